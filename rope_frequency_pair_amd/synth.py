"""Seeded synthetic inputs shaped like the pages' workloads.

Holds no part of the method's arithmetic: only shapes and seeded draws.  The
tests, the benchmark and the oracle checks all take their inputs from here.

Recipe: every tensor is iid N(0, 1) drawn in float32 from a torch.Generator
seeded with ``seed`` (draw order Q, K, V), then cast to the workload dtype
(bf16 with round-to-nearest-even).  Small workloads draw on the CPU generator,
large ones on the device generator of the GPU they run on.
"""

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str              # "prefill" | "decode" | "request"
    batch: int
    h_q: int
    h_kv: int
    head_dim: int
    rope_base: float
    k_turns: float
    n: int                 # prefill length / cache length
    dtype: torch.dtype
    seed: int
    splits: int = 0        # decode split-KV count
    chunk: int = 0         # chunked prefill chunk length (whole request)
    decode_steps: int = 0


# The five workloads of the pages' shapes (model-shaped attention layers).
WORKLOADS = {
    "single-head-1k": Workload("single-head-1k", "prefill", 1, 1, 1, 64, 1e4, 4.0, 1024,
                               torch.float32, 1000),
    "qwen2.5-0.5b-32k": Workload("qwen2.5-0.5b-32k", "prefill", 1, 14, 2, 64, 1e6, 8.0, 32768,
                                 torch.bfloat16, 1001),
    "llama-3.2-3b-128k": Workload("llama-3.2-3b-128k", "prefill", 1, 24, 8, 128, 5e5, 8.0, 131072,
                                  torch.bfloat16, 1002),
    "qwen2.5-7b-1m-decode-512k": Workload("qwen2.5-7b-1m-decode-512k", "decode", 8, 28, 4, 128, 1e7,
                                          8.0, 524288, torch.bfloat16, 1003, splits=64),
    "qwen2.5-7b-1m-request-1m": Workload("qwen2.5-7b-1m-request-1m", "request", 1, 28, 4, 128, 1e7,
                                         64.0, 1048576, torch.bfloat16, 1004, chunk=65536,
                                         decode_steps=128),
}


def _randn(shape, gen, device, dtype):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)


def generator(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def prefill_inputs(batch, h_q, h_kv, n_q, n_kv, head_dim, dtype, seed, device="cpu", gen_device=None):
    """(q, k, v) with q [B, Hq, Nq, d], k/v [B, Hkv, Nkv, d] on ``device``."""
    gen_device = gen_device or ("cpu" if device == "cpu" else device)
    g = generator(seed, gen_device)
    q = _randn((batch, h_q, n_q, head_dim), g, gen_device, dtype)
    k = _randn((batch, h_kv, n_kv, head_dim), g, gen_device, dtype)
    v = _randn((batch, h_kv, n_kv, head_dim), g, gen_device, dtype)
    return q.to(device), k.to(device), v.to(device)


def decode_inputs(batch, h_q, h_kv, cache_len, head_dim, dtype, seed, device="cpu", gen_device=None):
    """(q, k_cache, v_cache): q [B, Hq, d], caches [B, Hkv, L, d]; drawn per
    sequence (q, then each sequence's K, then V) to bound temporary memory."""
    gen_device = gen_device or ("cpu" if device == "cpu" else device)
    g = generator(seed, gen_device)
    q = _randn((batch, h_q, head_dim), g, gen_device, dtype).to(device)
    kc = torch.empty((batch, h_kv, cache_len, head_dim), dtype=dtype, device=device)
    vc = torch.empty((batch, h_kv, cache_len, head_dim), dtype=dtype, device=device)
    for b in range(batch):
        kc[b] = _randn((h_kv, cache_len, head_dim), g, gen_device, dtype).to(device)
    for b in range(batch):
        vc[b] = _randn((h_kv, cache_len, head_dim), g, gen_device, dtype).to(device)
    return q, kc, vc


def workload_prefill_inputs(w, device="cuda", n=None):
    """Inputs of a prefill workload (optionally at a different length n)."""
    n = n or w.n
    gen_device = "cpu" if w.n <= 32768 else device
    return prefill_inputs(w.batch, w.h_q, w.h_kv, n, n, w.head_dim, w.dtype, w.seed, device, gen_device)


def workload_decode_inputs(w, device="cuda"):
    return decode_inputs(w.batch, w.h_q, w.h_kv, w.n, w.head_dim, w.dtype, w.seed, device, device)


def request_inputs(w, device="cuda"):
    """Inputs of the whole-request workload: q [B, Hq, N, d] of the prompt,
    q_dec [steps, B, Hq, d] of the decode steps, and the caches k, v
    [B, Hkv, N + steps, d] (token N + s is the key / value the decode step s
    appends).  Drawn on the device generator in the order q, q_dec, k, v,
    per kv head for the caches."""
    g = generator(w.seed, device)
    n_all = w.n + w.decode_steps
    q = _randn((w.batch, w.h_q, w.n, w.head_dim), g, device, w.dtype)
    q_dec = _randn((w.decode_steps, w.batch, w.h_q, w.head_dim), g, device, w.dtype)
    k = torch.empty((w.batch, w.h_kv, n_all, w.head_dim), dtype=w.dtype, device=device)
    v = torch.empty((w.batch, w.h_kv, n_all, w.head_dim), dtype=w.dtype, device=device)
    for h in range(w.h_kv):
        k[:, h] = _randn((w.batch, n_all, w.head_dim), g, device, w.dtype)
    for h in range(w.h_kv):
        v[:, h] = _randn((w.batch, n_all, w.head_dim), g, device, w.dtype)
    return q, q_dec, k, v


def block_selection(batch, h_q, n_q, n_kv, seed, density=0.1, sink=1, local=4, block=64, q_pos0=0,
                    vertical=False):
    """Seeded boolean block selection [batch, h_q, ceil(n_q/block),
    ceil(n_kv/block)] with the structure block-sparse attention methods
    produce: the first `sink` key blocks, a local band of `local` key blocks
    ending at the block holding the query block's last position, and earlier
    key blocks with probability `density`: drawn independently per (batch,
    head, query block), or with vertical=True once per (batch, head) and
    shared by all its query blocks (vertical lines plus the diagonal band, the
    vertical-slash shape).  Blocks after the band stay unselected.  Drawn with
    numpy's PCG64 generator seeded with `seed` on the host."""
    import numpy as np
    n_qb, n_kb = -(-n_q // block), -(-n_kv // block)
    rng = np.random.default_rng(seed)
    if vertical:
        sel = np.broadcast_to(rng.random((batch, h_q, 1, n_kb), dtype=np.float32) < density,
                              (batch, h_q, n_qb, n_kb)).copy()
    else:
        sel = rng.random((batch, h_q, n_qb, n_kb), dtype=np.float32) < density
    kb = np.arange(n_kb)[None, :]
    last_pos = q_pos0 + np.minimum((np.arange(n_qb) + 1) * block, n_q) - 1
    diag = np.minimum(last_pos // block, n_kb - 1)[:, None]
    sel &= (kb <= diag)[None, None]
    band = (kb <= diag) & (kb > diag - local)
    sel |= (band | (kb < sink))[None, None]
    return torch.from_numpy(sel)


def decode_block_selection(batch, h_kv, kv_len, seed, density=0.05, sink=1, local=4, block=64):
    """Seeded boolean key-block selection for decode [batch, h_kv,
    ceil(max(kv_len)/block)]: the first `sink` blocks, the last `local` blocks
    of each sequence's keys, and every other block with probability
    `density`, independently per (sequence, kv head) -- the shape of a
    page-level top-k selection.  numpy PCG64 seeded with `seed`."""
    import numpy as np
    lens = [int(x) for x in (kv_len if hasattr(kv_len, "__len__") else [kv_len] * batch)]
    n_kb = -(-max(lens) // block)
    rng = np.random.default_rng(seed)
    sel = rng.random((batch, h_kv, n_kb), dtype=np.float32) < density
    kb = np.arange(n_kb)
    for b, n in enumerate(lens):
        last = -(-n // block)
        sel[b, :, kb >= last] = False
        sel[b, :, (kb < sink) | ((kb >= last - local) & (kb < last))] = True
    return torch.from_numpy(sel)

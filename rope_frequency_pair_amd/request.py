"""One attention layer of a whole request through libatw: chunked causal
prefill of the prompt, then single-token decode steps that append to the
cache ("ATFlash — Per-RoPE-Wavelength Attention Windows", README, "The
idea": one set of windows serves prefill and decode; the arXiv abstract's
end-to-end figure is a full request at a 1M-token context).

Host-side sequencing only: every computation is a libatw call.
"""

from . import binding


def decode_splits(w):
    """Split-KV count of the request's decode steps: the workload's own, else
    enough (sequence, kv head, split) work items for ~8 per CU of the 256 CUs
    (a single sequence with few kv heads would otherwise leave most CUs idle
    and the step bound by memory latency rather than bandwidth)."""
    if w.splits:
        return w.splits
    return max(64, -(-2048 // (w.batch * w.h_kv)))


class RequestBuffers:
    """Device buffers a request needs beyond its inputs, allocated once."""

    def __init__(self, w, device="cuda"):
        import torch
        n_all = w.n + w.decode_steps
        self.out_chunk = torch.empty((w.batch, w.h_q, w.chunk, w.head_dim), dtype=w.dtype, device=device)
        self.out_dec = torch.empty((w.decode_steps, w.batch, w.h_q, w.head_dim), dtype=w.dtype,
                                   device=device)
        self.ws_prefill = torch.empty(
            binding.prefill_workspace_bytes(binding.ATW_BF16, w.batch, w.h_kv, w.n, w.head_dim),
            dtype=torch.uint8, device=device)
        self.ws_decode = torch.empty(
            binding.decode_workspace_bytes(w.batch, w.h_q, w.head_dim, decode_splits(w)),
            dtype=torch.uint8, device=device)
        self.k_bands = torch.empty((w.batch, w.h_kv, w.head_dim // 16, n_all, 16), dtype=w.dtype,
                                   device=device)


def run_request(w, q, q_dec, k, v, bufs, *, window_on=True, stream=None, on_chunk=None):
    """Prefill the first w.n tokens in chunks of w.chunk (chunk c: queries
    [c*chunk, (c+1)*chunk) at their positions against keys [0, (c+1)*chunk)),
    band the prompt's keys, then run w.decode_steps steps: step s bands key
    w.n + s (its append) and attends with the query at position w.n + s over
    keys [0, w.n + s].  Returns (out of the last prefill chunk, decode outputs
    [steps, B, Hq, d]); on_chunk(c, out) is called after each chunk."""
    n, ch = w.n, w.chunk
    splits = decode_splits(w)
    for c in range(n // ch):
        binding.prefill(q[:, :, c * ch:(c + 1) * ch], k[:, :, :(c + 1) * ch], v[:, :, :(c + 1) * ch],
                        rope_base=w.rope_base, k_turns=w.k_turns, q_pos0=c * ch, causal=True,
                        window_on=window_on, out=bufs.out_chunk, workspace=bufs.ws_prefill,
                        stream=stream)
        if on_chunk is not None:
            on_chunk(c, bufs.out_chunk)
    binding.kcache_band(k, bufs.k_bands, t0=0, n_tokens=n, stream=stream)
    for s in range(w.decode_steps):
        pos = n + s
        binding.kcache_band(k, bufs.k_bands, t0=pos, n_tokens=1, stream=stream)
        binding.decode_banded(q_dec[s], bufs.k_bands, v, [pos + 1] * w.batch, [pos] * w.batch,
                              rope_base=w.rope_base, k_turns=w.k_turns, causal=True,
                              window_on=window_on, num_splits=splits, workspace=bufs.ws_decode,
                              out=bufs.out_dec[s], stream=stream)
    return bufs.out_chunk, bufs.out_dec

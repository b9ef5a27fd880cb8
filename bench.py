"""Benchmark of the windowed attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu]

One step = one call of atw_prefill (window planning + the windowed prefill
kernel) on the Llama-3.2-3B-shaped attention layer at 128K tokens
(batch 1, 24 query / 8 kv heads, d = 128, rope base 5e5, k = 8, causal, bf16,
inputs resident in HBM).  ``value`` is the algorithmic throughput of that
step: (2*d*C + 4*R) flops per (batch, query head), C = visible cells,
R = retained pair-terms, divided by the measured step time.

Also reported on the same line: the dense-equivalent rate, window ON/OFF
speedups (128K and the 32K/64K sweep, the Qwen2.5-0.5B 32K shape), the
split-KV decode HBM rate on the Qwen2.5-7B-1M-shaped 512K cache (8
sequences, 64 splits), the prefill kernel's roofline fraction from
per-launch HIP events, and the fp64 CPU oracle timed on a bounded sample.
Inputs are seeded synthetic N(0,1) tensors (see rope_frequency_pair_amd.synth).
"""

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
HEADLINE = "llama-3.2-3b-128k"
CPU_SHARE = 16                # cores of a one-GPU job on the GPU hosts
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "prefill_llama128k_traffic.json")
KERNEL_SOURCES = ["rope_frequency_pair_amd/csrc/prefill.hip", "rope_frequency_pair_amd/csrc/device_common.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# rope_scaling of the Llama-3.2-3B config (llama3 rule)
LLAMA32_SCALING = {"rope_type": "llama3", "factor": 32.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
                   "original_max_position_embeddings": 8192}


def prefill_flops(atw, n, d, h_q, batch, base, k_turns, window_on, rope_scaling=None):
    """(algorithmic, dense-equivalent) flops of one causal prefill of length n."""
    pruned, total = atw.pruned_terms(n, n, 0, d, base, k_turns, True, window_on, rope_scaling)
    h = d // 2
    cells = total // h
    retained = total - pruned
    per_head_alg = 2 * d * cells + 4 * retained
    per_head_dense = 4 * d * cells
    return per_head_alg * h_q * batch, per_head_dense * h_q * batch, pruned / total


def request_prefill_flops(atw, w):
    """Algorithmic and dense-equivalent flops of the whole request's chunked
    prefill (sum over chunks) and its pruned share."""
    h = w.head_dim // 2
    fo = fd = pr_all = tot_all = 0
    for c in range(w.n // w.chunk):
        pruned, total = atw.pruned_terms(w.chunk, (c + 1) * w.chunk, c * w.chunk, w.head_dim, w.rope_base,
                                         w.k_turns, True, True)
        cells = total // h
        fo += (2 * w.head_dim * cells + 4 * (total - pruned)) * w.h_q * w.batch
        fd += 4 * w.head_dim * cells * w.h_q * w.batch
        pr_all += pruned
        tot_all += total
    return fo, fd, pr_all / tot_all


def decode_bytes(atw, L, d, h_kv, batch, base, k_turns, window_on):
    """Algorithmic HBM bytes of one decode step: retained K pair slices
    (2 bytes per element, exact per-key window) + all of V, per kv head."""
    pruned, total = atw.pruned_terms(1, L, L, d, base, k_turns, True, window_on)
    h = d // 2
    k_bytes = 4 * (total - pruned)      # total pair-terms of the row = h * L; 2 elems * 2 B each
    v_bytes = 2 * d * L
    return (k_bytes + v_bytes) * h_kv * batch, pruned / total


def decode_line_bytes_banded(atw, L, q_pos, d, h_kv, batch, base, k_turns):
    """HBM bytes one decode step must move at the memory system's 128-byte
    line granularity with the pair-banded K cache (a line = one 8-pair band
    of 4 consecutive keys, fetched if the band is in the window for any of
    them) + all of V."""
    import numpy as np
    w = np.array(atw.window_widths(d, base, k_turns, True), dtype=np.int64)
    first = np.arange(0, L, 4)                       # first key of each line
    last = np.minimum(first + 3, L - 1)
    lines = sum(int((q_pos - last <= w[8 * c + 7]).sum()) for c in range(d // 16))
    return (lines * 128 + 2 * d * L) * h_kv * batch


def time_launches(fn, stream, n):
    """Per-launch durations (ms) from HIP events recorded on the launch stream."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def time_steps(fn, stream, n):
    """Mean duration (ms) of n back-to-back launches between two HIP events on
    the launch stream: the host work of each call overlaps the device work of
    the one before, as in a serving loop, so a short step is not charged for
    the host-side call (about 14 us per call through the Python binding)."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) / n]


def cpu_baseline(sample_rows=256):
    """Time the fp64 oracle on a bounded sample of the headline workload."""
    import multiprocessing as mp

    import numpy as np
    import torch

    from rope_frequency_pair_amd import synth
    w = synth.WORKLOADS[HEADLINE]
    # one single-threaded worker per core this process may run on, capped at
    # the 16-core share a one-GPU job gets on the GPU hosts (their
    # os.cpu_count() reports the whole machine)
    host_cores = os.cpu_count() or 1
    allowed = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else host_cores
    workers = max(1, min(CPU_SHARE, allowed, sample_rows))
    rng = np.random.default_rng(0)
    rows = sorted(int(x) for x in rng.integers(w.n // 2, w.n, size=sample_rows))
    # inputs of one (query head, kv head) pair on the CPU generator: same shape,
    # same distribution as the GPU draw
    g = synth.generator(w.seed)
    q = torch.randn((w.n, w.head_dim), generator=g)[rows].to(torch.bfloat16).float().numpy()
    k = torch.randn((w.n, w.head_dim), generator=g).to(torch.bfloat16).float().numpy()
    v = torch.randn((w.n, w.head_dim), generator=g).to(torch.bfloat16).float().numpy()
    chunks = [list(range(i, len(rows), workers)) for i in range(workers)]
    args = [(q[c], k, v, [rows[i] for i in c], w.rope_base, w.k_turns) for c in chunks if c]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(len(args)) as pool:
        pool.map(_oracle_rows, args)
    dt = time.perf_counter() - t0
    import oracle
    flops = 0
    for r in rows:
        p, t = oracle.pruned_terms(1, r + 1, r, w.head_dim, w.rope_base, w.k_turns)
        flops += 2 * w.head_dim * (r + 1) + 4 * (t - p)
    rate = flops / dt
    # the whole step at the sampled rate (rows sampled from the second half of
    # the sequence, so per-row cost is proportional to the flops counted)
    p_all, t_all = oracle.pruned_terms(w.n, w.n, 0, w.head_dim, w.rope_base, w.k_turns)
    full = w.batch * w.h_q * (2 * w.head_dim * (w.n * (w.n + 1) // 2) + 4 * (t_all - p_all))
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": len(args), "kind": "oracle",
            "host_cores": host_cores, "affinity_cores": allowed, "workers": len(args),
            "sample": f"{len(rows)} query rows (positions {rows[0]}..{rows[-1]}) of one head of the "
                      f"128K Llama-3.2-3B-shaped prefill, window on, float64 numpy; {dt:.1f} s wall; "
                      f"extrapolation to the whole step ({w.h_q} heads x {w.n} rows) at this rate: "
                      f"{full / rate / 3600:.1f} h"}


def _oracle_rows(a):
    os.environ["OMP_NUM_THREADS"] = "1"
    import numpy as np
    import oracle
    q, k, v, rows, base, k_turns = a
    for i, r in enumerate(rows):
        oracle.prefill(q[None, None, i:i + 1], k[None, None, :r + 1], v[None, None, :r + 1], r, base, k_turns)
    return len(rows)


def decode_profile_run(atw, synth, torch, dev):
    """The 512K decode step alone, for counter runs: row cache ON x2, OFF x2,
    then banded cache ON x2, OFF x2, in that launch order."""
    wd = synth.WORKLOADS["qwen2.5-7b-1m-decode-512k"]
    qd, kc, vc = synth.workload_decode_inputs(wd)
    L = wd.n
    ws = torch.empty(atw.decode_workspace_bytes(wd.batch, wd.h_q, wd.head_dim, wd.splits),
                     dtype=torch.uint8, device=dev)
    od = torch.empty((wd.batch, wd.h_q, wd.head_dim), dtype=torch.bfloat16, device=dev)
    kw = dict(rope_base=wd.rope_base, k_turns=wd.k_turns, num_splits=wd.splits, workspace=ws, out=od)
    for on in (True, True, False, False):
        atw.decode(qd, kc, vc, [L] * wd.batch, [L] * wd.batch, window_on=on, **kw)
    kb = atw.kcache_band(kc)
    for on in (True, True, False, False):
        atw.decode_banded(qd, kb, vc, [L] * wd.batch, [L] * wd.batch, window_on=on, **kw)
    torch.cuda.synchronize()
    by_on, _ = decode_bytes(atw, L, wd.head_dim, wd.h_kv, wd.batch, wd.rope_base, wd.k_turns, True)
    by_off, _ = decode_bytes(atw, L, wd.head_dim, wd.h_kv, wd.batch, wd.rope_base, wd.k_turns, False)
    by_line = decode_line_bytes_banded(atw, L, L, wd.head_dim, wd.h_kv, wd.batch, wd.rope_base, wd.k_turns)
    print(json.dumps({"decode_profile": wd.name, "bytes_on": by_on, "bytes_off": by_off,
                      "banded_line_bytes_on": by_line}), flush=True)


def single_profile_run(name, atw, synth, torch, dev):
    """One workload alone, window-on launches only, for counter runs:
    qwen32k (head_dim 64 prefill), sparse-independent (128K block-sparse
    prefill with per-query-block selections), sparse-decode (512K decode over
    a banded cache with a block selection)."""
    if name == "qwen32k":
        wq = synth.WORKLOADS["qwen2.5-0.5b-32k"]
        q1, k1, v1 = synth.workload_prefill_inputs(wq)
        o1 = torch.empty_like(q1)
        for _ in range(2):
            atw.prefill(q1, k1, v1, rope_base=wq.rope_base, k_turns=wq.k_turns, out=o1)
    elif name == "sparse-independent":
        w = synth.WORKLOADS[HEADLINE]
        q, k, v = synth.workload_prefill_inputs(w)
        out = torch.empty_like(q)
        sel = synth.block_selection(w.batch, w.h_q, w.n, w.n, w.seed + 100, vertical=False)
        smask = atw.pack_block_mask(sel).to(dev)
        for _ in range(2):
            atw.prefill_sparse(q, k, v, smask, rope_base=w.rope_base, k_turns=w.k_turns, out=out)
    elif name == "sparse-decode":
        wd = synth.WORKLOADS["qwen2.5-7b-1m-decode-512k"]
        qd, kc, vc = synth.workload_decode_inputs(wd)
        L = wd.n
        kb = atw.kcache_band(kc)
        del kc
        dsel = synth.decode_block_selection(wd.batch, wd.h_kv, L, wd.seed + 100)
        dmask = atw.pack_block_mask(dsel).to(dev)
        ws = torch.empty(atw.decode_workspace_bytes(wd.batch, wd.h_q, wd.head_dim, wd.splits),
                         dtype=torch.uint8, device=dev)
        od = torch.empty_like(qd)
        # 2 warm-up + 10 launches: a launch is ~0.1 ms, so a trace needs several
        for _ in range(12):
            atw.decode_sparse(qd, kb, vc, [L] * wd.batch, [L] * wd.batch, dmask, rope_base=wd.rope_base,
                              k_turns=wd.k_turns, num_splits=wd.splits, k_banded=True, workspace=ws, out=od)
    else:
        raise SystemExit(f"unknown profile workload {name}")
    torch.cuda.synchronize()
    print(json.dumps({"profile_run": name}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=6)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--quick", action="store_true", help="headline prefill only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--on-only", action="store_true",
                    help="profiling: window-on launches of the headline prefill only (no ON/OFF rounds)")
    ap.add_argument("--decode-only", action="store_true",
                    help="profiling: the 512K decode step only (row and banded cache, window on then "
                         "off, two launches each)")
    ap.add_argument("--profile", choices=["qwen32k", "sparse-independent", "sparse-decode"],
                    help="profiling: two window-on launches of one more workload only")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(each call runs on one device; prefill would shard over (batch, kv head) groups and "
              "decode over its key splits, with no change to the kernels)", file=sys.stderr)
        sys.exit(2)

    import torch
    import rope_frequency_pair_amd as atw
    from rope_frequency_pair_amd import synth

    atw.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    w = synth.WORKLOADS[HEADLINE]
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 1073741824 bytes read, 1073741824 bytes written")
        del src, dst
    if args.decode_only:
        decode_profile_run(atw, synth, torch, dev)
        return
    if args.profile:
        single_profile_run(args.profile, atw, synth, torch, dev)
        return
    log(f"[bench] {atw.version()} on {torch.cuda.get_device_name(0)}; inputs for {w.name}")
    q, k, v = synth.workload_prefill_inputs(w)
    out = torch.empty_like(q)

    def step(on=True, qq=q, kk=k, vv=v, oo=out, wl=w, sc=None):
        atw.prefill(qq, kk, vv, rope_base=wl.rope_base, k_turns=wl.k_turns, window_on=on, out=oo,
                    rope_scaling=sc)

    flops_on, dense, share = prefill_flops(atw, w.n, w.head_dim, w.h_q, w.batch, w.rope_base, w.k_turns, True)
    flops_off, _, _ = prefill_flops(atw, w.n, w.head_dim, w.h_q, w.batch, w.rope_base, w.k_turns, False)

    for _ in range(args.warmup):
        step(True)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    launch_ms = time_launches(lambda: step(True), stream, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    kern_ms = statistics.mean(launch_ms)
    value = flops_on / (ms_step * 1e-3) / 1e12

    # window ON vs OFF, interleaved, median of >= 6 rounds each
    rounds = 0 if args.on_only else max(6, args.steps)
    on_ms, off_ms = [], []
    for _ in range(rounds):
        on_ms += time_launches(lambda: step(True), stream, 1)
        off_ms += time_launches(lambda: step(False), stream, 1)
    if args.on_only:
        on_ms, off_ms = launch_ms, launch_ms
    med_on, med_off = statistics.median(on_ms), statistics.median(off_ms)
    ceiling = 2.0 / (1.0 + (1.0 - share))
    result = {
        "metric": "windowed prefill TFLOP/s (Llama-3.2-3B shape, 128K, window on)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.n, "h_q": w.h_q, "h_kv": w.h_kv,
                   "head_dim": w.head_dim, "rope_base": w.rope_base, "k": w.k_turns, "causal": True,
                   "parallelism": "none (1 GPU)"},
        "prefill_128k": {
            "pruned_share": round(share, 4),
            "tflops_algorithmic_on": round(flops_on / (med_on * 1e-3) / 1e12, 1),
            "tflops_dense_equiv_on": round(dense / (med_on * 1e-3) / 1e12, 1),
            "tflops_off": round(flops_off / (med_off * 1e-3) / 1e12, 1),
            "ms_on_median": round(med_on, 3),
            "ms_off_median": round(med_off, 3),
            "on_off_speedup": round(med_off / med_on, 3),
            "ceiling_2_over_1_plus_s": round(ceiling, 3),
        },
    }
    sha = kernel_sha()
    traffic = None
    if os.path.exists(PROFILE_TRAFFIC):
        with open(PROFILE_TRAFFIC) as f:
            prof = json.load(f)
        if prof.get("kernel_sha") == sha:
            traffic = prof.get("traffic_bytes")
    result["roofline"] = {"bound": "mfma", "achieved": round(flops_on / (kern_ms * 1e-3) / 1e12, 1),
                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(flops_on / (kern_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "traffic": traffic, "kernel": "prefill_bf16_kernel<128, false, true>",
                          "kernel_ms_mean": round(kern_ms, 3), "kernel_sha": sha}

    if not (args.quick or args.on_only):
        # ON/OFF sweep for "ON beats OFF at every context >= 32K"
        sweep = {}
        for n in (32768, 65536):
            qs, ks, vs = q[:, :, :n], k[:, :, :n], v[:, :, :n]
            os_ = out[:, :, :n]
            a, b = [], []
            # short launches: a few untimed pairs first, then 20 interleaved
            # rounds (the clock settles over the first few after the 128K runs)
            for _ in range(3):
                step(True, qs, ks, vs, os_)
                step(False, qs, ks, vs, os_)
            for _ in range(20):
                a += time_launches(lambda: step(True, qs, ks, vs, os_), stream, 1)
                b += time_launches(lambda: step(False, qs, ks, vs, os_), stream, 1)
            fo, _, sh = prefill_flops(atw, n, w.head_dim, w.h_q, w.batch, w.rope_base, w.k_turns, True)
            sweep[str(n)] = {"ms_on": round(statistics.median(a), 3), "ms_off": round(statistics.median(b), 3),
                             "on_off_speedup": round(statistics.median(b) / statistics.median(a), 3),
                             "tflops_algorithmic_on": round(fo / (statistics.median(a) * 1e-3) / 1e12, 1),
                             "pruned_share": round(sh, 4)}
        result["prefill_llama_sweep"] = sweep

        # the same 128K step with the model's own rope scaling (llama3 rule): the
        # windows come from the rescaled wavelengths
        a, b = [], []
        for _ in range(6):
            a += time_launches(lambda: step(True, sc=LLAMA32_SCALING), stream, 1)
            b += time_launches(lambda: step(False, sc=LLAMA32_SCALING), stream, 1)
        fo, _, sh = prefill_flops(atw, w.n, w.head_dim, w.h_q, w.batch, w.rope_base, w.k_turns, True,
                                  LLAMA32_SCALING)
        result["prefill_128k_llama3_scaling"] = {
            "rope_scaling": LLAMA32_SCALING, "pruned_share": round(sh, 4),
            "ms_on": round(statistics.median(a), 3), "ms_off": round(statistics.median(b), 3),
            "on_off_speedup": round(statistics.median(b) / statistics.median(a), 3),
            "tflops_algorithmic_on": round(fo / (statistics.median(a) * 1e-3) / 1e12, 1),
            "ceiling_2_over_1_plus_s": round(2.0 / (2.0 - sh), 3)}

        # the window on top of a block-sparse token selection (64x64 blocks:
        # the first key block, a local band of 4 blocks, and 10% of the earlier
        # blocks drawn once per head for all its query blocks (vertical-slash
        # shape) or independently per query block)
        sparse = {}
        for pattern, vertical in (("vertical_slash", True), ("independent_per_query_block", False)):
            log(f"[bench] block-sparse selection at 128K: {pattern}")
            sel = synth.block_selection(w.batch, w.h_q, w.n, w.n, w.seed + 100, vertical=vertical)
            smask = atw.pack_block_mask(sel).to(q.device)
            causal_blocks = (w.n // 64) * (w.n // 64 + 1) // 2 * w.h_q * w.batch
            density = float(sel.sum()) / causal_blocks
            del sel

            def sstep(on):
                atw.prefill_sparse(q, k, v, smask, rope_base=w.rope_base, k_turns=w.k_turns, window_on=on,
                                   out=out)

            sstep(True)
            sstep(False)
            a, b = [], []
            for _ in range(6):
                a += time_launches(lambda: sstep(True), stream, 1)
                b += time_launches(lambda: sstep(False), stream, 1)
            h = w.head_dim // 2
            pr = tot = 0
            for hq in range(w.h_q):
                p_, t_ = atw.pruned_terms_sparse(w.n, w.n, 0, w.head_dim, w.rope_base, w.k_turns,
                                                 smask[0, hq])
                pr += p_
                tot += t_
            cells = tot // h
            alg = (2 * w.head_dim * cells + 4 * (tot - pr)) * w.batch
            dense_s = 4 * w.head_dim * cells * w.batch
            sparse[pattern] = {
                "block_density_of_causal": round(density, 4), "pruned_share": round(pr / tot, 4),
                "ms_on": round(statistics.median(a), 3), "ms_off": round(statistics.median(b), 3),
                "on_off_speedup": round(statistics.median(b) / statistics.median(a), 3),
                "tflops_algorithmic_on": round(alg / (statistics.median(a) * 1e-3) / 1e12, 1),
                "tflops_dense_equiv_on": round(dense_s / (statistics.median(a) * 1e-3) / 1e12, 1),
                "ceiling_2_over_1_plus_s": round(2.0 / (2.0 - pr / tot), 3),
                "speedup_vs_dense_window_on": round(med_on / statistics.median(a), 2)}
            del smask
        sparse["selection"] = ("64x64 blocks: first key block + local band of 4 + 10% of earlier blocks "
                               "(vertical_slash: one draw per head; independent: one per query block)")
        result["prefill_128k_block_sparse"] = sparse
        del q, k, v, out
        torch.cuda.empty_cache()

        # Qwen2.5-0.5B shape, 32K, d = 64
        wq = synth.WORKLOADS["qwen2.5-0.5b-32k"]
        log(f"[bench] {wq.name}")
        q1, k1, v1 = synth.workload_prefill_inputs(wq)
        o1 = torch.empty_like(q1)
        a, b = [], []
        for _ in range(3):
            step(True, q1, k1, v1, o1, wq)
            step(False, q1, k1, v1, o1, wq)
        for _ in range(20):
            a += time_launches(lambda: step(True, q1, k1, v1, o1, wq), stream, 1)
            b += time_launches(lambda: step(False, q1, k1, v1, o1, wq), stream, 1)
        fo, fd, sh = prefill_flops(atw, wq.n, wq.head_dim, wq.h_q, wq.batch, wq.rope_base, wq.k_turns, True)
        result["prefill_qwen_32k"] = {"ms_on": round(statistics.median(a), 3),
                                      "ms_off": round(statistics.median(b), 3),
                                      "on_off_speedup": round(statistics.median(b) / statistics.median(a), 3),
                                      "tflops_algorithmic_on": round(fo / (statistics.median(a) * 1e-3) / 1e12, 1),
                                      "tflops_dense_equiv_on": round(fd / (statistics.median(a) * 1e-3) / 1e12, 1),
                                      "pruned_share": round(sh, 4)}
        del q1, k1, v1, o1
        torch.cuda.empty_cache()

        # Qwen2.5-7B-1M shape (28 / 4 heads, d = 128, base 1e7, k = 8): one
        # causal prefill call of 256K and of 512K tokens, window ON vs OFF
        wl7 = synth.WORKLOADS["qwen2.5-7b-1m-decode-512k"]
        longp = {}
        for n in (262144, 524288):
            log(f"[bench] Qwen2.5-7B-1M-shaped prefill, {n} tokens")
            ql, kl, vl = synth.prefill_inputs(1, wl7.h_q, wl7.h_kv, n, n, wl7.head_dim, torch.bfloat16,
                                              wl7.seed + 7, device=dev)
            ol = torch.empty_like(ql)
            step(True, ql, kl, vl, ol, wl7)
            step(False, ql, kl, vl, ol, wl7)
            a, b = [], []
            for _ in range(3):
                a += time_launches(lambda: step(True, ql, kl, vl, ol, wl7), stream, 1)
                b += time_launches(lambda: step(False, ql, kl, vl, ol, wl7), stream, 1)
            fo, fd, sh = prefill_flops(atw, n, wl7.head_dim, wl7.h_q, 1, wl7.rope_base, wl7.k_turns, True)
            longp[str(n)] = {"ms_on": round(statistics.median(a), 2), "ms_off": round(statistics.median(b), 2),
                             "on_off_speedup": round(statistics.median(b) / statistics.median(a), 3),
                             "tflops_algorithmic_on": round(fo / (statistics.median(a) * 1e-3) / 1e12, 1),
                             "tflops_dense_equiv_on": round(fd / (statistics.median(a) * 1e-3) / 1e12, 1),
                             "pruned_share": round(sh, 4), "ceiling_2_over_1_plus_s": round(2.0 / (2.0 - sh), 3)}
            del ql, kl, vl, ol
            torch.cuda.empty_cache()
        result["prefill_qwen7b_1m_shape_long"] = longp

        # split-KV decode, Qwen2.5-7B-1M shape, 512K cache, 8 sequences, 64 splits
        wd = synth.WORKLOADS["qwen2.5-7b-1m-decode-512k"]
        log(f"[bench] {wd.name}")
        qd, kc, vc = synth.workload_decode_inputs(wd)
        L = wd.n
        ws = torch.empty(atw.decode_workspace_bytes(wd.batch, wd.h_q, wd.head_dim, wd.splits),
                         dtype=torch.uint8, device=dev)
        od = torch.empty((wd.batch, wd.h_q, wd.head_dim), dtype=torch.bfloat16, device=dev)

        def dstep(on):
            atw.decode(qd, kc, vc, [L] * wd.batch, [L] * wd.batch, rope_base=wd.rope_base,
                       k_turns=wd.k_turns, window_on=on, num_splits=wd.splits, workspace=ws, out=od)

        for _ in range(3):
            dstep(True)
            dstep(False)
        a, b = [], []
        for _ in range(10):
            a += time_steps(lambda: dstep(True), stream, 10)
            b += time_steps(lambda: dstep(False), stream, 10)
        by_on, sh = decode_bytes(atw, L, wd.head_dim, wd.h_kv, wd.batch, wd.rope_base, wd.k_turns, True)
        by_off, _ = decode_bytes(atw, L, wd.head_dim, wd.h_kv, wd.batch, wd.rope_base, wd.k_turns, False)
        ma, mb = statistics.median(a), statistics.median(b)
        result["decode_512k"] = {"ms_on": round(ma, 4), "ms_off": round(mb, 4),
                                 "gbs_algorithmic_on": round(by_on / (ma * 1e-3) / 1e9, 1),
                                 "gbs_off": round(by_off / (mb * 1e-3) / 1e9, 1),
                                 "hbm_frac_on": round(by_on / (ma * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                 "hbm_frac_off": round(by_off / (mb * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                 "on_off_speedup": round(mb / ma, 3),
                                 "k_pair_terms_pruned": round(sh, 4),
                                 "bytes_on": by_on, "bytes_off": by_off}

        # the same step over a pair-banded K cache (whole 128-byte lines pruned)
        kb = atw.kcache_band(kc)
        del kc
        torch.cuda.synchronize()

        def bstep(on):
            atw.decode_banded(qd, kb, vc, [L] * wd.batch, [L] * wd.batch, rope_base=wd.rope_base,
                              k_turns=wd.k_turns, window_on=on, num_splits=wd.splits, workspace=ws,
                              out=od)

        for _ in range(3):
            bstep(True)
            bstep(False)
        a, b = [], []
        for _ in range(10):
            a += time_steps(lambda: bstep(True), stream, 10)
            b += time_steps(lambda: bstep(False), stream, 10)
        ma, mb = statistics.median(a), statistics.median(b)
        by_line = decode_line_bytes_banded(atw, L, L, wd.head_dim, wd.h_kv, wd.batch, wd.rope_base,
                                           wd.k_turns)
        result["decode_512k_banded"] = {
            "ms_on": round(ma, 4), "ms_off": round(mb, 4),
            "gbs_algorithmic_on": round(by_on / (ma * 1e-3) / 1e9, 1),
            "hbm_frac_on": round(by_on / (ma * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "gbs_line_bytes_on": round(by_line / (ma * 1e-3) / 1e9, 1),
            "on_off_speedup": round(mb / ma, 3),
            "on_vs_row_layout_off": round(result["decode_512k"]["ms_off"] / ma, 3),
            "line_bytes_on": by_line}

        # the window on top of a page-level block selection in decode (first
        # block, the last four blocks and 5% of the rest, per (sequence, kv
        # head)), banded cache
        dsel = synth.decode_block_selection(wd.batch, wd.h_kv, L, wd.seed + 100)
        dmask = atw.pack_block_mask(dsel).to(dev)
        del dsel

        def sdstep(on):
            atw.decode_sparse(qd, kb, vc, [L] * wd.batch, [L] * wd.batch, dmask, rope_base=wd.rope_base,
                              k_turns=wd.k_turns, window_on=on, num_splits=wd.splits, k_banded=True,
                              workspace=ws, out=od)

        for _ in range(3):
            sdstep(True)
            sdstep(False)
        a, b = [], []
        for _ in range(10):
            a += time_steps(lambda: sdstep(True), stream, 10)
            b += time_steps(lambda: sdstep(False), stream, 10)
        sb_on = sb_off = keys = 0
        for bi in range(wd.batch):
            for h in range(wd.h_kv):
                pr, tot = atw.pruned_terms_sparse(1, L, L, wd.head_dim, wd.rope_base, wd.k_turns,
                                                  dmask[bi, h][None])
                n_keys = tot // (wd.head_dim // 2)
                keys += n_keys
                sb_on += 4 * (tot - pr) + 2 * wd.head_dim * n_keys
                sb_off += 4 * tot + 2 * wd.head_dim * n_keys
        ma, mb = statistics.median(a), statistics.median(b)
        result["decode_512k_block_sparse_banded"] = {
            "selection": "64-key blocks: first, last four and 5% of the rest per (sequence, kv head)",
            "key_fraction": round(keys / (L * wd.h_kv * wd.batch), 4),
            "ms_on": round(ma, 4), "ms_off": round(mb, 4), "on_off_speedup": round(mb / ma, 3),
            "gbs_algorithmic_on": round(sb_on / (ma * 1e-3) / 1e9, 1),
            "gbs_algorithmic_off": round(sb_off / (mb * 1e-3) / 1e9, 1),
            "hbm_frac_on": round(sb_on / (ma * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_on": sb_on, "bytes_off": sb_off,
            "speedup_vs_dense_banded_on": round(result["decode_512k_banded"]["ms_on"] / ma, 2)}
        del dmask

        # multi-token decode (draft tokens verified in one step) on the same
        # banded cache: T tokens per sequence at positions L-T .. L-1
        multi = {}
        for T in (2, 4):
            qm = torch.randn((wd.batch, T, wd.h_q, wd.head_dim), generator=synth.generator(wd.seed + T),
                             device="cpu").to(torch.bfloat16).to(dev)
            om = torch.empty_like(qm)
            wsm = torch.empty(atw.decode_multi_workspace_bytes(wd.batch, T, wd.h_q, wd.head_dim, wd.splits),
                              dtype=torch.uint8, device=dev)

            def mstep(on, T=T, qm=qm, om=om, wsm=wsm):
                atw.decode_multi(qm, kb, vc, [L] * wd.batch, [L - T] * wd.batch, rope_base=wd.rope_base,
                                 k_turns=wd.k_turns, window_on=on, num_splits=wd.splits, k_banded=True,
                                 workspace=wsm, out=om)

            for _ in range(2):
                mstep(True)
                mstep(False)
            a, b = [], []
            for _ in range(6):
                a += time_steps(lambda: mstep(True), stream, 10)
                b += time_steps(lambda: mstep(False), stream, 10)
            passes = -(-T // (16 // (wd.h_q // wd.h_kv)))
            multi[str(T)] = {"ms_on": round(statistics.median(a), 4), "ms_off": round(statistics.median(b), 4),
                             "on_off_speedup": round(statistics.median(b) / statistics.median(a), 3),
                             "cache_passes": passes,
                             "ms_per_token_on": round(statistics.median(a) / T, 4)}
            del qm, om, wsm
        result["decode_512k_multi_token_banded"] = multi
        del qd, kb, vc
        torch.cuda.empty_cache()

        # whole request, Qwen2.5-7B-1M shape: 16 x 64K chunked prefill + 128 decode steps
        from rope_frequency_pair_amd import request as req
        wr = synth.WORKLOADS["qwen2.5-7b-1m-request-1m"]
        log(f"[bench] {wr.name}")
        qr, qdr, kr, vr = synth.request_inputs(wr)
        bufs = req.RequestBuffers(wr)
        times = {}
        for on in (True, False):
            marks = []

            def mark(c, _out):
                if c == wr.n // wr.chunk - 1:
                    ev = torch.cuda.Event(enable_timing=True)
                    ev.record(stream)
                    marks.append(ev)

            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            req.run_request(wr, qr, qdr, kr, vr, bufs, window_on=on, on_chunk=mark)
            e1.record(stream)
            torch.cuda.synchronize()
            times[on] = (e0.elapsed_time(e1), e0.elapsed_time(marks[0]))
            log(f"[bench] request window_on={on}: {times[on][0]:.1f} ms")
        fo, fd, sh = request_prefill_flops(atw, wr)
        result["request_1m"] = {
            "ms_on": round(times[True][0], 1), "ms_off": round(times[False][0], 1),
            "on_off_speedup": round(times[False][0] / times[True][0], 3),
            "prefill_ms_on": round(times[True][1], 1), "prefill_ms_off": round(times[False][1], 1),
            "decode_ms_on": round(times[True][0] - times[True][1], 2),
            "decode_ms_off": round(times[False][0] - times[False][1], 2),
            "prefill_tflops_algorithmic_on": round(fo / (times[True][1] * 1e-3) / 1e12, 1),
            "prefill_pruned_share": round(sh, 4)}
        del qr, qdr, kr, vr, bufs
        torch.cuda.empty_cache()

    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

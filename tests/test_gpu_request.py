"""The whole-request workload (Qwen2.5-7B-1M shape, one layer): chunked
causal prefill of 1,048,576 tokens in 64K chunks, then 128 decode steps that
append to the cache, window on and window off (the request is timed both
ways), through libatw; sampled outputs against the fp64 oracle, each row also
within a bound relative to its own magnitude (late rows are ~1e-3)."""

import pytest

import oracle
import rope_frequency_pair_amd as atw
from rope_frequency_pair_amd import request, synth
from tests.gpu_util import check_rows, say, sync, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("window_on", [True, False])
def test_request_1m_sampled(window_on):
    w = synth.WORKLOADS["qwen2.5-7b-1m-request-1m"]
    G = w.h_q // w.h_kv
    heads = [0, w.h_q - 1]                  # kv heads 0 and 3
    kvs = sorted({h // G for h in heads})
    hmap = [kvs.index(h // G) for h in heads]
    say(f"request 1m window_on={window_on}: generating inputs")
    q, q_dec, k, v = synth.request_inputs(w)
    bufs = request.RequestBuffers(w)
    # rows checked per chunk (offsets within the chunk)
    check = {0: [0, 1, 4097], w.n // w.chunk - 1: [0, 31337, w.chunk - 1]}
    got_rows = {}

    def keep(c, out):
        if c in check:
            got_rows[c] = to_np(out[:, heads][:, :, check[c]])
            say(f"request 1m: chunk {c} done")

    say(f"request 1m: running (window_on={window_on})")
    _, dec = request.run_request(w, q, q_dec, k, v, bufs, window_on=window_on, on_chunk=keep)
    sync()
    steps = [0, w.decode_steps - 1]
    got_dec = to_np(dec[steps][:, :, heads])
    kn, vn = to_np(k[:, kvs]), to_np(v[:, kvs])
    for c, offs in check.items():
        for i, off in enumerate(offs):
            pos = c * w.chunk + off
            say(f"request 1m: oracle prefill row {pos}")
            qn = to_np(q[:, heads][:, :, pos:pos + 1])
            ref = oracle.prefill(qn, kn[:, :, :pos + 1], vn[:, :, :pos + 1], pos, w.rope_base, w.k_turns,
                                 window_on=window_on, kv_head_of_q=hmap)[:, :, 0]
            check_rows(got_rows[c][:, :, i], ref, f"row {pos}")
    for j, s in enumerate(steps):
        pos = w.n + s
        say(f"request 1m: oracle decode step {s} (position {pos})")
        qn = to_np(q_dec[s][:, heads])
        ref = oracle.decode(qn, kn[:, :, :pos + 1], vn[:, :, :pos + 1], [pos + 1], [pos], w.rope_base,
                            w.k_turns, window_on=window_on, kv_head_of_q=hmap)
        check_rows(got_dec[j], ref, f"decode step {s}")


def test_one_shot_prefill_1m_sampled():
    """The 1M prompt of the same workload in one prefill call: the query and
    output tensors hold 28 x 2^20 x 128 = 3.8e9 elements, past 2^31, so the
    element offsets of the last rows need 64 bits.  Sampled rows of the first
    and last query heads against the fp64 oracle."""
    w = synth.WORKLOADS["qwen2.5-7b-1m-request-1m"]
    G = w.h_q // w.h_kv
    heads = [0, w.h_q - 1]
    kvs = sorted({h // G for h in heads})
    hmap = [kvs.index(h // G) for h in heads]
    say("one-shot 1m: generating inputs")
    q, _, k, v = synth.request_inputs(w)
    kp, vp = k[:, :, :w.n], v[:, :, :w.n]
    assert q.numel() > 2 ** 31
    say("one-shot 1m: prefill")
    out = atw.prefill(q, kp, vp, rope_base=w.rope_base, k_turns=w.k_turns, q_pos0=0)
    sync()
    rows = [0, 1, 65535, 65536, 524289, w.n - 1]
    got = to_np(out[:, heads][:, :, rows])
    del out
    kn, vn = to_np(kp[:, kvs]), to_np(vp[:, kvs])
    for i, pos in enumerate(rows):
        say(f"one-shot 1m: oracle row {pos}")
        qn = to_np(q[:, heads][:, :, pos:pos + 1])
        ref = oracle.prefill(qn, kn[:, :, :pos + 1], vn[:, :, :pos + 1], pos, w.rope_base, w.k_turns,
                             kv_head_of_q=hmap)[:, :, 0]
        check_rows(got[:, :, i], ref, f"row {pos}")

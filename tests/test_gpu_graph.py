"""HIP graph capture of the library's calls.  The entry points allocate
nothing, clear nothing with memset and never synchronize, so a prefill call
and a whole decode step (banding the appended key, split pass, combine) can
be captured on the current stream and replayed.  Every replay, with new query
values written eagerly between replays, must equal the eager call bit for bit.
"""

import pytest
import torch

import rope_frequency_pair_amd as atw
from rope_frequency_pair_amd import synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def test_prefill_graph_replays_match_eager():
    say("graph: prefill capture and replays")
    q, k, v = synth.prefill_inputs(1, 6, 2, 700, 700, 128, torch.bfloat16, 71, device="cuda")
    ws = torch.empty(atw.prefill_workspace_bytes(atw.ATW_BF16, 1, 2, 700, 128), dtype=torch.uint8,
                     device="cuda")
    out_g = torch.empty_like(q)
    out_e = torch.empty_like(q)
    kw = dict(rope_base=1e4, k_turns=0.5)
    atw.prefill(q, k, v, out=out_g, workspace=ws, **kw)          # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        atw.prefill(q, k, v, out=out_g, workspace=ws, **kw)
    torch.cuda.synchronize()
    for rep in range(3):
        q.copy_(synth.prefill_inputs(1, 6, 2, 700, 700, 128, torch.bfloat16, 72 + rep, device="cuda")[0])
        torch.cuda.synchronize()
        atw.prefill(q, k, v, out=out_e, **kw)                   # eager, own workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}"


def test_decode_step_graph_replays_match_eager():
    say("graph: decode step (band + split + combine) capture and replays")
    B, hq, hkv, L, d, splits = 2, 8, 2, 3000, 128, 16
    q, kc, vc = synth.decode_inputs(B, hq, hkv, L, d, torch.bfloat16, 73, device="cuda")
    kb = atw.kcache_band(kc, n_tokens=L - 1)                    # prompt banded; the step bands key L-1
    ws = torch.empty(atw.decode_workspace_bytes(B, hq, d, splits), dtype=torch.uint8, device="cuda")
    out_g = torch.empty((B, hq, d), dtype=torch.bfloat16, device="cuda")
    out_e = torch.empty_like(out_g)
    kw = dict(rope_base=1e7, k_turns=0.2, num_splits=splits)

    def step(out, workspace):
        atw.kcache_band(kc, kb, t0=L - 1, n_tokens=1)
        atw.decode_banded(q, kb, vc, [L] * B, [L - 1] * B, out=out, workspace=workspace, **kw)

    step(out_g, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out_g, ws)
    torch.cuda.synchronize()
    ws_e = torch.empty_like(ws)
    for rep in range(3):
        q.copy_(synth.decode_inputs(B, hq, hkv, 8, d, torch.bfloat16, 74 + rep, device="cuda")[0])
        kc[:, :, L - 1].normal_()                                # a new appended key each time
        torch.cuda.synchronize()
        step(out_e, ws_e)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}"

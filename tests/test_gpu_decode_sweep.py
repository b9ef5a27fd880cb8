"""Randomized GPU parity sweep of the decode entry points against the fp64
oracle: for each seed a random shape (head_dim 64 or 128, GQA ratio, batch,
ragged lengths from 1 to 3000 keys, query positions at or past the cache
end), window (k from 0.01 to 10 turns: from every pair pruned for most keys to
nothing pruned; window on or off), rope base, row or banded cache, split
count (1 to 17), draft-token count (1 to 4), and for single tokens sometimes a
random 64-key block selection (block-sparse decode).  The cases are drawn from a
seeded generator, so a failure names its seed and shape and reruns alike."""

import numpy as np
import pytest
import torch

import oracle
import rope_frequency_pair_amd as atw
from rope_frequency_pair_amd import synth
from tests.gpu_util import check_rows, say, sync, to_np

pytestmark = pytest.mark.gpu


def _case(seed):
    r = np.random.default_rng(seed)
    d = int(r.choice([64, 128]))
    h_kv = int(r.integers(1, 3))
    g = int(r.choice([1, 2, 4, 7, 16]))
    T = 1 if r.random() < 0.5 else int(r.integers(2, 5))
    while g * T > 16:
        T -= 1
    B = int(r.integers(1, 4))
    L = int(r.integers(1, 3001))
    kv_len = [int(x) for x in r.integers(1, L + 1, size=B)]
    kv_len[0] = L
    q_pos = [n - 1 + int(r.integers(0, 3)) for n in kv_len]      # at or past the cache end
    k_turns = float(np.exp(r.uniform(np.log(0.01), np.log(10.0))))
    base = float(r.choice([1e4, 5e5, 1e7]))
    return dict(d=d, h_kv=h_kv, h_q=g * h_kv, T=T, B=B, L=L, kv_len=kv_len, q_pos=q_pos,
                k_turns=k_turns, base=base, banded=bool(r.integers(0, 2)),
                window_on=bool(r.random() < 0.85), splits=int(r.integers(1, 18)),
                sparse=T == 1 and bool(r.random() < 0.5), density=float(r.choice([0.05, 0.3, 0.8])))


@pytest.mark.parametrize("seed", range(64))
def test_decode_random_sweep(seed):
    c = _case(2000 + seed)
    say(f"decode sweep seed {2000 + seed}: {c}")
    gen = synth.generator(3000 + seed)
    q = torch.randn((c["B"], c["T"], c["h_q"], c["d"]), generator=gen).to(torch.bfloat16).cuda()
    kc = torch.randn((c["B"], c["h_kv"], c["L"], c["d"]), generator=gen).to(torch.bfloat16).cuda()
    vc = torch.randn((c["B"], c["h_kv"], c["L"], c["d"]), generator=gen).to(torch.bfloat16).cuda()
    kk = atw.kcache_band(kc) if c["banded"] else kc
    kw = dict(rope_base=c["base"], k_turns=c["k_turns"], window_on=c["window_on"], num_splits=c["splits"])
    d = c["d"]
    if c["sparse"]:
        q1 = q[:, 0].contiguous()
        n_kb = -(-c["L"] // 64)
        sel = torch.from_numpy(np.random.default_rng(4000 + seed).random((c["B"], c["h_kv"], n_kb)) < c["density"])
        for b, n in enumerate(c["kv_len"]):
            sel[b, :, -(-n // 64):] = False          # blocks past a sequence's cache
        mask = atw.pack_block_mask(sel).cuda()
        out = atw.decode_sparse(q1, kk, vc, c["kv_len"], c["q_pos"], mask, k_banded=c["banded"], **kw)
        sync()
        ref = oracle.decode(to_np(q1), to_np(kc), to_np(vc), c["kv_len"], c["q_pos"], c["base"], c["k_turns"],
                            window_on=c["window_on"], key_blocks=sel.numpy())
        # a (sequence, kv head) with no selected block attends no key: its query heads give exactly 0
        empty = ~np.repeat(sel.any(dim=-1).numpy(), c["h_q"] // c["h_kv"], axis=1)
        if empty.any():
            assert (to_np(out)[empty] == 0).all(), f"seed {2000 + seed}: head attending no key is not 0"
            if empty.all():
                return
            check_rows(to_np(out)[~empty].reshape(-1, d), ref[~empty].reshape(-1, d), f"seed {2000 + seed}")
            return
    elif c["T"] == 1:
        q1 = q[:, 0].contiguous()
        fn = atw.decode_banded if c["banded"] else atw.decode
        out = fn(q1, kk, vc, c["kv_len"], c["q_pos"], **kw)
        sync()
        ref = oracle.decode(to_np(q1), to_np(kc), to_np(vc), c["kv_len"], c["q_pos"], c["base"], c["k_turns"],
                            window_on=c["window_on"])
    else:
        # draft tokens sit at q_pos .. q_pos + T - 1 and see the cache up to their own position
        q_pos = [max(p - c["T"] + 1, n - 1) for p, n in zip(c["q_pos"], c["kv_len"])]
        out = atw.decode_multi(q, kk, vc, c["kv_len"], q_pos, k_banded=c["banded"], **kw)
        sync()
        ref = oracle.decode_multi(to_np(q), to_np(kc), to_np(vc), c["kv_len"], q_pos, c["base"], c["k_turns"],
                                  window_on=c["window_on"])
    got = to_np(out).reshape(-1, d)
    assert np.isfinite(got).all()
    check_rows(got, ref.reshape(-1, d), f"seed {2000 + seed}")

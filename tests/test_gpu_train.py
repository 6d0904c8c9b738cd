"""GPU parity of training through a streaming rollout (block_sparse_attention_20_amd.train:
pbsa_block_gather, pbsa_attn_bwd and pbsa_grad_scatter through the C ABI)
against the fp64 oracle's rollout gradients, with the GPU's own routing and
pool decisions (teacher forcing).  Bar as for the single-chunk backward:
max-abs <= 2e-2 and max-abs / max|oracle| <= 2e-2 (bf16; the backward is
bf16 only)."""
import math
import sys

import numpy as np
import pytest
import torch

import pbsa_synth as syn
from oracle import rollout as orl

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_sparse_attention_20_amd import pbsa as P
    from block_sparse_attention_20_amd.train import TrainRollout


def _log(m):
    print(m, flush=True)
    sys.stdout.flush()


def _close(got, ref, what, bar):
    got = got.float().cpu().numpy() if hasattr(got, "cpu") else got
    err = np.abs(got - ref).max()
    scale = max(np.abs(ref).max(), 1e-30)
    _log(f"{what}: max-abs {err:.3e} normalised {err / scale:.3e}")
    assert not np.isnan(got).any(), what
    assert err <= bar and err / scale <= bar, (what, err, err / scale)


CASES = {
    # 6 chunks of 150 tokens (3 blocks of 64, the last ragged), window of 2
    # chunks, pool of 4 with one sink: pool blocks of several ages
    "bf16_d64_T64": (dict(n=6, B=1, H=2, d=64, T=64, Nq=150, C=4, topk=2, n_sink=1,
                          dtype=torch.bfloat16), 2e-2),
    "bf16_d128_T128_b2": (dict(n=5, B=2, H=1, d=128, T=128, Nq=300, C=3, topk=2, n_sink=0,
                               dtype=torch.bfloat16), 2e-2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_rollout_training_grads_match_oracle(name):
    c, bar = CASES[name]
    _log(f"rollout training case {name}")
    n = c["n"]
    shape = syn.Shape(B=c["B"], H=c["H"], d=c["d"], T=c["T"], Nq=c["Nq"], W=0, C=c["C"],
                      topk=c["topk"], dtype=c["dtype"])
    tr = TrainRollout(n, shape.B, shape.H, shape.d, shape.T, shape.Nq, shape.C, shape.topk,
                      n_sink=c["n_sink"], dtype=shape.dtype, device="cuda")
    sigma = 1.0
    qs, ks, vs, ds = [], [], [], []
    for t in range(n):
        u = syn.rollout_direction(9, 0, t, shape.d)
        ch = syn.make_chunk(shape, syn.rollout_seed(9, 0, t), u, sigma=sigma, shift=1.0, n_planted=1)
        dout = syn.make_dout(shape, 7000 + t)
        tr.forward(ch["q"].cuda(), ch["k"].cuda(), ch["v"].cuda())
        qs.append(ch["q"]); ks.append(ch["k"]); vs.append(ch["v"]); ds.append(dout)
    dq, gk, gv = tr.backward([x.cuda() for x in ds])
    torch.cuda.synchronize()
    assert tr.L.status_bits() == 0 and tr.D.status_bits() == 0
    plans = tr.plans()
    # the pool really carries blocks of older chunks into later attention
    assert any(len(plans[t][0][0][0]) > 0 for t in range(3, n))
    scale = 1 / math.sqrt(shape.d)
    ref = orl.rollout_attention_grads([x.float().numpy() for x in qs], [x.float().numpy() for x in ks],
                                      [x.float().numpy() for x in vs], plans, [x.float().numpy() for x in ds],
                                      scale, shape.T)
    for t in range(n):
        _close(tr.rec[t]["o"], ref["o"][t], f"{name} o[{t}]", bar)
        _close(dq[t], ref["dq"][t], f"{name} dq[{t}]", bar)
        _close(gk[t], ref["dk"][t], f"{name} dk[{t}]", bar)
        _close(gv[t], ref["dv"][t], f"{name} dv[{t}]", bar)


def test_gather_rebuilds_the_rollout_pool_bitwise():
    """The pool a chunk attended, rebuilt from the history by
    pbsa_block_gather, equals the rollout's own pool bytes at that point."""
    shape = syn.Shape(B=1, H=2, d=64, T=64, Nq=150, W=0, C=4, topk=2)
    n = 6
    tr = TrainRollout(n, 1, 2, 64, 64, 150, 4, 2, device="cuda")
    for t in range(n):
        u = syn.rollout_direction(3, 0, t, 64)
        ch = syn.make_chunk(shape, syn.rollout_seed(3, 0, t), u, sigma=1.0, shift=1.0, n_planted=1)
        tr.forward(ch["q"].cuda(), ch["k"].cuda(), ch["v"].cuda())
    L = tr.L  # pool after the last update
    out_k = torch.full_like(L.t["k_pool"], float("nan")); out_v = torch.full_like(out_k, float("nan"))
    ln = torch.full_like(L.t["pool_len"], -7)
    P.pbsa_block_gather(L.prob, L.t["pool_id"], 4, L.t["pool_count"], 4, tr.k_hist, tr.v_hist, n,
                        out_k, out_v, ln)
    torch.cuda.synchronize()
    cnt = L.t["pool_count"].cpu()
    for h in range(2):
        m = int(cnt[0, h])
        assert m > 0
        for p in range(m):
            n_ok = int(L.t["pool_len"][0, h, p])
            assert int(ln[0, h, p]) == n_ok
            assert torch.equal(out_k[0, h, p, :n_ok], L.t["k_pool"][0, h, p, :n_ok])
            assert torch.equal(out_v[0, h, p, :n_ok], L.t["v_pool"][0, h, p, :n_ok])
            assert (out_k[0, h, p, n_ok:] == 0).all()
        for p in range(m, 4):
            assert int(ln[0, h, p]) == 0 and (out_k[0, h, p] == 0).all()

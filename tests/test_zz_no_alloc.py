"""pbsa_select_static (the allocation-free select) against pbsa_select
through the C ABI: two calls in a row on one device, the second on a smaller
problem, each bit-identical to pbsa_select with its own workspace (the same
kernels, deterministic).  The outputs of the static call are poisoned first,
so every element must be written by it."""
import sys

import pytest
import torch

import pbsa_synth as syn

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_sparse_attention_20_amd import pbsa as P
    from block_sparse_attention_20_amd.layer import PBSALayer

OUTS = ("sel", "sel_count", "mass_pool", "mass_win", "kbar_cur")


def _select_both(shape, st):
    L = PBSALayer(shape.B, shape.H, shape.d, shape.T, shape.Nq, shape.W, shape.C, shape.topk,
                  dtype=shape.dtype, device="cuda").load(st)
    L.select()
    torch.cuda.synchronize()
    ref = {k: L.t[k].clone() for k in OUTS}
    for k in OUTS:
        if L.t[k].is_floating_point():
            L.t[k].fill_(float("nan"))
        else:
            L.t[k].fill_(-7)
    t = L.t
    P.pbsa_select_static(L.prob, t["q"], L.kv, t["sel"] if shape.topk > 0 else None, t["sel_count"],
                         t["mass_pool"] if shape.C > 0 else None, t["mass_win"] if shape.W > 0 else None)
    torch.cuda.synchronize()
    return L, ref


def test_select_static_matches_select_twice():
    big = syn.WAN_CHUNK
    small = syn.Shape(B=1, H=2, d=64, T=64, Nq=5 * 64 - 7, W=10, C=4, topk=3)
    cases = [(big, syn.wan_chunk_state(3)),
             (small, syn.make_state(small, 9, sigma=1.0, shift=1.5, n_planted=3,
                                    win_len=[64] * 4 + [33] + [64] * 4 + [1], pool_count=[4, 2]))]
    for n, (shape, st) in enumerate(cases):
        print(f"static select call {n}: H={shape.H} Nq={shape.Nq} W={shape.W} C={shape.C}", flush=True)
        sys.stdout.flush()
        L, ref = _select_both(shape, st)
        for k in OUTS:
            assert torch.equal(L.t[k], ref[k]), (n, k)
        assert L.status_bits() == 0

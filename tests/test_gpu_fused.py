"""pbsa_select_attn_fwd (routing + attention in one call) against
pbsa_select (no masses) followed by pbsa_attn_fwd, through the C ABI: the
same selection, key means, workspace scores, outputs and LSE, bit for bit.
Problems with d = T = 128 in bf16, C + topk <= 128 and no split of the
forward take the one-launch kernel; the rest take the two launches.  The
two-call results themselves are checked against the oracle elsewhere."""
import sys

import pytest
import torch

import pbsa_synth as syn

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_sparse_attention_20_amd.layer import PBSALayer
    from block_sparse_attention_20_amd import pbsa as P

from test_gpu_parity import CASES

OUT_KEYS = ("sel", "sel_count", "kbar_cur", "o", "lse")


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _two_calls_then_fused(shape, st, ws_fwd):
    """Outputs and select workspace of select + fwd, then of select_fwd on the
    same layer with every output poisoned first."""
    L = PBSALayer(shape.B, shape.H, shape.d, shape.T, shape.Nq, shape.W, shape.C, shape.topk,
                  dtype=shape.dtype, device="cuda", ws_fwd=ws_fwd).load(st)
    L.ws_select.fill_(0xAB)  # parts no call writes (the current-chunk scores) stay equal
    L.select(masses=False)
    L.fwd()
    torch.cuda.synchronize()
    ref = {k: L.t[k].clone() for k in OUT_KEYS}
    ref_ws = L.ws_select.clone()
    L.t["o"].fill_(float("nan"))
    L.t["lse"].fill_(float("nan"))
    L.t["kbar_cur"].fill_(float("nan"))
    L.t["sel_count"].fill_(-7)
    if shape.topk > 0:
        L.t["sel"].fill_(-7)
    L.ws_select.fill_(0xAB)
    L.select_fwd()
    torch.cuda.synchronize()
    return L, ref, ref_ws


def _assert_same(L, ref, ref_ws, what):
    for k in OUT_KEYS:
        assert torch.equal(L.t[k], ref[k]), (what, k)
    assert torch.equal(L.ws_select, ref_ws), (what, "select workspace")
    assert L.status_bits() == 0, what


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("with_fwd_ws", [False, True])
def test_select_attn_fwd_equals_two_calls(name, with_fwd_ws):
    shape, kw = CASES[name]
    _log(f"case {name} fwd_ws={with_fwd_ws}")
    st = syn.make_state(shape, 31, pad_value=float("nan"), **kw)
    L, ref, ref_ws = _two_calls_then_fused(shape, st, "own" if with_fwd_ws else None)
    _assert_same(L, ref, ref_ws, name)
    # the masses pbsa_block_mass forms from the fused call's workspace
    if shape.C + shape.W > 0:
        L.block_mass()
        torch.cuda.synchronize()
        m = {k: L.t[k].clone() for k in ("mass_pool", "mass_win")}
        L.select(masses=True)
        torch.cuda.synchronize()
        for k in ("mass_pool", "mass_win"):
            assert torch.equal(L.t[k], m[k]), (name, k)


@pytest.mark.parametrize("unscaled", [False, True])
def test_select_attn_fwd_wan_chunk(unscaled):
    """The Wan chunk (12 heads x 37 query blocks: one launch, no split) in
    the layer configuration the rollout uses, with and without a forward
    workspace (too many query blocks to split either way)."""
    shape = syn.WAN_CHUNK
    for ws_fwd in (None, "own"):
        _log(f"wan chunk unscaled={unscaled} fwd_ws={ws_fwd}")
        st = syn.wan_chunk_state(1, unscaled=unscaled)
        L, ref, ref_ws = _two_calls_then_fused(shape, st, ws_fwd)
        _assert_same(L, ref, ref_ws, f"wan chunk {ws_fwd}")


@pytest.mark.parametrize("W,C,topk", [(900, 4, 8), (200, 100, 40)])
def test_select_attn_fwd_past_the_one_launch_limits(W, C, topk):
    """A window past the routing scratch (W > 819) and a list past the 128
    entries held in LDS (C + topk > 128) take the two launches inside the
    call: still the same results as the separate calls."""
    shape = syn.Shape(B=1, H=2, d=128, T=128, Nq=2 * 128 + 17, W=W, C=C, topk=topk)
    _log(f"limits W={W} C={C} topk={topk}")
    st = syn.make_state(shape, 13, pad_value=float("nan"), sigma=1.0, shift=1.0, n_planted=3,
                        pool_count=[C, C // 2])
    L, ref, ref_ws = _two_calls_then_fused(shape, st, None)
    _assert_same(L, ref, ref_ws, f"W={W} C={C} topk={topk}")


def test_select_attn_fwd_bad_pool_count_is_flagged():
    """A pool_count above C is clamped and flagged by the fused call as by
    the separate ones, with the same outputs."""
    shape, kw = CASES["bf16_d128_T128_small"]
    st = syn.make_state(shape, 5, **kw)
    outs = []
    for fused in (False, True):
        L = PBSALayer(shape.B, shape.H, shape.d, shape.T, shape.Nq, shape.W, shape.C, shape.topk,
                      device="cuda", ws_fwd=None).load(st)
        L.t["pool_count"].fill_(99)
        if fused:
            L.select_fwd()
        else:
            L.select(masses=False)
            L.fwd()
        torch.cuda.synchronize()
        assert L.status_bits() & P.PBSA_STATUS_POOL_COUNT
        outs.append({k: L.t[k].clone() for k in OUT_KEYS})
    for k in OUT_KEYS:
        assert torch.equal(outs[0][k], outs[1][k]), k


def test_select_attn_fwd_requires_select_workspace():
    shape, kw = CASES["bf16_d128_T128_small"]
    st = syn.make_state(shape, 5, **kw)
    L = PBSALayer(shape.B, shape.H, shape.d, shape.T, shape.Nq, shape.W, shape.C, shape.topk,
                  device="cuda", ws_fwd=None).load(st)
    t = L.t
    with pytest.raises(P.PBSAError) as e:
        P.pbsa_select_attn_fwd(L.prob, t["q"], L.kv, t["sel"], t["sel_count"], t["o"], t["lse"], None)
    assert e.value.code == P.PBSA_ERR_WORKSPACE


def test_select_attn_fwd_and_static_select_replay_in_a_graph():
    """The calls make no allocation and no memset, so a caller can capture
    them: the one-launch routing + forward, and the allocation-free select
    followed by the forward, captured in a HIP graph and replayed three
    times (other work and synchronisation between replays) give the eager
    results bit for bit every time."""
    shape = syn.WAN_CHUNK
    st = syn.wan_chunk_state(2)
    L = PBSALayer(shape.B, shape.H, shape.d, shape.T, shape.Nq, shape.W, shape.C, shape.topk,
                  device="cuda", ws_fwd=None).load(st)
    t = L.t

    def fused():
        L.select_fwd()

    def static_then_fwd():
        P.pbsa_select_static(L.prob, t["q"], L.kv, t["sel"], t["sel_count"], None, None)
        L.fwd()

    for name, fn in (("fused", fused), ("static select + fwd", static_then_fwd)):
        _log(f"graph replay: {name}")
        fn()
        torch.cuda.synchronize()
        ref = {k: t[k].clone() for k in OUT_KEYS}
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            fn()  # warm-up on the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for r in range(3):
            for k in ("o", "lse"):
                t[k].fill_(float("nan"))
            t["sel"].fill_(-7)
            t["sel_count"].fill_(-7)
            g.replay()
            torch.cuda.synchronize()
            for k in OUT_KEYS:
                assert torch.equal(t[k], ref[k]), (name, r, k)
            fn()  # eager work between replays
            torch.cuda.synchronize()
        del g
    assert L.status_bits() == 0

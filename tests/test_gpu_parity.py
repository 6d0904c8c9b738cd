"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Bars (from the method's target numerics: bf16 inputs, fp32 accumulation):
  - selected window blocks: identical sets, except inside the tie band where
    the k-th and (k+1)-th coarse logits differ by <= 1e-4 relative (there
    any choice within the band is accepted and checked for validity);
  - block masses: fp32 vs fp64, rtol 1e-4;
  - attention outputs: max-abs <= 2e-2 AND max-abs / max|O_oracle| <= 2e-2
    on the bf16 path; <= 1e-4 max-abs on the fp32 path;
  - LSE: max-abs <= 2e-3 (bf16), 1e-5 (fp32);
  - memory update: pool membership, slot placement and copied bytes exact
    (teacher-forced on the GPU's own masses, so routing noise cannot cascade).
Attention and update are checked on the GPU's own selection (teacher forcing).
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import pbsa_synth as syn
from oracle import pbsa_oracle as po

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from block_sparse_attention_20_amd.layer import PBSALayer
    from block_sparse_attention_20_amd import pbsa as P

TIE_REL = 1e-4


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(shape, st, scale=0.0, device="cuda"):
    L = PBSALayer(shape.B, shape.H, shape.d, shape.T, shape.Nq, shape.W, shape.C, shape.topk,
                  dtype=shape.dtype, scale=scale, device=device).load(st)
    L.select()
    L.fwd()
    torch.cuda.synchronize()
    return L


def eff_scale(shape, scale):
    return scale if scale > 0 else 1.0 / math.sqrt(shape.d)


def check_selection(L, r, st, k):
    gsel = L.t["sel"].cpu().numpy()[..., :max(k, 1)]
    gcnt = L.t["sel_count"].cpu().numpy()
    np.testing.assert_array_equal(gcnt, r["sel_count"])
    win_id = np.asarray(st["win_id"])
    n_tie = 0
    for idx in np.ndindex(*gcnt.shape):
        g = [int(w) for w in gsel[idx][:gcnt[idx]]]
        o = [int(w) for w in r["sel"][idx][:r["sel_count"][idx]]]
        assert g == sorted(g), "selection must be in ascending slot order"
        assert all(w == -1 for w in gsel[idx][gcnt[idx]:k]), "padding must be -1"
        if g == o:
            continue
        # tie band: every slot in the symmetric difference scores within 1e-4
        # relative of the oracle's k-th score
        s = r["s_win"][idx]
        valid = [w for w in range(len(s)) if not np.isnan(s[w])]
        order = sorted(valid, key=lambda w: po.rank_key_desc(s[w], int(win_id[w])))
        kth = s[order[k - 1]]
        for w in set(g) ^ set(o):
            assert abs(s[w] - kth) <= TIE_REL * max(abs(s[w]), abs(kth)), (idx, w, s[w], kth)
        n_tie += 1
    return n_tie


def check_close_bf16(got, ref, what):
    ref = np.asarray(ref)
    m = ~np.isnan(ref)
    err = np.abs(got[m] - ref[m]).max()
    scale = np.abs(ref[m]).max()
    _log(f"{what}: max-abs {err:.3e}, normalised {err / scale:.3e}")
    assert err <= 2e-2, (what, err)
    assert err / scale <= 2e-2, (what, err / scale)
    return err


# ------------------------------------------------------------------- cases ---
CASES = {
    # ragged tail query block, empty + ragged window slots, pools of 3 and 1
    "bf16_d128_T128_small": (syn.Shape(B=1, H=2, d=128, T=128, Nq=3 * 128 - 40, W=6, C=3, topk=2),
                             dict(sigma=1.0, shift=1.0, n_planted=2, win_len=[128, 128, 88, 128, 0, 128],
                                  pool_count=[3, 1], pool_len=[128, 60, 128, 128, 128, 128])),
    # several tiles, d=64/T=64, batch 2, unscaled N(0,1)
    "bf16_d64_T64_multi": (syn.Shape(B=2, H=2, d=64, T=64, Nq=5 * 64 - 7, W=10, C=4, topk=3),
                           dict(sigma=1.0, shift=1.5, n_planted=3, win_len=[64] * 4 + [33] + [64] * 4 + [1],
                                pool_count=[4, 2, 0, 3])),
    "bf16_d64_T128": (syn.Shape(B=1, H=2, d=64, T=128, Nq=2 * 128 + 5, W=4, C=2, topk=2),
                      dict(sigma=1.0, n_planted=0, win_len=[128, 5, 128, 128], pool_count=[2, 1])),
    "bf16_d128_T64": (syn.Shape(B=1, H=1, d=128, T=64, Nq=4 * 64, W=8, C=4, topk=8),
                      dict(sigma=1.0, n_planted=2, shift=1.0, pool_count=4)),
    "f32_d64_T64": (syn.Shape(B=1, H=2, d=64, T=64, Nq=3 * 64 - 9, W=5, C=2, topk=2, dtype=torch.float32),
                    dict(sigma=1.0, n_planted=1, shift=1.0, win_len=[64, 64, 20, 64, 64], pool_count=[2, 1])),
    "f32_d128_T128": (syn.Shape(B=1, H=1, d=128, T=128, Nq=200, W=3, C=2, topk=1, dtype=torch.float32),
                      dict(sigma=1.0, pool_count=2)),
    # degenerate: no pool, no window blocks valid, single ragged query block
    "empty_pool_and_window": (syn.Shape(B=1, H=2, d=128, T=128, Nq=77, W=3, C=2, topk=2),
                              dict(sigma=1.0, win_len=[0, 0, 0], pool_count=0)),
    # k >= valid window slots: everything selected
    "topk_covers_window": (syn.Shape(B=1, H=1, d=128, T=128, Nq=256, W=4, C=1, topk=4),
                           dict(sigma=1.0, win_len=[128, 0, 128, 64], pool_count=1)),
    # W = 0, C = 0: the current chunk only
    "current_only": (syn.Shape(B=1, H=3, d=64, T=64, Nq=130, W=0, C=0, topk=0),
                     dict(sigma=1.0, win_len=[], pool_count=0)),
    # a one-entry block list (no pool, no window, one ragged query block):
    # the forward is never split, workspace or not
    "one_entry_list": (syn.Shape(B=1, H=2, d=128, T=128, Nq=100, W=0, C=0, topk=0),
                       dict(sigma=1.0, win_len=[], pool_count=0)),
    # a block list longer than the 128 entries staged in LDS (pool 12 + 140
    # selected + 3 current): the entries past it are resolved on the fly
    "long_list": (syn.Shape(B=1, H=2, d=128, T=64, Nq=3 * 64 - 5, W=150, C=12, topk=140),
                  dict(sigma=1.0, shift=1.0, n_planted=4,
                       win_len=[64] * 40 + [0, 30] + [64] * 100 + [17] + [64] * 7,
                       pool_count=[12, 7])),
    # the same at the benchmark's tile shape (d128, blocks of 128): pool 8 +
    # 130 selected + 2 current = 140 entries, past the 128 staged in LDS
    "long_list_d128_T128": (syn.Shape(B=1, H=1, d=128, T=128, Nq=2 * 128 - 30, W=140, C=8, topk=130),
                            dict(sigma=1.0, shift=1.0, n_planted=4,
                                 win_len=[128] * 60 + [0, 72] + [128] * 77 + [5], pool_count=8)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_select_and_fwd_match_oracle(name):
    shape, kw = CASES[name]
    _log(f"case {name}")
    st = syn.make_state(shape, 11, pad_value=float("nan"), **kw)
    L = run(shape, st)
    scale = eff_scale(shape, 0.0)
    r = po.select(st, shape.topk, scale, shape.T)
    if shape.topk > 0:
        check_selection(L, r, st, shape.topk)
    else:
        assert (L.t["sel_count"] == 0).all()
    # masses (fp32 vs fp64)
    if shape.C > 0:
        np.testing.assert_allclose(L.t["mass_pool"].cpu().numpy(), r["mass_pool"], rtol=1e-4, atol=1e-6)
    if shape.W > 0:
        np.testing.assert_allclose(L.t["mass_win"].cpu().numpy(), r["mass_win"], rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(L.t["kbar_cur"].cpu().numpy(), r["kbar_cur"], rtol=1e-5, atol=1e-5)
    # attention on the GPU's own selection
    gsel = L.t["sel"].cpu().numpy(); gcnt = L.t["sel_count"].cpu().numpy()
    f = po.attn_fwd(st, gsel, gcnt, scale, shape.T)
    o = L.t["o"].float().cpu().numpy()
    lse = L.t["lse"].cpu().numpy()
    if shape.dtype == torch.float32:
        assert np.abs(o - f["o"]).max() <= 1e-4
        assert np.abs(lse - f["lse"]).max() <= 1e-5
    else:
        check_close_bf16(o, f["o"], name)
        assert np.abs(lse - f["lse"]).max() <= 2e-3
    assert not np.isnan(o).any(), "padding rows leaked NaN into the output"
    assert L.status_bits() == 0


@pytest.mark.parametrize("name", ["bf16_d128_T128_small", "bf16_d64_T64_multi", "bf16_d64_T128",
                                  "bf16_d128_T64", "f32_d64_T64", "f32_d128_T128",
                                  "empty_pool_and_window", "topk_covers_window", "long_list",
                                  "long_list_d128_T128"])
def test_fine_mass_matches_oracle(name):
    """Exact block masses from the forward's lse against the fp64 oracle on
    the GPU's own selection.  Bar: 5e-3 of the largest mass (bf16 rounding is
    shared, so the residue is the fp32 accumulation and the forward's lse
    error, <= 2e-3 in these cases), 5e-5 for fp32; blocks no row attends are
    exact zeros."""
    shape, kw = CASES[name]
    _log(f"fine mass case {name}")
    st = syn.make_state(shape, 13, pad_value=float("nan"), **kw)
    L = run(shape, st)
    # poison the mass buffers: every element must be written
    L.t["mass_pool"].fill_(float("nan")); L.t["mass_win"].fill_(float("nan"))
    L.fine_mass()
    torch.cuda.synchronize()
    scale = eff_scale(shape, 0.0)
    gsel = L.t["sel"].cpu().numpy(); gcnt = L.t["sel_count"].cpu().numpy()
    ref = po.fine_mass(st, gsel, gcnt, scale, shape.T)
    rtol = 5e-5 if shape.dtype == torch.float32 else 5e-3
    for n, C in (("mass_pool", shape.C), ("mass_win", shape.W)):
        if C == 0:
            continue
        got = L.t[n].cpu().numpy()[..., :C]
        r = ref[n]
        assert not np.isnan(got).any(), f"{name}: {n} not fully written"
        bar = rtol * max(np.abs(r).max(), 1e-30) + 1e-7
        err = np.abs(got - r).max()
        _log(f"{name} {n}: max-abs {err:.3e} (bar {bar:.3e})")
        assert err <= bar, (name, n, err, bar)
        assert (got[r == 0] == 0).all(), f"{name}: {n} nonzero where no row attends"
    assert L.status_bits() == 0


@pytest.mark.parametrize("name", ["bf16_d128_T128_small", "bf16_d64_T64_multi", "bf16_d64_T128",
                                  "bf16_d128_T64", "f32_d64_T64", "f32_d128_T128",
                                  "empty_pool_and_window", "topk_covers_window", "long_list",
                                  "long_list_d128_T128", "current_only"])
def test_fwd_mass_matches_oracle(name):
    """The fused forward + exact block mass (pbsa_attn_fwd_mass): O and LSE
    as the plain forward (oracle bars), masses against the oracle's exact
    mass on the GPU's own selection (5e-3 of the largest mass for bf16, 5e-5
    for fp32, blocks no row attends exactly 0) and against the separate
    exact-mass pass (pbsa_fine_mass) to 1e-4 of the largest mass."""
    shape, kw = CASES[name]
    _log(f"fused fwd + mass case {name}")
    st = syn.make_state(shape, 13, pad_value=float("nan"), **kw)
    L = run(shape, st)
    L.fine_mass()
    torch.cuda.synchronize()
    sep = {n: L.t[n].clone() for n in ("mass_pool", "mass_win")}
    for n in ("mass_pool", "mass_win", "o", "lse"):
        L.t[n].fill_(float("nan"))
    L.fwd_mass()
    torch.cuda.synchronize()
    scale = eff_scale(shape, 0.0)
    gsel = L.t["sel"].cpu().numpy(); gcnt = L.t["sel_count"].cpu().numpy()
    f = po.attn_fwd(st, gsel, gcnt, scale, shape.T)
    o = L.t["o"].float().cpu().numpy(); lse = L.t["lse"].cpu().numpy()
    if shape.dtype == torch.float32:
        assert np.abs(o - f["o"]).max() <= 1e-4
        assert np.abs(lse - f["lse"]).max() <= 1e-5
    else:
        check_close_bf16(o, f["o"], f"{name} fused")
        assert np.abs(lse - f["lse"]).max() <= 2e-3
    ref = po.fine_mass(st, gsel, gcnt, scale, shape.T)
    rtol = 5e-5 if shape.dtype == torch.float32 else 5e-3
    for n, C in (("mass_pool", shape.C), ("mass_win", shape.W)):
        if C == 0:
            continue
        got = L.t[n].cpu().numpy()[..., :C]
        r = ref[n]
        assert not np.isnan(got).any(), f"{name}: {n} not fully written"
        top = max(np.abs(r).max(), 1e-30)
        err = np.abs(got - r).max()
        _log(f"{name} fused {n}: max-abs {err:.3e} (bar {rtol * top + 1e-7:.3e})")
        assert err <= rtol * top + 1e-7, (name, n, err)
        assert (got[r == 0] == 0).all(), f"{name}: {n} nonzero where no row attends"
        d_sep = np.abs(got - sep[n].cpu().numpy()[..., :C]).max()
        assert d_sep <= 1e-4 * top + 1e-7, (name, n, "vs pbsa_fine_mass", d_sep)
    assert L.status_bits() == 0


@pytest.mark.parametrize("unscaled", [False, True])
def test_fwd_mass_wan_chunk_full_size(unscaled):
    """The fused forward + exact mass at the Wan chunk, full size, in the
    benchmark's launch configuration: O and LSE equal to the plain forward's
    within rounding, two heads' masses against the oracle, every head's
    against the separate exact-mass pass."""
    _log(f"fused fwd + mass, wan chunk unscaled={unscaled}")
    shape = syn.WAN_CHUNK
    st = syn.wan_chunk_state(0, unscaled=unscaled)
    L = run(shape, st)
    o_plain = L.t["o"].float().cpu().numpy(); lse_plain = L.t["lse"].cpu().numpy()
    L.fine_mass()
    torch.cuda.synchronize()
    sep = {n: L.t[n].cpu().numpy() for n in ("mass_pool", "mass_win")}
    for n in ("mass_pool", "mass_win", "o", "lse"):
        L.t[n].fill_(float("nan"))
    L.fwd_mass()
    torch.cuda.synchronize()
    o = L.t["o"].float().cpu().numpy(); lse = L.t["lse"].cpu().numpy()
    assert np.abs(lse - lse_plain).max() <= 1e-5
    assert np.abs(o - o_plain).max() <= 1e-2 * np.abs(o_plain).max()
    mp = L.t["mass_pool"].cpu().numpy(); mw = L.t["mass_win"].cpu().numpy()
    for n, got in (("mass_pool", mp), ("mass_win", mw)):
        top = np.abs(sep[n]).max()
        assert np.abs(got - sep[n]).max() <= 1e-4 * top, n
    gsel = L.t["sel"].cpu().numpy(); gcnt = L.t["sel_count"].cpu().numpy()
    scale = 1 / math.sqrt(128)
    for h in (0, 7):
        ref = po.fine_mass(_one_head(st, h), gsel[:, h:h + 1], gcnt[:, h:h + 1], scale, shape.T)
        for n, got in (("mass_pool", mp[:, h:h + 1]), ("mass_win", mw[:, h:h + 1])):
            r = ref[n]
            err = np.abs(got - r).max()
            bar = 5e-3 * np.abs(r).max() + 1e-7
            _log(f"fused head {h} {n}: max-abs {err:.3e} (bar {bar:.3e})")
            assert err <= bar, (h, n, err, bar)
    assert L.status_bits() == 0


@pytest.mark.parametrize("name", ["bf16_d128_T128_small", "bf16_d64_T64_multi", "bf16_d128_T64",
                                  "bf16_d64_T128", "empty_pool_and_window", "one_entry_list"])
def test_fwd_split_and_one_block_per_workgroup_agree(name):
    """The forward with a split workspace (every query block's list cut into
    equal pieces, merged by a second kernel) and without one (one workgroup
    per query block) both match the oracle; on these small problems the
    split runs one list entry per piece.  A one-entry list is not split."""
    shape, kw = CASES[name]
    _log(f"case {name}")
    st = syn.make_state(shape, 23, pad_value=float("nan"), **kw)
    L = run(shape, st)
    assert L.ws_fwd is not None
    o_split = L.t["o"].float().cpu().numpy(); lse_split = L.t["lse"].cpu().numpy()
    L.ws_fwd, ws = None, L.ws_fwd
    L.fwd()
    torch.cuda.synchronize()
    L.ws_fwd = ws
    o_one = L.t["o"].float().cpu().numpy(); lse_one = L.t["lse"].cpu().numpy()
    gsel = L.t["sel"].cpu().numpy(); gcnt = L.t["sel_count"].cpu().numpy()
    f = po.attn_fwd(st, gsel, gcnt, eff_scale(shape, 0.0), shape.T)
    for o, lse, what in ((o_split, lse_split, "split"), (o_one, lse_one, "one per workgroup")):
        check_close_bf16(o, f["o"], f"{name} {what}")
        assert np.abs(lse - f["lse"]).max() <= 2e-3, what
    assert L.status_bits() == 0


@pytest.mark.parametrize("qb", [1, 8])
def test_short_chunk_split_matches_oracle(qb):
    """Short query chunks against the full-size Wan cache (12 heads x 128,
    window 74 slots with two ragged blocks, pool 32, top-16), the sizes
    bench.py --small-chunks times: the split forward with its merge kernel
    agrees with the one-workgroup-per-block launch (LSE within 1e-4, O
    within 1e-2 of max|O|) and with the oracle on every row of three heads."""
    base = syn.WAN_CHUNK
    shape = syn.Shape(B=1, H=base.H, d=base.d, T=base.T, Nq=qb * base.T, W=base.W, C=base.C,
                      topk=base.topk)
    _log(f"short chunk, {qb} query blocks")
    st = syn.make_state(shape, 6000 + qb, sigma=1 / math.sqrt(shape.d), shift=1.5, n_planted=8,
                        win_len=syn.chunk_window_lens(base.Nq, base.T, 2))
    L = run(shape, st)
    assert L.ws_fwd is not None and L.status_bits() == 0
    o_s = L.t["o"].float().cpu().numpy(); lse_s = L.t["lse"].cpu().numpy()
    L.ws_fwd, ws = None, L.ws_fwd
    L.fwd()
    torch.cuda.synchronize()
    L.ws_fwd = ws
    o_w = L.t["o"].float().cpu().numpy(); lse_w = L.t["lse"].cpu().numpy()
    assert np.abs(lse_s - lse_w).max() <= 1e-4
    assert np.abs(o_s - o_w).max() <= 1e-2 * np.abs(o_w).max()
    gsel = L.t["sel"].cpu().numpy(); gcnt = L.t["sel_count"].cpu().numpy()
    heads = (0, 5, 11)
    blocks = [(0, h, i) for h in heads for i in range(qb)]
    f = po.attn_fwd(st, gsel, gcnt, eff_scale(shape, 0.0), shape.T, blocks=blocks)
    for h in heads:
        check_close_bf16(o_s[0, h], f["o"][0, h], f"short chunk {qb} head {h}")
        assert np.abs(lse_s[0, h] - f["lse"][0, h]).max() <= 2e-3


def test_fwd_split_workspace_needs_no_initialisation():
    """The split forward's workspace may hold anything (here: bytes of an
    earlier use, then random bytes): every piece writes its partial before
    the merge kernel reads it, so the result matches a clean run."""
    shape, kw = CASES["bf16_d64_T64_multi"]
    st = syn.make_state(shape, 31, **kw)
    L = run(shape, st)
    ref_o = L.t["o"].clone(); ref_l = L.t["lse"].clone()
    g = torch.Generator(device="cuda").manual_seed(5)
    for _ in range(2):
        L.ws_fwd.copy_(torch.randint(0, 256, L.ws_fwd.shape, generator=g, device="cuda",
                                     dtype=torch.int32).to(torch.uint8))
        L.fwd()
        torch.cuda.synchronize()
        assert torch.equal(L.t["o"], ref_o) and torch.equal(L.t["lse"], ref_l)


def test_block_mass_later_equals_mass_in_select():
    """pbsa_select without mass buffers followed by pbsa_block_mass gives
    the masses of pbsa_select with them, bit for bit, and the same routing."""
    shape, kw = CASES["bf16_d128_T128_small"]
    st = syn.make_state(shape, 41, **kw)
    L = run(shape, st)
    ref = {k: L.t[k].clone() for k in ("mass_pool", "mass_win", "sel", "sel_count")}
    for k in ("mass_pool", "mass_win"):
        L.t[k].fill_(float("nan"))
    L.select(masses=False)
    torch.cuda.synchronize()
    assert torch.isnan(L.t["mass_pool"]).all() and torch.isnan(L.t["mass_win"]).all()
    assert torch.equal(L.t["sel"], ref["sel"]) and torch.equal(L.t["sel_count"], ref["sel_count"])
    L.block_mass()
    torch.cuda.synchronize()
    assert torch.equal(L.t["mass_pool"], ref["mass_pool"]) and torch.equal(L.t["mass_win"], ref["mass_win"])


def _topk_from_scores(srow_win, valid, ids, k):
    """Window slots of the k best valid scores under the total order (score
    descending, ties by id ascending, NaN after every number), ascending."""
    cand = [w for w in range(len(valid)) if valid[w]]
    cand.sort(key=lambda w: (bool(np.isnan(srow_win[w])),
                             0.0 if np.isnan(srow_win[w]) else -float(srow_win[w]), int(ids[w])))
    return sorted(cand[:min(k, len(cand))])


@pytest.mark.parametrize("k", [2, 5, 7, 36])
def test_topk_exact_on_kernel_scores(k):
    """The selection equals the top-k of the kernel's own fp32 coarse scores
    (read back from the select workspace), bit for bit, with exact ties:
    groups of window slots hold identical keys (so identical scores) and
    their ids are not in slot order, so only the id decides among them; two
    valid slots hold NaN keys and must rank after every number (k = 36 of 37
    valid slots leaves out exactly the NaN slot of the larger id); empty
    slots never count."""
    W, C, T, d = 40, 3, 64, 64
    shape = syn.Shape(B=1, H=2, d=d, T=T, Nq=3 * T - 9, W=W, C=C, topk=k)
    win_len = [T] * W
    for w in (3, 14, 27):
        win_len[w] = 0
    win_len[33] = 20
    rng = np.random.default_rng(5)
    ids = [int(x) for x in 100 + rng.permutation(W)]
    st = syn.make_state(shape, 29, sigma=1.0, shift=1.0, win_len=win_len, win_id=ids, pool_count=[3, 2])
    kw = st["k_win"].float()
    qm = st["q"].float().mean(dim=2)  # [B,H,d]: the queries' common direction
    top, second, nan_slots = (2, 9, 17, 30), (5, 22, 36), (11, 25)
    for w in top:
        kw[:, :, w, :] = 4.0 * qm[:, :, None, :]
    for w in second:
        kw[:, :, w, :] = 2.0 * qm[:, :, None, :]
    for w in nan_slots:
        kw[:, :, w, :] = float("nan")
    st["k_win"] = kw.to(shape.dtype)
    _log(f"top-k exact on kernel scores: k={k}")
    L = PBSALayer(shape.B, shape.H, shape.d, shape.T, shape.Nq, shape.W, shape.C, shape.topk,
                  dtype=shape.dtype, device="cuda").load(st)
    L.select(masses=False)
    torch.cuda.synchronize()
    QB = (shape.Nq + T - 1) // T
    bh = shape.B * shape.H
    off = (bh * QB * d * 4 + 255) // 256 * 256
    nj = C + W + QB
    srows = L.ws_select[off:off + bh * QB * nj * 4].view(torch.float32).cpu().numpy().reshape(bh, QB, nj)
    sel = L.t["sel"].cpu().numpy().reshape(bh, QB, k)
    cnt = L.t["sel_count"].cpu().numpy().reshape(bh, QB)
    valid = [x > 0 for x in win_len]
    n_valid = sum(valid)
    for b in range(bh):
        for i in range(QB):
            sw = srows[b, i, C:C + W]
            assert np.isnan(sw[list(nan_slots)]).all()
            assert len(set(float(sw[w]) for w in top)) == 1
            exp = _topk_from_scores(sw, valid, ids, k)
            assert int(cnt[b, i]) == min(k, n_valid)
            got = [int(x) for x in sel[b, i, :cnt[b, i]]]
            assert got == exp, (b, i, got, exp)
            assert (sel[b, i, cnt[b, i]:] == -1).all()
    if k == 2:
        # the top group is ahead of everything else in every row, so the two
        # smallest ids of the group are the selection
        want = sorted(sorted(top, key=lambda w: ids[w])[:2])
        assert all([int(x) for x in sel[b, i, :2]] == want for b in range(bh) for i in range(QB))


def test_fwd_deterministic_and_fully_written():
    shape, kw = CASES["bf16_d64_T64_multi"]
    st = syn.make_state(shape, 3, **kw)
    L = run(shape, st)
    o1 = L.t["o"].clone(); l1 = L.t["lse"].clone()
    L.t["o"].fill_(float("nan")); L.t["lse"].fill_(float("nan"))
    L.fwd()
    torch.cuda.synchronize()
    assert torch.equal(L.t["o"], o1) and torch.equal(L.t["lse"], l1)


def test_memory_update_matches_oracle():
    shape = syn.Shape(B=1, H=3, d=128, T=128, Nq=300, W=8, C=5, topk=3)
    st = syn.make_state(shape, 5, sigma=1.0, shift=1.0, n_planted=3,
                        win_len=[128, 128, 44, 128, 0, 128, 128, 17], pool_count=[5, 2, 0],
                        pool_len=[128, 128, 100, 128, 128] * 3, pool_id=list(range(5)) * 3,
                        win_id=list(range(10, 18)))
    L = run(shape, st)
    before = {k: L.t[k].clone() for k in ("k_pool", "v_pool", "kbar_pool", "pool_id", "pool_len")}
    leaving = [0, 1, 2, 3, 4, 7, 2]  # slot 4 empty, slot 2 listed twice
    mp = L.t["mass_pool"].cpu().numpy(); mw = L.t["mass_win"].cpu().numpy()
    kbw = L.t["kbar_win"].cpu().numpy(); kbp = L.t["kbar_pool"].cpu().numpy()
    L.update(torch.tensor(leaving, dtype=torch.int32, device="cuda"), n_sink=1)
    torch.cuda.synchronize()
    u = po.memory_update(st, mp, mw, leaving, 1, kbar_win=kbw, kbar_pool=kbp)
    np.testing.assert_array_equal(L.t["pool_count"].cpu().numpy(), u["pool_count"])
    cnt = u["pool_count"]
    for b, h in np.ndindex(shape.B, shape.H):
        n = cnt[b, h]
        np.testing.assert_array_equal(L.t["pool_id"][b, h, :n].cpu().numpy(), u["pool_id"][b, h, :n])
        np.testing.assert_array_equal(L.t["pool_len"][b, h, :n].cpu().numpy(), u["pool_len"][b, h, :n])
        np.testing.assert_array_equal(L.t["kbar_pool"][b, h, :n].cpu().numpy(), u["kbar_pool"][b, h, :n])
        # copied K/V are bit-exact copies of their window slot; survivors untouched
        for slot, w in u["admitted"][(b, h)]:
            assert torch.equal(L.t["k_pool"][b, h, slot], L.t["k_win"][b, h, w])
            assert torch.equal(L.t["v_pool"][b, h, slot], L.t["v_win"][b, h, w])
        admitted = {s for s, _ in u["admitted"][(b, h)]}
        for slot in range(shape.C):
            if slot not in admitted:
                assert torch.equal(L.t["k_pool"][b, h, slot], before["k_pool"][b, h, slot])
    assert L.status_bits() == 0


def test_memory_update_shared_matches_oracle():
    """Head-shared pool: every head ranks by the masses summed over heads
    and all heads end with the same pool.  The oracle decides on the same
    fp32 sums the kernel forms (ascending head order), so near-ties order
    alike; the oracle's own head summation agrees with them to rounding."""
    shape = syn.Shape(B=2, H=3, d=128, T=128, Nq=300, W=8, C=5, topk=3)
    st = syn.make_state(shape, 7, sigma=1.0, shift=1.0, n_planted=3,
                        win_len=[128, 128, 44, 128, 0, 128, 128, 17], pool_count=4,
                        pool_len=[128, 128, 100, 128, 128], pool_id=list(range(5)),
                        win_id=list(range(10, 18)))
    L = run(shape, st)
    leaving = [0, 1, 2, 3, 4, 7, 2]
    mp = L.t["mass_pool"].cpu().numpy(); mw = L.t["mass_win"].cpu().numpy()
    kbw = L.t["kbar_win"].cpu().numpy(); kbp = L.t["kbar_pool"].cpu().numpy()
    L.update(torch.tensor(leaving, dtype=torch.int32, device="cuda"), n_sink=1, shared=True)
    torch.cuda.synchronize()
    # the kernel's fp32 sums, broadcast to every head
    sp = np.zeros_like(mp); sw = np.zeros_like(mw)
    for b in range(shape.B):
        accp = np.zeros(shape.C, np.float32); accw = np.zeros(shape.W, np.float32)
        for h in range(shape.H):
            accp = (accp + mp[b, h]).astype(np.float32); accw = (accw + mw[b, h]).astype(np.float32)
        sp[b] = accp; sw[b] = accw
    ref_p, ref_w = po.head_shared_masses(st, mp, mw)
    np.testing.assert_allclose(ref_p[:, :, :4], sp[:, :, :4], rtol=1e-6)
    np.testing.assert_allclose(ref_w, sw, rtol=1e-6)
    u = po.memory_update(st, sp, sw, leaving, 1, kbar_win=kbw, kbar_pool=kbp)
    np.testing.assert_array_equal(L.t["pool_count"].cpu().numpy(), u["pool_count"])
    for b, h in np.ndindex(shape.B, shape.H):
        n = u["pool_count"][b, h]
        np.testing.assert_array_equal(L.t["pool_id"][b, h, :n].cpu().numpy(), u["pool_id"][b, h, :n])
        np.testing.assert_array_equal(L.t["pool_id"][b, h].cpu().numpy(), L.t["pool_id"][b, 0].cpu().numpy())
        for slot, w in u["admitted"][(b, h)]:
            assert torch.equal(L.t["k_pool"][b, h, slot], L.t["k_win"][b, h, w])
    assert L.status_bits() == 0
    # heads that disagree are flagged
    L.t["pool_id"][1, 2, 0] = 99
    L.update(torch.tensor([5], dtype=torch.int32, device="cuda"), shared=True)
    torch.cuda.synchronize()
    assert L.status_bits() & P.PBSA_STATUS_SHARED


def test_window_append_copies_chunk():
    shape = syn.Shape(B=1, H=2, d=64, T=64, Nq=150, W=6, C=1, topk=1)
    st = syn.make_state(shape, 2, win_len=[64, 64, 22, 0, 0, 0], pool_count=1)
    L = run(shape, st)
    L.append_window(3, 1000)
    torch.cuda.synchronize()
    assert L.t["win_len"].cpu().tolist() == [64, 64, 22, 64, 64, 22]
    assert L.t["win_id"].cpu().tolist()[3:] == [1000, 1001, 1002]
    for j, n in enumerate([64, 64, 22]):
        assert torch.equal(L.t["k_win"][:, :, 3 + j, :n], L.t["k_cur"][:, :, 64 * j:64 * j + n])
        assert torch.equal(L.t["v_win"][:, :, 3 + j, :n], L.t["v_cur"][:, :, 64 * j:64 * j + n])
        assert torch.equal(L.t["kbar_win"][:, :, 3 + j], L.t["kbar_cur"][:, :, j])


def test_bad_device_metadata_is_clamped_and_flagged():
    shape = syn.Shape(B=1, H=1, d=64, T=64, Nq=64, W=3, C=2, topk=2)
    st = syn.make_state(shape, 1, pool_count=2)
    L = run(shape, st)
    o_ref = L.t["o"].clone()
    L.t["pool_count"].fill_(99)        # > C: clamped to C
    L.t["sel"][0, 0, 0, 1] = 1000      # outside [0, W): skipped
    L.fwd()
    torch.cuda.synchronize()
    bits = L.status_bits()
    assert bits & P.PBSA_STATUS_POOL_COUNT and bits & P.PBSA_STATUS_SEL
    assert not torch.isnan(L.t["o"].float()).any()
    del o_ref


# ------------------------------------------------------- Wan-shaped chunk ---
@pytest.mark.parametrize("unscaled", [False, True])
def test_wan_chunk_full_size(unscaled):
    """The Wan2.1-1.3B-shaped chunk (12 heads, 4680 tokens, window 74, pool 32,
    top-16) at full size, in the launch configuration the benchmark times:
    full selection and masses against the oracle, and O / LSE of every row
    of every head (all 444 query blocks)."""
    _log(f"wan chunk unscaled={unscaled}")
    shape = syn.WAN_CHUNK
    st = syn.wan_chunk_state(0, unscaled=unscaled)
    L = run(shape, st)
    scale = 1 / math.sqrt(128)
    r = po.select(st, shape.topk, scale, shape.T)
    n_tie = check_selection(L, r, st, shape.topk)
    _log(f"tie-band rows: {n_tie}")
    # planted blocks are recalled by every query block
    gsel = L.t["sel"].cpu().numpy(); gcnt = L.t["sel_count"].cpu().numpy()
    for idx in np.ndindex(*gcnt.shape):
        assert set(st["planted"]) <= set(gsel[idx].tolist())
    np.testing.assert_allclose(L.t["mass_pool"].cpu().numpy(), r["mass_pool"], rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(L.t["mass_win"].cpu().numpy(), r["mass_win"], rtol=1e-4, atol=1e-6)
    f = po.attn_fwd(st, gsel, gcnt, scale, shape.T)
    o = L.t["o"].float().cpu().numpy()
    assert not np.isnan(f["o"]).any()
    check_close_bf16(o, f["o"], f"wan chunk, all rows (unscaled={unscaled})")
    lse = L.t["lse"].cpu().numpy()
    assert np.abs(lse - f["lse"]).max() <= 2e-3
    assert L.status_bits() == 0


def test_tiny_f32_config_matches_oracle():
    """The tiny fp32 configuration itself (1 head of 64, blocks of 64, a
    256-token chunk, window 32, pool 4, top-4, seed 0, two planted window
    blocks): selection, pooled keys and masses, the forward (<= 1e-4) on the
    fp32 path, and the Top-C update with window slots 0-3 leaving, all
    against the oracle."""
    shape = syn.TINY_F32
    st = syn.tiny_f32_state()
    L = run(shape, st)
    scale = eff_scale(shape, 0.0)
    r = po.select(st, shape.topk, scale, shape.T)
    gsel = L.t["sel"].cpu().numpy(); gcnt = L.t["sel_count"].cpu().numpy()
    n_tie = check_selection(L, r, st, shape.topk)
    assert n_tie == 0
    for idx in np.ndindex(*gcnt.shape):
        assert set(st["planted"]) <= set(gsel[idx].tolist())
    np.testing.assert_allclose(L.t["kbar_cur"].cpu().numpy(), r["kbar_cur"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(L.t["kbar_win"].cpu().numpy(), r["kbar_win"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(L.t["mass_pool"].cpu().numpy(), r["mass_pool"], rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(L.t["mass_win"].cpu().numpy(), r["mass_win"], rtol=1e-4, atol=1e-6)
    f = po.attn_fwd(st, gsel, gcnt, scale, shape.T)
    o = L.t["o"].cpu().numpy()
    err = np.abs(o - f["o"]).max()
    _log(f"tiny fp32 forward: max-abs {err:.3e}")
    assert err <= 1e-4
    assert np.abs(L.t["lse"].cpu().numpy() - f["lse"]).max() <= 1e-5
    # the update: the oldest four window slots leave, the pool (4, full) keeps
    # the four best of 8 candidates
    mp = L.t["mass_pool"].cpu().numpy(); mw = L.t["mass_win"].cpu().numpy()
    kbw = L.t["kbar_win"].cpu().numpy(); kbp = L.t["kbar_pool"].cpu().numpy()
    before_k = L.t["k_pool"].clone()
    leaving = [0, 1, 2, 3]
    L.update(torch.tensor(leaving, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    u = po.memory_update(st, mp, mw, leaving, 0, kbar_win=kbw, kbar_pool=kbp)
    np.testing.assert_array_equal(L.t["pool_count"].cpu().numpy(), u["pool_count"])
    n = int(u["pool_count"][0, 0])
    np.testing.assert_array_equal(L.t["pool_id"][0, 0, :n].cpu().numpy(), u["pool_id"][0, 0, :n])
    np.testing.assert_array_equal(L.t["pool_len"][0, 0, :n].cpu().numpy(), u["pool_len"][0, 0, :n])
    np.testing.assert_array_equal(L.t["kbar_pool"][0, 0, :n].cpu().numpy(), u["kbar_pool"][0, 0, :n])
    admitted = {s_ for s_, _ in u["admitted"][(0, 0)]}
    for slot, w in u["admitted"][(0, 0)]:
        assert torch.equal(L.t["k_pool"][0, 0, slot], L.t["k_win"][0, 0, w])
        assert torch.equal(L.t["v_pool"][0, 0, slot], L.t["v_win"][0, 0, w])
    for slot in range(shape.C):
        if slot not in admitted:
            assert torch.equal(L.t["k_pool"][0, 0, slot], before_k[0, 0, slot])
    assert L.status_bits() == 0


def _one_head(st, h):
    """State of head h alone (B = 1): per-head tensors sliced, shared ones kept."""
    out = {}
    for k, v in st.items():
        if k in ("win_len", "win_id", "planted", "u"):
            out[k] = v
        elif hasattr(v, "dim") and v.dim() >= 2:
            out[k] = v[:, h:h + 1]
        else:
            out[k] = v
    return out


@pytest.mark.parametrize("unscaled", [False, True])
def test_fine_mass_wan_chunk_full_size(unscaled):
    """Exact block masses at the Wan chunk, full size: two heads against the
    oracle (all their query blocks), every head checked for the identity
    sum of pool + window masses <= query rows, and the planted window
    blocks (chosen by every query block) holding more mass than the rest."""
    _log(f"fine mass wan chunk unscaled={unscaled}")
    shape = syn.WAN_CHUNK
    st = syn.wan_chunk_state(0, unscaled=unscaled)
    L = run(shape, st)
    L.t["mass_pool"].fill_(float("nan")); L.t["mass_win"].fill_(float("nan"))
    L.fine_mass()
    torch.cuda.synchronize()
    mp = L.t["mass_pool"].cpu().numpy(); mw = L.t["mass_win"].cpu().numpy()
    assert not np.isnan(mp).any() and not np.isnan(mw).any()
    tot = mp.sum(-1) + mw.sum(-1)
    assert (tot > 0).all() and (tot <= shape.Nq * (1 + 1e-3)).all()
    gsel = L.t["sel"].cpu().numpy(); gcnt = L.t["sel_count"].cpu().numpy()
    scale = 1 / math.sqrt(128)
    for h in (0, 7):
        ref = po.fine_mass(_one_head(st, h), gsel[:, h:h + 1], gcnt[:, h:h + 1], scale, shape.T)
        for n, got in (("mass_pool", mp[:, h:h + 1]), ("mass_win", mw[:, h:h + 1])):
            r = ref[n]
            err = np.abs(got - r).max()
            bar = 5e-3 * np.abs(r).max() + 1e-7
            _log(f"head {h} {n}: max-abs {err:.3e} (bar {bar:.3e}), max {np.abs(r).max():.3e}")
            assert err <= bar, (h, n, err, bar)
    planted = st["planted"]
    others = [w for w in range(shape.W) if w not in planted]
    assert mw[0][:, planted].min() > mw[0][:, others].max()


def test_maximum_sizes():
    """W = C = 1024 (the largest window and pool), k = 1000: routing, the
    forward over 2,026 blocks per query block, exact masses and a full
    update (1,024 pool blocks + 1,024 leaving candidates) against the oracle."""
    shape = syn.Shape(B=1, H=1, d=64, T=64, Nq=2 * 64 - 9, W=1024, C=1024, topk=1000)
    wl = [64] * 1024
    wl[5] = 0; wl[700] = 13
    pl = [64] * 1024
    pl[3] = 40
    st = syn.make_state(shape, 17, sigma=1.0, shift=1.0, n_planted=6, win_len=wl, pool_count=1024,
                        pool_len=pl, win_id=list(range(2000, 3024)))
    _log("max sizes: select + fwd")
    L = run(shape, st)
    scale = eff_scale(shape, 0.0)
    r = po.select(st, shape.topk, scale, shape.T)
    check_selection(L, r, st, shape.topk)
    np.testing.assert_allclose(L.t["mass_pool"].cpu().numpy(), r["mass_pool"], rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(L.t["mass_win"].cpu().numpy(), r["mass_win"], rtol=1e-4, atol=1e-6)
    gsel = L.t["sel"].cpu().numpy(); gcnt = L.t["sel_count"].cpu().numpy()
    f = po.attn_fwd(st, gsel, gcnt, scale, shape.T)
    check_close_bf16(L.t["o"].float().cpu().numpy(), f["o"], "max sizes")
    assert np.abs(L.t["lse"].cpu().numpy() - f["lse"]).max() <= 2e-3
    _log("max sizes: fine mass")
    mp0 = L.t["mass_pool"].clone(); mw0 = L.t["mass_win"].clone()
    L.fine_mass()
    torch.cuda.synchronize()
    ref = po.fine_mass(st, gsel, gcnt, scale, shape.T)
    for n in ("mass_pool", "mass_win"):
        got = L.t[n].cpu().numpy(); rr = ref[n]
        assert np.abs(got - rr).max() <= 5e-3 * np.abs(rr).max() + 1e-7, n
    _log("max sizes: update")
    L.t["mass_pool"].copy_(mp0); L.t["mass_win"].copy_(mw0)
    leaving = list(range(1024))
    mp = mp0.cpu().numpy(); mw = mw0.cpu().numpy()
    L.update(torch.tensor(leaving, dtype=torch.int32, device="cuda"), n_sink=0)
    torch.cuda.synchronize()
    u = po.memory_update(st, mp, mw, leaving, 0)
    np.testing.assert_array_equal(L.t["pool_count"].cpu().numpy(), u["pool_count"])
    n = int(u["pool_count"][0, 0])
    np.testing.assert_array_equal(L.t["pool_id"][0, 0, :n].cpu().numpy(), u["pool_id"][0, 0, :n])
    assert L.status_bits() == 0

"""Pins of the fp64 oracle against facts that do not come from the oracle:
closed forms, brute force over tiny inputs, textbook dense attention (torch
fp64 library routines), central finite differences, and invariants.

Every function of ``oracle/pbsa_oracle.py`` has at least one pin here, chosen
so that a dropped term, a wrong sign, index or transposed operand fails one of
them (see ``test_pins_catch_planted_mistakes`` for mistakes planted on purpose
into copies of the oracle's functions).
"""
import itertools
import math

import numpy as np
import pytest
import torch

import pbsa_synth as syn
from oracle import pbsa_oracle as po
from oracle import rollout as orl
from oracle.rollout import OracleRollout


def small_state(B=1, H=2, d=8, T=4, Nq=10, W=6, C=3, topk=2, seed=0, win_len=None,
                pool_count=None, pool_len=None, pad_value=float("nan"), sigma=1.0):
    shape = syn.Shape(B=B, H=H, d=d, T=T, Nq=Nq, W=W, C=C, topk=topk, dtype=torch.float32)
    st = syn.make_state(shape, seed, sigma=sigma, win_len=win_len, pool_count=pool_count,
                        pool_len=pool_len, pad_value=pad_value)
    return shape, st


# ---------------------------------------------------------------- pooling ---
def test_block_mean_closed_form():
    # rows r*a + c (r = 0..n-1): mean = a (n-1)/2 + c, exactly
    a = np.array([1.0, -2.0, 0.5]); c = np.array([3.0, 0.0, -1.0])
    for n in (1, 2, 5, 72):
        rows = np.arange(n)[:, None] * a + c
        np.testing.assert_allclose(po.block_mean(rows), a * (n - 1) / 2 + c, rtol=0, atol=1e-12)


def test_pooled_queries_ragged_tail():
    # Nq = 10, T = 4: blocks of 4, 4, 2 rows; constant rows per block
    q = np.zeros((1, 1, 10, 3))
    q[0, 0, :4] = 1.0; q[0, 0, 4:8] = 2.0; q[0, 0, 8:] = 7.0
    q[0, 0, 9, 0] = 9.0   # tail block: rows 8 (7) and 9 (9) in column 0 -> 8
    qb = po.pooled_queries(q, 4)
    assert qb.shape == (1, 1, 3, 3)
    np.testing.assert_array_equal(qb[0, 0, :, 1], [1.0, 2.0, 7.0])
    assert qb[0, 0, 2, 0] == 8.0


def test_pooled_slots_ragged_closed_form():
    # slot rows r*a + c for r < len (mean a (len-1)/2 + c, exactly); the
    # padding rows after len hold a large finite value, so a mean that reads
    # them, or divides a short slot's sum by T, is off by far more than the
    # tolerance.  An empty slot has no representative (NaN).
    T, d = 8, 3
    a = np.array([1.0, -2.0, 0.5]); c = np.array([3.0, 0.0, -1.0])
    lens = np.array([8, 3, 1, 0, 5])
    k = np.full((1, 1, len(lens), T, d), 1000.0)
    for w, n in enumerate(lens):
        k[0, 0, w, :n] = np.arange(n)[:, None] * a + c
    got = po.pooled_slots(k, lens[None, None, :])
    for w, n in enumerate(lens):
        if n == 0:
            assert np.isnan(got[0, 0, w]).all()
        else:
            np.testing.assert_allclose(got[0, 0, w], a * (n - 1) / 2 + c, rtol=0, atol=1e-12)
    # the same means seen through the coarse logits of select(): all queries
    # are e0, so slot w's logit is scale * (its mean's first coordinate)
    W = len(lens)
    shape, st = small_state(B=1, H=1, d=d, T=T, Nq=2 * T, W=W, C=2, topk=2,
                            win_len=lens.tolist(), pool_count=0, pad_value=0.0)
    st["q"][:] = 0; st["q"][..., 0] = 1.0
    st["k_win"][:] = torch.from_numpy(k.astype(np.float32))
    r = po.select(st, 2, 0.5, T)
    for w, n in enumerate(lens):
        if n > 0:
            np.testing.assert_allclose(r["s_win"][0, 0, :, w], 0.5 * (a[0] * (n - 1) / 2 + c[0]),
                                       rtol=0, atol=1e-12)
        else:
            assert np.isnan(r["s_win"][0, 0, :, w]).all()


def test_coarse_scores_with_T1_are_token_logits():
    # T = 1: every block is one token, so coarse logits are the token logits
    shape, st = small_state(T=1, Nq=5, W=6, C=2, topk=6, d=8, H=1)
    r = po.select(st, 6, 0.3, 1)
    q = st["q"].double()[0, 0]; kw = st["k_win"].double()[0, 0, :, 0]
    ref = 0.3 * (q @ kw.T)
    np.testing.assert_allclose(r["s_win"][0, 0], ref.numpy(), rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ top-k ---
def _const_key_state(cw, ids, lens, topk, d=4, T=3, Nq=6, n_pool=0):
    """Window slot w has every key row = cw[w] * e0 and every query = e0, so
    the coarse logit of slot w is exactly scale * cw[w]."""
    W = len(cw)
    shape, st = small_state(B=1, H=1, d=d, T=T, Nq=Nq, W=W, C=2, topk=topk, win_len=lens,
                            pool_count=n_pool, pad_value=0.0)
    st["q"][:] = 0; st["q"][..., 0] = 1.0
    for w in range(W):
        st["k_win"][0, 0, w] = 0.0
        st["k_win"][0, 0, w, :, 0] = cw[w]
    st["win_id"] = torch.tensor(ids, dtype=torch.int64)
    return st


def test_topk_constructed_order_and_tiebreak():
    cw = [0.5, 0.1, 0.9, 0.5, -1.0, float("nan"), 0.7, 0.2]
    ids = [10, 11, 12, 3, 14, 15, 16, 17]
    lens = [3, 3, 3, 3, 3, 3, 0, 2]          # slot 6 empty: never selected
    st = _const_key_state(cw, ids, lens, topk=3)
    r = po.select(st, 3, 1.0, 3)
    # valid: 0(.5,id10) 1(.1) 2(.9) 3(.5,id3) 4(-1) 5(nan) 7(.2)
    # order: 2 (.9), then tie .5: id 3 (slot 3) before id 10 (slot 0) -> {2,3,0}
    assert r["sel"][0, 0, 0].tolist() == [0, 2, 3]
    assert r["sel_count"][0, 0, 0] == 3
    # k = 6 of 7 valid: NaN ranks last, so slot 5 is the one left out
    r6 = po.select(st, 6, 1.0, 3)
    assert r6["sel"][0, 0, 0].tolist() == [0, 1, 2, 3, 4, 7]
    # k >= valid slots: all 7 valid slots, padded with -1
    r9 = po.select(st, 9, 1.0, 3)
    assert r9["sel"][0, 0, 0].tolist() == [0, 1, 2, 3, 4, 5, 7, -1, -1]
    assert r9["sel_count"][0, 0, 0] == 7
    # k = 0 selects nothing
    r0 = po.select(st, 0, 1.0, 3)
    assert r0["sel_count"][0, 0, 0] == 0


def test_topk_scale_sign_matters():
    # a negative scale reverses the order: catches a dropped or misplaced scale
    cw = [0.5, 0.1, 0.9, 0.3]
    st = _const_key_state(cw, [0, 1, 2, 3], [3, 3, 3, 3], topk=1)
    assert po.select(st, 1, -1.0, 3)["sel"][0, 0, 0].tolist() == [1]
    assert po.select(st, 1, 2.0, 3)["sel"][0, 0, 0].tolist() == [2]


@pytest.mark.parametrize("which", ["tiny", "wan_like"])
def test_planted_blocks_are_recalled(which):
    if which == "tiny":
        st = syn.tiny_f32_state()
        k, scale, T = 4, 1 / 8, 64
    else:   # Wan chunk geometry and generator, 2 heads and a 3-block chunk for speed
        shape = syn.Shape(B=1, H=2, d=128, T=128, Nq=3 * 128 - 56, W=6, C=4, topk=4)
        st = syn.make_state(shape, 1000, sigma=1 / math.sqrt(128), shift=1.5, n_planted=3,
                            win_len=[128, 128, 72, 128, 128, 72])
        k, scale, T = 4, 1 / math.sqrt(128), 128
    r = po.select(st, k, scale, T)
    for b, h, i in np.ndindex(*r["sel_count"].shape):
        assert set(st["planted"]) <= set(r["sel"][b, h, i].tolist())


# --------------------------------------------------------------- attention ---
def _sdpa64(q, k, v, scale, mask=None):
    """Textbook softmax attention in fp64 through torch's library routine."""
    return torch.nn.functional.scaled_dot_product_attention(
        q[None, None], k[None, None], v[None, None], attn_mask=mask, scale=scale)[0, 0]


def test_fwd_dense_limit_equals_textbook_attention():
    # every valid window slot selected + pool attended => dense attention over
    # [valid pool tokens; valid window tokens; current chunk]
    lens = [4, 2, 0, 4, 3, 1]
    shape, st = small_state(H=2, d=8, T=4, Nq=10, W=6, C=3, win_len=lens,
                            pool_count=[2, 3], pool_len=[4, 1, 3, 4, 4, 2])
    scale = 0.37
    r = po.select(st, 6, scale, 4)
    f = po.attn_fwd(st, r["sel"], r["sel_count"], scale, 4)
    for h in range(2):
        n_pool = int(st["pool_count"][0, h])
        ks, vs = [], []
        for p in range(n_pool):
            n = int(st["pool_len"][0, h, p])
            ks.append(st["k_pool"][0, h, p, :n]); vs.append(st["v_pool"][0, h, p, :n])
        for w in range(6):
            ks.append(st["k_win"][0, h, w, :lens[w]]); vs.append(st["v_win"][0, h, w, :lens[w]])
        ks.append(st["k_cur"][0, h]); vs.append(st["v_cur"][0, h])
        K = torch.cat(ks).double(); V = torch.cat(vs).double()
        ref = _sdpa64(st["q"][0, h].double(), K, V, scale)
        np.testing.assert_allclose(f["o"][0, h], ref.numpy(), rtol=1e-12, atol=1e-12)
        lse = torch.logsumexp(scale * st["q"][0, h].double() @ K.T, dim=1)
        np.testing.assert_allclose(f["lse"][0, h], lse.numpy(), rtol=1e-12, atol=1e-12)


def _flat_token_mask(st, sel, sel_count, T, C, W):
    """Independent brute force: one flat token axis [pool C*T | window W*T |
    current Nq] and a boolean mask per query row, built token by token."""
    B, H, nq, d = st["q"].shape
    n_tok = C * T + W * T + nq
    mask = np.zeros((B, H, nq, n_tok), dtype=bool)
    for b, h, r in np.ndindex(B, H, nq):
        i = r // T
        chosen = set(int(w) for w in sel[b, h, i, :sel_count[b, h, i]])
        for p in range(C):
            for t in range(T):
                mask[b, h, r, p * T + t] = p < int(st["pool_count"][b, h]) and t < int(st["pool_len"][b, h, p])
        for w in range(W):
            for t in range(T):
                mask[b, h, r, C * T + w * T + t] = (w in chosen) and t < int(st["win_len"][w])
        mask[b, h, r, C * T + W * T:] = True
    K = torch.cat([st["k_pool"].reshape(B, H, C * T, d), st["k_win"].reshape(B, H, W * T, d),
                   st["k_cur"]], dim=2).double()
    V = torch.cat([st["v_pool"].reshape(B, H, C * T, d), st["v_win"].reshape(B, H, W * T, d),
                   st["v_cur"]], dim=2).double()
    return mask, torch.nan_to_num(K), torch.nan_to_num(V)


@pytest.mark.parametrize("T,d", [(2, 4), (4, 8)])
def test_fwd_matches_bruteforce_token_mask(T, d):
    W, C = 5, 3
    lens = [T, 1, 0, T, T - 1 if T > 1 else 1]
    shape, st = small_state(B=2, H=2, d=d, T=T, Nq=3 * T - 1, W=W, C=C, topk=2, win_len=lens,
                            pool_count=[0, 1, 3, 2], pool_len=[T, 1, T] * 4, seed=3)
    scale = 0.5
    r = po.select(st, 2, scale, T)
    f = po.attn_fwd(st, r["sel"], r["sel_count"], scale, T)
    mask, K, V = _flat_token_mask(st, r["sel"], r["sel_count"], T, C, W)
    q = st["q"].double()
    z = scale * q @ K.transpose(-1, -2)
    z = z.masked_fill(~torch.from_numpy(mask), float("-inf"))
    ref = torch.softmax(z, dim=-1) @ V
    np.testing.assert_allclose(f["o"], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_fwd_invariants_ones_and_zero_queries():
    shape, st = small_state(H=1, d=8, T=4, Nq=7, W=5, C=2, win_len=[4, 3, 4, 0, 2],
                            pool_count=2, pool_len=[4, 2])
    for name in ("v_cur", "v_win", "v_pool"):
        v = st[name]
        st[name] = torch.where(torch.isnan(v), v, torch.ones_like(v))
    r = po.select(st, 2, 0.4, 4)
    f = po.attn_fwd(st, r["sel"], r["sel_count"], 0.4, 4)
    np.testing.assert_allclose(f["o"], 1.0, atol=1e-14)            # V == 1 => O == 1
    # Q == 0: all logits 0 -> uniform weights, LSE = ln |U_i|, O = mean of V over U_i
    st["q"][:] = 0
    f = po.attn_fwd(st, r["sel"], r["sel_count"], 0.4, 4)
    for i in range(2):
        n_u = 4 + 2 + sum([4, 3, 4, 0, 2][w] for w in r["sel"][0, 0, i] if w >= 0) + 7
        rows = po.query_block_rows(7, 4, i)
        np.testing.assert_allclose(f["lse"][0, 0, rows.start:rows.stop], math.log(n_u), atol=1e-13)


def test_fwd_single_block_is_plain_attention():
    # no pool, k = 0, a single current block: ordinary attention over the chunk
    shape, st = small_state(H=1, d=8, T=8, Nq=8, W=3, C=2, pool_count=0, seed=5)
    r = po.select(st, 0, 0.25, 8)
    f = po.attn_fwd(st, r["sel"], r["sel_count"], 0.25, 8)
    ref = _sdpa64(st["q"][0, 0].double(), st["k_cur"][0, 0].double(), st["v_cur"][0, 0].double(), 0.25)
    np.testing.assert_allclose(f["o"][0, 0], ref.numpy(), rtol=1e-13, atol=1e-13)


def test_fwd_golden_hand_example():
    # tests/golden/fwd_hand.txt: a worked example derived by hand
    g = _read_golden("fwd_hand.txt")
    shape, st = small_state(B=1, H=1, d=2, T=1, Nq=1, W=1, C=1, topk=1, win_len=[1],
                            pool_count=1, pool_len=[1], pad_value=0.0)
    st = {k: (v.double() if torch.is_tensor(v) and v.is_floating_point() else v) for k, v in st.items()}
    st["q"][0, 0, 0] = torch.tensor(g["q"], dtype=torch.float64)
    st["k_pool"][0, 0, 0, 0] = torch.tensor(g["k_pool"], dtype=torch.float64); st["v_pool"][0, 0, 0, 0] = torch.tensor(g["v_pool"], dtype=torch.float64)
    st["k_win"][0, 0, 0, 0] = torch.tensor(g["k_win"], dtype=torch.float64); st["v_win"][0, 0, 0, 0] = torch.tensor(g["v_win"], dtype=torch.float64)
    st["k_cur"][0, 0, 0] = torch.tensor(g["k_cur"], dtype=torch.float64); st["v_cur"][0, 0, 0] = torch.tensor(g["v_cur"], dtype=torch.float64)
    r = po.select(st, 1, 1.0, 1)
    f = po.attn_fwd(st, r["sel"], r["sel_count"], 1.0, 1)
    np.testing.assert_allclose(f["o"][0, 0, 0], g["o"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(f["lse"][0, 0, 0], g["lse"][0], rtol=1e-14)


def _read_golden(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    out = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, vals = line.split("=")
        out[key.strip()] = [float(eval(x, {"math": math})) for x in vals.split(",")]
    return out


# ---------------------------------------------------------------- backward ---
def _loss(st, sel, sel_count, dout, scale, T):
    f = po.attn_fwd(st, sel, sel_count, scale, T)
    return float((f["o"] * dout).sum())


def test_bwd_matches_central_finite_differences():
    T, d = 2, 3
    shape, st = small_state(B=1, H=1, d=d, T=T, Nq=3, W=3, C=2, topk=1, win_len=[2, 1, 2],
                            pool_count=2, pool_len=[2, 1], pad_value=0.0, seed=11)
    st = po.as_f64_state(st)
    scale = 0.7
    r = po.select(st, 1, scale, T)
    sel, sc = r["sel"], r["sel_count"]
    dout = np.random.default_rng(1).standard_normal(st["q"].shape)
    g = po.attn_bwd(st, sel, sc, dout, scale, T)
    eps = 1e-6
    checks = [("q", "dq"), ("k_cur", "dk_cur"), ("v_cur", "dv_cur"), ("k_win", "dk_win"),
              ("v_win", "dv_win"), ("k_pool", "dk_pool"), ("v_pool", "dv_pool")]
    n_nonzero = 0
    for name, gname in checks:
        x = st[name]
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps; lp = _loss(st, sel, sc, dout, scale, T)
            x[idx] = old - eps; lm = _loss(st, sel, sc, dout, scale, T)
            x[idx] = old
            fd = (lp - lm) / (2 * eps)
            an = g[gname][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, an)
            n_nonzero += abs(an) > 1e-9
    assert n_nonzero > 20


def test_bwd_matches_torch_autograd_dense_masked_form():
    T, d, W, C = 4, 8, 5, 3
    lens = [4, 2, 4, 0, 3]
    shape, st = small_state(B=1, H=2, d=d, T=T, Nq=9, W=W, C=C, topk=2, win_len=lens,
                            pool_count=[3, 1], pool_len=[4, 3, 2, 1, 4, 4], seed=7)
    scale = 0.45
    r = po.select(st, 2, scale, T)
    dout = torch.randn(st["q"].shape, generator=torch.Generator().manual_seed(2), dtype=torch.float64)
    g = po.attn_bwd(st, r["sel"], r["sel_count"], dout.numpy(), scale, T)
    mask, K, V = _flat_token_mask(st, r["sel"], r["sel_count"], T, C, W)
    q = st["q"].double().clone().requires_grad_(True)
    K = K.clone().requires_grad_(True); V = V.clone().requires_grad_(True)
    z = scale * q @ K.transpose(-1, -2)
    z = z.masked_fill(~torch.from_numpy(mask), float("-inf"))
    o = torch.softmax(z, dim=-1) @ V
    (o * dout).sum().backward()
    np.testing.assert_allclose(g["dq"], q.grad.numpy(), rtol=1e-11, atol=1e-11)
    B, H = 1, 2
    dk = K.grad.numpy(); dv = V.grad.numpy()
    np.testing.assert_allclose(g["dk_pool"].reshape(B, H, C * T, d), dk[:, :, :C * T], atol=1e-11)
    np.testing.assert_allclose(g["dv_win"].reshape(B, H, W * T, d), dv[:, :, C * T:C * T + W * T], atol=1e-11)
    np.testing.assert_allclose(g["dk_cur"], dk[:, :, C * T + W * T:], atol=1e-11)
    np.testing.assert_allclose(g["dv_cur"], dv[:, :, C * T + W * T:], atol=1e-11)


def test_bwd_invariants():
    shape, st = small_state(B=1, H=1, d=8, T=4, Nq=10, W=6, C=3, topk=2, pad_value=0.0, seed=9)
    r = po.select(st, 2, 0.3, 4)
    dout = np.random.default_rng(3).standard_normal(st["q"].shape)
    g = po.attn_bwd(st, r["sel"], r["sel_count"], dout, 0.3, 4)
    # every row's weights sum to one => sum over all tokens of dV = sum over rows of dO
    tot = g["dv_cur"].sum(axis=(0, 1, 2)) + g["dv_win"].sum(axis=(0, 1, 2, 3)) + g["dv_pool"].sum(axis=(0, 1, 2, 3))
    np.testing.assert_allclose(tot, dout.sum(axis=(0, 1, 2)), atol=1e-12)
    # rows of dS sum to zero => sum of dK is scale * sum_r (sum_u dS_ru) Q_r = 0
    totk = g["dk_cur"].sum(axis=(0, 1, 2)) + g["dk_win"].sum(axis=(0, 1, 2, 3)) + g["dk_pool"].sum(axis=(0, 1, 2, 3))
    np.testing.assert_allclose(totk, 0.0, atol=1e-12)
    # unselected window slots get no gradient
    chosen = set(r["sel"][0, 0].ravel().tolist()) - {-1}
    for w in range(6):
        if w not in chosen:
            assert not g["dk_win"][0, 0, w].any() and not g["dv_win"][0, 0, w].any()


# -------------------------------------------------------------- block mass ---
def test_mass_uniform_when_scores_equal():
    # Q == 0 => every coarse logit is 0 => pi = 1/|J| => M_j = QB/|J|
    shape, st = small_state(H=1, d=8, T=4, Nq=10, W=6, C=3, win_len=[4, 4, 0, 1, 4, 4],
                            pool_count=2, pool_len=[4, 4, 4])
    st["q"][:] = 0
    r = po.select(st, 2, 1.0, 4)
    n_j = 2 + 5 + 3
    np.testing.assert_allclose(r["mass_pool"][0, 0, :2], 3 / n_j, rtol=1e-14)
    assert r["mass_pool"][0, 0, 2] == 0
    np.testing.assert_allclose(r["mass_win"][0, 0, [0, 1, 3, 4, 5]], 3 / n_j, rtol=1e-14)
    assert r["mass_win"][0, 0, 2] == 0


def test_mass_two_candidates_logistic():
    # one pool block, no window slot, one current block: pi_pool = sigmoid(s_p - s_c)
    shape, st = small_state(H=1, d=4, T=4, Nq=4, W=1, C=1, win_len=[0], pool_count=1,
                            pool_len=[4], pad_value=0.0, seed=2)
    scale = 0.9
    r = po.select(st, 1, scale, 4)
    qb = st["q"][0, 0].double().mean(0); kp = st["k_pool"][0, 0, 0].double().mean(0)
    kc = st["k_cur"][0, 0].double().mean(0)
    expect = 1.0 / (1.0 + math.exp(-scale * float(qb @ kp - qb @ kc)))
    assert abs(r["mass_pool"][0, 0, 0] - expect) < 1e-14


def test_mass_sums_to_query_blocks_when_current_is_negligible():
    # current-chunk keys pushed far away: their softmax weight vanishes, so the
    # pool + window masses sum to QB (rows of pi sum to one)
    shape, st = small_state(H=1, d=4, T=4, Nq=12, W=5, C=2, pool_count=2, pad_value=0.0, seed=4)
    st["q"][:] = 1.0
    st["k_cur"][:] = -50.0
    r = po.select(st, 2, 1.0, 4)
    total = r["mass_pool"].sum() + r["mass_win"].sum()
    assert abs(total - 3.0) < 1e-12


# ---------------------------------------------- fine-grained block mass ---
def test_fine_mass_uniform_when_queries_are_zero():
    # Q == 0 => every row attends its set U_i uniformly => a block j in U_i
    # receives rows_i * len_j / |U_i| from query block i
    T, nq = 4, 10
    lens = [4, 4, 0, 1, 4, 3]
    shape, st = small_state(H=2, d=8, T=T, Nq=nq, W=6, C=3, win_len=lens,
                            pool_count=[2, 3], pool_len=[4, 2, 4, 4, 1, 3])
    st["q"][:] = 0
    sel = np.array([[[[0, 3, -1], [1, 4, 5], [5, -1, -1]],
                     [[2, 4, -1], [0, 1, 3], [3, 4, -1]]]])
    cnt = np.array([[[2, 3, 1], [2, 3, 2]]])
    r = po.fine_mass(st, sel, cnt, 0.7, T)
    for h in range(2):
        n_pool = int(st["pool_count"][0, h])
        plen = [int(x) for x in st["pool_len"][0, h]]
        ep = np.zeros(3); ew = np.zeros(6); ec = np.zeros(3)
        for i in range(3):
            rows = min(T, nq - i * T)
            chosen = [w for w in sel[0, h, i, :cnt[0, h, i]]]
            n_u = sum(plen[:n_pool]) + sum(lens[w] for w in chosen) + nq
            for p_ in range(n_pool):
                ep[p_] += rows * plen[p_] / n_u
            for w in chosen:
                ew[w] += rows * lens[w] / n_u
            for c in range(3):
                ec[c] += rows * min(T, nq - c * T) / n_u
        np.testing.assert_allclose(r["mass_pool"][0, h], ep, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(r["mass_win"][0, h], ew, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(r["mass_cur"][0, h], ec, rtol=1e-13, atol=1e-15)


def test_fine_mass_rows_sum_to_one():
    # every valid query row distributes exactly one unit of mass
    shape, st = small_state(H=2, d=8, T=4, Nq=11, W=5, C=2, win_len=[4, 3, 4, 0, 4],
                            pool_count=[2, 1], pool_len=[4, 2, 4, 4], seed=6)
    r = po.select(st, 2, 0.5, 4)
    f = po.fine_mass(st, r["sel"], r["sel_count"], 0.5, 4)
    total = f["mass_pool"].sum(-1) + f["mass_win"].sum(-1) + f["mass_cur"].sum(-1)
    np.testing.assert_allclose(total, 11.0, rtol=1e-13)
    assert (f["mass_pool"] >= 0).all() and (f["mass_win"] >= 0).all()


@pytest.mark.parametrize("T,d", [(2, 4), (4, 8)])
def test_fine_mass_matches_bruteforce_token_mask(T, d):
    # flat token axis [pool C*T | window W*T | current Nq], masked softmax by
    # torch's library routine, then summed over each block's token range
    C, W, nq = 3, 5, 3 * T + 1
    shape, st = small_state(H=2, d=d, T=T, Nq=nq, W=W, C=C,
                            win_len=[T, 1, 0, T, T - 1], pool_count=[3, 1],
                            pool_len=[T, 1, T, T, T, T], seed=8)
    scale = 0.8
    r = po.select(st, 2, scale, T)
    sel, cnt = r["sel"], r["sel_count"]
    f = po.fine_mass(st, sel, cnt, scale, T)
    mask, K, _ = _flat_token_mask(st, sel, cnt, T, C, W)
    z = scale * torch.einsum("bhrd,bhud->bhru", st["q"].double(), K)
    z = z.masked_fill(~torch.from_numpy(mask), float("-inf"))
    P = torch.softmax(z, dim=-1).numpy()
    col = P.sum(axis=2)                                    # [B,H,n_tok]
    for h in range(2):
        np.testing.assert_allclose(f["mass_pool"][0, h], col[0, h, :C * T].reshape(C, T).sum(-1),
                                   rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(f["mass_win"][0, h],
                                   col[0, h, C * T:C * T + W * T].reshape(W, T).sum(-1),
                                   rtol=1e-12, atol=1e-14)
        cur = col[0, h, C * T + W * T:]
        np.testing.assert_allclose(f["mass_cur"][0, h],
                                   [cur[c * T:(c + 1) * T].sum() for c in range(4)],
                                   rtol=1e-12, atol=1e-14)


# ------------------------------------------------- training through a rollout ---
def _random_rollout(n, B, H, d, T, Nq, seed):
    g = torch.Generator().manual_seed(seed)
    QB = -(-Nq // T)
    mk = lambda: [torch.randn(B, H, Nq, d, generator=g, dtype=torch.float64) for _ in range(n)]
    q, k, v, dout = mk(), mk(), mk(), mk()
    rng = np.random.default_rng(seed)
    plans = [[[[sorted(int(x) for x in rng.choice(t * QB, size=rng.integers(0, t * QB + 1),
                                                   replace=False)) if t else []
                for _ in range(QB)] for _ in range(H)] for _ in range(B)] for t in range(n)]
    return q, k, v, dout, plans, QB


def test_rollout_grads_match_autograd_of_flat_masked_attention():
    # every chunk's keys on one flat axis [chunk 0 | chunk 1 | ...]; a query
    # row of chunk t sees its planned history blocks and all of chunk t; torch
    # autograd of sum <dO, O> is the reference
    n, B, H, d, T, Nq = 4, 1, 2, 4, 2, 5
    q, k, v, dout, plans, QB = _random_rollout(n, B, H, d, T, Nq, 11)
    scale = 0.6
    r = orl.rollout_attention_grads([x.numpy() for x in q], [x.numpy() for x in k],
                                [x.numpy() for x in v], plans, [x.numpy() for x in dout], scale, T)
    qs = [x.clone().requires_grad_() for x in q]
    K = torch.cat([x.clone() for x in k], dim=2).requires_grad_()
    V = torch.cat([x.clone() for x in v], dim=2).requires_grad_()
    loss = 0
    for t in range(n):
        mask = torch.zeros(B, H, Nq, n * Nq, dtype=torch.bool)
        for b, h, row in itertools.product(range(B), range(H), range(Nq)):
            for x_id in plans[t][b][h][row // T]:
                c, j = divmod(x_id, QB)
                mask[b, h, row, c * Nq + j * T:c * Nq + min(Nq, (j + 1) * T)] = True
            mask[b, h, row, t * Nq:(t + 1) * Nq] = True
        z = scale * qs[t] @ K.transpose(-1, -2)
        P = torch.softmax(z.masked_fill(~mask, float("-inf")), dim=-1)
        loss = loss + (dout[t] * (P @ V)).sum()
    loss.backward()
    for t in range(n):
        np.testing.assert_allclose(r["dq"][t], qs[t].grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(r["dk"][t], K.grad[:, :, t * Nq:(t + 1) * Nq].numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(r["dv"][t], V.grad[:, :, t * Nq:(t + 1) * Nq].numpy(), rtol=1e-10, atol=1e-12)


def test_rollout_grads_single_chunk_is_the_chunk_backward():
    n, B, H, d, T, Nq = 1, 1, 2, 8, 4, 10
    q, k, v, dout, plans, QB = _random_rollout(n, B, H, d, T, Nq, 3)
    r = orl.rollout_attention_grads([x.numpy() for x in q], [x.numpy() for x in k],
                                [x.numpy() for x in v], plans, [x.numpy() for x in dout], 0.4, T)
    shape = syn.Shape(B=B, H=H, d=d, T=T, Nq=Nq, W=0, C=0, topk=0, dtype=torch.float32)
    st = syn.make_state(shape, 0, win_len=[], pool_count=0)
    st["q"], st["k_cur"], st["v_cur"] = q[0], k[0], v[0]
    g = po.attn_bwd(st, np.zeros((B, H, QB, 1), int), np.zeros((B, H, QB), int), dout[0].numpy(), 0.4, T)
    np.testing.assert_allclose(r["dq"][0], g["dq"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dk"][0], g["dk_cur"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dv"][0], g["dv_cur"], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------- memory update ---
def test_update_matches_best_subset_bruteforce():
    rng = np.random.default_rng(0)
    C = 4
    for trial in range(40):
        pool_ids = [int(x) for x in rng.choice(50, size=4, replace=False)]
        cand_ids = [int(x) for x in rng.choice(np.arange(50, 100), size=4, replace=False)]
        n_sink = int(rng.integers(0, 3)) * 10      # at most 4 pinned (pool ids < 50)
        pm = rng.random(4).tolist(); cm = rng.random(4).tolist()
        assign, new_ids, status = po.memory_update_one(pool_ids, pm, cand_ids, cm, C, n_sink)
        X = list(zip(pool_ids + cand_ids, pm + cm))
        pinned = {i for i, _ in X if i < n_sink}
        best, best_val = None, -1
        for sub in itertools.combinations(X, C):
            ids = {i for i, _ in sub}
            if not pinned <= ids:
                continue
            val = sum(m for _, m in sub)
            if val > best_val:
                best, best_val = ids, val
        assert set(new_ids) == best, trial
        # invariants
        kept_m = {i: m for i, m in X if i in best and i not in pinned}
        ev_m = [m for i, m in X if i not in best]
        if kept_m and ev_m:
            assert min(kept_m.values()) >= max(ev_m)
        assert status == 0


def test_update_head_shared_pool_is_best_subset_of_summed_mass():
    # head-shared pool: heads hold the same blocks; the kept set must be the
    # best C-subset by the mass summed over heads (brute force), and every
    # head ends with the same pool
    rng = np.random.default_rng(3)
    C, H, W = 4, 3, 6
    for trial in range(20):
        shape, st = small_state(H=H, d=4, T=2, Nq=4, W=W, C=C, win_len=[2] * W,
                                pool_count=4, pool_len=[2] * C, seed=trial)
        st["pool_id"][:] = torch.tensor([3, 9, 14, 20])
        st["win_id"][:] = torch.arange(30, 30 + W)
        mp = rng.random((1, H, C)); mw = rng.random((1, H, W))
        leaving = [1, 2, 4]
        r = po.memory_update(st, mp, mw, leaving, 0, shared_heads=True)
        ids = [3, 9, 14, 20] + [30 + w for w in leaving]
        summed = dict(zip(ids, list(mp[0].sum(0)) + [mw[0, :, w].sum() for w in leaving]))
        best = max(itertools.combinations(ids, C), key=lambda sub: sum(summed[i] for i in sub))
        for h in range(H):
            n = int(r["pool_count"][0, h])
            assert set(r["pool_id"][0, h, :n].tolist()) == set(best), trial
            np.testing.assert_array_equal(r["pool_id"][0, h], r["pool_id"][0, 0])


def test_update_head_shared_pool_with_one_head_is_the_plain_update():
    shape, st = small_state(H=1, d=4, T=2, Nq=4, W=5, C=3, win_len=[2, 2, 0, 2, 1],
                            pool_count=3, pool_len=[2, 2, 2], seed=5)
    rng = np.random.default_rng(1)
    mp = rng.random((1, 1, 3)); mw = rng.random((1, 1, 5))
    a = po.memory_update(st, mp, mw, [0, 1, 3, 4], 0)
    b = po.memory_update(st, mp, mw, [0, 1, 3, 4], 0, shared_heads=True)
    for k in ("pool_id", "pool_count", "pool_len", "k_pool"):
        np.testing.assert_array_equal(a[k], b[k])


def test_update_placement_golden():
    g = _read_golden("update_hand.txt")
    assign, new_ids, status = po.memory_update_one(
        [int(x) for x in g["pool_ids"]], g["pool_mass"], [int(x) for x in g["cand_ids"]],
        g["cand_mass"], int(g["C"][0]), int(g["n_sink"][0]))
    assert new_ids == [int(x) for x in g["new_ids"]]
    assert [s for s, _ in assign] == [int(x) for x in g["admit_slots"]]


def test_update_small_pool_keeps_everything_and_fills_tail():
    assign, new_ids, st = po.memory_update_one([5, 9], [0.1, 0.2], [30, 20, 9], [0.0, 0.5, 0.9], 6, 0)
    # 9 already pooled: not a second candidate; 20 and 30 go to slots 2, 3 by id
    assert new_ids == [5, 9, 20, 30] and assign == [(2, 1), (3, 0)] and st == 0


def test_update_duplicate_leaving_ids_count_once():
    # the same block listed twice among the leaving blocks is one candidate
    assign, new_ids, _ = po.memory_update_one([1], [0.1], [5, 5, 6], [0.9, 0.9, 0.2], 3, 0)
    assert new_ids == [1, 5, 6] and assign == [(1, 0), (2, 2)]


def test_update_ties_and_nan():
    # equal mass: smaller id wins; NaN mass ranks last
    assign, new_ids, _ = po.memory_update_one([7, 3], [0.5, float("nan")], [4, 8], [0.5, 0.5], 2, 0)
    assert sorted(new_ids) == [4, 7]


def test_update_sink_overflow_flag():
    assign, new_ids, st = po.memory_update_one([0, 1], [0.1, 0.1], [2, 50], [0.9, 0.9], 2, 10)
    assert st == po.STATUS_SINK_OVERFLOW and sorted(new_ids) == [0, 1]


def test_update_copies_blocks_bitexactly_and_leaves_survivors():
    shape, st = small_state(B=1, H=2, d=4, T=3, Nq=6, W=4, C=3, pool_count=[3, 1],
                            win_len=[3, 2, 3, 1], pad_value=0.0, seed=8)
    st = po.as_f64_state(st)
    mp = np.array([[[0.9, 0.1, 0.5]], [[0.2, 0.0, 0.0]]]).reshape(1, 2, 3)
    mw = np.array([[[0.3, 0.8, 0.05, 0.7]], [[0.6, 0.1, 0.3, 0.2]]]).reshape(1, 2, 4)
    u = po.memory_update(st, mp, mw, [1, 3], 0)
    # head 0: X = pool{0:.9, 1:.1, 2:.5} + win{1:.8, 3:.7} -> keep .9 .8 .7 ; evict slots 1, 2
    assert u["pool_count"][0, 0] == 3
    np.testing.assert_array_equal(u["k_pool"][0, 0, 0], st["k_pool"][0, 0, 0])
    assert u["admitted"][(0, 0)] == [(1, 1), (2, 3)]
    np.testing.assert_array_equal(u["k_pool"][0, 0, 1], st["k_win"][0, 0, 1])
    np.testing.assert_array_equal(u["v_pool"][0, 0, 2], st["v_win"][0, 0, 3])
    assert u["pool_len"][0, 0, 1] == 2 and u["pool_len"][0, 0, 2] == 1
    # head 1: count 1 + 2 candidates <= C: all kept, candidates to slots 1, 2
    assert u["pool_count"][0, 1] == 3 and u["admitted"][(0, 1)] == [(1, 1), (2, 3)]


# ----------------------------------------------------------------- rollout ---
def test_rollout_dense_limit_is_chunk_causal_attention():
    # k >= window slots and C >= all history blocks: each chunk attends every
    # earlier token plus itself -> textbook attention with a chunk-causal mask
    B, H, d, T, Nq, n_chunks = 1, 2, 8, 4, 10, 5
    qb = po.n_blocks(Nq, T)
    ro = OracleRollout(B, H, d, T, Nq, C=n_chunks * qb, topk=2 * qb, scale=0.35)
    g = torch.Generator().manual_seed(0)
    qs, ks, vs = [], [], []
    for t in range(n_chunks):
        q = torch.randn(B, H, Nq, d, generator=g, dtype=torch.float64)
        k = torch.randn(B, H, Nq, d, generator=g, dtype=torch.float64)
        v = torch.randn(B, H, Nq, d, generator=g, dtype=torch.float64)
        qs.append(q); ks.append(k); vs.append(v)
        out = ro.step(q.numpy(), k.numpy(), v.numpy())
        K = torch.cat(ks, dim=2); V = torch.cat(vs, dim=2)
        ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=0.35)
        np.testing.assert_allclose(out["attn"]["o"], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_rollout_pool_trajectory_and_flat_work():
    # pool fills with the chunk that leaves the window, then saturates; from
    # then on the attended token count per query block is constant
    B, H, d, T, Nq = 1, 1, 4, 4, 10
    qb = po.n_blocks(Nq, T)
    C, k = 5, 2
    ro = OracleRollout(B, H, d, T, Nq, C=C, topk=k, scale=0.5)
    g = np.random.default_rng(0)
    counts, work = [], []
    for t in range(7):
        q, kk, v = (g.standard_normal((B, H, Nq, d)) for _ in range(3))
        out = ro.step(q, kk, v, run_attention=False)
        counts.append(int(out["pool_count_before"][0, 0]))
        pool_tokens = sum(int(ro.pool_len[0, 0, p]) for p in range(int(out["pool_count_before"][0, 0])))
        work.append(int(out["sel_count"].sum()))
    assert counts == [0, 0, 0, qb, C, C, C]
    assert work[0] == 0 and work[1] == qb * min(k, qb) and work[2:] == [qb * k] * 5

"""fp64 oracle of a PBSA streaming rollout (window ring + persistent pool).

TEST INFRASTRUCTURE: used only by the tests and the benchmark's CPU-baseline
leg.  Shares no code with the HIP library or its rollout driver.

Per chunk t of Nq tokens (QB blocks), following the per-chunk flow described
on "Sparse Forcing: Native Trainable Sparse Attention for Real-time
Autoregressive Diffusion Video Generation" (shd-paper.top summary,
"方法详解" / technical framework: select blocks -> sparse attention -> update
the KV cache -> next chunk) and the memory structure of the gist.science/es
explainer (sec. 2, "Arquitectura Propuesta": local sliding window L_t plus a
persistent memory P_t updated by Top-C retention):

  1. select + attention with the current window (chunks t-2 and t-1) and pool;
  2. once the window is full (t >= 2), the blocks of chunk t-2 leave the
     window: Top-C update of the pool with this chunk's block masses;
  3. chunk t's keys/values are written into the window slots chunk t-2 held
     (ring position t mod 2); block ids are t*QB + j.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import pbsa_oracle as po


class OracleRollout:
    def __init__(self, B: int, H: int, d: int, T: int, Nq: int, C: int, topk: int,
                 scale: float, n_sink: int = 0, window_chunks: int = 2):
        self.B, self.H, self.d, self.T, self.Nq, self.C = B, H, d, T, Nq, C
        self.topk, self.scale, self.n_sink = topk, scale, n_sink
        self.QB = po.n_blocks(Nq, T)
        self.window_chunks = window_chunks
        self.W = window_chunks * self.QB
        W = self.W
        self.k_win = np.zeros((B, H, W, T, d)); self.v_win = np.zeros((B, H, W, T, d))
        self.win_len = np.zeros(W, dtype=np.int64); self.win_id = np.full(W, -1, dtype=np.int64)
        self.k_pool = np.zeros((B, H, C, T, d)); self.v_pool = np.zeros((B, H, C, T, d))
        self.pool_len = np.zeros((B, H, C), dtype=np.int64)
        self.pool_id = np.full((B, H, C), -1, dtype=np.int64)
        self.pool_count = np.zeros((B, H), dtype=np.int64)
        self.t = 0

    def ring_slots(self, chunk: int) -> list:
        pos = chunk % self.window_chunks
        return list(range(pos * self.QB, (pos + 1) * self.QB))

    def state(self, q, k, v) -> dict:
        return dict(q=q, k_cur=k, v_cur=v, k_win=self.k_win, v_win=self.v_win,
                    win_len=self.win_len, win_id=self.win_id, k_pool=self.k_pool,
                    v_pool=self.v_pool, pool_len=self.pool_len, pool_id=self.pool_id,
                    pool_count=self.pool_count)

    def step(self, q, k, v, *, sel_override=None, sel_count_override=None,
             mass_override: Optional[tuple] = None, run_attention: bool = True,
             attn_blocks=None) -> dict:
        """One chunk.  ``sel_override``/``mass_override`` (mass_pool, mass_win)
        replace the oracle's own routing (teacher forcing on another
        implementation's decisions, so a tie-band divergence cannot cascade)."""
        st = po.as_f64_state(self.state(q, k, v))
        r = po.select(st, self.topk, self.scale, self.T)
        sel = r["sel"] if sel_override is None else np.asarray(sel_override)
        sel_count = r["sel_count"] if sel_count_override is None else np.asarray(sel_count_override)
        out = dict(select=r, sel=sel, sel_count=sel_count, chunk=self.t,
                   pool_count_before=self.pool_count.copy())
        if run_attention:
            out["attn"] = po.attn_fwd(st, sel, sel_count, self.scale, self.T, blocks=attn_blocks)
        mp, mw = (r["mass_pool"], r["mass_win"]) if mass_override is None else mass_override
        t = self.t
        if t >= self.window_chunks:
            leaving = self.ring_slots(t - self.window_chunks)
            u = po.memory_update(st, mp, mw, leaving, self.n_sink)
            self.k_pool, self.v_pool = u["k_pool"], u["v_pool"]
            self.pool_len, self.pool_id, self.pool_count = u["pool_len"], u["pool_id"], u["pool_count"]
            out["update"] = u
        # ring advance: chunk t takes the slots chunk t - window_chunks held
        kk = st["k_cur"]; vv = st["v_cur"]
        for j, w in enumerate(self.ring_slots(t)):
            rows = po.query_block_rows(self.Nq, self.T, j)
            n = len(rows)
            self.k_win[:, :, w, :n] = kk[:, :, rows.start:rows.stop]
            self.v_win[:, :, w, :n] = vv[:, :, rows.start:rows.stop]
            self.win_len[w] = n
            self.win_id[w] = t * self.QB + j
        self.t += 1
        return out


# ----------------------------------------------------------------------------
# Training through a rollout (R21): the loss sum_t <dO_t, O_t> differentiated
# through every chunk's attention with the routing and pool decisions held
# fixed (stop-gradient, as for the single-chunk backward).  A stored block is
# a copy of rows of the chunk that produced it (R14), so the gradient a pool
# or window slot receives belongs to those rows of that chunk's K/V.
# ----------------------------------------------------------------------------
def _history_rows(x: np.ndarray, ids, Nq: int, T: int, QB: int, b: int, h: int) -> tuple:
    """Rows of the history blocks `ids` (block id c*QB + j = rows
    [j T, min(Nq, (j+1) T)) of chunk c), concatenated, and their
    (chunk, row) origins."""
    rows, origin = [], []
    for x_id in ids:
        c, j = divmod(int(x_id), QB)
        r0, r1 = j * T, min(Nq, (j + 1) * T)
        rows.append(x[c][b, h, r0:r1])
        origin += [(c, r) for r in range(r0, r1)]
    if not rows:
        return np.zeros((0, x[0].shape[-1])), origin
    return np.concatenate(rows, axis=0), origin


def rollout_attention_grads(q: list, k: list, v: list, plans: list, dout: list, scale: float,
                            T: int) -> dict:
    """Gradients of L = sum_t sum_rows <dO_t, O_t> over the chunks of a
    rollout.  q, k, v, dout: per chunk [B,H,Nq,d] arrays; plans[t][b][h][i]:
    the history block ids query block i of chunk t attends (pool blocks and
    selected window blocks); chunk t itself is attended in full.  Returns
    per-chunk dq, dk, dv (fp64) and the outputs o."""
    q = [po._f64(x) for x in q]; k = [po._f64(x) for x in k]
    v = [po._f64(x) for x in v]; dout = [po._f64(x) for x in dout]
    n = len(q)
    B, H, Nq, d = q[0].shape
    QB = po.n_blocks(Nq, T)
    dq = [np.zeros_like(x) for x in q]
    dk = [np.zeros_like(x) for x in k]
    dv = [np.zeros_like(x) for x in v]
    o = [np.zeros_like(x) for x in q]
    for t in range(n):
        for b in range(B):
            for h in range(H):
                for i in range(QB):
                    r0, r1 = i * T, min(Nq, (i + 1) * T)
                    ids = plans[t][b][h][i]
                    Kh, org = _history_rows(k, ids, Nq, T, QB, b, h)
                    Vh, _ = _history_rows(v, ids, Nq, T, QB, b, h)
                    K = np.concatenate([Kh, k[t][b, h]], axis=0)
                    V = np.concatenate([Vh, v[t][b, h]], axis=0)
                    org = org + [(t, r) for r in range(Nq)]
                    Q = q[t][b, h, r0:r1]
                    dO = dout[t][b, h, r0:r1]
                    z = scale * (Q @ K.T)
                    e = np.exp(z - z.max(axis=1, keepdims=True))
                    P = e / e.sum(axis=1, keepdims=True)
                    O = P @ V
                    o[t][b, h, r0:r1] = O
                    Dr = (dO * O).sum(axis=1, keepdims=True)
                    dS = P * (dO @ V.T - Dr)
                    dq[t][b, h, r0:r1] += scale * (dS @ K)
                    dK = scale * (dS.T @ Q)
                    dV = P.T @ dO
                    for u, (c, r) in enumerate(org):
                        dk[c][b, h, r] += dK[u]
                        dv[c][b, h, r] += dV[u]
    return dict(dq=dq, dk=dk, dv=dv, o=o)

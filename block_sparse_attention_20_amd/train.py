"""Training through a streaming rollout (one layer).

The sparse attention of "Sparse Forcing: Native Trainable Sparse Attention
for Real-time Autoregressive Diffusion Video Generation" is trainable
(shd-paper.top summary; gist.science/es explainer, sec. 2): a chunk's queries
attend pool and window blocks that are copies of earlier chunks' keys and
values, so the loss of a rollout reaches those chunks through the cache.

``TrainRollout.forward`` runs the chunks in order through the streaming
driver (select, attention, Top-C update, window append) and records what
each chunk attended: its selection, the pool and window ids, O and LSE.
``backward`` then differentiates sum_t <dO_t, O_t> with every routing and
pool decision held fixed: per chunk it rebuilds the attended pool and window
slots from the kept history (pbsa_block_gather), runs pbsa_attn_bwd, and adds
each slot's gradient to the rows of the chunk that produced the block
(pbsa_grad_scatter) in fp32 accumulators.  Every step runs in libpbsa.so;
the Python code only moves pointers.
"""
from __future__ import annotations

from typing import List

import torch

from . import pbsa as P
from .layer import PBSALayer
from .rollout import Rollout


class TrainRollout:
    def __init__(self, n_chunks: int, B: int, H: int, d: int, T: int, Nq: int, C: int, topk: int,
                 n_sink: int = 0, window_chunks: int = 2, dtype=torch.bfloat16, scale: float = 0.0,
                 device="cuda"):
        self.n = n_chunks
        self.ro = Rollout(1, B, H, d, T, Nq, C, topk, n_sink=n_sink, window_chunks=window_chunks,
                          dtype=dtype, scale=scale, device=device)
        self.L = self.ro.layers[0]
        self.B, self.H, self.d, self.T, self.Nq, self.C = B, H, d, T, Nq, C
        self.QB, self.W = self.ro.QB, self.ro.W
        z = dict(dtype=dtype, device=device)
        self.q_hist = torch.zeros(n_chunks, B, H, Nq, d, **z)
        self.k_hist = torch.zeros(n_chunks, B, H, Nq, d, **z)
        self.v_hist = torch.zeros(n_chunks, B, H, Nq, d, **z)
        self.rec: List[dict] = []
        # the layer the backward rebuilds each chunk's attended state in
        self.D = PBSALayer(B, H, d, T, Nq, self.W, C, topk, dtype=dtype, scale=scale, device=device,
                           ws_fwd=None)
        self.device = device

    def forward(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> torch.Tensor:
        """The next chunk (in order); returns its O (a copy)."""
        t = self.ro.t
        assert t < self.n, "more chunks than the history holds"
        self.q_hist[t].copy_(q)
        self.k_hist[t].copy_(k)
        self.v_hist[t].copy_(v)
        L = self.L
        self.ro.set_inputs(0, q, k, v)
        snap = {n: L.t[n].clone() for n in ("pool_id", "pool_count", "win_id", "win_len")}
        self.ro.run_layer(0)
        snap.update({n: L.t[n].clone() for n in ("sel", "sel_count", "o", "lse")})
        self.rec.append(snap)
        self.ro.advance()
        return snap["o"]

    def backward(self, douts: List[torch.Tensor]):
        """Gradients of sum_t <dO_t, O_t>: dq per chunk (problem dtype) and
        dk, dv for every chunk as fp32 [n_chunks,B,H,Nq,d]."""
        n = len(self.rec)
        gk = torch.zeros(self.n, self.B, self.H, self.Nq, self.d, dtype=torch.float32, device=self.device)
        gv = torch.zeros_like(gk)
        D = self.D
        dq, grads = [], None
        for t in range(n):
            r = self.rec[t]
            for name, src in (("q", self.q_hist[t]), ("k_cur", self.k_hist[t]), ("v_cur", self.v_hist[t]),
                              ("sel", r["sel"]), ("sel_count", r["sel_count"]), ("o", r["o"]),
                              ("lse", r["lse"]), ("win_id", r["win_id"]), ("win_len", r["win_len"]),
                              ("pool_id", r["pool_id"]), ("pool_count", r["pool_count"])):
                D.t[name].copy_(src)
            # the window and pool slots chunk t attended, rebuilt from the history
            if self.W > 0:
                P.pbsa_block_gather(D.prob, r["win_id"], 0, None, self.W, self.k_hist, self.v_hist,
                                    self.n, D.t["k_win"], D.t["v_win"], None)
            if self.C > 0:
                P.pbsa_block_gather(D.prob, r["pool_id"], self.C, r["pool_count"], self.C, self.k_hist,
                                    self.v_hist, self.n, D.t["k_pool"], D.t["v_pool"], D.t["pool_len"])
            grads = D.bwd(douts[t], grads)
            dq.append(grads["dq"].clone())
            cur_ids = torch.arange(t * self.QB, (t + 1) * self.QB, dtype=torch.int64, device=self.device)
            P.pbsa_grad_scatter(D.prob, cur_ids, 0, None, self.QB, 1, grads["dk_cur"], grads["dv_cur"],
                                gk, gv, self.n)
            if self.W > 0:
                P.pbsa_grad_scatter(D.prob, r["win_id"], 0, None, self.W, 0, grads["dk_win"],
                                    grads["dv_win"], gk, gv, self.n)
            if self.C > 0:
                P.pbsa_grad_scatter(D.prob, r["pool_id"], self.C, r["pool_count"], self.C, 0,
                                    grads["dk_pool"], grads["dv_pool"], gk, gv, self.n)
        return dq, gk, gv

    def plans(self) -> list:
        """Per chunk, batch element, head and query block: the history block
        ids attended (pool blocks, then selected window blocks)."""
        out = []
        for r in self.rec:
            pid, pc = r["pool_id"].cpu(), r["pool_count"].cpu()
            sel, sc, wid = r["sel"].cpu(), r["sel_count"].cpu(), r["win_id"].cpu()
            out.append([[[[int(x) for x in pid[b, h, :int(pc[b, h])]] +
                          [int(wid[int(w)]) for w in sel[b, h, i, :int(sc[b, h, i])]]
                          for i in range(self.QB)] for h in range(self.H)] for b in range(self.B)])
        return out

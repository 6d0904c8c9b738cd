"""Streaming rollout driver: chunk after chunk, layer after layer, on one GPU.

The per-chunk flow follows "Sparse Forcing: Native Trainable Sparse
Attention for Real-time Autoregressive Diffusion Video Generation"
(shd-paper.top summary, method details / technical framework: select the
important blocks, run PBSA, update the KV cache, move to the next chunk) with
the memory layout of the gist.science/es explainer (sec. 2 "Arquitectura
Propuesta": a local window of the most recent blocks plus a bounded
persistent memory updated by Top-C retention).

Per layer and chunk t (all device work is libpbsa.so; nothing syncs):
  1. pbsa_select and pbsa_attn_fwd against the window (chunks t-2, t-1) and
     the pool;
  2. once the window is full (t >= window_chunks), pbsa_memory_update with
     the slots of chunk t-2 as the leaving blocks;
  3. pbsa_window_append writes chunk t into those slots (ring position
     t mod window_chunks), block ids t*QB + j.
The state of a layer is plain device tensors (``PBSALayer.t``), so it can be
saved and restored with ``state_dict`` / ``load_state_dict``.
"""
from __future__ import annotations

from typing import List, Optional

import torch

from .layer import PBSALayer

STATE_KEYS = ("k_win", "v_win", "win_len", "win_id", "kbar_win", "k_pool", "v_pool", "pool_len",
              "pool_id", "pool_count", "kbar_pool")


class Rollout:
    def __init__(self, n_layers: int, B: int, H: int, d: int, T: int, Nq: int, C: int, topk: int,
                 n_sink: int = 0, window_chunks: int = 2, dtype=torch.bfloat16, scale: float = 0.0,
                 device="cuda"):
        self.QB = (Nq + T - 1) // T
        self.window_chunks = window_chunks
        self.W = window_chunks * self.QB
        self.n_sink = n_sink
        self.layers: List[PBSALayer] = [
            PBSALayer(B, H, d, T, Nq, self.W, C, topk, dtype=dtype, scale=scale, device=device)
            for _ in range(n_layers)]
        self.leaving = [torch.arange(p * self.QB, (p + 1) * self.QB, dtype=torch.int32, device=device)
                        for p in range(window_chunks)]
        self.t = 0

    def first_slot(self, chunk: int) -> int:
        return (chunk % self.window_chunks) * self.QB

    def set_inputs(self, layer: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
        L = self.layers[layer]
        L.t["q"].copy_(q)
        L.t["k_cur"].copy_(k)
        L.t["v_cur"].copy_(v)

    def run_layer(self, layer: int, attention: bool = True):
        """PBSA work of one layer for the current chunk (inputs already set)."""
        L = self.layers[layer]
        t = self.t
        L.select()
        if attention:
            L.fwd()
        if t >= self.window_chunks:
            L.update(self.leaving[t % self.window_chunks], self.n_sink)
        L.append_window(self.first_slot(t), t * self.QB)

    def run_chunk(self, attention: bool = True):
        for l in range(len(self.layers)):
            self.run_layer(l, attention)
        self.advance()

    def advance(self):
        self.t += 1

    # -- checkpoint / resume ---------------------------------------------------
    def state_dict(self) -> dict:
        return {"t": self.t,
                "layers": [{k: L.t[k].clone() for k in STATE_KEYS} for L in self.layers]}

    def load_state_dict(self, sd: dict):
        self.t = int(sd["t"])
        for L, s in zip(self.layers, sd["layers"]):
            for k in STATE_KEYS:
                L.t[k].copy_(s[k])

    # -- accounting ------------------------------------------------------------
    def attended_tokens(self, layer: int) -> int:
        """Sum over (b, h, query row) of the attended key tokens (sync)."""
        return attended_tokens(self.layers[layer])


def attended_tokens(L: PBSALayer) -> int:
    """Sum over (b, h, query row) of the valid key tokens each row attends:
    pool slots [0, count) + selected window slots + the whole chunk."""
    t = L.t
    T, Nq, QB = L.T, L.Nq, L.QB
    rows = torch.tensor([min(T, Nq - i * T) for i in range(QB)], dtype=torch.int64,
                        device=t["sel"].device)
    cnt = t["pool_count"].long()                                         # [B,H]
    C = L.C
    if C > 0:
        slot = torch.arange(C, device=cnt.device)
        pool_tok = (t["pool_len"].long() * (slot[None, None, :] < cnt[..., None])).sum(-1)  # [B,H]
    else:
        pool_tok = torch.zeros_like(cnt)
    if L.topk > 0 and L.W > 0:
        sel = t["sel"].long()
        valid = (torch.arange(sel.shape[-1], device=sel.device)[None, None, None, :]
                 < t["sel_count"].long()[..., None])
        wl = t["win_len"].long()[sel.clamp(min=0)] * valid
        win_tok = wl.sum(-1)                                             # [B,H,QB]
    else:
        win_tok = torch.zeros(L.B, L.H, QB, dtype=torch.int64, device=cnt.device)
    per_block = pool_tok[..., None] + win_tok + Nq                       # [B,H,QB]
    return int((per_block * rows[None, None, :]).sum().item())

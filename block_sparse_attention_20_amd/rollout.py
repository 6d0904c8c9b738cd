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
  2. once the window is full (t >= window_chunks), the block masses
     (pbsa_block_mass, or inside pbsa_select without a side stream) and
     pbsa_memory_update with the slots of chunk t-2 as the leaving blocks;
  3. pbsa_window_append writes chunk t into those slots (ring position
     t mod window_chunks), block ids t*QB + j.
The state of a layer is plain device tensors (``PBSALayer.t``), so it can be
saved and restored with ``state_dict`` / ``load_state_dict``.

With ``mass="fine"`` the update ranks blocks by their exact attention mass
instead of the coarse mass: the forward of each layer is pbsa_attn_fwd_mass,
which records the masses during its own walk; with
``shared_pool=True`` all heads of a layer keep one pool, ranked by the masses
summed over heads (pbsa_memory_update_shared).

With ``overlap=True`` steps 2-3 go to a side stream: the next layer needs
only this layer's output O, while the masses and the updated pool and window
are needed by the next *chunk*.  The side stream waits for the layer's
forward (the update rewrites pool slots the forward reads); the next chunk's
select of the layer (which rewrites the scores the masses are computed from)
and the next write of its inputs wait for the side work.  Both streams keep
the default priority.  ``side_group`` layers share one launch of side work
(and one event on each stream); every layer's side work is launched by the
time the chunk advances.
"""
from __future__ import annotations

from typing import List, Optional

import torch

from . import pbsa as P
from .layer import PBSALayer

STATE_KEYS = ("k_win", "v_win", "win_len", "win_id", "kbar_win", "k_pool", "v_pool", "pool_len",
              "pool_id", "pool_count", "kbar_pool")


class Rollout:
    def __init__(self, n_layers: int, B: int, H: int, d: int, T: int, Nq: int, C: int, topk: int,
                 n_sink: int = 0, window_chunks: int = 2, dtype=torch.bfloat16, scale: float = 0.0,
                 device="cuda", overlap: bool = False, mass: str = "coarse",
                 shared_pool: bool = False, fused: bool = True, side_group: int = 1):
        if mass not in ("coarse", "fine"):
            raise ValueError(f"mass must be 'coarse' or 'fine', not {mass!r}")
        self.mass = mass
        # select + forward through pbsa_select_attn_fwd (one launch where the
        # problem allows) instead of pbsa_select then pbsa_attn_fwd
        self.fused = fused
        self.shared_pool = shared_pool
        self.QB = (Nq + T - 1) // T
        self.window_chunks = window_chunks
        self.W = window_chunks * self.QB
        self.n_sink = n_sink
        first = PBSALayer(B, H, d, T, Nq, self.W, C, topk, dtype=dtype, scale=scale, device=device)
        # the forwards of all layers run on one stream: one split workspace
        self.layers: List[PBSALayer] = [first] + [
            PBSALayer(B, H, d, T, Nq, self.W, C, topk, dtype=dtype, scale=scale, device=device,
                      ws_fwd=first.ws_fwd)
            for _ in range(n_layers - 1)]
        if mass == "fine":   # one fused forward + mass workspace for all layers (one stream)
            ws = P.workspace(first.prob, P.PBSA_OP_FWD_MASS, device)
            for L in self.layers:
                L.ws_fwd_mass = ws
        self.leaving = [torch.arange(p * self.QB, (p + 1) * self.QB, dtype=torch.int32, device=device)
                        for p in range(window_chunks)]
        self.t = 0
        self.side = torch.cuda.Stream(device=device) if overlap else None
        # side_group: layers whose side work goes to the side stream together,
        # behind one event on each stream (fewer event packets between the
        # forwards on the critical stream)
        if side_group < 1:
            raise ValueError("side_group must be >= 1")
        self.side_group = side_group
        self._pend: List[int] = []       # layers run whose side work is not launched yet
        self._side_ev: List[Optional[torch.cuda.Event]] = [None] * n_layers
        self._attended = [True] * n_layers

    def _wait_side(self, layer: int):
        """The current stream waits for the side work that covers ``layer``
        (and so for every layer launched with it)."""
        if self.side is None:
            return
        if layer in self._pend:
            self._flush_side()
        ev = self._side_ev[layer]
        if ev is not None:
            torch.cuda.current_stream().wait_event(ev)
            for l, e in enumerate(self._side_ev):
                if e is ev:
                    self._side_ev[l] = None

    def _flush_side(self):
        """Launch the side work of the pending layers on the side stream,
        after everything enqueued so far on the current stream."""
        if not self._pend:
            return
        ev_fwd = torch.cuda.Event()
        ev_fwd.record()
        ev_side = torch.cuda.Event()
        with torch.cuda.stream(self.side):
            self.side.wait_event(ev_fwd)
            for l in self._pend:
                self._side_work(self.layers[l], self.t, self._attended[l])
            ev_side.record(self.side)
        for l in self._pend:
            self._side_ev[l] = ev_side
        self._pend = []

    def first_slot(self, chunk: int) -> int:
        return (chunk % self.window_chunks) * self.QB

    def set_inputs(self, layer: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
        self._wait_side(layer)   # the window append still reads k_cur / v_cur
        L = self.layers[layer]
        L.t["q"].copy_(q)
        L.t["k_cur"].copy_(k)
        L.t["v_cur"].copy_(v)

    def run_layer(self, layer: int, attention: bool = True, fwd_events=None):
        """PBSA work of one layer for the current chunk (inputs already set).
        ``fwd_events``: optional (start, end) events recorded around the
        forward launch on the current stream."""
        L = self.layers[layer]
        t = self.t
        self._wait_side(layer)
        fine_now = self.mass == "fine" and t >= self.window_chunks
        fused = self.fused and attention and not fine_now
        # with a side stream the block masses (needed only by the update) are
        # computed there, off the attention's critical path
        if not fused:
            L.select(masses=self.side is None and self.mass == "coarse")
        self._attended[layer] = attention
        if attention:
            if fwd_events is not None:
                fwd_events[0].record()
            if fused:
                L.select_fwd()       # routing + attention, one launch where possible
            elif fine_now:
                L.fwd_mass()         # the update after this chunk ranks by these masses
            else:
                L.fwd()
            if fwd_events is not None:
                fwd_events[1].record()
        if fused and self.side is None and self.mass == "coarse" and t >= self.window_chunks:
            L.block_mass()           # the fused call leaves the masses to block_mass
        if self.side is None:
            self._side_work(L, t, attention)
            return
        self._pend.append(layer)
        if len(self._pend) >= self.side_group or layer == len(self.layers) - 1:
            self._flush_side()

    def _side_work(self, L, t, attended):
        if t >= self.window_chunks:
            if self.mass == "fine" and attended:
                pass                 # pbsa_attn_fwd_mass wrote the masses
            elif self.side is not None or self.mass == "fine":
                L.block_mass()       # coarse masses from the select scores
            L.update(self.leaving[t % self.window_chunks], self.n_sink, shared=self.shared_pool)
        L.append_window(self.first_slot(t), t * self.QB)

    def sync_side(self):
        """Make the current stream wait for every layer's side work."""
        if self.side is not None:
            self._flush_side()
        for l in range(len(self.layers)):
            self._wait_side(l)

    def run_chunk(self, attention: bool = True):
        for l in range(len(self.layers)):
            self.run_layer(l, attention)
        self.advance()

    def advance(self):
        if self.side is not None:
            self._flush_side()   # side work of this chunk's layers, before t moves on
        self.t += 1

    # -- checkpoint / resume ---------------------------------------------------
    def state_dict(self) -> dict:
        self.sync_side()
        return {"t": self.t,
                "layers": [{k: L.t[k].clone() for k in STATE_KEYS} for L in self.layers]}

    def load_state_dict(self, sd: dict):
        self.sync_side()
        self.t = int(sd["t"])
        for L, s in zip(self.layers, sd["layers"]):
            for k in STATE_KEYS:
                L.t[k].copy_(s[k])

    # -- accounting ------------------------------------------------------------
    def attended_tokens(self, layer: int) -> int:
        """Sum over (b, h, query row) of the attended key tokens (sync)."""
        return attended_tokens(self.layers[layer])


def attended_tokens(L: PBSALayer, pool_count=None, pool_len=None, sel=None, sel_count=None) -> int:
    """Sum over (b, h, query row) of the valid key tokens each row attends:
    pool slots [0, count) + selected window slots + the whole chunk.
    ``pool_count`` / ``pool_len`` / ``sel`` / ``sel_count``: the pool and
    routing as a forward saw them, when the layer has moved on since
    (default: the layer's current ones)."""
    t = dict(L.t)
    if pool_count is not None:
        t["pool_count"], t["pool_len"] = pool_count, pool_len
    if sel is not None:
        t["sel"], t["sel_count"] = sel, sel_count
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

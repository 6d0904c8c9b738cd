"""One layer's PBSA state on the device and the calls that drive it.

Host-side bookkeeping only (allocating buffers, marshalling pointers); every
computation is a call into libpbsa.so through ``pbsa.py``.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import pbsa as P

KV_FIELDS = ("k_cur", "v_cur", "k_win", "v_win", "win_len", "win_id", "kbar_win", "k_pool",
             "v_pool", "pool_len", "pool_id", "pool_count", "kbar_pool", "kbar_cur")


class PBSALayer:
    """Device buffers of one layer: current chunk, window ring, pool, pooled
    key caches, routing outputs and attention outputs."""

    def __init__(self, B, H, d, T, Nq, W, C, topk, dtype=torch.bfloat16, scale=0.0,
                 device="cuda", with_status=True, ws_fwd="own"):
        self.B, self.H, self.d, self.T, self.Nq, self.W, self.C, self.topk = B, H, d, T, Nq, W, C, topk
        self.dtype, self.device = dtype, device
        self.QB = (Nq + T - 1) // T
        self.status = torch.zeros(4, dtype=torch.int32, device=device) if with_status else None
        self.prob = P.problem(B, H, d, T, Nq, W, C, topk, P.dtype_code(dtype), scale, self.status)
        z = dict(device=device)
        self.t = {
            "q": torch.zeros(B, H, Nq, d, dtype=dtype, **z),
            "k_cur": torch.zeros(B, H, Nq, d, dtype=dtype, **z),
            "v_cur": torch.zeros(B, H, Nq, d, dtype=dtype, **z),
            "k_win": torch.zeros(B, H, W, T, d, dtype=dtype, **z),
            "v_win": torch.zeros(B, H, W, T, d, dtype=dtype, **z),
            "win_len": torch.zeros(W, dtype=torch.int32, **z),
            "win_id": torch.full((W,), -1, dtype=torch.int64, **z),
            "kbar_win": torch.zeros(B, H, W, d, dtype=torch.float32, **z),
            "k_pool": torch.zeros(B, H, C, T, d, dtype=dtype, **z),
            "v_pool": torch.zeros(B, H, C, T, d, dtype=dtype, **z),
            "pool_len": torch.zeros(B, H, C, dtype=torch.int32, **z),
            "pool_id": torch.full((B, H, C), -1, dtype=torch.int64, **z),
            "pool_count": torch.zeros(B, H, dtype=torch.int32, **z),
            "kbar_pool": torch.zeros(B, H, C, d, dtype=torch.float32, **z),
            "kbar_cur": torch.zeros(B, H, self.QB, d, dtype=torch.float32, **z),
            "sel": torch.zeros(B, H, self.QB, max(topk, 1), dtype=torch.int32, **z),
            "sel_count": torch.zeros(B, H, self.QB, dtype=torch.int32, **z),
            "mass_pool": torch.zeros(B, H, max(C, 1), dtype=torch.float32, **z),
            "mass_win": torch.zeros(B, H, max(W, 1), dtype=torch.float32, **z),
            "o": torch.zeros(B, H, Nq, d, dtype=dtype, **z),
            "lse": torch.zeros(B, H, Nq, dtype=torch.float32, **z),
        }
        self.ws_select = P.workspace(self.prob, P.PBSA_OP_SELECT, device)
        self.ws_update = P.workspace(self.prob, P.PBSA_OP_UPDATE, device)
        self.ws_bwd = P.workspace(self.prob, P.PBSA_OP_BWD, device)
        # forward workspace: "own" allocates one (split launch for few query blocks), None
        # runs one workgroup per query block, a tensor is shared (layers that
        # run one after another on one stream can share it)
        self.ws_fwd = P.workspace(self.prob, P.PBSA_OP_FWD, device) if isinstance(ws_fwd, str) else ws_fwd
        self.ws_fine = None  # allocated on first use of fine_mass()
        self.ws_fwd_mass = None  # allocated on first use of fwd_mass() (or shared, set by the owner)
        self._kv = None

    # -- state ---------------------------------------------------------------
    def load(self, st: dict) -> "PBSALayer":
        """Copy a state dict (tensors on any device) into the layer and
        compute the pooled-key caches of the window and pool slots."""
        for k in ("q", "k_cur", "v_cur", "k_win", "v_win", "win_len", "win_id", "k_pool", "v_pool",
                  "pool_len", "pool_id", "pool_count"):
            if k in st:
                self.t[k].copy_(st[k].to(self.t[k].dtype))
        self.refresh_kbar()
        return self

    @property
    def kv(self) -> P.KV:
        if self._kv is None:
            self._kv = P.make_kv(self.t)
        return self._kv

    def refresh_kbar(self):
        if self.W > 0:
            self._win_lens = self.t["win_len"].repeat(self.B * self.H)  # per stored block
            P.pbsa_block_mean(self.prob, self.t["k_win"], self._win_lens, self.B * self.H * self.W,
                              self.t["kbar_win"])
        if self.C > 0:
            P.pbsa_block_mean(self.prob, self.t["k_pool"], self.t["pool_len"],
                              self.B * self.H * self.C, self.t["kbar_pool"])

    # -- the four calls ------------------------------------------------------
    def select(self, masses: bool = True):
        """Routing; with masses=False the block masses are left to
        block_mass() (which reads the scores this call leaves in ws_select)."""
        t = self.t
        P.pbsa_select(self.prob, t["q"], self.kv, t["sel"] if self.topk > 0 else None,
                      t["sel_count"], t["mass_pool"] if masses and self.C > 0 else None,
                      t["mass_win"] if masses and self.W > 0 else None, self.ws_select)

    def select_fwd(self, with_lse=True):
        """select(masses=False) then fwd() as one call (pbsa_select_attn_fwd):
        one launch where the problem allows, the same results bit for bit."""
        t = self.t
        P.pbsa_select_attn_fwd(self.prob, t["q"], self.kv, t["sel"] if self.topk > 0 else None,
                               t["sel_count"], t["o"], t["lse"] if with_lse else None,
                               self.ws_select, self.ws_fwd)

    def block_mass(self):
        t = self.t
        P.pbsa_block_mass(self.prob, t["mass_pool"] if self.C > 0 else None,
                          t["mass_win"] if self.W > 0 else None, self.ws_select)

    def fine_mass(self, stream=None):
        """Exact block masses from the last fwd's lse (pbsa_fine_mass) into
        mass_pool / mass_win, in place of the coarse ones; the update reads
        whichever was written last."""
        t = self.t
        if self.ws_fine is None:
            self.ws_fine = P.workspace(self.prob, P.PBSA_OP_FINE_MASS, self.device)
        P.pbsa_fine_mass(self.prob, t["q"], self.kv, t["sel"] if self.topk > 0 else None,
                         t["sel_count"], t["lse"], t["mass_pool"] if self.C > 0 else None,
                         t["mass_win"] if self.W > 0 else None, self.ws_fine, stream)

    def fwd(self, with_lse=True):
        t = self.t
        P.pbsa_attn_fwd(self.prob, t["q"], self.kv, t["sel"] if self.topk > 0 else None,
                        t["sel_count"], t["o"], t["lse"] if with_lse else None, self.ws_fwd)

    def fwd_mass(self):
        """Forward plus the exact block masses from the forward's own walk
        (pbsa_attn_fwd_mass) into mass_pool / mass_win."""
        t = self.t
        if self.ws_fwd_mass is None:
            self.ws_fwd_mass = P.workspace(self.prob, P.PBSA_OP_FWD_MASS, self.device)
        P.pbsa_attn_fwd_mass(self.prob, t["q"], self.kv, t["sel"] if self.topk > 0 else None,
                             t["sel_count"], t["o"], t["lse"], t["mass_pool"] if self.C > 0 else None,
                             t["mass_win"] if self.W > 0 else None, self.ws_fwd_mass)

    def bwd(self, dout: torch.Tensor, grads: Optional[dict] = None) -> dict:
        t = self.t
        if grads is None:
            grads = {"dq": torch.empty_like(t["q"])}
            for n in ("k_cur", "v_cur", "k_win", "v_win", "k_pool", "v_pool"):
                grads["d" + n] = torch.empty_like(t[n])
        P.pbsa_attn_bwd(self.prob, t["q"], self.kv, t["sel"] if self.topk > 0 else None,
                        t["sel_count"], t["o"], t["lse"], dout, grads["dq"], P.make_grad(grads),
                        self.ws_bwd)
        return grads

    def update(self, leaving: torch.Tensor, n_sink: int = 0, shared: bool = False):
        """Top-C update; shared=True ranks by the masses summed over heads
        (pbsa_memory_update_shared: one pool for all heads)."""
        t = self.t
        fn = P.pbsa_memory_update_shared if shared else P.pbsa_memory_update
        fn(self.prob, self.kv, t["mass_pool"] if self.C > 0 else None,
           t["mass_win"] if self.W > 0 else None, leaving, leaving.numel(), n_sink, self.ws_update)

    def append_window(self, first_slot: int, first_id: int):
        t = self.t
        P.pbsa_window_append(self.prob, self.kv, t["k_win"], t["v_win"], t["kbar_win"],
                             t["win_len"], t["win_id"], first_slot, first_id)

    def status_bits(self) -> int:
        return 0 if self.status is None else int(self.status[0].item())

"""Seeded synthetic inputs for Persistent Block-Sparse Attention (PBSA).

This module only draws random numbers and lays them out; it contains none of
the method's arithmetic (no pooling, scoring, selection, attention or pool
update).  Both the fp64 oracle (``oracle/``) and the HIP library
(``block_sparse_attention_20_amd``) are fed from here, so the two sides always
consume the same bytes.

Workload shape follows the method description on the pages
"Sparse Forcing: Native Trainable Sparse Attention for Real-time
Autoregressive Diffusion Video Generation" (gist.science/es explainer,
sec. 2 "Observacion Empirica Clave"): a few historical blocks act as
persistent salient anchors.  We mimic that by *planting* salient key blocks:
their keys and every query are shifted by ``shift * u`` along a random unit
direction ``u``, so the planted blocks win the coarse block scoring.

Draw order (fixed, so a seed names one input): u, planted slots, Q, K_cur,
V_cur, K_win, V_win, K_pool, V_pool.  Values are drawn in fp32 (torch's
seeded generator), shifted, and rounded once to the storage dtype (bf16 RNE).
Rows past a block's valid length are padding and hold ``pad_value``
(NaN in poison tests, so a kernel that reads them shows it).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch


@dataclasses.dataclass
class Shape:
    B: int
    H: int
    d: int
    T: int
    Nq: int
    W: int
    C: int
    topk: int
    dtype: torch.dtype = torch.bfloat16

    @property
    def QB(self) -> int:
        return (self.Nq + self.T - 1) // self.T


# Named workloads (sizes from the pages' Wan2.1-T2V-1.3B setting: 12 heads of
# 128, 1560 tokens per latent frame, 3 frames per chunk).
TINY_F32 = Shape(B=1, H=1, d=64, T=64, Nq=256, W=32, C=4, topk=4, dtype=torch.float32)
WAN_CHUNK = Shape(B=1, H=12, d=128, T=128, Nq=4680, W=74, C=32, topk=16)
WAN_TRAIN = Shape(B=2, H=12, d=128, T=128, Nq=4680, W=74, C=32, topk=16)
ROLLOUT_POOL_CAP = 64


def chunk_window_lens(nq: int, t: int, n_chunks: int) -> list:
    """Valid token counts of the window slots holding ``n_chunks`` chunks of
    ``nq`` tokens, each chunk cut into ceil(nq/t) contiguous blocks (the last
    one ragged)."""
    qb = (nq + t - 1) // t
    one = [min(t, nq - j * t) for j in range(qb)]
    return one * n_chunks


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, sigma):
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * sigma


def make_state(
    shape: Shape,
    seed: int,
    *,
    sigma: float = 1.0,
    shift: float = 0.0,
    n_planted: int = 0,
    win_len: Optional[Sequence[int]] = None,
    win_id: Optional[Sequence[int]] = None,
    pool_count: Optional[Sequence[int]] = None,
    pool_len: Optional[Sequence[int]] = None,
    pool_id: Optional[Sequence[int]] = None,
    pad_value: float = 0.0,
    device="cpu",
) -> dict:
    """One layer's inputs: the current chunk (Q, K_cur, V_cur), the window
    ring slots and the persistent pool.

    Defaults: every window slot full (len T); pool full (count C), every pool
    block full; block ids are non-negative, pool ids 0..C-1 (older) and window
    ids C..C+W-1.
    ``pool_count``/``pool_len``/``pool_id`` may be given per (b, h) flattened
    or as a single value broadcast to every head.
    """
    B, H, d, T, Nq, W, C = shape.B, shape.H, shape.d, shape.T, shape.Nq, shape.W, shape.C
    g = _gen(seed, device)
    wl = torch.tensor(list(win_len) if win_len is not None else [T] * W, dtype=torch.int32)
    wi = torch.tensor(list(win_id) if win_id is not None else list(range(C, C + W)),
                      dtype=torch.int64)
    assert wl.numel() == W and wi.numel() == W

    def per_head(v, default, dt, extra=()):
        if v is None:
            v = default
        t = torch.tensor(v, dtype=dt)
        full = (B, H) + tuple(extra)
        if t.numel() == 1:
            return t.reshape(()).expand(full).clone()
        if t.numel() == int(torch.tensor(full).prod()):
            return t.reshape(full).clone()
        if extra and t.numel() == extra[0]:
            return t.reshape(1, 1, -1).expand(full).clone()
        raise ValueError("bad per-head array size")

    pc = per_head(pool_count, C, torch.int32)
    pl = per_head(pool_len, T, torch.int32, (C,))
    pid = per_head(pool_id, list(range(C)), torch.int64, (C,))

    # 1. direction shared by the planted keys and the queries
    u = torch.randn(d, generator=g, device=device, dtype=torch.float32)
    u = u / u.norm()
    # 2. planted window slots: distinct, full
    full_slots = [w for w in range(W) if int(wl[w]) == T]
    planted = []
    if n_planted > 0:
        assert n_planted <= len(full_slots)
        perm = torch.randperm(len(full_slots), generator=g, device=device).cpu().tolist()
        planted = sorted(full_slots[j] for j in perm[:n_planted])
    # 3. tensors
    q = _randn((B, H, Nq, d), g, device, sigma)
    k_cur = _randn((B, H, Nq, d), g, device, sigma)
    v_cur = _randn((B, H, Nq, d), g, device, sigma)
    k_win = _randn((B, H, W, T, d), g, device, sigma)
    v_win = _randn((B, H, W, T, d), g, device, sigma)
    k_pool = _randn((B, H, C, T, d), g, device, sigma)
    v_pool = _randn((B, H, C, T, d), g, device, sigma)
    if shift != 0.0:
        q += shift * u
        for w in planted:
            k_win[:, :, w] += shift * u
    # padding rows
    wl_d = wl.to(device)
    tok = torch.arange(T, device=device)
    wpad = (tok[None, :] >= wl_d[:, None])  # [W,T]
    k_win[:, :, wpad] = pad_value
    v_win[:, :, wpad] = pad_value
    ppad = (tok[None, None, None, :] >= pl.to(device)[..., None])  # [B,H,C,T]
    k_pool[ppad] = pad_value
    v_pool[ppad] = pad_value
    dt = shape.dtype
    return dict(
        q=q.to(dt), k_cur=k_cur.to(dt), v_cur=v_cur.to(dt),
        k_win=k_win.to(dt), v_win=v_win.to(dt),
        win_len=wl.to(device), win_id=wi.to(device),
        k_pool=k_pool.to(dt), v_pool=v_pool.to(dt),
        pool_len=pl.to(device), pool_id=pid.to(device), pool_count=pc.to(device),
        planted=planted, u=u,
    )


def make_dout(shape: Shape, seed: int, sigma: float = 1.0, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return _randn((shape.B, shape.H, shape.Nq, shape.d), g, device, sigma).to(shape.dtype)


def make_chunk(shape: Shape, seed: int, u: torch.Tensor, *, sigma: float, shift: float,
               n_planted: int, device="cpu") -> dict:
    """One new chunk of a streaming rollout: Q, K, V of Nq tokens.  ``n_planted``
    of its full blocks get their keys shifted by ``shift*u``; every query is
    shifted too.  The planted blocks become salient window/pool blocks later."""
    B, H, d, T, Nq = shape.B, shape.H, shape.d, shape.T, shape.Nq
    g = _gen(seed, device)
    qb = shape.QB
    full_blocks = [j for j in range(qb) if min(T, Nq - j * T) == T]
    planted = []
    if n_planted > 0:
        perm = torch.randperm(len(full_blocks), generator=g, device=device).cpu().tolist()
        planted = sorted(full_blocks[j] for j in perm[:n_planted])
    q = _randn((B, H, Nq, d), g, device, sigma)
    k = _randn((B, H, Nq, d), g, device, sigma)
    v = _randn((B, H, Nq, d), g, device, sigma)
    if shift != 0.0:
        q += shift * u.to(device)
        for j in planted:
            k[:, :, j * T:(j + 1) * T] += shift * u.to(device)
    dt = shape.dtype
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), planted=planted)


def rollout_direction(config_id: int, layer: int, chunk: int, d: int, redraw_every: int = 8,
                      device="cpu") -> torch.Tensor:
    """Unit direction for the planted saliency of a rollout; re-drawn every
    ``redraw_every`` chunks (the salient content drifts slowly)."""
    g = _gen(config_id * 10**6 + layer * 10**3 + 900 + chunk // redraw_every, device)
    u = torch.randn(d, generator=g, device=device, dtype=torch.float32)
    return u / u.norm()


def rollout_seed(config_id: int, layer: int, chunk: int) -> int:
    return config_id * 10**6 + layer * 10**3 + chunk


def wan_chunk_state(layer: int, device="cpu", pad_value: float = 0.0, shape: Shape = WAN_CHUNK,
                    unscaled: bool = False) -> dict:
    """The Wan2.1-1.3B-shaped chunk: 12 heads x 128, 4680-token chunk in 37
    blocks of 128 (last block 72 tokens), a window of the two previous chunks
    (74 slots, two of them ragged), a full pool of 32 blocks, top-16.
    Values N(0,1)/sqrt(128) (N(0,1) when ``unscaled``); 8 planted full window
    blocks get +1.5 along the shared direction.  Layer l uses seed 1000+l."""
    sigma = 1.0 if unscaled else 1.0 / math.sqrt(shape.d)
    wl = chunk_window_lens(shape.Nq, shape.T, 2)
    assert len(wl) == shape.W
    return make_state(shape, 1000 + layer, sigma=sigma, shift=1.5, n_planted=8,
                      win_len=wl, win_id=list(range(2 * shape.QB, 4 * shape.QB)),
                      pool_id=list(range(0, shape.C)), pad_value=pad_value, device=device)


def tiny_f32_state(device="cpu", pad_value: float = 0.0) -> dict:
    """The tiny fp32 case: 1 head, d=64, blocks of 64, a 256-token chunk,
    a 32-block window, a pool of 4, top-4; N(0,1) with 2 planted window
    blocks at +2.0.  Seed 0."""
    return make_state(TINY_F32, 0, sigma=1.0, shift=2.0, n_planted=2, pad_value=pad_value,
                      device=device)

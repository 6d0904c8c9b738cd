"""ctypes binding of the PBSA C ABI (include/pbsa.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every computation runs in the HIP kernels of libpbsa.so.
The functions keep the C names and raise ``PBSAError`` on a non-zero status.
There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpbsa.so")

PBSA_BF16, PBSA_F32 = 0, 1
PBSA_OP_SELECT, PBSA_OP_FWD, PBSA_OP_BWD, PBSA_OP_UPDATE, PBSA_OP_FINE_MASS = 0, 1, 2, 3, 4
PBSA_OP_FWD_MASS = 5
PBSA_STATUS_POOL_COUNT, PBSA_STATUS_WIN_LEN, PBSA_STATUS_SEL, PBSA_STATUS_SINK = 1, 2, 4, 8
(PBSA_OK, PBSA_ERR_NULL, PBSA_ERR_SHAPE, PBSA_ERR_DTYPE, PBSA_ERR_ALIGN, PBSA_ERR_WORKSPACE,
 PBSA_ERR_HIP, PBSA_ERR_UNSUPPORTED) = 0, -1, -2, -3, -4, -5, -6, -7
PBSA_STATUS_SHARED = 16

# every exported symbol declared in include/pbsa.h
EXPORTS = ("pbsa_select", "pbsa_select_static", "pbsa_block_mass", "pbsa_attn_fwd",
           "pbsa_attn_fwd_mass", "pbsa_select_attn_fwd", "pbsa_attn_bwd", "pbsa_memory_update",
           "pbsa_fine_mass", "pbsa_memory_update_shared", "pbsa_block_gather", "pbsa_grad_scatter",
           "pbsa_block_mean", "pbsa_window_append", "pbsa_workspace_size", "pbsa_validate",
           "pbsa_strerror", "pbsa_last_error")


class PBSAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"PBSA error {code}: {msg}")
        self.code = code


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
                ("T", ctypes.c_int32), ("Nq", ctypes.c_int32), ("W", ctypes.c_int32),
                ("C", ctypes.c_int32), ("topk", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dev_status", ctypes.c_void_p)]

    @property
    def QB(self) -> int:
        return (self.Nq + self.T - 1) // self.T


class KV(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "k_cur", "v_cur", "k_win", "v_win", "win_len", "win_id", "kbar_win", "k_pool", "v_pool",
        "pool_len", "pool_id", "pool_count", "kbar_pool", "kbar_cur")]


class KVGrad(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "dk_cur", "dv_cur", "dk_win", "dv_win", "dk_pool", "dv_pool")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libpbsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise PBSAError(-6, f"{LIB_PATH} is missing: build it first "
                                "(python -m block_sparse_attention_20_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        P, K, G = ctypes.POINTER(Problem), ctypes.POINTER(KV), ctypes.POINTER(KVGrad)
        sig = {
            "pbsa_select": (ctypes.c_int, [P, vp, K, vp, vp, vp, vp, vp, sz, vp]),
            "pbsa_select_static": (ctypes.c_int, [P, vp, K, vp, vp, vp, vp, vp]),
            "pbsa_block_mass": (ctypes.c_int, [P, vp, vp, vp, sz, vp]),
            "pbsa_attn_fwd": (ctypes.c_int, [P, vp, K, vp, vp, vp, vp, vp, sz, vp]),
            "pbsa_attn_fwd_mass": (ctypes.c_int, [P, vp, K, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "pbsa_select_attn_fwd": (ctypes.c_int, [P, vp, K, vp, vp, vp, vp, vp, sz, vp, sz, vp]),
            "pbsa_attn_bwd": (ctypes.c_int, [P, vp, K, vp, vp, vp, vp, vp, vp, G, vp, sz, vp]),
            "pbsa_memory_update": (ctypes.c_int, [P, K, vp, vp, vp, i32, i64, vp, sz, vp]),
            "pbsa_fine_mass": (ctypes.c_int, [P, vp, K, vp, vp, vp, vp, vp, vp, sz, vp]),
            "pbsa_memory_update_shared": (ctypes.c_int, [P, K, vp, vp, vp, i32, i64, vp, sz, vp]),
            "pbsa_block_gather": (ctypes.c_int, [P, vp, i64, vp, i32, vp, vp, i32, vp, vp, vp, vp]),
            "pbsa_grad_scatter": (ctypes.c_int, [P, vp, i64, vp, i32, i32, vp, vp, vp, vp, i32, vp]),
            "pbsa_block_mean": (ctypes.c_int, [P, vp, vp, i64, vp, vp]),
            "pbsa_window_append": (ctypes.c_int, [P, K, vp, vp, vp, vp, vp, i32, i64, vp]),
            "pbsa_workspace_size": (sz, [P, ctypes.c_int]),
            "pbsa_validate": (ctypes.c_int, [P, ctypes.c_int]),
            "pbsa_strerror": (ctypes.c_char_p, [ctypes.c_int]),
            "pbsa_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != 0:
        L = lib()
        raise PBSAError(rc, f"{L.pbsa_strerror(rc).decode()}: {L.pbsa_last_error().decode()}")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    return torch.cuda.current_stream().cuda_stream


def problem(B, H, d, T, Nq, W, C, topk, dtype=PBSA_BF16, scale=0.0, dev_status=None) -> Problem:
    return Problem(B, H, d, T, Nq, W, C, topk, dtype, float(scale), _p(dev_status))


def dtype_code(t: torch.dtype) -> int:
    return {torch.bfloat16: PBSA_BF16, torch.float32: PBSA_F32}[t]


def make_kv(st: dict) -> KV:
    """KV struct from a dict of tensors (missing entries become NULL)."""
    return KV(*[_p(st.get(n)) for n, _ in KV._fields_])


def make_grad(g: dict) -> KVGrad:
    return KVGrad(*[_p(g.get(n)) for n, _ in KVGrad._fields_])


# --- the C entry points --------------------------------------------------------
def pbsa_workspace_size(prob: Problem, op: int) -> int:
    return int(lib().pbsa_workspace_size(ctypes.byref(prob), op))


def pbsa_validate(prob: Problem, op: int) -> int:
    return int(lib().pbsa_validate(ctypes.byref(prob), op))


def pbsa_select(prob, q, kv: KV, sel, sel_count, mass_pool, mass_win, ws, stream=None):
    _check(lib().pbsa_select(ctypes.byref(prob), _p(q), ctypes.byref(kv), _p(sel), _p(sel_count),
                             _p(mass_pool), _p(mass_win), _p(ws),
                             0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def pbsa_select_static(prob, q, kv: KV, sel, sel_count, mass_pool, mass_win, stream=None):
    _check(lib().pbsa_select_static(ctypes.byref(prob), _p(q), ctypes.byref(kv), _p(sel),
                                    _p(sel_count), _p(mass_pool), _p(mass_win), _stream(stream)))


def pbsa_attn_fwd(prob, q, kv: KV, sel, sel_count, o, lse, ws=None, stream=None):
    _check(lib().pbsa_attn_fwd(ctypes.byref(prob), _p(q), ctypes.byref(kv), _p(sel), _p(sel_count),
                               _p(o), _p(lse), _p(ws),
                               0 if ws is None else ws.numel() * ws.element_size(),
                               _stream(stream)))


def pbsa_select_attn_fwd(prob, q, kv: KV, sel, sel_count, o, lse, ws, fwd_ws=None, stream=None):
    _check(lib().pbsa_select_attn_fwd(ctypes.byref(prob), _p(q), ctypes.byref(kv), _p(sel),
                                      _p(sel_count), _p(o), _p(lse), _p(ws),
                                      0 if ws is None else ws.numel() * ws.element_size(),
                                      _p(fwd_ws),
                                      0 if fwd_ws is None else fwd_ws.numel() * fwd_ws.element_size(),
                                      _stream(stream)))


def pbsa_attn_fwd_mass(prob, q, kv: KV, sel, sel_count, o, lse, mass_pool, mass_win, ws,
                       stream=None):
    _check(lib().pbsa_attn_fwd_mass(ctypes.byref(prob), _p(q), ctypes.byref(kv), _p(sel),
                                    _p(sel_count), _p(o), _p(lse), _p(mass_pool), _p(mass_win),
                                    _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream)))


def pbsa_attn_bwd(prob, q, kv: KV, sel, sel_count, o, lse, dout, dq, grad: KVGrad, ws,
                  stream=None):
    _check(lib().pbsa_attn_bwd(ctypes.byref(prob), _p(q), ctypes.byref(kv), _p(sel),
                               _p(sel_count), _p(o), _p(lse), _p(dout), _p(dq),
                               ctypes.byref(grad), _p(ws),
                               0 if ws is None else ws.numel() * ws.element_size(),
                               _stream(stream)))


def pbsa_memory_update(prob, kv: KV, mass_pool, mass_win, leaving, n_leave, n_sink, ws,
                       stream=None):
    _check(lib().pbsa_memory_update(ctypes.byref(prob), ctypes.byref(kv), _p(mass_pool),
                                    _p(mass_win), _p(leaving), int(n_leave), int(n_sink), _p(ws),
                                    0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream)))


def pbsa_fine_mass(prob, q, kv: KV, sel, sel_count, lse, mass_pool, mass_win, ws, stream=None):
    _check(lib().pbsa_fine_mass(ctypes.byref(prob), _p(q), ctypes.byref(kv), _p(sel), _p(sel_count),
                                _p(lse), _p(mass_pool), _p(mass_win), _p(ws),
                                0 if ws is None else ws.numel() * ws.element_size(),
                                _stream(stream)))


def pbsa_memory_update_shared(prob, kv: KV, mass_pool, mass_win, leaving, n_leave, n_sink, ws,
                              stream=None):
    _check(lib().pbsa_memory_update_shared(ctypes.byref(prob), ctypes.byref(kv), _p(mass_pool),
                                           _p(mass_win), _p(leaving), int(n_leave), int(n_sink),
                                           _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                           _stream(stream)))


def pbsa_block_gather(prob, ids, ids_bh_stride, count, n_slots, k_hist, v_hist, n_chunks, k_out,
                      v_out, len_out=None, stream=None):
    _check(lib().pbsa_block_gather(ctypes.byref(prob), _p(ids), int(ids_bh_stride), _p(count),
                                   int(n_slots), _p(k_hist), _p(v_hist), int(n_chunks), _p(k_out),
                                   _p(v_out), _p(len_out), _stream(stream)))


def pbsa_grad_scatter(prob, ids, ids_bh_stride, count, n_slots, src_is_chunk, dk, dv, gk, gv,
                      n_chunks, stream=None):
    _check(lib().pbsa_grad_scatter(ctypes.byref(prob), _p(ids), int(ids_bh_stride), _p(count),
                                   int(n_slots), int(src_is_chunk), _p(dk), _p(dv), _p(gk), _p(gv),
                                   int(n_chunks), _stream(stream)))


def pbsa_block_mass(prob, mass_pool, mass_win, ws, stream=None):
    _check(lib().pbsa_block_mass(ctypes.byref(prob), _p(mass_pool), _p(mass_win), _p(ws),
                                 0 if ws is None else ws.numel() * ws.element_size(),
                                 _stream(stream)))


def pbsa_block_mean(prob, x, length, n_blocks, out, stream=None):
    _check(lib().pbsa_block_mean(ctypes.byref(prob), _p(x), _p(length), int(n_blocks), _p(out),
                                 _stream(stream)))


def pbsa_window_append(prob, kv: KV, k_win, v_win, kbar_win, win_len, win_id, first_slot,
                       first_id, stream=None):
    _check(lib().pbsa_window_append(ctypes.byref(prob), ctypes.byref(kv), _p(k_win), _p(v_win),
                                    _p(kbar_win), _p(win_len), _p(win_id), int(first_slot),
                                    int(first_id), _stream(stream)))


def workspace(prob: Problem, op: int, device="cuda") -> Optional[torch.Tensor]:
    n = pbsa_workspace_size(prob, op)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device) if n > 0 else None

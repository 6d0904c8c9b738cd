"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and host-side validation returns the documented codes before
anything is launched (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_20_amd import pbsa as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pbsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(P.LIB_PATH),
                                reason="libpbsa.so not built (run __graft_entry__.build())")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pbsa_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert set(names) == set(P.EXPORTS), names
    L = P.lib()
    for n in names:
        assert hasattr(L, n), n


def test_header_compiles_as_plain_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "pbsa.h"\nint main(void){pbsa_problem p; (void)p; return 0;}\n')
    import subprocess
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                        "-c", str(src), "-o", str(tmp_path / "t.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def wan():
    return P.problem(1, 12, 128, 128, 4680, 74, 32, 16, P.PBSA_BF16)


@pytest.mark.parametrize("field,value,code", [
    ("dtype", 7, -3), ("B", 0, -2), ("H", 0, -2), ("Nq", 0, -2), ("W", 2000, -2),
    ("C", -1, -2), ("topk", 75, -2), ("topk", -1, -2), ("d", 96, -7), ("T", 32, -7),
    ("scale", -1.0, -2), ("scale", float("inf"), -2),
])
def test_validate_codes(field, value, code):
    p = wan()
    assert P.pbsa_validate(p, P.PBSA_OP_FWD) == 0
    setattr(p, field, value)
    assert P.pbsa_validate(p, P.PBSA_OP_FWD) == code
    assert P.lib().pbsa_last_error().decode() != ""


def test_validate_select_size_limit():
    p = P.problem(1, 1, 128, 64, 64 * 12000, 10, 10, 2, P.PBSA_BF16)
    assert P.pbsa_validate(p, P.PBSA_OP_SELECT) == -2
    assert P.pbsa_validate(p, P.PBSA_OP_FWD) == 0


def test_workspace_sizes():
    p = wan()
    # forward: optional split workspace - partial O^T (fp32, 64 per thread)
    # and (max, sum) for each of at most 512 pieces of 256 threads
    ws_fwd = P.pbsa_workspace_size(p, P.PBSA_OP_FWD)
    assert ws_fwd >= 512 * 256 * 64 * 4 + 512 * 256 * 2 * 4
    # the fp32 path splits the same way, with the same partial layout
    f32 = wan(); f32.dtype = P.PBSA_F32
    assert P.pbsa_workspace_size(f32, P.PBSA_OP_FWD) == ws_fwd
    ws_sel = P.pbsa_workspace_size(p, P.PBSA_OP_SELECT)
    # qbar [12,37,128] f32 + per-row softmax [12,37,106] f32, 256-byte aligned
    assert ws_sel >= 12 * 37 * 128 * 4 + 12 * 37 * 106 * 4
    assert P.pbsa_workspace_size(p, P.PBSA_OP_UPDATE) >= 2 * 12 * 32 * 4 + 12 * 4
    bad = wan(); bad.d = 96
    assert P.pbsa_workspace_size(bad, P.PBSA_OP_SELECT) == 0
    # fine mass: one fp32 partial sum per (b, h, query block, wave slot, entry)
    assert P.pbsa_workspace_size(p, P.PBSA_OP_FINE_MASS) >= 12 * 37 * 4 * (32 + 16) * 4
    assert P.pbsa_validate(p, P.PBSA_OP_FINE_MASS) == 0
    assert P.pbsa_validate(p, P.PBSA_OP_FWD_MASS) == 0
    assert P.pbsa_validate(p, P.PBSA_OP_FWD_MASS + 1) == -2
    # fused forward + exact mass: one log-sum-exp per (row, scored entry), then
    # the forward's split workspace
    assert P.pbsa_workspace_size(p, P.PBSA_OP_FWD_MASS) >= 12 * 37 * 48 * 128 * 4 + ws_fwd


def test_entry_points_reject_before_launch():
    """Every entry point validates on the host and returns without touching
    the device (these calls are safe without a GPU)."""
    L = P.lib()
    p = wan()
    kv = P.KV()
    # NULL problem / q / kv fields
    assert L.pbsa_attn_fwd(None, None, ctypes.byref(kv), None, None, None, None, None, 0, None) == -1
    assert L.pbsa_attn_fwd(ctypes.byref(p), None, ctypes.byref(kv), None, None, None, None, None, 0, None) == -1
    fake = 0x10000  # never dereferenced: validation fails first
    kv2 = P.KV(*([fake] * 14))
    assert L.pbsa_attn_fwd(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, None, None, None, 0, None) == -1
    assert "o" in L.pbsa_last_error().decode()
    # misaligned pointer
    assert L.pbsa_attn_fwd(ctypes.byref(p), fake + 2, ctypes.byref(kv2), fake, fake, fake, None, None, 0, None) == -4
    # select: masses are optional only as a pair
    need = L.pbsa_workspace_size(ctypes.byref(p), P.PBSA_OP_SELECT)
    assert L.pbsa_select(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, fake, None, fake, need, None) == -1
    assert L.pbsa_select(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, None, fake, fake, need, None) == -1
    # block mass: both mass buffers and the select workspace
    assert L.pbsa_block_mass(ctypes.byref(p), None, fake, fake, need, None) == -1
    assert L.pbsa_block_mass(ctypes.byref(p), fake, None, fake, need, None) == -1
    assert L.pbsa_block_mass(ctypes.byref(p), fake, fake, None, 0, None) == -5
    assert L.pbsa_block_mass(ctypes.byref(p), fake, fake, fake, need - 1, None) == -5
    # select without workspace
    assert L.pbsa_select(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, fake, fake, None, 0, None) == -5
    need = L.pbsa_workspace_size(ctypes.byref(p), P.PBSA_OP_SELECT)
    assert L.pbsa_select(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, fake, fake, fake, need - 1, None) == -5
    # allocation-free select: same checks, and problems whose select
    # workspace exceeds the static scratch are refused before any launch
    assert L.pbsa_select_static(ctypes.byref(p), fake, ctypes.byref(kv2), fake, None, fake, fake, None) == -1
    big = P.problem(1, 256, 128, 128, 128 * 64, 0, 64, 0, P.PBSA_BF16)
    assert L.pbsa_workspace_size(ctypes.byref(big), P.PBSA_OP_SELECT) > 8 << 20
    assert L.pbsa_select_static(ctypes.byref(big), fake, ctypes.byref(kv2), None, fake, fake, None, None) == -5
    assert "static scratch" in L.pbsa_last_error().decode()
    # update: n_leave out of range, negative n_sink
    assert L.pbsa_memory_update(ctypes.byref(p), ctypes.byref(kv2), fake, fake, fake, 75, 0, fake, 1 << 20, None) == -2
    assert L.pbsa_memory_update(ctypes.byref(p), ctypes.byref(kv2), fake, fake, fake, 37, -1, fake, 1 << 20, None) == -2
    # window append outside the ring
    assert L.pbsa_window_append(ctypes.byref(p), ctypes.byref(kv2), fake, fake, fake, fake, fake, 40, 0, None) == -2
    # bwd needs every gradient buffer
    g = P.KVGrad()
    assert L.pbsa_attn_bwd(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, fake, fake, fake, fake,
                           ctypes.byref(g), fake, 1 << 30, None) == -1
    # fine mass: lse and both mass buffers required, workspace sized
    need = L.pbsa_workspace_size(ctypes.byref(p), P.PBSA_OP_FINE_MASS)
    assert L.pbsa_fine_mass(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, None, fake, fake, fake,
                            need, None) == -1
    assert L.pbsa_fine_mass(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, fake, None, fake, fake,
                            need, None) == -1
    assert L.pbsa_fine_mass(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, fake, fake, fake, fake,
                            need - 1, None) == -5
    # select + forward in one call: o and the select workspace required,
    # an optional forward workspace must be aligned
    need = L.pbsa_workspace_size(ctypes.byref(p), P.PBSA_OP_SELECT)
    assert L.pbsa_select_attn_fwd(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, None, fake,
                                  fake, need, None, 0, None) == -1
    assert L.pbsa_select_attn_fwd(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, fake, fake,
                                  None, 0, None, 0, None) == -5
    assert L.pbsa_select_attn_fwd(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, fake, fake,
                                  fake, need - 1, None, 0, None) == -5
    assert L.pbsa_select_attn_fwd(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, fake, fake,
                                  fake, need, fake + 8, 1 << 30, None) == -4
    assert L.pbsa_select_attn_fwd(ctypes.byref(p), fake, ctypes.byref(kv2), None, fake, fake, fake,
                                  fake, need, None, 0, None) == -1
    # fused forward + mass: lse, both mass buffers and the workspace required
    need = L.pbsa_workspace_size(ctypes.byref(p), P.PBSA_OP_FWD_MASS)
    assert L.pbsa_attn_fwd_mass(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, fake, None, fake,
                                fake, fake, need, None) == -1
    assert L.pbsa_attn_fwd_mass(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, fake, fake, None,
                                fake, fake, need, None) == -1
    assert L.pbsa_attn_fwd_mass(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, fake, fake, fake,
                                fake, fake, need - 1, None) == -5
    assert L.pbsa_attn_fwd_mass(ctypes.byref(p), fake, ctypes.byref(kv2), fake, fake, fake, fake, fake,
                                fake, None, 0, None) == -5
    # gather / scatter: slot counts, id strides, chunk counts, required pointers
    assert L.pbsa_block_gather(ctypes.byref(p), fake, 0, None, 70000, fake, fake, 2, fake, fake, None, None) == -2
    assert L.pbsa_block_gather(ctypes.byref(p), fake, 3, None, 4, fake, fake, 2, fake, fake, None, None) == -2
    assert L.pbsa_block_gather(ctypes.byref(p), fake, 0, None, 4, fake, fake, 0, fake, fake, None, None) == -2
    assert L.pbsa_block_gather(ctypes.byref(p), None, 0, None, 4, fake, fake, 2, fake, fake, None, None) == -1
    assert L.pbsa_grad_scatter(ctypes.byref(p), fake, 0, None, 4, 2, fake, fake, fake, fake, 2, None) == -2
    assert L.pbsa_grad_scatter(ctypes.byref(p), fake, 0, None, 4, 0, fake, fake, None, fake, 2, None) == -1
    # the backward is bf16 only, refused on the host
    f32 = wan(); f32.dtype = P.PBSA_F32
    assert L.pbsa_attn_bwd(ctypes.byref(f32), fake, ctypes.byref(kv2), fake, fake, fake, fake, fake, fake,
                           ctypes.byref(g), fake, 1 << 30, None) == -7
    assert L.pbsa_strerror(-5).decode().startswith("workspace")

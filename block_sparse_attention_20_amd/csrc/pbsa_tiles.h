// LDS tile staging shared by the PBSA attention kernels (gfx950).
#pragma once

#include "pbsa_common.h"

namespace pbsa {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// s_waitcnt immediate: vmcnt <= n, expcnt and lgkmcnt unconstrained (gfx9 encoding)
#define PBSA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14)))

// LDS swizzles (gfx950 LDS: 64 banks of 4 bytes; a 16-byte read serves 16
// lanes per cycle, an 8-byte read 32 lanes).  Rows are 16-byte chunks; the
// physical chunk of logical chunk c in row r is c ^ swz(r).
//  K (read as MFMA A rows: 16 consecutive rows, one chunk each):
//    d = 128: r & 15 (16 distinct chunks); d = 64: (r >> 1) & 7 with two rows
//    per 256-byte bank line.
//  V (read with ds_read_b64_tr_b16: 4 consecutive rows x 64 bytes per 32
//    lanes): d = 128: 4 (r & 3) moves each row's 64-byte group to its own
//    quarter of the bank line; d = 64: 2 (r & 3).
//  U (read both ways: 16 consecutive rows of one chunk, and 4 rows x 4
//    chunks): d = 128: the two 2-bit halves of r & 15 swapped; d = 64:
//    ((r >> 1) & 1) << 2 | ((r >> 2) & 3).
enum { kSwzK = 0, kSwzV = 1, kSwzU = 2 };

template <int D, int MODE>
__device__ __forceinline__ int lds_swz(int r) {
  if constexpr (MODE == kSwzV) return D == 128 ? 4 * (r & 3) : 2 * (r & 3);
  else if constexpr (MODE == kSwzK) return D == 128 ? (r & 15) : ((r >> 1) & 7);
  else return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Stage one [BT][D] bf16 tile (rows >= valid read as zeros) into LDS,
// swizzled as above.  Each wave moves IPW chunks of 1 KB with
// buffer_load_dwordx4 ... lds (lane l lands at base + 16 l), so the whole
// tile is in flight without touching VGPRs.  The source is a buffer
// descriptor over the tile's valid rows only: a lane whose row is past the
// end is out of range and writes zeros, so padding rows never reach the
// MFMAs (and NaN padding in HBM cannot leak).  Instruction `it` of a wave
// covers rows row0 + it*RPI + lane/CPR; every wave's first row is a multiple
// of 16, so a lane's offset within its 16-row band repeats every 16/RPI
// instructions: dma_lane_offsets() computes those few byte offsets once, and
// each band gets its own descriptor (group), so the per-instruction offset
// is a fixed VGPR and the rest is scalar.
template <int D, int BT, int NW>
struct DmaGeom {
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;          // rows per 1 KB instruction
  static constexpr int IPW = BT * D * 2 / 1024 / NW;
  static constexpr int NVAR = 16 / RPI < IPW ? 16 / RPI : IPW;  // distinct lane offsets
  static constexpr int NGRP = IPW / NVAR;       // 16-row bands per wave
  static_assert((IPW * RPI) % 16 == 0, "wave row ranges must start at multiples of 16");
  static_assert(IPW % NVAR == 0, "whole bands per wave");
};

template <int D, int BT, int NW, int MODE>
__device__ __forceinline__ void dma_lane_offsets(int lane, uint32_t (&ofs)[DmaGeom<D, BT, NW>::NVAR]) {
  using G = DmaGeom<D, BT, NW>;
  const int p = lane % G::CPR, rsub = lane / G::CPR;
#pragma unroll
  for (int v = 0; v < G::NVAR; ++v) {
    const int rl = v * G::RPI + rsub;
    ofs[v] = (uint32_t)((rl * D + (p ^ lds_swz<D, MODE>(rl)) * 8) * 2);
  }
}

// One wave's bands of a tile: rows [0, valid) of `src`; band grp starts at
// row wave * IPW * RPI + 16 grp and may read `bytes` bytes from there.
// (Plain pointers and sizes; the buffer descriptors are formed where they
// are used, in scalar registers.)
template <int D, int BT, int NW>
struct TileSrc {
  const uint16_t *base[DmaGeom<D, BT, NW>::NGRP];
  int bytes[DmaGeom<D, BT, NW>::NGRP];
};

template <int D, int BT, int NW>
struct TileDma {
  using G = DmaGeom<D, BT, NW>;

  // `p` and `valid` are the same in every lane of the wave; reading them
  // from the first lane says so to the compiler, which then keeps the
  // descriptors in scalar registers instead of looping over lane values.
  __device__ static __forceinline__ TileSrc<D, BT, NW> src(const uint16_t *p, int valid, int wave) {
    const uint64_t pu = reinterpret_cast<uint64_t>(p);
    p = reinterpret_cast<const uint16_t *>(
        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)pu) |
        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(pu >> 32)) << 32));
    valid = __builtin_amdgcn_readfirstlane(valid);
    TileSrc<D, BT, NW> t;
#pragma unroll
    for (int grp = 0; grp < G::NGRP; ++grp) {
      const int row0 = wave * G::IPW * G::RPI + grp * 16;
      t.base[grp] = p + (size_t)row0 * D;
      t.bytes[grp] = valid > row0 ? (valid - row0) * D * 2 : 0;
    }
    return t;
  }

  // Instruction `it` (< IPW) of this wave's share of a tile: a raw buffer
  // load (stride 0) whose descriptor covers the band's valid bytes, so lanes
  // past them write zeros.
  __device__ static __forceinline__ void one(uint16_t *lds, const TileSrc<D, BT, NW> &t, int wave,
                                             int it, const uint32_t *ofs) {
    const int grp = it / G::NVAR;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(t.base[grp]), (short)0, t.bytes[grp],
                                          0x00020000),
        (lds_void *)(lds + wave * G::IPW * 512 + it * 512), 16, ofs[it % G::NVAR], 0, 0, 0);
  }

  // The whole tile: rows [0, valid) of `p`, zeros after.
  __device__ static __forceinline__ void tile(uint16_t *lds, const uint16_t *p, int valid, int wave,
                                              const uint32_t *ofs) {
    const TileSrc<D, BT, NW> t = src(p, valid, wave);
#pragma unroll
    for (int it = 0; it < G::IPW; ++it) one(lds, t, wave, it, ofs);
  }
};

// A = V^T / K^T / Q^T fragment of a 32x32x16 MFMA read from a row-major
// [rows][D] tile with ds_read_b64_tr_b16: two 4-row bands (rows r1 and
// r1 + 8 of the caller's layout), 4 elements each.
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t *tile, int r1, int stride8) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&tile[r1]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&tile[r1 + stride8]));
  return __builtin_bit_cast(bf16x8, (__attribute__((__vector_size__(8 * sizeof(short)))) short){
                                        lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// Which stored block is entry j of query block i's attended list, and how
// many of its rows are valid.  Order: pool slots, selected window slots,
// current-chunk blocks.
template <typename TIn, int D, int BT, typename Args>
__device__ __forceinline__ void resolve_block(const Args &a, size_t bh, int i, int n_pool,
                                              int sc, int j, const TIn *&kp, const TIn *&vp,
                                              int &len) {
  if (j < n_pool) {
    const size_t off = (bh * a.C + j) * (size_t)(BT * D);
    kp = (const TIn *)a.k_pool + off;
    vp = (const TIn *)a.v_pool + off;
    len = a.pool_len[bh * a.C + j];
  } else if (j < n_pool + sc) {
    const int w = a.sel[(bh * a.QB + i) * (size_t)a.topk + (j - n_pool)];
    if (w < 0 || w >= a.W) {
      set_status(a.status, PBSA_STATUS_SEL);
      kp = (const TIn *)a.k_win;
      vp = (const TIn *)a.v_win;
      len = 0;
      return;
    }
    const size_t off = (bh * a.W + w) * (size_t)(BT * D);
    kp = (const TIn *)a.k_win + off;
    vp = (const TIn *)a.v_win + off;
    len = a.win_len[w];
  } else {
    const int c = j - n_pool - sc;
    const size_t off = (bh * a.Nq + (size_t)c * BT) * D;
    kp = (const TIn *)a.k_cur + off;
    vp = (const TIn *)a.v_cur + off;
    len = min(BT, a.Nq - c * BT);
  }
  if (len < 0 || len > BT) {
    set_status(a.status, PBSA_STATUS_WIN_LEN);
    len = max(0, min(len, BT));
  }
}

template <typename Args>
__device__ __forceinline__ int clamp_counts(const Args &a, size_t bh, int i, int &n_pool,
                                            int &sc) {
  n_pool = a.pool_count[bh];
  if (n_pool < 0 || n_pool > a.C) {
    set_status(a.status, PBSA_STATUS_POOL_COUNT);
    n_pool = max(0, min(n_pool, a.C));
  }
  sc = a.sel_count[bh * a.QB + i];
  if (sc < 0 || sc > a.topk) {
    set_status(a.status, PBSA_STATUS_SEL);
    sc = max(0, min(sc, a.topk));
  }
  return n_pool + sc + a.QB;
}

// The pool and selected-window part of a query block's list, resolved once
// per workgroup into LDS: element offset of the block in its region and
// (len | window << 16).  Entries past kMaxList fall back to resolve_block.
constexpr int kMaxList = 128;

struct BlockList {
  int64_t off[kMaxList];
  int32_t meta[kMaxList];
};

// selrow: the query block's selected window slots; nullptr = its row of
// a.sel.  lens: the window slots' lengths then this (b, h)'s pool slots'
// (as in a.win_len / a.pool_len); nullptr = read them there.
template <int D, int BT, typename Args>
__device__ __forceinline__ void preload_list(const Args &a, size_t bh, int i, int n_pool, int sc,
                                             BlockList &bl, int t, int nt,
                                             const int32_t *selrow = nullptr,
                                             const int *lens = nullptr) {
  const int n = min(n_pool + sc, kMaxList);
  for (int j = t; j < n; j += nt) {
    int64_t off;
    int len, win = 0;
    if (j < n_pool) {
      off = (int64_t)(bh * a.C + j) * (BT * D);
      len = lens ? lens[a.W + j] : a.pool_len[bh * a.C + j];
    } else {
      const int w = selrow ? selrow[j - n_pool] : a.sel[(bh * a.QB + i) * (size_t)a.topk + (j - n_pool)];
      win = 1;
      if (w < 0 || w >= a.W) {
        set_status(a.status, PBSA_STATUS_SEL);
        off = 0;
        len = 0;
      } else {
        off = (int64_t)(bh * a.W + w) * (BT * D);
        len = lens ? lens[w] : a.win_len[w];
      }
    }
    if (len < 0 || len > BT) {
      set_status(a.status, PBSA_STATUS_WIN_LEN);
      len = max(0, min(len, BT));
    }
    bl.off[j] = off;
    bl.meta[j] = len | (win << 16);
  }
}

template <int D, int BT, typename Args>
__device__ __forceinline__ void list_block(const Args &a, const BlockList &bl, size_t bh, int i,
                                           int n_pool, int sc, int j, const uint16_t *&kp,
                                           const uint16_t *&vp, int &len) {
  if (j < n_pool + sc && j < kMaxList) {
    const int64_t off = __builtin_amdgcn_readfirstlane((int)(bl.off[j] & 0xffffffff)) |
                        ((int64_t)__builtin_amdgcn_readfirstlane((int)(bl.off[j] >> 32)) << 32);
    const int meta = __builtin_amdgcn_readfirstlane(bl.meta[j]);
    len = meta & 0xffff;
    if (meta >> 16) {
      kp = (const uint16_t *)a.k_win + off;
      vp = (const uint16_t *)a.v_win + off;
    } else {
      kp = (const uint16_t *)a.k_pool + off;
      vp = (const uint16_t *)a.v_pool + off;
    }
  } else {
    resolve_block<uint16_t, D, BT>(a, bh, i, n_pool, sc, j, kp, vp, len);
  }
}

}  // namespace pbsa

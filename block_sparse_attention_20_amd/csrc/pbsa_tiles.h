// LDS tile staging shared by the PBSA attention kernels (gfx950).
#pragma once

#include "pbsa_common.h"

namespace pbsa {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// s_waitcnt immediate: vmcnt <= n, expcnt and lgkmcnt unconstrained (gfx9 encoding)
#define PBSA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14)))

// 256 bytes of zeros: the DMA source for rows past a block's valid length
// (padding rows and the tail of the last current block), so that they land
// in LDS as zeros without a register round trip.
static __device__ __attribute__((aligned(256))) uint32_t g_zero_rows[64];

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

// Stage one [BT][D] bf16 block (rows >= len read as zeros) into LDS,
// swizzled as above.  Each wave moves IPW chunks of 1 KB with
// global_load_lds_dwordx4 (lane l lands at base + 16 l), so the whole block
// is in flight without touching VGPRs.  Instruction `it` of a wave covers
// rows row0 + it*RPI + lane/CPR; every wave's first row is a multiple of 16,
// so a lane's source offset within its row band repeats every 16/RPI
// instructions: dma_lane_offsets() computes those few byte offsets once.
template <int D, int BT, int NW>
struct DmaGeom {
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;          // rows per 1 KB instruction
  static constexpr int IPW = BT * D * 2 / 1024 / NW;
  static constexpr int NVAR = 16 / RPI < IPW ? 16 / RPI : IPW;  // distinct lane offsets
  static_assert((IPW * RPI) % 16 == 0, "wave row ranges must start at multiples of 16");
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

// Ragged block (len < BT): rows past len come from the zero page.
template <int D, int BT, int NW>
__device__ __forceinline__ void dma_block_ragged(uint16_t *dst, const char *base, int row0,
                                                          int len, int lane,
                                                          const uint32_t *ofs) {
  using G = DmaGeom<D, BT, NW>;
  const int rsub = lane / G::CPR, p = lane % G::CPR;
#pragma unroll
  for (int it = 0; it < G::IPW; ++it) {
    const bool ok = row0 + it * G::RPI + rsub < len;
    const char *g = ok ? base + (it / G::NVAR) * (G::NVAR * G::RPI * D * 2) + ofs[it % G::NVAR]
                       : reinterpret_cast<const char *>(g_zero_rows + p * 4);
    __builtin_amdgcn_global_load_lds(g, (lds_void *)(dst + it * 512), 16, 0, 0);
  }
}

template <int D, int BT, int NW, int MODE>
__device__ __forceinline__ void dma_block(uint16_t *lds, const uint16_t *src, int len, int wave,
                                          int lane, const uint32_t (&ofs)[DmaGeom<D, BT, NW>::NVAR]) {
  using G = DmaGeom<D, BT, NW>;
  const int row0 = wave * G::IPW * G::RPI;
  const char *base = reinterpret_cast<const char *>(src + (size_t)row0 * D);
  uint16_t *dst = lds + wave * G::IPW * 512;
  if (len >= BT) {
#pragma unroll
    for (int it = 0; it < G::IPW; ++it) {
      const char *g = base + (it / G::NVAR) * (G::NVAR * G::RPI * D * 2) + ofs[it % G::NVAR];
      __builtin_amdgcn_global_load_lds(g, (lds_void *)(dst + it * 512), 16, 0, 0);
    }
  } else {
    dma_block_ragged<D, BT, NW>(dst, base, row0, len, lane, ofs);
  }
}


// A = V^T / K^T / Q^T fragment of a 32x32x16 MFMA read from a row-major
// [rows][D] tile with ds_read_b64_tr_b16: two 4-row bands (rows r1 and
// r1 + 8 of the caller's layout), 4 elements each.
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t *tile, int r1, int stride8) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&tile[r1]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&tile[r1 + stride8]));
  return __builtin_bit_cast(bf16x8, (__attribute__((__vector_size__(8 * sizeof(short)))) short){
                                        lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

}  // namespace pbsa

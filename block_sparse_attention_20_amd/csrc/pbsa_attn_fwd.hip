// PBSA hybrid attention forward.
//
// Method: "Sparse Forcing: Native Trainable Sparse Attention for Real-time
// Autoregressive Diffusion Video Generation" (gist.science/es explainer,
// sec. 2 "Persistente Block-Sparse Attention (PBSA)": the kernel computes
// dense attention over the persistent memory and sparse attention over the
// local window).  Query block i attends every valid pool slot, its selected
// window slots and the whole current chunk; softmax over all of them.
//
// bf16 path (gfx950 MFMA), one workgroup per (b, h, query block), two
// workgroups per CU (64 KB LDS and <= 256 VGPRs each):
//   - T/32 waves, wave w owns query rows [32w, 32w+32) of the block;
//   - the block list (pool, selected window slots, current chunk) is walked
//     in order.  K and V of a block are moved HBM -> LDS by raw buffer loads
//     with the LDS flag (no register round trip) into row-major tiles whose
//     16-byte chunks are XOR-swizzled per row; each buffer descriptor covers
//     only the valid rows, so lanes past them write zeros and padding can
//     never inject NaN;
//   - the list is walked in 64-token tiles, double buffered (separate K0/K1,
//     V0/V1 arrays indexed at compile time), one barrier per tile: the next
//     tile's DMA is issued one instruction per k-step of the current tile's
//     S MFMAs;
//   - S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held
//     in registers for the whole kernel), so each lane owns one query column
//     and the row softmax is in-lane (four independent max chains) plus one
//     lane-half swap (v_permlane32_swap);
//   - online softmax in the log2 domain; the running max only moves when a
//     block raises it by more than 8 (P <= 2^8), so O is rarely rescaled;
//   - P is rounded to bf16 in registers and is directly the B operand of
//     O^T = V^T P^T; the V^T A operand is read from the row-major V tile with
//     ds_read_b64_tr_b16 (two 4x16 transposed reads per fragment); this part
//     runs at raised wave priority;
//   - work items are mapped XCD-aware: consecutive query blocks of a head
//     run on the same XCD and share its L2 for the pool/current K/V;
//   - with a workspace and at most half the resident slots' worth of query
//     blocks, the list visits are split evenly over up to 8 workgroups per
//     query block; each piece writes a partial and attn_fwd_merge_kernel
//     combines them after the launch, in a fixed order.
// fp32 path: vector FMA version of the same walk (small problems).
#include "pbsa_common.h"
#include "pbsa_internal.h"
#include "pbsa_tiles.h"

#include <atomic>
#include <type_traits>

namespace pbsa {

struct FwdArgs {
  const void *q, *k_cur, *v_cur, *k_win, *v_win, *k_pool, *v_pool;
  const int32_t *win_len, *pool_len, *pool_count, *sel, *sel_count;
  void *o;
  float *lse;
  int32_t *status;
  int H, Nq, W, C, topk, QB, n_items, per_xcd;
  float sl2;  // scale * log2(e)
  // balanced split: NB list entries per item, G workgroups sharing
  // U = n_items * NB block visits; partial results of items cut between
  // workgroups go to part_o / part_ml, and attn_fwd_merge_kernel combines
  // them after the forward launch.
  int split, NB, G;
  int P;  // pieces per query block in the split launch
  float *part_o, *part_ml;
};

__device__ __forceinline__ void item_of_block(const FwdArgs &a, int &item) {
  const int n = blockIdx.x;
  item = (n & 7) * a.per_xcd + (n >> 3);
}

// K/V move through LDS in tiles of 64 tokens (a 128-token block is two
// tiles; a block with <= 64 valid tokens is one), double buffered: the next
// tile's DMA is issued as soon as the barrier at the top of a tile has
// released the buffer of the previous one, so a whole tile of compute hides
// it, with a single barrier per tile.  Four 16 KB buffers keep two
// workgroups per CU.
constexpr int kTile = 64;

// Split launch: every query block's list cut into P equal ranges of
// entries; workgroup wg takes range wg / n_items of query block
// wg % n_items, so the pieces in flight together (consecutive workgroups,
// one XCD) are the same range of consecutive query blocks of a head and
// share its pool and current blocks in L2.  Piece wg writes partial slot wg.
__device__ __forceinline__ int piece_start(const FwdArgs &a, int pc) {
  return (int)((int64_t)pc * a.NB / a.P);
}

template <int D, int BT>
struct FwdLds {
  BlockList blist;
};

// Entries [j0, j1) of item `item`'s block list.  A whole item (0, NB)
// writes O and LSE; a piece writes its unnormalised O^T, running max and row
// sum to its partial slot for attn_fwd_merge_kernel.
// max of x over lanes l and l ^ 32 (v_permlane32_swap exchanges the two
// lane halves of a register; no LDS round trip)
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int D, int BT>
__device__ __forceinline__ void fwd_segment(const FwdArgs &a, FwdLds<D, BT> &sh, uint16_t *K0,
                                            uint16_t *K1, uint16_t *V0, uint16_t *V1, int wg, int item,
                                            int j0, int j1) {
  constexpr int NW = BT / 32;  // waves; wave w owns query rows [32w, 32w+32)
  constexpr int TT = kTile;
  using G = DmaGeom<D, TT, NW>;
  // four separate LDS arrays (not one [2][..] array), so that the compiler
  // sees that this tile's reads and the next tile's DMA touch different
  // objects and inserts no wait for the DMA in front of the reads
  uint16_t *const Kb[2] = {K0, K1};
  uint16_t *const Vb[2] = {V0, V1};
  BlockList &blist = sh.blist;
  const int i = item % a.QB;
  const size_t bh = item / a.QB;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  int n_pool, sc;
  const int nb = clamp_counts(a, bh, i, n_pool, sc);
  const int jend = min(j1, nb);

  // this lane's query column, held as MFMA B fragments for the whole kernel
  const int qrow = i * BT + wave * 32 + l32;
  bf16x8 qf[D / 16];
  {
    const uint16_t *qp = (const uint16_t *)a.q + (bh * a.Nq + (qrow < a.Nq ? qrow : 0)) * (size_t)D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 v = {0, 0, 0, 0};
      if (qrow < a.Nq) v = *reinterpret_cast<const u32x4 *>(qp + kk * 16 + g * 8);
      qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  // running max (log2 units) and row sum, the sum as four partial sums so
  // that the adds of a tile are not one dependent chain
  float m = -INFINITY, l4[4] = {0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.sl2;

  // Per-lane LDS element offsets, fixed for the whole kernel.
  // K fragment (A of S^T): tile row tt*32 + l32, logical chunk 2kk + g.
  int koff[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koff[kk] = l32 * D + (((2 * kk + g) ^ lds_swz<D, kSwzK>(l32)) * 8);
  // V^T fragment via ds_read_b64_tr_b16: in each 16-lane group, lane gi
  // addresses row gi/4 of a 4-row band (rows 16*step + 4g + gi/4, and the
  // band 8 rows further) and 4 of the group's 16 dims; it receives dim gi of
  // the 4 rows.
  const int gi = lane & 15, q16 = (lane >> 4) & 1;
  const int vr = gi >> 2, vq = gi & 3;
  const int vsw = lds_swz<D, kSwzV>(4 * g + vr);
  int voff[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
    voff[dt] = (4 * g + vr) * D + (((4 * dt + 2 * q16 + (vq >> 1)) ^ vsw) * 8) + (vq & 1) * 4;
  uint32_t kdma[G::NVAR], vdma[G::NVAR];
  dma_lane_offsets<D, TT, NW, kSwzK>(lane, kdma);
  dma_lane_offsets<D, TT, NW, kSwzV>(lane, vdma);
  __syncthreads();  // the previous segment of this workgroup is done with LDS
  preload_list<D, BT>(a, bh, i, n_pool, sc, blist, t, 2 * BT);
  __syncthreads();

  // tile stream: (block j, half h); tile rows = min(64, len_j - 64 h)
  int j = j0, h = 0;
  const uint16_t *kb, *vb;
  int blen = 0, tlen = 0;
  if (j0 < jend) {
    list_block<D, BT>(a, blist, bh, i, n_pool, sc, j0, kb, vb, blen);
    tlen = min(TT, blen);
    TileDma<D, TT, NW>::tile(Kb[0], kb, tlen, wave, kdma);
    TileDma<D, TT, NW>::tile(Vb[0], vb, tlen, wave, vdma);
  }
  // the two LDS buffers alternate; each is a compile-time index so that
  // tile addresses are immediate offsets
  auto step = [&](auto bufc) __attribute__((always_inline)) -> bool {
    constexpr int buf = decltype(bufc)::value;
    PBSA_WAIT_VM(0);  // this tile has landed (own loads) ...
    __syncthreads();  // ... for every wave, and every wave is done with the other buffer
    // next tile
    int jn = j, hn = h + 1, nlen = 0;
    const uint16_t *kn = kb, *vn = vb;
    int bn = blen;
    if (hn * TT >= blen || hn * TT >= BT) {
      jn = j + 1;
      hn = 0;
      if (jn < jend) list_block<D, BT>(a, blist, bh, i, n_pool, sc, jn, kn, vn, bn);
    }
    const bool more = jn < jend;
    // the next tile's DMA is spread over the k-steps of S below, between
    // the MFMAs (issued as one burst it stalls the wave on the vector-memory
    // queue); its descriptors cover the valid rows only.  After the last
    // tile they cover nothing: the loads then only write zeros into the idle
    // buffer, which keeps the k-step loop free of branches.
    if (more) nlen = min(TT, bn - hn * TT);
    const TileSrc<D, TT, NW> ksrc = TileDma<D, TT, NW>::src(kn + hn * TT * D, nlen, wave);
    const TileSrc<D, TT, NW> vsrc = TileDma<D, TT, NW>::src(vn + hn * TT * D, nlen, wave);
    const uint16_t *Kl = Kb[buf];
    const uint16_t *Vl = Vb[buf];

    // ---- S^T[token][query] = K Q^T over this tile's 64 tokens
    f32x16 sacc[TT / 32];
#pragma unroll
    for (int tt = 0; tt < TT / 32; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[tt][e] = 0.f;
    {
      constexpr int PD = 2;  // K fragments PD k-steps ahead of the MFMAs
      bf16x8 ka[PD + 1][TT / 32];
#pragma unroll
      for (int k0 = 0; k0 < PD; ++k0)
#pragma unroll
        for (int tt = 0; tt < TT / 32; ++tt)
          ka[k0][tt] = *reinterpret_cast<const bf16x8 *>(&Kl[tt * 32 * D + koff[k0]]);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        if (kk + PD < D / 16) {
#pragma unroll
          for (int tt = 0; tt < TT / 32; ++tt)
            ka[(kk + PD) % (PD + 1)][tt] = *reinterpret_cast<const bf16x8 *>(&Kl[tt * 32 * D + koff[kk + PD]]);
        }
        // this k-step's share of the next tile's DMA (2 IPW instructions
        // over D/16 steps)
        {
          constexpr int NI = 2 * G::IPW, PER = (NI + D / 16 - 1) / (D / 16);
#pragma unroll
          for (int q = 0; q < PER; ++q) {
            const int it2 = kk * PER + q;
            if (it2 < G::IPW)
              TileDma<D, TT, NW>::one(Kb[buf ^ 1], ksrc, wave, it2, kdma);
            else if (it2 < NI)
              TileDma<D, TT, NW>::one(Vb[buf ^ 1], vsrc, wave, it2 - G::IPW, vdma);
          }
        }
#pragma unroll
        for (int tt = 0; tt < TT / 32; ++tt) {
          // an empty asm on the fragment keeps this MFMA after the reads above
          asm volatile("" : "+v"(ka[kk % (PD + 1)][tt]));
          sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk % (PD + 1)][tt], qf[kk], sacc[tt], 0, 0, 0);
        }
      }
    }
    // The softmax and P V part of a tile (exponentials interleaved with
    // MFMAs) runs at raised wave priority: of the two waves sharing a SIMD
    // (one per workgroup), the one in this part issues first, and the other
    // one's S MFMAs fill the matrix pipe around it (measured: 7% faster than
    // equal priorities).
    __builtin_amdgcn_s_setprio(1);
    // ---- online softmax (log2 domain); the running max only moves when a
    // tile raises it by more than 8, so O is rarely rescaled and P <= 2^8.
    if (tlen < TT) {
#pragma unroll
      for (int tt = 0; tt < TT / 32; ++tt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int tok = tt * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
          if (tok >= tlen) sacc[tt][e] = -INFINITY;
        }
    }
    // row max: four independent chains, then the two lane halves (which
    // hold the two 4-token interleaves of the same query column) combined
    // by one lane-half swap
    float mc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int tt = 0; tt < TT / 32; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mc[(2 * tt + (e >> 3)) & 3] = fmaxf(mc[(2 * tt + (e >> 3)) & 3], sacc[tt][e]);
    float mx = fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3]));
    mx = half_swap_max(mx) * sl2;
    if (__ballot(mx > m + 8.f)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);  // m = -inf -> 0
      m = mnew;
#pragma unroll
      for (int k = 0; k < 4; ++k) l4[k] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
    }
    const float muse = m == -INFINITY ? 0.f : m;
    // ---- O^T += V^T P^T  (V^T fragments read one step ahead)
    {
      auto vfrag = [&](int step, int dt) -> bf16x8 {
        const int r1 = step * 16 * D + voff[dt];
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&Vl[r1]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&Vl[r1 + 8 * D]));
        return __builtin_bit_cast(bf16x8, (__attribute__((__vector_size__(8 * sizeof(short)))) short){
                                              lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      };
      bf16x8 va[2][D / 32];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) va[0][dt] = vfrag(0, dt);
#pragma unroll
      for (int st = 0; st < TT / 16; ++st) {
        const int tt = st >> 1, hh = st & 1;
        if (st + 1 < TT / 16) {
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) va[(st + 1) & 1][dt] = vfrag(st + 1, dt);
        }
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(sacc[tt][8 * hh + e] * sl2 - muse);
          l4[st & 3] += p;
          pf[e] = static_cast<__bf16>(p);
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[st & 1][dt], pf, oacc[dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (!more) return false;
    j = jn;
    h = hn;
    kb = kn;
    vb = vn;
    blen = bn;
    tlen = nlen;
    return true;
  };
  if (j0 < jend) {
    while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
    }
    PBSA_WAIT_VM(0);  // the empty loads after the last tile have landed
  }
  float l = (l4[0] + l4[1]) + (l4[2] + l4[3]);
  l += __shfl_xor(l, 32);
  if (j0 > 0 || j1 < a.NB) {
    // piece of a split item: its partial goes to slot wg, laid out
    // [slot][dt][thread][16] so that the merge of one dt reads a contiguous
    // 16 KB
    const int slot = wg;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      float *po = a.part_o + (((size_t)slot * (D / 32) + dt) * (2 * BT) + t) * 16;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        *reinterpret_cast<f32x4 *>(po + 4 * e4) =
            f32x4{oacc[dt][4 * e4], oacc[dt][4 * e4 + 1], oacc[dt][4 * e4 + 2], oacc[dt][4 * e4 + 3]};
    }
    float *pm = a.part_ml + ((size_t)slot * (2 * BT) + t) * 2;
    pm[0] = m;
    pm[1] = l;
    return;
  }
  // O = O^T / l, LSE = ln(sum exp(scale s))
  const float inv = 1.f / l;
  if (qrow < a.Nq) {
    uint16_t *op = (uint16_t *)a.o + (bh * a.Nq + qrow) * (size_t)D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 pk;
        pk[0] = pack_bf16x2(oacc[dt][4 * jj] * inv, oacc[dt][4 * jj + 1] * inv);
        pk[1] = pack_bf16x2(oacc[dt][4 * jj + 2] * inv, oacc[dt][4 * jj + 3] * inv);
        *reinterpret_cast<u32x2 *>(op + dt * 32 + 8 * jj + 4 * g) = pk;
      }
    if (g == 0 && a.lse) a.lse[bh * a.Nq + qrow] = (m + __log2f(l)) * kLn2;
  }
}

template <int D, int BT>
__global__ __launch_bounds__(2 * BT, BT == 128 ? 2 : 1) void attn_fwd_bf16_kernel(FwdArgs a) {
  __shared__ FwdLds<D, BT> sh;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[kTile * D], K1[kTile * D];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[kTile * D], V1[kTile * D];
  int wg;
  item_of_block(a, wg);
  if (!a.split) {
    if (wg < a.n_items) fwd_segment<D, BT>(a, sh, K0, K1, V0, V1, wg, wg, 0, a.NB);
    return;
  }
  if (wg >= a.G) return;
  const int pc = wg / a.n_items;
  fwd_segment<D, BT>(a, sh, K0, K1, V0, V1, wg, wg % a.n_items, piece_start(a, pc), piece_start(a, pc + 1));
}

// Merge of the split pieces, one workgroup per (query block, 32 of the d
// output columns); thread t holds the same rows and columns as thread t of
// the forward.  Two passes over the pieces in workgroup order: the max M of
// their running maxima, then O = sum_g 2^(m_g - M) O_g / sum_g 2^(m_g - M) l_g.
// The order is fixed, so the result does not depend on timing; the kernel
// boundary orders the pieces' stores before these loads.  A split launch
// cuts every query block into P >= 2 non-empty pieces, so each has a partial.
template <int D, int BT>
__global__ __launch_bounds__(2 * BT) void attn_fwd_merge_kernel(FwdArgs a) {
  const int item = blockIdx.x / (D / 32), dt = blockIdx.x % (D / 32);
  if (item >= a.n_items) return;
  const int i = item % a.QB;
  const size_t bh = item / a.QB;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int qrow = i * BT + wave * 32 + l32;
  auto slot_of = [&](int pc) -> size_t { return (size_t)pc * a.n_items + item; };
  const int ga = 0, gb = a.P - 1;
  float M = -INFINITY;
  for (int gg = ga; gg <= gb; ++gg) M = fmaxf(M, a.part_ml[(slot_of(gg) * (2 * BT) + t) * 2]);
  float L = 0.f;
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll 2
  for (int gg = ga; gg <= gb; ++gg) {
    const size_t sl = slot_of(gg);
    const float mg = a.part_ml[(sl * (2 * BT) + t) * 2], lg = a.part_ml[(sl * (2 * BT) + t) * 2 + 1];
    const float w = mg == -INFINITY ? 0.f : exp2f(mg - M);
    L += w * lg;
    const float *po = a.part_o + ((sl * (D / 32) + dt) * (2 * BT) + t) * 16;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(po + 4 * e4);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[4 * e4 + k] += w * v[k];
    }
  }
  if (qrow >= a.Nq) return;
  const float inv = 1.f / L;
  uint16_t *op = (uint16_t *)a.o + (bh * a.Nq + qrow) * (size_t)D;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    u32x2 pk;
    pk[0] = pack_bf16x2(acc[4 * jj] * inv, acc[4 * jj + 1] * inv);
    pk[1] = pack_bf16x2(acc[4 * jj + 2] * inv, acc[4 * jj + 3] * inv);
    *reinterpret_cast<u32x2 *>(op + dt * 32 + 8 * jj + 4 * g) = pk;
  }
  if (dt == 0 && g == 0 && a.lse) a.lse[bh * a.Nq + qrow] = (M + log2f(L)) * kLn2;
}

// fp32 vector path: kF32Tpr threads per query row, each owning D / kF32Tpr
// of the dims (a dot product is a partial sum per thread, reduced over the
// row's lanes with xor shuffles).  One workgroup per query block; K and V
// of one list block staged in LDS at a time; online softmax per 16 keys.
// On the tiny configuration (1 head x 64, 4 query blocks of 64) 8 threads
// per row took 171 us, 16 threads 205 us, 2 threads 415 us.
constexpr int kF32Tpr = 8;

template <int D, int BT>
__global__ __launch_bounds__(kF32Tpr * BT) void attn_fwd_f32_kernel(FwdArgs a) {
  constexpr int NT = kF32Tpr * BT;
  constexpr int DH = D / kF32Tpr;
  __shared__ __attribute__((aligned(16))) float Ks[BT * D];
  __shared__ __attribute__((aligned(16))) float Vs[BT * D];
  int item;
  item_of_block(a, item);
  if (item >= a.n_items) return;
  const int i = item % a.QB;
  const size_t bh = item / a.QB;
  const int t = threadIdx.x, r = t / kF32Tpr, part = t % kF32Tpr;
  int n_pool, sc;
  const int nb = clamp_counts(a, bh, i, n_pool, sc);
  const int qrow = i * BT + r;
  float qv[DH], ov[DH];
  const float *qp = (const float *)a.q + (bh * a.Nq + qrow) * (size_t)D + part * DH;
#pragma unroll
  for (int x = 0; x < DH; ++x) {
    qv[x] = qrow < a.Nq ? qp[x] : 0.f;
    ov[x] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float sl2 = a.sl2;
  for (int j = 0; j < nb; ++j) {
    const float *kp, *vp;
    int len;
    resolve_block<float, D, BT>(a, bh, i, n_pool, sc, j, kp, vp, len);
    __syncthreads();
    for (int e = t * 4; e < BT * D; e += NT * 4) {
      const int row = e / D;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (row < len) {
        kv = *reinterpret_cast<const f32x4 *>(kp + e);
        vv = *reinterpret_cast<const f32x4 *>(vp + e);
      }
      *reinterpret_cast<f32x4 *>(&Ks[e]) = kv;
      *reinterpret_cast<f32x4 *>(&Vs[e]) = vv;
    }
    __syncthreads();
    for (int u0 = 0; u0 < len; u0 += 16) {
      float s[16];
      float mx = -INFINITY;
#pragma unroll
      for (int uu = 0; uu < 16; ++uu) {
        const int u = u0 + uu;
        const float *kr = &Ks[(u < BT ? u : 0) * D + part * DH];
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < DH; ++x) acc += qv[x] * kr[x];
#pragma unroll
        for (int o = 1; o < kF32Tpr; o <<= 1) acc += __shfl_xor(acc, o);
        s[uu] = u < len ? acc * sl2 : -INFINITY;
        mx = fmaxf(mx, s[uu]);
      }
      const float mnew = fmaxf(m, mx);
      const float muse = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = exp2f(m - muse);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int x = 0; x < DH; ++x) ov[x] *= alpha;
#pragma unroll
      for (int uu = 0; uu < 16; ++uu) {
        const int u = u0 + uu;
        const float p = exp2f(s[uu] - muse);
        l += p;
        const float *vr = &Vs[(u < BT ? u : 0) * D + part * DH];
#pragma unroll
        for (int x = 0; x < DH; ++x) ov[x] += p * vr[x];
      }
    }
  }
  if (qrow < a.Nq) {
    float *op = (float *)a.o + (bh * a.Nq + qrow) * (size_t)D + part * DH;
    const float inv = 1.f / l;
#pragma unroll
    for (int x = 0; x < DH; ++x) op[x] = ov[x] * inv;
    if (part == 0 && a.lse) a.lse[bh * a.Nq + qrow] = (m + log2f(l)) * kLn2;
  }
}

// Resident workgroups of the split launch: two per CU (LDS and VGPR
// budget of the bf16 kernel), at most kSplitSlots.  A split launch runs at
// most that many pieces, one workspace partial each.
constexpr int kSplitSlots = 512;
// Most pieces per query block in the split launch (fewer when fewer
// resident slots per query block are free).  More pieces keep more loads
// in flight but each adds a partial to write and merge: forward on 1-4
// query blocks x 12 heads of the Wan cache took 41-51 us (cold caches)
// with 8, against 57-58 with 4 and 50-70 with 16.
constexpr int kMaxPieces = 8;

static int split_slots() {
  // per device, filled on first use; concurrent first calls store the same
  // value, and the atomics keep that free of data races
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kSplitSlots;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = kSplitSlots / 2;
    v = 2 * n < kSplitSlots ? 2 * n : kSplitSlots;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

static size_t split_part_o_bytes(const pbsa_problem &p) {
  return align256((size_t)kSplitSlots * (2 * p.T) * (p.d / 2) * sizeof(float));
}
static size_t split_part_ml_bytes(const pbsa_problem &p) {
  return align256((size_t)kSplitSlots * (2 * p.T) * 2 * sizeof(float));
}

size_t fwd_ws_bytes(const pbsa_problem &p) {
  if (p.dtype != PBSA_BF16) return 0;
  return split_part_o_bytes(p) + split_part_ml_bytes(p);
}

hipError_t launch_attn_fwd(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                           const int32_t *sel, const int32_t *sel_count, void *o, float *lse,
                           void *ws, size_t ws_bytes, hipStream_t st) {
  FwdArgs a;
  a.q = q;
  a.k_cur = kv.k_cur; a.v_cur = kv.v_cur; a.k_win = kv.k_win; a.v_win = kv.v_win;
  a.k_pool = kv.k_pool; a.v_pool = kv.v_pool;
  a.win_len = kv.win_len; a.pool_len = kv.pool_len; a.pool_count = kv.pool_count;
  a.sel = sel; a.sel_count = sel_count; a.o = o; a.lse = lse; a.status = p.dev_status;
  a.H = p.H; a.Nq = p.Nq; a.W = p.W; a.C = p.C; a.topk = p.topk;
  a.QB = (p.Nq + p.T - 1) / p.T;
  a.n_items = p.B * p.H * a.QB;
  a.NB = p.C + p.topk + a.QB;
  a.sl2 = scale * kLog2e;
  a.split = 0;
  a.G = 0;
  a.P = 1;
  a.part_o = a.part_ml = nullptr;
  int n_wg = a.n_items;
  const int64_t slots = split_slots();
  // The split pays off only when one workgroup per query block would leave
  // most resident slots idle; otherwise the partials and their merge only
  // add traffic.  It needs at least two pieces of at least one list entry
  // each (a one-entry list is never split).
  int64_t pcs = slots / a.n_items;
  if (pcs > kMaxPieces) pcs = kMaxPieces;
  if (pcs > a.NB) pcs = a.NB;
  if (p.dtype == PBSA_BF16 && ws != nullptr && ws_bytes >= fwd_ws_bytes(p) && pcs >= 2) {
    a.split = 1;
    a.P = (int)pcs;
    a.G = a.n_items * a.P;
    char *w = reinterpret_cast<char *>(ws);
    a.part_o = reinterpret_cast<float *>(w);
    a.part_ml = reinterpret_cast<float *>(w + split_part_o_bytes(p));
    n_wg = a.G;
  }
  a.per_xcd = (n_wg + 7) / 8;
  const dim3 grid(8 * a.per_xcd);
  const dim3 block(2 * p.T);
#define PBSA_FWD_CASE(DT, D_, T_, KERN)                                              \
  if (p.dtype == DT && p.d == D_ && p.T == T_) {                                     \
    KERN<D_, T_><<<grid, block, 0, st>>>(a);                                         \
    if (a.split)                                                                     \
      attn_fwd_merge_kernel<D_, T_><<<dim3(a.n_items * (D_ / 32)), block, 0, st>>>(a); \
    return hipGetLastError();                                                        \
  }
  PBSA_FWD_CASE(PBSA_BF16, 128, 128, attn_fwd_bf16_kernel)
  PBSA_FWD_CASE(PBSA_BF16, 64, 128, attn_fwd_bf16_kernel)
  PBSA_FWD_CASE(PBSA_BF16, 128, 64, attn_fwd_bf16_kernel)
  PBSA_FWD_CASE(PBSA_BF16, 64, 64, attn_fwd_bf16_kernel)
#undef PBSA_FWD_CASE
  const dim3 block_f32(kF32Tpr * p.T);
#define PBSA_FWD_F32_CASE(D_, T_)                                            \
  if (p.dtype == PBSA_F32 && p.d == D_ && p.T == T_) {                       \
    attn_fwd_f32_kernel<D_, T_><<<grid, block_f32, 0, st>>>(a);              \
    return hipGetLastError();                                                \
  }
  PBSA_FWD_F32_CASE(128, 128)
  PBSA_FWD_F32_CASE(64, 128)
  PBSA_FWD_F32_CASE(128, 64)
  PBSA_FWD_F32_CASE(64, 64)
#undef PBSA_FWD_F32_CASE
  return hipErrorInvalidValue;
}

}  // namespace pbsa

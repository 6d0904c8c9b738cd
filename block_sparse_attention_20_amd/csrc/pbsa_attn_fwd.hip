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
// fp32 path: the same walk on fp32 MFMA (v_mfma_f32_32x32x2_f32), with the
// same split and merge (small problems).
#include "pbsa_common.h"
#include "pbsa_internal.h"
#include "pbsa_select_dev.h"
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
  // NB: list entries per item (an upper bound: C + topk + QB).  Split
  // launch (split = 1): every item's entries cut into P ranges, one per
  // workgroup, G = n_items * P workgroups; each piece writes its partial to
  // part_o / part_ml and attn_fwd_merge_kernel combines them after the
  // forward launch.
  int split, NB, G;
  int P;  // pieces per query block in the split launch
  float *part_o, *part_ml;
  // exact block mass (the MASS kernels): for every query row r and scored
  // list entry j (pool slots and selected window slots), the block's
  // log2-sum-exp log2 sum_{u in j} 2^(s_ru scale log2 e), absolute (not
  // relative to a running max), at blse[((item * E) + j) * BT + row]
  float *blse;
  int E;  // C + topk entries per item
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

// x over lanes l and l ^ 32, summed
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// No routing: the selection is read from a.sel / a.sel_count.
struct NoRoute {
  __device__ int operator()() const { return 0; }
};

// route (the fused select + forward): routes the query block into sel_lds,
// leaves the window and pool slot lengths in lens ([W] then [C]) and
// returns the selection's size; it runs after this workgroup's query
// fragments are in flight and may use K1 and V1 (the first tile goes to K0
// and V0, issued once the routing is done).
template <int D, int BT, bool MASS, typename Route = NoRoute>
__device__ __forceinline__ void fwd_segment(const FwdArgs &a, FwdLds<D, BT> &sh, uint16_t *K0,
                                            uint16_t *K1, uint16_t *V0, uint16_t *V1, int wg, int item,
                                            int j0, int j1, const int32_t *sel_lds = nullptr,
                                            Route route = Route{}, const int *lens = nullptr) {
  constexpr bool ROUTED = !std::is_same<Route, NoRoute>::value;
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
  int n_pool, sc = 0, nb = 0;
  if constexpr (ROUTED) {
    n_pool = a.pool_count[bh];
    n_pool = max(0, min(n_pool, a.C));  // the routing flags a bad count
  } else {
    nb = clamp_counts(a, bh, i, n_pool, sc);
  }

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
  // MASS: the row sum (both lane halves, relative to m) when the previous
  // block ended; a block's own sum is the difference.  Pool and window
  // entries come first in the list, so the sum is still small there and the
  // difference loses little.
  float lprev = 0.f;

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
  // the previous segment of this workgroup is done with LDS (a routed
  // segment is the workgroup's first: no wait, so the query fragments stay
  // in flight through the routing)
  if constexpr (!ROUTED) __syncthreads();
  if constexpr (ROUTED) {
    sc = route();
    nb = n_pool + sc + a.QB;
  }
  const int jend = min(j1, nb);
  const int n_scored = n_pool + sc;

  // tile stream: (block j, half h); tile rows = min(64, len_j - 64 h)
  int j = j0, h = 0;
  const uint16_t *kb = nullptr, *vb = nullptr;
  int blen = 0, tlen = 0;
  bool first_issued = false;
  if constexpr (ROUTED) {
    // a non-empty pool heads the list: its first tile moves while the list
    // is resolved (the routing left the slot lengths in LDS)
    if (j0 == 0 && n_pool > 0) {
      const size_t off = (bh * a.C) * (size_t)(BT * D);
      kb = (const uint16_t *)a.k_pool + off;
      vb = (const uint16_t *)a.v_pool + off;
      blen = max(0, min(__builtin_amdgcn_readfirstlane(lens[a.W]), BT));
      tlen = min(TT, blen);
      TileDma<D, TT, NW>::tile(Kb[0], kb, tlen, wave, kdma);
      TileDma<D, TT, NW>::tile(Vb[0], vb, tlen, wave, vdma);
      first_issued = true;
    }
  }
  preload_list<D, BT>(a, bh, i, n_pool, sc, blist, t, 2 * BT, sel_lds, lens);
  __syncthreads();
  if (j0 < jend && !first_issued) {
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
      if constexpr (MASS) lprev *= alpha;
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
    if constexpr (MASS) {
      // this tile ends block j: its log2-sum-exp for this lane's row
      if (jn != j && j < n_scored) {
        const float ls = half_swap_sum((l4[0] + l4[1]) + (l4[2] + l4[3]));
        const float bs = ls - lprev;
        lprev = ls;
        if (g == 0 && qrow < a.Nq)
          a.blse[((size_t)item * a.E + j) * BT + wave * 32 + l32] = bs > 0.f ? m + __log2f(bs) : -INFINITY;
      }
    }
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

template <int D, int BT, bool MASS>
__global__ __launch_bounds__(2 * BT, BT == 128 ? 2 : 1) void attn_fwd_bf16_kernel(FwdArgs a) {
  __shared__ FwdLds<D, BT> sh;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[kTile * D], K1[kTile * D];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[kTile * D], V1[kTile * D];
  int wg;
  item_of_block(a, wg);
  if (!a.split) {
    if (wg < a.n_items) fwd_segment<D, BT, MASS>(a, sh, K0, K1, V0, V1, wg, wg, 0, a.NB);
    return;
  }
  if (wg >= a.G) return;
  const int pc = wg / a.n_items;
  fwd_segment<D, BT, MASS>(a, sh, K0, K1, V0, V1, wg, wg % a.n_items, piece_start(a, pc),
                           piece_start(a, pc + 1));
}

// Select + forward in one launch (d = T = 128, bf16, no split): each
// workgroup first routes its own query block (select_query_block: the same
// code and order as the select kernel, so sel, sel_count, the means and the
// score rows are bit-identical), then attends with the selection it holds
// in LDS.  The routing's scratch borrows the second K and V tile buffers,
// which the walk first fills during the first tile (after the routing is
// done); it needs 16 KB of each: 2 x 256 x 8 floats of partial sums (then
// the slot lengths), and 20 B per window slot (W <= 819).  The block list
// takes at most 128 entries (C + topk <= 128), all resolved from LDS.  The
// current block's key mean, which nothing in the launch reads, is taken at
// the end (its rows are in L2 by then), so the routing's HBM burst holds
// only the query rows.
constexpr int kFusedMaxW = (kTile * 128 * 2) / 20;

template <int D, int BT>
__global__ __launch_bounds__(2 * BT, 2) void attn_fwd_sel_bf16_kernel(FwdArgs a,
                                                                      SelArgs<uint16_t> s) {
  static_assert(D == 128 && BT == 128, "the routing runs on 256 threads with 16 KB tile buffers");
  __shared__ FwdLds<D, BT> sh;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[kTile * D], K1[kTile * D];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[kTile * D], V1[kTile * D];
  __shared__ __attribute__((aligned(16))) float qv[128];
  __shared__ float both[256];
  __shared__ int nvalid, wcnt[4], n_sel;
  __shared__ int32_t sel_lds[kMaxList];
  __shared__ uint64_t kout[2];  // where the key mean goes (kept out of scalar registers)
  int wg;
  item_of_block(a, wg);
  if (wg >= a.n_items) return;
  const int i = wg % a.QB;
  const size_t bh = wg / a.QB;
  if (threadIdx.x == 0) {
    kout[0] = reinterpret_cast<uint64_t>(s.kbar_cur + (bh * a.QB + i) * D);
    kout[1] = reinterpret_cast<uint64_t>(s.kbarc_out + (bh * a.QB + i) * D);
  }
  int *lens = reinterpret_cast<int *>(K1);
  const SelLds L{qv, reinterpret_cast<float *>(K1), both, V1, &nvalid, wcnt, sel_lds, &n_sel, lens};
  auto route = [&]() -> int {
    select_query_block<uint16_t, false>(s, i, bh, L);
    return n_sel;
  };
  fwd_segment<D, BT, false>(a, sh, K0, K1, V0, V1, wg, wg, 0, a.NB, sel_lds, route, lens);
  // the walk's last DMA (zeros into the idle buffer) has landed before K1
  // is reused
  PBSA_WAIT_VM(0);
  __syncthreads();
  float *kbar = reinterpret_cast<float *>(kout[0]);
  float *kbarc = reinterpret_cast<float *>(kout[1]);
  key_block_mean<uint16_t>((const uint16_t *)a.k_cur + (bh * a.Nq + (size_t)i * BT) * D,
                           min(BT, a.Nq - i * BT), D, kbar, kbarc, reinterpret_cast<float *>(K1), both);
}

// Merge of the split pieces, one workgroup per (query block, 32 of the d
// output columns); thread t holds the same rows and columns as thread t of
// the forward.  The running max and row sum of every piece are loaded at
// once (at most kMergePieces), then O = sum_g 2^(m_g - M) O_g / sum_g
// 2^(m_g - M) l_g with M the max of the m_g, the partial O loads four pieces
// at a time.  Sums run over the pieces in workgroup order, so the result
// does not depend on timing; the kernel boundary orders the pieces' stores
// before these loads.  A split launch cuts every query block into P >= 2
// non-empty pieces, so each has a partial.
constexpr int kMergePieces = 16;

template <int D, int BT, typename TOut>
__global__ __launch_bounds__(2 * BT) void attn_fwd_merge_kernel(FwdArgs a) {
  const int item = blockIdx.x / (D / 32), dt = blockIdx.x % (D / 32);
  if (item >= a.n_items) return;
  const int i = item % a.QB;
  const size_t bh = item / a.QB;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int qrow = i * BT + wave * 32 + l32;
  auto slot_of = [&](int pc) -> size_t { return (size_t)pc * a.n_items + item; };
  float mg[kMergePieces], lg[kMergePieces];
#pragma unroll
  for (int gg = 0; gg < kMergePieces; ++gg) {
    mg[gg] = -INFINITY;
    lg[gg] = 0.f;
    if (gg < a.P) {
      const float *pm = a.part_ml + (slot_of(gg) * (2 * BT) + t) * 2;
      mg[gg] = pm[0];
      lg[gg] = pm[1];
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int gg = 0; gg < kMergePieces; ++gg) M = fmaxf(M, mg[gg]);
  float L = 0.f;
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
  for (int g0 = 0; g0 < kMergePieces; g0 += 4) {
    if (g0 >= a.P) break;
    f32x4 v[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float *po = a.part_o + ((slot_of(g0 + u < a.P ? g0 + u : g0) * (D / 32) + dt) * (2 * BT) + t) * 16;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) v[u][e4] = *reinterpret_cast<const f32x4 *>(po + 4 * e4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (g0 + u < a.P) {
        const float w = mg[g0 + u] == -INFINITY ? 0.f : exp2f(mg[g0 + u] - M);
        L += w * lg[g0 + u];
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[4 * e4 + k] += w * v[u][e4][k];
      }
    }
  }
  if (qrow >= a.Nq) return;
  const float inv = 1.f / L;
  if constexpr (std::is_same<TOut, float>::value) {
    float *op = (float *)a.o + (bh * a.Nq + qrow) * (size_t)D;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      *reinterpret_cast<f32x4 *>(op + dt * 32 + 8 * jj + 4 * g) =
          f32x4{acc[4 * jj] * inv, acc[4 * jj + 1] * inv, acc[4 * jj + 2] * inv, acc[4 * jj + 3] * inv};
  } else {
    uint16_t *op = (uint16_t *)a.o + (bh * a.Nq + qrow) * (size_t)D;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2 pk;
      pk[0] = pack_bf16x2(acc[4 * jj] * inv, acc[4 * jj + 1] * inv);
      pk[1] = pack_bf16x2(acc[4 * jj + 2] * inv, acc[4 * jj + 3] * inv);
      *reinterpret_cast<u32x2 *>(op + dt * 32 + 8 * jj + 4 * g) = pk;
    }
  }
  if (dt == 0 && g == 0 && a.lse) a.lse[bh * a.Nq + qrow] = (M + log2f(L)) * kLn2;
}

// fp32 path (v_mfma_f32_32x32x2_f32), for the small fp32 problems.  Same
// work split as the bf16 kernel (a whole query block, or a piece of its list
// in the split launch, per workgroup; wave w owns query rows [32w, 32w+32))
// and the same accumulator layout, so the pieces go through the same merge.
//   - the contraction order over d is free, so k-step s of S^T = K Q^T takes
//     dims s (lanes 0-31) and D/2 + s (lanes 32-63): a lane's Q values and
//     its K reads are then contiguous runs (16-byte LDS reads, four k-steps
//     each), and Q stays in D/2 registers per lane;
//   - likewise k-step s of O^T = V^T P^T takes, in lane half g, the token
//     held in S^T accumulator element s of that half, so P needs no exchange
//     between lanes: the exponential of element s is the B operand as is;
//   - K and V go through LDS in 64-token tiles with padded rows (K: D + 4,
//     V: D + 8 floats), which makes both read patterns bank-conflict free.
template <int D, int BT, bool MASS>
__device__ __forceinline__ void fwd_f32_segment(const FwdArgs &a, float *Ks, float *Vs, int wg,
                                                int item, int j0, int j1) {
  constexpr int NT = 2 * BT, TT = 64;
  constexpr int SK = D + 4, SV = D + 8;
  const int i = item % a.QB;
  const size_t bh = item / a.QB;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  int n_pool, sc;
  const int nb = clamp_counts(a, bh, i, n_pool, sc);
  const int jend = min(j1, nb);
  const int qrow = i * BT + wave * 32 + l32;
  // this lane's query row: dims [g D/2, g D/2 + D/2), the B operand of S^T
  float qv[D / 2];
  {
    const float *qp = (const float *)a.q + (bh * a.Nq + (qrow < a.Nq ? qrow : 0)) * (size_t)D + g * (D / 2);
#pragma unroll
    for (int s4 = 0; s4 < D / 8; ++s4) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (qrow < a.Nq) v = *reinterpret_cast<const f32x4 *>(qp + 4 * s4);
#pragma unroll
      for (int c = 0; c < 4; ++c) qv[4 * s4 + c] = v[c];
    }
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float sl2 = a.sl2;
  for (int j = j0; j < jend; ++j) {
    const float *kp, *vp;
    int len;
    resolve_block<float, D, BT>(a, bh, i, n_pool, sc, j, kp, vp, len);
    float bsum = 0.f;  // MASS: this block's sum of P (this lane's tokens, relative to m)
    for (int h0 = 0; h0 < len; h0 += TT) {
      const int tlen = min(TT, len - h0);
      __syncthreads();  // every wave is done with the previous tile
      for (int e = t; e < TT * D / 4; e += NT) {
        const int row = e / (D / 4), c4 = e % (D / 4);
        f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
        if (row < tlen) {  // rows past the block's length are zeros, never its padding
          kv = *reinterpret_cast<const f32x4 *>(kp + (size_t)(h0 + row) * D + 4 * c4);
          vv = *reinterpret_cast<const f32x4 *>(vp + (size_t)(h0 + row) * D + 4 * c4);
        }
        *reinterpret_cast<f32x4 *>(&Ks[row * SK + 4 * c4]) = kv;
        *reinterpret_cast<f32x4 *>(&Vs[row * SV + 4 * c4]) = vv;
      }
      __syncthreads();
      // S^T[token][query] over the tile's two 32-token halves
      f32x16 sacc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[tt][e] = 0.f;
        const float *kr = &Ks[(tt * 32 + l32) * SK + g * (D / 2)];
#pragma unroll
        for (int s4 = 0; s4 < D / 8; ++s4) {
          const f32x4 kf = *reinterpret_cast<const f32x4 *>(kr + 4 * s4);
#pragma unroll
          for (int c = 0; c < 4; ++c)
            sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[c], qv[4 * s4 + c], sacc[tt], 0, 0, 0);
        }
      }
      // element e of half tt is token tt*32 + 8 (e / 4) + 4 g + e % 4
      float mx = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int tok = tt * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
          if (tok >= tlen) sacc[tt][e] = -INFINITY;
          mx = fmaxf(mx, sacc[tt][e]);
        }
      mx = half_swap_max(mx) * sl2;
      const float mnew = fmaxf(m, mx);
      const float muse = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m - muse);  // m = -inf -> 0
      m = mnew;
      l *= alpha;
      if constexpr (MASS) bsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
      // O^T += V^T P^T: k-step s of half tt pairs the tokens of element s
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const float p = __builtin_amdgcn_exp2f(sacc[tt][s] * sl2 - muse);
          l += p;
          if constexpr (MASS) bsum += p;
          const int tok = tt * 32 + 8 * (s >> 2) + 4 * g + (s & 3);
          const float *vr = &Vs[tok * SV + l32];
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[dt * 32], p, oacc[dt], 0, 0, 0);
        }
    }
    if constexpr (MASS) {
      if (j < n_pool + sc) {
        const float bs = half_swap_sum(bsum);
        if (g == 0 && qrow < a.Nq)
          a.blse[((size_t)item * a.E + j) * BT + wave * 32 + l32] = bs > 0.f ? m + __log2f(bs) : -INFINITY;
      }
    }
  }
  l += __shfl_xor(l, 32);
  if (j0 > 0 || j1 < a.NB) {
    // piece of a split item: partial slot wg, the bf16 kernel's layout
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      float *po = a.part_o + (((size_t)wg * (D / 32) + dt) * (2 * BT) + t) * 16;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        *reinterpret_cast<f32x4 *>(po + 4 * e4) =
            f32x4{oacc[dt][4 * e4], oacc[dt][4 * e4 + 1], oacc[dt][4 * e4 + 2], oacc[dt][4 * e4 + 3]};
    }
    float *pm = a.part_ml + ((size_t)wg * (2 * BT) + t) * 2;
    pm[0] = m;
    pm[1] = l;
    return;
  }
  if (qrow < a.Nq) {
    float *op = (float *)a.o + (bh * a.Nq + qrow) * (size_t)D;
    const float inv = 1.f / l;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<f32x4 *>(op + dt * 32 + 8 * jj + 4 * g) =
            f32x4{oacc[dt][4 * jj] * inv, oacc[dt][4 * jj + 1] * inv, oacc[dt][4 * jj + 2] * inv,
                  oacc[dt][4 * jj + 3] * inv};
    if (g == 0 && a.lse) a.lse[bh * a.Nq + qrow] = (m + log2f(l)) * kLn2;
  }
}

template <int D, int BT, bool MASS>
__global__ __launch_bounds__(2 * BT) void attn_fwd_f32_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) float Ks[64 * (D + 4)];
  __shared__ __attribute__((aligned(16))) float Vs[64 * (D + 8)];
  int wg;
  item_of_block(a, wg);
  if (!a.split) {
    if (wg < a.n_items) fwd_f32_segment<D, BT, MASS>(a, Ks, Vs, wg, wg, 0, a.NB);
    return;
  }
  if (wg >= a.G) return;
  const int pc = wg / a.n_items;
  fwd_f32_segment<D, BT, MASS>(a, Ks, Vs, wg, wg % a.n_items, piece_start(a, pc),
                               piece_start(a, pc + 1));
}

// Exact block masses from the forward's per-(row, block) log2-sum-exp and
// the final lse: M_j = sum over query rows r attending j of
// 2^(blse_rj - lse_r log2 e), the attention probability the rows put on
// block j.  One workgroup per (stored slot, b, h): pool slot c sums entry c
// of every query block; window slot w sums, for every query block, the
// entries at which it selected w.  Each thread sums its own (query block,
// row) pairs in a fixed order, then a fixed tree over the threads: the
// result is deterministic, and every output element is written (0 where no
// row attends).  grid (B*H, C + W), 256 threads.
template <int BT>
__global__ __launch_bounds__(256) void fwd_mass_reduce_kernel(FwdArgs a, float *mass_pool,
                                                              float *mass_win) {
  constexpr int QPP = 256 / BT;  // query blocks per pass
  __shared__ int first[256], count[256];
  __shared__ float red[256];
  const size_t bh = blockIdx.x;
  const int slot = blockIdx.y;
  const int t = threadIdx.x;
  int n_pool = a.pool_count[bh];
  n_pool = max(0, min(n_pool, a.C));
  const bool is_pool = slot < a.C;
  const int w = slot - a.C;
  float acc = 0.f;
  if (!is_pool || slot < n_pool) {
    for (int i0 = 0; i0 < a.QB; i0 += 256) {
      // matching list entries of query blocks i0 .. i0 + 255
      if (i0 + t < a.QB) {
        const int i = i0 + t;
        int f = -1, c = 0;
        if (is_pool) {
          f = slot;
          c = 1;
        } else {
          const int sc = max(0, min(a.sel_count[bh * a.QB + i], a.topk));
          const int32_t *sl = a.sel + (bh * a.QB + i) * (size_t)a.topk;
          for (int e0 = 0; e0 < sc; e0 += 4) {
            int32_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = e0 + u < sc ? sl[e0 + u] : -1;
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (v[u] == w) {
                if (c == 0) f = n_pool + e0 + u;
                ++c;
              }
          }
        }
        first[t] = f;
        count[t] = c;
      }
      __syncthreads();
      const int ni = min(256, a.QB - i0);
      const int r = t % BT;
      // four of this thread's (query block, row) pairs per round, their loads
      // in flight together; terms added in ascending query block order
      for (int il0 = t / BT; il0 < ni; il0 += 4 * QPP) {
        float bv[4], lv[4];
        int cnt[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int il = il0 + u * QPP, i = i0 + il;
          cnt[u] = il < ni && i * BT + r < a.Nq ? count[il] : 0;
          bv[u] = -INFINITY;
          lv[u] = 0.f;
          if (cnt[u] > 0) lv[u] = a.lse[bh * a.Nq + (size_t)i * BT + r];
          if (cnt[u] == 1) bv[u] = a.blse[((bh * a.QB + i) * (size_t)a.E + first[il]) * BT + r];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (cnt[u] == 1) {
            acc += exp2f(bv[u] - lv[u] * kLog2e);
          } else if (cnt[u] > 1) {  // a slot listed more than once is attended once per listing
            const int i = i0 + il0 + u * QPP;
            const float *bl = a.blse + (((bh * a.QB + i) * (size_t)a.E) * BT) + r;
            const int32_t *sl = a.sel + (bh * a.QB + i) * (size_t)a.topk;
            const int sc = max(0, min(a.sel_count[bh * a.QB + i], a.topk));
            for (int e = 0; e < sc; ++e)
              if (sl[e] == w) acc += exp2f(bl[(size_t)(n_pool + e) * BT] - lv[u] * kLog2e);
          }
        }
      }
      __syncthreads();
    }
  }
  red[t] = acc;
  __syncthreads();
#pragma unroll
  for (int off = 128; off > 0; off >>= 1) {
    if (t < off) red[t] += red[t + off];
    __syncthreads();
  }
  if (t == 0) {
    if (is_pool)
      mass_pool[bh * a.C + slot] = red[0];
    else
      mass_win[bh * a.W + w] = red[0];
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
// with 8, against 57-58 with 4.  16 pieces pay off only while every piece
// has a CU to itself (1 query block x 12 heads: 36 us against 39; at 2,
// 43 against 40).
constexpr int kMaxPieces = 8;
constexpr int kMaxPiecesAlone = 16;
// The fp32 path serves small problems, where a query block's list is a few
// blocks: one piece per list entry, up to this many.
constexpr int kMaxPiecesF32 = 16;
static_assert(kMaxPieces <= kMergePieces && kMaxPiecesAlone <= kMergePieces &&
                  kMaxPiecesF32 <= kMergePieces,
              "the merge loads every piece's running max and row sum at once");

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
  return split_part_o_bytes(p) + split_part_ml_bytes(p);
}

static size_t blse_bytes(const pbsa_problem &p) {
  const size_t QB = (p.Nq + p.T - 1) / p.T;
  const size_t E = (size_t)p.C + p.topk > 0 ? (size_t)p.C + p.topk : 1;
  return align256((size_t)p.B * p.H * QB * E * p.T * sizeof(float));
}

static hipError_t launch_attn_fwd_impl(const pbsa_problem &p, float scale, const void *q,
                                       const pbsa_kv &kv, const int32_t *sel,
                                       const int32_t *sel_count, void *o, float *lse, void *ws,
                                       size_t ws_bytes, float *blse, float *mass_pool,
                                       float *mass_win, hipStream_t st);

// the block log2-sum-exps first, then the split workspace
size_t fwd_mass_ws_bytes(const pbsa_problem &p) { return blse_bytes(p) + fwd_ws_bytes(p); }

hipError_t launch_attn_fwd_mass(const pbsa_problem &p, float scale, const void *q,
                                const pbsa_kv &kv, const int32_t *sel, const int32_t *sel_count,
                                void *o, float *lse, float *mass_pool, float *mass_win, void *ws,
                                size_t ws_bytes, hipStream_t st) {
  char *w = reinterpret_cast<char *>(ws);
  const size_t nb = blse_bytes(p);
  return launch_attn_fwd_impl(p, scale, q, kv, sel, sel_count, o, lse, w + nb, ws_bytes - nb,
                              reinterpret_cast<float *>(w), mass_pool, mass_win, st);
}

hipError_t launch_attn_fwd(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                           const int32_t *sel, const int32_t *sel_count, void *o, float *lse,
                           void *ws, size_t ws_bytes, hipStream_t st) {
  return launch_attn_fwd_impl(p, scale, q, kv, sel, sel_count, o, lse, ws, ws_bytes, nullptr,
                              nullptr, nullptr, st);
}

// The forward's arguments, unsplit.
static FwdArgs fwd_args(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                        const int32_t *sel, const int32_t *sel_count, void *o, float *lse,
                        float *blse) {
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
  a.blse = blse;
  a.E = p.C + p.topk > 0 ? p.C + p.topk : 1;
  a.per_xcd = (a.n_items + 7) / 8;
  return a;
}

// Pieces per query block a split launch would cut (given a workspace): the
// split pays off only when one workgroup per query block would leave most
// resident slots idle; otherwise the partials and their merge only add
// traffic.  It needs at least two pieces of at least one list entry each
// (a one-entry list is never split).
static int64_t split_pieces(const pbsa_problem &p, const FwdArgs &a) {
  const int64_t slots = split_slots();
  int64_t pcs = slots / a.n_items;
  int max_pieces = kMaxPiecesF32;
  if (p.dtype == PBSA_BF16)
    max_pieces = (int64_t)a.n_items * kMaxPiecesAlone <= slots / 2 ? kMaxPiecesAlone : kMaxPieces;
  if (pcs > max_pieces) pcs = max_pieces;
  if (pcs > a.NB) pcs = a.NB;
  return pcs;
}

hipError_t launch_select_attn_fwd(const pbsa_problem &p, float scale, const void *q,
                                  const pbsa_kv &kv, int32_t *sel, int32_t *sel_count, void *o,
                                  float *lse, void *ws, void *fwd_ws, size_t fwd_bytes,
                                  hipStream_t st) {
  FwdArgs a = fwd_args(p, scale, q, kv, sel, sel_count, o, lse, nullptr);
  const bool would_split = fwd_ws != nullptr && fwd_bytes >= fwd_ws_bytes(p) &&
                           split_pieces(p, a) >= 2;
  const bool fused = p.dtype == PBSA_BF16 && p.d == 128 && p.T == 128 &&
                     p.C + p.topk <= kMaxList && p.W <= kFusedMaxW && !would_split;
  if (!fused) {
    hipError_t e = launch_select(p, scale, q, kv, sel, sel_count, nullptr, nullptr, false, ws, st);
    if (e != hipSuccess) return e;
    return launch_attn_fwd(p, scale, q, kv, sel, sel_count, o, lse, fwd_ws, fwd_bytes, st);
  }
  attn_fwd_sel_bf16_kernel<128, 128><<<dim3(8 * a.per_xcd), dim3(256), 0, st>>>(
      a, sel_args<uint16_t>(p, scale, q, kv, sel, sel_count, ws));
  return hipGetLastError();
}

// blse == nullptr: plain forward; else the MASS kernels and the reduce into
// mass_pool / mass_win (lse required)
static hipError_t launch_attn_fwd_impl(const pbsa_problem &p, float scale, const void *q,
                                       const pbsa_kv &kv, const int32_t *sel,
                                       const int32_t *sel_count, void *o, float *lse, void *ws,
                                       size_t ws_bytes, float *blse, float *mass_pool,
                                       float *mass_win, hipStream_t st) {
  FwdArgs a = fwd_args(p, scale, q, kv, sel, sel_count, o, lse, blse);
  int n_wg = a.n_items;
  const int64_t pcs = split_pieces(p, a);
  if (ws != nullptr && ws_bytes >= fwd_ws_bytes(p) && pcs >= 2) {
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
#define PBSA_FWD_CASE(DT, TOUT, D_, T_, KERN)                                                \
  if (p.dtype == DT && p.d == D_ && p.T == T_) {                                             \
    if (blse)                                                                                \
      KERN<D_, T_, true><<<grid, block, 0, st>>>(a);                                         \
    else                                                                                     \
      KERN<D_, T_, false><<<grid, block, 0, st>>>(a);                                        \
    if (a.split)                                                                             \
      attn_fwd_merge_kernel<D_, T_, TOUT><<<dim3(a.n_items * (D_ / 32)), block, 0, st>>>(a);   \
    if (blse && p.C + p.W > 0)                                                               \
      fwd_mass_reduce_kernel<T_><<<dim3(p.B * p.H, p.C + p.W), 256, 0, st>>>(a, mass_pool,   \
                                                                             mass_win);      \
    return hipGetLastError();                                                                \
  }
  PBSA_FWD_CASE(PBSA_BF16, uint16_t, 128, 128, attn_fwd_bf16_kernel)
  PBSA_FWD_CASE(PBSA_BF16, uint16_t, 64, 128, attn_fwd_bf16_kernel)
  PBSA_FWD_CASE(PBSA_BF16, uint16_t, 128, 64, attn_fwd_bf16_kernel)
  PBSA_FWD_CASE(PBSA_BF16, uint16_t, 64, 64, attn_fwd_bf16_kernel)
  PBSA_FWD_CASE(PBSA_F32, float, 128, 128, attn_fwd_f32_kernel)
  PBSA_FWD_CASE(PBSA_F32, float, 64, 128, attn_fwd_f32_kernel)
  PBSA_FWD_CASE(PBSA_F32, float, 128, 64, attn_fwd_f32_kernel)
  PBSA_FWD_CASE(PBSA_F32, float, 64, 64, attn_fwd_f32_kernel)
#undef PBSA_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace pbsa

// PBSA fine-grained block mass.
//
// Method: "Sparse Forcing: Native Trainable Sparse Attention for Real-time
// Autoregressive Diffusion Video Generation" (gist.science/es explainer,
// sec. 2 "Arquitectura Propuesta": dynamic pool blocks are kept by their
// relevance to the current step).  The coarse block mass scores a block by
// pooled representatives; this is the exact alternative: for every stored
// block j, the attention probability the chunk's query rows actually put on
// its tokens,
//   M_j = sum_r sum_{u in j} exp(scale <Q_r, K_u> - lse_r),
// with lse_r the forward's log-sum-exp of row r (so the probabilities are
// those of the forward, normalised over the row's whole attended set).  A
// block a query block does not attend gets nothing from it.
//
// Two launches, deterministic (no atomics on outputs):
//   1. per (b, h, query block): walk the pool and selected-window entries of
//      the block list (the forward's order), S^T = K Q^T on MFMA from LDS
//      tiles, P summed over the tile's valid tokens; each wave writes its
//      sum per entry to a partial slot (fp32 path: one thread per row).
//   2. per (b, h): mass_pool[c] / mass_win[w] = partial slots summed over
//      query blocks (ascending) and waves (ascending).
#include "pbsa_common.h"
#include "pbsa_internal.h"
#include "pbsa_tiles.h"

#include <math.h>

#include <type_traits>

namespace pbsa {

struct FineArgs {
  // block-list resolution reads the v_* fields too; they alias k_*
  const void *q, *k_cur, *v_cur, *k_win, *v_win, *k_pool, *v_pool;
  const int32_t *win_len, *pool_len, *pool_count, *sel, *sel_count;
  const float *lse;
  float *part;  // [B*H*QB][kFineSlots][E] partial sums, E = C + topk entries
  int32_t *status;
  int H, Nq, W, C, topk, QB, n_items, per_xcd, E;
  float sl2, scale;
};

constexpr int kFineSlots = 4;  // partial sums per (query block, entry): one per wave
constexpr int kFineTile = 64;  // K tile rows in LDS

// sum of v over the 64 lanes: the two lane halves first (one lane-half
// swap), then a butterfly over 32 lanes; every lane gets the total
__device__ __forceinline__ float wave_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Zero the partial slots of this item that no wave writes: waves that do
// not exist (fewer than kFineSlots) and entries past n_entries.
__device__ __forceinline__ void zero_unwritten(const FineArgs &a, float *part, int n_waves,
                                               int n_entries, int t, int nt) {
  for (int x = t; x < kFineSlots * a.E; x += nt) {
    const int w = x / a.E, e = x % a.E;
    if (w >= n_waves || e >= n_entries) part[x] = 0.f;
  }
}

template <int D, int BT>
__global__ __launch_bounds__(2 * BT) void fine_mass_bf16_kernel(FineArgs a) {
  constexpr int NW = BT / 32, TT = kFineTile;
  using G = DmaGeom<D, TT, NW>;
  __shared__ BlockList blist;
  // two separate arrays, indexed at compile time, so that reads of one are
  // not made to wait for the DMA into the other
  __shared__ __attribute__((aligned(1024))) uint16_t K0[TT * D], K1[TT * D];
  const int item = (blockIdx.x & 7) * a.per_xcd + (blockIdx.x >> 3);
  if (item >= a.n_items) return;
  const int i = item % a.QB;
  const size_t bh = item / a.QB;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  int n_pool, sc;
  clamp_counts(a, bh, i, n_pool, sc);
  const int ne = n_pool + sc;  // pool and selected window entries
  float *part = a.part + (size_t)item * kFineSlots * a.E;
  zero_unwritten(a, part, NW, ne, t, 2 * BT);
  if (ne == 0) return;

  // this lane's query column as MFMA B fragments; rows past Nq put no mass
  const int qrow = i * BT + wave * 32 + l32;
  const bool qok = qrow < a.Nq;
  bf16x8 qf[D / 16];
  {
    const uint16_t *qp = (const uint16_t *)a.q + (bh * a.Nq + (qok ? qrow : 0)) * (size_t)D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 v = {0, 0, 0, 0};
      if (qok) v = *reinterpret_cast<const u32x4 *>(qp + kk * 16 + g * 8);
      qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const float L2 = qok ? a.lse[bh * a.Nq + qrow] * kLog2e : INFINITY;
  const float sl2 = a.sl2;
  // K fragment (A of S^T): tile row tt*32 + l32, logical chunk 2kk + g
  int koff[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koff[kk] = l32 * D + (((2 * kk + g) ^ lds_swz<D, kSwzK>(l32)) * 8);
  uint32_t kdma[G::NVAR];
  dma_lane_offsets<D, TT, NW, kSwzK>(lane, kdma);
  preload_list<D, BT>(a, bh, i, n_pool, sc, blist, t, 2 * BT);
  __syncthreads();

  // tile stream: (entry j, half h); tile rows = min(64, len_j - 64 h)
  int j = 0, h = 0, blen = 0;
  const uint16_t *kb, *vb;
  list_block<D, BT>(a, blist, bh, i, n_pool, sc, 0, kb, vb, blen);
  int tlen = min(TT, blen);
  TileDma<D, TT, NW>::tile(K0, kb, tlen, wave, kdma);
  float acc = 0.f;  // this lane's P sum over the current entry
  auto step = [&](auto bufc) __attribute__((always_inline)) -> bool {
    constexpr int buf = decltype(bufc)::value;
    uint16_t *const Kl = buf ? K1 : K0;
    uint16_t *const Kn = buf ? K0 : K1;
    PBSA_WAIT_VM(0);  // this tile has landed (own loads) ...
    __syncthreads();  // ... for every wave, and every wave is done with the other buffer
    int jn = j, hn = h + 1, bn = blen, nlen = 0;
    const uint16_t *kn = kb, *vn = vb;
    if (hn * TT >= blen || hn * TT >= BT) {
      jn = j + 1;
      hn = 0;
      if (jn < ne) list_block<D, BT>(a, blist, bh, i, n_pool, sc, jn, kn, vn, bn);
    }
    const bool more = jn < ne;
    if (more) {
      nlen = min(TT, bn - hn * TT);
      TileDma<D, TT, NW>::tile(Kn, kn + hn * TT * D, nlen, wave, kdma);
    }
    if (tlen > 0) {
      f32x16 s[TT / 32];
#pragma unroll
      for (int tt = 0; tt < TT / 32; ++tt)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[tt][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
        for (int tt = 0; tt < TT / 32; ++tt) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(&Kl[tt * 32 * D + koff[kk]]);
          s[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s[tt], 0, 0, 0);
        }
      // element e of accumulator tt is token tt*32 + 8 (e / 4) + 4 g + e % 4
      float p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < TT / 32; ++tt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int tok = tt * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
          const float p = __builtin_amdgcn_exp2f(s[tt][e] * sl2 - L2);
          p4[e & 3] += tok < tlen ? p : 0.f;
        }
      acc += (p4[0] + p4[1]) + (p4[2] + p4[3]);
    }
    if (jn != j) {  // entry j is complete
      const float tot = wave_sum(acc);
      if (lane == 0) part[wave * a.E + j] = tot;
      acc = 0.f;
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
  while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
  }
}

// fp32 inputs (small problems): one thread per query row, K rows read from
// global memory (every thread of the block reads the same row), one block
// sum per entry through LDS in a fixed tree order; slot 0 holds it.
template <int D, int BT>
__global__ __launch_bounds__(BT) void fine_mass_f32_kernel(FineArgs a) {
  __shared__ float red[BT];
  const int item = blockIdx.x;
  if (item >= a.n_items) return;
  const int i = item % a.QB;
  const size_t bh = item / a.QB;
  const int t = threadIdx.x;
  int n_pool, sc;
  clamp_counts(a, bh, i, n_pool, sc);
  const int ne = n_pool + sc;
  float *part = a.part + (size_t)item * kFineSlots * a.E;
  zero_unwritten(a, part, 1, ne, t, BT);
  const int qrow = i * BT + t;
  const bool qok = qrow < a.Nq;
  float qv[D];
  const float *qp = (const float *)a.q + (bh * a.Nq + (qok ? qrow : 0)) * (size_t)D;
#pragma unroll
  for (int c = 0; c < D; ++c) qv[c] = qok ? qp[c] * a.scale : 0.f;
  const float lse = qok ? a.lse[bh * a.Nq + qrow] : INFINITY;
  for (int j = 0; j < ne; ++j) {
    const float *kp, *vp;
    int len;
    resolve_block<float, D, BT>(a, bh, i, n_pool, sc, j, kp, vp, len);
    float acc = 0.f;
    for (int u = 0; u < len; ++u) {
      const float *kr = kp + (size_t)u * D;
      float z = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) z = fmaf(qv[c], kr[c], z);
      acc += __expf(z - lse);
    }
    red[t] = acc;
    __syncthreads();
    for (int n = BT / 2; n > 0; n >>= 1) {
      if (t < n) red[t] += red[t + n];
      __syncthreads();
    }
    if (t == 0) part[j] = red[0];
    __syncthreads();
  }
}

// mass_pool[b,h,c] and mass_win[b,h,w] from the partial slots: query blocks
// ascending, then slots ascending (fixed order, so results are reproducible)
__global__ __launch_bounds__(256) void fine_mass_reduce_kernel(FineArgs a, float *mass_pool,
                                                               float *mass_win) {
  const size_t bh = blockIdx.x;
  const int t = threadIdx.x;
  const int n_pool = max(0, min(a.pool_count[bh], a.C));
  const float *part = a.part + bh * (size_t)a.QB * kFineSlots * a.E;
  for (int c = t; c < a.C; c += 256) {
    float s = 0.f;
    if (c < n_pool)
      for (int i = 0; i < a.QB; ++i)
#pragma unroll
        for (int w4 = 0; w4 < kFineSlots; ++w4) s += part[((size_t)i * kFineSlots + w4) * a.E + c];
    mass_pool[bh * a.C + c] = s;
  }
  for (int w = t; w < a.W; w += 256) {
    float s = 0.f;
    for (int i = 0; i < a.QB; ++i) {
      const int sc = max(0, min(a.sel_count[bh * a.QB + i], a.topk));
      const int32_t *sl = a.sel + (bh * a.QB + i) * (size_t)a.topk;
      for (int e = 0; e < sc; ++e)
        if (sl[e] == w)
#pragma unroll
          for (int w4 = 0; w4 < kFineSlots; ++w4)
            s += part[((size_t)i * kFineSlots + w4) * a.E + n_pool + e];
    }
    mass_win[bh * a.W + w] = s;
  }
}

size_t fine_ws_bytes(const pbsa_problem &p) {
  const size_t QB = (p.Nq + p.T - 1) / p.T;
  const size_t E = (size_t)p.C + p.topk > 0 ? (size_t)p.C + p.topk : 1;
  return align256((size_t)p.B * p.H * QB * kFineSlots * E * sizeof(float));
}

hipError_t launch_fine_mass(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                            const int32_t *sel, const int32_t *sel_count, const float *lse,
                            float *mass_pool, float *mass_win, void *ws, hipStream_t st) {
  FineArgs a;
  a.q = q;
  a.k_cur = a.v_cur = kv.k_cur;
  a.k_win = a.v_win = kv.k_win;
  a.k_pool = a.v_pool = kv.k_pool;
  a.win_len = kv.win_len;
  a.pool_len = kv.pool_len;
  a.pool_count = kv.pool_count;
  a.sel = sel;
  a.sel_count = sel_count;
  a.lse = lse;
  a.part = reinterpret_cast<float *>(ws);
  a.status = p.dev_status;
  a.H = p.H;
  a.Nq = p.Nq;
  a.W = p.W;
  a.C = p.C;
  a.topk = p.topk;
  a.QB = (p.Nq + p.T - 1) / p.T;
  a.n_items = p.B * p.H * a.QB;
  a.per_xcd = (a.n_items + 7) / 8;
  a.E = p.C + p.topk > 0 ? p.C + p.topk : 1;
  a.scale = scale;
  a.sl2 = scale * kLog2e;
  if (p.dtype == PBSA_BF16) {
    const dim3 grid(8 * a.per_xcd);
#define PBSA_FINE_BF16(D_, T_) fine_mass_bf16_kernel<D_, T_><<<grid, 2 * T_, 0, st>>>(a)
    if (p.d == 128 && p.T == 128) PBSA_FINE_BF16(128, 128);
    else if (p.d == 64 && p.T == 128) PBSA_FINE_BF16(64, 128);
    else if (p.d == 128 && p.T == 64) PBSA_FINE_BF16(128, 64);
    else PBSA_FINE_BF16(64, 64);
#undef PBSA_FINE_BF16
  } else {
    const dim3 grid(a.n_items);
#define PBSA_FINE_F32(D_, T_) fine_mass_f32_kernel<D_, T_><<<grid, T_, 0, st>>>(a)
    if (p.d == 128 && p.T == 128) PBSA_FINE_F32(128, 128);
    else if (p.d == 64 && p.T == 128) PBSA_FINE_F32(64, 128);
    else if (p.d == 128 && p.T == 64) PBSA_FINE_F32(128, 64);
    else PBSA_FINE_F32(64, 64);
#undef PBSA_FINE_F32
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  fine_mass_reduce_kernel<<<p.B * p.H, 256, 0, st>>>(a, mass_pool, mass_win);
  return hipGetLastError();
}

}  // namespace pbsa

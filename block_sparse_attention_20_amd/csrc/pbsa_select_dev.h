// PBSA coarse routing of one query block, as device code shared by the
// select kernel and the fused select + forward kernel (both compute exactly
// this, in this order, so their results are bit-identical).
//
// Method: "Sparse Forcing: Native Trainable Sparse Attention for Real-time
// Autoregressive Diffusion Video Generation" (gist.science/es explainer,
// sec. 2 "Persistente Block-Sparse Attention (PBSA)": blocks are compressed
// by pooling into representatives for a cheap coarse routing;
// "Arquitectura Propuesta": Top-K window blocks per query).
// Representatives are plain means of the valid rows; the coarse logit is
// scale * <qbar, kbar>.
#pragma once

#include "pbsa_common.h"
#include "pbsa_internal.h"

namespace pbsa {

// Means of the first n rows of NBLK [rows, d] blocks a (and b) (row stride
// d), both blocks' loads in flight together; fp32 sums in a fixed order,
// the same for a block averaged alone or with another.  256 threads, 16-byte
// loads; red: LDS, >= NBLK*256*8 floats.  Threads [0, d) write out_a[t],
// threads [d, 2d) out_b[t - d]; the means also go to both[0, NBLK*d) (LDS,
// for the caller after a sync).
template <typename TIn, int NBLK = 2>
__device__ void two_block_means(const TIn *__restrict__ a, const TIn *__restrict__ b, int n, int d,
                                float *out_a, float *out_b, float *red, float *both) {
  constexpr int E = 16 / sizeof(TIn);
  const int tpr = d / E, rpp = 256 / tpr;
  const int t = threadIdx.x;
  const int rg = t / tpr, cg = t % tpr;
  const TIn *src[2] = {a, b};
  float acc[NBLK][E];
#pragma unroll
  for (int k = 0; k < NBLK; ++k)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[k][e] = 0.f;
#pragma unroll 8
  for (int r = rg; r < n; r += rpp) {
    u32x4 v[NBLK];
#pragma unroll
    for (int k = 0; k < NBLK; ++k) v[k] = *reinterpret_cast<const u32x4 *>(src[k] + (size_t)r * d + cg * E);
#pragma unroll
    for (int k = 0; k < NBLK; ++k) {
      if constexpr (sizeof(TIn) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[k][2 * e] += bflo(v[k][e]);
          acc[k][2 * e + 1] += bfhi(v[k][e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[k][e] += __uint_as_float(v[k][e]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < NBLK; ++k)
#pragma unroll
    for (int e = 0; e < E; ++e) red[k * 256 * 8 + rg * d + cg * E + e] = acc[k][e];
  __syncthreads();
  if (t < NBLK * d) {
    const int c = t % d, w = t / d;
    float s = 0.f;
    for (int g = 0; g < rpp; ++g) s += red[w * 256 * 8 + g * d + c];
    const float v = n > 0 ? s / (float)n : 0.f;
    if (w == 0) out_a[c] = v; else out_b[c] = v;
    both[t] = v;
  }
}

// Inputs and outputs of the routing of one query block (plain pointers).
template <typename TIn>
struct SelArgs {
  const TIn *q, *k_cur;
  float *qbar_out, *kbarc_out, *kbar_cur;
  const float *kbar_pool, *kbar_win;
  const int32_t *pool_count, *win_len, *pool_len;
  const int64_t *win_id;
  int32_t *sel, *sel_count;
  float *srow_out;
  int H, Nq, d, T, W, C, QB, topk;
  float scale;
  int32_t *status;
};

// The routing's arguments for problem p; the workspace ws is laid out as
// select_ws_layout says.
template <typename TIn>
inline SelArgs<TIn> sel_args(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                             int32_t *sel, int32_t *sel_count, const void *ws) {
  SelArgs<TIn> s;
  float *qbar, *srows, *kbarc;
  select_ws_layout(p, ws, qbar, srows, kbarc);
  s.q = (const TIn *)q;
  s.k_cur = (const TIn *)kv.k_cur;
  s.qbar_out = qbar;
  s.kbarc_out = kbarc;
  s.kbar_cur = kv.kbar_cur;
  s.kbar_pool = kv.kbar_pool;
  s.kbar_win = kv.kbar_win;
  s.pool_count = kv.pool_count;
  s.win_len = kv.win_len;
  s.pool_len = kv.pool_len;
  s.win_id = kv.win_id;
  s.sel = sel;
  s.sel_count = sel_count;
  s.srow_out = srows;
  s.H = p.H;
  s.Nq = p.Nq;
  s.d = p.d;
  s.T = p.T;
  s.W = p.W;
  s.C = p.C;
  s.QB = (p.Nq + p.T - 1) / p.T;
  s.topk = p.topk;
  s.scale = scale;
  s.status = p.dev_status;
  return s;
}

// LDS the routing works in (all of it dead once it returns, except
// sel_lds / n_sel_lds).  dyn: W * (8 + 4 + 4 + 4) bytes, 8-byte aligned.
struct SelLds {
  float *qv;       // [128]
  float *red;      // [2 * 256 * 8]
  float *both;     // [256]
  void *dyn;       // window ids [W] int64, keys [W], flags [W], ranks [W]
  int *nvalid;     // [1]
  int *wcnt;       // [4]
  int32_t *sel_lds;  // optional [topk]: the selection, as written to sel
  int *n_sel_lds;    // optional [1]: its count
  // optional [W + C]: the window slots' and pool slots' lengths, as read
  // (unclamped), written over red once the means are done (needs
  // W <= 4 * 256, C <= 256)
  int *lens;
};

// 16 candidates per pass; 7 passes cover the 106 pool and window candidates
// of the Wan chunk (pool 32 + window 74) with one batch of loads.
constexpr int kScorePasses = 7;

// Own-block means, coarse scores + window top-k of query block i of (b, h)
// row bh, by one 256-thread workgroup:
//  - the query block's Q rows and K rows (the current chunk's block i) are
//    averaged together: qbar_i to LDS and to the workspace (for the block
//    mass), kbar_cur_i to its cache;
//  - candidates [pool C | window W], 16 lanes per candidate (coalesced
//    16-byte reads of kbar, 4 shuffles); the first batch of candidate loads
//    is issued before the means are reduced;
//  - the score row's pool and window part goes to the workspace for the
//    block-mass kernel (which adds the current-chunk part);
//  - top-k is rank based: a valid window slot is selected iff fewer than k
//    valid slots rank before it in the total order (score desc, id asc, NaN
//    last); its output position is the number of selected slots below it.
//    Exact and order-independent, hence deterministic.  Scores enter the
//    ranking as order keys (order_key; 0 = invalid slot), so the pairwise
//    comparisons are branch free.
// KMEAN = false leaves kbar_cur_i and its workspace copy to key_block_mean
// (the same bits, later).  Ends with the workgroup synchronised.
template <typename TIn, bool KMEAN = true>
__device__ __forceinline__ void select_query_block(const SelArgs<TIn> &s, int i, size_t bh,
                                                   const SelLds &L) {
  const int H = s.H, Nq = s.Nq, d = s.d, T = s.T, W = s.W, C = s.C, QB = s.QB, topk = s.topk;
  (void)H;
  int64_t *wid = reinterpret_cast<int64_t *>(L.dyn);     // [W]
  uint32_t *key = reinterpret_cast<uint32_t *>(wid + W);  // [W]: order keys
  int *flag = reinterpret_cast<int *>(key + W);           // [W]: 1 valid, 2 selected
  int *rank = flag + W;                                    // [W]
  float *qv = L.qv;
  int &nvalid_sh = *L.nvalid;
  int *wcnt = L.wcnt;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int n_pool = s.pool_count[bh];
  if (n_pool < 0 || n_pool > C) {
    if (t == 0) set_status(s.status, PBSA_STATUS_POOL_COUNT);
    n_pool = max(0, min(n_pool, C));
  }
  int nv = 0;
  int wl[4] = {0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int w = t + 256 * u;
    if (w < W) {
      const int len = s.win_len[w];
      if (len > T) set_status(s.status, PBSA_STATUS_WIN_LEN);
      flag[w] = len > 0 ? 1 : 0;
      nv += len > 0;
      wid[w] = s.win_id[w];
      wl[u] = len;
    }
  }
  for (int w = t + 1024; w < W; w += 256) {
    const int len = s.win_len[w];
    if (len > T) set_status(s.status, PBSA_STATUS_WIN_LEN);
    flag[w] = len > 0 ? 1 : 0;
    nv += len > 0;
    wid[w] = s.win_id[w];
  }
  const int pl = (L.lens && t < C) ? s.pool_len[bh * C + t] : 0;
  if (t == 0) nvalid_sh = 0;
  const int nj = C + W;                 // candidates scored here
  const int nrow = C + W + QB;          // score row length (current part: block mass)
  const int sub = lane >> 4, sl = lane & 15;
  const int per = d / 16;  // floats per lane (8 or 4)
  float *srow = s.srow_out + (bh * QB + i) * (size_t)nrow;
  // one batch of candidate loads (the first kScorePasses * 16 candidates).
  // Every stored slot's representative is loaded (in bounds whether or not
  // the slot is valid), so the loads wait for no metadata; an invalid
  // slot's score is replaced by -inf below.
  auto load_batch = [&](int base, f32x4 (&k0)[kScorePasses], f32x4 (&k1)[kScorePasses],
                        bool (&ok)[kScorePasses]) __attribute__((always_inline)) {
#pragma unroll
    for (int ps = 0; ps < kScorePasses; ++ps) {
      const int j = base + ps * 16 + sub;
      const float *kb = nullptr;
      bool valid = false;
      if (j < C) {
        valid = j < n_pool;
        kb = s.kbar_pool + (bh * C + j) * d;
      } else if (j < nj) {
        valid = s.win_len[j - C] > 0;
        kb = s.kbar_win + (bh * W + (j - C)) * d;
      }
      ok[ps] = valid;
      k0[ps] = f32x4{0.f, 0.f, 0.f, 0.f};
      k1[ps] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j < nj) {
        k0[ps] = *reinterpret_cast<const f32x4 *>(kb + sl * per);
        if (per == 8) k1[ps] = *reinterpret_cast<const f32x4 *>(kb + sl * per + 4);
      }
    }
  };
  f32x4 k0[kScorePasses], k1[kScorePasses];
  bool ok[kScorePasses];
  int base = wave * 4;
  load_batch(base, k0, k1, ok);
  // the block's own means (Q -> qbar, K -> kbar_cur)
  {
    const int r0 = i * T, n = min(T, Nq - r0);
    if constexpr (KMEAN)
      two_block_means<TIn>(s.q + (bh * Nq + r0) * d, s.k_cur + (bh * Nq + r0) * d, n, d, qv,
                           s.kbar_cur + (bh * QB + i) * d, L.red, L.both);
    else
      two_block_means<TIn, 1>(s.q + (bh * Nq + r0) * d, nullptr, n, d, qv, nullptr, L.red, L.both);
  }
  __syncthreads();
  if (t < d) {
    s.qbar_out[(bh * QB + i) * d + t] = qv[t];
    if constexpr (KMEAN) s.kbarc_out[(bh * QB + i) * d + t] = L.both[d + t];
  }
  if (L.lens) {  // red is dead from here on
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (t + 256 * u < W) L.lens[t + 256 * u] = wl[u];
    if (t < C) L.lens[W + t] = pl;
  }
  for (int o = 32; o > 0; o >>= 1) nv += __shfl_xor(nv, o);
  if (lane == 0) atomicAdd(&nvalid_sh, nv);
  for (;;) {
#pragma unroll
    for (int ps = 0; ps < kScorePasses; ++ps) {
      const int j = base + ps * 16 + sub;
      const float *qq = qv + sl * per;
      float acc = qq[0] * k0[ps][0] + qq[1] * k0[ps][1] + qq[2] * k0[ps][2] + qq[3] * k0[ps][3];
      if (per == 8) acc += qq[4] * k1[ps][0] + qq[5] * k1[ps][1] + qq[6] * k1[ps][2] + qq[7] * k1[ps][3];
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      acc += __shfl_xor(acc, 4);
      acc += __shfl_xor(acc, 8);
      if (sl == 0 && j < nj) {
        const float v = ok[ps] ? acc * s.scale : -INFINITY;
        srow[j] = v;
        if (j >= C) key[j - C] = ok[ps] ? order_key(v) : 0u;
      }
    }
    base += 16 * kScorePasses;
    if (base >= nj) break;
    load_batch(base, k0, k1, ok);
  }
  __syncthreads();

  // rank-based top-k over the valid window slots: a slot is selected iff
  // fewer than k valid slots rank before it.  The comparisons are split
  // over the four waves (each takes a quarter of the v range for every w);
  // partial ranks meet in LDS.
  for (int w = t; w < W; w += 256) rank[w] = 0;
  __syncthreads();
  {
    const int vq = (W + 3) / 4, v0 = wave * vq, v1 = min(W, v0 + vq);
    for (int w = lane; w < W; w += 64) {
      const uint32_t kw = key[w];
      const int64_t iw = wid[w];
      int r = 0;
      // an invalid v has key 0 and never ranks before a valid w; v == w
      // fails both terms
#pragma unroll 8
      for (int v = v0; v < v1; ++v) {
        const uint32_t kv = key[v];
        r += (int)((kv > kw) | ((kv == kw) & (wid[v] < iw)));
      }
      if (r && kw != 0) atomicAdd(&rank[w], r);
    }
  }
  __syncthreads();
  for (int w = t; w < W; w += 256)
    if ((flag[w] & 1) && rank[w] < topk) flag[w] |= 2;
  __syncthreads();
  const int n_sel = min(topk, nvalid_sh);
  int32_t *selrow = s.sel + (bh * QB + i) * (size_t)topk;
  // positions: ascending slot order, by ballot prefix counts per 256 slots
  int carry = 0;
  for (int base = 0; base < W; base += 256) {
    const int w = base + t;
    const bool bit = w < W && (flag[w] & 2);
    const unsigned long long m = __ballot(bit);
    if (lane == 0) wcnt[wave] = __popcll(m);
    __syncthreads();
    int before = carry;
    for (int q = 0; q < wave; ++q) before += wcnt[q];
    const int pos = before + __popcll(m & ((1ull << lane) - 1ull));
    if (bit && pos < topk) {  // more than k only with duplicate ids
      selrow[pos] = w;
      if (L.sel_lds) L.sel_lds[pos] = w;
    }
    carry += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    __syncthreads();
  }
  for (int p = n_sel + t; p < topk; p += 256) {
    selrow[p] = -1;
    if (L.sel_lds) L.sel_lds[p] = -1;
  }
  if (t == 0) {
    s.sel_count[bh * QB + i] = n_sel;
    if (L.n_sel_lds) *L.n_sel_lds = n_sel;
  }
  __syncthreads();
}

// kbar_cur_i and its workspace copy, as select_query_block<TIn, true>
// computes them (same loads and summation order), from the current block's
// K rows.  red: >= 256*8 floats of LDS, both: >= d floats.  Ends with the
// workgroup synchronised.
template <typename TIn>
__device__ __forceinline__ void key_block_mean(const TIn *k_rows, int n, int d, float *kbar_out,
                                               float *kbarc_out, float *red, float *both) {
  two_block_means<TIn, 1>(k_rows, nullptr, n, d, kbar_out, nullptr, red, both);
  __syncthreads();
  if (threadIdx.x < d) kbarc_out[threadIdx.x] = both[threadIdx.x];
  __syncthreads();
}

}  // namespace pbsa

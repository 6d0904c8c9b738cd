// PBSA sparse attention backward (bf16 MFMA, deterministic, no atomics).
//
// Method: "Sparse Forcing: Native Trainable Sparse Attention for Real-time
// Autoregressive Diffusion Video Generation" - the title's *trainable*
// sparse attention: training runs with the sparse mechanism in the loop
// (gist.science/es explainer, sec. 2 "Entrenamiento"), so gradients flow
// through the fixed block mask while the routing itself is not
// differentiated.
//
// With P the forward weights (recomputed from the saved LSE),
// D_r = <dO_r, O_r> and dS = P (dO V^T - D):
//   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO.
// Four launches:
//   1. D = rowsum(dO * O) per query row;
//   2. inverse selection lists: for every window slot, the query blocks that
//      selected it (CSR, ascending query block, built per (b, h));
//   3. dQ: one workgroup per (b, h, query block), walking the same block
//      list as the forward (S^T, dP^T and dQ^T on MFMA; P and dS fed from
//      the accumulators as B operands);
//   4. dK/dV: one workgroup per stored KV block (pool slot, window slot,
//      current block); it loops over the query blocks that attend it (all of
//      them for pool and current blocks, the CSR list for window slots) and
//      keeps its K/V in registers.  Blocks nobody attends get zeros.
// Every gradient element is written by exactly one workgroup, in a fixed
// order, so results are bitwise reproducible.
#include "pbsa_common.h"
#include "pbsa_internal.h"

namespace pbsa {

struct BwdArgs {
  const uint16_t *q, *k_cur, *v_cur, *k_win, *v_win, *k_pool, *v_pool, *o, *dout;
  const int32_t *win_len, *pool_len, *pool_count, *sel, *sel_count;
  const float *lse;
  uint16_t *dq, *dk_cur, *dv_cur, *dk_win, *dv_win, *dk_pool, *dv_pool;
  float *Dv;
  int32_t *qptr, *qidx;
  int32_t *status;
  int H, Nq, W, C, topk, QB, n_items;
  float scale, sl2;
};

__device__ __forceinline__ int perm4b(int rg) { return (rg & ~3) | ((rg & 1) << 1) | ((rg >> 1) & 1); }

// rows [ROWS][D] -> LDS, row stride D+8, rows >= len zero
template <int D, int ROWS, int NT>
__device__ __forceinline__ void stage_rows(uint16_t *lds, const uint16_t *src, int len, int t) {
  constexpr int CH = ROWS * D / 8;
#pragma unroll
  for (int c = t; c < CH; c += NT) {
    const int row = c / (D / 8), col = c % (D / 8);
    u32x4 v = {0, 0, 0, 0};
    if (row < len) v = *reinterpret_cast<const u32x4 *>(src + row * D + col * 8);
    *reinterpret_cast<u32x4 *>(lds + row * (D + 8) + col * 8) = v;
  }
}

// rows [ROWS][D] -> LDS transposed [D][ROWS+8]; within every 16 rows the
// 4-row groups 1 and 2 swap places, so that the rows one MFMA lane needs
// (the accumulator layout of a 32x32 tile) are 8 contiguous elements.
template <int D, int ROWS, int NT>
__device__ __forceinline__ void stage_cols(uint16_t *lds, const uint16_t *src, int len, int t) {
  constexpr int UN = (ROWS / 4) * (D / 8);
  constexpr int VS = ROWS + 8;
#pragma unroll
  for (int u = t; u < UN; u += NT) {
    const int rg = u % (ROWS / 4), dg = u / (ROWS / 4);
    u32x4 v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = rg * 4 + e;
      v[e] = u32x4{0, 0, 0, 0};
      if (row < len) v[e] = *reinterpret_cast<const u32x4 *>(src + row * D + dg * 8);
    }
    uint16_t *dst = lds + (dg * 8) * VS + perm4b(rg) * 4;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int wd = c >> 1;
      u32x2 pk;
      if (c & 1) {
        pk[0] = (v[0][wd] >> 16) | (v[1][wd] & 0xffff0000u);
        pk[1] = (v[2][wd] >> 16) | (v[3][wd] & 0xffff0000u);
      } else {
        pk[0] = (v[0][wd] & 0xffffu) | (v[1][wd] << 16);
        pk[1] = (v[2][wd] & 0xffffu) | (v[3][wd] << 16);
      }
      *reinterpret_cast<u32x2 *>(dst + c * VS) = pk;
    }
  }
}

// ---------------------------------------------------------------------------
// 1. D_r = <dO_r, O_r>.  grid (ceil(rows/16)), 256 threads, 16 rows per block
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const uint16_t *__restrict__ o,
                                                         const uint16_t *__restrict__ dout,
                                                         float *__restrict__ Dv, size_t rows) {
  constexpr int TPR = D / 8;  // threads per row
  const size_t r = (size_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (r < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(o + r * D + c * 8);
    const u32x4 b = *reinterpret_cast<const u32x4 *>(dout + r * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += bflo(a[e]) * bflo(b[e]) + bfhi(a[e]) * bfhi(b[e]);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (r < rows && c == 0) Dv[r] = acc;
}

// ---------------------------------------------------------------------------
// 2. inverse selection lists.  grid (H, B), 256 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_csr_kernel(const int32_t *__restrict__ sel,
                                                      const int32_t *__restrict__ sel_count,
                                                      int32_t *__restrict__ qptr,
                                                      int32_t *__restrict__ qidx, int H, int W,
                                                      int QB, int topk) {
  __shared__ int32_t cnt[1025];
  const size_t bh = (size_t)blockIdx.y * H + blockIdx.x;
  const int t = threadIdx.x;
  const int32_t *sb = sel + bh * QB * (size_t)topk;
  const int32_t *cb = sel_count + bh * QB;
  for (int w = t; w < W; w += 256) {
    int n = 0;
    for (int i = 0; i < QB; ++i) {
      const int sc = max(0, min(cb[i], topk));
      for (int s = 0; s < sc; ++s) n += sb[(size_t)i * topk + s] == w;
    }
    cnt[w] = n;
  }
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      const int n = cnt[w];
      cnt[w] = run;
      run += n;
    }
    cnt[W] = run;
  }
  __syncthreads();
  int32_t *qp = qptr + bh * (W + 1);
  int32_t *qi = qidx + bh * QB * (size_t)topk;
  for (int w = t; w <= W; w += 256) qp[w] = cnt[w];
  for (int w = t; w < W; w += 256) {
    int pos = cnt[w];
    for (int i = 0; i < QB; ++i) {
      const int sc = max(0, min(cb[i], topk));
      for (int s = 0; s < sc; ++s)
        if (sb[(size_t)i * topk + s] == w) qi[pos++] = i;
    }
  }
}

// block j of query block i's list (as the forward)
template <int D, int BT>
__device__ __forceinline__ void bwd_resolve(const BwdArgs &a, size_t bh, int i, int n_pool, int sc,
                                            int j, const uint16_t *&kp, const uint16_t *&vp,
                                            int &len) {
  if (j < n_pool) {
    const size_t off = (bh * a.C + j) * (size_t)(BT * D);
    kp = a.k_pool + off;
    vp = a.v_pool + off;
    len = a.pool_len[bh * a.C + j];
  } else if (j < n_pool + sc) {
    const int w = a.sel[(bh * a.QB + i) * (size_t)a.topk + (j - n_pool)];
    if (w < 0 || w >= a.W) {
      set_status(a.status, PBSA_STATUS_SEL);
      kp = a.k_win;
      vp = a.v_win;
      len = 0;
      return;
    }
    const size_t off = (bh * a.W + w) * (size_t)(BT * D);
    kp = a.k_win + off;
    vp = a.v_win + off;
    len = a.win_len[w];
  } else {
    const int c = j - n_pool - sc;
    const size_t off = (bh * a.Nq + (size_t)c * BT) * D;
    kp = a.k_cur + off;
    vp = a.v_cur + off;
    len = min(BT, a.Nq - c * BT);
  }
  len = max(0, min(len, BT));
}

__device__ __forceinline__ int bwd_item(const BwdArgs &a) {
  const int per = (a.n_items + 7) / 8;
  return (blockIdx.x & 7) * per + (blockIdx.x >> 3);
}

// ---------------------------------------------------------------------------
// 3. dQ per (b, h, query block).
// ---------------------------------------------------------------------------
template <int D, int BT>
__global__ __launch_bounds__(2 * BT) void bwd_dq_kernel(BwdArgs a) {
  constexpr int NT = 2 * BT;
  constexpr int KS = D + 8, TS = BT + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * TS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BT * KS];
  const int item = bwd_item(a);
  if (item >= a.n_items) return;
  const int i = item % a.QB;
  const size_t bh = item / a.QB;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l32 = lane & 31, g = lane >> 5;
  int n_pool = max(0, min(a.pool_count[bh], a.C));
  int sc = max(0, min(a.sel_count[bh * a.QB + i], a.topk));
  const int nb = n_pool + sc + a.QB;
  const int qrow = i * BT + wave * 32 + l32;
  const bool qok = qrow < a.Nq;
  bf16x8 qf[D / 16], df[D / 16];
  {
    const size_t base = (bh * a.Nq + (qok ? qrow : 0)) * (size_t)D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 v = {0, 0, 0, 0}, w = {0, 0, 0, 0};
      if (qok) {
        v = *reinterpret_cast<const u32x4 *>(a.q + base + kk * 16 + g * 8);
        w = *reinterpret_cast<const u32x4 *>(a.dout + base + kk * 16 + g * 8);
      }
      qf[kk] = __builtin_bit_cast(bf16x8, v);
      df[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const float lse2 = qok ? a.lse[bh * a.Nq + qrow] * kLog2e : INFINITY;
  const float Dq = qok ? a.Dv[bh * a.Nq + qrow] : 0.f;
  f32x16 dqacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqacc[dt][e] = 0.f;

  for (int j = 0; j < nb; ++j) {
    const uint16_t *kp, *vp;
    int len;
    bwd_resolve<D, BT>(a, bh, i, n_pool, sc, j, kp, vp, len);
    __syncthreads();
    stage_rows<D, BT, NT>(Ks, kp, len, t);
    stage_cols<D, BT, NT>(Kt, kp, len, t);
    stage_rows<D, BT, NT>(Vs, vp, len, t);
    __syncthreads();
    f32x16 sacc[BT / 32], pacc[BT / 32];
#pragma unroll
    for (int tt = 0; tt < BT / 32; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[tt][e] = pacc[tt][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int tt = 0; tt < BT / 32; ++tt) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(&Ks[(tt * 32 + l32) * KS + kk * 16 + g * 8]);
        const bf16x8 va = *reinterpret_cast<const bf16x8 *>(&Vs[(tt * 32 + l32) * KS + kk * 16 + g * 8]);
        sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], sacc[tt], 0, 0, 0);
        pacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[kk], pacc[tt], 0, 0, 0);
      }
    // dS^T = P^T (dP^T - D), padding tokens masked
#pragma unroll
    for (int tt = 0; tt < BT / 32; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int tok = tt * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
        const float p = tok < len ? __builtin_amdgcn_exp2f(sacc[tt][e] * a.sl2 - lse2) : 0.f;
        sacc[tt][e] = p * (pacc[tt][e] - Dq);
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int tt = 0; tt < BT / 32; ++tt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 sf;
#pragma unroll
        for (int e = 0; e < 8; ++e) sf[e] = static_cast<__bf16>(sacc[tt][8 * h + e]);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(&Kt[(dt * 32 + l32) * TS + tt * 32 + h * 16 + g * 8]);
          dqacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, sf, dqacc[dt], 0, 0, 0);
        }
      }
  }
  if (qok) {
    uint16_t *op = a.dq + (bh * a.Nq + qrow) * (size_t)D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 pk;
        pk[0] = pack_bf16x2(dqacc[dt][4 * jj] * a.scale, dqacc[dt][4 * jj + 1] * a.scale);
        pk[1] = pack_bf16x2(dqacc[dt][4 * jj + 2] * a.scale, dqacc[dt][4 * jj + 3] * a.scale);
        *reinterpret_cast<u32x2 *>(op + dt * 32 + 8 * jj + 4 * g) = pk;
      }
  }
}

// ---------------------------------------------------------------------------
// 4. dK, dV per stored KV block.  Items: [pool C | window W | current QB]
//    per (b, h).
// ---------------------------------------------------------------------------
template <int D, int BT>
__global__ __launch_bounds__(2 * BT) void bwd_dkv_kernel(BwdArgs a) {
  constexpr int NT = 2 * BT;
  constexpr int KS = D + 8, TS = BT + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[BT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[D * TS];
  __shared__ __attribute__((aligned(16))) uint16_t Os[BT * KS];  // dO rows
  __shared__ __attribute__((aligned(16))) uint16_t Ot[D * TS];   // dO transposed
  __shared__ float lse2s[BT], Ds[BT];
  const int item = bwd_item(a);
  if (item >= a.n_items) return;
  const int nj = a.C + a.W + a.QB;
  const int jb = item % nj;
  const size_t bh = item / nj;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l32 = lane & 31, g = lane >> 5;
  const int n_pool = max(0, min(a.pool_count[bh], a.C));

  const uint16_t *kp = nullptr, *vp = nullptr;
  uint16_t *dkp, *dvp;
  int len, nq = 0, list_base = 0;
  bool all_q = false;
  if (jb < a.C) {
    const size_t off = (bh * a.C + jb) * (size_t)(BT * D);
    kp = a.k_pool + off; vp = a.v_pool + off; dkp = a.dk_pool + off; dvp = a.dv_pool + off;
    len = jb < n_pool ? max(0, min(a.pool_len[bh * a.C + jb], BT)) : 0;
    all_q = true;
  } else if (jb < a.C + a.W) {
    const int w = jb - a.C;
    const size_t off = (bh * a.W + w) * (size_t)(BT * D);
    kp = a.k_win + off; vp = a.v_win + off; dkp = a.dk_win + off; dvp = a.dv_win + off;
    len = max(0, min(a.win_len[w], BT));
    list_base = a.qptr[bh * (a.W + 1) + w];
    nq = a.qptr[bh * (a.W + 1) + w + 1] - list_base;
  } else {
    const int c = jb - a.C - a.W;
    const size_t off = (bh * a.Nq + (size_t)c * BT) * D;
    kp = a.k_cur + off; vp = a.v_cur + off; dkp = a.dk_cur + off; dvp = a.dv_cur + off;
    len = min(BT, a.Nq - c * BT);
    all_q = true;
  }
  if (all_q) nq = len > 0 ? a.QB : 0;
  const bool is_cur = jb >= a.C + a.W;

  // this lane's key token, held as B fragments (K^T and V^T columns)
  const int tok = wave * 32 + l32;
  const bool tok_ok = tok < len;
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 v = {0, 0, 0, 0}, w = {0, 0, 0, 0};
    if (tok_ok) {
      v = *reinterpret_cast<const u32x4 *>(kp + tok * D + kk * 16 + g * 8);
      w = *reinterpret_cast<const u32x4 *>(vp + tok * D + kk * 16 + g * 8);
    }
    kf[kk] = __builtin_bit_cast(bf16x8, v);
    vf[kk] = __builtin_bit_cast(bf16x8, w);
  }
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) dkacc[dt][e] = dvacc[dt][e] = 0.f;

  for (int n = 0; n < nq; ++n) {
    const int i = all_q ? n : a.qidx[bh * a.QB * (size_t)a.topk + list_base + n];
    const int r0 = i * BT;
    const int qlen = min(BT, a.Nq - r0);
    const size_t roff = (bh * a.Nq + r0) * (size_t)D;
    __syncthreads();
    stage_rows<D, BT, NT>(Qs, a.q + roff, qlen, t);
    stage_cols<D, BT, NT>(Qt, a.q + roff, qlen, t);
    stage_rows<D, BT, NT>(Os, a.dout + roff, qlen, t);
    stage_cols<D, BT, NT>(Ot, a.dout + roff, qlen, t);
    for (int r = t; r < BT; r += NT) {
      lse2s[r] = r < qlen ? a.lse[bh * a.Nq + r0 + r] * kLog2e : INFINITY;
      Ds[r] = r < qlen ? a.Dv[bh * a.Nq + r0 + r] : 0.f;
    }
    __syncthreads();
    // S[q][tok] = Q K^T and dP[q][tok] = dO V^T
    f32x16 sacc[BT / 32], pacc[BT / 32];
#pragma unroll
    for (int qt = 0; qt < BT / 32; ++qt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[qt][e] = pacc[qt][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int qt = 0; qt < BT / 32; ++qt) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(&Qs[(qt * 32 + l32) * KS + kk * 16 + g * 8]);
        const bf16x8 oa = *reinterpret_cast<const bf16x8 *>(&Os[(qt * 32 + l32) * KS + kk * 16 + g * 8]);
        sacc[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], sacc[qt], 0, 0, 0);
        pacc[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[kk], pacc[qt], 0, 0, 0);
      }
    // P and dS (element (qt, e) is query row qt*32 + 8(e/4) + 4g + e%4)
#pragma unroll
    for (int qt = 0; qt < BT / 32; ++qt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int qr = qt * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
        const float p = tok_ok ? __builtin_amdgcn_exp2f(sacc[qt][e] * a.sl2 - lse2s[qr]) : 0.f;
        sacc[qt][e] = p;
        pacc[qt][e] = p * (pacc[qt][e] - Ds[qr]);
      }
    // dV^T += dO^T P ; dK^T += Q^T dS
#pragma unroll
    for (int qt = 0; qt < BT / 32; ++qt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 pf, sf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pf[e] = static_cast<__bf16>(sacc[qt][8 * h + e]);
          sf[e] = static_cast<__bf16>(pacc[qt][8 * h + e]);
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int off = (dt * 32 + l32) * TS + qt * 32 + h * 16 + g * 8;
          const bf16x8 oa = *reinterpret_cast<const bf16x8 *>(&Ot[off]);
          const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(&Qt[off]);
          dvacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, pf, dvacc[dt], 0, 0, 0);
          dkacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, sf, dkacc[dt], 0, 0, 0);
        }
      }
  }
  // write this lane's token row (zeros for padding rows of stored slots)
  if (is_cur && !tok_ok) return;
  uint16_t *dk = dkp + tok * (size_t)D;
  uint16_t *dv = dvp + tok * (size_t)D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2 pk, pv;
      pk[0] = pack_bf16x2(dkacc[dt][4 * jj] * a.scale, dkacc[dt][4 * jj + 1] * a.scale);
      pk[1] = pack_bf16x2(dkacc[dt][4 * jj + 2] * a.scale, dkacc[dt][4 * jj + 3] * a.scale);
      pv[0] = pack_bf16x2(dvacc[dt][4 * jj], dvacc[dt][4 * jj + 1]);
      pv[1] = pack_bf16x2(dvacc[dt][4 * jj + 2], dvacc[dt][4 * jj + 3]);
      *reinterpret_cast<u32x2 *>(dk + dt * 32 + 8 * jj + 4 * g) = pk;
      *reinterpret_cast<u32x2 *>(dv + dt * 32 + 8 * jj + 4 * g) = pv;
    }
}

size_t bwd_ws_bytes(const pbsa_problem &p) {
  const size_t bh = (size_t)p.B * p.H;
  const size_t QB = (p.Nq + p.T - 1) / p.T;
  return align256(bh * p.Nq * sizeof(float)) + align256(bh * (p.W + 1) * sizeof(int32_t)) +
         align256(bh * QB * (size_t)(p.topk > 0 ? p.topk : 1) * sizeof(int32_t));
}

hipError_t launch_attn_bwd(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                           const int32_t *sel, const int32_t *sel_count, const void *o,
                           const float *lse, const void *dout, void *dq, const pbsa_kv_grad &g,
                           void *ws, hipStream_t st) {
  if (p.dtype != PBSA_BF16) return hipErrorNotSupported;
  BwdArgs a;
  a.q = (const uint16_t *)q;
  a.k_cur = (const uint16_t *)kv.k_cur; a.v_cur = (const uint16_t *)kv.v_cur;
  a.k_win = (const uint16_t *)kv.k_win; a.v_win = (const uint16_t *)kv.v_win;
  a.k_pool = (const uint16_t *)kv.k_pool; a.v_pool = (const uint16_t *)kv.v_pool;
  a.o = (const uint16_t *)o; a.dout = (const uint16_t *)dout;
  a.win_len = kv.win_len; a.pool_len = kv.pool_len; a.pool_count = kv.pool_count;
  a.sel = sel; a.sel_count = sel_count; a.lse = lse;
  a.dq = (uint16_t *)dq;
  a.dk_cur = (uint16_t *)g.dk_cur; a.dv_cur = (uint16_t *)g.dv_cur;
  a.dk_win = (uint16_t *)g.dk_win; a.dv_win = (uint16_t *)g.dv_win;
  a.dk_pool = (uint16_t *)g.dk_pool; a.dv_pool = (uint16_t *)g.dv_pool;
  a.status = p.dev_status;
  a.H = p.H; a.Nq = p.Nq; a.W = p.W; a.C = p.C; a.topk = p.topk;
  a.QB = (p.Nq + p.T - 1) / p.T;
  a.scale = scale;
  a.sl2 = scale * kLog2e;
  const size_t bh = (size_t)p.B * p.H;
  char *w = reinterpret_cast<char *>(ws);
  a.Dv = reinterpret_cast<float *>(w);
  w += align256(bh * p.Nq * sizeof(float));
  a.qptr = reinterpret_cast<int32_t *>(w);
  w += align256(bh * (p.W + 1) * sizeof(int32_t));
  a.qidx = reinterpret_cast<int32_t *>(w);

  const size_t rows = bh * p.Nq;
  const unsigned rblocks = (unsigned)((rows + (256 / (p.d / 8)) - 1) / (256 / (p.d / 8)));
  if (p.d == 128)
    bwd_rowdot_kernel<128><<<rblocks, 256, 0, st>>>(a.o, a.dout, a.Dv, rows);
  else
    bwd_rowdot_kernel<64><<<rblocks, 256, 0, st>>>(a.o, a.dout, a.Dv, rows);
  if (p.W > 0) bwd_csr_kernel<<<dim3(p.H, p.B), 256, 0, st>>>(sel, sel_count, a.qptr, a.qidx, p.H, p.W, a.QB, p.topk);

  const dim3 block(2 * p.T);
#define PBSA_BWD_CASE(D_, T_)                                               \
  if (p.d == D_ && p.T == T_) {                                             \
    a.n_items = (int)(bh * a.QB);                                           \
    bwd_dq_kernel<D_, T_><<<dim3(8 * ((a.n_items + 7) / 8)), block, 0, st>>>(a); \
    a.n_items = (int)(bh * (p.C + p.W + a.QB));                             \
    bwd_dkv_kernel<D_, T_><<<dim3(8 * ((a.n_items + 7) / 8)), block, 0, st>>>(a); \
    return hipGetLastError();                                               \
  }
  PBSA_BWD_CASE(128, 128)
  PBSA_BWD_CASE(64, 128)
  PBSA_BWD_CASE(128, 64)
  PBSA_BWD_CASE(64, 64)
#undef PBSA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace pbsa

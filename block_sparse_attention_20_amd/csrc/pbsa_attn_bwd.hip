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
//   1. per query row: L = log2(e) lse and -D, into arrays padded to whole
//      query blocks (padding rows hold zeros);
//   2. inverse selection lists: for every window slot, the query blocks that
//      selected it (CSR, ascending query block, built per (b, h) from the
//      selection staged in LDS);
//   3. dQ: one workgroup per (b, h, query block), walking the same block
//      list as the forward; K and V tiles of 64 tokens are moved to LDS by
//      DMA, double buffered.  S^T = K Q^T and dP^T = V dO^T take K and V rows
//      as A operands; dQ^T += K^T dS^T reads K^T from the same tile with
//      ds_read_b64_tr_b16.
//   4. dK/dV: one workgroup per stored KV block (pool slot, current block,
//      window slot - the ones attended by every query block first), looping
//      over the query blocks that attend it (all of them for pool and current
//      blocks, the CSR list for window slots) in 32-row Q/dO tiles, DMA
//      staged and double buffered (separate buffers indexed at compile time,
//      so no read waits for the next tile's DMA); K and V stay in
//      registers.  Blocks nobody attends get zeros.
// Every gradient element is written by exactly one workgroup, in a fixed
// order, so results are bitwise reproducible.
//
// Tiles that are read both as rows (A operand, 16 lanes x 16 bytes per
// cycle) and transposed (ds_read_b64_tr_b16, 4 rows x 64 bytes) use the
// two-way swizzle kSwzU; tiles read only as rows use kSwzK.
#include "pbsa_common.h"
#include "pbsa_internal.h"
#include "pbsa_tiles.h"

#include <type_traits>

namespace pbsa {

struct BwdArgs {
  const uint16_t *q, *k_cur, *v_cur, *k_win, *v_win, *k_pool, *v_pool, *o, *dout;
  const int32_t *win_len, *pool_len, *pool_count, *sel, *sel_count;
  const float *lse;
  uint16_t *dq, *dk_cur, *dv_cur, *dk_win, *dv_win, *dk_pool, *dv_pool;
  float *LDp;  // [bh][QB*T][2]: (log2(e) lse, -D) per query row, zero padded
  int32_t *qptr, *qidx;
  int32_t *status;
  int H, Nq, W, C, topk, QB, n_items, per_xcd;
  float scale, sl2;
};

constexpr int kTileB = 64;  // rows of every staged tile

// consecutive items on the same XCD (workgroup n runs on XCD n % 8)
__device__ __forceinline__ int bwd_item(const BwdArgs &a) {
  return (blockIdx.x & 7) * a.per_xcd + (blockIdx.x >> 3);
}

// ---------------------------------------------------------------------------
// 1. L_r = log2(e) lse_r and -D_r = -<dO_r, O_r>.  grid (ceil(bh*QB*T / rows
//    per block)), 256 threads; rows past Nq of each (b, h) get zeros.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_rows_kernel(const uint16_t *__restrict__ o,
                                                       const uint16_t *__restrict__ dout,
                                                       const float *__restrict__ lse,
                                                       float *__restrict__ LDp, size_t rows_p,
                                                       int Nq, int NqP) {
  constexpr int TPR = D / 8;  // threads per row
  const size_t rp = (size_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  const size_t bh = rp / NqP;
  const int r = (int)(rp % NqP);
  const bool ok = rp < rows_p && r < Nq;
  const size_t src = bh * Nq + r;
  float acc = 0.f;
  if (ok) {
    const u32x4 x = *reinterpret_cast<const u32x4 *>(o + src * D + c * 8);
    const u32x4 y = *reinterpret_cast<const u32x4 *>(dout + src * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += bflo(x[e]) * bflo(y[e]) + bfhi(x[e]) * bfhi(y[e]);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (rp < rows_p && c == 0) {
    LDp[2 * rp] = ok ? lse[src] * kLog2e : 0.f;
    LDp[2 * rp + 1] = -acc;
  }
}

// ---------------------------------------------------------------------------
// 2. inverse selection lists.  grid (H, B), 256 threads; thread t owns the
//    window slots t, t + 256, t + 512, t + 768.  The selection rows are
//    staged in LDS (invalid entries -1) and scanned in order, so each slot's
//    list is in ascending query block order.
// ---------------------------------------------------------------------------
constexpr int kCsrChunk = 8192;

// entries [base, base + m) into sl[0, m), padded with -1 to a multiple of 16
__device__ __forceinline__ int csr_stage(int32_t *sl, const int32_t *sb, const int32_t *cb,
                                         int base, int m, int topk, int W, int t) {
  const int mp = (m + 15) & ~15;
  for (int e = t; e < mp; e += 256) {
    int w = -1;
    if (e < m) {
      const int idx = base + e;
      const int i = idx / topk, s = idx - i * topk;
      w = s < cb[i] ? sb[idx] : -1;
    }
    sl[e] = w >= 0 && w < W ? w : -1;  // out-of-range slots select nothing
  }
  return mp;
}

// In place: start[0..W) holds per-slot counts (W <= 1024); afterwards
// start[w] is the exclusive prefix sum and start[W] the total.  256 threads;
// thread t sums slots 4t..4t+3, then a wave scan and a scan of wave totals.
__device__ __forceinline__ void csr_exclusive_scan(int32_t *start, int32_t *wsum, int W, int t) {
  const int lane = t & 63, wave = t >> 6;
  __syncthreads();
  int v[4], s = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[k] = 4 * t + k < W ? start[4 * t + k] : 0;
    s += v[k];
  }
  int incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int run = incl - s;
  for (int w2 = 0; w2 < wave; ++w2) run += wsum[w2];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    start[4 * t + k] = run;
    run += v[k];
  }
  if (t == 255) start[1024] = run;
  __syncthreads();
  if (t == 0) start[W] = start[1024];
  __syncthreads();
}

// Small problems (QB * W <= kCsrMat): per (query block, slot) selection
// counts in LDS; each slot's list is then a scan over query blocks.
constexpr int kCsrMat = 12288;

__global__ __launch_bounds__(256) void bwd_csr_mat_kernel(const int32_t *__restrict__ sel,
                                                          const int32_t *__restrict__ sel_count,
                                                          int32_t *__restrict__ qptr,
                                                          int32_t *__restrict__ qidx, int H, int W,
                                                          int QB, int topk) {
  __shared__ int32_t mat[kCsrMat];
  __shared__ int32_t start[1024 + 1];
  __shared__ int32_t wsum[4];
  const size_t bh = (size_t)blockIdx.y * H + blockIdx.x;
  const int t = threadIdx.x;
  const int32_t *sb = sel + bh * QB * (size_t)topk;
  const int32_t *cb = sel_count + bh * QB;
  for (int e = t; e < QB * W; e += 256) mat[e] = 0;
  __syncthreads();
  for (int e = t; e < QB * topk; e += 256) {
    const int i = e / topk, s = e - i * topk;
    if (s < cb[i]) {
      const int w = sb[e];
      if (w >= 0 && w < W) atomicAdd(&mat[i * W + w], 1);  // out-of-range slots select nothing
    }
  }
  __syncthreads();
  for (int w = t; w < 1024; w += 256) {
    int c = 0;
    if (w < W)
      for (int i = 0; i < QB; ++i) c += mat[i * W + w];
    start[w] = c;
  }
  csr_exclusive_scan(start, wsum, W, t);
  int32_t *qp = qptr + bh * (W + 1);
  int32_t *qi = qidx + bh * QB * (size_t)topk;
  for (int w = t; w <= W; w += 256) qp[w] = start[w];
  for (int w = t; w < W; w += 256) {
    int pos = start[w];
    for (int i = 0; i < QB; ++i)
      for (int c = mat[i * W + w]; c > 0; --c) qi[pos++] = i;
  }
}

__global__ __launch_bounds__(256) void bwd_csr_kernel(const int32_t *__restrict__ sel,
                                                      const int32_t *__restrict__ sel_count,
                                                      int32_t *__restrict__ qptr,
                                                      int32_t *__restrict__ qidx, int H, int W,
                                                      int QB, int topk) {
  __shared__ __attribute__((aligned(16))) int32_t sl[kCsrChunk];
  __shared__ int32_t start[1024 + 1];
  __shared__ int32_t wsum[4];
  const size_t bh = (size_t)blockIdx.y * H + blockIdx.x;
  const int t = threadIdx.x;
  const int32_t *sb = sel + bh * QB * (size_t)topk;
  const int32_t *cb = sel_count + bh * QB;
  const int n = QB * topk;
  int c0 = 0, c1 = 0, c2 = 0, c3 = 0;
  for (int base = 0; base < n; base += kCsrChunk) {
    const int m = min(kCsrChunk, n - base);
    __syncthreads();
    const int mp = csr_stage(sl, sb, cb, base, m, topk, W, t);
    __syncthreads();
    for (int e = 0; e < mp; e += 16) {
      int4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = *reinterpret_cast<const int4 *>(&sl[e + 4 * k]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int ws[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int w = ws[q];
          c0 += w == t;
          c1 += w == t + 256;
          c2 += w == t + 512;
          c3 += w == t + 768;
        }
      }
    }
  }
  __syncthreads();
  start[t] = c0;
  start[t + 256] = c1;
  start[t + 512] = c2;
  start[t + 768] = c3;
  csr_exclusive_scan(start, wsum, W, t);
  int32_t *qp = qptr + bh * (W + 1);
  for (int w = t; w <= W; w += 256) qp[w] = start[w];
  int p0 = start[t], p1 = start[t + 256], p2 = start[t + 512], p3 = start[t + 768];
  int32_t *qi = qidx + bh * QB * (size_t)topk;
  for (int base = 0; base < n; base += kCsrChunk) {
    const int m = min(kCsrChunk, n - base);
    __syncthreads();
    const int mp = csr_stage(sl, sb, cb, base, m, topk, W, t);
    __syncthreads();
    if (t >= W) continue;  // owns no slot (W <= 1024, so t < W covers every owner)
    for (int e = 0; e < mp; e += 16) {
      int4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = *reinterpret_cast<const int4 *>(&sl[e + 4 * k]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int ws[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int w = ws[q];
          if (w >= 0 && (w & 255) == t) {  // w < W <= 1024 here
            const int i = (base + e + 4 * k + q) / topk;
            const int kk = w >> 8;
            const int pos = kk == 0 ? p0++ : kk == 1 ? p1++ : kk == 2 ? p2++ : p3++;
            qi[pos] = i;
          }
        }
      }
    }
  }
}

// Element offsets of the transposed (tr16) A fragments of a 32x32x16 MFMA
// over a [64][D] tile swizzled with kSwzU: for 16 tile rows starting at a
// multiple of 16, lane (gi = lane & 15) of each 16-lane group addresses row
// 4g + gi/4 (lo) and the row 8 further (hi), dims 32 dt + 16 q16 + 4 (gi & 3).
// Because the swizzle XORs whole chunks, the offsets of dims tile dt are the
// dt = 0 offset XOR 32 dt, and the hi row's is the lo one XOR 16 plus 8 rows:
// one base per lane (tr_base) and two XORs per fragment (tr_frag_u).
template <int D>
__device__ __forceinline__ int tr_base(int lane) {
  const int g = lane >> 5, gi = lane & 15, q16 = (lane >> 4) & 1, vr = gi >> 2, vq = gi & 3;
  const int rlo = 4 * g + vr;
  return rlo * D + (((2 * q16 + (vq >> 1)) ^ lds_swz<D, kSwzU>(rlo)) * 8) + (vq & 1) * 4;
}

__device__ __forceinline__ bf16x8 tr_read(const uint16_t *tile, int lo, int hi) {
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&tile[lo]));
  const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&tile[hi]));
  return __builtin_bit_cast(bf16x8, (__attribute__((__vector_size__(8 * sizeof(short)))) short){
                                        x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]});
}

template <int D>
__device__ __forceinline__ bf16x8 tr_frag_u(const uint16_t *tile, int base, int dt) {
  const int lo = base ^ (32 * dt);
  return tr_read(tile, lo, (lo ^ 16) + 8 * D);
}

// this lane's row as MFMA B fragments (dims 16 kk + 8 g .. + 7)
template <int D>
__device__ __forceinline__ void load_bfrag(bf16x8 (&f)[D / 16], const uint16_t *row, bool ok, int g) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 v = {0, 0, 0, 0};
    if (ok) v = *reinterpret_cast<const u32x4 *>(row + kk * 16 + g * 8);
    f[kk] = __builtin_bit_cast(bf16x8, v);
  }
}

// ---------------------------------------------------------------------------
// 3. dQ per (b, h, query block).
// ---------------------------------------------------------------------------
template <int D, int BT>
__global__ __launch_bounds__(2 * BT, BT == 128 ? 2 : 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int NW = BT / 32, TT = kTileB;
  using G = DmaGeom<D, TT, NW>;
  __shared__ __attribute__((aligned(1024))) uint16_t Kb[2][TT * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Vb[2][TT * D];
  __shared__ BlockList blist;
  const int item = bwd_item(a);
  if (item >= a.n_items) return;
  const int i = item % a.QB;
  const size_t bh = item / a.QB;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  int n_pool, sc;
  const int nb = clamp_counts(a, bh, i, n_pool, sc);

  // this lane's query column: Q and dO rows as B fragments
  const int qrow = i * BT + wave * 32 + l32;
  const bool qok = qrow < a.Nq;
  bf16x8 qf[D / 16], df[D / 16];
  {
    const size_t base = (bh * a.Nq + (qok ? qrow : 0)) * (size_t)D;
    load_bfrag<D>(qf, a.q + base, qok, g);
    load_bfrag<D>(df, a.dout + base, qok, g);
  }
  const size_t prow = bh * (size_t)(a.QB * BT) + qrow;
  const float Lq = a.LDp[2 * prow];
  const float Dn = a.LDp[2 * prow + 1];  // -D of this query row
  const float sl2 = a.sl2;
  f32x16 dqacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqacc[dt][e] = 0.f;

  // A = K / V rows: tile row 32 half + l32, logical chunk 2 kk + g
  int koff[D / 16], voff[D / 16];
  {
    const int ks = lds_swz<D, kSwzU>(l32), vs = lds_swz<D, kSwzK>(l32);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      koff[kk] = l32 * D + (((2 * kk + g) ^ ks) * 8);
      voff[kk] = l32 * D + (((2 * kk + g) ^ vs) * 8);
    }
  }
  const int tbase = tr_base<D>(lane);
  uint32_t kdma[G::NVAR], vdma[G::NVAR];
  dma_lane_offsets<D, TT, NW, kSwzU>(lane, kdma);
  dma_lane_offsets<D, TT, NW, kSwzK>(lane, vdma);
  preload_list<D, BT>(a, bh, i, n_pool, sc, blist, t, 2 * BT);
  __syncthreads();

  int j = 0, h = 0;
  const uint16_t *kb, *vb;
  int blen;
  list_block<D, BT>(a, blist, bh, i, n_pool, sc, 0, kb, vb, blen);
  int tlen = min(TT, blen);
  TileDma<D, TT, NW>::tile(Kb[0], kb, tlen, wave, kdma);
  TileDma<D, TT, NW>::tile(Vb[0], vb, tlen, wave, vdma);
  int buf = 0;

  while (true) {
    PBSA_WAIT_VM(0);
    __syncthreads();
    int jn = j, hn = h + 1, nlen = 0;
    const uint16_t *kn = kb, *vn = vb;
    int bn = blen;
    if (hn * TT >= blen || hn * TT >= BT) {
      jn = j + 1;
      hn = 0;
      if (jn < nb) list_block<D, BT>(a, blist, bh, i, n_pool, sc, jn, kn, vn, bn);
    }
    const bool more = jn < nb;
    if (more) {
      nlen = min(TT, bn - hn * TT);
      TileDma<D, TT, NW>::tile(Kb[buf ^ 1], kn + hn * TT * D, nlen, wave, kdma);
      TileDma<D, TT, NW>::tile(Vb[buf ^ 1], vn + hn * TT * D, nlen, wave, vdma);
    }
    const uint16_t *Kl = Kb[buf];
    const uint16_t *Vl = Vb[buf];

#pragma unroll
    for (int hf = 0; hf < TT / 32; ++hf) {
      if (hf * 32 < tlen) {
        // S^T = K Q^T and dP^T = V dO^T over 32 tokens
        f32x16 sacc, pacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = pacc[e] = 0.f;
        // K / V fragments read PD k-steps ahead of their MFMAs (an empty asm
        // on each keeps the MFMA behind the reads)
        constexpr int PD = 2;
        bf16x8 kfr[PD + 1], vfr[PD + 1];
#pragma unroll
        for (int k0 = 0; k0 < PD; ++k0) {
          kfr[k0] = *reinterpret_cast<const bf16x8 *>(&Kl[hf * 32 * D + koff[k0]]);
          vfr[k0] = *reinterpret_cast<const bf16x8 *>(&Vl[hf * 32 * D + voff[k0]]);
        }
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          if (kk + PD < D / 16) {
            kfr[(kk + PD) % (PD + 1)] = *reinterpret_cast<const bf16x8 *>(&Kl[hf * 32 * D + koff[kk + PD]]);
            vfr[(kk + PD) % (PD + 1)] = *reinterpret_cast<const bf16x8 *>(&Vl[hf * 32 * D + voff[kk + PD]]);
          }
          asm volatile("" : "+v"(kfr[kk % (PD + 1)]), "+v"(vfr[kk % (PD + 1)]));
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[kk % (PD + 1)], qf[kk], sacc, 0, 0, 0);
          pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[kk % (PD + 1)], df[kk], pacc, 0, 0, 0);
        }
        // the exponentials and dQ MFMAs run at raised wave priority (as in
        // the forward: the other workgroup's S / dP MFMAs fill around them)
        __builtin_amdgcn_s_setprio(1);
        // dS^T = P^T (dP^T - D); tokens past the tile's length (only in the
        // ragged last tile of a block) get P = 0
        if (tlen >= hf * 32 + 32) {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            sacc[e] = __builtin_amdgcn_exp2f(sacc[e] * sl2 - Lq) * (pacc[e] + Dn);
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float p = __builtin_amdgcn_exp2f(sacc[e] * sl2 - Lq);
            if (hf * 32 + 8 * (e >> 2) + 4 * g + (e & 3) >= tlen) p = 0.f;
            sacc[e] = p * (pacc[e] + Dn);
          }
        }
        // dQ^T += K^T dS^T, 16 tokens per step
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x8 sf;
#pragma unroll
          for (int e = 0; e < 8; ++e) sf[e] = static_cast<__bf16>(sacc[8 * hh + e]);
          const uint16_t *Kst = Kl + (2 * hf + hh) * 16 * D;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
            dqacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag_u<D>(Kst, tbase, dt), sf,
                                                                dqacc[dt], 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
      }
    }
    if (!more) break;
    j = jn;
    h = hn;
    kb = kn;
    vb = vn;
    blen = bn;
    tlen = nlen;
    buf ^= 1;
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
// 4. dK, dV per stored KV block.  Items per (b, h):
//    [pool C | current QB | window W].
// ---------------------------------------------------------------------------

// (L, -D) of query rows [r0, r0 + 32) into LD[0..63] (row r at 2r, 2r+1)
// with one buffer load by wave 0: lanes 0..15 move the 256 bytes, lanes
// 16..63 are past the descriptor's range and write zeros to LD[64..255].
__device__ __forceinline__ void dma_rows_ld32(float *LD, const float *src, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(src), (short)0, 256, 0x00020000),
      (lds_void *)LD, 16, (uint32_t)lane * 16, 0, 0, 0);
}

template <int D, int BT>
__global__ __launch_bounds__(2 * BT, BT == 128 ? 2 : 1) void bwd_dkv_kernel(BwdArgs a) {
  // 32-row Q / dO tiles, two of the waves moving each (16 rows apiece);
  // separate LDS arrays per buffer half, indexed at compile time, so that
  // the compiler sees this tile's reads and the next tile's DMA touch
  // different objects
  constexpr int TT = 32, NWD = 2;
  using G = DmaGeom<D, TT, NWD>;
  __shared__ __attribute__((aligned(1024))) uint16_t Q0[TT * D], Q1[TT * D];
  __shared__ __attribute__((aligned(1024))) uint16_t O0[TT * D], O1[TT * D];  // dO rows
  __shared__ __attribute__((aligned(1024))) float LD0[256], LD1[256];  // (L, -D) per row, 64..255 zero
  uint16_t *const Qb[2] = {Q0, Q1};
  uint16_t *const Ob[2] = {O0, O1};
  float *const LD[2] = {LD0, LD1};
  const int item = bwd_item(a);
  if (item >= a.n_items) return;
  const int nj = a.C + a.W + a.QB;
  const int jb = item % nj;
  const size_t bh = item / nj;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  int n_pool = a.pool_count[bh];
  n_pool = max(0, min(n_pool, a.C));

  const uint16_t *kp, *vp;
  uint16_t *dkp, *dvp;
  int len, nq, list_base = 0;
  bool all_q = true, is_cur = false;
  if (jb < a.C) {
    const size_t off = (bh * a.C + jb) * (size_t)(BT * D);
    kp = a.k_pool + off; vp = a.v_pool + off; dkp = a.dk_pool + off; dvp = a.dv_pool + off;
    len = jb < n_pool ? max(0, min(a.pool_len[bh * a.C + jb], BT)) : 0;
  } else if (jb < a.C + a.QB) {
    const int c = jb - a.C;
    const size_t off = (bh * a.Nq + (size_t)c * BT) * D;
    kp = a.k_cur + off; vp = a.v_cur + off; dkp = a.dk_cur + off; dvp = a.dv_cur + off;
    len = min(BT, a.Nq - c * BT);
    is_cur = true;
  } else {
    const int w = jb - a.C - a.QB;
    const size_t off = (bh * a.W + w) * (size_t)(BT * D);
    kp = a.k_win + off; vp = a.v_win + off; dkp = a.dk_win + off; dvp = a.dv_win + off;
    len = max(0, min(a.win_len[w], BT));
    all_q = false;
    // with topk == 0 no query block selects any window slot, and the
    // inverse lists are not built (the launcher skips them): read nothing
    nq = 0;
    if (a.topk > 0) {
      list_base = a.qptr[bh * (a.W + 1) + w];
      nq = a.qptr[bh * (a.W + 1) + w + 1] - list_base;
    }
  }
  if (all_q) nq = a.QB;
  if (len == 0) nq = 0;
  const int32_t *ql = a.qidx + bh * a.QB * (size_t)a.topk + list_base;

  // this lane's key token: K and V rows as B fragments
  const int tok = wave * 32 + l32;
  const bool tok_ok = tok < len;
  bf16x8 kf[D / 16], vf[D / 16];
  load_bfrag<D>(kf, kp + (tok_ok ? tok : 0) * (size_t)D, tok_ok, g);
  load_bfrag<D>(vf, vp + (tok_ok ? tok : 0) * (size_t)D, tok_ok, g);
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) dkacc[dt][e] = dvacc[dt][e] = 0.f;
  const float sl2 = a.sl2;

  if (nq > 0) {
    // A = Q / dO rows: tile row 32 qs + l32, logical chunk 2 kk + g
    // (chunk 2 kk + g) ^ s = (g ^ s) ^ 2 kk: one base offset, XOR 16 kk per step
    const int rbase = l32 * D + ((g ^ lds_swz<D, kSwzU>(l32)) * 8);
    const int tbase = tr_base<D>(lane);
    uint32_t rdma[G::NVAR];
    dma_lane_offsets<D, TT, NWD, kSwzU>(lane, rdma);
    const size_t NqP = (size_t)a.QB * BT;

    // query tile stream: list entry n (query block qi), half h
    int n = 0, h = 0;
    int qi = all_q ? 0 : __builtin_amdgcn_readfirstlane(ql[0]);
    int qlen = min(BT, a.Nq - qi * BT);
    int tlen = min(TT, qlen);
    if (wave < NWD) {
      const size_t r0 = bh * a.Nq + (size_t)qi * BT;
      TileDma<D, TT, NWD>::tile(Qb[0], a.q + r0 * D, tlen, wave, rdma);
      TileDma<D, TT, NWD>::tile(Ob[0], a.dout + r0 * D, tlen, wave, rdma);
      if (wave == 0) dma_rows_ld32(LD[0], a.LDp + 2 * (bh * NqP + qi * BT), lane);
    }
    int rb = rbase, tb = tbase;
    auto step = [&](auto bufc) __attribute__((always_inline)) -> bool {
      constexpr int buf = decltype(bufc)::value;
      PBSA_WAIT_VM(0);
      __syncthreads();
      // per-step copies of the lane offsets: values derived from them are
      // formed inside the step, not held across it
      asm volatile("" : "+v"(rb), "+v"(tb));
      const int rbase = rb, tbase = tb;
      int nn = n, hn = h + 1, qin = qi, qlenn = qlen, nlen = 0;
      if (hn * TT >= qlen || hn * TT >= BT) {
        nn = n + 1;
        hn = 0;
        if (nn < nq) {
          qin = all_q ? nn : __builtin_amdgcn_readfirstlane(ql[nn]);
          qlenn = min(BT, a.Nq - qin * BT);
        }
      }
      const bool more = nn < nq;
      if (more && wave < NWD) {
        nlen = min(TT, qlenn - hn * TT);
        const size_t r0 = bh * a.Nq + (size_t)qin * BT + hn * TT;
        TileDma<D, TT, NWD>::tile(Qb[buf ^ 1], a.q + r0 * D, nlen, wave, rdma);
        TileDma<D, TT, NWD>::tile(Ob[buf ^ 1], a.dout + r0 * D, nlen, wave, rdma);
        if (wave == 0) dma_rows_ld32(LD[buf ^ 1], a.LDp + 2 * (bh * NqP + (size_t)qin * BT + hn * TT), lane);
      }
      if (more) nlen = min(TT, qlenn - hn * TT);
      const uint16_t *Ql = Qb[buf];
      const uint16_t *Ol = Ob[buf];
      const float *LDl = LD[buf];
      {
        constexpr int qs = 0;
        if (qs * 32 < tlen) {
          // S = Q K^T and dP = dO V^T over 32 query rows (element e of a
          // lane is query row 32 qs + 8 (e / 4) + 4 g + e % 4)
          // dP accumulates onto -D, so it ends as dP - D (element e of a
          // lane and float e % 4 of the LD read 4 (e / 4) share their row)
          f32x16 sacc, pacc;
#pragma unroll
          for (int m4 = 0; m4 < 4; ++m4) {
            const int r = qs * 32 + 8 * m4 + 4 * g;  // rows r .. r+3: (L, -D) pairs
            sacc[4 * m4] = sacc[4 * m4 + 1] = sacc[4 * m4 + 2] = sacc[4 * m4 + 3] = 0.f;
            pacc[4 * m4] = LDl[2 * r + 1];  // (scalar reads: fewer live registers
            pacc[4 * m4 + 1] = LDl[2 * r + 3];  //  than two 16-byte reads)
            pacc[4 * m4 + 2] = LDl[2 * r + 5];
            pacc[4 * m4 + 3] = LDl[2 * r + 7];
          }
#pragma unroll
          for (int kk = 0; kk < D / 16; ++kk) {
            const int ro = qs * 32 * D + (rbase ^ (16 * kk));
            const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(&Ql[ro]);
            const bf16x8 oa = *reinterpret_cast<const bf16x8 *>(&Ol[ro]);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], sacc, 0, 0, 0);
            pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[kk], pacc, 0, 0, 0);
          }
          // P and dS.  Rows past the query block are zero in Q, dO, L and D,
          // so they contribute nothing (P = 1, dS = 0 there).
#pragma unroll
          for (int m4 = 0; m4 < 4; ++m4) {
            const int r = qs * 32 + 8 * m4 + 4 * g;
            const f32x4 lo = *reinterpret_cast<const f32x4 *>(&LDl[2 * r]);
            const f32x4 hi = *reinterpret_cast<const f32x4 *>(&LDl[2 * r + 4]);
            const float L4[4] = {lo[0], lo[2], hi[0], hi[2]};
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const int e = 4 * m4 + e4;
              const float p = __builtin_amdgcn_exp2f(sacc[e] * sl2 - L4[e4]);
              sacc[e] = p;
              pacc[e] = p * pacc[e];
            }
          }
          // dV^T += dO^T P and dK^T += Q^T dS, 16 query rows per step
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            bf16x8 pf, sf;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              pf[e] = static_cast<__bf16>(sacc[8 * hh + e]);
              sf[e] = static_cast<__bf16>(pacc[8 * hh + e]);
            }
            const int st = (2 * qs + hh) * 16 * D;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
              dvacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag_u<D>(Ol + st, tbase, dt), pf,
                                                                  dvacc[dt], 0, 0, 0);
              dkacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag_u<D>(Ql + st, tbase, dt), sf,
                                                                  dkacc[dt], 0, 0, 0);
            }
          }
        }
      }
      if (!more) return false;
      n = nn;
      h = hn;
      qi = qin;
      qlen = qlenn;
      tlen = nlen;
      return true;
    };
    while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
    }
  }
  // this lane's token row.  Padding rows of stored slots get zeros: their
  // accumulator columns hold whatever P gave for zero K/V rows (possibly
  // not finite), so they are replaced, not scaled.  Rows past Nq of the
  // last current block do not exist.
  if (is_cur && !tok_ok) return;
  if (!tok_ok) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) dkacc[dt][e] = dvacc[dt][e] = 0.f;
  }
  uint16_t *dk = dkp + tok * (size_t)D;
  uint16_t *dv = dvp + tok * (size_t)D;
  const float ks = a.scale;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2 pk, pv;
      pk[0] = pack_bf16x2(dkacc[dt][4 * jj] * ks, dkacc[dt][4 * jj + 1] * ks);
      pk[1] = pack_bf16x2(dkacc[dt][4 * jj + 2] * ks, dkacc[dt][4 * jj + 3] * ks);
      pv[0] = pack_bf16x2(dvacc[dt][4 * jj], dvacc[dt][4 * jj + 1]);
      pv[1] = pack_bf16x2(dvacc[dt][4 * jj + 2], dvacc[dt][4 * jj + 3]);
      *reinterpret_cast<u32x2 *>(dk + dt * 32 + 8 * jj + 4 * g) = pk;
      *reinterpret_cast<u32x2 *>(dv + dt * 32 + 8 * jj + 4 * g) = pv;
    }
}

size_t bwd_ws_bytes(const pbsa_problem &p) {
  const size_t bh = (size_t)p.B * p.H;
  const size_t QB = (p.Nq + p.T - 1) / p.T;
  const size_t rows_p = bh * QB * p.T;
  return align256(2 * rows_p * sizeof(float)) + align256(bh * (p.W + 1) * sizeof(int32_t)) +
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
  const size_t rows_p = bh * a.QB * p.T;
  char *w = reinterpret_cast<char *>(ws);
  a.LDp = reinterpret_cast<float *>(w);
  w += align256(2 * rows_p * sizeof(float));
  a.qptr = reinterpret_cast<int32_t *>(w);
  w += align256(bh * (p.W + 1) * sizeof(int32_t));
  a.qidx = reinterpret_cast<int32_t *>(w);

  const int rpb = 256 / (p.d / 8);
  const unsigned rblocks = (unsigned)((rows_p + rpb - 1) / rpb);
  const int NqP = a.QB * p.T;
  if (p.d == 128)
    bwd_rows_kernel<128><<<rblocks, 256, 0, st>>>(a.o, a.dout, lse, a.LDp, rows_p, p.Nq, NqP);
  else
    bwd_rows_kernel<64><<<rblocks, 256, 0, st>>>(a.o, a.dout, lse, a.LDp, rows_p, p.Nq, NqP);
  if (p.W > 0 && p.topk > 0) {
    if ((int64_t)a.QB * p.W <= kCsrMat)
      bwd_csr_mat_kernel<<<dim3(p.H, p.B), 256, 0, st>>>(sel, sel_count, a.qptr, a.qidx, p.H, p.W,
                                                         a.QB, p.topk);
    else
      bwd_csr_kernel<<<dim3(p.H, p.B), 256, 0, st>>>(sel, sel_count, a.qptr, a.qidx, p.H, p.W,
                                                     a.QB, p.topk);
  }

  const dim3 block(2 * p.T);
#define PBSA_BWD_CASE(D_, T_)                                                     \
  if (p.d == D_ && p.T == T_) {                                                   \
    a.n_items = (int)(bh * a.QB);                                                 \
    a.per_xcd = (a.n_items + 7) / 8;                                              \
    bwd_dq_kernel<D_, T_><<<dim3(8 * a.per_xcd), block, 0, st>>>(a);              \
    a.n_items = (int)(bh * (p.C + p.W + a.QB));                                   \
    a.per_xcd = (a.n_items + 7) / 8;                                              \
    bwd_dkv_kernel<D_, T_><<<dim3(8 * a.per_xcd), block, 0, st>>>(a);             \
    return hipGetLastError();                                                     \
  }
  PBSA_BWD_CASE(128, 128)
  PBSA_BWD_CASE(64, 128)
  PBSA_BWD_CASE(128, 64)
  PBSA_BWD_CASE(64, 64)
#undef PBSA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace pbsa

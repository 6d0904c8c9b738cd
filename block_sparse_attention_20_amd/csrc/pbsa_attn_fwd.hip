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
//     in order.  K and V of a block are moved HBM -> LDS by
//     global_load_lds_dwordx4 (no register round trip) into row-major tiles
//     whose 16-byte chunks are XOR-swizzled per row; rows past the valid
//     length come from a zero page, so padding can never inject NaN;
//   - the next block's K is in flight while the softmax and P V of the
//     current block run, and its V while the next S is computed (one K and
//     one V buffer, four barriers per block);
//   - S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held
//     in registers for the whole kernel), so each lane owns one query column
//     and the row softmax is in-lane plus one cross-half exchange;
//   - online softmax in the log2 domain; the running max only moves when a
//     block raises it by more than 8 (P <= 2^8), so O is rarely rescaled;
//   - P is rounded to bf16 in registers and is directly the B operand of
//     O^T = V^T P^T; the V^T A operand is read from the row-major V tile with
//     ds_read_b64_tr_b16 (two 4x16 transposed reads per fragment);
//   - work items are mapped XCD-aware: consecutive query blocks of a head
//     run on the same XCD and share its L2 for the pool/current K/V.
// fp32 path: plain vector FMA version of the same walk (small problems).
#include "pbsa_common.h"
#include "pbsa_internal.h"

namespace pbsa {

struct FwdArgs {
  const void *q, *k_cur, *v_cur, *k_win, *v_win, *k_pool, *v_pool;
  const int32_t *win_len, *pool_len, *pool_count, *sel, *sel_count;
  void *o;
  float *lse;
  int32_t *status;
  int H, Nq, W, C, topk, QB, n_items, per_xcd;
  float sl2;  // scale * log2(e)
};

// Which stored block is entry j of query block i's attended list, and how
// many of its rows are valid.  Order: pool slots, selected window slots,
// current-chunk blocks.
template <typename TIn, int D, int BT>
__device__ __forceinline__ void resolve_block(const FwdArgs &a, size_t bh, int i, int n_pool,
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

__device__ __forceinline__ void item_of_block(const FwdArgs &a, int &item) {
  const int n = blockIdx.x;
  item = (n & 7) * a.per_xcd + (n >> 3);
}

__device__ __forceinline__ int clamp_counts(const FwdArgs &a, size_t bh, int i, int &n_pool,
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

// 256 bytes of zeros: the DMA source for rows past a block's valid length
// (padding rows and the tail of the last current block), so that they land
// in LDS as zeros without a register round trip.
__device__ __attribute__((aligned(256))) uint32_t g_zero_rows[64];

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// s_waitcnt immediate: vmcnt <= n, expcnt and lgkmcnt unconstrained (gfx9 encoding)
#define PBSA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14)))

// Stage one [BT][D] bf16 block (rows >= len read as zeros) into LDS with the
// 16-byte chunks of each row XOR-permuted by a row-dependent swizzle (K:
// row & 7; V: 2 (row & 7), or 2 (row & 3) when a row has 8 chunks).  Each
// wave moves IPW chunks of 1 KB with global_load_lds_dwordx4 (lane l lands
// at base + 16 l), so the whole block is in flight without touching VGPRs.
// Every wave's first row is a multiple of 8, so the swizzle depends only on
// the lane and the instruction index.
template <int D, int BT, int NW, bool VSWZ>
__device__ __forceinline__ void dma_block(uint16_t *lds, const uint16_t *src, int len, int wave,
                                          int lane) {
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;         // rows per 1 KB instruction
  constexpr int IPW = BT * D * 2 / 1024 / NW;
  static_assert((IPW * RPI) % 8 == 0, "wave row ranges must start at multiples of 8");
  const int p = lane % CPR, rsub = lane / CPR;
  const int row0 = wave * IPW * RPI;
  uint16_t *dst = lds + wave * IPW * 512;
  if (len >= BT) {
#pragma unroll
    for (int it = 0; it < IPW; ++it) {
      const int rl = it * RPI + rsub;  // row - row0
      const int sw = VSWZ ? (CPR == 16 ? 2 * (rl & 7) : 2 * (rl & 3)) : (rl & 7);
      __builtin_amdgcn_global_load_lds(src + (size_t)(row0 + rl) * D + (p ^ sw) * 8,
                                       (lds_void *)(dst + it * 512), 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int it = 0; it < IPW; ++it) {
      const int rl = it * RPI + rsub;
      const int sw = VSWZ ? (CPR == 16 ? 2 * (rl & 7) : 2 * (rl & 3)) : (rl & 7);
      const void *g = row0 + rl < len ? (const void *)(src + (size_t)(row0 + rl) * D + (p ^ sw) * 8)
                                      : (const void *)(g_zero_rows + p * 4);
      __builtin_amdgcn_global_load_lds(g, (lds_void *)(dst + it * 512), 16, 0, 0);
    }
  }
}

template <int D, int BT>
__global__ __launch_bounds__(2 * BT, 2) void attn_fwd_bf16_kernel(FwdArgs a) {
  constexpr int NW = BT / 32;               // waves; wave w owns query rows [32w, 32w+32)
  constexpr int CPR = D / 8;
  constexpr int IPW = BT * D * 2 / 1024 / NW;
  __shared__ __attribute__((aligned(1024))) uint16_t Kl[BT * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Vl[BT * D];

  int item;
  item_of_block(a, item);
  if (item >= a.n_items) return;
  const int i = item % a.QB;
  const size_t bh = item / a.QB;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  int n_pool, sc;
  const int nb = clamp_counts(a, bh, i, n_pool, sc);

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
  float m = -INFINITY, l = 0.f;
  const float sl2 = a.sl2;

  // Per-lane LDS element offsets, fixed for the whole kernel (the swizzle of
  // a row depends only on row & 7, which is fixed by the lane).
  // K fragment (A of S^T): row tt*32 + l32, logical chunk 2kk + g.
  int koff[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koff[kk] = l32 * D + (((2 * kk + g) ^ (l32 & 7)) * 8);
  // V^T fragment via ds_read_b64_tr_b16: in each 16-lane group, lane gi
  // addresses row gi/4 of a 4-row band (rows tt*32 + 16h + 4g + gi/4, and the
  // band 8 rows further) and 4 of the group's 16 dims; it receives dim gi of
  // the 4 rows.
  const int gi = lane & 15, q16 = (lane >> 4) & 1;
  const int vr = gi >> 2, vq = gi & 3;
  const int vsw = CPR == 16 ? 2 * ((4 * g + vr) & 7) : 2 * ((4 * g + vr) & 3);
  int voff[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
    voff[dt] = (4 * g + vr) * D + (((4 * dt + 2 * q16 + (vq >> 1)) ^ vsw) * 8) + (vq & 1) * 4;

  const uint16_t *kp, *vp;
  int len;
  resolve_block<uint16_t, D, BT>(a, bh, i, n_pool, sc, 0, kp, vp, len);
  dma_block<D, BT, NW, false>(Kl, kp, len, wave, lane);
  dma_block<D, BT, NW, true>(Vl, vp, len, wave, lane);
  PBSA_WAIT_VM(0);
  __syncthreads();

  for (int j = 0; j < nb; ++j) {
    const int len_cur = len;
    // ---- S^T[token][query] = K Q^T
    f32x16 sacc[BT / 32];
#pragma unroll
    for (int tt = 0; tt < BT / 32; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[tt][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int tt = 0; tt < BT / 32; ++tt) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(&Kl[tt * 32 * D + koff[kk]]);
        sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], sacc[tt], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave is done with K
    const bool more = j + 1 < nb;
    if (more) {
      resolve_block<uint16_t, D, BT>(a, bh, i, n_pool, sc, j + 1, kp, vp, len);
      dma_block<D, BT, NW, false>(Kl, kp, len, wave, lane);
    }
    // ---- online softmax (log2 domain); the running max only moves when a
    // block raises it by more than 8, so O is rarely rescaled and P <= 2^8.
    if (len_cur < BT) {
#pragma unroll
      for (int tt = 0; tt < BT / 32; ++tt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int tok = tt * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
          if (tok >= len_cur) sacc[tt][e] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < BT / 32; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[tt][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
    if (__ballot(mx > m + 8.f)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);  // m = -inf -> 0
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
    }
    const float muse = m == -INFINITY ? 0.f : m;
    if (!more) PBSA_WAIT_VM(0);
    else PBSA_WAIT_VM(IPW);  // V of this block has landed (K of the next may be in flight)
    __syncthreads();
    // ---- O^T += V^T P^T
#pragma unroll
    for (int tt = 0; tt < BT / 32; ++tt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(sacc[tt][8 * h + e] * sl2 - muse);
          l += p;
          pf[e] = static_cast<__bf16>(p);
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int r1 = (tt * 32 + 16 * h) * D + voff[dt];
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&Vl[r1]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&Vl[r1 + 8 * D]));
          const bf16x8 va = __builtin_bit_cast(
              bf16x8, (__attribute__((__vector_size__(8 * sizeof(short)))) short){
                          lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf, oacc[dt], 0, 0, 0);
        }
      }
    }
    if (more) {
      __syncthreads();  // every wave is done with V
      dma_block<D, BT, NW, true>(Vl, vp, len, wave, lane);
      PBSA_WAIT_VM(IPW);  // the next K has landed
      __syncthreads();
    }
  }

  // epilogue: O = O^T / l, LSE = ln(sum exp(scale s))
  l += __shfl_xor(l, 32);
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

// fp32 vector path: two threads per query row, each owns half of the dims.
template <int D, int BT>
__global__ __launch_bounds__(2 * BT) void attn_fwd_f32_kernel(FwdArgs a) {
  constexpr int NT = 2 * BT;
  constexpr int DH = D / 2;
  __shared__ __attribute__((aligned(16))) float Ks[BT * D];
  __shared__ __attribute__((aligned(16))) float Vs[BT * D];
  int item;
  item_of_block(a, item);
  if (item >= a.n_items) return;
  const int i = item % a.QB;
  const size_t bh = item / a.QB;
  const int t = threadIdx.x, r = t >> 1, hf = t & 1;
  int n_pool, sc;
  const int nb = clamp_counts(a, bh, i, n_pool, sc);
  const int qrow = i * BT + r;
  float qv[DH], ov[DH];
  const float *qp = (const float *)a.q + (bh * a.Nq + qrow) * (size_t)D + hf * DH;
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
        const float *kr = &Ks[(u < BT ? u : 0) * D + hf * DH];
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < DH; ++x) acc += qv[x] * kr[x];
        acc += __shfl_xor(acc, 1);
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
        const float *vr = &Vs[(u < BT ? u : 0) * D + hf * DH];
#pragma unroll
        for (int x = 0; x < DH; ++x) ov[x] += p * vr[x];
      }
    }
  }
  if (qrow < a.Nq) {
    float *op = (float *)a.o + (bh * a.Nq + qrow) * (size_t)D + hf * DH;
    const float inv = 1.f / l;
#pragma unroll
    for (int x = 0; x < DH; ++x) op[x] = ov[x] * inv;
    if (hf == 0 && a.lse) a.lse[bh * a.Nq + qrow] = (m + log2f(l)) * kLn2;
  }
}

hipError_t launch_attn_fwd(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                           const int32_t *sel, const int32_t *sel_count, void *o, float *lse,
                           hipStream_t st) {
  FwdArgs a;
  a.q = q;
  a.k_cur = kv.k_cur; a.v_cur = kv.v_cur; a.k_win = kv.k_win; a.v_win = kv.v_win;
  a.k_pool = kv.k_pool; a.v_pool = kv.v_pool;
  a.win_len = kv.win_len; a.pool_len = kv.pool_len; a.pool_count = kv.pool_count;
  a.sel = sel; a.sel_count = sel_count; a.o = o; a.lse = lse; a.status = p.dev_status;
  a.H = p.H; a.Nq = p.Nq; a.W = p.W; a.C = p.C; a.topk = p.topk;
  a.QB = (p.Nq + p.T - 1) / p.T;
  a.n_items = p.B * p.H * a.QB;
  a.per_xcd = (a.n_items + 7) / 8;
  a.sl2 = scale * kLog2e;
  const dim3 grid(8 * a.per_xcd);
  const dim3 block(2 * p.T);
#define PBSA_FWD_CASE(DT, D_, T_, KERN)                         \
  if (p.dtype == DT && p.d == D_ && p.T == T_) {                \
    KERN<D_, T_><<<grid, block, 0, st>>>(a);                    \
    return hipGetLastError();                                   \
  }
  PBSA_FWD_CASE(PBSA_BF16, 128, 128, attn_fwd_bf16_kernel)
  PBSA_FWD_CASE(PBSA_BF16, 64, 128, attn_fwd_bf16_kernel)
  PBSA_FWD_CASE(PBSA_BF16, 128, 64, attn_fwd_bf16_kernel)
  PBSA_FWD_CASE(PBSA_BF16, 64, 64, attn_fwd_bf16_kernel)
  PBSA_FWD_CASE(PBSA_F32, 128, 128, attn_fwd_f32_kernel)
  PBSA_FWD_CASE(PBSA_F32, 64, 128, attn_fwd_f32_kernel)
  PBSA_FWD_CASE(PBSA_F32, 128, 64, attn_fwd_f32_kernel)
  PBSA_FWD_CASE(PBSA_F32, 64, 64, attn_fwd_f32_kernel)
#undef PBSA_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace pbsa

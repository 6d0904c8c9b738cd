// PBSA coarse routing: block pooling, coarse scores, window top-k, block mass.
//
// Method: "Sparse Forcing: Native Trainable Sparse Attention for Real-time
// Autoregressive Diffusion Video Generation" (gist.science/es explainer,
// sec. 2 "Persistente Block-Sparse Attention (PBSA)": latents are split into
// blocks and compressed by pooling into representatives used for a cheap
// coarse routing; "Arquitectura Propuesta": Top-K window blocks per query,
// dynamic pool blocks chosen by a coarse score of relevance to the current
// step).  Representatives are plain means of the valid rows; the coarse
// logit is scale * <qbar, kbar>; the block mass used by the pool update is
// the coarse softmax over everything the chunk sees, summed over the
// chunk's query blocks.
//
// All of this is HBM/latency bound and tiny next to the attention: three
// launches, each far below a microsecond of arithmetic per workgroup.
#include "pbsa_common.h"
#include "pbsa_internal.h"

namespace pbsa {

// ---------------------------------------------------------------------------
// Mean of the first n rows of a [rows, d] block (row stride d), fp32 sums in a
// fixed order (deterministic).  One 256-thread workgroup per block; each
// thread loads 16 B vectors.
// ---------------------------------------------------------------------------
template <typename TIn>
__device__ void block_mean_wg(const TIn *__restrict__ src, int n, int d, float *__restrict__ out,
                              float *red /* LDS, >= 256*8 floats */) {
  constexpr int E = 16 / sizeof(TIn);  // elements per 16-byte load
  const int tpr = d / E;               // threads per row
  const int rpp = 256 / tpr;           // rows per pass
  const int t = threadIdx.x;
  const int rg = t / tpr, cg = t % tpr;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int r = rg; r < n; r += rpp) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(src + (size_t)r * d + cg * E);
    if constexpr (sizeof(TIn) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bflo(v[e]);
        acc[2 * e + 1] += bfhi(v[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(v[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[rg * d + cg * E + e] = acc[e];
  __syncthreads();
  if (t < d) {
    float s = 0.f;
    for (int g = 0; g < rpp; ++g) s += red[g * d + t];
    out[t] = n > 0 ? s / (float)n : 0.f;
  }
  __syncthreads();
}

// grid (QB, H, B*2): z even = Q -> qbar (workspace), z odd = K_cur -> kbar_cur
template <typename TIn>
__global__ __launch_bounds__(256) void chunk_means_kernel(const TIn *__restrict__ q,
                                                          const TIn *__restrict__ k,
                                                          float *__restrict__ qbar,
                                                          float *__restrict__ kbar, int H, int Nq,
                                                          int d, int T, int QB) {
  __shared__ float red[256 * 8];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z >> 1, which = blockIdx.z & 1;
  const size_t bh = (size_t)b * H + h;
  const int r0 = i * T;
  const int n = min(T, Nq - r0);
  const TIn *src = (which ? k : q) + (bh * Nq + r0) * d;
  float *dst = (which ? kbar : qbar) + (bh * QB + i) * d;
  block_mean_wg<TIn>(src, n, d, dst, red);
}

// grid (n_blocks): means of stored slot blocks [n, T, d] with lengths
template <typename TIn>
__global__ __launch_bounds__(256) void slot_means_kernel(const TIn *__restrict__ x,
                                                         const int32_t *__restrict__ len,
                                                         float *__restrict__ out, int d, int T,
                                                         int32_t *status) {
  __shared__ float red[256 * 8];
  const size_t blk = blockIdx.x;
  int n = len ? len[blk] : T;
  if (n < 0 || n > T) {
    if (threadIdx.x == 0) set_status(status, PBSA_STATUS_WIN_LEN);
    n = max(0, min(n, T));
  }
  block_mean_wg<TIn>(x + blk * (size_t)T * d, n, d, out + blk * d, red);
}

// ---------------------------------------------------------------------------
// Coarse scores + window top-k + per-row block softmax.
// grid (QB, H, B), 256 threads.  Dynamic LDS: s[C+W+QB] floats, flags.
// Top-k is rank based: a valid window slot is selected iff fewer than k
// valid slots rank before it in the total order (score desc, id asc, NaN
// last); its output position is the number of selected slots below it.
// This is exact and order-independent, so it is deterministic.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void score_topk_kernel(
    const float *__restrict__ qbar, const float *__restrict__ kbar_pool,
    const float *__restrict__ kbar_win, const float *__restrict__ kbar_cur,
    const int32_t *__restrict__ pool_count, const int32_t *__restrict__ win_len,
    const int64_t *__restrict__ win_id, int32_t *__restrict__ sel, int32_t *__restrict__ sel_count,
    float *__restrict__ pi, int H, int d, int T, int W, int C, int QB, int topk, float scale,
    int32_t *status) {
  extern __shared__ float smem[];
  float *qv = smem;                     // [d]
  float *s = qv + 128;                  // [C + W + QB]
  int *flag = reinterpret_cast<int *>(s + C + W + QB);  // [W]: 1 valid, 2 selected
  __shared__ float red[8];
  __shared__ int nvalid_sh;

  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * H + h;
  const int t = threadIdx.x;
  int n_pool = pool_count[bh];
  if (n_pool < 0 || n_pool > C) {
    if (t == 0) set_status(status, PBSA_STATUS_POOL_COUNT);
    n_pool = max(0, min(n_pool, C));
  }
  if (t < d) qv[t] = qbar[(bh * QB + i) * d + t];
  if (t == 0) nvalid_sh = 0;
  __syncthreads();

  const int nj = C + W + QB;  // candidate layout: [pool C | window W | current QB]
  for (int j = t; j < nj; j += 256) {
    const float *kb = nullptr;
    bool valid;
    if (j < C) {
      valid = j < n_pool;
      kb = kbar_pool + (bh * C + j) * d;
    } else if (j < C + W) {
      const int w = j - C;
      const int len = win_len[w];
      valid = len > 0;
      if (len > T && t == 0) set_status(status, PBSA_STATUS_WIN_LEN);
      kb = kbar_win + (bh * W + w) * d;
      flag[w] = valid ? 1 : 0;
    } else {
      valid = true;
      kb = kbar_cur + (bh * QB + (j - C - W)) * d;
    }
    float acc = 0.f;
    if (valid) {
      for (int e = 0; e < d; e += 4) {
        const f32x4 kv4 = *reinterpret_cast<const f32x4 *>(kb + e);
        acc += qv[e] * kv4[0];
        acc += qv[e + 1] * kv4[1];
        acc += qv[e + 2] * kv4[2];
        acc += qv[e + 3] * kv4[3];
      }
      acc *= scale;
    }
    s[j] = valid ? acc : -INFINITY;
  }
  __syncthreads();

  // row max / sum over the valid candidates (NaN propagates through the sum)
  float mx = -INFINITY;
  for (int j = t; j < nj; j += 256) mx = fmaxf(mx, s[j]);
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (int j = t; j < nj; j += 256) sum += expf(s[j] - mx);  // invalid: exp(-inf) = 0
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if ((t & 63) == 0) red[4 + (t >> 6)] = sum;
  __syncthreads();
  sum = (red[4] + red[5]) + (red[6] + red[7]);
  const float inv = 1.f / sum;
  float *pirow = pi + (bh * QB + i) * (size_t)(C + W);
  for (int j = t; j < C + W; j += 256) pirow[j] = expf(s[j] - mx) * inv;

  // rank-based top-k over the valid window slots
  int cnt = 0;
  for (int w = t; w < W; w += 256) cnt += flag[w] & 1;
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  if ((t & 63) == 0) atomicAdd(&nvalid_sh, cnt);
  for (int w = t; w < W; w += 256) {
    if (!(flag[w] & 1)) continue;
    const float sw = s[C + w];
    const int64_t iw = win_id[w];
    int rank = 0;
    for (int v = 0; v < W; ++v)
      if ((flag[v] & 1) && v != w && ranks_before(s[C + v], win_id[v], sw, iw)) ++rank;
    if (rank < topk) flag[w] |= 2;
  }
  __syncthreads();
  const int n_sel = min(topk, nvalid_sh);
  int32_t *selrow = sel + (bh * QB + i) * (size_t)topk;
  for (int w = t; w < W; w += 256) {
    if (!(flag[w] & 2)) continue;
    int pos = 0;
    for (int v = 0; v < w; ++v) pos += (flag[v] >> 1) & 1;
    selrow[pos] = w;
  }
  for (int p = n_sel + t; p < topk; p += 256) selrow[p] = -1;
  if (t == 0) sel_count[bh * QB + i] = n_sel;
}

// mass[j] = sum_i pi[i][j] in ascending i (deterministic).  grid (H, B).
__global__ __launch_bounds__(256) void mass_reduce_kernel(const float *__restrict__ pi,
                                                          float *__restrict__ mass_pool,
                                                          float *__restrict__ mass_win, int H,
                                                          int W, int C, int QB) {
  const size_t bh = (size_t)blockIdx.y * H + blockIdx.x;
  const int CW = C + W;
  for (int j = threadIdx.x; j < CW; j += 256) {
    const float *col = pi + bh * QB * (size_t)CW + j;
    float s = 0.f;
    for (int i = 0; i < QB; ++i) s += col[(size_t)i * CW];
    if (j < C)
      mass_pool[bh * C + j] = s;
    else
      mass_win[bh * W + (j - C)] = s;
  }
}

// ---------------------------------------------------------------------------
// Ring advance: copy the current chunk's blocks into window slots.
// grid (QB, H, B), 256 threads.
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ __launch_bounds__(256) void window_append_kernel(
    const TIn *__restrict__ k_cur, const TIn *__restrict__ v_cur, const float *__restrict__ kbar_cur,
    TIn *__restrict__ k_win, TIn *__restrict__ v_win, float *__restrict__ kbar_win,
    int32_t *__restrict__ win_len, int64_t *__restrict__ win_id, int H, int Nq, int d, int T,
    int W, int QB, int first_slot, int64_t first_id) {
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * H + h;
  const int slot = first_slot + j;
  const int n = min(T, Nq - j * T);
  constexpr int E = 16 / sizeof(TIn);
  const size_t nvec = (size_t)n * d / E;
  const u32x4 *ks = reinterpret_cast<const u32x4 *>(k_cur + (bh * Nq + (size_t)j * T) * d);
  const u32x4 *vs = reinterpret_cast<const u32x4 *>(v_cur + (bh * Nq + (size_t)j * T) * d);
  u32x4 *kd = reinterpret_cast<u32x4 *>(k_win + (bh * W + slot) * (size_t)T * d);
  u32x4 *vd = reinterpret_cast<u32x4 *>(v_win + (bh * W + slot) * (size_t)T * d);
  for (size_t e = threadIdx.x; e < nvec; e += 256) {
    kd[e] = ks[e];
    vd[e] = vs[e];
  }
  for (int e = threadIdx.x; e < d; e += 256)
    kbar_win[(bh * W + slot) * d + e] = kbar_cur[(bh * QB + j) * d + e];
  if (bh == 0 && threadIdx.x == 0) {
    win_len[slot] = n;
    win_id[slot] = first_id + j;
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
size_t select_ws_bytes(const pbsa_problem &p) {
  const size_t QB = (p.Nq + p.T - 1) / p.T;
  const size_t bh = (size_t)p.B * p.H;
  return align256(bh * QB * p.d * sizeof(float)) + align256(bh * QB * (p.C + p.W) * sizeof(float));
}

size_t select_lds_bytes(const pbsa_problem &p) {
  const int QB = (p.Nq + p.T - 1) / p.T;
  return (128 + (size_t)p.C + p.W + QB) * sizeof(float) + (size_t)p.W * sizeof(int);
}

hipError_t launch_select(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                         int32_t *sel, int32_t *sel_count, float *mass_pool, float *mass_win,
                         void *ws, hipStream_t st) {
  const int QB = (p.Nq + p.T - 1) / p.T;
  const size_t bh = (size_t)p.B * p.H;
  float *qbar = reinterpret_cast<float *>(ws);
  float *pi = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) +
                                        align256(bh * QB * p.d * sizeof(float)));
  dim3 g1(QB, p.H, p.B * 2);
  if (p.dtype == PBSA_BF16)
    chunk_means_kernel<uint16_t><<<g1, 256, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)kv.k_cur, qbar, kv.kbar_cur, p.H, p.Nq, p.d, p.T, QB);
  else
    chunk_means_kernel<float><<<g1, 256, 0, st>>>((const float *)q, (const float *)kv.k_cur, qbar,
                                                  kv.kbar_cur, p.H, p.Nq, p.d, p.T, QB);
  dim3 g2(QB, p.H, p.B);
  score_topk_kernel<<<g2, 256, select_lds_bytes(p), st>>>(
      qbar, kv.kbar_pool, kv.kbar_win, kv.kbar_cur, kv.pool_count, kv.win_len, kv.win_id, sel,
      sel_count, pi, p.H, p.d, p.T, p.W, p.C, QB, p.topk, scale, p.dev_status);
  dim3 g3(p.H, p.B);
  mass_reduce_kernel<<<g3, 256, 0, st>>>(pi, mass_pool, mass_win, p.H, p.W, p.C, QB);
  return hipGetLastError();
}

hipError_t launch_block_mean(const pbsa_problem &p, const void *x, const int32_t *len,
                             int64_t n_blocks, float *out, hipStream_t st) {
  if (n_blocks == 0) return hipSuccess;
  if (p.dtype == PBSA_BF16)
    slot_means_kernel<uint16_t><<<dim3((unsigned)n_blocks), 256, 0, st>>>(
        (const uint16_t *)x, len, out, p.d, p.T, p.dev_status);
  else
    slot_means_kernel<float><<<dim3((unsigned)n_blocks), 256, 0, st>>>((const float *)x, len, out,
                                                                        p.d, p.T, p.dev_status);
  return hipGetLastError();
}

hipError_t launch_window_append(const pbsa_problem &p, const pbsa_kv &kv, void *k_win, void *v_win,
                                float *kbar_win, int32_t *win_len, int64_t *win_id,
                                int first_slot, int64_t first_id, hipStream_t st) {
  const int QB = (p.Nq + p.T - 1) / p.T;
  dim3 g(QB, p.H, p.B);
  if (p.dtype == PBSA_BF16)
    window_append_kernel<uint16_t><<<g, 256, 0, st>>>(
        (const uint16_t *)kv.k_cur, (const uint16_t *)kv.v_cur, kv.kbar_cur, (uint16_t *)k_win,
        (uint16_t *)v_win, kbar_win, win_len, win_id, p.H, p.Nq, p.d, p.T, p.W, QB, first_slot,
        first_id);
  else
    window_append_kernel<float><<<g, 256, 0, st>>>(
        (const float *)kv.k_cur, (const float *)kv.v_cur, kv.kbar_cur, (float *)k_win,
        (float *)v_win, kbar_win, win_len, win_id, p.H, p.Nq, p.d, p.T, p.W, QB, first_slot,
        first_id);
  return hipGetLastError();
}

}  // namespace pbsa

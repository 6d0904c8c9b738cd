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
// All of this is HBM/latency bound and tiny next to the attention.  The
// window top-k of a query block needs only the block's own query mean and
// the cached pool/window representatives, so the critical path is one
// launch per query block: its own query and key means, pool and window
// scores, top-k.  The scores against the current chunk's blocks (whose means
// are spread over all the query blocks' workgroups) are needed only for the
// block masses, and are formed by the block-mass kernel, which runs later.
#include "pbsa_common.h"
#include "pbsa_internal.h"
#include "pbsa_select_dev.h"

#include <mutex>

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
#pragma unroll 4
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
// Own-block means, coarse scores + window top-k (select_query_block, shared
// with the fused select + forward kernel).  grid (QB, H, B), 256 threads.
// Dynamic LDS: window ids [W] int64, keys [W], flags [W], ranks [W].
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ __launch_bounds__(256) void score_topk_kernel(SelArgs<TIn> s) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ __attribute__((aligned(16))) float qv[128];
  __shared__ float red[2 * 256 * 8];
  __shared__ float both[256];
  __shared__ int nvalid_sh;
  __shared__ int wcnt[4];
  const SelLds L{qv, red, both, smem, &nvalid_sh, wcnt, nullptr, nullptr, nullptr};
  select_query_block<TIn>(s, blockIdx.x, (size_t)blockIdx.z * s.H + blockIdx.y, L);
}

// ---------------------------------------------------------------------------
// Block mass per (b, h): M_j = sum_i softmax_j(s_i.), the softmax over every
// candidate of query block i (pool, window and current blocks); written for
// the pool and window slots (0 where invalid).  One workgroup of 1024
// threads per (b, h) (latency bound: many waves in flight); the score rows
// are staged into LDS in chunks of rows; sums run over i in ascending order
// (deterministic).  grid (H, B).
// ---------------------------------------------------------------------------
constexpr int kMassLds = 12288;  // floats of staged scores
constexpr int kMassThreads = 1024;

__global__ __launch_bounds__(kMassThreads) void block_mass_kernel(
    const float *__restrict__ srows, const float *__restrict__ qbar, const float *__restrict__ kbarc,
    float *__restrict__ mass_pool, float *__restrict__ mass_win, int H, int W, int C, int QB, int d,
    float scale) {
  __shared__ float sbuf[kMassLds];
  __shared__ float rmax[kMassThreads / 64 * 16], rinv[kMassThreads / 64 * 16];
  const size_t bh = (size_t)blockIdx.y * H + blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  constexpr int NWV = kMassThreads / 64;
  const int sub = lane >> 4, sl = lane & 15, per = d / 16;
  const int nj = C + W + QB;
  const int rows_per = max(1, min(NWV * 16, kMassLds / nj));
  const float *src = srows + bh * QB * (size_t)nj;
  float acc[2] = {0.f, 0.f};  // columns t and t + 1024 (C + W <= 2048)
  for (int r0 = 0; r0 < QB; r0 += rows_per) {
    const int nr = min(rows_per, QB - r0);
    __syncthreads();
    const float *s0 = src + (size_t)r0 * nj;
    // pool and window scores from the select kernel ...
#pragma unroll 8
    for (int e = t; e < nr * nj; e += kMassThreads)
      if (e % nj < C + W) sbuf[e] = s0[e];
    // ... and the current-chunk scores s_rj = scale <qbar_r, kbar_cur_j>,
    // 16 lanes per dot product (the select kernel's summation order).  A
    // wave takes a row (its query mean loaded once), its four 16-lane groups
    // columns j = sub, sub + 4, ..., with kMassU column loads in flight.
    constexpr int kMassU = 4;
    for (int r = wave; r < nr; r += NWV) {
      const float *qq = qbar + (bh * QB + r0 + r) * (size_t)d + sl * per;
      const f32x4 q0 = *reinterpret_cast<const f32x4 *>(qq);
      f32x4 q1 = {0.f, 0.f, 0.f, 0.f};
      if (per == 8) q1 = *reinterpret_cast<const f32x4 *>(qq + 4);
      for (int j0 = sub; j0 < QB; j0 += 4 * kMassU) {
        f32x4 k0[kMassU], k1[kMassU];
#pragma unroll
        for (int u = 0; u < kMassU; ++u) {
          const int j = j0 + 4 * u;
          k0[u] = k1[u] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (j < QB) {
            const float *kk = kbarc + (bh * QB + j) * (size_t)d + sl * per;
            k0[u] = *reinterpret_cast<const f32x4 *>(kk);
            if (per == 8) k1[u] = *reinterpret_cast<const f32x4 *>(kk + 4);
          }
        }
#pragma unroll
        for (int u = 0; u < kMassU; ++u) {
          const int j = j0 + 4 * u;
          if (j < QB) {  // the same for all 16 lanes of a group
            float acc = q0[0] * k0[u][0] + q0[1] * k0[u][1] + q0[2] * k0[u][2] + q0[3] * k0[u][3];
            if (per == 8)
              acc += q1[0] * k1[u][0] + q1[1] * k1[u][1] + q1[2] * k1[u][2] + q1[3] * k1[u][3];
            acc += __shfl_xor(acc, 1);
            acc += __shfl_xor(acc, 2);
            acc += __shfl_xor(acc, 4);
            acc += __shfl_xor(acc, 8);
            if (sl == 0) sbuf[r * nj + C + W + j] = acc * scale;
          }
        }
      }
    }
    __syncthreads();
    // per-row max and 1/sum, one wave per row
    for (int r = wave; r < nr; r += NWV) {
      float mx = -INFINITY;
      for (int j = lane; j < nj; j += 64) mx = fmaxf(mx, sbuf[r * nj + j]);
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      float sm = 0.f;
      for (int j = lane; j < nj; j += 64) sm += __expf(sbuf[r * nj + j] - mx);
      for (int o = 32; o > 0; o >>= 1) sm += __shfl_xor(sm, o);
      if (lane == 0) {
        rmax[r] = mx;
        rinv[r] = 1.f / sm;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = t + kMassThreads * q;
      if (j < C + W) {
        float a = acc[q];
#pragma unroll 4
        for (int r = 0; r < nr; ++r) a += __expf(sbuf[r * nj + j] - rmax[r]) * rinv[r];
        acc[q] = a;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int j = t + kMassThreads * q;
    if (j < C)
      mass_pool[bh * C + j] = acc[q];
    else if (j < C + W)
      mass_win[bh * W + (j - C)] = acc[q];
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
// Select workspace: query-block means [bh][QB][d], score rows
// [bh][QB][C + W + QB] (pool, window, current), copies of the current
// blocks' key means [bh][QB][d] for the block-mass kernel.
size_t select_ws_bytes(const pbsa_problem &p) {
  const size_t QB = (p.Nq + p.T - 1) / p.T;
  const size_t bh = (size_t)p.B * p.H;
  return 2 * align256(bh * QB * p.d * sizeof(float)) +
         align256(bh * QB * (p.C + p.W + QB) * sizeof(float));
}

void select_ws_layout(const pbsa_problem &p, const void *ws, float *&qbar, float *&srows,
                      float *&kbarc) {
  const size_t QB = (p.Nq + p.T - 1) / p.T;
  const size_t bh = (size_t)p.B * p.H;
  char *w = reinterpret_cast<char *>(const_cast<void *>(ws));
  qbar = reinterpret_cast<float *>(w);
  w += align256(bh * QB * p.d * sizeof(float));
  srows = reinterpret_cast<float *>(w);
  w += align256(bh * QB * (p.C + p.W + QB) * sizeof(float));
  kbarc = reinterpret_cast<float *>(w);
}

size_t select_lds_bytes(const pbsa_problem &p) {
  return (size_t)p.W * (sizeof(uint32_t) + 2 * sizeof(int) + sizeof(int64_t));
}

hipError_t launch_select(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                         int32_t *sel, int32_t *sel_count, float *mass_pool, float *mass_win,
                         bool masses, void *ws, hipStream_t st) {
  const int QB = (p.Nq + p.T - 1) / p.T;
  const dim3 g(QB, p.H, p.B);
  if (p.dtype == PBSA_BF16)
    score_topk_kernel<uint16_t><<<g, 256, select_lds_bytes(p), st>>>(
        sel_args<uint16_t>(p, scale, q, kv, sel, sel_count, ws));
  else
    score_topk_kernel<float><<<g, 256, select_lds_bytes(p), st>>>(
        sel_args<float>(p, scale, q, kv, sel, sel_count, ws));
  if (masses) return launch_block_mass(p, scale, mass_pool, mass_win, ws, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Allocation-free select: the same launches with their workspace in a
// file-scope device array.  Each GPU the library runs on holds its own copy
// of the array, at its own address, until the process ends; its address on
// a device comes from hipGetSymbolAddress with that device current (taken
// on the first call on the device and kept).  The array's name is a host
// stand-in and is never passed to a kernel.  Calls on one device share the
// array, so calls that overlap in time on one device race.  Every byte the
// kernels read is written earlier in the same call, so nothing needs
// clearing between calls.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kSelectScratchBytes];

constexpr int kMaxScratchDevices = 64;

static hipError_t scratch_address(void **out) {
  static std::mutex mu;
  static void *addr[kMaxScratchDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_select_static(const pbsa_problem &p, float scale, const void *q,
                                const pbsa_kv &kv, int32_t *sel, int32_t *sel_count,
                                float *mass_pool, float *mass_win, bool masses, hipStream_t st) {
  if (select_ws_bytes(p) > kSelectScratchBytes) return hipErrorInvalidValue;
  void *ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_select(p, scale, q, kv, sel, sel_count, mass_pool, mass_win, masses, ws, st);
}

hipError_t launch_block_mass(const pbsa_problem &p, float scale, float *mass_pool,
                             float *mass_win, const void *ws, hipStream_t st) {
  const int QB = (p.Nq + p.T - 1) / p.T;
  float *qbar, *srows, *kbarc;
  select_ws_layout(p, ws, qbar, srows, kbarc);
  if (p.C + p.W > 0)
    block_mass_kernel<<<dim3(p.H, p.B), kMassThreads, 0, st>>>(srows, qbar, kbarc, mass_pool,
                                                                mass_win, p.H, p.W, p.C, QB, p.d,
                                                                scale);
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

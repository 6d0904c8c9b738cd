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
// launches (block means; scores + top-k per query block; block mass per
// head), each written so its global loads are in flight together.
#include "pbsa_common.h"
#include "pbsa_internal.h"

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

// grid (QB, H, B*2): z even = Q -> qbar (workspace), z odd = K_cur -> kbar_cur.
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
// Coarse scores + window top-k.  grid (QB, H, B), 256 threads.
//  - candidates [pool C | window W | current QB], 16 lanes per candidate
//    (coalesced 16-byte reads of kbar, 4 shuffles); all of a pass's loads
//    are issued before any is used;
//  - the score row goes to the workspace for the block-mass kernel;
//  - top-k is rank based: a valid window slot is selected iff fewer than k
//    valid slots rank before it in the total order (score desc, id asc, NaN
//    last); its output position is the number of selected slots below it.
//    Exact and order-independent, hence deterministic.  Scores enter the
//    ranking as order keys (order_key; 0 = invalid slot), so the pairwise
//    comparisons are branch free.
// Dynamic LDS: q[128] floats, window ids [W] int64, keys [W], flags [W],
// ranks [W].
// ---------------------------------------------------------------------------
// 16 candidates per pass; 9 passes cover the 143 candidates of the Wan
// chunk (pool 32 + window 74 + 37 current blocks) with one batch of loads:
// 16.3 us for means + scores + top-k there, against 18.6 us with 8 (which
// needs a second, almost empty batch) and 16.5 us with 3 or 5.
constexpr int kScorePasses = 9;

__global__ __launch_bounds__(256) void score_topk_kernel(
    const float *__restrict__ qbar, const float *__restrict__ kbar_pool,
    const float *__restrict__ kbar_win, const float *__restrict__ kbar_cur,
    const int32_t *__restrict__ pool_count, const int32_t *__restrict__ win_len,
    const int64_t *__restrict__ win_id, int32_t *__restrict__ sel, int32_t *__restrict__ sel_count,
    float *__restrict__ srow_out, int H, int d, int T, int W, int C, int QB, int topk, float scale,
    int32_t *status) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float *qv = smem;                                        // [128]
  int64_t *wid = reinterpret_cast<int64_t *>(qv + 128);   // [W]
  uint32_t *key = reinterpret_cast<uint32_t *>(wid + W);  // [W]: order keys
  int *flag = reinterpret_cast<int *>(key + W);           // [W]: 1 valid, 2 selected
  int *rank = flag + W;                                    // [W]
  __shared__ int nvalid_sh;
  __shared__ int wcnt[4];

  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * H + h;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int n_pool = pool_count[bh];
  if (n_pool < 0 || n_pool > C) {
    if (t == 0) set_status(status, PBSA_STATUS_POOL_COUNT);
    n_pool = max(0, min(n_pool, C));
  }
  if (t < d) qv[t] = qbar[(bh * QB + i) * d + t];
  int nv = 0;
  for (int w = t; w < W; w += 256) {
    const int len = win_len[w];
    if (len > T) set_status(status, PBSA_STATUS_WIN_LEN);
    flag[w] = len > 0 ? 1 : 0;
    nv += len > 0;
    wid[w] = win_id[w];
  }
  if (t == 0) nvalid_sh = 0;
  __syncthreads();
  for (int o = 32; o > 0; o >>= 1) nv += __shfl_xor(nv, o);
  if (lane == 0) atomicAdd(&nvalid_sh, nv);

  const int nj = C + W + QB;
  const int sub = lane >> 4, sl = lane & 15;
  const int per = d / 16;  // floats per lane (8 or 4)
  float *srow = srow_out + (bh * QB + i) * (size_t)nj;
  for (int base = wave * 4; base < nj; base += 16 * kScorePasses) {
    f32x4 k0[kScorePasses], k1[kScorePasses];
    bool ok[kScorePasses];
#pragma unroll
    for (int ps = 0; ps < kScorePasses; ++ps) {
      const int j = base + ps * 16 + sub;
      const float *kb = kbar_pool;
      bool valid = false;
      if (j < C) {
        valid = j < n_pool;
        kb = kbar_pool + (bh * C + j) * d;
      } else if (j < C + W) {
        valid = flag[j - C] != 0;
        kb = kbar_win + (bh * W + (j - C)) * d;
      } else if (j < nj) {
        valid = true;
        kb = kbar_cur + (bh * QB + (j - C - W)) * d;
      }
      ok[ps] = valid;
      k0[ps] = f32x4{0.f, 0.f, 0.f, 0.f};
      k1[ps] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (valid) {
        k0[ps] = *reinterpret_cast<const f32x4 *>(kb + sl * per);
        if (per == 8) k1[ps] = *reinterpret_cast<const f32x4 *>(kb + sl * per + 4);
      }
    }
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
        const float v = ok[ps] ? acc * scale : -INFINITY;
        srow[j] = v;
        if (j >= C && j < C + W) key[j - C] = ok[ps] ? order_key(v) : 0u;
      }
    }
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
  int32_t *selrow = sel + (bh * QB + i) * (size_t)topk;
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
    if (bit && pos < topk) selrow[pos] = w;  // more than k only with duplicate ids
    carry += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    __syncthreads();
  }
  for (int p = n_sel + t; p < topk; p += 256) selrow[p] = -1;
  if (t == 0) sel_count[bh * QB + i] = n_sel;
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

__global__ __launch_bounds__(kMassThreads) void block_mass_kernel(const float *__restrict__ srows,
                                                                  float *__restrict__ mass_pool,
                                                                  float *__restrict__ mass_win,
                                                                  int H, int W, int C, int QB) {
  __shared__ float sbuf[kMassLds];
  __shared__ float rmax[kMassThreads / 64 * 16], rinv[kMassThreads / 64 * 16];
  const size_t bh = (size_t)blockIdx.y * H + blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  constexpr int NWV = kMassThreads / 64;
  const int nj = C + W + QB;
  const int rows_per = max(1, min(NWV * 16, kMassLds / nj));
  const float *src = srows + bh * QB * (size_t)nj;
  float acc[2] = {0.f, 0.f};  // columns t and t + 1024 (C + W <= 2048)
  for (int r0 = 0; r0 < QB; r0 += rows_per) {
    const int nr = min(rows_per, QB - r0);
    __syncthreads();
    const float *s0 = src + (size_t)r0 * nj;
#pragma unroll 8
    for (int e = t; e < nr * nj; e += kMassThreads) sbuf[e] = s0[e];
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
size_t select_ws_bytes(const pbsa_problem &p) {
  const size_t QB = (p.Nq + p.T - 1) / p.T;
  const size_t bh = (size_t)p.B * p.H;
  return align256(bh * QB * p.d * sizeof(float)) +
         align256(bh * QB * (p.C + p.W + QB) * sizeof(float));
}

size_t select_lds_bytes(const pbsa_problem &p) {
  return 128 * sizeof(float) + (size_t)p.W * (sizeof(uint32_t) + 2 * sizeof(int) + sizeof(int64_t));
}

hipError_t launch_select(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                         int32_t *sel, int32_t *sel_count, float *mass_pool, float *mass_win,
                         bool masses, void *ws, hipStream_t st) {
  const int QB = (p.Nq + p.T - 1) / p.T;
  const size_t bh = (size_t)p.B * p.H;
  float *qbar = reinterpret_cast<float *>(ws);
  char *wsb = reinterpret_cast<char *>(ws);
  float *srows = reinterpret_cast<float *>(wsb + align256(bh * QB * p.d * sizeof(float)));
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
      sel_count, srows, p.H, p.d, p.T, p.W, p.C, QB, p.topk, scale, p.dev_status);
  if (masses) return launch_block_mass(p, mass_pool, mass_win, ws, st);
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

hipError_t launch_block_mass(const pbsa_problem &p, float *mass_pool, float *mass_win,
                             const void *ws, hipStream_t st) {
  const int QB = (p.Nq + p.T - 1) / p.T;
  const size_t bh = (size_t)p.B * p.H;
  const char *wsb = reinterpret_cast<const char *>(ws);
  const float *srows = reinterpret_cast<const float *>(wsb + align256(bh * QB * p.d * sizeof(float)));
  if (p.C + p.W > 0)
    block_mass_kernel<<<dim3(p.H, p.B), kMassThreads, 0, st>>>(srows, mass_pool, mass_win, p.H, p.W,
                                                                p.C, QB);
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

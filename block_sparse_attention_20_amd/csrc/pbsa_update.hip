// PBSA persistent-memory update: Top-C retention with pinned sinks, slot
// placement, and bit-exact block copies.
//
// Method: "Sparse Forcing: Native Trainable Sparse Attention for Real-time
// Autoregressive Diffusion Video Generation" (gist.science/es explainer,
// sec. 2 "Arquitectura Propuesta": the persistent memory holds sink blocks
// (fixed global anchors) and dynamic blocks chosen by coarse scoring; Top-C
// retention keeps the C best-scored blocks and discards the less relevant
// blocks leaving the local window).  The kernel is the "selective cache
// update" the same page credits the PBSA kernel with.
//
// Two launches: a decision kernel per (b, h) that ranks the candidates and
// computes where each admitted block goes, and an HBM-bound copy kernel
// (one workgroup per admitted block) that moves K/V/kbar.
#include "pbsa_common.h"
#include "pbsa_internal.h"

namespace pbsa {

constexpr int kMaxC = 1024;
constexpr int kMaxLeave = 1024;
constexpr int kMaxX = kMaxC + kMaxLeave;

__global__ __launch_bounds__(256) void update_decide_kernel(
    const float *__restrict__ mass_pool, const float *__restrict__ mass_win,
    const int32_t *__restrict__ leaving, int n_leave, const int32_t *__restrict__ win_len,
    const int64_t *__restrict__ win_id, int32_t *__restrict__ pool_len,
    int64_t *__restrict__ pool_id, int32_t *__restrict__ pool_count, int32_t *__restrict__ a_slot,
    int32_t *__restrict__ a_src, int32_t *__restrict__ a_count, int H, int W, int C, int T,
    int64_t n_sink, int shared, int32_t *status) {
  __shared__ int64_t xid[kMaxX];
  __shared__ uint32_t xk[kMaxX];   // order key of the candidate's mass (order_key)
  __shared__ int32_t xsrc[kMaxX];   // >= 0: pool slot; < 0: window slot -1-w
  __shared__ int8_t xkeep[kMaxX];
  __shared__ int8_t cflag[kMaxLeave];
  __shared__ int32_t free_slot[kMaxC];
  __shared__ int32_t lw[kMaxLeave], lwl[kMaxLeave];
  __shared__ int64_t lid[kMaxLeave];
  __shared__ int red[4];

  const int t = threadIdx.x;
  const size_t bh = (size_t)blockIdx.y * H + blockIdx.x;
  int n_pool = pool_count[bh];
  if (n_pool < 0 || n_pool > C) {
    if (t == 0) set_status(status, PBSA_STATUS_POOL_COUNT);
    n_pool = max(0, min(n_pool, C));
  }
  // head-shared pool: every head of batch element b ranks by the masses
  // summed over its heads (ascending h, so every head computes the same
  // sums); the heads hold the same blocks in the same slots
  const size_t b0 = (size_t)blockIdx.y * H;
  for (int p = t; p < n_pool; p += 256) {
    xid[p] = pool_id[bh * C + p];
    float m = mass_pool[bh * C + p];
    if (shared) {
      m = 0.f;
      for (int h2 = 0; h2 < H; ++h2) m += mass_pool[(b0 + h2) * C + p];
    }
    xk[p] = order_key(m);
    xsrc[p] = p;
  }
  // stage the leaving slots' metadata (wl = -1 marks a slot out of range)
  for (int c = t; c < n_leave; c += 256) {
    const int w = leaving[c];
    const bool inr = w >= 0 && w < W;
    if (!inr) set_status(status, PBSA_STATUS_SEL);
    lw[c] = w;
    lwl[c] = inr ? win_len[w] : -1;
    lid[c] = inr ? win_id[w] : -1;
  }
  __syncthreads();
  // candidate filter: slot in range, non-empty, not pooled, first of its id
  for (int c = t; c < n_leave; c += 256) {
    const int64_t id = lid[c];
    bool ok = lwl[c] > 0;
#pragma unroll 8
    for (int p = 0; p < n_pool; ++p) ok &= xid[p] != id;
#pragma unroll 8
    for (int c2 = 0; c2 < c; ++c2) ok &= !((lwl[c2] > 0) & (lid[c2] == id));
    cflag[c] = ok ? 1 : 0;
  }
  __syncthreads();
  for (int c = t; c < n_leave; c += 256) {
    if (!cflag[c]) continue;
    int pos = n_pool;
#pragma unroll 8
    for (int c2 = 0; c2 < c; ++c2) pos += cflag[c2];
    const int w = lw[c];
    xid[pos] = lid[c];
    float m = mass_win[bh * W + w];
    if (shared) {
      m = 0.f;
      for (int h2 = 0; h2 < H; ++h2) m += mass_win[(b0 + h2) * W + w];
    }
    xk[pos] = order_key(m);
    xsrc[pos] = -1 - w;
  }
  int nc = 0, np = 0;
  for (int c = t; c < n_leave; c += 256) nc += cflag[c];
  for (int o = 32; o > 0; o >>= 1) nc += __shfl_xor(nc, o);
  if ((t & 63) == 0) red[t >> 6] = nc;
  __syncthreads();
  const int n_x = n_pool + red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  for (int x = t; x < n_x; x += 256) np += xid[x] < n_sink;
  for (int o = 32; o > 0; o >>= 1) np += __shfl_xor(np, o);
  if ((t & 63) == 0) red[t >> 6] = np;
  __syncthreads();
  const int n_pin = red[0] + red[1] + red[2] + red[3];
  if (n_x > C && n_pin > C && t == 0) set_status(status, PBSA_STATUS_SINK);
  for (int x = t; x < n_x; x += 256) {
    bool keep;
    const bool pin = xid[x] < n_sink;
    if (n_x <= C) {
      keep = true;
    } else if (n_pin > C) {  // more sinks than room: the C smallest ids
      int r = 0;
      for (int y = 0; y < n_x; ++y) r += (int)((xid[y] < n_sink) & (xid[y] < xid[x]));
      keep = pin && r < C;
    } else if (pin) {
      keep = true;
    } else {
      int r = 0;
      const uint32_t kxx = xk[x];
      const int64_t ixx = xid[x];
      // branch free: candidate y ranks before x iff its key is larger, or
      // equal with a smaller id (mass descending, id ascending, NaN last)
#pragma unroll 8
      for (int y = 0; y < n_x; ++y) {
        const uint32_t ky = xk[y];
        const int64_t iy = xid[y];
        r += (int)((iy >= n_sink) & ((ky > kxx) | ((ky == kxx) & (iy < ixx))));
      }
      keep = r < C - n_pin;
    }
    xkeep[x] = keep ? 1 : 0;
  }
  __syncthreads();
  // free slots: evicted pool slots and the unused tail, ascending
  for (int s = t; s < C; s += 256) {
    const bool fr = s >= n_pool || !xkeep[s];
    if (!fr) continue;
    int pos = 0;
#pragma unroll 8
    for (int s2 = 0; s2 < s; ++s2) pos += (int)((s2 >= n_pool) | !xkeep[s2]);
    free_slot[pos] = s;
  }
  __syncthreads();
  int nk = 0, na = 0;
  for (int x = t; x < n_x; x += 256) {
    nk += xkeep[x];
    if (x < n_pool || !xkeep[x]) continue;
    int pos = 0;  // rank among the admitted by id (ids are unique)
    const int64_t ixx = xid[x];
#pragma unroll 8
    for (int y = n_pool; y < n_x; ++y) pos += (int)((xkeep[y] != 0) & (xid[y] < ixx));
    const int slot = free_slot[pos];
    const int w = -1 - xsrc[x];
    a_slot[bh * C + pos] = slot;
    a_src[bh * C + pos] = w;
    pool_len[bh * C + slot] = min(max(win_len[w], 0), T);
    pool_id[bh * C + slot] = xid[x];
    ++na;
  }
  for (int o = 32; o > 0; o >>= 1) {
    nk += __shfl_xor(nk, o);
    na += __shfl_xor(na, o);
  }
  __syncthreads();
  if ((t & 63) == 0) red[t >> 6] = nk;
  __syncthreads();
  if (t == 0) pool_count[bh] = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  if ((t & 63) == 0) red[t >> 6] = na;
  __syncthreads();
  if (t == 0) a_count[bh] = red[0] + red[1] + red[2] + red[3];
}

// Head-shared pool precondition, checked before the decisions (which then
// rewrite the pool metadata): every head of batch element blockIdx.x holds
// head 0's count and ids; otherwise PBSA_STATUS_SHARED.
__global__ __launch_bounds__(256) void update_shared_check_kernel(const int64_t *__restrict__ pool_id,
                                                                  const int32_t *__restrict__ pool_count,
                                                                  int H, int C, int32_t *status) {
  const size_t b0 = (size_t)blockIdx.x * H;
  const int n0 = pool_count[b0];
  bool bad = false;
  for (int x = threadIdx.x; x < H * C; x += 256) {
    const int h = x / C, p = x % C;
    if (p == 0 && pool_count[b0 + h] != n0) bad = true;
    if (p < n0 && p < C && pool_id[(b0 + h) * C + p] != pool_id[b0 * C + p]) bad = true;
  }
  if (bad) set_status(status, PBSA_STATUS_SHARED);
}

// grid (A, H, B): workgroup a copies admitted block a of (b, h) from its
// window slot into its pool slot (K and V: all T rows; kbar: d floats).
__global__ __launch_bounds__(256) void update_copy_kernel(
    const uint8_t *__restrict__ k_win, const uint8_t *__restrict__ v_win,
    const float *__restrict__ kbar_win, uint8_t *__restrict__ k_pool, uint8_t *__restrict__ v_pool,
    float *__restrict__ kbar_pool, const int32_t *__restrict__ a_slot,
    const int32_t *__restrict__ a_src, const int32_t *__restrict__ a_count, int H, int W, int C,
    int d, size_t block_bytes) {
  const int a = blockIdx.x;
  const size_t bh = (size_t)blockIdx.z * H + blockIdx.y;
  if (a >= a_count[bh]) return;
  const int slot = a_slot[bh * C + a];
  const int w = a_src[bh * C + a];
  const size_t nvec = block_bytes / 16;
  const u32x4 *ks = reinterpret_cast<const u32x4 *>(k_win + (bh * W + w) * block_bytes);
  const u32x4 *vs = reinterpret_cast<const u32x4 *>(v_win + (bh * W + w) * block_bytes);
  u32x4 *kd = reinterpret_cast<u32x4 *>(k_pool + (bh * C + slot) * block_bytes);
  u32x4 *vd = reinterpret_cast<u32x4 *>(v_pool + (bh * C + slot) * block_bytes);
  for (size_t e = threadIdx.x; e < nvec; e += 256) {
    const u32x4 x = ks[e];
    const u32x4 y = vs[e];
    kd[e] = x;
    vd[e] = y;
  }
  for (int e = threadIdx.x; e < d; e += 256) kbar_pool[(bh * C + slot) * d + e] = kbar_win[(bh * W + w) * d + e];
}

size_t update_ws_bytes(const pbsa_problem &p) {
  const size_t bh = (size_t)p.B * p.H;
  return 2 * align256(bh * p.C * sizeof(int32_t)) + align256(bh * sizeof(int32_t));
}

hipError_t launch_memory_update(const pbsa_problem &p, const pbsa_kv &kv, const float *mass_pool,
                                const float *mass_win, const int32_t *leaving, int n_leave,
                                int64_t n_sink, bool shared, void *ws, hipStream_t st) {
  const size_t bh = (size_t)p.B * p.H;
  char *w = reinterpret_cast<char *>(ws);
  int32_t *a_slot = reinterpret_cast<int32_t *>(w);
  int32_t *a_src = reinterpret_cast<int32_t *>(w + align256(bh * p.C * sizeof(int32_t)));
  int32_t *a_count = reinterpret_cast<int32_t *>(w + 2 * align256(bh * p.C * sizeof(int32_t)));
  if (shared && p.dev_status)
    update_shared_check_kernel<<<p.B, 256, 0, st>>>(kv.pool_id, kv.pool_count, p.H, p.C, p.dev_status);
  update_decide_kernel<<<dim3(p.H, p.B), 256, 0, st>>>(
      mass_pool, mass_win, leaving, n_leave, kv.win_len, kv.win_id, kv.pool_len, kv.pool_id,
      kv.pool_count, a_slot, a_src, a_count, p.H, p.W, p.C, p.T, n_sink, shared ? 1 : 0,
      p.dev_status);
  const int A = n_leave < p.C ? n_leave : p.C;
  if (A > 0) {
    const size_t esz = p.dtype == PBSA_BF16 ? 2 : 4;
    update_copy_kernel<<<dim3(A, p.H, p.B), 256, 0, st>>>(
        (const uint8_t *)kv.k_win, (const uint8_t *)kv.v_win, kv.kbar_win, (uint8_t *)kv.k_pool,
        (uint8_t *)kv.v_pool, kv.kbar_pool, a_slot, a_src, a_count, p.H, p.W, p.C, p.d,
        (size_t)p.T * p.d * esz);
  }
  return hipGetLastError();
}

}  // namespace pbsa

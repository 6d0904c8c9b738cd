// Training through a streaming rollout: moving stored blocks and their
// gradients between the rollout's history and the pool / window slots.
//
// Method: "Sparse Forcing: Native Trainable Sparse Attention for Real-time
// Autoregressive Diffusion Video Generation" (gist.science/es explainer,
// sec. 2 "Arquitectura Propuesta" and "Persistente Block-Sparse Attention
// (PBSA)"; shd-paper.top summary: the sparse attention is trainable).  A
// pool or window slot holds a bit-exact copy of a block of an earlier chunk
// (block id = chunk * QB + j: rows [j T, min(Nq, (j + 1) T)) of that chunk's
// K and V), so
//   - block_gather rebuilds the slots a chunk attended from the history, and
//   - grad_scatter adds the gradient a slot received (pbsa_attn_bwd's
//     dk/dv_win, dk/dv_pool, or dk/dv_cur for the chunk itself) to those rows
//     of the chunk's fp32 gradient accumulator.
// Both are HBM-bound copies: one workgroup per (slot, head, batch element),
// 16-byte vector accesses.
#include "pbsa_common.h"
#include "pbsa_internal.h"

namespace pbsa {

struct SlotMap {
  const int64_t *ids;  // block id per slot; < 0 = empty
  int64_t ids_bh_stride;  // 0: one id list for every (b, h)
  const int32_t *count;   // optional [B,H]: slots >= count are skipped / empty
  int n_slots, H, Nq, T, d, QB, n_chunks, B;
  int32_t *status;
};

// rows of slot `slot` of (b, h): chunk c, first row r0, n valid rows (0 =
// empty or skipped)
__device__ __forceinline__ void slot_rows(const SlotMap &m, size_t bh, int slot, int &c, int &r0,
                                          int &n) {
  n = 0;
  c = 0;
  r0 = 0;
  if (m.count) {
    const int cnt = m.count[bh];
    if (slot >= cnt) return;
  }
  const int64_t id = m.ids[bh * m.ids_bh_stride + slot];
  if (id < 0) return;
  const int64_t cc = id / m.QB;
  if (cc >= m.n_chunks) {
    set_status(m.status, PBSA_STATUS_SEL);
    return;
  }
  c = (int)cc;
  const int j = (int)(id % m.QB);
  r0 = j * m.T;
  n = min(m.T, m.Nq - r0);
}

// grid (n_slots, H, B): slot rows from the history into [B,H,n_slots,T,d];
// rows past the block's length are zeroed; len_out (optional) gets n
__global__ __launch_bounds__(256) void block_gather_kernel(SlotMap m, const uint8_t *__restrict__ k_hist,
                                                           const uint8_t *__restrict__ v_hist,
                                                           uint8_t *__restrict__ k_out,
                                                           uint8_t *__restrict__ v_out,
                                                           int32_t *__restrict__ len_out, int esz) {
  const int slot = blockIdx.x;
  const size_t bh = (size_t)blockIdx.z * m.H + blockIdx.y;
  int c, r0, n;
  slot_rows(m, bh, slot, c, r0, n);
  const size_t row_bytes = (size_t)m.d * esz;
  const size_t nv_all = (size_t)m.T * row_bytes / 16, nv = (size_t)n * row_bytes / 16;
  const size_t src = (((size_t)c * m.B * m.H + bh) * m.Nq + r0) * row_bytes;
  const size_t dst = (bh * m.n_slots + slot) * (size_t)m.T * row_bytes;
  const u32x4 *ks = reinterpret_cast<const u32x4 *>(k_hist + src);
  const u32x4 *vs = reinterpret_cast<const u32x4 *>(v_hist + src);
  u32x4 *kd = reinterpret_cast<u32x4 *>(k_out + dst);
  u32x4 *vd = reinterpret_cast<u32x4 *>(v_out + dst);
  const u32x4 z = {0, 0, 0, 0};
  for (size_t e = threadIdx.x; e < nv_all; e += 256) {
    const bool in = e < nv;
    kd[e] = in ? ks[e] : z;
    vd[e] = in ? vs[e] : z;
  }
  if (len_out && threadIdx.x == 0) len_out[bh * m.n_slots + slot] = n;
}

// grid (n_slots, H, B): g[c][b,h,r0 + r,:] += src rows of the slot, for its
// valid rows r.  The source is slot-shaped [B,H,n_slots,T,d] (rows of slot s
// start at s T) or chunk-shaped [B,H,Nq,d] (rows of block j start at j T).
template <typename TIn>
__global__ __launch_bounds__(256) void grad_scatter_kernel(SlotMap m, const TIn *__restrict__ dk,
                                                           const TIn *__restrict__ dv,
                                                           float *__restrict__ gk,
                                                           float *__restrict__ gv, int src_is_chunk) {
  const int slot = blockIdx.x;
  const size_t bh = (size_t)blockIdx.z * m.H + blockIdx.y;
  int c, r0, n;
  slot_rows(m, bh, slot, c, r0, n);
  if (n == 0) return;
  const size_t cnt = (size_t)n * m.d;  // elements, a multiple of 4
  const size_t src = src_is_chunk ? (bh * m.Nq + r0) * (size_t)m.d
                                  : (bh * m.n_slots + slot) * (size_t)m.T * m.d;
  const size_t dst = (((size_t)c * m.B * m.H + bh) * m.Nq + r0) * m.d;
  for (size_t e = 4 * threadIdx.x; e < cnt; e += 4 * 256) {
    f32x4 a = *reinterpret_cast<const f32x4 *>(gk + dst + e);
    f32x4 b = *reinterpret_cast<const f32x4 *>(gv + dst + e);
    if constexpr (sizeof(TIn) == 2) {
      const u32x2 xk = *reinterpret_cast<const u32x2 *>(dk + src + e);
      const u32x2 xv = *reinterpret_cast<const u32x2 *>(dv + src + e);
      a[0] += bflo(xk[0]); a[1] += bfhi(xk[0]); a[2] += bflo(xk[1]); a[3] += bfhi(xk[1]);
      b[0] += bflo(xv[0]); b[1] += bfhi(xv[0]); b[2] += bflo(xv[1]); b[3] += bfhi(xv[1]);
    } else {
      const f32x4 xk = *reinterpret_cast<const f32x4 *>(dk + src + e);
      const f32x4 xv = *reinterpret_cast<const f32x4 *>(dv + src + e);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        a[x] += xk[x];
        b[x] += xv[x];
      }
    }
    *reinterpret_cast<f32x4 *>(gk + dst + e) = a;
    *reinterpret_cast<f32x4 *>(gv + dst + e) = b;
  }
}

static SlotMap make_map(const pbsa_problem &p, const int64_t *ids, int64_t ids_bh_stride,
                        const int32_t *count, int n_slots, int n_chunks) {
  SlotMap m;
  m.ids = ids;
  m.ids_bh_stride = ids_bh_stride;
  m.count = count;
  m.n_slots = n_slots;
  m.H = p.H;
  m.B = p.B;
  m.Nq = p.Nq;
  m.T = p.T;
  m.d = p.d;
  m.QB = (p.Nq + p.T - 1) / p.T;
  m.n_chunks = n_chunks;
  m.status = p.dev_status;
  return m;
}

hipError_t launch_block_gather(const pbsa_problem &p, const int64_t *ids, int64_t ids_bh_stride,
                               const int32_t *count, int n_slots, const void *k_hist,
                               const void *v_hist, int n_chunks, void *k_out, void *v_out,
                               int32_t *len_out, hipStream_t st) {
  if (n_slots == 0) return hipSuccess;
  const SlotMap m = make_map(p, ids, ids_bh_stride, count, n_slots, n_chunks);
  const int esz = p.dtype == PBSA_BF16 ? 2 : 4;
  block_gather_kernel<<<dim3(n_slots, p.H, p.B), 256, 0, st>>>(
      m, (const uint8_t *)k_hist, (const uint8_t *)v_hist, (uint8_t *)k_out, (uint8_t *)v_out,
      len_out, esz);
  return hipGetLastError();
}

hipError_t launch_grad_scatter(const pbsa_problem &p, const int64_t *ids, int64_t ids_bh_stride,
                               const int32_t *count, int n_slots, int src_is_chunk,
                               const void *dk, const void *dv, float *gk, float *gv, int n_chunks,
                               hipStream_t st) {
  if (n_slots == 0) return hipSuccess;
  const SlotMap m = make_map(p, ids, ids_bh_stride, count, n_slots, n_chunks);
  const dim3 grid(n_slots, p.H, p.B);
  const int ch = src_is_chunk ? 1 : 0;
  if (p.dtype == PBSA_BF16)
    grad_scatter_kernel<uint16_t><<<grid, 256, 0, st>>>(m, (const uint16_t *)dk, (const uint16_t *)dv,
                                                        gk, gv, ch);
  else
    grad_scatter_kernel<float><<<grid, 256, 0, st>>>(m, (const float *)dk, (const float *)dv, gk, gv, ch);
  return hipGetLastError();
}

}  // namespace pbsa

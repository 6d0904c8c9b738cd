// Internal launcher declarations shared by the PBSA host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pbsa.h"

namespace pbsa {

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t select_ws_bytes(const pbsa_problem &p);
// largest select workspace the allocation-free select holds (8 MiB: the
// Wan chunk needs 0.5 MB, batch 8 of it 3.9 MB)
constexpr size_t kSelectScratchBytes = size_t(8) << 20;
size_t select_lds_bytes(const pbsa_problem &p);
// select workspace: query-block means, score rows, current-block key means
void select_ws_layout(const pbsa_problem &p, const void *ws, float *&qbar, float *&srows,
                      float *&kbarc);
size_t update_ws_bytes(const pbsa_problem &p);
size_t fwd_ws_bytes(const pbsa_problem &p);
size_t fwd_mass_ws_bytes(const pbsa_problem &p);
size_t bwd_ws_bytes(const pbsa_problem &p);
size_t fine_ws_bytes(const pbsa_problem &p);

hipError_t launch_select(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                         int32_t *sel, int32_t *sel_count, float *mass_pool, float *mass_win,
                         bool masses, void *ws, hipStream_t st);
hipError_t launch_select_static(const pbsa_problem &p, float scale, const void *q,
                                const pbsa_kv &kv, int32_t *sel, int32_t *sel_count,
                                float *mass_pool, float *mass_win, bool masses, hipStream_t st);
hipError_t launch_block_mass(const pbsa_problem &p, float scale, float *mass_pool,
                             float *mass_win, const void *ws, hipStream_t st);
hipError_t launch_block_mean(const pbsa_problem &p, const void *x, const int32_t *len,
                             int64_t n_blocks, float *out, hipStream_t st);
hipError_t launch_window_append(const pbsa_problem &p, const pbsa_kv &kv, void *k_win, void *v_win,
                                float *kbar_win, int32_t *win_len, int64_t *win_id,
                                int first_slot, int64_t first_id, hipStream_t st);
hipError_t launch_attn_fwd(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                           const int32_t *sel, const int32_t *sel_count, void *o, float *lse,
                           void *ws, size_t ws_bytes, hipStream_t st);
// select (no masses) + forward in one launch where the problem allows it
// (bf16, d = T = 128, C + topk <= 128, W <= 819, no split), else the two
// launches; ws = the select workspace, fwd_ws the forward's (optional)
hipError_t launch_select_attn_fwd(const pbsa_problem &p, float scale, const void *q,
                                  const pbsa_kv &kv, int32_t *sel, int32_t *sel_count, void *o,
                                  float *lse, void *ws, void *fwd_ws, size_t fwd_ws_bytes,
                                  hipStream_t st);
hipError_t launch_attn_fwd_mass(const pbsa_problem &p, float scale, const void *q,
                                const pbsa_kv &kv, const int32_t *sel, const int32_t *sel_count,
                                void *o, float *lse, float *mass_pool, float *mass_win, void *ws,
                                size_t ws_bytes, hipStream_t st);
hipError_t launch_attn_bwd(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                           const int32_t *sel, const int32_t *sel_count, const void *o,
                           const float *lse, const void *dout, void *dq, const pbsa_kv_grad &g,
                           void *ws, hipStream_t st);
hipError_t launch_fine_mass(const pbsa_problem &p, float scale, const void *q, const pbsa_kv &kv,
                            const int32_t *sel, const int32_t *sel_count, const float *lse,
                            float *mass_pool, float *mass_win, void *ws, hipStream_t st);
hipError_t launch_block_gather(const pbsa_problem &p, const int64_t *ids, int64_t ids_bh_stride,
                               const int32_t *count, int n_slots, const void *k_hist,
                               const void *v_hist, int n_chunks, void *k_out, void *v_out,
                               int32_t *len_out, hipStream_t st);
hipError_t launch_grad_scatter(const pbsa_problem &p, const int64_t *ids, int64_t ids_bh_stride,
                               const int32_t *count, int n_slots, int src_is_chunk,
                               const void *dk, const void *dv, float *gk, float *gv, int n_chunks,
                               hipStream_t st);
hipError_t launch_memory_update(const pbsa_problem &p, const pbsa_kv &kv, const float *mass_pool,
                                const float *mass_win, const int32_t *leaving, int n_leave,
                                int64_t n_sink, bool shared, void *ws, hipStream_t st);

}  // namespace pbsa

// PBSA C ABI: host-side validation, error reporting, workspace sizing and
// dispatch to the kernels.  Everything here runs on the host; nothing
// synchronises.  See include/pbsa.h for the contract of each entry point.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "pbsa_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return PBSA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

#define REQ(ptr)                                                         \
  do {                                                                   \
    if (!(ptr)) return fail(PBSA_ERR_NULL, "%s must not be NULL", #ptr); \
    if (!aligned16(ptr))                                                 \
      return fail(PBSA_ERR_ALIGN, "%s is not 16-byte aligned", #ptr);    \
  } while (0)

int check_problem(const pbsa_problem *p, int op) {
  if (!p) return fail(PBSA_ERR_NULL, "problem must not be NULL");
  if (p->dtype != PBSA_BF16 && p->dtype != PBSA_F32)
    return fail(PBSA_ERR_DTYPE, "dtype %d is neither PBSA_BF16 nor PBSA_F32", p->dtype);
  if (p->B < 1 || p->H < 1) return fail(PBSA_ERR_SHAPE, "B=%d H=%d must be >= 1", p->B, p->H);
  if (p->d < 1 || p->T < 1) return fail(PBSA_ERR_SHAPE, "d=%d T=%d must be >= 1", p->d, p->T);
  if (p->Nq < 1) return fail(PBSA_ERR_SHAPE, "Nq=%d must be >= 1", p->Nq);
  if (p->W < 0 || p->W > 1024) return fail(PBSA_ERR_SHAPE, "W=%d outside [0, 1024]", p->W);
  if (p->C < 0 || p->C > 1024) return fail(PBSA_ERR_SHAPE, "C=%d outside [0, 1024]", p->C);
  if (p->topk < 0 || p->topk > p->W)
    return fail(PBSA_ERR_SHAPE, "topk=%d outside [0, W=%d]", p->topk, p->W);
  if (!(p->scale >= 0.f) || isinf(p->scale))
    return fail(PBSA_ERR_SHAPE, "scale must be finite and >= 0 (0 = 1/sqrt(d))");
  if ((p->d != 64 && p->d != 128) || (p->T != 64 && p->T != 128))
    return fail(PBSA_ERR_UNSUPPORTED, "d=%d T=%d: supported d in {64,128}, T in {64,128}",
                p->d, p->T);
  const long long QB = (p->Nq + (long long)p->T - 1) / p->T;
  const long long rows = (long long)p->B * p->H * QB;
  if (rows > (1LL << 30)) return fail(PBSA_ERR_SHAPE, "B*H*QB=%lld too large", rows);
  if (op == PBSA_OP_SELECT && QB + p->C + p->W > 12000)
    return fail(PBSA_ERR_SHAPE, "QB+C+W=%lld exceeds the coarse-routing limit 12000",
                QB + p->C + p->W);
  if (p->dev_status && !aligned16(p->dev_status) && (reinterpret_cast<uintptr_t>(p->dev_status) & 3))
    return fail(PBSA_ERR_ALIGN, "dev_status must be 4-byte aligned");
  return PBSA_OK;
}

float eff_scale(const pbsa_problem *p) { return p->scale > 0.f ? p->scale : 1.f / sqrtf((float)p->d); }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return ok();
  return fail(PBSA_ERR_HIP, "HIP error %d: %s", (int)e, hipGetErrorString(e));
}

int check_ws(const pbsa_problem *p, int op, const void *ws, size_t ws_bytes) {
  const size_t need = pbsa_workspace_size(p, op);
  if (need == 0) return PBSA_OK;
  if (!ws) return fail(PBSA_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (!aligned16(ws)) return fail(PBSA_ERR_ALIGN, "ws is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(PBSA_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
  return PBSA_OK;
}

int check_kv_common(const pbsa_kv *kv, const pbsa_problem *p) {
  if (!kv) return fail(PBSA_ERR_NULL, "kv must not be NULL");
  REQ(kv->k_cur);
  REQ(kv->v_cur);
  REQ(kv->pool_count);
  if (p->W > 0) {
    REQ(kv->k_win);
    REQ(kv->v_win);
    REQ(kv->win_len);
    REQ(kv->win_id);
  }
  if (p->C > 0) {
    REQ(kv->k_pool);
    REQ(kv->v_pool);
    REQ(kv->pool_len);
    REQ(kv->pool_id);
  }
  return PBSA_OK;
}

}  // namespace

extern "C" {

const char *pbsa_last_error(void) { return g_err; }

const char *pbsa_strerror(int status) {
  switch (status) {
    case PBSA_OK: return "ok";
    case PBSA_ERR_NULL: return "NULL pointer";
    case PBSA_ERR_SHAPE: return "size out of range";
    case PBSA_ERR_DTYPE: return "unknown dtype";
    case PBSA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PBSA_ERR_WORKSPACE: return "workspace missing or too small";
    case PBSA_ERR_HIP: return "HIP runtime error";
    case PBSA_ERR_UNSUPPORTED: return "unsupported configuration";
    default: return "unknown status";
  }
}

int pbsa_validate(const pbsa_problem *p, int op) {
  if (op < PBSA_OP_SELECT || op > PBSA_OP_FWD_MASS) return fail(PBSA_ERR_SHAPE, "unknown op %d", op);
  int rc = check_problem(p, op);
  return rc ? rc : ok();
}

size_t pbsa_workspace_size(const pbsa_problem *p, int op) {
  if (!p || check_problem(p, op) != PBSA_OK) return 0;
  switch (op) {
    case PBSA_OP_SELECT: return pbsa::select_ws_bytes(*p);
    case PBSA_OP_FWD: return pbsa::fwd_ws_bytes(*p);
    case PBSA_OP_BWD: return pbsa::bwd_ws_bytes(*p);
    case PBSA_OP_UPDATE: return pbsa::update_ws_bytes(*p);
    case PBSA_OP_FINE_MASS: return pbsa::fine_ws_bytes(*p);
    case PBSA_OP_FWD_MASS: return pbsa::fwd_mass_ws_bytes(*p);
    default: return 0;
  }
}

int pbsa_select(const pbsa_problem *p, const void *q, const pbsa_kv *kv, int32_t *sel,
                int32_t *sel_count, float *mass_pool, float *mass_win, void *ws,
                size_t ws_bytes, pbsa_stream_t stream) {
  int rc = check_problem(p, PBSA_OP_SELECT);
  if (rc) return rc;
  REQ(q);
  if ((rc = check_kv_common(kv, p))) return rc;
  REQ(kv->kbar_cur);
  if (p->W > 0) REQ(kv->kbar_win);
  if (p->C > 0) REQ(kv->kbar_pool);
  if (p->topk > 0) REQ(sel);
  REQ(sel_count);
  const bool masses = mass_pool != nullptr || mass_win != nullptr;
  if (masses && p->C > 0) REQ(mass_pool);
  if (masses && p->W > 0) REQ(mass_win);
  if ((rc = check_ws(p, PBSA_OP_SELECT, ws, ws_bytes))) return rc;
  return hip_status(pbsa::launch_select(*p, eff_scale(p), q, *kv, sel, sel_count,
                                        masses ? mass_pool : nullptr, masses ? mass_win : nullptr,
                                        masses, ws, (hipStream_t)stream));
}

int pbsa_select_static(const pbsa_problem *p, const void *q, const pbsa_kv *kv, int32_t *sel,
                       int32_t *sel_count, float *mass_pool, float *mass_win,
                       pbsa_stream_t stream) {
  int rc = check_problem(p, PBSA_OP_SELECT);
  if (rc) return rc;
  REQ(q);
  if ((rc = check_kv_common(kv, p))) return rc;
  REQ(kv->kbar_cur);
  if (p->W > 0) REQ(kv->kbar_win);
  if (p->C > 0) REQ(kv->kbar_pool);
  if (p->topk > 0) REQ(sel);
  REQ(sel_count);
  const bool masses = mass_pool != nullptr || mass_win != nullptr;
  if (masses && p->C > 0) REQ(mass_pool);
  if (masses && p->W > 0) REQ(mass_win);
  const size_t need = pbsa::select_ws_bytes(*p);
  if (need > pbsa::kSelectScratchBytes)
    return fail(PBSA_ERR_WORKSPACE,
                "this problem needs %zu bytes of select scratch; the static scratch holds %zu "
                "(use pbsa_select with a workspace)",
                need, pbsa::kSelectScratchBytes);
  return hip_status(pbsa::launch_select_static(*p, eff_scale(p), q, *kv, sel, sel_count,
                                               masses ? mass_pool : nullptr,
                                               masses ? mass_win : nullptr, masses,
                                               (hipStream_t)stream));
}

int pbsa_block_mass(const pbsa_problem *p, float *mass_pool, float *mass_win, const void *ws,
                    size_t ws_bytes, pbsa_stream_t stream) {
  int rc = check_problem(p, PBSA_OP_SELECT);
  if (rc) return rc;
  if (p->C > 0) REQ(mass_pool);
  if (p->W > 0) REQ(mass_win);
  if ((rc = check_ws(p, PBSA_OP_SELECT, ws, ws_bytes))) return rc;
  return hip_status(pbsa::launch_block_mass(*p, eff_scale(p), mass_pool, mass_win, ws,
                                            (hipStream_t)stream));
}

int pbsa_attn_fwd(const pbsa_problem *p, const void *q, const pbsa_kv *kv, const int32_t *sel,
                  const int32_t *sel_count, void *o, float *lse, void *ws, size_t ws_bytes,
                  pbsa_stream_t stream) {
  int rc = check_problem(p, PBSA_OP_FWD);
  if (rc) return rc;
  REQ(q);
  if ((rc = check_kv_common(kv, p))) return rc;
  if (p->topk > 0) REQ(sel);
  REQ(sel_count);
  REQ(o);
  if (lse && !aligned16(lse)) return fail(PBSA_ERR_ALIGN, "lse is not 16-byte aligned");
  if (ws != nullptr && !aligned16(ws)) return fail(PBSA_ERR_ALIGN, "ws is not 16-byte aligned");
  return hip_status(pbsa::launch_attn_fwd(*p, eff_scale(p), q, *kv, sel, sel_count, o, lse, ws,
                                          ws_bytes, (hipStream_t)stream));
}

int pbsa_select_attn_fwd(const pbsa_problem *p, const void *q, const pbsa_kv *kv, int32_t *sel,
                         int32_t *sel_count, void *o, float *lse, void *ws, size_t ws_bytes,
                         void *fwd_ws, size_t fwd_ws_bytes, pbsa_stream_t stream) {
  int rc = check_problem(p, PBSA_OP_SELECT);
  if (rc) return rc;
  REQ(q);
  if ((rc = check_kv_common(kv, p))) return rc;
  REQ(kv->kbar_cur);
  if (p->W > 0) REQ(kv->kbar_win);
  if (p->C > 0) REQ(kv->kbar_pool);
  if (p->topk > 0) REQ(sel);
  REQ(sel_count);
  REQ(o);
  if (lse && !aligned16(lse)) return fail(PBSA_ERR_ALIGN, "lse is not 16-byte aligned");
  if ((rc = check_ws(p, PBSA_OP_SELECT, ws, ws_bytes))) return rc;
  if (fwd_ws != nullptr && !aligned16(fwd_ws))
    return fail(PBSA_ERR_ALIGN, "fwd_ws is not 16-byte aligned");
  return hip_status(pbsa::launch_select_attn_fwd(*p, eff_scale(p), q, *kv, sel, sel_count, o, lse,
                                                 ws, fwd_ws, fwd_ws_bytes, (hipStream_t)stream));
}

int pbsa_attn_bwd(const pbsa_problem *p, const void *q, const pbsa_kv *kv, const int32_t *sel,
                  const int32_t *sel_count, const void *o, const float *lse, const void *dout,
                  void *dq, const pbsa_kv_grad *g, void *ws, size_t ws_bytes,
                  pbsa_stream_t stream) {
  int rc = check_problem(p, PBSA_OP_BWD);
  if (rc) return rc;
  if (p->dtype != PBSA_BF16) return fail(PBSA_ERR_UNSUPPORTED, "pbsa_attn_bwd supports bf16 only");
  REQ(q);
  if ((rc = check_kv_common(kv, p))) return rc;
  if (p->topk > 0) REQ(sel);
  REQ(sel_count);
  REQ(o);
  REQ(lse);
  REQ(dout);
  REQ(dq);
  if (!g) return fail(PBSA_ERR_NULL, "g must not be NULL");
  REQ(g->dk_cur);
  REQ(g->dv_cur);
  if (p->W > 0) {
    REQ(g->dk_win);
    REQ(g->dv_win);
  }
  if (p->C > 0) {
    REQ(g->dk_pool);
    REQ(g->dv_pool);
  }
  if ((rc = check_ws(p, PBSA_OP_BWD, ws, ws_bytes))) return rc;
  return hip_status(pbsa::launch_attn_bwd(*p, eff_scale(p), q, *kv, sel, sel_count, o, lse, dout,
                                          dq, *g, ws, (hipStream_t)stream));
}

int pbsa_fine_mass(const pbsa_problem *p, const void *q, const pbsa_kv *kv, const int32_t *sel,
                   const int32_t *sel_count, const float *lse, float *mass_pool, float *mass_win,
                   void *ws, size_t ws_bytes, pbsa_stream_t stream) {
  int rc = check_problem(p, PBSA_OP_FINE_MASS);
  if (rc) return rc;
  REQ(q);
  if ((rc = check_kv_common(kv, p))) return rc;
  if (p->topk > 0) REQ(sel);
  REQ(sel_count);
  REQ(lse);
  if (p->C > 0) REQ(mass_pool);
  if (p->W > 0) REQ(mass_win);
  if ((rc = check_ws(p, PBSA_OP_FINE_MASS, ws, ws_bytes))) return rc;
  return hip_status(pbsa::launch_fine_mass(*p, eff_scale(p), q, *kv, sel, sel_count, lse, mass_pool,
                                           mass_win, ws, (hipStream_t)stream));
}

int pbsa_attn_fwd_mass(const pbsa_problem *p, const void *q, const pbsa_kv *kv,
                       const int32_t *sel, const int32_t *sel_count, void *o, float *lse,
                       float *mass_pool, float *mass_win, void *ws, size_t ws_bytes,
                       pbsa_stream_t stream) {
  int rc = check_problem(p, PBSA_OP_FWD_MASS);
  if (rc) return rc;
  REQ(q);
  if ((rc = check_kv_common(kv, p))) return rc;
  if (p->topk > 0) REQ(sel);
  REQ(sel_count);
  REQ(o);
  REQ(lse);
  if (p->C > 0) REQ(mass_pool);
  if (p->W > 0) REQ(mass_win);
  if ((rc = check_ws(p, PBSA_OP_FWD_MASS, ws, ws_bytes))) return rc;
  return hip_status(pbsa::launch_attn_fwd_mass(*p, eff_scale(p), q, *kv, sel, sel_count, o, lse,
                                               mass_pool, mass_win, ws, ws_bytes,
                                               (hipStream_t)stream));
}

static int memory_update_impl(const pbsa_problem *p, const pbsa_kv *kv, const float *mass_pool,
                              const float *mass_win, const int32_t *leaving, int32_t n_leave,
                              int64_t n_sink, void *ws, size_t ws_bytes, pbsa_stream_t stream,
                              bool shared) {
  int rc = check_problem(p, PBSA_OP_UPDATE);
  if (rc) return rc;
  if ((rc = check_kv_common(kv, p))) return rc;
  if (n_leave < 0 || n_leave > p->W)
    return fail(PBSA_ERR_SHAPE, "n_leave=%d outside [0, W=%d]", n_leave, p->W);
  if (n_sink < 0) return fail(PBSA_ERR_SHAPE, "n_sink must be >= 0");
  if (p->C > 0) {
    REQ(mass_pool);
    REQ(kv->kbar_pool);
  }
  if (n_leave > 0) {
    REQ(mass_win);
    REQ(leaving);
    REQ(kv->kbar_win);
  }
  if ((rc = check_ws(p, PBSA_OP_UPDATE, ws, ws_bytes))) return rc;
  return hip_status(pbsa::launch_memory_update(*p, *kv, mass_pool, mass_win, leaving, n_leave,
                                               n_sink, shared, ws, (hipStream_t)stream));
}

int pbsa_memory_update(const pbsa_problem *p, const pbsa_kv *kv, const float *mass_pool,
                       const float *mass_win, const int32_t *leaving, int32_t n_leave,
                       int64_t n_sink, void *ws, size_t ws_bytes, pbsa_stream_t stream) {
  return memory_update_impl(p, kv, mass_pool, mass_win, leaving, n_leave, n_sink, ws, ws_bytes,
                            stream, false);
}

int pbsa_memory_update_shared(const pbsa_problem *p, const pbsa_kv *kv, const float *mass_pool,
                              const float *mass_win, const int32_t *leaving, int32_t n_leave,
                              int64_t n_sink, void *ws, size_t ws_bytes, pbsa_stream_t stream) {
  return memory_update_impl(p, kv, mass_pool, mass_win, leaving, n_leave, n_sink, ws, ws_bytes,
                            stream, true);
}

static int check_slots(const pbsa_problem *p, const int64_t *ids, int64_t ids_bh_stride,
                       int32_t n_slots, int32_t n_chunks) {
  if (n_slots < 0 || n_slots > 65535) return fail(PBSA_ERR_SHAPE, "n_slots=%d outside [0, 65535]", n_slots);
  if (ids_bh_stride != 0 && ids_bh_stride < n_slots)
    return fail(PBSA_ERR_SHAPE, "ids_bh_stride=%lld must be 0 or >= n_slots=%d",
                (long long)ids_bh_stride, n_slots);
  if (n_chunks < 1 || (long long)n_chunks * p->B * p->H * p->Nq > (1LL << 40))
    return fail(PBSA_ERR_SHAPE, "n_chunks=%d out of range", n_chunks);
  if (n_slots > 0) REQ(ids);
  return PBSA_OK;
}

int pbsa_block_gather(const pbsa_problem *p, const int64_t *ids, int64_t ids_bh_stride,
                      const int32_t *count, int32_t n_slots, const void *k_hist, const void *v_hist,
                      int32_t n_chunks, void *k_out, void *v_out, int32_t *len_out,
                      pbsa_stream_t stream) {
  int rc = check_problem(p, PBSA_OP_BWD);
  if (rc) return rc;
  if ((rc = check_slots(p, ids, ids_bh_stride, n_slots, n_chunks))) return rc;
  REQ(k_hist);
  REQ(v_hist);
  REQ(k_out);
  REQ(v_out);
  if (count && !aligned16(count)) return fail(PBSA_ERR_ALIGN, "count is not 16-byte aligned");
  if (len_out && !aligned16(len_out)) return fail(PBSA_ERR_ALIGN, "len_out is not 16-byte aligned");
  return hip_status(pbsa::launch_block_gather(*p, ids, ids_bh_stride, count, n_slots, k_hist, v_hist,
                                              n_chunks, k_out, v_out, len_out, (hipStream_t)stream));
}

int pbsa_grad_scatter(const pbsa_problem *p, const int64_t *ids, int64_t ids_bh_stride,
                      const int32_t *count, int32_t n_slots, int32_t src_is_chunk, const void *dk,
                      const void *dv, float *gk, float *gv, int32_t n_chunks, pbsa_stream_t stream) {
  int rc = check_problem(p, PBSA_OP_BWD);
  if (rc) return rc;
  if ((rc = check_slots(p, ids, ids_bh_stride, n_slots, n_chunks))) return rc;
  if (src_is_chunk != 0 && src_is_chunk != 1)
    return fail(PBSA_ERR_SHAPE, "src_is_chunk must be 0 or 1");
  REQ(dk);
  REQ(dv);
  REQ(gk);
  REQ(gv);
  if (count && !aligned16(count)) return fail(PBSA_ERR_ALIGN, "count is not 16-byte aligned");
  return hip_status(pbsa::launch_grad_scatter(*p, ids, ids_bh_stride, count, n_slots, src_is_chunk,
                                              dk, dv, gk, gv, n_chunks, (hipStream_t)stream));
}

int pbsa_block_mean(const pbsa_problem *p, const void *x, const int32_t *len, int64_t n_blocks,
                    float *out, pbsa_stream_t stream) {
  int rc = check_problem(p, PBSA_OP_SELECT);
  if (rc) return rc;
  if (n_blocks < 0 || n_blocks > (1LL << 31) - 1)
    return fail(PBSA_ERR_SHAPE, "n_blocks=%lld out of range", (long long)n_blocks);
  if (n_blocks == 0) return ok();
  REQ(x);
  REQ(out);
  if (len && !aligned16(len)) return fail(PBSA_ERR_ALIGN, "len is not 16-byte aligned");
  return hip_status(pbsa::launch_block_mean(*p, x, len, n_blocks, out, (hipStream_t)stream));
}

int pbsa_window_append(const pbsa_problem *p, const pbsa_kv *kv, void *k_win, void *v_win,
                       float *kbar_win, int32_t *win_len, int64_t *win_id, int32_t first_slot,
                       int64_t first_id, pbsa_stream_t stream) {
  int rc = check_problem(p, PBSA_OP_SELECT);
  if (rc) return rc;
  if (!kv) return fail(PBSA_ERR_NULL, "kv must not be NULL");
  REQ(kv->k_cur);
  REQ(kv->v_cur);
  REQ(kv->kbar_cur);
  REQ(k_win);
  REQ(v_win);
  REQ(kbar_win);
  REQ(win_len);
  REQ(win_id);
  const int QB = (p->Nq + p->T - 1) / p->T;
  if (first_slot < 0 || first_slot + QB > p->W)
    return fail(PBSA_ERR_SHAPE, "slots [%d, %d) outside the window of %d", first_slot,
                first_slot + QB, p->W);
  if (first_id < 0) return fail(PBSA_ERR_SHAPE, "first_id must be >= 0");
  return hip_status(pbsa::launch_window_append(*p, *kv, k_win, v_win, kbar_win, win_len, win_id,
                                               first_slot, first_id, (hipStream_t)stream));
}

}  // extern "C"

/*
 * pbsa.h - Persistent Block-Sparse Attention (PBSA) for AMD Instinct MI355X
 * (gfx950), C ABI.
 *
 * The method is described on the pages "Sparse Forcing: Native Trainable
 * Sparse Attention for Real-time Autoregressive Diffusion Video Generation"
 * (gist.science/es explainer, sec. 2 "Metodologia": "Arquitectura Propuesta"
 * and "Persistente Block-Sparse Attention (PBSA)"; English abstract on the
 * shd-paper.top summary page).  Per autoregressive chunk, each query block
 * attends (1) every block of a small persistent pool P_t, (2) the top-k
 * blocks of the local sliding window L_t, chosen by coarse routing on
 * mean-pooled block representatives, and (3) the current chunk itself.
 * After the chunk, the blocks leaving the window compete with the pool by
 * pooled attention mass (Top-C retention); sink blocks are pinned.
 *
 * Conventions
 *  - Every pointer is a DEVICE pointer unless stated otherwise.  Tensors are
 *    dense, row-major, contiguous, head-major (index order as written).
 *  - "bf16" data is raw bfloat16 bits (uint16); dtype PBSA_F32 uses float.
 *    Q, K, V, O, dO, dQ, dK, dV share the problem's dtype; pooled means,
 *    masses and LSE are always fp32; indices int32; block ids int64 (>= 0).
 *  - The caller owns and allocates every buffer, including the workspace.
 *    The library allocates nothing, keeps no state between calls and never
 *    synchronises the host: each call only enqueues kernels on `stream`
 *    (a hipStream_t; NULL = the null stream).  Calls are thread-safe.
 *  - Pointers must be 16-byte aligned.
 *  - Return value: PBSA_OK (0) or a negative PBSA_ERR_* code.  Arguments are
 *    validated on the host before anything is enqueued; on error nothing is
 *    launched and outputs are untouched.  pbsa_last_error() gives a
 *    thread-local detail string.  No C++ exception crosses the ABI.
 *  - Device-resident metadata (pool_count, win_len, sel) cannot be checked
 *    on the host without a sync; kernels clamp bad values instead of
 *    faulting and OR a PBSA_STATUS_* bit into *problem.dev_status (if not
 *    NULL).
 *
 * Shapes (QB = ceil(Nq / T) query blocks; the last block may be short):
 *   q, k_cur, v_cur, o, dout, dq, dk_cur, dv_cur  [B, H, Nq, d]
 *   k_win, v_win, dk_win, dv_win                  [B, H, W, T, d]   ring slots
 *   win_len [W] int32 (0 = empty slot), win_id [W] int64
 *   k_pool, v_pool, dk_pool, dv_pool              [B, H, C, T, d]
 *   pool_len [B, H, C] int32, pool_id [B, H, C] int64,
 *   pool_count [B, H] int32 (valid pool slots are exactly [0, count))
 *   kbar_win [B, H, W, d], kbar_pool [B, H, C, d], kbar_cur [B, H, QB, d]
 *   sel [B, H, QB, topk] int32, sel_count [B, H, QB] int32
 *   mass_pool [B, H, C], mass_win [B, H, W], lse [B, H, Nq]  (fp32)
 *
 * Supported: dtype PBSA_BF16 with d in {64, 128} and T in {64, 128}
 * (bf16 MFMA, fp32 accumulate and softmax); dtype PBSA_F32 with d in
 * {64, 128}, T in {64, 128} (fp32 MFMA, fp32 softmax) for every call except
 * pbsa_attn_bwd, which is bf16 only (PBSA_ERR_UNSUPPORTED otherwise).
 * W <= 1024, C <= 1024, 0 <= topk <= W.
 */
#ifndef PBSA_H
#define PBSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *pbsa_stream_t; /* hipStream_t */

enum { PBSA_BF16 = 0, PBSA_F32 = 1 };

enum {
  PBSA_OK = 0,
  PBSA_ERR_NULL = -1,        /* a required pointer is NULL */
  PBSA_ERR_SHAPE = -2,       /* a size is out of range */
  PBSA_ERR_DTYPE = -3,       /* unknown dtype */
  PBSA_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  PBSA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required */
  PBSA_ERR_HIP = -6,         /* the HIP runtime reported an error */
  PBSA_ERR_UNSUPPORTED = -7  /* valid but not implemented (e.g. d = 96) */
};

enum { PBSA_OP_SELECT = 0, PBSA_OP_FWD = 1, PBSA_OP_BWD = 2, PBSA_OP_UPDATE = 3,
       PBSA_OP_FINE_MASS = 4, PBSA_OP_FWD_MASS = 5 };

/* Bits OR-ed into *dev_status by kernels (device-side metadata faults). */
enum {
  PBSA_STATUS_POOL_COUNT = 1,  /* pool_count outside [0, C]: clamped */
  PBSA_STATUS_WIN_LEN = 2,     /* a win_len / pool_len outside [0, T]: clamped */
  PBSA_STATUS_SEL = 4,         /* sel entry outside [0, W) or sel_count > topk: skipped/clamped */
  PBSA_STATUS_SINK = 8,        /* more pinned sink blocks than C: kept the C smallest ids */
  PBSA_STATUS_SHARED = 16      /* head-shared update: the heads of a batch element hold different pools */
};

typedef struct {
  int32_t B, H;      /* batch, heads; every (b, h) is independent */
  int32_t d;         /* head dim */
  int32_t T;         /* tokens per block (also the query-block height) */
  int32_t Nq;        /* tokens of the current chunk (>= 1) */
  int32_t W;         /* window ring slots */
  int32_t C;         /* pool capacity in blocks */
  int32_t topk;      /* window blocks selected per query block */
  int32_t dtype;     /* PBSA_BF16 or PBSA_F32 */
  float scale;       /* logit scale; 0 means 1/sqrt(d) */
  int32_t *dev_status; /* optional device int32 for PBSA_STATUS_* bits; may be NULL */
} pbsa_problem;

/* One layer's KV state; every buffer is caller-owned. */
typedef struct {
  const void *k_cur, *v_cur;  /* [B,H,Nq,d] current chunk */
  const void *k_win, *v_win;  /* [B,H,W,T,d] window ring */
  const int32_t *win_len;     /* [W] valid tokens per slot, 0 = empty (shared by all b,h) */
  const int64_t *win_id;      /* [W] global block id of each slot */
  const float *kbar_win;      /* [B,H,W,d] mean of each window slot's valid keys */
  void *k_pool, *v_pool;      /* [B,H,C,T,d] persistent pool */
  int32_t *pool_len;          /* [B,H,C] */
  int64_t *pool_id;           /* [B,H,C] */
  int32_t *pool_count;        /* [B,H] */
  float *kbar_pool;           /* [B,H,C,d] */
  float *kbar_cur;            /* [B,H,QB,d] written by pbsa_select */
} pbsa_kv;

/* Gradient buffers, same shapes as the matching pbsa_kv fields. */
typedef struct {
  void *dk_cur, *dv_cur, *dk_win, *dv_win, *dk_pool, *dv_pool;
} pbsa_kv_grad;

/*
 * pbsa_select - block compression by pooling and coarse routing
 * (gist.science/es, sec. 2 "Persistente Block-Sparse Attention (PBSA)":
 * pooled block representatives for coarse routing; "Arquitectura
 * Propuesta": Top-K window blocks per query, coarse scoring of relevance).
 *   qbar_i   = mean of the rows of query block i            (fp32)
 *   kbar_cur = mean of the key rows of each current block   (fp32, written to kv->kbar_cur)
 *   s_ij     = scale * <qbar_i, kbar_j> for j in the valid pool slots, the
 *              valid window slots and the current blocks
 *   sel[i]   = the min(topk, #valid window slots) window slots with the
 *              largest s_ij (ties: smaller win_id; NaN last), ascending
 *              slot order, padded with -1; sel_count[i] = their number
 *   mass_pool / mass_win[j] = sum over query blocks i of softmax_j(s_i.)
 *              (the softmax runs over pool + window + current); 0 for
 *              invalid slots.  These are the scores of the Top-C update.
 * mass_pool and mass_win are optional as a pair: with both NULL the masses
 * are not computed here (the attention needs only sel); pbsa_block_mass
 * computes them later from the scores this call leaves in ws.  Otherwise
 * mass_pool is required when C > 0 and mass_win when W > 0.
 * Workspace: pbsa_workspace_size(p, PBSA_OP_SELECT) bytes.
 */
int pbsa_select(const pbsa_problem *p, const void *q, const pbsa_kv *kv, int32_t *sel,
                int32_t *sel_count, float *mass_pool, float *mass_win, void *ws,
                size_t ws_bytes, pbsa_stream_t stream);

/*
 * pbsa_select_static - pbsa_select for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and results, with the workspace taken
 * from a static device array of 8 MiB that the library holds on each GPU it
 * runs on until the process ends.  The caller passes inputs and outputs as
 * for pbsa_select; nothing is allocated and nothing needs clearing.
 * Problems whose select workspace (pbsa_workspace_size(p, PBSA_OP_SELECT))
 * exceeds 8 MiB are refused with PBSA_ERR_WORKSPACE before any launch.
 * Every call on one GPU uses that GPU's one array: calls that overlap in
 * time on one GPU (several streams or threads) race, and pbsa_block_mass
 * cannot read the scores this call leaves (it takes a workspace).
 */
int pbsa_select_static(const pbsa_problem *p, const void *q, const pbsa_kv *kv, int32_t *sel,
                       int32_t *sel_count, float *mass_pool, float *mass_win,
                       pbsa_stream_t stream);

/*
 * pbsa_block_mass - the block masses of pbsa_select (same definition and
 * section) from the coarse scores the last pbsa_select call left in ws
 * (same problem, ws untouched since), so that a rollout can take them off
 * the attention's critical path and compute them on the stream that runs the
 * Top-C update.  mass_pool [B,H,C] required when C > 0, mass_win [B,H,W]
 * when W > 0 (fp32, written in full).
 * Workspace: the pbsa_select workspace, read only.
 */
int pbsa_block_mass(const pbsa_problem *p, float *mass_pool, float *mass_win, const void *ws,
                    size_t ws_bytes, pbsa_stream_t stream);

/*
 * pbsa_attn_fwd - hybrid attention (same section: dense attention over the
 * persistent memory, sparse attention over the window).  For row r of query
 * block i, over the tokens U_i = valid tokens of pool slots [0, count),
 * of the window slots sel[i][0:sel_count[i]], and of the whole current chunk:
 *   O_r = softmax_u(scale * <Q_r, K_u>) V_u,   lse_r = log sum_u exp(scale <Q_r,K_u>)
 * (natural log).  o: [B,H,Nq,d] in the problem dtype; lse may be NULL.
 * Workspace: optional.  With ws == NULL (or ws_bytes below
 * pbsa_workspace_size(p, PBSA_OP_FWD)) each query block runs in one
 * workgroup.  With a large enough 16-byte-aligned ws and at most half the
 * GPU's resident workgroups' worth of query blocks, every query block's list
 * is cut into 2 to 8 equal ranges (bf16: up to 16 while every piece can have
 * a CU to itself; fp32: up to 16, at most one list
 * entry each), one workgroup each;
 * each piece leaves a partial in ws (fp32 O, running max and row sum of
 * its 2T threads; at most 512 pieces) and a second kernel, enqueued by the
 * same call, merges them in a fixed order, so results stay bitwise
 * reproducible.  ws needs no initialisation; calls that share one ws must
 * not overlap in time (one stream is fine).
 */
int pbsa_attn_fwd(const pbsa_problem *p, const void *q, const pbsa_kv *kv, const int32_t *sel,
                  const int32_t *sel_count, void *o, float *lse, void *ws, size_t ws_bytes,
                  pbsa_stream_t stream);

/*
 * pbsa_select_attn_fwd - pbsa_select without masses followed by
 * pbsa_attn_fwd (the same sections: coarse routing of each query block,
 * then the hybrid attention over what it selected), with the same results
 * bit for bit: sel, sel_count, kv->kbar_cur, o and lse (lse may be NULL).
 * Where the problem allows (bf16, d = T = 128, C + topk <= 128, W <= 819,
 * and no split of the forward) it is one launch in which each workgroup
 * routes its own query block and then attends, so no launch boundary
 * separates the two; otherwise the two launches of the separate calls.
 * ws: the pbsa_select workspace (required), left as pbsa_select leaves it,
 * so pbsa_block_mass can be given it afterwards.  fwd_ws: optional, as the
 * workspace of pbsa_attn_fwd (it decides whether the forward splits).
 * Calls that share a workspace must not overlap in time.
 */
int pbsa_select_attn_fwd(const pbsa_problem *p, const void *q, const pbsa_kv *kv, int32_t *sel,
                         int32_t *sel_count, void *o, float *lse, void *ws, size_t ws_bytes,
                         void *fwd_ws, size_t fwd_ws_bytes, pbsa_stream_t stream);

/*
 * pbsa_attn_bwd - gradients through the fixed block mask (the trainable
 * sparse attention of the paper's title; selection is not differentiated).
 * With P the forward weights (recomputed from lse), D_r = <dO_r, O_r>,
 * dS = P (dO V^T - D):  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
 * each landing on the storage slot of its token.  Every element of every
 * gradient buffer is written (zero where no query attends).  dq and every
 * pbsa_kv_grad field are required.  bf16 only.
 * Workspace: pbsa_workspace_size(p, PBSA_OP_BWD) bytes.
 */
int pbsa_attn_bwd(const pbsa_problem *p, const void *q, const pbsa_kv *kv, const int32_t *sel,
                  const int32_t *sel_count, const void *o, const float *lse, const void *dout,
                  void *dq, const pbsa_kv_grad *g, void *ws, size_t ws_bytes,
                  pbsa_stream_t stream);

/*
 * pbsa_fine_mass - exact block mass, an alternative score for the Top-C
 * update ("Arquitectura Propuesta": dynamic pool blocks are kept by their
 * relevance to the current step; this scores that relevance with the
 * attention itself instead of pooled representatives).  For every stored
 * block j of (b, h):
 *   M_j = sum over the chunk's query rows r of sum_{u in j} P_ru,
 *   P_ru = exp(scale <Q_r, K_u> - lse_r),
 * with lse the natural-log output of pbsa_attn_fwd for the same problem,
 * q, kv, sel and sel_count, so that P is the forward's attention.  mass_pool
 * [B,H,C] covers pool slots [0, count) (0 elsewhere); mass_win [B,H,W] sums
 * over the query blocks that selected the slot (0 if none did).  Both are
 * required (when C > 0 / W > 0), fp32, written in full, and can be passed
 * to pbsa_memory_update in place of the coarse masses.
 * Workspace: pbsa_workspace_size(p, PBSA_OP_FINE_MASS) bytes (partial sums;
 * no initialisation needed).
 */
int pbsa_fine_mass(const pbsa_problem *p, const void *q, const pbsa_kv *kv, const int32_t *sel,
                   const int32_t *sel_count, const float *lse, float *mass_pool, float *mass_win,
                   void *ws, size_t ws_bytes, pbsa_stream_t stream);

/*
 * pbsa_attn_fwd_mass - pbsa_attn_fwd and the exact block masses of
 * pbsa_fine_mass (same definitions and sections) in one call: the forward's
 * own walk records, for every query row and every pool or selected window
 * block it attends, the block's log-sum-exp of the row's logits, and a small
 * kernel then forms M_j = sum_r exp(blse_rj - lse_r) with the final lse, so
 * the masses cost no second pass over K.  o and lse as pbsa_attn_fwd (lse
 * required here); mass_pool / mass_win as pbsa_fine_mass (required when
 * C > 0 / W > 0, fp32, written in full, deterministic).
 * Workspace: pbsa_workspace_size(p, PBSA_OP_FWD_MASS) bytes, required (the
 * per-row block log-sum-exps, then the forward's split workspace); no
 * initialisation needed; calls that share one ws must not overlap in time.
 */
int pbsa_attn_fwd_mass(const pbsa_problem *p, const void *q, const pbsa_kv *kv,
                       const int32_t *sel, const int32_t *sel_count, void *o, float *lse,
                       float *mass_pool, float *mass_win, void *ws, size_t ws_bytes,
                       pbsa_stream_t stream);

/*
 * pbsa_memory_update - Top-C retention of the persistent pool ("Arquitectura
 * Propuesta": sink blocks as fixed anchors, dynamic blocks by coarse score,
 * Top-C keeps the C best and discards the rest of the blocks leaving the
 * window).  Per (b, h): candidates X = valid pool blocks + the window slots
 * listed in `leaving` (device int32 [n_leave], slots with win_len 0 and ids
 * already in the pool are skipped).  If |X| <= C all are kept; otherwise the
 * blocks with id < n_sink are pinned and the rest ranked by mass (desc, then
 * id asc, NaN last).  Survivors keep their slots; admitted blocks fill the
 * freed slots, then the unused tail, in ascending slot order and ascending
 * id order, copying K, V (all T rows), kbar, len and id bit-exactly.
 * pool_count becomes |kept|.  Reads kv->k_win/v_win/kbar_win/win_*.
 * Workspace: pbsa_workspace_size(p, PBSA_OP_UPDATE) bytes.  n_leave <= W.
 */
int pbsa_memory_update(const pbsa_problem *p, const pbsa_kv *kv, const float *mass_pool,
                       const float *mass_win, const int32_t *leaving, int32_t n_leave,
                       int64_t n_sink, void *ws, size_t ws_bytes, pbsa_stream_t stream);

/*
 * pbsa_memory_update_shared - the same update with a head-shared pool (a
 * policy variant the pages leave open; same section): every head of a batch
 * element ranks the candidates by the block's mass summed over the heads
 * (slot-wise for pool blocks, window slots are shared), in ascending head
 * order, so all heads make the same decision and keep the same blocks in the
 * same slots.  Precondition: the heads of each batch element hold the same
 * pool (count and ids), as after every update so far being shared; a
 * violation sets PBSA_STATUS_SHARED in dev_status (checked when dev_status is
 * given) and the heads then decide on sums of different blocks' masses.
 * Arguments, workspace and copies as pbsa_memory_update.
 */
int pbsa_memory_update_shared(const pbsa_problem *p, const pbsa_kv *kv, const float *mass_pool,
                              const float *mass_win, const int32_t *leaving, int32_t n_leave,
                              int64_t n_sink, void *ws, size_t ws_bytes, pbsa_stream_t stream);

/*
 * Training through a streaming rollout (the sparse attention is trainable;
 * same pages).  A pool or window slot holds a copy of block j of an earlier
 * chunk c, block id c*QB + j: rows [j T, min(Nq, (j+1) T)) of that chunk's
 * K and V.  With the routing and pool decisions of every chunk held fixed,
 * the gradient a slot receives in pbsa_attn_bwd belongs to those rows.
 * History and gradient accumulators hold all chunks of the rollout:
 * k_hist / v_hist [n_chunks,B,H,Nq,d] in the problem dtype, gk / gv
 * [n_chunks,B,H,Nq,d] fp32.  Slot ids: ids[(b*H + h) * ids_bh_stride + s]
 * for slot s (ids_bh_stride 0: one list for every (b, h), as for the window;
 * otherwise >= n_slots); id < 0 = empty slot; count (optional, [B,H]) makes
 * the slots >= count[b,h] empty.  An id whose chunk is >= n_chunks is
 * treated as empty and sets PBSA_STATUS_SEL.
 *
 * pbsa_block_gather - rebuild slots from the history: k_out / v_out
 * [B,H,n_slots,T,d] get the block's rows, zeros after its length (empty
 * slots: all zeros); len_out (optional, [B,H,n_slots] int32) its length.
 *
 * pbsa_grad_scatter - gk[c][b,h,rows] += dk of the slot (and gv, dv): with
 * src_is_chunk = 0, dk / dv are slot-shaped [B,H,n_slots,T,d] (the pool or
 * window gradients of pbsa_attn_bwd); with src_is_chunk = 1 they are
 * chunk-shaped [B,H,Nq,d] and block j's rows are read at j T (the chunk's own
 * dk_cur / dv_cur, ids c*QB + j).  The non-negative ids of one (b, h) must be
 * distinct within a call (each destination row is added by one workgroup);
 * successive calls accumulate in call order.
 */
int pbsa_block_gather(const pbsa_problem *p, const int64_t *ids, int64_t ids_bh_stride,
                      const int32_t *count, int32_t n_slots, const void *k_hist, const void *v_hist,
                      int32_t n_chunks, void *k_out, void *v_out, int32_t *len_out,
                      pbsa_stream_t stream);
int pbsa_grad_scatter(const pbsa_problem *p, const int64_t *ids, int64_t ids_bh_stride,
                      const int32_t *count, int32_t n_slots, int32_t src_is_chunk, const void *dk,
                      const void *dv, float *gk, float *gv, int32_t n_chunks, pbsa_stream_t stream);

/*
 * pbsa_block_mean - pooled representative (mean of the valid rows) of
 * n_blocks stored blocks: x [n_blocks, T, d] in the problem dtype, len
 * [n_blocks] int32 (or NULL = all T), out [n_blocks, d] fp32.  Blocks with
 * len 0 get 0.  Used to fill kbar caches for a state built outside a
 * rollout (same pooling as pbsa_select).
 */
int pbsa_block_mean(const pbsa_problem *p, const void *x, const int32_t *len, int64_t n_blocks,
                    float *out, pbsa_stream_t stream);

/*
 * pbsa_window_append - the ring advance of a rollout: write the current
 * chunk (k_cur/v_cur of kv, kbar_cur) into QB consecutive window slots
 * [first_slot, first_slot + QB) and set their win_len (block length) and
 * win_id (first_id + j).  win_len/win_id are passed writable here.
 */
int pbsa_window_append(const pbsa_problem *p, const pbsa_kv *kv, void *k_win, void *v_win,
                       float *kbar_win, int32_t *win_len, int64_t *win_id, int32_t first_slot,
                       int64_t first_id, pbsa_stream_t stream);

/* Bytes of workspace an op needs (0 if none). */
size_t pbsa_workspace_size(const pbsa_problem *p, int op);

/* Host-only validation of the problem for an op (same checks the entry
 * points run first).  Returns PBSA_OK or a PBSA_ERR_* code. */
int pbsa_validate(const pbsa_problem *p, int op);

const char *pbsa_strerror(int status);
const char *pbsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PBSA_H */

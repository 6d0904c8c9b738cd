"""fp64 CPU oracle of Persistent Block-Sparse Attention (PBSA).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg use this module.  It shares no code with the HIP library and
imports nothing from it; the product path never calls it.

Sources (the pages are secondary descriptions of the method; there are no
equations or listings for PBSA on them):
  [SF-es]  "Sparse Forcing: Native Trainable Sparse Attention for Real-time
           Autoregressive Diffusion Video Generation", gist.science/es
           explainer: sec. 2 "Metodologia" -> "Arquitectura Propuesta"
           (persistent memory P_t = sink blocks + dynamic blocks D_t chosen by
           coarse scoring, Top-C retention, local window L_t with Top-K block
           selection) and "Persistente Block-Sparse Attention (PBSA)" (block
           compression by pooling, coarse routing, hybrid attention: dense over
           the persistent memory, sparse over the window).
  [SF-abs] the same paper's English abstract ("摘要（原文）" on the
           shd-paper.top summary page): compress, preserve and update
           persistent blocks; restrict each window's computation to a
           dynamically selected local neighbourhood; kernel accelerates
           sparse attention and memory updates.
  [LF-it]  "Light Forcing: Accelerating Autoregressive Video Diffusion via
           Sparse Attention", gist.science/it, sec. 2.2 (HSA): block
           representatives by mean pooling (related work; supports reading R2).

Every step below is written in fp64 from the inputs' exact values (bf16/fp32
widened).  Where the pages leave a step open, the plainest reading is taken;
each reading is tagged R<n> and listed with its basis in the design notes:
  R1  selection is per query block (all rows of a block share one set)
  R2  pooled representative = arithmetic mean of the block's valid rows
  R3  coarse logit = scale * <qbar, kbar>, same scale as the token logits
  R4  every (batch, head) is independent, with its own pool
  R5  the window holds the blocks before the current chunk; the current chunk
      is always attended in full, without a causal mask inside it
  R6  pool attention is dense over every valid pool slot
  R7  a chunk is cut into contiguous blocks of T tokens; the last may be short
  R8  short blocks: only valid tokens are attended, averaged, scored
  R9  fewer valid window slots than k: all are selected
  R10 top-k order: score descending, then block id ascending; NaN ranks last
  R11 block mass = coarse softmax over everything the chunk can see, summed
      over the chunk's query blocks
  R12 update candidates = valid pool blocks + blocks leaving the window
      (a leaving block whose id is already pooled, or listed earlier among
      the leaving blocks, is not a second candidate)
  R13 Top-C order: mass descending, then id ascending; NaN last; blocks with
      id < n_sink are pinned (sinks)
  R14 a block enters the pool as a bit-exact copy of its K/V/mean/len/id
  R15 placement: survivors keep their slots; freed slots, then the unused
      tail, are filled in ascending order by the admitted blocks in
      ascending id order; valid pool slots are always [0, count)
  R21 training through a rollout: the routing and pool decisions of every
      chunk are held fixed; a stored block's gradient belongs to the rows of
      the chunk that produced it
  R20 head-shared pool (a policy variant): every head of a batch element
      ranks the candidates by the block's masses summed over the heads
  R19 fine-grained block mass (an alternative to R11's coarse mass): the
      exact attention probability the chunk's query rows put on the block's
      tokens, summed over the rows; a block a row does not attend gets
      nothing from it
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

F64 = np.float64


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=F64)


def n_blocks(nq: int, t: int) -> int:
    return (nq + t - 1) // t


def query_block_rows(nq: int, t: int, i: int) -> range:
    """Rows of query block i (R7)."""
    return range(i * t, min(nq, (i + 1) * t))


# ----------------------------------------------------------------------------
# Block compression by pooling  [SF-es, "PBSA": pooled representatives]  (R2)
# ----------------------------------------------------------------------------
def block_mean(rows: np.ndarray) -> np.ndarray:
    """Mean of the valid rows of one block, [n, d] -> [d]."""
    rows = _f64(rows)
    n = rows.shape[0]
    if n == 0:
        raise ValueError("empty block has no representative")
    return rows.sum(axis=0) / n


def pooled_queries(q: np.ndarray, t: int) -> np.ndarray:
    """qbar[b,h,i] = mean of the rows of query block i.  q: [B,H,Nq,d]."""
    q = _f64(q)
    B, H, nq, d = q.shape
    qb = n_blocks(nq, t)
    out = np.empty((B, H, qb, d))
    for b in range(B):
        for h in range(H):
            for i in range(qb):
                r = query_block_rows(nq, t, i)
                out[b, h, i] = block_mean(q[b, h, r.start:r.stop])
    return out


def pooled_slots(k_slots: np.ndarray, lens: np.ndarray) -> np.ndarray:
    """Means of slot blocks [..., S, T, d] with valid lengths broadcastable to
    [..., S]; empty slots get NaN (they are never used)."""
    k_slots = _f64(k_slots)
    lens = np.broadcast_to(np.asarray(lens), k_slots.shape[:-2])
    out = np.full(k_slots.shape[:-2] + (k_slots.shape[-1],), np.nan)
    for idx in np.ndindex(*k_slots.shape[:-2]):
        n = int(lens[idx])
        if n > 0:
            out[idx] = block_mean(k_slots[idx][:n])
    return out


# ----------------------------------------------------------------------------
# Coarse routing: scores, window top-k, block mass
#   [SF-es "Arquitectura Propuesta": Top-K block selection in the window,
#    dynamic blocks by coarse scoring of relevance to the current step]
# ----------------------------------------------------------------------------
def coarse_logit(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> float:
    """R3: s = scale * <qbar, kbar>."""
    return float(scale * np.dot(_f64(qbar), _f64(kbar)))


def rank_key_desc(score: float, block_id: int):
    """Total order used by top-k (R10) and Top-C (R13): larger score first,
    ties to the smaller id, NaN after every number."""
    if math.isnan(score):
        return (1, 0.0, block_id)
    return (0, -score, block_id)


def topk_window(scores: dict, ids: dict, k: int) -> list:
    """Top-k of the candidate window slots.

    scores/ids: slot -> coarse logit / global block id, valid slots only.
    Returns the chosen slots in ascending slot order (R9, R10)."""
    order = sorted(scores.keys(), key=lambda w: rank_key_desc(scores[w], int(ids[w])))
    return sorted(order[:max(0, k)])


def softmax(x: np.ndarray) -> np.ndarray:
    x = _f64(x)
    m = np.max(x)
    e = np.exp(x - m)
    return e / e.sum()


def select(st: dict, topk: int, scale: float, t: int) -> dict:
    """Block pooling, coarse scores, per-query-block window top-k and block
    mass for one layer.

    ``st`` holds the layer's inputs (numpy or torch CPU arrays): q, k_cur
    [B,H,Nq,d]; k_win [B,H,W,T,d], win_len [W], win_id [W]; k_pool
    [B,H,C,T,d], pool_len [B,H,C], pool_id [B,H,C], pool_count [B,H].

    Returns sel [B,H,QB,topk] (ascending slots, -1 padding), sel_count
    [B,H,QB], mass_pool [B,H,C], mass_win [B,H,W] (0 where not a candidate),
    the pooled representatives, and the window logits s_win [B,H,QB,W]
    (NaN where the slot is empty) for tie analysis.
    """
    st = as_f64_state(st)
    q = st["q"]; k_cur = st["k_cur"]
    k_win = st["k_win"]; k_pool = st["k_pool"]
    win_len = np.asarray(st["win_len"]).astype(np.int64)
    win_id = np.asarray(st["win_id"]).astype(np.int64)
    pool_len = np.asarray(st["pool_len"]).astype(np.int64)
    pool_count = np.asarray(st["pool_count"]).astype(np.int64)
    B, H, nq, d = q.shape
    W = k_win.shape[2]
    C = k_pool.shape[2]
    qb = n_blocks(nq, t)

    qbar = pooled_queries(q, t)
    kbar_cur = pooled_queries(k_cur, t)           # current-chunk blocks share the partition (R7)
    kbar_win = pooled_slots(k_win, win_len[None, None, :])
    kbar_pool = np.full((B, H, C, d), np.nan)
    for b in range(B):
        for h in range(H):
            for p in range(int(pool_count[b, h])):
                kbar_pool[b, h, p] = block_mean(k_pool[b, h, p, :pool_len[b, h, p]])

    sel = np.full((B, H, qb, topk), -1, dtype=np.int64)
    sel_count = np.zeros((B, H, qb), dtype=np.int64)
    mass_pool = np.zeros((B, H, C))
    mass_win = np.zeros((B, H, W))
    s_win = np.full((B, H, qb, W), np.nan)
    valid_w = [w for w in range(W) if win_len[w] > 0]
    for b in range(B):
        for h in range(H):
            n_pool = int(pool_count[b, h])
            for i in range(qb):
                sp = [coarse_logit(qbar[b, h, i], kbar_pool[b, h, p], scale) for p in range(n_pool)]
                sw = {w: coarse_logit(qbar[b, h, i], kbar_win[b, h, w], scale) for w in valid_w}
                sc = [coarse_logit(qbar[b, h, i], kbar_cur[b, h, j], scale) for j in range(qb)]
                for w, v in sw.items():
                    s_win[b, h, i, w] = v
                chosen = topk_window(sw, {w: win_id[w] for w in valid_w}, topk)
                sel[b, h, i, :len(chosen)] = chosen
                sel_count[b, h, i] = len(chosen)
                # R11: softmax over J = pool-valid, window-valid, current blocks
                pi = softmax(np.array(sp + [sw[w] for w in valid_w] + sc))
                mass_pool[b, h, :n_pool] += pi[:n_pool]
                for n, w in enumerate(valid_w):
                    mass_win[b, h, w] += pi[n_pool + n]
    return dict(sel=sel, sel_count=sel_count, mass_pool=mass_pool, mass_win=mass_win,
                qbar=qbar, kbar_cur=kbar_cur, kbar_win=kbar_win, kbar_pool=kbar_pool,
                s_win=s_win)


# ----------------------------------------------------------------------------
# Hybrid attention  [SF-es "PBSA": dense over the persistent memory, sparse
# (selected blocks) over the local window; plus the current chunk (R5)]
# ----------------------------------------------------------------------------
def attended_segments(st: dict, b: int, h: int, sel_i: Iterable[int]) -> list:
    """U_i as storage segments (region, slot, n_valid) with region in
    {'pool', 'win', 'cur'}: every valid pool slot (R6), the selected window
    slots, and the whole current chunk (R5).  Token u of a segment is row u
    of that slot (or of the chunk).  The order does not change the result."""
    pool_len = np.asarray(st["pool_len"]); win_len = np.asarray(st["win_len"])
    n_pool = int(np.asarray(st["pool_count"])[b, h])
    nq = st["q"].shape[2]
    seg = [("pool", p, int(pool_len[b, h, p])) for p in range(n_pool)]
    seg += [("win", int(w), int(win_len[int(w)])) for w in sel_i if int(w) >= 0]
    seg.append(("cur", 0, nq))
    return [s for s in seg if s[2] > 0]


def _gather(st: dict, b: int, h: int, seg: list, which: str) -> np.ndarray:
    """Rows of K (which='k') or V (which='v') of the segments, concatenated."""
    rows = []
    for reg, slot, n in seg:
        if reg == "cur":
            rows.append(st[which + "_cur"][b, h, :n])
        else:
            rows.append(st[which + "_" + reg][b, h, slot, :n])
    return np.concatenate(rows, axis=0)


def _block_operands(st, b, h, sel_i):
    seg = attended_segments(st, b, h, sel_i)
    return seg, _gather(st, b, h, seg, "k"), _gather(st, b, h, seg, "v")


def as_f64_state(st: dict) -> dict:
    """Widen every float array of a state to fp64 numpy (exact for bf16 and
    fp32 inputs); integer arrays become int64 numpy."""
    out = {}
    for key, v in st.items():
        if hasattr(v, "detach"):
            v = v.detach().to("cpu")
            v = v.double().numpy() if v.is_floating_point() else v.long().numpy()
        elif isinstance(v, np.ndarray):
            v = v.astype(F64, copy=False) if v.dtype.kind == "f" else v.astype(np.int64, copy=False)
        out[key] = v
    return out


def attn_fwd(st: dict, sel: np.ndarray, sel_count: np.ndarray, scale: float, t: int,
             blocks: Optional[Iterable] = None) -> dict:
    """O and LSE of every query row.

    For row r of query block i: z_u = scale*<Q_r, K_u> over u in U_i;
    P = softmax(z); O_r = sum_u P_u V_u; LSE_r = max z + ln sum exp(z - max z).
    ``blocks``: optional iterable of (b, h, i) to compute; other rows stay NaN.
    """
    st = as_f64_state(st)
    q = st["q"]
    B, H, nq, d = q.shape
    qb = n_blocks(nq, t)
    o = np.full((B, H, nq, d), np.nan)
    lse = np.full((B, H, nq), np.nan)
    todo = blocks if blocks is not None else [(b, h, i) for b in range(B) for h in range(H)
                                              for i in range(qb)]
    sel = np.asarray(sel); sel_count = np.asarray(sel_count)
    for b, h, i in todo:
        rows = query_block_rows(nq, t, i)
        _, K, V = _block_operands(st, b, h, sel[b, h, i, :int(sel_count[b, h, i])])
        z = scale * (q[b, h, rows.start:rows.stop] @ K.T)        # [rows, |U|]
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        l = e.sum(axis=1, keepdims=True)
        o[b, h, rows.start:rows.stop] = (e / l) @ V
        lse[b, h, rows.start:rows.stop] = (m + np.log(l))[:, 0]
    return dict(o=o, lse=lse)


def fine_mass(st: dict, sel: np.ndarray, sel_count: np.ndarray, scale: float, t: int) -> dict:
    """Fine-grained block mass (R19): for every stored block j,
    M_j = sum over the chunk's query rows r of sum_{u in j} P_ru, where P_r is
    row r's attention distribution over its attended set U_i (the same one
    attn_fwd normalises over).  Returns mass_pool [B,H,C], mass_win [B,H,W]
    and, for the identity sum_j M_j = number of query rows, mass_cur
    [B,H,QB] (current-chunk block c holds tokens [c t, c t + t))."""
    st = as_f64_state(st)
    q = st["q"]
    B, H, nq, d = q.shape
    qb = n_blocks(nq, t)
    C = st["k_pool"].shape[2]
    W = st["k_win"].shape[2]
    mass_pool = np.zeros((B, H, C))
    mass_win = np.zeros((B, H, W))
    mass_cur = np.zeros((B, H, qb))
    sel = np.asarray(sel); sel_count = np.asarray(sel_count)
    for b in range(B):
        for h in range(H):
            for i in range(qb):
                rows = query_block_rows(nq, t, i)
                seg, K, _ = _block_operands(st, b, h, sel[b, h, i, :int(sel_count[b, h, i])])
                z = scale * (q[b, h, rows.start:rows.stop] @ K.T)
                e = np.exp(z - z.max(axis=1, keepdims=True))
                P = e / e.sum(axis=1, keepdims=True)  # each row sums to 1
                col_mass = P.sum(axis=0)             # per attended token
                u0 = 0
                for reg, slot, n in seg:
                    m = col_mass[u0:u0 + n]
                    if reg == "pool":
                        mass_pool[b, h, slot] += m.sum()
                    elif reg == "win":
                        mass_win[b, h, slot] += m.sum()
                    else:
                        for c in range(qb):
                            mass_cur[b, h, c] += m[c * t:min(n, (c + 1) * t)].sum()
                    u0 += n
    return dict(mass_pool=mass_pool, mass_win=mass_win, mass_cur=mass_cur)


def attn_bwd(st: dict, sel: np.ndarray, sel_count: np.ndarray, dout: np.ndarray, scale: float,
             t: int, blocks: Optional[Iterable] = None) -> dict:
    """Gradients of sum(dO * O) through the fixed block mask (selection is
    not differentiated).

    D_r = <dO_r, O_r>; dS_ru = P_ru (<dO_r, V_u> - D_r); dQ_r = scale sum_u
    dS_ru K_u; dK_u = scale sum_r dS_ru Q_r; dV_u = sum_r P_ru dO_r, each
    landing on the storage slot of token u.  Unattended slots get zero.
    ``blocks``: restrict the query blocks that contribute (b, h, i)."""
    st = as_f64_state(st)
    q = st["q"]; dout = as_f64_state({"x": dout})["x"]
    B, H, nq, d = q.shape
    qb = n_blocks(nq, t)
    g = {name: np.zeros_like(st[name]) for name in
         ("k_cur", "v_cur", "k_win", "v_win", "k_pool", "v_pool")}
    dq = np.zeros_like(q)
    todo = blocks if blocks is not None else [(b, h, i) for b in range(B) for h in range(H)
                                              for i in range(qb)]
    sel = np.asarray(sel); sel_count = np.asarray(sel_count)
    for b, h, i in todo:
        rows = query_block_rows(nq, t, i)
        seg, K, V = _block_operands(st, b, h, sel[b, h, i, :int(sel_count[b, h, i])])
        Q = q[b, h, rows.start:rows.stop]
        dO = dout[b, h, rows.start:rows.stop]
        z = scale * (Q @ K.T)
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        P = e / e.sum(axis=1, keepdims=True)
        O = P @ V
        D = (dO * O).sum(axis=1, keepdims=True)
        dS = P * (dO @ V.T - D)
        dq[b, h, rows.start:rows.stop] = scale * (dS @ K)
        dK = scale * (dS.T @ Q)
        dV = P.T @ dO
        off = 0
        for reg, slot, n in seg:
            if reg == "cur":
                g["k_cur"][b, h, :n] += dK[off:off + n]
                g["v_cur"][b, h, :n] += dV[off:off + n]
            else:
                g["k_" + reg][b, h, slot, :n] += dK[off:off + n]
                g["v_" + reg][b, h, slot, :n] += dV[off:off + n]
            off += n
    return dict(dq=dq, dk_cur=g["k_cur"], dv_cur=g["v_cur"], dk_win=g["k_win"],
                dv_win=g["v_win"], dk_pool=g["k_pool"], dv_pool=g["v_pool"])


# ----------------------------------------------------------------------------
# Persistent-memory update  [SF-es "Arquitectura Propuesta": Top-C retention,
# sink blocks as fixed anchors; SF-abs: preserve and update persistent blocks]
# ----------------------------------------------------------------------------
STATUS_POOL_COUNT = 1
STATUS_WIN_LEN = 2
STATUS_SEL_RANGE = 4
STATUS_SINK_OVERFLOW = 8


def memory_update_one(pool_ids: list, pool_mass: list, cand_ids: list, cand_mass: list,
                      C: int, n_sink: int):
    """Top-C decision for one (batch, head).

    pool_ids/pool_mass: the valid pool blocks, slot p = position p.
    cand_ids/cand_mass: the blocks leaving the window (R12).
    Returns (slot_of_admitted, new_ids_by_slot, status) where
    slot_of_admitted is a list of (slot, candidate index) and new_ids_by_slot
    the pool's id list after the update, and status is 0 or
    STATUS_SINK_OVERFLOW.
    """
    n_pool = len(pool_ids)
    seen = set(int(x) for x in pool_ids)
    X = [("pool", p, int(pool_ids[p]), float(pool_mass[p])) for p in range(n_pool)]
    for c in range(len(cand_ids)):
        if int(cand_ids[c]) in seen:       # R12: already resident or already listed
            continue
        seen.add(int(cand_ids[c]))
        X.append(("cand", c, int(cand_ids[c]), float(cand_mass[c])))
    status = 0
    if len(X) <= C:
        kept = X
    else:
        pinned = [x for x in X if x[2] < n_sink]            # R13 sinks
        rest = [x for x in X if x[2] >= n_sink]
        if len(pinned) > C:
            status = STATUS_SINK_OVERFLOW
            kept = sorted(pinned, key=lambda x: x[2])[:C]
        else:
            rest = sorted(rest, key=lambda x: rank_key_desc(x[3], x[2]))
            kept = pinned + rest[:C - len(pinned)]
    kept_pool = {x[1] for x in kept if x[0] == "pool"}
    admitted = sorted([x for x in kept if x[0] == "cand"], key=lambda x: x[2])
    free = [p for p in range(n_pool) if p not in kept_pool] + list(range(n_pool, C))
    free = sorted(free)                                     # R15
    assign = [(free[n], x[1]) for n, x in enumerate(admitted)]
    new_ids = {p: int(pool_ids[p]) for p in kept_pool}
    for slot, c in assign:
        new_ids[slot] = int(cand_ids[c])
    count = len(kept)
    assert sorted(new_ids.keys()) == list(range(count)), "valid slots must be [0, count)"
    return assign, [new_ids[p] for p in range(count)], status


def head_shared_masses(st: dict, mass_pool: np.ndarray, mass_win: np.ndarray):
    """R20 (head-shared pool): the score of a block for batch element b is
    the sum of its masses over the heads, matched by block id: per head, the
    pool slot holding the id, or the window slot (shared by all heads).
    Returns mass arrays of the input shapes holding those sums."""
    st = as_f64_state(st)
    pool_id = np.asarray(st["pool_id"]); pool_count = np.asarray(st["pool_count"])
    win_id = np.asarray(st["win_id"])
    B, H, C = pool_id.shape
    W = win_id.shape[0]
    mp = np.zeros((B, H, C)); mw = np.zeros((B, H, W))
    for b in range(B):
        tot = {}
        for h in range(H):
            for p in range(int(pool_count[b, h])):
                x = int(pool_id[b, h, p])
                tot[x] = tot.get(x, 0.0) + float(mass_pool[b, h, p])
        for w in range(W):
            x = int(win_id[w])
            tot[x] = tot.get(x, 0.0) + float(sum(mass_win[b, h, w] for h in range(H)))
        for h in range(H):
            for p in range(int(pool_count[b, h])):
                mp[b, h, p] = tot[int(pool_id[b, h, p])]
            for w in range(W):
                mw[b, h, w] = tot[int(win_id[w])]
    return mp, mw


def memory_update(st: dict, mass_pool: np.ndarray, mass_win: np.ndarray, leaving: Iterable[int],
                  n_sink: int, kbar_win: Optional[np.ndarray] = None,
                  kbar_pool: Optional[np.ndarray] = None, shared_heads: bool = False) -> dict:
    """Apply the Top-C update to every (b, h) and return the new pool state
    (copies; the inputs are not modified).  Leaving slots that are empty
    (len 0) are not candidates.  Pool K/V/len/id (and the pooled means if
    given) of admitted blocks are bit-exact copies of their window slot (R14).
    With ``shared_heads`` every head ranks by the head-summed masses (R20),
    so heads that hold the same pool make the same decision.
    """
    if shared_heads:
        mass_pool, mass_win = head_shared_masses(st, mass_pool, mass_win)
    st = as_f64_state(st)
    k_pool = np.array(st["k_pool"], copy=True); v_pool = np.array(st["v_pool"], copy=True)
    pool_len = np.array(st["pool_len"], copy=True); pool_id = np.array(st["pool_id"], copy=True)
    pool_count = np.array(st["pool_count"], copy=True)
    k_win = np.asarray(st["k_win"]); v_win = np.asarray(st["v_win"])
    win_len = np.asarray(st["win_len"]); win_id = np.asarray(st["win_id"])
    kp = None if kbar_pool is None else np.array(kbar_pool, copy=True)
    B, H, C = pool_len.shape
    leaving = [int(w) for w in leaving if int(win_len[int(w)]) > 0]
    status = np.zeros((B, H), dtype=np.int64)
    admitted_map = {}
    for b in range(B):
        for h in range(H):
            n = int(pool_count[b, h])
            ids = [int(pool_id[b, h, p]) for p in range(n)]
            pm = [float(mass_pool[b, h, p]) for p in range(n)]
            cids = [int(win_id[w]) for w in leaving]
            cm = [float(mass_win[b, h, w]) for w in leaving]
            assign, new_ids, stt = memory_update_one(ids, pm, cids, cm, C, n_sink)
            status[b, h] = stt
            for slot, c in assign:
                w = leaving[c]
                k_pool[b, h, slot] = k_win[b, h, w]
                v_pool[b, h, slot] = v_win[b, h, w]
                pool_len[b, h, slot] = win_len[w]
                pool_id[b, h, slot] = win_id[w]
                if kp is not None:
                    kp[b, h, slot] = kbar_win[b, h, w]
            pool_count[b, h] = len(new_ids)
            admitted_map[(b, h)] = [(slot, leaving[c]) for slot, c in assign]
    return dict(k_pool=k_pool, v_pool=v_pool, pool_len=pool_len, pool_id=pool_id,
                pool_count=pool_count, kbar_pool=kp, status=status, admitted=admitted_map)

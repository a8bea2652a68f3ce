"""CPU oracle for the DSV dynamic block-sparse attention path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it, and it
shares no code with the library: it is a plain, slow, float64 NumPy statement
of what the path computes, used to judge the GPU results.

Sources.  Two machine-written explainer pages of the same paper, both titled
"DSV: Exploiting Dynamic Sparsity to Accelerate Large-Scale Video DiT
Training": the German one (gist.science/de/paper/2502.07590, cited "[de]") and
the Spanish one (gist.science/es/paper/2502.07590, cited "[es]").  Section
numbers refer to the technical summaries on those pages.  The pages state the
method in prose only (no equations, no listings); where they leave a step open
the reading taken is named in the function that takes it.

The path, in the pages' order:
  1. per-head low-rank predictor matrices W^Q_lr, W^K_lr whose product
     approximates Q K^T of that head ([es] §2.A; [de] §2.A);
  2. the predicted attention mass of each (query group, KV block) pair, computed
     without keeping the full N x N matrix ([de] §2.A; §2.B, the fused matmul and top-k;
     [es] §2.B);
  3. top-k selection of the critical KV blocks per query group ([de] §2.B;
     [es] §2.B); neighbouring queries form one group ([es] §2.B, query
     grouping; [de] §2.B);
  4. exact softmax attention restricted to the selected KV blocks, forward and
     backward, because the method trains with it ([es] §3; [de] §2.A, stage 2).

Readings where the pages are silent, ambiguous or garbled:
  R1 the predictor acts on each head's Q and K: Q_lr = Q W^Q_lr, K_lr = K W^K_lr
     with W in R^{d x r};
  R2 predicted logits are pred_scale * <Q_lr_i, K_lr_j> (pred_scale defaults to
     1/sqrt(d)); there is no causal mask (video DiT self-attention is full);
  R3 the two operands of the logit product are rounded once to the run's
     storage dtype (bf16: nearest, ties to even; fp32 runs keep them exact).  The
     query operand carries the logit scale, in base-2 units, before that rounding:
     Q~ = rho(pred_scale * log2(e) * Q W^Q_lr), K_lr = rho(K W^K_lr), and the
     logit is l_ij = ln(2) * <Q~_i, K_lr_j> (in fp32 runs exactly R2's
     pred_scale * <Q_lr_i, K_lr_j>);
  R4-R5 a block score is the predicted softmax mass of the query block on the KV
     block, SUMMED over the block's Bq rows (each score row sums to Bq);
  R6 every query row of a group contributes (the Spanish page's joint
     processing); the representative-row variant of the German page is a
     separate function;
  R7 fixed k per query block; ties go to the smaller KV-block index; the list
     is emitted ascending and duplicate-free; no block is forced in;
  R8 the sparse softmax is renormalised over the selected keys only; LSE is a
     natural log of the scaled logits;
  R9 N must be a multiple of Bq and of Bk, and Bq a multiple of Bk;
  R13 mass-threshold selection (the pages' own rule: keep the critical KV blocks that
     carry ~90% of the score, [de] §2.A, [es] §2.A): per query block, the smallest
     set of KV blocks, taken by descending score (ties to the smaller index), whose
     scores sum to at least tau times the row's total score; capped at kmax blocks,
     never empty.  Lists are ascending and padded with -1 to kmax; a negative entry
     of any block list means "no block", and a query block whose list is empty has
     O = 0, LSE = -inf and no gradient;
  R14 per-block activation of sparse attention (the pages switch a block to sparse
     attention once it is sparse enough, [de] §2.A, stage 2; [es] §2.A): the measure
     is a head's selected density, the selected KV blocks summed over its query
     blocks divided by (query blocks x KV blocks); the head is flagged dense when
     that sum exceeds floor(dense_above * query blocks * KV blocks), an integer
     comparison.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

# --------------------------------------------------------------------------
# storage rounding (R3)
# --------------------------------------------------------------------------


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value of each float64 element (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range; below
    2**-126 the spacing is fixed at 2**-133 (subnormals); beyond the largest
    finite value the result is +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)                   # xf = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)               # subnormal range: fixed quantum 2**-133
    quantum = np.ldexp(1.0, e - 8)        # spacing of 8-bit significands at this exponent
    r = np.rint(xf / quantum) * quantum   # np.rint rounds half to even
    big = np.abs(r) > 3.3895313892515355e38  # largest finite bfloat16
    r[big] = np.copysign(np.inf, r[big])
    out[fin] = r
    return out


def rho(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage rounding of the predictor projections (R3)."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


def _check_blocks(n: int, bq: int, bk: int) -> None:
    if n % bq or n % bk or bq % bk:
        raise ValueError(f"N={n} must be a multiple of Bq={bq} and Bk={bk}, and Bq of Bk (R9)")


# --------------------------------------------------------------------------
# 1. predictor projection ([es] §2.A low-rank estimators; [de] §2.A)
# --------------------------------------------------------------------------


def project(x: np.ndarray, w: np.ndarray, dtype: str) -> np.ndarray:
    """Low-rank projection of one head: rho(x @ w), x [N, d], w [d, r] -> [N, r] (R1, R3)."""
    return rho(np.asarray(x, np.float64) @ np.asarray(w, np.float64), dtype)


LOG2E = 1.0 / math.log(2.0)
LN2 = math.log(2.0)


def project_query(x: np.ndarray, w: np.ndarray, pred_scale: float, dtype: str) -> np.ndarray:
    """Query operand of the predictor (R1-R3): rho(pred_scale * log2(e) * (x @ w)).

    The logit scale in base-2 units is applied before the one rounding, so the
    logit of R2 is ln(2) * <Q~_i, K_lr_j>: pass ``LN2`` as the scale of the score
    functions below when they are given Q~.
    """
    return rho(pred_scale * LOG2E * (np.asarray(x, np.float64) @ np.asarray(w, np.float64)), dtype)


# --------------------------------------------------------------------------
# 2. predicted block mass ([de] §2.A, §2.B; [es] §2.A-B)
# --------------------------------------------------------------------------


def block_scores_qblock(q_lr_blk: np.ndarray, k_lr: np.ndarray, bk: int, pred_scale: float) -> np.ndarray:
    """Predicted softmax mass of one query block on every KV block -> [nkb] (R2, R4-R5, R6).

    Every row i of the block gets the full predicted softmax over all N keys,
    P_ij = exp(l_ij - max_j l) / sum_j exp(l_ij - max_j l) with
    l_ij = pred_scale * <q_lr_i, k_lr_j>; the block score is the sum of P_ij
    over the block's rows i and the KV block's keys j.  Only Bq x N logits are
    held at once (the method never keeps the N x N matrix).
    """
    n = k_lr.shape[0]
    logits = pred_scale * (np.asarray(q_lr_blk, np.float64) @ np.asarray(k_lr, np.float64).T)
    shifted = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(shifted)
    p = e / e.sum(axis=1, keepdims=True)
    return p.reshape(p.shape[0], n // bk, bk).sum(axis=(0, 2))


def block_scores_head(q_lr: np.ndarray, k_lr: np.ndarray, bq: int, bk: int, pred_scale: float) -> np.ndarray:
    """[nqb, nkb] block scores of one head from its projections."""
    n = q_lr.shape[0]
    _check_blocks(n, bq, bk)
    return np.stack([block_scores_qblock(q_lr[qb * bq:(qb + 1) * bq], k_lr, bk, pred_scale)
                     for qb in range(n // bq)])


def predict(q, k, wq, wk, bq: int, bk: int, pred_scale: float, dtype: str):
    """Full predictor over [B, H, N, d] inputs and [H, d, r] weights.

    Returns (scores [B, H, nqb, nkb], q~ [B, H, N, r], k_lr [B, H, N, r]), q~ the
    scaled query operand of R3 (logits ln(2) <q~_i, k_lr_j>).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    b_, h_, n, _ = q.shape
    _check_blocks(n, bq, bk)
    r = wq.shape[-1]
    q_lr = np.empty((b_, h_, n, r))
    k_lr = np.empty((b_, h_, n, r))
    scores = np.empty((b_, h_, n // bq, n // bk))
    for b in range(b_):
        for h in range(h_):
            q_lr[b, h] = project_query(q[b, h], wq[h], pred_scale, dtype)
            k_lr[b, h] = project(k[b, h], wk[h], dtype)
            scores[b, h] = block_scores_head(q_lr[b, h], k_lr[b, h], bq, bk, LN2)
    return scores, q_lr, k_lr


def representative_scores_head(q_lr: np.ndarray, k_lr: np.ndarray, bq: int, bk: int, pred_scale: float,
                               rep: int = 0) -> np.ndarray:
    """Representative-row variant ([de] §2.B, query grouping): the group's estimate is the
    predicted softmax mass of its row ``rep`` alone -> [nqb, nkb] (each row sums to 1)."""
    n = q_lr.shape[0]
    _check_blocks(n, bq, bk)
    return np.stack([block_scores_qblock(q_lr[qb * bq + rep:qb * bq + rep + 1], k_lr, bk, pred_scale)
                     for qb in range(n // bq)])


# --------------------------------------------------------------------------
# 3. top-k selection ([de] §2.B, top-k selection; [es] §2.B)
# --------------------------------------------------------------------------


def select_topk_row(scores_row: np.ndarray, k: int) -> np.ndarray:
    """The k highest-scoring KV blocks of one query block, ties to the smaller index,
    returned ascending (R7)."""
    n = scores_row.shape[0]
    if not 1 <= k <= n:
        raise ValueError(f"k={k} out of range [1, {n}]")
    order = np.lexsort((np.arange(n), -np.asarray(scores_row, np.float64)))
    return np.sort(order[:k]).astype(np.int32)


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """[..., nkb] scores -> [..., k] int32 ascending block lists."""
    flat = scores.reshape(-1, scores.shape[-1])
    out = np.stack([select_topk_row(r, k) for r in flat])
    return out.reshape(scores.shape[:-1] + (k,))


def topk_gap(scores: np.ndarray, k: int) -> np.ndarray:
    """s_(k) - s_(k+1) of each row (the k-th minus the (k+1)-th largest score); +inf when k = nkb."""
    s = -np.sort(-scores.reshape(-1, scores.shape[-1]), axis=1)
    if k >= s.shape[1]:
        gap = np.full(s.shape[0], np.inf)
    else:
        gap = s[:, k - 1] - s[:, k]
    return gap.reshape(scores.shape[:-1])


def select_mass_row(scores_row: np.ndarray, tau: float, kmax: int) -> np.ndarray:
    """Mass-threshold selection of one query block (R13): the smallest descending-score prefix
    (ties to the smaller index) whose sum reaches tau * sum(scores_row), at most kmax blocks and
    at least one; returned ascending."""
    n = scores_row.shape[0]
    if not 1 <= kmax <= n:
        raise ValueError(f"kmax={kmax} out of range [1, {n}]")
    s = np.asarray(scores_row, np.float64)
    order = np.lexsort((np.arange(n), -s))
    csum = np.cumsum(s[order])
    reached = np.nonzero(csum >= tau * s.sum())[0]
    m = int(reached[0]) + 1 if reached.size else n
    m = max(1, min(m, kmax))
    return np.sort(order[:m]).astype(np.int32)


def select_mass(scores: np.ndarray, tau: float, kmax: int) -> Tuple[np.ndarray, np.ndarray]:
    """[..., nkb] scores -> ([..., kmax] int32 ascending lists padded with -1, [...] int32 counts)."""
    flat = scores.reshape(-1, scores.shape[-1])
    idx = np.full((flat.shape[0], kmax), -1, np.int32)
    cnt = np.zeros(flat.shape[0], np.int32)
    for i, r in enumerate(flat):
        sel = select_mass_row(r, tau, kmax)
        idx[i, :sel.size] = sel
        cnt[i] = sel.size
    return idx.reshape(scores.shape[:-1] + (kmax,)), cnt.reshape(scores.shape[:-1])


def mass_margin(scores: np.ndarray, tau: float) -> np.ndarray:
    """How far the uncapped cut of each row is from being decided otherwise: with c_m the sum of
    the m largest scores and m the selected count, min(c_m - T, T - c_{m-1}) for the target
    T = tau * row total (c_0 = -inf).  A cut with a small margin can legitimately move by one
    block when the sums are formed in another precision or order."""
    flat = np.asarray(scores, np.float64).reshape(-1, scores.shape[-1])
    out = np.empty(flat.shape[0])
    for i, r in enumerate(flat):
        t = tau * r.sum()
        c = np.cumsum(np.sort(r)[::-1])
        reached = np.nonzero(c >= t)[0]
        m = int(reached[0]) + 1 if reached.size else r.size
        above = c[m - 1] - t if reached.size else np.inf
        below = t - c[m - 2] if m >= 2 else np.inf
        out[i] = min(above, below)
    return out.reshape(scores.shape[:-1])


def head_density(counts: Optional[np.ndarray], k: int, nqb: int, nkb: int, dense_above: float):
    """Selected density of each head and its dense flag (R14).

    counts [B, H, nqb] list lengths (clamped to [0, k]) or None (every list holds k blocks).
    Returns (density [B, H] float64, dense [B, H] bool)."""
    if counts is None:
        raise ValueError("pass counts, or use np.full((B, H, nqb), k)")
    c = np.clip(np.asarray(counts, np.int64), 0, k)
    total = c.sum(axis=-1)                     # exact integer sums
    cells = nqb * nkb
    density = total / cells
    limit = math.floor(dense_above * cells)    # dense_above * cells in float64, then floor
    return density, total > limit


def block_recall(q, k, idx, bq: int, bk: int, sm_scale: float) -> np.ndarray:
    """True attention mass captured by the selected blocks (R15; [de] §2.A: the critical KV carry
    most of the score; the profiler's question is how much): per query block, the mean over its rows of
    sum_{j selected} softmax(sm_scale q_i K^T)_j, with the softmax over ALL keys.
    q, k [B, H, N, d]; idx [B, H, nqb, k] (negative entries select nothing) -> [B, H, nqb]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    b_, h_, n, _ = q.shape
    nqb = n // bq
    out = np.zeros((b_, h_, nqb))
    for b in range(b_):
        for h in range(h_):
            for qb in range(nqb):
                s = sm_scale * (q[b, h, qb * bq:(qb + 1) * bq] @ k[b, h].T)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                keys = selected_keys(idx[b, h, qb], bk)
                out[b, h, qb] = p[:, keys].sum(axis=1).mean()
    return out


def pack_selected(idx: np.ndarray, counts: Optional[np.ndarray], qb_begin: int, qb_end: int, nkb: int):
    """Sequence-parallel send list ([de] §2.C, [es] §2.C: context parallelism that moves only the
    KV the selection needs): per (b, h) the union of the KV blocks selected by query blocks
    [qb_begin, qb_end), ascending.

    idx [B, H, nqb, k], counts [B, H, nqb] or None (all k).  Returns
      blocks [B, H, nkb]  the union ascending, then -1;   count [B, H];
      remapped [B, H, qb_end - qb_begin, k]  each list entry's position in the union (-1 past
      the row's count or for an out-of-range entry)."""
    b_, h_, nqb, k = idx.shape
    blocks = np.full((b_, h_, nkb), -1, np.int32)
    count = np.zeros((b_, h_), np.int32)
    remapped = np.full((b_, h_, qb_end - qb_begin, k), -1, np.int32)
    for b in range(b_):
        for h in range(h_):
            lens = [k if counts is None else int(np.clip(counts[b, h, qb], 0, k)) for qb in range(nqb)]
            sel = sorted({int(x) for qb in range(qb_begin, qb_end) for x in idx[b, h, qb, :lens[qb]] if 0 <= x < nkb})
            blocks[b, h, :len(sel)] = sel
            count[b, h] = len(sel)
            where = {kb: u for u, kb in enumerate(sel)}
            for qb in range(qb_begin, qb_end):
                for j in range(lens[qb]):
                    x = int(idx[b, h, qb, j])
                    if 0 <= x < nkb:
                        remapped[b, h, qb - qb_begin, j] = where[x]
    return blocks, count, remapped


def pack_rows(x: np.ndarray, blocks: np.ndarray, count: np.ndarray, bk: int) -> np.ndarray:
    """[B, H, N, d] rows of the packed KV blocks: rows [u*bk, (u+1)*bk) of the result hold block
    blocks[b, h, u] of x, for u < count; later rows are left zero."""
    out = np.zeros_like(x)
    for b in range(x.shape[0]):
        for h in range(x.shape[1]):
            for u in range(int(count[b, h])):
                kb = int(blocks[b, h, u])
                out[b, h, u * bk:(u + 1) * bk] = x[b, h, kb * bk:(kb + 1) * bk]
    return out


# --------------------------------------------------------------------------
# 4. sparse attention over the selected blocks ([es] §3; [de] §2.A, stage 2)
# --------------------------------------------------------------------------


def selected_keys(idx_row: np.ndarray, bk: int, nkb: Optional[int] = None) -> np.ndarray:
    """Token indices of the selected KV blocks, block by block in list order (negative
    entries pad a ragged list and select nothing, R13).

    R7: a list names each selected block once.  With ``nkb`` given, a list whose non-negative
    entries repeat a block or reach past the last block (>= nkb) is rejected: the attention is
    defined only for distinct in-range lists."""
    idx_row = np.asarray(idx_row, np.int64)
    idx_row = idx_row[idx_row >= 0]
    if nkb is not None and (np.any(idx_row >= nkb) or np.unique(idx_row).size != idx_row.size):
        raise ValueError(f"block list {idx_row.tolist()} repeats a block or exceeds the {nkb} KV blocks (R7)")
    return (idx_row[:, None] * bk + np.arange(bk)[None, :]).reshape(-1)


def attn_fwd_qblock(q_blk, k, v, idx_row, bk: int, sm_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of one query block over its selected keys only (R8).

    Returns (O [Bq, d], LSE [Bq]) with LSE_i = log sum_j exp(sm_scale <q_i, k_j>).  An empty
    list (R13) defines O = 0 and LSE = -inf.
    """
    keys = selected_keys(idx_row, bk, np.shape(k)[0] // bk)
    if keys.size == 0:
        return np.zeros((np.shape(q_blk)[0], np.shape(v)[-1])), np.full(np.shape(q_blk)[0], -np.inf)
    s = sm_scale * (np.asarray(q_blk, np.float64) @ np.asarray(k, np.float64)[keys].T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e / l) @ np.asarray(v, np.float64)[keys]
    return o, (m + np.log(l))[:, 0]


def sparse_attn_fwd(q, k, v, idx, bq: int, bk: int, sm_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """[B, H, N, d] inputs, idx [B, H, nqb, k] -> (O [B, H, N, d], LSE [B, H, N])."""
    q = np.asarray(q, np.float64)
    b_, h_, n, d = q.shape
    _check_blocks(n, bq, bk)
    o = np.empty((b_, h_, n, v.shape[-1]))
    lse = np.empty((b_, h_, n))
    for b in range(b_):
        for h in range(h_):
            for qb in range(n // bq):
                rows = slice(qb * bq, (qb + 1) * bq)
                o[b, h, rows], lse[b, h, rows] = attn_fwd_qblock(q[b, h, rows], k[b, h], v[b, h],
                                                                 idx[b, h, qb], bk, sm_scale)
    return o, lse


def attn_bwd_qblock(q_blk, k, v, do_blk, idx_row, bk: int, sm_scale: float):
    """Gradients of L = <O, dO> for one query block with respect to its inputs.

    With S = sm_scale Q K_J^T, P = softmax_row(S), O = P V_J (J = selected keys):
      dV_J = P^T dO,   dP = dO V_J^T,   dS = P o (dP - rowsum(P o dP)),
      dQ = sm_scale dS K_J,   dK_J = sm_scale dS^T Q.
    Returns (dQ [Bq, d], dK_J [|J|, d], dV_J [|J|, d], J); an empty list has no gradient.
    """
    keys = selected_keys(idx_row, bk, np.shape(k)[0] // bk)
    if keys.size == 0:
        dq = np.zeros(np.shape(q_blk))
        return dq, np.zeros((0, np.shape(k)[-1])), np.zeros((0, np.shape(v)[-1])), keys
    q_blk = np.asarray(q_blk, np.float64)
    kj = np.asarray(k, np.float64)[keys]
    vj = np.asarray(v, np.float64)[keys]
    do_blk = np.asarray(do_blk, np.float64)
    s = sm_scale * (q_blk @ kj.T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    dv = p.T @ do_blk
    dp = do_blk @ vj.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = sm_scale * (ds @ kj)
    dk = sm_scale * (ds.T @ q_blk)
    return dq, dk, dv, keys


def sparse_attn_bwd(q, k, v, do, idx, bq: int, bk: int, sm_scale: float):
    """[B, H, N, d] inputs -> (dQ, dK, dV), each [B, H, N, d]; idx is a constant."""
    q = np.asarray(q, np.float64)
    b_, h_, n, d = q.shape
    _check_blocks(n, bq, bk)
    dq = np.zeros_like(q)
    dk = np.zeros((b_, h_, n, k.shape[-1]))
    dv = np.zeros((b_, h_, n, v.shape[-1]))
    for b in range(b_):
        for h in range(h_):
            for qb in range(n // bq):
                rows = slice(qb * bq, (qb + 1) * bq)
                g_q, g_k, g_v, keys = attn_bwd_qblock(q[b, h, rows], k[b, h], v[b, h], do[b, h, rows],
                                                      idx[b, h, qb], bk, sm_scale)
                dq[b, h, rows] = g_q
                np.add.at(dk[b, h], keys, g_k)
                np.add.at(dv[b, h], keys, g_v)
    return dq, dk, dv


def attn_bwd_kvblock(q, k, v, do, idx, kb: int, bq: int, bk: int, sm_scale: float):
    """dK, dV of one KV block of one head ([N, d] inputs, idx [nqb, k]) -> ([Bk, d], [Bk, d]).

    Sums the contributions of every query block whose list holds ``kb``; used to
    check sampled KV blocks at sizes where the full backward is too slow.
    """
    n = q.shape[0]
    dk = np.zeros((bk, k.shape[-1]))
    dv = np.zeros((bk, v.shape[-1]))
    for qb in range(n // bq):
        row = np.asarray(idx[qb])
        hit = np.nonzero(row == kb)[0]
        if hit.size == 0:
            continue
        rows = slice(qb * bq, (qb + 1) * bq)
        _, g_k, g_v, _ = attn_bwd_qblock(q[rows], k, v, do[rows], row, bk, sm_scale)
        pos = int(np.sum(row[:hit[0]] >= 0))  # position among the list's valid entries
        dk += g_k[pos * bk:(pos + 1) * bk]
        dv += g_v[pos * bk:(pos + 1) * bk]
    return dk, dv


# --------------------------------------------------------------------------
# the whole step
# --------------------------------------------------------------------------


def default_scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)


def dsv_step(q, k, v, do, wq, wk, bq: int, bk: int, topk: int, dtype: str,
             sm_scale: Optional[float] = None, pred_scale: Optional[float] = None):
    """predict -> select -> sparse forward -> sparse backward, all in float64."""
    d = q.shape[-1]
    ps = default_scale(d, pred_scale)
    ss = default_scale(d, sm_scale)
    scores, q_lr, k_lr = predict(q, k, wq, wk, bq, bk, ps, dtype)
    idx = select_topk(scores, topk)
    o, lse = sparse_attn_fwd(q, k, v, idx, bq, bk, ss)
    grads = sparse_attn_bwd(q, k, v, do, idx, bq, bk, ss) if do is not None else None
    return {"scores": scores, "q_lr": q_lr, "k_lr": k_lr, "idx": idx, "o": o, "lse": lse, "grads": grads}

"""CPU oracle for the DSA hot path (lightning indexer -> top-k -> sparse GQA attention).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links this
module; only the tests, the smoke check and the CPU-baseline leg of the benchmark do.
It shares no code, table or constant with the HIP library.

What is computed, and where it comes from:

* Source A: the digest of the Kwai Keye-VL-2.0-30B-A3B technical report on mqxn.cn
  (news item 1966), section 一 ("why long video is hard"): a light "scout" module, the
  Lightning Indexer, scans every position and scores which deserve attention; it uses an
  MQA-style shared design (one key per position for all indexer heads); for every query
  token the 2048 most relevant positions of the context are kept; attention then runs only
  between the query and those positions, turning O(L^2) work into O(L*k).  The same section
  says the base model is GQA and that DSA was adapted to GQA for the first time.
* Source A, section 八 (inference engineering): top-k must be deterministic so that
  training and inference select identical sets.
* Source B: the aihot summary page "快手开源 Kwai Keye-VL-2.0-30B-A3B ..." (abstract):
  DSA adapted to a GQA multimodal architecture, lossless 256K context.
* Source C: the QbitAI re-post on news.chathome.org "將DSA注意力引入多模態 ...": DSA is run
  in a variable-length (packed) sequence mode.

The pages print no formula.  Readings adopted where they are silent (each one is also
listed in the design notes):
  R1  indexer score   I[t,s] = sum_j w[t,j] * max(0, <q_I[t,j,:], k_I[s,:]>), no extra scale
  R2  w is per (token, head)
  R3  causal prefix includes the diagonal: s in [0, t]
  R4  a prefix shorter than k is taken whole; the index list is padded with -1
  R5  ties go to the lower position; -0 equals +0
  R6  selected positions are returned in ascending order
  R21 the torch.topk-shaped variant orders the same set by descending score, then position
  R22 the backward recomputes the softmax over the selected keys; every index entry is one key
  R23 warm-up target = head-mean of the dense causal attention distribution; KL(target || indexer),
      summed over rows; the target is fixed (the attention is not trained in that stage)
  R8  GQA head h reads KV head h // (Hq // Hkv)
  R9  softmax scale passed explicitly (1/sqrt(D) by default), lse is natural-log and
      includes the scale
  R11 positions are sequence-local; no attention across packed sequences
  R12 a decode cache of length n holds the new token at position n-1
  R25 adjacent-query dedup: blocks of 16 consecutive packed rows; the union is over packed KV
      rows, each row keeps its own distinct valid positions through a 16-bit mask

Everything is float64.  Loops run per query row so that each step reads like its
definition; speed is not a goal.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "index_scores_row",
    "index_scores",
    "select_topk_row",
    "sparse_gqa_attention_row",
    "prefill",
    "decode",
    "default_softmax_scale",
    "adjacent_query_union",
    "sparse_gqa_attention_union",
]


def default_softmax_scale(head_dim: int) -> float:
    """1/sqrt(D) (reading R9)."""
    return 1.0 / math.sqrt(head_dim)


def index_scores_row(q_idx_row: np.ndarray, w_row: np.ndarray, k_idx_prefix: np.ndarray) -> np.ndarray:
    """Lightning-indexer scores of one query token against its causal prefix.

    Source A, section 一: one shared key per position (MQA), several indexer heads.
    Reading R1: I[s] = sum_j w[j] * ReLU(<q_I[j], k_I[s]>).

    q_idx_row    [H_I, d_I]  indexer query heads of the token
    w_row        [H_I]       per-head weights of the token
    k_idx_prefix [n, d_I]    indexer keys of positions 0..n-1 (n = t+1)
    returns      [n] float64
    """
    q = np.asarray(q_idx_row, dtype=np.float64)
    w = np.asarray(w_row, dtype=np.float64)
    k = np.asarray(k_idx_prefix, dtype=np.float64)
    logits = q @ k.T                      # [H_I, n]: <q_I[j], k_I[s]>
    relu = np.maximum(logits, 0.0)        # ReLU per (head, position)
    return w @ relu                       # weighted sum over heads -> [n]


def index_scores(q_idx: np.ndarray, k_idx: np.ndarray, w: np.ndarray, cu_seqlens) -> list:
    """Scores of every packed query row against its own sequence's causal prefix.

    Returns a list with one float64 vector of length t+1 per packed row (reading R3, R11).
    """
    cu = [int(x) for x in cu_seqlens]
    out = []
    for b in range(len(cu) - 1):
        o, n = cu[b], cu[b + 1] - cu[b]
        for t in range(n):
            out.append(index_scores_row(q_idx[o + t], w[o + t], k_idx[o:o + t + 1]))
    return out


def select_topk_row(scores: np.ndarray, k: int) -> np.ndarray:
    """Per-query top-k (source A, section 一: keep the k most relevant positions).

    Readings R4-R6: a prefix of length <= k is kept whole; otherwise positions are ranked by
    (-score, position) so equal scores favour the lower position; the kept positions are
    returned in ascending order and padded with -1 to length k.  -0.0 and +0.0 compare equal
    under the float comparison used by the sort, so no special case is needed.
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    out = np.full(k, -1, dtype=np.int64)
    if n <= k:
        out[:n] = np.arange(n)
        return out
    # A stable sort on -score keeps equal scores in ascending position order.
    order = np.argsort(-s, kind="stable")
    chosen = np.sort(order[:k])
    out[:] = chosen
    return out


def select_topk_sorted_row(scores: np.ndarray, k: int):
    """Deterministic top-k in the shape of torch.topk(sorted=True) (source A, section 八: a
    deterministic top-k takes the place of torch.topk so that training and inference keep
    identical sets).

    Reading R21: the kept set is the one select_topk_row keeps; it is returned ordered by
    descending score and, among equal scores, ascending position, with the scores alongside;
    a row shorter than k is padded at the end with position -1 and score -inf.
    returns (idx [k] int64, values [k] float64)
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    m = min(n, k)
    idx = np.full(k, -1, dtype=np.int64)
    val = np.full(k, -np.inf, dtype=np.float64)
    # The same stable ranking as select_topk_row, kept in rank order instead of position order.
    order = np.argsort(-s, kind="stable")[:m]
    idx[:m] = order
    val[:m] = s[order]
    return idx, val


def sparse_gqa_attention_row(q_row: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray,
                             idx_row: np.ndarray, softmax_scale: float):
    """Attention of one token over its selected positions only (source A, section 一),
    with GQA sharing (source B; reading R8): query head h uses KV head h // G, and every
    query head of the token uses the same index set.

    q_row   [Hq, D]
    k_seq   [S, Hkv, D]   keys of the token's sequence (local positions)
    v_seq   [S, Hkv, D]
    idx_row [k]           selected local positions, negative entries are padding
    returns (O [Hq, D] float64, lse [Hq] float64, weight_sums [Hq] float64)
    """
    q = np.asarray(q_row, dtype=np.float64)
    hq, d = q.shape
    hkv = k_seq.shape[1]
    g_size = hq // hkv
    sel = np.asarray([int(i) for i in idx_row if int(i) >= 0], dtype=np.int64)
    o = np.zeros((hq, d), dtype=np.float64)
    lse = np.full(hq, -np.inf, dtype=np.float64)
    wsum = np.zeros(hq, dtype=np.float64)
    if sel.size == 0:
        return o, lse, wsum
    for h in range(hq):
        g = h // g_size
        keys = np.asarray(k_seq[sel, g, :], dtype=np.float64)    # [n_sel, D]
        vals = np.asarray(v_seq[sel, g, :], dtype=np.float64)
        z = softmax_scale * (keys @ q[h])                         # [n_sel]
        m = z.max()
        e = np.exp(z - m)
        denom = e.sum()
        p = e / denom
        o[h] = p @ vals
        lse[h] = m + math.log(denom)
        wsum[h] = p.sum()
    return o, lse, wsum


def sparse_gqa_attention_row_grad(q_row: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray,
                                  idx_row: np.ndarray, softmax_scale: float, dout_row: np.ndarray):
    """Gradients of the selected-position attention of one token (the sparse adaptation stage
    of source A, section 一, trains the whole model through this attention; reading R22).

    Same arguments as sparse_gqa_attention_row plus dout_row [Hq, D], the gradient of the loss
    with respect to O.  Per query head, with p the softmax weights over the selected keys:
        dp_s = <dO, v_s>,   dz_s = p_s (dp_s - sum_u p_u dp_u)      (softmax backward)
        dq   = scale * sum_s dz_s k_s
        dk_s += scale * dz_s q,   dv_s += p_s dO                   (summed over the group's heads)
    Each index entry is one key, so a repeated entry contributes once per occurrence.
    returns (dq [Hq, D], dk_seq [S, Hkv, D], dv_seq [S, Hkv, D]) float64: this row's contributions
    """
    q = np.asarray(q_row, dtype=np.float64)
    do = np.asarray(dout_row, dtype=np.float64)
    hq, d = q.shape
    n_pos, hkv = k_seq.shape[0], k_seq.shape[1]
    g_size = hq // hkv
    sel = np.asarray([int(i) for i in idx_row if 0 <= int(i) < n_pos], dtype=np.int64)
    dq = np.zeros((hq, d), dtype=np.float64)
    dk = np.zeros((n_pos, hkv, d), dtype=np.float64)
    dv = np.zeros((n_pos, hkv, d), dtype=np.float64)
    if sel.size == 0:
        return dq, dk, dv
    for h in range(hq):
        g = h // g_size
        keys = np.asarray(k_seq[sel, g, :], dtype=np.float64)    # [n_sel, D]
        vals = np.asarray(v_seq[sel, g, :], dtype=np.float64)
        z = softmax_scale * (keys @ q[h])
        e = np.exp(z - z.max())
        p = e / e.sum()
        dp = vals @ do[h]
        dz = p * (dp - p @ dp)
        dq[h] = softmax_scale * (dz @ keys)
        np.add.at(dk[:, g, :], sel, softmax_scale * np.outer(dz, q[h]))
        np.add.at(dv[:, g, :], sel, np.outer(p, do[h]))
    return dq, dk, dv


def sparse_attention_grad(q, k, v, idx, cu_seqlens, dout, softmax_scale=None):
    """Backward of the sparse GQA attention over packed sequences (reading R22): dq for every
    row, dk and dv summed over every row and head that selected each position.  Entries of
    idx outside a row's causal prefix are ignored, as in the forward."""
    q = np.asarray(q, dtype=np.float64)
    total, hq, d = q.shape
    scale = default_softmax_scale(d) if softmax_scale is None else softmax_scale
    cu = [int(x) for x in cu_seqlens]
    dq = np.zeros_like(q)
    dk = np.zeros(np.shape(k), dtype=np.float64)
    dv = np.zeros(np.shape(v), dtype=np.float64)
    for b in range(len(cu) - 1):
        o = cu[b]
        for t in range(cu[b + 1] - o):
            r = o + t
            gq, gk, gv = sparse_gqa_attention_row_grad(q[r], k[o:o + t + 1], v[o:o + t + 1], idx[r], scale, dout[r])
            dq[r] = gq
            dk[o:o + t + 1] += gk
            dv[o:o + t + 1] += gv
    return dq, dk, dv


def attention_head_mean_row(q_row: np.ndarray, k_prefix: np.ndarray, softmax_scale: float) -> np.ndarray:
    """Target of the indexer's dense warm-up (source A, section 一: with the full attention left
    unchanged, the indexer is trained to follow the full attention distribution, the gap measured
    by KL divergence; reading R23): the causal softmax of every query head over the whole prefix,
    averaged over the query heads (GQA head h reads KV head h // G).

    q_row [Hq, D], k_prefix [n, Hkv, D] -> [n] float64, summing to 1
    """
    q = np.asarray(q_row, dtype=np.float64)
    hq = q.shape[0]
    g_size = hq // k_prefix.shape[1]
    acc = np.zeros(k_prefix.shape[0], dtype=np.float64)
    for h in range(hq):
        z = softmax_scale * (np.asarray(k_prefix[:, h // g_size, :], dtype=np.float64) @ q[h])
        e = np.exp(z - z.max())
        acc += e / e.sum()
    return acc / hq


def indexer_kl_row(scores_row: np.ndarray, target_row: np.ndarray):
    """KL(target || softmax(scores)) over one causal prefix, and its gradient with respect to
    the scores (reading R23; the target is fixed):
        r = softmax(I),  loss = sum_s p_s (log p_s - log r_s)  (terms with p_s = 0 are 0),
        dloss/dI_s = r_s - p_s
    returns (loss float, grad [n] float64)
    """
    i_row = np.asarray(scores_row, dtype=np.float64)
    p = np.asarray(target_row, dtype=np.float64)
    m = i_row.max()
    lse = m + math.log(np.exp(i_row - m).sum())
    log_r = i_row - lse
    pos = p > 0
    loss = float((p[pos] * (np.log(p[pos]) - log_r[pos])).sum())
    return loss, np.exp(log_r) - p


def index_scores_row_grad(q_idx_row: np.ndarray, w_row: np.ndarray, k_idx_prefix: np.ndarray,
                          dscores: np.ndarray):
    """Backward of index_scores_row (reading R1) for one query row: with c[j, s] = <q_j, k_s>,
        dw_j = sum_s dI_s max(0, c[j, s])
        dq_j = w_j sum_s dI_s [c[j, s] > 0] k_s
        dk_s = dI_s sum_j w_j [c[j, s] > 0] q_j
    (the ReLU's derivative is taken as 0 at 0).
    returns (dq [H_I, d_I], dw [H_I], dk [n, d_I]) float64
    """
    q = np.asarray(q_idx_row, dtype=np.float64)
    w = np.asarray(w_row, dtype=np.float64)
    k = np.asarray(k_idx_prefix, dtype=np.float64)
    d_i = np.asarray(dscores, dtype=np.float64)
    c = q @ k.T                                   # [H_I, n]
    dw = np.maximum(c, 0.0) @ d_i
    gmat = (w[:, None] * d_i[None, :]) * (c > 0)  # d loss / d c
    return gmat @ k, dw, gmat.T @ q


def indexer_warmup_loss_grads(q, k, q_idx, k_idx, w, cu_seqlens, softmax_scale=None):
    """Dense warm-up loss of the indexer (reading R23) over packed sequences: the sum over rows
    of KL(head-mean causal attention distribution || softmax of the row's indexer scores), and
    its gradients with respect to q_idx, k_idx and w (the attention inputs are not trained).
    returns (row_loss [T], dq_idx [T, H_I, d_I], dk_idx [T, d_I], dw [T, H_I]) float64
    """
    q = np.asarray(q, dtype=np.float64)
    total, hq, d = q.shape
    scale = default_softmax_scale(d) if softmax_scale is None else softmax_scale
    cu = [int(x) for x in cu_seqlens]
    row_loss = np.zeros(total, dtype=np.float64)
    dq_idx = np.zeros(np.shape(q_idx), dtype=np.float64)
    dk_idx = np.zeros(np.shape(k_idx), dtype=np.float64)
    dw = np.zeros(np.shape(w), dtype=np.float64)
    for b in range(len(cu) - 1):
        o = cu[b]
        for t in range(cu[b + 1] - o):
            r = o + t
            target = attention_head_mean_row(q[r], k[o:o + t + 1], scale)
            scores = index_scores_row(q_idx[r], w[r], k_idx[o:o + t + 1])
            row_loss[r], d_i = indexer_kl_row(scores, target)
            gq, gw, gk = index_scores_row_grad(q_idx[r], w[r], k_idx[o:o + t + 1], d_i)
            dq_idx[r] = gq
            dw[r] = gw
            dk_idx[o:o + t + 1] += gk
    return row_loss, dq_idx, dk_idx, dw


def _seq_of_row(cu: list, r: int) -> int:
    for b in range(len(cu) - 1):
        if cu[b] <= r < cu[b + 1]:
            return b
    raise IndexError(r)


def adjacent_query_union(idx, cu_seqlens, block_rows=16, blocks=None):
    """Merged index sets of neighbouring query rows (source A, section 八: adjacent queries
    choose largely the same positions, so their top-k sets are de-duplicated and every KV row
    of the merged set is fetched once; a mask keeps each query to its own positions).

    Reading R25: block b holds the packed rows block_rows*b .. block_rows*b + block_rows - 1
    (the last block may be shorter, and a block may span two sequences).  Entry p of row r,
    whose sequence starts at packed row o and whose local position is t = r - o, counts when
    0 <= p <= t and stands for the packed KV row o + p.  The block's union is the set of those
    KV rows in ascending order; bit j of a KV row's mask is set when row block_rows*b + j
    selected it.  A position listed twice by one row appears once.

    idx [total_rows, k] (any integers), cu_seqlens [B+1].
    Returns one (kv_rows int64 [U], masks int64 [U]) pair per block in `blocks` (all if None).
    """
    cu = [int(x) for x in cu_seqlens]
    total = cu[-1]
    n_blocks = (total + block_rows - 1) // block_rows
    blocks = range(n_blocks) if blocks is None else [int(b) for b in blocks]
    result = []
    for b in blocks:
        mask_of = {}
        for j in range(block_rows):
            r = b * block_rows + j
            if r >= total:
                break
            s = _seq_of_row(cu, r)
            t = r - cu[s]
            for p in idx[r]:
                p = int(p)
                if 0 <= p <= t:
                    kv = cu[s] + p
                    mask_of[kv] = mask_of.get(kv, 0) | (1 << j)
        kv_rows = sorted(mask_of)
        result.append((np.asarray(kv_rows, dtype=np.int64),
                       np.asarray([mask_of[x] for x in kv_rows], dtype=np.int64)))
    return result


def sparse_gqa_attention_union(q, k, v, kv_rows, masks, first_row, n_rows, softmax_scale):
    """Attention of the rows first_row .. first_row + n_rows - 1 of one block computed from the
    block's merged set (reading R25): row first_row + j attends over the packed KV rows whose
    mask has bit j, with the softmax and GQA sharing of sparse_gqa_attention_row.

    q [T, Hq, D], k / v [T, Hkv, D] over all packed rows; kv_rows, masks from
    adjacent_query_union.  Returns (O [n_rows, Hq, D], lse [n_rows, Hq]) in float64.
    """
    hq, d = q.shape[1], q.shape[2]
    out = np.zeros((n_rows, hq, d), dtype=np.float64)
    lse = np.zeros((n_rows, hq), dtype=np.float64)
    kv_rows = np.asarray(kv_rows, dtype=np.int64)
    masks = np.asarray(masks, dtype=np.int64)
    for j in range(n_rows):
        mine = kv_rows[((masks >> j) & 1) == 1]
        # The selected rows are addressed directly in the packed K / V (local position = the
        # packed row itself when the "sequence" starts at row 0).
        o, l, _ = sparse_gqa_attention_row(q[first_row + j], k, v, mine, softmax_scale)
        out[j], lse[j] = o, l
    return out, lse


def prefill(q, k, v, q_idx, k_idx, w, cu_seqlens, top_k, softmax_scale=None, rows=None):
    """The whole prefill path for the packed rows listed in `rows` (all rows if None).

    For each row r of sequence b (offset o, local position t = r - o):
      1. scores over the prefix [0, t] of sequence b     (index_scores_row)
      2. top-k positions, ascending, -1 padded           (select_topk_row)
      3. GQA attention over those positions              (sparse_gqa_attention_row)

    Returns dict with 'rows', 'idx' [n_rows, top_k] int64, 'out' [n_rows, Hq, D] float64,
    'lse' [n_rows, Hq] float64, 'wsum' [n_rows, Hq] float64.
    """
    cu = [int(x) for x in cu_seqlens]
    total = cu[-1]
    hq, d = q.shape[1], q.shape[2]
    if softmax_scale is None:
        softmax_scale = default_softmax_scale(d)
    rows = list(range(total)) if rows is None else [int(r) for r in rows]
    idx = np.full((len(rows), top_k), -1, dtype=np.int64)
    out = np.zeros((len(rows), hq, d), dtype=np.float64)
    lse = np.zeros((len(rows), hq), dtype=np.float64)
    wsum = np.zeros((len(rows), hq), dtype=np.float64)
    for i, r in enumerate(rows):
        b = _seq_of_row(cu, r)
        o0, t = cu[b], r - cu[b]
        sc = index_scores_row(q_idx[r], w[r], k_idx[o0:o0 + t + 1])
        sel = select_topk_row(sc, top_k)
        oo, ll, ws = sparse_gqa_attention_row(q[r], k[o0:cu[b + 1]], v[o0:cu[b + 1]], sel, softmax_scale)
        idx[i], out[i], lse[i], wsum[i] = sel, oo, ll, ws
    return {"rows": rows, "idx": idx, "out": out, "lse": lse, "wsum": wsum}


def decode(q, q_idx, w, k_cache, v_cache, k_idx_cache, seq_lens, top_k, softmax_scale=None, batch=None):
    """One decode step per sequence (reading R12: the new token sits at position n-1 of a
    cache of length n and sees positions 0..n-1).

    q [B, Hq, D], q_idx [B, H_I, d_I], w [B, H_I],
    k_cache/v_cache [B, S_max, Hkv, D], k_idx_cache [B, S_max, d_I], seq_lens [B].
    Returns dict with 'batch', 'idx' [n, top_k], 'out' [n, Hq, D], 'lse' [n, Hq], 'wsum', 'scores'
    (list of float64 score vectors, one per sequence).
    """
    bsz = q.shape[0]
    hq, d = q.shape[1], q.shape[2]
    if softmax_scale is None:
        softmax_scale = default_softmax_scale(d)
    batch = list(range(bsz)) if batch is None else [int(b) for b in batch]
    idx = np.full((len(batch), top_k), -1, dtype=np.int64)
    out = np.zeros((len(batch), hq, d), dtype=np.float64)
    lse = np.zeros((len(batch), hq), dtype=np.float64)
    wsum = np.zeros((len(batch), hq), dtype=np.float64)
    scores = []
    for i, b in enumerate(batch):
        n = int(seq_lens[b])
        sc = index_scores_row(q_idx[b], w[b], k_idx_cache[b, :n])
        sel = select_topk_row(sc, top_k)
        oo, ll, ws = sparse_gqa_attention_row(q[b], k_cache[b, :n], v_cache[b, :n], sel, softmax_scale)
        idx[i], out[i], lse[i], wsum[i] = sel, oo, ll, ws
        scores.append(sc)
    return {"batch": batch, "idx": idx, "out": out, "lse": lse, "wsum": wsum, "scores": scores}

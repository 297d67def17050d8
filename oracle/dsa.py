"""MLA-DSA (indexer -> top-k -> sparse attention) oracle, float64.  TEST INFRASTRUCTURE ONLY.

What the pages fix ([P1] §二.1, [P3] §架構創新 1):
  * a lightweight indexer scores every history position for each query;
  * only the top-k positions by that score are kept;
  * exact (core) attention runs over those positions only, so its per-query
    cost does not grow with the context;
  * MLA heads are 256 wide.

Readings taken where the pages are silent:
  * indexer score(i, s) = sum_h w[i, h] * max(0, <q_I[i, h], k_I[s]>), one
    indexer key per position shared by the indexer heads, one weight per
    (query, head), no scale;
  * candidates of query i at position p_i are the positions s <= p_i
    (causal, self included);
  * selection order is score descending, then position ascending (ties go to
    the lower position); -0.0 ranks equal to +0.0; when p_i + 1 <= k every
    candidate is kept;
  * the index list is returned in ascending position order, padded with -1;
  * attention is multi-query: all query heads share one K and one V row per
    position; scale = 1/sqrt(D) unless given.

CSA variant (the compressed alternative the pages contrast with DSA; the
library's reading): the indexer keys, K and V are block means over `ratio`
consecutive tokens (4 in the pages' description), and the query at token
position t sees the compressed entries j < floor((t+1)/ratio), i.e. the blocks
that end at or before t.  Indexer, top-k and sparse attention then run over
compressed entries exactly as DSA runs over positions; ratio = 1 is DSA.
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def n_candidates(p, ratio, S):
    """Number of keys visible to the query at token position p: keys s < floor((p+1)/ratio), at most S."""
    return max(0, min((p + 1) // ratio, S))


def dsa_indexer_scores(q_idx, k_idx, w, q_pos=None, ratio=1):
    """Indexer scores for every (query, history position) pair.

    q_idx: [B, T, Hi, Di]; k_idx: [B, S, Di]; w: [B, T, Hi];
    q_pos: [B] position of query row 0 (row i sits at q_pos[b] + i);
    None means row i sits at position i.  ratio: keys are entries of `ratio`
    tokens (CSA); 1 for DSA.
    Returns [B, T, S] float64; entries that are not candidates are NaN.
    """
    q_idx, k_idx, w = map(_f64, (q_idx, k_idx, w))
    B, T, Hi, Di = q_idx.shape
    S = k_idx.shape[1]
    out = np.full((B, T, S), np.nan)
    for b in range(B):
        base = 0 if q_pos is None else int(q_pos[b])
        # dots[i, h, s] = <q_idx[b, i, h], k_idx[b, s]>
        dots = (q_idx[b].reshape(T * Hi, Di) @ k_idx[b].T).reshape(T, Hi, S)
        score = (w[b][:, :, None] * np.maximum(dots, 0.0)).sum(axis=1)
        for i in range(T):
            n = n_candidates(base + i, ratio, S)
            out[b, i, :n] = score[i, :n]
    return out


def dsa_topk(scores, k, q_pos=None, ratio=1):
    """Top-k history positions per query row.

    scores: [B, T, S]; row i of batch b sits at token position
    p_i = q_pos[b] + i (or i) and has candidates s < n_candidates(p_i, ratio, S)
    (s <= p_i for ratio 1).  Selection: the first min(k, n) candidates in the
    order (score descending, position ascending).  Returned ascending, padded
    with -1.  Output int64 [B, T, k].
    """
    scores = _f64(scores)
    B, T, S = scores.shape
    idx = np.full((B, T, k), -1, dtype=np.int64)
    for b in range(B):
        base = 0 if q_pos is None else int(q_pos[b])
        for i in range(T):
            n_cand = n_candidates(base + i, ratio, S)
            cand = scores[b, i, :n_cand] + 0.0  # -0.0 + 0.0 == +0.0
            pos = np.arange(n_cand)
            # lexsort: last key is primary -> score descending, then position ascending
            order = np.lexsort((pos, -cand))
            sel = np.sort(order[: min(k, n_cand)])
            idx[b, i, : sel.size] = sel
    return idx


def dsa_sparse_attention(q, k, v, idx, scale=None):
    """Exact multi-query attention over the selected positions only.

    q: [B, T, Hq, D]; k, v: [B, S, D] (one KV head shared by all Hq query
    heads); idx: [B, T, kk] with -1 entries skipped.
    Returns (o [B, T, Hq, D], lse [B, T, Hq]) in float64.  A row with no
    selected position returns o = 0 and lse = -inf.
    """
    q, k, v = map(_f64, (q, k, v))
    B, T, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.zeros((B, T, Hq, D))
    lse = np.full((B, T, Hq), -np.inf)
    for b in range(B):
        for i in range(T):
            sel = idx[b, i]
            sel = sel[sel >= 0]
            if sel.size == 0:
                continue
            logits = scale * (q[b, i] @ k[b, sel].T)  # [Hq, n]
            m = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - m)
            l = p.sum(axis=1, keepdims=True)
            o[b, i] = (p @ v[b, sel]) / l
            lse[b, i] = (m + np.log(l))[:, 0]
    return o, lse


def dsa_sparse_attention_bwd(q, k, v, idx, do, scale=None):
    """Gradients of dsa_sparse_attention for an upstream gradient do of o.

    The pages train these layers ([P1] §二.1 notes DSA's training speed) but
    print no backward formula; this is the chain rule applied to the forward's
    definition, entry by entry of idx (an entry listed twice counts twice).
    The selection idx is discrete and receives no gradient.  Per row, with
    the row's entries s_1..s_n, K = k[s_j], V = v[s_j]:
      P  = softmax_j(scale * q_h . k_{s_j})      (the forward's weights)
      dP = do_h . v_{s_j}
      dS = P * (dP - sum_j P dP)                 (softmax derivative)
      dq_h        = scale * sum_j dS_hj k_{s_j}
      dk[s_j]    += scale * sum_h dS_hj q_h
      dv[s_j]    += sum_h P_hj do_h
    Returns (dq [B, T, Hq, D], dk [B, S, D], dv [B, S, D]) in float64; rows
    without an entry contribute nothing.
    """
    q, k, v, do = map(_f64, (q, k, v, do))
    B, T, Hq, D = q.shape
    S = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.zeros((B, T, Hq, D))
    dk = np.zeros((B, S, D))
    dv = np.zeros((B, S, D))
    for b in range(B):
        for i in range(T):
            sel = idx[b, i]
            sel = sel[sel >= 0]
            if sel.size == 0:
                continue
            kr, vr = k[b, sel], v[b, sel]
            logits = scale * (q[b, i] @ kr.T)  # [Hq, n]
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = do[b, i] @ vr.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, i] = scale * (ds @ kr)
            np.add.at(dk[b], sel, scale * (ds.T @ q[b, i]))
            np.add.at(dv[b], sel, p.T @ do[b, i])
    return dq, dk, dv


def csa_attention(q_idx, k_idx, w, q, k, v, ratio, topk, scale=None):
    """CSA forward for one layer over token-level inputs (see the module docstring).

    q_idx [B,T,Hi,Di], k_idx [B,T,Di], w [B,T,Hi], q [B,T,Hq,D], k, v [B,T,D]:
    block means over `ratio` tokens of k_idx, k and v (complete blocks only),
    indexer scores and top-`topk` over the visible compressed entries, sparse
    attention over the selected entries.  Returns (o, lse, idx).
    """
    from .hca import hca_compress

    kc_idx = hca_compress(k_idx, ratio)
    kc, vc = hca_compress(k, ratio), hca_compress(v, ratio)
    idx = dsa_topk(dsa_indexer_scores(q_idx, kc_idx, w, ratio=ratio), topk, ratio=ratio)
    o, lse = dsa_sparse_attention(q, kc, vc, idx, scale)
    return o, lse, idx

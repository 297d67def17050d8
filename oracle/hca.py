"""HCA (Heavily Compressed Attention) oracle, float64.  TEST INFRASTRUCTURE ONLY.

What the pages fix ([P1] §二.1, [P2] §混合稀疏注意力, [P3] §架構創新 1):
  * every 128 consecutive tokens become one cache entry (128x compression);
  * a query attends over all compressed history entries plus a short window
    of recent, uncompressed tokens;
  * HCA heads are 512 wide.

Readings taken where the pages are silent (each one is stated again in the
function that uses it):
  * the compression operator is the arithmetic mean of the block's K (and V)
    rows; Q is not compressed;
  * the window is the W most recent tokens, including the query's own token;
  * a compressed entry j (tokens j*blk .. j*blk+blk-1) is visible to query t
    iff the whole block lies at or before t-W, i.e. (j+1)*blk-1 <= t-W; the
    window covers t-W < s <= t.  The two sets never overlap; the tokens of the
    block that straddles t-W and lie outside the window are seen by neither;
  * one softmax over the union of both key sets, logits scale*<q, key> with
    scale = 1/sqrt(d) unless given; no sink, bias or gate.

Head shapes.  The plain shape has q, k, v all d = 512 wide.  [P3] §預訓練資料工程
item 3 (FlashMask-4) names a wider query/key head than value head, qk 576 and
v 512; every function here takes the query/key width from q and the value
width from v, and the default scale is 1/sqrt(query/key width).
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def hca_compress(x, blk):
    """Mean of each complete block of ``blk`` consecutive tokens.

    [P1] §二.1 / [P3] §架構創新 1: each run of 128 tokens is pressed into one
    cache entry.  Reading: the entry is the arithmetic mean of the block's
    rows.  Incomplete trailing tokens (fewer than ``blk``) form no entry.

    x: [..., T, d]  ->  [..., T // blk, d]  (float64, no rounding of the mean)
    """
    x = _f64(x)
    T, d = x.shape[-2], x.shape[-1]
    n = T // blk
    lead = x.shape[:-2]
    blocks = x[..., : n * blk, :].reshape(*lead, n, blk, d)
    return blocks.sum(axis=-2) / blk


def hca_visible_blocks(t, blk, window):
    """Number of compressed entries visible to the query at position t.

    Entry j is visible iff (j+1)*blk - 1 <= t - window, so the count is
    max(0, floor((t - window + 1) / blk)).
    """
    return max(0, (t - window + 1) // blk)


def hca_window_range(t, window):
    """Raw positions the query at position t sees uncompressed: (t-window, t], s >= 0."""
    return max(0, t - window + 1), t + 1  # half-open [lo, hi)


def hca_key_set(t, blk, window, n_entries=None):
    """(visible compressed entry ids, visible raw positions) for query t."""
    nc = hca_visible_blocks(t, blk, window)
    if n_entries is not None:
        nc = min(nc, n_entries)
    lo, hi = hca_window_range(t, window)
    return np.arange(nc), np.arange(lo, hi)


def _attend(q, keys, vals, scale):
    """One softmax over the given keys for a batch of heads.

    q: [H, d]; keys: [H, n, d]; vals: [H, n, dv].  Returns (o [H, dv], lse [H]).
    lse is the natural-log normaliser of the scaled logits.
    """
    logits = scale * np.einsum("hd,hnd->hn", q, keys)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    l = p.sum(axis=1, keepdims=True)
    o = np.einsum("hn,hnd->hd", p, vals) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def hca_attention_prefill(q, k, v, kc, vc, blk, window, scale=None, rows=None):
    """HCA prefill attention for the query positions ``rows``.

    [P1] §二.1: attention runs over the compressed entries plus a window of
    the most recent uncompressed tokens.  [P3] §架構創新 1: the query attends
    to all compressed history entries and the short recent window.

    q, k: [B, H, T, d]; v: [B, H, T, dv]; kc: [B, H, Nc, d], vc: [B, H, Nc, dv]
    (the compressed cache; for the plain method Nc = T // blk and
    kc = hca_compress(k, blk)).  dv may be smaller than d (qk 576 / v 512).
    rows: iterable of query positions (default: all of 0..T-1).
    Returns (o [B, H, len(rows), dv], lse [B, H, len(rows)]) in float64.
    """
    q, k, v, kc, vc = map(_f64, (q, k, v, kc, vc))
    B, H, T, d = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = list(range(T)) if rows is None else [int(t) for t in rows]
    o = np.zeros((B, H, len(rows), dv))
    lse = np.zeros((B, H, len(rows)))
    for b in range(B):
        for r, t in enumerate(rows):
            cj, rs = hca_key_set(t, blk, window, n_entries=kc.shape[2])
            keys = np.concatenate([kc[b][:, cj], k[b][:, rs]], axis=1)
            vals = np.concatenate([vc[b][:, cj], v[b][:, rs]], axis=1)
            o[b, :, r], lse[b, :, r] = _attend(q[b, :, t], keys, vals, scale)
    return o, lse


def hca_attention_decode(q, kc, vc, ring_k, ring_v, pos, blk, window, scale=None):
    """HCA decode: one query per sequence at position pos[b].

    Same key set as prefill row t = pos[b] ([P1] §二.1): compressed entries
    j < min(visible(t), Nc) from the cache, and the window positions
    t-window < s <= t read from a ring buffer of ``window`` slots where
    position s lives in slot s mod window.

    q: [B, H, d]; kc: [B, H, Nc, d]; vc: [B, H, Nc, dv]; ring_k: [B, H, window, d];
    ring_v: [B, H, window, dv].
    Returns (o [B, H, dv], lse [B, H]).
    """
    q, kc, vc, ring_k, ring_v = map(_f64, (q, kc, vc, ring_k, ring_v))
    B, H, d = q.shape
    dv = vc.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((B, H, dv))
    lse = np.zeros((B, H))
    for b in range(B):
        t = int(pos[b])
        cj, rs = hca_key_set(t, blk, window, n_entries=kc.shape[2])
        slots = rs % window
        keys = np.concatenate([kc[b][:, cj], ring_k[b][:, slots]], axis=1)
        vals = np.concatenate([vc[b][:, cj], ring_v[b][:, slots]], axis=1)
        o[b], lse[b] = _attend(q[b], keys, vals, scale)
    return o, lse


def hca_attention_bwd(q, k, v, kc, vc, blk, window, do, scale=None, rows=None):
    """Gradients of hca_attention_prefill (every row) for an upstream gradient do of o.

    The pages train the HCA layers (FlashMask-4, [P3] §預訓練資料工程 item 3, ships
    a backward pass) but print no backward formula; this is the chain rule of
    the forward's definition.  Per row t, with the row's keys (visible
    compressed entries, then the window positions) and P the forward's
    softmax weights over them:
      dP = do_t . value,   dS = P * (dP - sum P dP)      (softmax derivative)
      dq_t          = scale * sum dS * key
      d(key)       += scale * dS * q_t      (into dkc for an entry, dk for a window token)
      d(value)     += P * do_t              (into dvc, dv likewise)
    q, k: [B, H, T, d]; v, do: [B, H, T, dv]; kc: [B, H, Nc, d]; vc: [B, H, Nc, dv],
    treated as independent inputs.  Returns (dq, dk, dv, dkc, dvc) in float64:
    dk, dv hold only the window path; the path through the compression is
    hca_compress_bwd(dkc) (hca_layer_bwd adds both).
    rows: the query rows whose terms are summed (default: every row); dq of
    the other rows is left 0 and dk, dv, dkc, dvc hold only the listed rows'
    contributions (complete for a position s when rows covers s .. s+window-1).
    """
    q, k, v, kc, vc, do = map(_f64, (q, k, v, kc, vc, do))
    B, H, T, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    dkc, dvc = np.zeros(kc.shape), np.zeros(vc.shape)
    rows = range(T) if rows is None else [int(t) for t in rows]
    for b in range(B):
        for t in rows:
            cj, rs = hca_key_set(t, blk, window, n_entries=kc.shape[2])
            nc = cj.size
            keys = np.concatenate([kc[b][:, cj], k[b][:, rs]], axis=1)  # [H, n, d]
            vals = np.concatenate([vc[b][:, cj], v[b][:, rs]], axis=1)  # [H, n, dv]
            logits = scale * np.einsum("hd,hnd->hn", q[b, :, t], keys)
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = np.einsum("hd,hnd->hn", do[b, :, t], vals)
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, :, t] = scale * np.einsum("hn,hnd->hd", ds, keys)
            dkey = scale * ds[:, :, None] * q[b, :, t][:, None, :]  # [H, n, d]
            dval = p[:, :, None] * do[b, :, t][:, None, :]          # [H, n, dv]
            dkc[b][:, cj] += dkey[:, :nc]
            dvc[b][:, cj] += dval[:, :nc]
            dk[b][:, rs] += dkey[:, nc:]
            dv[b][:, rs] += dval[:, nc:]
    return dq, dk, dv, dkc, dvc


def hca_compress_bwd(dxc, blk, T):
    """Gradient of hca_compress: entry j is the mean of tokens j*blk .. j*blk+blk-1, so each of
    them receives dxc[j] / blk; trailing tokens of an incomplete block receive nothing.

    dxc: [..., Nc, d] with Nc <= T // blk  ->  [..., T, d]
    """
    dxc = _f64(dxc)
    nc, d = dxc.shape[-2], dxc.shape[-1]
    out = np.zeros(dxc.shape[:-2] + (T, d))
    for j in range(nc):
        out[..., j * blk: (j + 1) * blk, :] = dxc[..., j: j + 1, :] / blk
    return out


def hca_layer_bwd(q, k, v, blk, window, do, scale=None):
    """Gradients of the whole HCA layer (K and V compressed with hca_compress, then
    hca_attention_prefill) with respect to the raw q, k, v: the window path plus the
    compression path.  Returns (dq, dk, dv, dkc, dvc) in float64."""
    T = np.shape(k)[-2]
    kc, vc = hca_compress(k, blk), hca_compress(v, blk)
    dq, dk, dv, dkc, dvc = hca_attention_bwd(q, k, v, kc, vc, blk, window, do, scale)
    return dq, dk + hca_compress_bwd(dkc, blk, T), dv + hca_compress_bwd(dvc, blk, T), dkc, dvc

"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each one.

Every mutation replaces one function of the oracle with a subtly wrong copy:
an off-by-one in the visibility rule or the window, a dropped scale, a wrong
mean divisor, a dropped ReLU, transposed head weights, the wrong tie-break,
padding entries not skipped.  The pin suite must fail for every one.
"""

import numpy as np
import pytest

import oracle
import oracle.dsa as odsa
import oracle.fp8 as ofp8
import oracle.hca as ohca
import oracle_pins


def _run_all_pins():
    """(pins whose assertions fail, pins that raised anything else).  Only an AssertionError counts
    as a catch: a mutant that merely crashes a pin (a wrong signature, an empty key set) is not
    detected by that pin."""
    failed, crashed = [], []
    for name, fn in sorted(oracle_pins.ALL_PINS.items()):
        try:
            fn()
        except AssertionError:
            failed.append(name)
        except Exception as e:  # noqa: BLE001 -- recorded, never counted as a catch
            crashed.append(f"{name}: {type(e).__name__}")
    return failed, crashed


def _mut_visible_off_by_one(t, blk, window):
    return max(0, (t - window) // blk)


def _mut_window_one_short(t, window):
    return max(0, t - window + 2), t + 1


def _mut_window_one_long(t, window):
    return max(0, t - window), t + 1


def _mut_attend_no_scale(q, keys, vals, scale):
    return _orig_attend(q, keys, vals, 1.0)


def _mut_compress_wrong_divisor(x, blk):
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape[-2], x.shape[-1]
    n = T // blk
    blocks = x[..., : n * blk, :].reshape(*x.shape[:-2], n, blk, d)
    return blocks.sum(axis=-2) / (blk + 1)


def _mut_compress_includes_tail(x, blk):
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[-2]
    n = -(-T // blk)
    out = [x[..., j * blk: (j + 1) * blk, :].mean(axis=-2) for j in range(n)]
    return np.stack(out, axis=-2)


_orig_attend = ohca._attend
_orig_encode = ofp8.e4m3_encode


def _mut_e4m3_bias8(code):
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e, m = (c >> 3) & 0xF, c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -10, (1.0 + m / 8.0) * np.exp2(e - 8.0))
    return sign * np.where((e == 15) & (m == 7), np.nan, mag)


def _mut_e4m3_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x80, 0)
    a = np.abs(x)
    _, ex = np.frexp(a)
    e = np.where(a > 0, np.maximum(ex - 1, -6), -6)
    n = np.floor(np.ldexp(a, -(e - 3)))
    return (sign | (8 * (e + 7) + (n.astype(np.int64) - 8))).astype(np.uint8)


def _mut_e4m3_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x80, 0)
    a = np.abs(x)
    _, ex = np.frexp(a)
    e = np.where(a > 0, np.maximum(ex - 1, -6), -6)
    n = np.floor(np.ldexp(a, -(e - 3)) + 0.5)
    return (sign | (8 * (e + 7) + (n.astype(np.int64) - 8))).astype(np.uint8)


def _mut_csa_partial_block_visible(p, ratio, S):
    return max(0, min(-(-(p + 1) // ratio), S))


def _mut_quantize_scale_inverted(x):
    codes, scales = _orig_quantize(x)
    with np.errstate(divide="ignore"):
        return codes, np.where(scales > 0, np.float32(1) / scales, 0).astype(np.float32)


_orig_prefill = ohca.hca_attention_prefill


def _mut_prefill_scale_from_v(q, k, v, kc, vc, blk, window, scale=None, rows=None):
    if scale is None:
        scale = 1.0 / np.sqrt(np.shape(v)[-1])
    return _orig_prefill(q, k, v, kc, vc, blk, window, scale, rows)


def _mut_prefill_qk_cut_to_v(q, k, v, kc, vc, blk, window, scale=None, rows=None):
    dv = np.shape(v)[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(np.shape(q)[-1])
    return _orig_prefill(np.asarray(q)[..., :dv], np.asarray(k)[..., :dv], v, np.asarray(kc)[..., :dv], vc, blk, window,
                         scale, rows)


_orig_quantize = ofp8.quantize_fp8_rows
_orig_scores = odsa.dsa_indexer_scores
_orig_topk = odsa.dsa_topk
_orig_sparse = odsa.dsa_sparse_attention
_orig_sparse_bwd = odsa.dsa_sparse_attention_bwd


def _mut_scores_no_relu(q_idx, k_idx, w, q_pos=None, ratio=1):
    q_idx, k_idx, w = (np.asarray(a, dtype=np.float64) for a in (q_idx, k_idx, w))
    B, T, Hi, Di = q_idx.shape
    S = k_idx.shape[1]
    out = np.full((B, T, S), np.nan)
    for b in range(B):
        base = 0 if q_pos is None else int(q_pos[b])
        dots = np.einsum("thd,sd->ths", q_idx[b], k_idx[b])
        score = (w[b][:, :, None] * dots).sum(axis=1)
        for i in range(T):
            n = odsa.n_candidates(base + i, ratio, S)
            out[b, i, :n] = score[i, :n]
    return out


def _mut_scores_weights_reversed(q_idx, k_idx, w, q_pos=None, ratio=1):
    w = np.asarray(w)[:, :, ::-1]
    return _orig_scores(q_idx, k_idx, w, q_pos, ratio)


def _mut_topk_ties_high(scores, k, q_pos=None, ratio=1):
    scores = np.asarray(scores, dtype=np.float64)
    B, T, S = scores.shape
    idx = np.full((B, T, k), -1, dtype=np.int64)
    for b in range(B):
        base = 0 if q_pos is None else int(q_pos[b])
        for i in range(T):
            n = odsa.n_candidates(base + i, ratio, S)
            cand = scores[b, i, :n] + 0.0
            order = np.lexsort((-np.arange(n), -cand))
            sel = np.sort(order[: min(k, n)])
            idx[b, i, : sel.size] = sel
    return idx


def _mut_topk_descending_output(scores, k, q_pos=None, ratio=1):
    idx = _orig_topk(scores, k, q_pos, ratio)
    out = idx.copy()
    for b in range(idx.shape[0]):
        for i in range(idx.shape[1]):
            valid = idx[b, i][idx[b, i] >= 0]
            out[b, i, : valid.size] = valid[::-1]
    return out


def _mut_sparse_keeps_padding(q, k, v, idx, scale=None):
    idx = np.where(np.asarray(idx) < 0, 0, idx)
    return _orig_sparse(q, k, v, idx, scale)


def _sparse_bwd_parts(q, k, v, idx, do, scale, ds_fn, dk_scale, dv_from_ds):
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    B, T, Hq, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(B):
        for i in range(T):
            sel = idx[b, i][idx[b, i] >= 0]
            if sel.size == 0:
                continue
            lg = scale * (q[b, i] @ k[b, sel].T)
            p = np.exp(lg - lg.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            ds = ds_fn(p, do[b, i] @ v[b, sel].T)
            dq[b, i] = scale * ds @ k[b, sel]
            np.add.at(dk[b], sel, dk_scale(scale) * (ds.T @ q[b, i]))
            np.add.at(dv[b], sel, (ds if dv_from_ds else p).T @ do[b, i])
    return dq, dk, dv


def _mut_sparse_bwd_no_rowsum(q, k, v, idx, do, scale=None):
    return _sparse_bwd_parts(q, k, v, idx, do, scale, lambda p, dp: p * dp, lambda s: s, False)


def _mut_sparse_bwd_dk_unscaled(q, k, v, idx, do, scale=None):
    return _sparse_bwd_parts(q, k, v, idx, do, scale, lambda p, dp: p * (dp - (p * dp).sum(1, keepdims=True)),
                             lambda s: 1.0, False)


def _mut_sparse_bwd_dv_from_ds(q, k, v, idx, do, scale=None):
    return _sparse_bwd_parts(q, k, v, idx, do, scale, lambda p, dp: p * (dp - (p * dp).sum(1, keepdims=True)),
                             lambda s: s, True)


_orig_hca_bwd = ohca.hca_attention_bwd


def _hca_bwd_variant(q, k, v, kc, vc, blk, window, do, scale, ds_fn, entry_scale, dval_from_ds):
    q, k, v, kc, vc, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, kc, vc, do))
    B, H, T, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    dkc, dvc = np.zeros(kc.shape), np.zeros(vc.shape)
    for b in range(B):
        for t in range(T):
            cj, rs = ohca.hca_key_set(t, blk, window, n_entries=kc.shape[2])
            nc = cj.size
            keys = np.concatenate([kc[b][:, cj], k[b][:, rs]], axis=1)
            vals = np.concatenate([vc[b][:, cj], v[b][:, rs]], axis=1)
            lg = scale * np.einsum("hd,hnd->hn", q[b, :, t], keys)
            p = np.exp(lg - lg.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            ds = ds_fn(p, np.einsum("hd,hnd->hn", do[b, :, t], vals))
            dq[b, :, t] = scale * np.einsum("hn,hnd->hd", ds, keys)
            dkey = ds[:, :, None] * q[b, :, t][:, None, :]
            dval = (ds if dval_from_ds else p)[:, :, None] * do[b, :, t][:, None, :]
            dkc[b][:, cj] += entry_scale(scale) * dkey[:, :nc]
            dvc[b][:, cj] += dval[:, :nc]
            dk[b][:, rs] += scale * dkey[:, nc:]
            dv[b][:, rs] += dval[:, nc:]
    return dq, dk, dv, dkc, dvc


def _ds_ok(p, dp):
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def _mut_hca_bwd_no_rowsum(q, k, v, kc, vc, blk, window, do, scale=None):
    return _hca_bwd_variant(q, k, v, kc, vc, blk, window, do, scale, lambda p, dp: p * dp, lambda s: s, False)


def _mut_hca_bwd_entry_unscaled(q, k, v, kc, vc, blk, window, do, scale=None):
    return _hca_bwd_variant(q, k, v, kc, vc, blk, window, do, scale, _ds_ok, lambda s: 1.0, False)


def _mut_hca_bwd_dv_from_ds(q, k, v, kc, vc, blk, window, do, scale=None):
    return _hca_bwd_variant(q, k, v, kc, vc, blk, window, do, scale, _ds_ok, lambda s: s, True)


def _mut_compress_bwd_no_divisor(dxc, blk, T):
    return _orig_compress_bwd(dxc, blk, T) * blk


def _mut_compress_bwd_into_tail(dxc, blk, T):
    out = _orig_compress_bwd(dxc, blk, T)
    nc = np.shape(dxc)[-2]
    if nc * blk < T:
        out[..., nc * blk:, :] = np.asarray(dxc, dtype=np.float64)[..., -1:, :] / blk
    return out


_orig_compress_bwd = ohca.hca_compress_bwd


MUTATIONS = {
    "visible_off_by_one": (ohca, "hca_visible_blocks", _mut_visible_off_by_one),
    "window_one_short": (ohca, "hca_window_range", _mut_window_one_short),
    "window_one_long": (ohca, "hca_window_range", _mut_window_one_long),
    "attend_no_scale": (ohca, "_attend", _mut_attend_no_scale),
    "compress_wrong_divisor": (ohca, "hca_compress", _mut_compress_wrong_divisor),
    "compress_includes_tail": (ohca, "hca_compress", _mut_compress_includes_tail),
    "scores_no_relu": (odsa, "dsa_indexer_scores", _mut_scores_no_relu),
    "scores_weights_reversed": (odsa, "dsa_indexer_scores", _mut_scores_weights_reversed),
    "topk_ties_high": (odsa, "dsa_topk", _mut_topk_ties_high),
    "topk_descending_output": (odsa, "dsa_topk", _mut_topk_descending_output),
    "sparse_keeps_padding": (odsa, "dsa_sparse_attention", _mut_sparse_keeps_padding),
    "sparse_bwd_no_rowsum": (odsa, "dsa_sparse_attention_bwd", _mut_sparse_bwd_no_rowsum),
    "sparse_bwd_dk_unscaled": (odsa, "dsa_sparse_attention_bwd", _mut_sparse_bwd_dk_unscaled),
    "sparse_bwd_dv_from_ds": (odsa, "dsa_sparse_attention_bwd", _mut_sparse_bwd_dv_from_ds),
    "e4m3_bias8": (ofp8, "e4m3_value", _mut_e4m3_bias8),
    "e4m3_truncate": (ofp8, "e4m3_encode", _mut_e4m3_truncate),
    "e4m3_ties_away": (ofp8, "e4m3_encode", _mut_e4m3_ties_away),
    "quantize_scale_inverted": (ofp8, "quantize_fp8_rows", _mut_quantize_scale_inverted),
    "csa_partial_block_visible": (odsa, "n_candidates", _mut_csa_partial_block_visible),
    "prefill_scale_from_v": (ohca, "hca_attention_prefill", _mut_prefill_scale_from_v),
    "prefill_qk_cut_to_v": (ohca, "hca_attention_prefill", _mut_prefill_qk_cut_to_v),
    "hca_bwd_no_rowsum": (ohca, "hca_attention_bwd", _mut_hca_bwd_no_rowsum),
    "hca_bwd_entry_unscaled": (ohca, "hca_attention_bwd", _mut_hca_bwd_entry_unscaled),
    "hca_bwd_dv_from_ds": (ohca, "hca_attention_bwd", _mut_hca_bwd_dv_from_ds),
    "compress_bwd_no_divisor": (ohca, "hca_compress_bwd", _mut_compress_bwd_no_divisor),
    "compress_bwd_into_tail": (ohca, "hca_compress_bwd", _mut_compress_bwd_into_tail),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_pins_catch_mutation(mutation, monkeypatch):
    mod, attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(mod, attr, fn)
    # the package namespace re-exports the public functions: patch it too
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    failed, crashed = _run_all_pins()
    assert failed, f"no pin's assertion caught mutation {mutation} (crashed: {crashed})"

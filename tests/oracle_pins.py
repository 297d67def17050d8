"""Pins for the float64 oracle: checks against facts other than the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a closed form, a hand-derived golden value, a library routine (torch CPU
scaled_dot_product_attention, NumPy matmul / sorted), an invariant of the
definition, or brute force on tiny inputs.  tests/test_oracle_pins.py runs
them against the oracle; tests/test_oracle_mutations.py plants plausible
mistakes in the oracle and checks that at least one pin then fails.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa_causal(q, k, v):
    """Dense causal attention from torch's CPU float64 library routine.  q,k,v: [B,H,T,d]."""
    import torch
    import torch.nn.functional as F

    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)) for a in (q, k, v))
    return F.scaled_dot_product_attention(tq, tk, tv, is_causal=True).numpy()


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err} > {tol}"


# ---------------------------------------------------------------------------
# hca_compress
# ---------------------------------------------------------------------------


def pin_compress_constant_blocks():
    """A block whose rows all equal one dyadic value compresses to it exactly."""
    rng = _rng(1)
    blk, n, d = 8, 5, 3
    c = rng.integers(-1000, 1000, size=(2, n, d)) / 64.0
    x = np.repeat(c, blk, axis=1)  # [2, n*blk, d]
    out = oracle.hca_compress(x, blk)
    assert out.shape == (2, n, d)
    assert np.array_equal(out, c), "constant blocks must compress exactly"


def pin_compress_ramp():
    """x[t] = t compresses to the block midpoint j*blk + (blk-1)/2 (exact)."""
    for blk in (1, 4, 128):
        T = 5 * blk + (blk // 2)  # ragged tail that must be ignored
        x = np.arange(T, dtype=np.float64)[:, None] * np.ones((1, 2))
        out = oracle.hca_compress(x, blk)
        assert out.shape == (T // blk, 2)
        want = np.arange(T // blk) * blk + (blk - 1) / 2.0
        assert np.array_equal(out[:, 0], want), f"ramp midpoint blk={blk}"


def pin_compress_bruteforce():
    rng = _rng(2)
    B, H, T, d, blk = 2, 3, 13, 4, 3
    x = rng.standard_normal((B, H, T, d))
    out = oracle.hca_compress(x, blk)
    assert out.shape == (B, H, T // blk, d)
    for b in range(B):
        for h in range(H):
            for j in range(T // blk):
                for e in range(d):
                    s = 0.0
                    for i in range(blk):
                        s += float(x[b, h, j * blk + i, e])
                    assert abs(out[b, h, j, e] - s / blk) < 1e-14


def pin_compress_pages_ratio():
    """The pages: one cache entry per 128 tokens, context up to 1,048,576 tokens."""
    c = _load("pages_constants.json")
    blk = c["tokens_per_compressed_entry"]["value"]
    for n_tok in (c["pretraining_context_tokens"]["value"], c["max_context_tokens"]["value"]):
        x = np.zeros((n_tok, 1), dtype=np.float32)
        assert oracle.hca_compress(x, blk).shape[0] * blk == n_tok


# ---------------------------------------------------------------------------
# HCA attention
# ---------------------------------------------------------------------------


def _hca_inputs(seed, B, H, T, d, blk):
    rng = _rng(seed)
    q, k, v = (rng.standard_normal((B, H, T, d)) for _ in range(3))
    return q, k, v, oracle.hca_compress(k, blk), oracle.hca_compress(v, blk)


def pin_hca_blk1_is_dense_causal():
    """blk = 1: visible entries and window tile 0..t exactly once -> dense causal."""
    B, H, T, d = 1, 2, 23, 8
    for window in (1, 3, 7, 40):
        q, k, v, kc, vc = _hca_inputs(3, B, H, T, d, 1)
        o, _ = oracle.hca_attention_prefill(q, k, v, kc, vc, 1, window)
        _close(o, _sdpa_causal(q, k, v), 1e-12, f"blk=1 window={window}")


def pin_hca_window_ge_T_is_dense_causal():
    B, H, T, d = 2, 2, 19, 8
    for blk in (2, 4, 16):
        q, k, v, kc, vc = _hca_inputs(4, B, H, T, d, blk)
        o, _ = oracle.hca_attention_prefill(q, k, v, kc, vc, blk, T)
        _close(o, _sdpa_causal(q, k, v), 1e-12, f"window>=T blk={blk}")


def pin_hca_rows_below_window_are_dense():
    B, H, T, d, blk, window = 1, 2, 40, 8, 4, 9
    q, k, v, kc, vc = _hca_inputs(5, B, H, T, d, blk)
    rows = list(range(window))
    o, _ = oracle.hca_attention_prefill(q, k, v, kc, vc, blk, window, rows=rows)
    _close(o, _sdpa_causal(q, k, v)[:, :, :window], 1e-12, "rows t < window")


def pin_hca_constant_v():
    B, H, T, d, blk, window = 1, 2, 50, 4, 4, 6
    q, k, _, kc, _ = _hca_inputs(6, B, H, T, d, blk)
    v = np.full((B, H, T, d), 0.375)
    vc = oracle.hca_compress(v, blk)
    o, _ = oracle.hca_attention_prefill(q, k, v, kc, vc, blk, window)
    _close(o, np.full_like(o, 0.375), 1e-14, "constant V")


def _literal_weights(q, k, blk, window, t, scale):
    """Brute force: enumerate every (block, token) and test the visibility rule literally.

    Returns the attention weight each raw token receives (compressed entries
    spread their weight evenly over their block's tokens)."""
    T = k.shape[0]
    keys = []  # (logit, list of (token, share))
    for j in range(T // blk):
        end = j * blk + blk - 1  # last token of block j
        if end <= t - window:
            mean = [sum(k[j * blk + i][e] for i in range(blk)) / blk for e in range(k.shape[1])]
            keys.append((scale * sum(a * b for a, b in zip(q, mean)), [(j * blk + i, 1.0 / blk) for i in range(blk)]))
    for s in range(T):
        if t - window < s <= t:
            keys.append((scale * sum(a * b for a, b in zip(q, k[s])), [(s, 1.0)]))
    m = max(lg for lg, _ in keys)
    z = sum(math.exp(lg - m) for lg, _ in keys)
    wts = [0.0] * T
    for lg, toks in keys:
        p = math.exp(lg - m) / z
        for s, share in toks:
            wts[s] += p * share
    return wts


def pin_hca_identity_v_weights():
    """V = identity exposes each query's weight on every raw token; compare with brute force."""
    T, d, blk, window = 24, 24, 4, 6
    rng = _rng(7)
    q = rng.standard_normal((1, 1, T, d))
    k = rng.standard_normal((1, 1, T, d))
    v = np.eye(T)[None, None]
    kc, vc = oracle.hca_compress(k, blk), oracle.hca_compress(v, blk)
    o, _ = oracle.hca_attention_prefill(q, k, v, kc, vc, blk, window)
    scale = 1.0 / math.sqrt(d)
    for t in range(T):
        w = o[0, 0, t]
        assert abs(w.sum() - 1.0) < 1e-12, "weights sum to one"
        assert np.all(w[t + 1:] == 0.0), "no weight on future tokens"
        ref = _literal_weights(q[0, 0, t], k[0, 0], blk, window, t, scale)
        _close(w, ref, 1e-12, f"identity-V weights t={t}")
        # gap tokens: in the block straddling t-window, outside the window
        lo = max(0, t - window + 1)
        nvis = max(0, (t - window + 1) // blk)
        for s in range(nvis * blk, lo):
            assert w[s] == 0.0, f"gap token {s} of query {t} must get no weight"


def pin_hca_uniform_golden():
    """q = 0 makes attention uniform; hand-derived outputs in tests/golden/hca_uniform_q0.json."""
    g = _load("hca_uniform_q0.json")
    T, blk, window = g["T"], g["blk"], g["window"]
    v = np.arange(T, dtype=np.float64).reshape(1, 1, T, 1)
    k = _rng(8).standard_normal((1, 1, T, 1))
    q = np.zeros((1, 1, T, 1))
    o, lse = oracle.hca_attention_prefill(q, k, v, oracle.hca_compress(k, blk), oracle.hca_compress(v, blk), blk, window)
    for row in g["rows"]:
        t = row["t"]
        want = float(Fraction(*row["o"]))
        assert abs(o[0, 0, t, 0] - want) < 1e-12, f"t={t}: {o[0, 0, t, 0]} != {want}"
        assert abs(lse[0, 0, t] - math.log(row["n_keys"])) < 1e-12, f"lse t={t}"
        cj, rs = oracle.hca_key_set(t, blk, window)
        assert list(cj) == row["visible_blocks"], f"visible blocks t={t}"
        assert [int(rs[0]), int(rs[-1])] == row["window"], f"window t={t}"


def pin_hca_decode_equals_prefill_row():
    """Decode at position t with the ring holding positions t-window+1..t equals prefill row t."""
    B, H, T, d, blk, window = 2, 3, 37, 8, 4, 6
    q, k, v, kc, vc = _hca_inputs(9, B, H, T, d, blk)
    rows = [0, 3, 5, 6, 11, 20, 36]
    o_pre, lse_pre = oracle.hca_attention_prefill(q, k, v, kc, vc, blk, window, rows=rows)
    for r, t in enumerate(rows):
        ring_k = np.zeros((B, H, window, d))
        ring_v = np.zeros((B, H, window, d))
        for s in range(max(0, t - window + 1), t + 1):
            ring_k[:, :, s % window] = k[:, :, s]
            ring_v[:, :, s % window] = v[:, :, s]
        o_dec, lse_dec = oracle.hca_attention_decode(q[:, :, t], kc, vc, ring_k, ring_v, [t] * B, blk, window)
        _close(o_dec, o_pre[:, :, r], 1e-12, f"decode vs prefill t={t}")
        _close(lse_dec, lse_pre[:, :, r], 1e-12, f"decode lse t={t}")


def pin_hca_head_permutation():
    B, H, T, d, blk, window = 1, 4, 30, 4, 4, 5
    q, k, v, kc, vc = _hca_inputs(10, B, H, T, d, blk)
    perm = [2, 0, 3, 1]
    o, _ = oracle.hca_attention_prefill(q, k, v, kc, vc, blk, window)
    op, _ = oracle.hca_attention_prefill(q[:, perm], k[:, perm], v[:, perm], kc[:, perm], vc[:, perm], blk, window)
    _close(op, o[:, perm], 1e-14, "head permutation")


def _sdpa_causal_grads(q, k, v, do):
    """Dense causal attention's gradients (dq, dk, dv) for upstream do, from torch's CPU float64
    autograd of its library routine.  q,k,v,do: [B,H,T,d]."""
    import torch
    import torch.nn.functional as F

    tq, tk, tv = (torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True) for a in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    o.backward(torch.from_numpy(np.ascontiguousarray(do, dtype=np.float64)))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def _central_diff(loss, args, which, h=1e-6):
    """Central differences of loss(*args) with respect to args[which], entry by entry."""
    x = args[which]
    fd = np.zeros_like(x)
    for j in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[j] += h
        xm[j] -= h
        fd[j] = (loss(*[xp if i == which else a for i, a in enumerate(args)]) -
                 loss(*[xm if i == which else a for i, a in enumerate(args)])) / (2 * h)
    return fd


def pin_hca_bwd_finite_differences():
    """Every gradient of hca_attention_bwd (q, the window path of k and v, and the compressed
    entries kc, vc as independent inputs) equals a central difference of the forward oracle's
    loss sum(do * o); a query/key width above the value width, rows with no visible entry, rows
    with a gap between entries and window, and an entry past every query's reach included."""
    rng = _rng(61)
    B, H, T, d, dv, blk, window = 1, 2, 11, 3, 2, 2, 3
    q, k = rng.standard_normal((B, H, T, d)), rng.standard_normal((B, H, T, d))
    v, do = rng.standard_normal((B, H, T, dv)), rng.standard_normal((B, H, T, dv))
    kc, vc = rng.standard_normal((B, H, T // blk, d)), rng.standard_normal((B, H, T // blk, dv))
    got = oracle.hca_attention_bwd(q, k, v, kc, vc, blk, window, do)

    def loss(q_, k_, v_, kc_, vc_):
        return float((oracle.hca_attention_prefill(q_, k_, v_, kc_, vc_, blk, window)[0] * do).sum())

    args = [q, k, v, kc, vc]
    for i, name in enumerate(("dq", "dk", "dv", "dkc", "dvc")):
        _close(got[i], _central_diff(loss, args, i), 1e-7, f"{name} vs central differences")
    # entry 4 (tokens 8, 9) is visible from t = 12 on: no query sees it
    assert np.all(got[3][:, :, 4] == 0) and np.all(got[4][:, :, 4] == 0), "unreached entry has a gradient"


def pin_hca_layer_bwd_finite_differences():
    """hca_layer_bwd's dk, dv (window path plus the block mean's 1/blk spread; the ragged tail gets
    the window path only) equal central differences of the whole layer, compression included."""
    rng = _rng(62)
    # (13, 3, 4): the last entry is out of every query's reach; (14, 3, 1): it is seen, next to a
    # two-token tail that must get the window path only.
    for T, blk, window in ((13, 3, 4), (14, 3, 1)):
        B, H, d = 1, 2, 3
        q, k, v, do = (rng.standard_normal((B, H, T, d)) for _ in range(4))
        dq, dk, dv, _, _ = oracle.hca_layer_bwd(q, k, v, blk, window, do)

        def loss(q_, k_, v_):
            o = oracle.hca_attention_prefill(q_, k_, v_, oracle.hca_compress(k_, blk), oracle.hca_compress(v_, blk),
                                             blk, window)[0]
            return float((o * do).sum())

        for i, (name, g) in enumerate((("dq", dq), ("dk", dk), ("dv", dv))):
            _close(g, _central_diff(loss, [q, k, v], i), 1e-7, f"T={T} window={window} layer {name} vs central differences")


def pin_hca_layer_bwd_blk1_is_dense_causal():
    """blk = 1 (any window): the layer is dense causal attention, so its gradients are those of
    torch's float64 SDPA; window >= T: no entry is visible (dkc = dvc = 0) and the same holds."""
    rng = _rng(63)
    B, H, T, d = 2, 2, 17, 5
    q, k, v, do = (rng.standard_normal((B, H, T, d)) for _ in range(4))
    want = _sdpa_causal_grads(q, k, v, do)
    for blk, window in ((1, 1), (1, 4), (1, 30), (4, T), (16, T + 5)):
        dq, dk, dv, dkc, dvc = oracle.hca_layer_bwd(q, k, v, blk, window, do)
        for name, g, w in (("dq", dq, want[0]), ("dk", dk, want[1]), ("dv", dv, want[2])):
            _close(g, w, 1e-12, f"blk={blk} window={window} {name}")
        if window >= T:
            assert not dkc.any() and not dvc.any(), "window >= T: no entry gradient"


def pin_hca_bwd_sum_identities():
    """The softmax derivative sums to 0 over a row's keys and the weights sum to 1: summed over
    keys (window tokens and entries), dk is 0 and dv is the sum of do over the rows."""
    rng = _rng(64)
    B, H, T, d, blk, window = 2, 3, 40, 4, 4, 6
    q, k, v, do = (rng.standard_normal((B, H, T, d)) for _ in range(4))
    kc, vc = oracle.hca_compress(k, blk), oracle.hca_compress(v, blk)
    dq, dk, dv, dkc, dvc = oracle.hca_attention_bwd(q, k, v, kc, vc, blk, window, do)
    _close(dk.sum(axis=2) + dkc.sum(axis=2), np.zeros((B, H, d)), 1e-12, "sum of dk")
    _close(dv.sum(axis=2) + dvc.sum(axis=2), do.sum(axis=2), 1e-12, "sum of dv")


def _sdpa_causal_dv(q, k, v):
    """torch CPU float64 SDPA with a value width different from the query/key width (scale 1/sqrt(qk width))."""
    return _sdpa_causal(q, k, v)


def pin_hca_wide_qk_dense():
    """qk wider than v (the 576/512 shape, scaled down): blk = 1 and window >= T reduce to dense causal
    attention, checked against torch's SDPA, which scales by 1/sqrt(query width) and allows Ev != E."""
    rng = _rng(44)
    B, H, T, dk, dv = 1, 2, 21, 12, 8
    q, k = rng.standard_normal((B, H, T, dk)), rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    want = _sdpa_causal_dv(q, k, v)
    assert want.shape == (B, H, T, dv)
    for blk, window in ((1, 1), (1, 5), (4, T), (8, T + 3)):
        o, _ = oracle.hca_attention_prefill(q, k, v, oracle.hca_compress(k, blk), oracle.hca_compress(v, blk), blk, window)
        _close(o, want, 1e-12, f"wide qk blk={blk} window={window}")


def pin_hca_wide_qk_decode_equals_prefill_row():
    """Decode with qk wider than v equals the prefill row at the same position."""
    rng = _rng(45)
    B, H, T, dk, dv, blk, window = 2, 2, 29, 10, 6, 4, 5
    q, k = rng.standard_normal((B, H, T, dk)), rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    kc, vc = oracle.hca_compress(k, blk), oracle.hca_compress(v, blk)
    for t in (0, 4, 9, 17, 28):
        o_pre, lse_pre = oracle.hca_attention_prefill(q, k, v, kc, vc, blk, window, rows=[t])
        ring_k, ring_v = np.zeros((B, H, window, dk)), np.zeros((B, H, window, dv))
        for s_ in range(max(0, t - window + 1), t + 1):
            ring_k[:, :, s_ % window] = k[:, :, s_]
            ring_v[:, :, s_ % window] = v[:, :, s_]
        o_dec, lse_dec = oracle.hca_attention_decode(q[:, :, t], kc, vc, ring_k, ring_v, [t] * B, blk, window)
        _close(o_dec, o_pre[:, :, 0], 1e-12, f"wide qk decode t={t}")
        _close(lse_dec, lse_pre[:, :, 0], 1e-12, f"wide qk decode lse t={t}")


# ---------------------------------------------------------------------------
# DSA indexer
# ---------------------------------------------------------------------------


def pin_indexer_single_head_is_matmul():
    """Hi = 1, w = 1, non-negative inputs: ReLU is inactive, scores = q @ k^T."""
    rng = _rng(11)
    T, S, Di = 9, 9, 5
    qi = np.abs(rng.standard_normal((1, T, 1, Di)))
    ki = np.abs(rng.standard_normal((1, S, Di)))
    sc = oracle.dsa_indexer_scores(qi, ki, np.ones((1, T, 1)))
    ref = qi[0, :, 0] @ ki[0].T
    for i in range(T):
        _close(sc[0, i, : i + 1], ref[i, : i + 1], 1e-12, f"matmul row {i}")
        assert np.all(np.isnan(sc[0, i, i + 1:])), "non-candidates are NaN"


def pin_indexer_integer_grid_exact():
    """Inputs on a quarter grid with signs: exact rational brute force (pure Python Fractions)."""
    rng = _rng(12)
    B, T, S, Hi, Di = 2, 5, 8, 3, 4
    qi = rng.integers(-3, 4, size=(B, T, Hi, Di)) / 4.0
    ki = rng.integers(-3, 4, size=(B, S, Di)) / 4.0
    w = rng.integers(0, 5, size=(B, T, Hi)) / 4.0
    q_pos = [2, 0]
    sc = oracle.dsa_indexer_scores(qi, ki, w, q_pos=q_pos)
    for b in range(B):
        for i in range(T):
            p = q_pos[b] + i
            for s in range(S):
                if s > p:
                    assert np.isnan(sc[b, i, s])
                    continue
                tot = Fraction(0)
                for h in range(Hi):
                    dot = sum(Fraction(qi[b, i, h, e]) * Fraction(ki[b, s, e]) for e in range(Di))
                    tot += Fraction(w[b, i, h]) * max(dot, Fraction(0))
                assert Fraction(sc[b, i, s]) == tot, f"b={b} i={i} s={s}"


# ---------------------------------------------------------------------------
# DSA top-k
# ---------------------------------------------------------------------------


def _brute_topk_row(row, n_cand, k):
    cands = sorted(range(n_cand), key=lambda s: (-(row[s] + 0.0), s))
    sel = sorted(cands[: min(k, n_cand)])
    return sel + [-1] * (k - len(sel))


def pin_topk_bruteforce():
    rng = _rng(13)
    B, T, S = 2, 12, 12
    for k in (1, 3, 5, 12, 20):
        sc = rng.integers(0, 4, size=(B, T, S)).astype(np.float64)  # heavy ties
        idx = oracle.dsa_topk(sc, k)
        for b in range(B):
            for i in range(T):
                assert list(idx[b, i]) == _brute_topk_row(sc[b, i], i + 1, k), f"k={k} b={b} i={i}"


def pin_topk_short_rows_keep_all():
    sc = _rng(14).standard_normal((1, 6, 6))
    idx = oracle.dsa_topk(sc, 8)
    for i in range(6):
        assert list(idx[0, i]) == list(range(i + 1)) + [-1] * (8 - i - 1)


def pin_topk_constant_scores_take_lowest():
    sc = np.full((1, 1, 50), 0.25)
    idx = oracle.dsa_topk(sc, 7, q_pos=[49])
    assert list(idx[0, 0]) == list(range(7))


def pin_topk_signed_zero_ties():
    row = np.array([-0.0, 0.0, -0.0, 0.5, 0.0, -1.0])
    idx = oracle.dsa_topk(row.reshape(1, 1, 6), 3, q_pos=[5])
    assert list(idx[0, 0]) == [0, 1, 3], list(idx[0, 0])


# ---------------------------------------------------------------------------
# DSA sparse attention
# ---------------------------------------------------------------------------


def pin_sparse_all_positions_is_dense_mqa():
    rng = _rng(15)
    B, T, Hq, D = 1, 17, 4, 8
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, T, D))
    v = rng.standard_normal((B, T, D))
    idx = np.full((B, T, T + 3), -1)
    for i in range(T):
        idx[0, i, : i + 1] = np.arange(i + 1)
    o, _ = oracle.dsa_sparse_attention(q, k, v, idx)
    qh = q.transpose(0, 2, 1, 3)
    kh = np.repeat(k[:, None], Hq, axis=1)
    vh = np.repeat(v[:, None], Hq, axis=1)
    ref = _sdpa_causal(qh, kh, vh).transpose(0, 2, 1, 3)
    _close(o, ref, 1e-12, "dense MQA")


def pin_sparse_single_position():
    rng = _rng(16)
    B, T, S, Hq, D = 1, 3, 10, 2, 4
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, S, D))
    v = rng.standard_normal((B, S, D))
    idx = np.array([[[7, -1, -1], [-1, 2, -1], [-1, -1, -1]]])
    o, lse = oracle.dsa_sparse_attention(q, k, v, idx)
    _close(o[0, 0], np.repeat(v[0, 7][None], Hq, 0), 1e-15, "single -> v[s]")
    _close(o[0, 1], np.repeat(v[0, 2][None], Hq, 0), 1e-15, "single -> v[s]")
    _close(lse[0, 0], q[0, 0] @ k[0, 7] / 2.0, 1e-14, "single lse = scaled logit")
    assert np.all(o[0, 2] == 0) and np.all(np.isneginf(lse[0, 2])), "empty row"


def pin_sparse_identity_support():
    rng = _rng(17)
    S, Hq = 12, 3
    q = rng.standard_normal((1, 1, Hq, S))
    k = rng.standard_normal((1, S, S))
    v = np.eye(S)[None]
    sel = [1, 4, 5, 9]
    idx = np.array([[sel + [-1]]])
    o, _ = oracle.dsa_sparse_attention(q, k, v, idx)
    for h in range(Hq):
        w = o[0, 0, h]
        assert abs(w.sum() - 1) < 1e-12
        assert set(np.nonzero(w)[0]) == set(sel)
        logits = np.array([q[0, 0, h] @ k[0, s] for s in sel]) / math.sqrt(S)
        p = np.exp(logits - logits.max())
        _close(w[sel], p / p.sum(), 1e-12, "identity-V weights")


def _sparse_bwd_case(seed, B, T, S, Hq, D, kk):
    rng = _rng(seed)
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, S, D))
    v = rng.standard_normal((B, S, D))
    do = rng.standard_normal((B, T, Hq, D))
    idx = np.stack([np.stack([rng.choice(S, kk, replace=False) for _ in range(T)]) for _ in range(B)])
    return q, k, v, do, idx


def pin_sparse_bwd_finite_differences():
    """Every gradient entry equals a central difference of the forward oracle's loss sum(do * o)
    (the forward is pinned on its own); padding, a repeated entry and an empty row included."""
    q, k, v, do, idx = _sparse_bwd_case(31, 1, 4, 9, 2, 3, 4)
    idx[0, 1, 2] = -1
    idx[0, 2, 3] = idx[0, 2, 0]  # one position listed twice
    idx[0, 3] = -1               # empty row
    dq, dk, dv = oracle.dsa_sparse_attention_bwd(q, k, v, idx, do)
    loss = lambda q_, k_, v_: float((oracle.dsa_sparse_attention(q_, k_, v_, idx)[0] * do).sum())
    h = 1e-6
    for name, x, g in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
        fd = np.zeros_like(x)
        for j in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[j] += h
            xm[j] -= h
            args_p = [xp if a is x else a for a in (q, k, v)]
            args_m = [xm if a is x else a for a in (q, k, v)]
            fd[j] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        _close(g, fd, 1e-7, f"{name} vs central differences")


def pin_sparse_bwd_sum_identities():
    """Softmax weights sum to 1 and their derivative rows sum to 0: summed over positions, dk is 0
    and dv is the sum of do over every (token, head) whose row has an entry."""
    q, k, v, do, idx = _sparse_bwd_case(32, 2, 5, 11, 3, 4, 5)
    idx[1, 2] = -1
    dq, dk, dv = oracle.dsa_sparse_attention_bwd(q, k, v, idx, do)
    live = (idx >= 0).any(axis=2)
    _close(dk.sum(axis=1), np.zeros((2, 4)), 1e-12, "sum of dk")
    _close(dv.sum(axis=1), (do * live[:, :, None, None]).sum(axis=(1, 2)), 1e-12, "sum of dv")
    assert np.all(dq[1, 2] == 0), "empty row has no dq"


def pin_sparse_bwd_single_entry():
    """One entry per row: its weight is 1 for any logits, so dq = 0, dk = 0 and dv[s] collects
    the row's do summed over heads."""
    q, k, v, do, idx = _sparse_bwd_case(33, 1, 3, 6, 2, 4, 1)
    idx[0, :, 0] = [4, 1, 4]
    dq, dk, dv = oracle.dsa_sparse_attention_bwd(q, k, v, idx, do)
    assert np.all(dq == 0) and np.all(dk == 0)
    ref = np.zeros((6, 4))
    for t, s in enumerate([4, 1, 4]):
        ref[s] += do[0, t].sum(axis=0)
    _close(dv[0], ref, 1e-14, "single-entry dv")


def pin_dsa_end_to_end_k_ge_context_is_dense():
    rng = _rng(18)
    T, Hi, Di, Hq, D = 14, 2, 4, 3, 8
    qi = rng.standard_normal((1, T, Hi, Di))
    ki = rng.standard_normal((1, T, Di))
    w = rng.random((1, T, Hi))
    q = rng.standard_normal((1, T, Hq, D))
    k = rng.standard_normal((1, T, D))
    v = rng.standard_normal((1, T, D))
    idx = oracle.dsa_topk(oracle.dsa_indexer_scores(qi, ki, w), T)
    o, _ = oracle.dsa_sparse_attention(q, k, v, idx)
    ref = _sdpa_causal(q.transpose(0, 2, 1, 3), np.repeat(k[:, None], Hq, 1), np.repeat(v[:, None], Hq, 1))
    _close(o, ref.transpose(0, 2, 1, 3), 1e-12, "k >= context")


# ---------------------------------------------------------------------------
# CSA variant: DSA over block-mean compressed entries
# ---------------------------------------------------------------------------
def pin_csa_bruteforce():
    """Tiny CSA layer written out from the reading with plain loops: block means of 4 tokens,
    entry j visible to token t iff its block ends at or before t (4j+3 <= t), scores, top-k by
    (score desc, entry asc), softmax over the selected entries."""
    rng = _rng(41)
    T, r, Hi, Di, Hq, D, kk = 23, 4, 2, 4, 3, 8, 3
    qi, ki, w = rng.standard_normal((1, T, Hi, Di)), rng.standard_normal((1, T, Di)), rng.random((1, T, Hi))
    q, k, v = rng.standard_normal((1, T, Hq, D)), rng.standard_normal((1, T, D)), rng.standard_normal((1, T, D))
    o, lse, idx = oracle.csa_attention(qi, ki, w, q, k, v, r, kk)
    nb = T // r
    mean = lambda x, j: sum(x[0, r * j + u] for u in range(r)) / r
    kci = [mean(ki, j) for j in range(nb)]
    kc = [mean(k, j) for j in range(nb)]
    vc = [mean(v, j) for j in range(nb)]
    for t in range(T):
        vis = [j for j in range(nb) if r * j + r - 1 <= t]
        sc = {j: sum(w[0, t, h] * max(0.0, float(qi[0, t, h] @ kci[j])) for h in range(Hi)) for j in vis}
        sel = sorted(sorted(vis, key=lambda j: (-sc[j], j))[:kk])
        assert list(idx[0, t][idx[0, t] >= 0]) == sel, (t, idx[0, t], sel)
        for h in range(Hq):
            if not sel:
                assert np.all(o[0, t, h] == 0) and lse[0, t, h] == -np.inf
                continue
            logits = np.array([q[0, t, h] @ kc[j] / math.sqrt(D) for j in sel])
            p_ = np.exp(logits - logits.max())
            want = sum(p_[n] * vc[j] for n, j in enumerate(sel)) / p_.sum()
            _close(o[0, t, h], want, 1e-12, "CSA output")
            _close(lse[0, t, h], logits.max() + math.log(p_.sum()), 1e-12, "CSA lse")


def pin_csa_ratio_one_is_dsa():
    """ratio 1: block means of one token are the tokens, and the visible set is s <= t."""
    rng = _rng(42)
    T, Hi, Di, Hq, D, kk = 19, 2, 4, 2, 8, 5
    qi, ki, w = rng.standard_normal((1, T, Hi, Di)), rng.standard_normal((1, T, Di)), rng.random((1, T, Hi))
    q, k, v = rng.standard_normal((1, T, Hq, D)), rng.standard_normal((1, T, D)), rng.standard_normal((1, T, D))
    o, lse, idx = oracle.csa_attention(qi, ki, w, q, k, v, 1, kk)
    idx_d = oracle.dsa_topk(oracle.dsa_indexer_scores(qi, ki, w), kk)
    assert np.array_equal(idx, idx_d)
    o_d, lse_d = oracle.dsa_sparse_attention(q, k, v, idx_d)
    _close(o, o_d, 1e-12, "ratio 1 output")


def pin_indexer_ratio_rows_are_single_query_calls():
    """Row t of the ratio-4 scores equals a one-query DSA call whose last position is its last visible entry."""
    rng = _rng(43)
    T, S, Hi, Di = 30, 7, 2, 4
    qi, ki, w = rng.standard_normal((1, T, Hi, Di)), rng.standard_normal((1, S, Di)), rng.random((1, T, Hi))
    sc = oracle.dsa_indexer_scores(qi, ki, w, ratio=4)
    for t in range(T):
        n = min((t + 1) // 4, S)
        assert np.all(np.isnan(sc[0, t, n:])), t
        if n == 0:
            continue
        one = oracle.dsa_indexer_scores(qi[:, t:t + 1], ki, w[:, t:t + 1], q_pos=[n - 1])
        _close(sc[0, t, :n], one[0, 0, :n], 0.0, f"row {t}")


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3 "fn") decode cache -- the library's own format reading
# ---------------------------------------------------------------------------
def _torch_e4m3_decode(codes):
    import torch

    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_e4m3_encode(x):
    import torch

    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_values_are_torch_float8():
    """Every code decodes as torch's float8_e4m3fn does (NaN for S.1111.111 only)."""
    codes = np.arange(256)
    got = oracle.e4m3_value(codes)
    ref = _torch_e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "NaN codes"
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]), "E4M3 values"
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok])), "signs"


def pin_e4m3_golden_codes():
    """Facts of the OCP E4M3 layout: bias 7, 3 mantissa bits, subnormals m*2^-9, max 448."""
    v = oracle.e4m3_value
    golden = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
              0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, want in golden.items():
        assert v(c) == want, (hex(c), v(c), want)
    assert np.signbit(v(0x80)) and v(0x80) == 0.0, "0x80 is -0.0"
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF)), "S.1111.111 is NaN"
    pos = v(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E increase"


def pin_e4m3_encode_round_trip_and_ties():
    """encode(value(c)) == c for every finite code; a midpoint goes to the even code."""
    codes = np.arange(256)
    vals = oracle.e4m3_value(codes)
    ok = ~np.isnan(vals)
    assert np.array_equal(oracle.e4m3_encode(vals[ok]), codes[ok].astype(np.uint8)), "round trip"
    # midpoints between neighbours 0x38|0x39 (1.0625) and 0x39|0x3A (1.1875), 0x00|0x01, 0x7D|0x7E
    for x, want in ((1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (432.0, 0x7E),
                    (-1.0625, 0xB8), (464.0, 0x7E)):
        assert oracle.e4m3_encode(np.array([x]))[0] == want, (x, hex(oracle.e4m3_encode(np.array([x]))[0]), hex(want))


def pin_e4m3_encode_is_torch_conversion():
    """Round to nearest even, as torch's float32/64 -> float8_e4m3fn conversion, over normal,
    subnormal and midpoint values."""
    rng = _rng(31)
    vals = oracle.e4m3_value(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([rng.uniform(-448, 448, 5000), rng.uniform(-0.03, 0.03, 5000), mids, -mids,
                        rng.standard_normal(2000) * 10])
    x = x[np.abs(x) <= 448]
    assert np.array_equal(oracle.e4m3_encode(x), _torch_e4m3_encode(x)), "E4M3 rounding"


def pin_quantize_rows_invariants():
    """Per-row scaling: the row's largest magnitude maps to +-448, the scale is amax/448 in fp32,
    every value is within half a step of its code, zero rows give zero codes and scale."""
    rng = _rng(32)
    x = (rng.standard_normal((6, 512)) * np.array([1.0, 1e-3, 50.0, 1e-6, 3.0, 0.2])[:, None]).astype(np.float32)
    x[1, :] = 0.0
    x[1, 7] = -2.5  # a single nonzero value
    x[4, :] = 0.75  # constant row
    x = np.concatenate([x, np.zeros((1, 512), np.float32)])
    codes, scales = oracle.quantize_fp8_rows(x)
    assert scales.dtype == np.float32 and codes.dtype == np.uint8
    amax = np.max(np.abs(x), axis=-1)
    assert np.array_equal(scales, (amax / np.float32(448)).astype(np.float32)), "scale = amax/448"
    for r in range(x.shape[0]):
        if amax[r] == 0:
            assert np.all(codes[r] == 0) and scales[r] == 0, "zero row"
            continue
        j = int(np.argmax(np.abs(x[r])))
        assert codes[r, j] in (0x7E, 0xFE), ("row max maps to 448", r, hex(codes[r, j]))
        inv = np.float64(np.float32(448) / amax[r])
        scaled = x[r].astype(np.float64) * inv
        err = np.abs(oracle.e4m3_value(codes[r]) - scaled)
        step = np.where(np.abs(scaled) >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(np.abs(scaled), 2.0 ** -6))) - 3),
                        2.0 ** -9)
        assert np.all(err <= step / 2 + 1e-9 * np.abs(scaled)), ("half a step", r)
    assert np.all(codes[4] == 0x7E), "constant row"
    deq = oracle.dequantize_fp8_rows(codes, scales)
    assert np.all(np.abs(deq - x) <= np.abs(x) * 2.0 ** -4 + scales[:, None] * 2.0 ** -9 + 1e-30), "dequantized rows"


ALL_PINS = {name: fn for name, fn in globals().items() if name.startswith("pin_") and callable(fn)}

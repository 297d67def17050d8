"""Backward of the DSA sparse attention (dsa_sparse_attention_bwd) against the float64 oracle.

The GPU works from the forward's bf16 output o and fp32 log-sum-exp; the oracle rebuilds everything in
float64 from the same bf16 inputs.  Tolerance: an element-wise bound derived from the roundings the
kernels make, computed in float64 beside the reference (per token, from the exact weights P, their
derivative dS = P (dP - D) and D = sum P dP):
  * D_h comes from the forward's bf16 output o: dS is off by P |dD_h|, dD_h = do_h . (o_gpu - o_exact)
    computed exactly here;
  * P and dS are rounded to bf16 (relative 2^-9) for the dq, dk, dv products (2^-8 covers it with room);
  * P is rebuilt from fp32 scores and the forward's fp32 log-sum-exp (relative 1e-5 covers it);
  * each entry's dk and dv rows are rounded to bf16 (relative 2^-9) before the per-position sums.
So with e_hj = P |dD_h| + 2^-8 |dS| + 1e-5 P (|dP| + |D|): |error of dq_h| <= scale sum_j e_hj |k_j|,
|error of dk[s]| <= sum over the entries at s of (scale sum_h e_hj |q_h| + 2^-9 |dk row|), and
|error of dv[s]| <= sum over the entries at s of ((2^-8 + 1e-5) sum_h P_hj |do_h| + 2^-9 |dv row|).
Checked with a margin of 2 and an absolute floor of 1e-6 of the reference's largest magnitude.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, f64, require_gpu

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


def _inputs(B, T, S, seed, sigma=1.0):
    q = synth.np_normal((B, T, 64, 256), sigma, "bf16", seed, 0)
    k = synth.np_normal((B, S, 256), sigma, "bf16", seed, 1)
    v = synth.np_normal((B, S, 256), sigma, "bf16", seed, 2)
    do = synth.np_normal((B, T, 64, 256), 1.0, "bf16", seed, 3)
    return q, k, v, do


def _causal_idx(B, T, S, kk, g):
    """Row i (position S - T + i) keeps min(pos + 1, kk) distinct positions <= pos, ascending, -1 padded."""
    idx = np.full((B, T, kk), -1, dtype=np.int64)
    for b in range(B):
        for i in range(T):
            pos = S - T + i
            n = min(pos + 1, kk)
            idx[b, i, :n] = np.sort(g.choice(pos + 1, n, replace=False))
    return idx


def _token_terms(q_i, k_b, v_b, o_i, do_i, sel, scale):
    """Float64 terms of one token: (dq_i, per-entry dk rows, dv rows) and their error bounds."""
    K, V = k_b[sel], v_b[sel]
    lg = scale * (q_i @ K.T)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = do_i @ V.T
    D = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - D)
    dD = np.abs((do_i * (o_i - p @ V)).sum(axis=1, keepdims=True))
    e = p * dD + U * np.abs(ds) + 1e-5 * p * (np.abs(dp) + np.abs(D))
    ck, cv = scale * (ds.T @ q_i), p.T @ do_i
    eq = scale * (e @ np.abs(K))
    ek = scale * (e.T @ np.abs(q_i)) + 2.0 ** -9 * np.abs(ck)
    ev = (U + 1e-5) * (p.T @ np.abs(do_i)) + 2.0 ** -9 * np.abs(cv)
    return scale * (ds @ K), ck, cv, eq, ek, ev


def _bounds(q, k, v, o_gpu, do, idx, scale=None):
    """Element-wise error bounds (dq, dk, dv) for the whole call (float64)."""
    q, k, v, o_gpu, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, o_gpu, do))
    B, T, Hq, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    eq, ek, ev = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(B):
        for i in range(T):
            sel = idx[b, i][(idx[b, i] >= 0) & (idx[b, i] < k.shape[1])]
            if sel.size == 0:
                continue
            _, _, _, eq[b, i], eki, evi = _token_terms(q[b, i], k[b], v[b], o_gpu[b, i], do[b, i], sel, scale)
            np.add.at(ek[b], sel, eki)
            np.add.at(ev[b], sel, evi)
    return eq, ek, ev


def _check(name, got, ref, bound):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    floor = 1e-6 * max(float(np.abs(ref).max()), 1e-30)
    worst = float(np.max(err / (2 * bound + floor)))
    print(f"  {name}: max abs err {err.max():.3e}, max |ref| {np.abs(ref).max():.3e}, "
          f"worst err / (2 bound + floor) {worst:.3f}", flush=True)
    assert worst <= 1.0, f"{name}: error above the derived bound ({worst:.3f})"


def _gpu(sa, q, k, v, do, idx):
    t = lambda a: synth.to_torch(a, "bf16", DEV)
    ti = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    tq, tk, tv = t(q), t(k), t(v)
    o, lse = sa.dsa_sparse_attention_fwd(tq, tk, tv, ti, return_lse=True)
    dq, dk, dv = sa.dsa_sparse_attention_bwd(tq, tk, tv, ti, o, lse, t(do))
    torch.cuda.synchronize()
    return f64(dq), f64(dk), f64(dv), f64(o)


def _compare_all(sa, q, k, v, do, idx):
    dq, dk, dv, o = _gpu(sa, q, k, v, do, idx)
    S = k.shape[1]
    clean = np.where((idx >= 0) & (idx < S), idx, -1)
    rq, rk, rv = oracle.dsa_sparse_attention_bwd(q, k, v, clean, do)
    eq, ek, ev = _bounds(q, k, v, o, do, clean)
    _check("dq", dq, rq, eq)
    _check("dk", dk, rk, ek)
    _check("dv", dv, rv, ev)
    return dq


@pytest.mark.parametrize("B,T,S,kk", [(1, 40, 100, 48), (2, 9, 300, 21), (1, 20, 2100, 2048), (1, 33, 33, 16),
                                      (2, 1500, 1600, 64)])
def test_sparse_bwd_matches_oracle(B, T, S, kk):
    """Element-wise against the oracle; (2, 1500, 1600, 64) has 3000 tokens, so two chunks of the
    per-position sums (2048 tokens each) and a batch boundary inside the first chunk."""
    sa = require_gpu()
    print(f"[dsa_bwd] B={B} T={T} S={S} kk={kk}", flush=True)
    q, k, v, do = _inputs(B, T, S, 60 + kk)
    idx = _causal_idx(B, T, S, kk, np.random.default_rng(61 + kk))
    _compare_all(sa, q, k, v, do, idx)


def test_sparse_bwd_padding_duplicates_and_empty_rows():
    """Out-of-range entries are skipped, a repeated entry counts twice, an empty row gives dq = 0."""
    sa = require_gpu()
    B, T, S, kk = 1, 5, 120, 37
    q, k, v, do = _inputs(B, T, S, 62)
    idx = np.full((B, T, kk), -1, dtype=np.int64)
    idx[0, 0, :6] = [3, 150, 7, -9, 99, 7]  # 150 and -9 out of range; 7 twice
    idx[0, 1, 10:12] = [42, 43]
    idx[0, 3, :] = np.arange(kk)
    idx[0, 4, :] = np.arange(kk) + 80
    dq = _compare_all(sa, q, k, v, do, idx)
    assert np.all(dq[0, 2] == 0)


def test_sparse_bwd_long_segment_of_one_position():
    """One position listed 8192 times within a chunk (every entry of 64 tokens is position 5, most of
    another position 9): more entries than the per-position sort holds, so the ordered scan adds them."""
    sa = require_gpu()
    B, T, S, kk = 1, 64, 40, 128
    q, k, v, do = _inputs(B, T, S, 65)
    idx = np.full((B, T, kk), 5, dtype=np.int64)
    idx[0, 10:20, 1::2] = 9
    idx[0, 30, -3:] = -1
    _compare_all(sa, q, k, v, do, idx)


def test_sparse_bwd_bit_reproducible():
    """Entries are added per position in ascending (token, entry) order: two runs give identical bits."""
    sa = require_gpu()
    B, T, S, kk = 2, 2500, 2600, 256
    q, k, v, do = _inputs(B, T, S, 66)
    idx = _causal_idx(B, T, S, kk, np.random.default_rng(67))
    t = lambda a: synth.to_torch(a, "bf16", DEV)
    ti = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    tq, tk, tv, tdo = t(q), t(k), t(v), t(do)
    o, lse = sa.dsa_sparse_attention_fwd(tq, tk, tv, ti, return_lse=True)
    a = sa.dsa_sparse_attention_bwd(tq, tk, tv, ti, o, lse, tdo)
    b = sa.dsa_sparse_attention_bwd(tq, tk, tv, ti, o, lse, tdo)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_sparse_bwd_user_stream_and_graph():
    """The call forks its inverse index to a second stream and joins it back with events.  On a
    non-default stream, with the index list written by the work just before the call on that stream,
    and captured in a graph (replayed three times with eager work between), it gives the bits of the
    plain call."""
    sa = require_gpu()
    B, T, S, kk = 1, 3000, 3100, 128
    q, k, v, do = _inputs(B, T, S, 71)
    idx = _causal_idx(B, T, S, kk, np.random.default_rng(72))
    t = lambda a: synth.to_torch(a, "bf16", DEV)
    ti = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    tq, tk, tv, tdo = t(q), t(k), t(v), t(do)
    o, lse = sa.dsa_sparse_attention_fwd(tq, tk, tv, ti, return_lse=True)
    ref = sa.dsa_sparse_attention_bwd(tq, tk, tv, ti, o, lse, tdo)
    torch.cuda.synchronize()
    ws = torch.empty(sa.dsa_sparse_attention_bwd_workspace_size(B, T, S, kk), dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ti2 = torch.full_like(ti, -1)
        ti2.copy_(ti)  # written on s just before the call: the index must see it
        got = sa.dsa_sparse_attention_bwd(tq, tk, tv, ti2, o, lse, tdo, workspace=ws)
    torch.cuda.synchronize()
    for x, y in zip(got, ref):
        assert torch.equal(x, y)
    # Graph capture (the forked stream joins the capture through the events).
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        sa.dsa_sparse_attention_bwd(tq, tk, tv, ti, o, lse, tdo, workspace=ws)  # warm-up outside the graph
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        cap = sa.dsa_sparse_attention_bwd(tq, tk, tv, ti, o, lse, tdo, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in cap:
            x.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(cap, ref):
            assert torch.equal(x, y), rep
        eager = sa.dsa_sparse_attention_bwd(tq, tk, tv, ti, o, lse, tdo)  # eager work between replays
        torch.cuda.synchronize()
        for x, y in zip(eager, ref):
            assert torch.equal(x, y), rep


def _sampled_check(q, k, v, o, do, idx, dq, dk, dv, rows, positions, scale):
    """dq of sampled rows, and dk, dv at sampled positions from every token that lists them."""
    B = q.shape[0]
    kn, vn = f64(k), f64(v)
    idx_np = idx.cpu().numpy().astype(np.int64)
    for i in rows:
        qi, oi, doi = f64(q[0, i]), f64(o[0, i]), f64(do[0, i])
        sel = idx_np[0, i][idx_np[0, i] >= 0]
        rq, _, _, eq, _, _ = _token_terms(qi, kn[0], vn[0], oi, doi, sel, scale)
        _check(f"dq row {i}", f64(dq[0, i]), rq, eq)
    for s in positions:
        toks = np.nonzero((idx_np[0] == s).any(axis=1))[0]
        rk, rv, ek, ev = (np.zeros(256) for _ in range(4))
        for i in toks:
            sel = idx_np[0, i][idx_np[0, i] >= 0]
            _, ck, cv, _, eki, evi = _token_terms(f64(q[0, i]), kn[0], vn[0], f64(o[0, i]), f64(do[0, i]), sel, scale)
            m = sel == s
            rk += ck[m].sum(axis=0)
            rv += cv[m].sum(axis=0)
            ek += eki[m].sum(axis=0)
            ev += evi[m].sum(axis=0)
        print(f"  position {s}: listed by {toks.size} tokens", flush=True)
        _check(f"dk[{s}]", f64(dk[0, s]), rk, ek)
        _check(f"dv[{s}]", f64(dv[0, s]), rv, ev)


@pytest.mark.parametrize("sigma", [1.0, 1.0 / 16])
def test_sparse_bwd_32768_top2048(sigma):
    """The bench's configuration: T = S = 32768, top-2048 chosen by the indexer and top-k, inputs at unit
    variance and at the workload's N(0,1)/16, do N(0,1).  dq of sampled rows and dk, dv at sampled
    positions (every token that lists them, found from the index) against the oracle within the derived
    bound, and the sum identities over every position."""
    sa = require_gpu()
    T, kk = 32768, 2048
    qi = synth.torch_normal((1, T, 4, 128), 128 ** -0.5, torch.bfloat16, 401, DEV)
    ki = synth.torch_normal((1, T, 128), 128 ** -0.5, torch.bfloat16, 402, DEV)
    wi = synth.torch_uniform((1, T, 4), 403, DEV)
    idx = sa.dsa_indexer_topk(qi, ki, wi, kk)
    del qi, ki, wi
    q = synth.torch_normal((1, T, 64, 256), sigma, torch.bfloat16, 404, DEV)
    k = synth.torch_normal((1, T, 256), sigma, torch.bfloat16, 405, DEV)
    v = synth.torch_normal((1, T, 256), sigma, torch.bfloat16, 406, DEV)
    do = synth.torch_normal((1, T, 64, 256), 1.0, torch.bfloat16, 407, DEV)
    o, lse = sa.dsa_sparse_attention_fwd(q, k, v, idx, return_lse=True)
    dq, dk, dv = sa.dsa_sparse_attention_bwd(q, k, v, idx, o, lse, do)
    torch.cuda.synchronize()
    dk64, dv64 = dk.double(), dv.double()
    err_k = float((dk64.sum(dim=1).abs() / dk64.abs().sum(dim=1)).max())
    err_v = float(((dv64.sum(dim=1) - do.double().sum(dim=(1, 2))).abs() / dv64.abs().sum(dim=1)).max())
    print(f"sigma {sigma}: |sum dk| / mass {err_k:.3e}; |sum dv - sum do| / mass {err_v:.3e}", flush=True)
    assert err_k <= 1e-2 and err_v <= 1e-3  # every row has at least one entry
    rows = [0, 1, 2047, 2048, 16384, 32767]
    positions = [32500, 32000, 31000, 28000]
    _sampled_check(q, k, v, o, do, idx, dq, dk, dv, rows, positions, 1.0 / 16)

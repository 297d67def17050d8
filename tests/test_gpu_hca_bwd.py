"""GPU parity: HCA prefill backward (HIP library through the C ABI) vs the float64 oracle.

The GPU gets bf16 q, k, v, dO, its own bf16 compressed cache (hca_compress) and its own forward output o and
log-sum-exp; the oracle's hca_attention_bwd gets the same bf16 values (k_c, v_c as independent inputs).

Tolerance: an element-wise bound derived from the roundings the kernels make, computed in float64 beside
the reference (a per-row walk of the definition with absolute values).  With P, dS the exact weights and
their derivative for the GPU's own inputs:
  * D_t comes from the forward's bf16 output o (not the exact one): dS is off by P * |dD_t| with
    dD_t = dO_t . (o_gpu - o_exact) computed exactly here;
  * P and dS are rounded to bf16 (relative 2^-9) before the dq, dk, dv products: 2^-8 covers it with room;
  * P is rebuilt from fp32 scores and the forward's fp32 log-sum-exp: relative 1e-5 covers it.
So the error of dq[t] is at most scale * sum_j e_tj |key_j| with e_tj = P |dD_t| + 2^-8 |dS| +
1e-5 P (|dP| + |D_t|), of dk (window or entry) scale * sum_t e_tj |q_t|, of dv 2^-8-and-1e-5 weighted
sum_t P |dO_t|, and through the compression the entry bound spread by 1/blk.  Checked with a margin of 2 and
an absolute floor of 1e-6 of the reference's largest magnitude (fp32 summation).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, f64, require_gpu

pytestmark = pytest.mark.gpu


def _bounds(q, k, v, kc, vc, o_gpu, do, blk, window, scale=None, rows=None):
    """Element-wise error bounds (dq, dk_window, dv_window, dkc, dvc) for one batch's heads, float64, summed
    over the given query rows (default all)."""
    q, k, v, kc, vc, o_gpu, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, kc, vc, o_gpu, do))
    H, T, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    rows = list(range(T)) if rows is None else [int(t) for t in rows]
    o_rows, _ = oracle.hca_attention_prefill(q[None], k[None], v[None], kc[None], vc[None], blk, window, scale, rows)
    o_ex = np.zeros(o_gpu.shape)
    o_ex[:, rows] = o_rows[0]
    u = 2.0 ** -8
    eq, ek, ev = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    ekc, evc = np.zeros(kc.shape), np.zeros(vc.shape)
    for t in rows:
        cj, rs = oracle.hca_key_set(t, blk, window, n_entries=kc.shape[1])
        nc = cj.size
        keys = np.concatenate([kc[:, cj], k[:, rs]], axis=1)
        vals = np.concatenate([vc[:, cj], v[:, rs]], axis=1)
        lg = scale * np.einsum("hd,hnd->hn", q[:, t], keys)
        p = np.exp(lg - lg.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dp = np.einsum("hd,hnd->hn", do[:, t], vals)
        D = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - D)
        dD = np.abs((do[:, t] * (o_gpu[:, t] - o_ex[:, t])).sum(axis=1, keepdims=True))
        e = p * dD + u * np.abs(ds) + 1e-5 * p * (np.abs(dp) + np.abs(D))
        ep = u * p + 1e-5 * p
        eq[:, t] = scale * np.einsum("hn,hnd->hd", e, np.abs(keys))
        ekey = scale * e[:, :, None] * np.abs(q[:, t])[:, None, :]
        eval_ = ep[:, :, None] * np.abs(do[:, t])[:, None, :]
        ekc[:, cj] += ekey[:, :nc]
        evc[:, cj] += eval_[:, :nc]
        ek[:, rs] += ekey[:, nc:]
        ev[:, rs] += eval_[:, nc:]
    return eq, ek, ev, ekc, evc


def _check(name, got, ref, bound):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    floor = 1e-6 * max(float(np.abs(ref).max()), 1e-30)
    worst = float(np.max(err / (2 * bound + floor)))
    print(f"  {name}: max abs err {err.max():.3e}, max |ref| {np.abs(ref).max():.3e}, "
          f"worst err / (2 bound + floor) {worst:.3f}", flush=True)
    assert worst <= 1.0, f"{name}: error above the derived bound ({worst:.3f})"


def _run(sa, B, H, T, blk, window, seed, through, sigma=1.0):
    qn, kn, vn, don = (synth.np_normal((B, H, T, 512), sigma, "bf16", seed, i) for i in range(4))
    tq, tk, tv, tdo = (synth.to_torch(a, "bf16", DEV) for a in (qn, kn, vn, don))
    kc, vc = sa.hca_compress(tk, blk), sa.hca_compress(tv, blk)
    o, lse = sa.hca_attention_fwd(sa.HCA_PREFILL, tq, tk, tv, kc, vc, blk, window, return_lse=True)
    grads = sa.hca_attention_bwd(tq, tk, tv, kc, vc, o, lse, tdo, blk, window, through_compress=through)
    torch.cuda.synchronize()
    return (qn, kn, vn, don), (f64(kc), f64(vc), f64(o)), [f64(g) for g in grads]


@pytest.mark.parametrize("B,H,T,blk,window,through", [
    (1, 2, 300, 128, 128, True),   # ragged T, one entry seen by the last rows
    (1, 2, 300, 128, 128, False),
    (2, 1, 700, 64, 100, True),    # window not a multiple of 32, two sequences
    (1, 1, 200, 1, 16, True),      # blk = 1: every past token also an entry
    (1, 2, 150, 128, 256, True),   # window >= T: no entry visible
    (1, 1, 260, 32, 1, True),      # window 1: self only, entries up to t - 1
    (1, 3, 1100, 128, 128, True),  # several chunks of query tiles per entry tile pair
])
def test_hca_bwd_small(B, H, T, blk, window, through):
    sa = require_gpu()
    print(f"[hca_bwd] B={B} H={H} T={T} blk={blk} window={window} through={through}", flush=True)
    (q, k, v, do), (kc, vc, o), (dq, dk, dv, dkc, dvc) = _run(sa, B, H, T, blk, window, 8100 + T + blk, through)
    for b in range(B):
        r = oracle.hca_attention_bwd(q[b:b + 1], k[b:b + 1], v[b:b + 1], kc[b:b + 1], vc[b:b + 1], blk, window, do[b:b + 1])
        r = [x[0] for x in r]
        e = _bounds(q[b], k[b], v[b], kc[b], vc[b], o[b], do[b], blk, window)
        if through:
            r[1] = r[1] + oracle.hca_compress_bwd(r[3], blk, T)
            r[2] = r[2] + oracle.hca_compress_bwd(r[4], blk, T)
            e = list(e)
            e[1] = e[1] + oracle.hca_compress_bwd(e[3], blk, T)
            e[2] = e[2] + oracle.hca_compress_bwd(e[4], blk, T)
        for name, got, ref, bound in zip(("dq", "dk", "dv", "dkc", "dvc"), (dq[b], dk[b], dv[b], dkc[b], dvc[b]), r, e):
            if ref.size:
                _check(name, got, ref, bound)
        if window >= T:
            assert not dkc[b].any() and not dvc[b].any()


def test_hca_bwd_bit_reproducible():
    """Fixed-order sums and no atomics: two runs give identical bits."""
    sa = require_gpu()
    B, H, T, blk, window = 1, 4, 2500, 128, 128
    qn, kn, vn, don = (synth.np_normal((B, H, T, 512), 1.0, "bf16", 8200, i) for i in range(4))
    tq, tk, tv, tdo = (synth.to_torch(a, "bf16", DEV) for a in (qn, kn, vn, don))
    kc, vc = sa.hca_compress(tk, blk), sa.hca_compress(tv, blk)
    o, lse = sa.hca_attention_fwd(sa.HCA_PREFILL, tq, tk, tv, kc, vc, blk, window, return_lse=True)
    a = sa.hca_attention_bwd(tq, tk, tv, kc, vc, o, lse, tdo, blk, window)
    b = sa.hca_attention_bwd(tq, tk, tv, kc, vc, o, lse, tdo, blk, window)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("sigma", [1.0, 512 ** -0.5])
def test_hca_bwd_full_config(sigma):
    """T = 32768, 64 heads, d = 512, block 128, window 128 (the prefill workload), at unit variance and at
    the workload's own N(0,1)/sqrt(512): sampled outputs of two heads against the oracle within the derived
    bound, and every head and dim against the sum identities (relative to the summed magnitudes)."""
    sa = require_gpu()
    B, H, T, blk, window = 1, 64, 32768, 128, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(8300)
    tq, tk, tv, tdo = ((torch.randn((B, H, T, 512), generator=g, device=DEV) * sigma).to(torch.bfloat16)
                       for _ in range(4))
    kc, vc = sa.hca_compress(tk, blk), sa.hca_compress(tv, blk)
    o, lse = sa.hca_attention_fwd(sa.HCA_PREFILL, tq, tk, tv, kc, vc, blk, window, return_lse=True)
    dq, dk, dv, dkc, dvc = sa.hca_attention_bwd(tq, tk, tv, kc, vc, o, lse, tdo, blk, window, through_compress=False)
    torch.cuda.synchronize()
    # Sum identities over every head and dim (window tokens and entries together): sum dk = 0 and
    # sum dv = sum do, each relative to the summed magnitudes of the terms.
    mk = dk.double().abs().sum(dim=2) + dkc.double().abs().sum(dim=2)
    mv = dv.double().abs().sum(dim=2) + dvc.double().abs().sum(dim=2)
    sk = ((dk.double().sum(dim=2) + dkc.double().sum(dim=2)).abs() / mk).max().item()
    sv = ((dv.double().sum(dim=2) + dvc.double().sum(dim=2) - tdo.double().sum(dim=2)).abs() / mv).max().item()
    print(f"[hca_bwd full] sigma={sigma:.4f}: |sum dk| / mass {sk:.3e}, |sum dv - sum do| / mass {sv:.3e}", flush=True)
    assert sk <= 1e-2 and sv <= 1e-3
    # Sampled outputs of two heads, each against the oracle summed over exactly the rows that reach it:
    # dq on spread rows (first tokens, block and window edges, the last token); dk, dv (window path) at
    # sampled positions from the rows s .. s+127 that see them; dkc, dvc of late entries (t >= 128 j + 255).
    rng = np.random.default_rng(8301)
    q_rows = sorted(set([0, 1, 127, 128, 254, 255, 256, 383, 4095, 16384, T - 2, T - 1] +
                        rng.integers(0, T, 36).tolist()))
    s_pos = sorted(set([0, 1, 130, 255, 12345, T - 1] + rng.integers(0, T, 6).tolist()))
    entries = [247, 250, 253, 254]
    t_first = (entries[0] + 1) * blk + window - 1
    for h in (5, 61):
        print(f"[hca_bwd full] head {h}", flush=True)
        qh, kh, vh, doh = (f64(x[0, h]) for x in (tq, tk, tv, tdo))
        kch, vch, oh = f64(kc[0, h]), f64(vc[0, h]), f64(o[0, h])
        args = (qh[None, None], kh[None, None], vh[None, None], kch[None, None], vch[None, None], blk, window,
                doh[None, None])
        bargs = (qh[None], kh[None], vh[None], kch[None], vch[None], oh[None], doh[None], blk, window)
        r = oracle.hca_attention_bwd(*args, rows=q_rows)
        e = _bounds(*bargs, rows=q_rows)
        _check("dq rows", f64(dq[0, h, q_rows]), r[0][0, 0, q_rows], e[0][0, q_rows])
        for s in s_pos:
            rows = list(range(s, min(T, s + window)))
            r = oracle.hca_attention_bwd(*args, rows=rows)
            e = _bounds(*bargs, rows=rows)
            _check(f"dk[{s}]", f64(dk[0, h, s]), r[1][0, 0, s], e[1][0, s])
            _check(f"dv[{s}]", f64(dv[0, h, s]), r[2][0, 0, s], e[2][0, s])
        rows = list(range(t_first, T))
        r = oracle.hca_attention_bwd(*args, rows=rows)
        e = _bounds(*bargs, rows=rows)
        _check("dkc late entries", f64(dkc[0, h, entries]), r[3][0, 0, entries], e[3][0, entries])
        _check("dvc late entries", f64(dvc[0, h, entries]), r[4][0, 0, entries], e[4][0, entries])

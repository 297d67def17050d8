"""Backward of the DSA sparse attention (dsa_sparse_attention_bwd) against the float64 oracle.

The kernel works from the forward's bf16 output o and fp32 log-sum-exp and accumulates in fp32;
the oracle rebuilds everything in float64 from the same bf16 inputs.  Tolerances, as a fraction
of the output's largest magnitude, 1e-2 for each gradient:
  * dq and dk go through dS = P (dP - D_h) with D_h = sum_d do*o taken from the forward's o, which
    carries bf16 rounding (of P in the PV product and of o itself, each relative 2^-9 = 2e-3); the
    error of D_h is of that order relative to dP and passes to dS, dq and dk;
  * the kernel rounds dS and P to bf16 (relative 2^-9) for the dq, dk and dv sums, as the forward
    rounds P for its PV product; summed over many terms of either sign these errors stay of that
    order (measured: dq, dk up to 2.2e-3 before this rounding; dv about 1e-6 without it).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, f64, max_abs_err, require_gpu

pytestmark = pytest.mark.gpu

REL_TOL = {"dq": 1e-2, "dk": 1e-2, "dv": 1e-2}


def _inputs(B, T, S, seed):
    q = synth.np_normal((B, T, 64, 256), 1.0, "bf16", seed, 0)
    k = synth.np_normal((B, S, 256), 1.0, "bf16", seed, 1)
    v = synth.np_normal((B, S, 256), 1.0, "bf16", seed, 2)
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


def _gpu(sa, q, k, v, do, idx):
    t = lambda a: synth.to_torch(a, "bf16", DEV)
    ti = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    tq, tk, tv = t(q), t(k), t(v)
    o, lse = sa.dsa_sparse_attention_fwd(tq, tk, tv, ti, return_lse=True)
    return sa.dsa_sparse_attention_bwd(tq, tk, tv, ti, o, lse, t(do))


def _check(got, ref, what):
    err = max_abs_err(f64(got), ref)
    scale = float(np.abs(ref).max())
    print(f"{what}: max abs err {err:.3e}, max |ref| {scale:.3e}", flush=True)
    assert err <= REL_TOL[what.split()[0]] * scale, what


@pytest.mark.parametrize("B,T,S,kk", [(1, 40, 100, 48), (2, 9, 300, 21), (1, 20, 2100, 2048), (1, 33, 33, 16)])
def test_sparse_bwd_matches_oracle(B, T, S, kk):
    sa = require_gpu()
    q, k, v, do = _inputs(B, T, S, 60 + kk)
    idx = _causal_idx(B, T, S, kk, np.random.default_rng(61 + kk))
    dq, dk, dv = _gpu(sa, q, k, v, do, idx)
    rq, rk, rv = oracle.dsa_sparse_attention_bwd(q, k, v, idx, do)
    _check(dq, rq, "dq")
    _check(dk, rk, "dk")
    _check(dv, rv, "dv")


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
    dq, dk, dv = _gpu(sa, q, k, v, do, idx)
    clean = np.where((idx >= 0) & (idx < S), idx, -1)
    rq, rk, rv = oracle.dsa_sparse_attention_bwd(q, k, v, clean, do)
    _check(dq, rq, "dq")
    _check(dk, rk, "dk")
    _check(dv, rv, "dv")
    assert torch.all(dq[0, 2] == 0)


def test_sparse_bwd_4096_sums_and_sampled_rows():
    """T = S = 4096, k = 2048: the sum identities of the gradients (sum of dk = 0, sum of dv = sum
    of do over the rows with an entry) and dq of sampled rows against the oracle row by row."""
    sa = require_gpu()
    B, T, S, kk = 1, 4096, 4096, 2048
    g = np.random.default_rng(63)
    q, k, v, do = _inputs(B, T, S, 64)
    idx = _causal_idx(B, T, S, kk, g)
    dq, dk, dv = _gpu(sa, q, k, v, do, idx)
    dk64, dv64 = f64(dk), f64(dv)
    _check_sum = lambda got, want, mag, what: (print(f"{what}: {np.abs(got - want).max():.3e} vs {mag:.3e}"),
                                              np.abs(got - want).max() <= REL_TOL[what.split()[1]] * mag)
    # sum of dk: each row's dS sums to D_h-error terms only, so its sum is small against sum |dk|
    assert _check_sum(dk64.sum(axis=1), 0.0, np.abs(dk64).sum(axis=1).max(), "sum dk")[1]
    want_v = do.astype(np.float64).sum(axis=(1, 2))
    assert _check_sum(dv64.sum(axis=1), want_v, np.abs(dv64).sum(axis=1).max(), "sum dv")[1]
    rows = [0, 1, 2047, 2048, 3000, 4095]  # row 0 has one entry: its dq is exactly 0
    refs = [oracle.dsa_sparse_attention_bwd(q[:, i:i + 1], k, v, idx[:, i:i + 1], do[:, i:i + 1])[0] for i in rows]
    mag = max(float(np.abs(r).max()) for r in refs)
    for i, rq in zip(rows, refs):
        err = max_abs_err(f64(dq[:, i:i + 1]), rq)
        print(f"dq row {i}: max abs err {err:.3e} (largest sampled |dq| {mag:.3e})", flush=True)
        assert err <= REL_TOL["dq"] * mag, i


def test_sparse_bwd_32768_top2048_sums_and_sampled_rows():
    """The bench's configuration: T = S = 32768, top-2048 chosen by the indexer and top-k, inputs
    N(0,1)/16 and do N(0,1).  The sum identities over every position and dq of sampled rows
    against the oracle row by row."""
    sa = require_gpu()
    T, kk = 32768, 2048
    qi = synth.torch_normal((1, T, 4, 128), 128 ** -0.5, torch.bfloat16, 401, DEV)
    ki = synth.torch_normal((1, T, 128), 128 ** -0.5, torch.bfloat16, 402, DEV)
    wi = synth.torch_uniform((1, T, 4), 403, DEV)
    idx = sa.dsa_indexer_topk(qi, ki, wi, kk)
    del qi, ki, wi
    q = synth.torch_normal((1, T, 64, 256), 1.0 / 16, torch.bfloat16, 404, DEV)
    k = synth.torch_normal((1, T, 256), 1.0 / 16, torch.bfloat16, 405, DEV)
    v = synth.torch_normal((1, T, 256), 1.0 / 16, torch.bfloat16, 406, DEV)
    do = synth.torch_normal((1, T, 64, 256), 1.0, torch.bfloat16, 407, DEV)
    o, lse = sa.dsa_sparse_attention_fwd(q, k, v, idx, return_lse=True)
    dq, dk, dv = sa.dsa_sparse_attention_bwd(q, k, v, idx, o, lse, do)
    dk64, dv64 = dk.double(), dv.double()
    err_k = float(dk64.sum(dim=1).abs().max())
    mag_k = float(dk64.abs().sum(dim=1).max())
    err_v = float((dv64.sum(dim=1) - do.double().sum(dim=(1, 2))).abs().max())
    mag_v = float(dv64.abs().sum(dim=1).max())
    print(f"sum dk: {err_k:.3e} vs {mag_k:.3e}; sum dv: {err_v:.3e} vs {mag_v:.3e}", flush=True)
    assert err_k <= REL_TOL["dk"] * mag_k
    assert err_v <= REL_TOL["dv"] * mag_v  # every row has at least one entry
    kn, vn = f64(k), f64(v)
    rows = [0, 1, 2047, 2048, 16384, 32767]
    refs = []
    for i in rows:
        r = oracle.dsa_sparse_attention_bwd(f64(q[:, i:i + 1]), kn, vn, idx[:, i:i + 1].cpu().numpy().astype(np.int64),
                                            f64(do[:, i:i + 1]))
        refs.append(r[0])
    mag = max(float(np.abs(r).max()) for r in refs)
    for i, rq in zip(rows, refs):
        err = max_abs_err(f64(dq[:, i:i + 1]), rq)
        print(f"dq row {i}: max abs err {err:.3e} (largest sampled |dq| {mag:.3e})", flush=True)
        assert err <= REL_TOL["dq"] * mag, i

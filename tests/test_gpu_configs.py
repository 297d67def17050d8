"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The oracle cannot run these workloads whole, so each test checks sampled
outputs that the oracle computes one by one (chosen rows / heads / sequences,
including the first and last positions and the block and window edges).
Inputs come from the seeded device generators in synth.py; the oracle gets
the same bits by copying the needed slices to the host.

Tolerances: fp32 workloads 1e-5 normwise relative; bf16 workloads 2e-2
max-abs on unit-variance inputs, and 2e-2 * sigma_V on the workloads' own
N(0,1)/sqrt(d) inputs.  Top-k is bit-exact on the GPU's own scores, and
against the oracle's float64 scores with positions within 1e-6 of the k-th
score excluded.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import BF16_ABS_TOL, DEV, f64, max_abs_err, require_gpu

pytestmark = pytest.mark.gpu

BLK = WIN = 128


def _spread_rows(T, n, seed, edges):
    """At least n distinct rows: the given edges, an even spread over [0, T) and seeded random rows."""
    rows = set(int(x) for x in edges)
    rows |= set(int(x) for x in np.linspace(0, T - 1, n // 2).round())
    g = np.random.default_rng(seed)
    while len(rows) < n:
        rows.add(int(g.integers(0, T)))
    return sorted(rows)


def _hca_prefill_case(sa, sigma, seed, dqk=512):
    """Sampled outputs of the full prefill: 256+ spread rows (block and window edges, first and last
    tokens) of three heads against the oracle's prefill (its own compression of those heads), and every
    head of four rows against the oracle's decode over the GPU's compressed cache and the rows' windows
    (decode at position t equals prefill row t)."""
    T, H, d = 32768, 64, 512
    q = synth.torch_normal((1, H, T, dqk), sigma, torch.bfloat16, seed, DEV)
    k = synth.torch_normal((1, H, T, dqk), sigma, torch.bfloat16, seed + 1, DEV)
    v = synth.torch_normal((1, H, T, d), sigma, torch.bfloat16, seed + 2, DEV)
    kc = sa.hca_compress(k, BLK)
    vc = sa.hca_compress(v, BLK)
    o, lse = sa.hca_attention_fwd(sa.HCA_PREFILL, q, k, v, kc, vc, BLK, WIN, return_lse=True)
    torch.cuda.synchronize()
    edges = [0, 1, 126, 127, 128, 254, 255, 256, 383, 1000, 4097, 16384, 20000, 32639, 32640, 32767]
    rows = _spread_rows(T, 256, seed, edges)
    worst = 0.0
    for h in (0, 37, 63):
        qh, kh, vh = f64(q[:, h:h + 1]), f64(k[:, h:h + 1]), f64(v[:, h:h + 1])
        ow, lw = oracle.hca_attention_prefill(qh, kh, vh, oracle.hca_compress(kh, BLK), oracle.hca_compress(vh, BLK),
                                              BLK, WIN, rows=rows)
        got = f64(o[:, h:h + 1, rows])
        worst = max(worst, max_abs_err(got, ow))
        assert max_abs_err(f64(lse[:, h:h + 1, rows]), lw) <= 1e-2
        print(f"[hca prefill full] head {h}: {len(rows)} rows, max err {worst:.3e}", flush=True)
    kch, vch = f64(kc), f64(vc)
    for t in (127, 128, 20000, T - 1):
        lo = max(0, t - WIN + 1)
        ring_k = np.zeros((1, H, WIN, dqk))
        ring_v = np.zeros((1, H, WIN, d))
        pos = np.arange(lo, t + 1)
        ring_k[0][:, pos % WIN] = f64(k[0, :, lo:t + 1])
        ring_v[0][:, pos % WIN] = f64(v[0, :, lo:t + 1])
        ow, lw = oracle.hca_attention_decode(f64(q[:, :, t]), kch, vch, ring_k, ring_v, [t], BLK, WIN)
        worst = max(worst, max_abs_err(f64(o[:, :, t]), ow))
        assert max_abs_err(f64(lse[:, :, t]), lw) <= 1e-2, t
    print(f"[hca prefill full] all 64 heads of 4 rows: max err {worst:.3e}", flush=True)
    del q, k, v, kc, vc, o, lse
    torch.cuda.empty_cache()
    return worst


def test_hca_prefill_32768x64x512_unit_variance():
    sa = require_gpu()
    assert _hca_prefill_case(sa, 1.0, 1200) <= BF16_ABS_TOL


def test_hca_prefill_32768x64x512_config_distribution():
    sa = require_gpu()
    sigma = 1.0 / math.sqrt(512)
    assert _hca_prefill_case(sa, sigma, 1300) <= BF16_ABS_TOL * sigma


def test_hca_prefill_32768x64_qk576_v512_unit_variance():
    """The wider query/key head (qk 576, v 512) at the prefill workload's size."""
    sa = require_gpu()
    assert _hca_prefill_case(sa, 1.0, 1250, dqk=576) <= BF16_ABS_TOL


@pytest.mark.parametrize("B,ncap,pos,sigma,dqk", [(64, 1024, 131071, 1.0, 512), (64, 1024, 131071, 512 ** -0.5, 512),
                                                  (4, 8192, 1048575, 1.0, 512), (64, 1024, 131071, 1.0, 576),
                                                  (4, 8192, 1048575, 1.0, 576)])
def test_hca_decode_full(B, ncap, pos, sigma, dqk):
    sa = require_gpu()
    H, d = 64, 512
    q = synth.torch_normal((B, H, dqk), sigma, torch.bfloat16, 1400, DEV)
    kc = synth.torch_normal((B, H, ncap, dqk), sigma, torch.bfloat16, 1401, DEV)
    vc = synth.torch_normal((B, H, ncap, d), sigma, torch.bfloat16, 1402, DEV)
    rk = synth.torch_normal((B, H, WIN, dqk), sigma, torch.bfloat16, 1403, DEV)
    rv = synth.torch_normal((B, H, WIN, d), sigma, torch.bfloat16, 1404, DEV)
    posd = torch.full((B,), pos, dtype=torch.int64, device=DEV)
    o, lse = sa.hca_attention_fwd(sa.HCA_DECODE, q, rk, rv, kc, vc, BLK, WIN, pos=posd, return_lse=True)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (B - 1, 63), (B // 2, 17), (1, 40)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ow, lw = oracle.hca_attention_decode(f64(q[sl]), f64(kc[sl]), f64(vc[sl]), f64(rk[sl]), f64(rv[sl]), [pos],
                                             BLK, WIN)
        assert max_abs_err(f64(o[sl]), ow) <= BF16_ABS_TOL * sigma, (b, h)
        assert max_abs_err(f64(lse[sl]), lw) <= 1e-2


@pytest.mark.parametrize("B,ncap,pos", [(64, 1024, 131071), (4, 8192, 1048575)])
def test_hca_decode_fp8_full(B, ncap, pos):
    """FP8 cache at the decode configs' full sizes: GPU encoding bit-exact against the oracle on sampled
    (b, h) rows, GPU FP8 decode against the oracle over the dequantized cache."""
    sa = require_gpu()
    H, d = 64, 512
    q = synth.torch_normal((B, H, d), 1.0, torch.bfloat16, 1410, DEV)
    cache = {n: synth.torch_normal(shape, 1.0, torch.bfloat16, 1411 + i, DEV) for i, (n, shape) in enumerate(
        (("kc", (B, H, ncap, d)), ("vc", (B, H, ncap, d)), ("rk", (B, H, WIN, d)), ("rv", (B, H, WIN, d))))}
    enc = {n: sa.hca_quantize_fp8(t) for n, t in cache.items()}
    posd = torch.full((B,), pos, dtype=torch.int64, device=DEV)
    o, lse = sa.hca_decode_fp8(q, *enc["rk"], *enc["rv"], *enc["kc"], *enc["vc"], BLK, WIN, posd, return_lse=True)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (B - 1, 63), (B // 2, 17), (1, 40)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        deq = {}
        for n, t in cache.items():
            want_c, want_s = oracle.quantize_fp8_rows(f64(t[sl]))
            assert np.array_equal(enc[n][0][sl].cpu().numpy(), want_c), (n, b, h)
            assert np.array_equal(enc[n][1][sl].cpu().numpy(), want_s), (n, b, h)
            deq[n] = oracle.dequantize_fp8_rows(want_c, want_s)
        ow, lw = oracle.hca_attention_decode(f64(q[sl]), deq["kc"], deq["vc"], deq["rk"], deq["rv"], [pos], BLK, WIN)
        assert max_abs_err(f64(o[sl]), ow) <= BF16_ABS_TOL, (b, h)
        assert max_abs_err(f64(lse[sl]), lw) <= 1e-2


def _band_compare(got_idx, oracle_scores, k):
    """Top-k vs the oracle's float64 scores: positions within 1e-6 of the k-th score are excluded."""
    valid = np.isfinite(oracle_scores)
    cand = np.nonzero(valid)[0]
    want = oracle.dsa_topk(oracle_scores.reshape(1, 1, -1), k, q_pos=[cand.size - 1])[0, 0]
    got = got_idx[got_idx >= 0]
    want = want[want >= 0]
    if cand.size <= k:
        assert np.array_equal(got, want)
        return 0
    kth = np.sort(oracle_scores[cand])[::-1][k - 1]
    band = set(np.nonzero(np.abs(oracle_scores - kth) <= 1e-6)[0].tolist())
    g = set(got.tolist()) - band
    w = set(want.tolist()) - band
    assert g == w, (len(g ^ w), len(band))
    return len(band)


def _dsa_inputs(B, T, S, sigma, seed):
    qi = synth.torch_normal((B, T, 4, 128), 128 ** -0.5, torch.bfloat16, seed, DEV)
    ki = synth.torch_normal((B, S, 128), 128 ** -0.5, torch.bfloat16, seed + 1, DEV)
    w = synth.torch_uniform((B, T, 4), seed + 2, DEV)
    q = synth.torch_normal((B, T, 64, 256), sigma, torch.bfloat16, seed + 3, DEV)
    k = synth.torch_normal((B, S, 256), sigma, torch.bfloat16, seed + 4, DEV)
    v = synth.torch_normal((B, S, 256), sigma, torch.bfloat16, seed + 5, DEV)
    return qi, ki, w, q, k, v


@pytest.mark.parametrize("sigma", [1.0, 1.0 / 16])
def test_dsa_prefill_32768_top2048(sigma):
    sa = require_gpu()
    T = S = 32768
    kk = 2048
    qi, ki, w, q, k, v = _dsa_inputs(1, T, S, sigma, 1500)
    sc = sa.dsa_indexer_scores(qi, ki, w)
    idx = sa.dsa_topk(sc, kk)
    o, lse = sa.dsa_sparse_attention_fwd(q, k, v, idx, return_lse=True)
    torch.cuda.synchronize()
    # 256 spread rows at the workload's own distribution, 96 at unit variance (every row checks all 64 heads)
    edges = [0, 1, 2046, 2047, 2048, 2049, 4095, 8191, 8192, 10000, 16383, 16384, 32767]
    rows = _spread_rows(T, 256 if sigma < 1.0 else 96, 1501, edges)
    ki_h, q_h, k_h, v_h = f64(ki), None, f64(k), f64(v)
    for n_done, i in enumerate(rows):
        if n_done % 64 == 0:
            print(f"[dsa prefill full] sigma={sigma}: row {n_done} of {len(rows)}", flush=True)
        sc_row = sc[0, i, : i + 1].cpu().numpy().astype(np.float64)
        want_sc = oracle.dsa_indexer_scores(f64(qi[:, i:i + 1]), ki_h[:, : i + 1], f64(w[:, i:i + 1]), q_pos=[i])[0, 0]
        assert np.max(np.abs(sc_row - want_sc)) <= 2e-6, i
        got_idx = idx[0, i].cpu().numpy().astype(np.int64)
        # bit-exact on the GPU's own scores
        assert np.array_equal(got_idx, oracle.dsa_topk(sc_row.reshape(1, 1, -1), kk, q_pos=[i])[0, 0]), i
        # band comparison against the oracle's float64 scores
        _band_compare(got_idx, want_sc, kk)
        # attention on the GPU's indices
        ow, lw = oracle.dsa_sparse_attention(f64(q[:, i:i + 1]), k_h, v_h, got_idx.reshape(1, 1, -1))
        assert max_abs_err(f64(o[:, i:i + 1]), ow) <= BF16_ABS_TOL * sigma, i
        assert max_abs_err(f64(lse[:, i:i + 1]), lw) <= 1e-2, i


def test_csa_prefill_32768_ratio4_top2048():
    """CSA variant at the DSA prefill's size: block-4 means (8192 entries), indexer, top-2048 and sparse
    attention on the GPU; sampled rows against the oracle (scores within fp32 rounding, selection
    bit-exact on the GPU's scores, attention on the GPU's entries and cache within 2e-2)."""
    sa = require_gpu()
    T, ratio, kk = 32768, 4, 2048
    S = T // ratio
    qi, ki, w, q, k, v = _dsa_inputs(1, T, T, 1.0, 1600)
    kci = sa.hca_compress(ki[:, None], ratio)[:, 0].contiguous()
    kc = sa.hca_compress(k[:, None], ratio)[:, 0].contiguous()
    vc = sa.hca_compress(v[:, None], ratio)[:, 0].contiguous()
    sc = sa.csa_indexer_scores(qi, kci, w, ratio)
    idx = sa.csa_topk(sc, kk, ratio)
    o, lse = sa.dsa_sparse_attention_fwd(q, kc, vc, idx, return_lse=True)
    torch.cuda.synchronize()
    kci_h, kc_h, vc_h = f64(kci), f64(kc), f64(vc)
    rows = [0, 3, 8194, 8195, 20000, T - 1] + [int(x) for x in np.random.default_rng(1601).integers(8196, T, size=4)]
    for i in rows:
        n = oracle.n_candidates(i, ratio, S)
        if n == 0:  # no complete block yet: nothing selected, o = 0
            assert (idx[0, i] == -1).all() and (o[0, i] == 0).all(), i
            continue
        want_sc = oracle.dsa_indexer_scores(f64(qi[:, i:i + 1]), kci_h[:, :n], f64(w[:, i:i + 1]), q_pos=[n - 1])[0, 0]
        sc_row = sc[0, i, :n].cpu().numpy().astype(np.float64)
        assert np.max(np.abs(sc_row - want_sc)) <= 2e-6, i
        got_idx = idx[0, i].cpu().numpy().astype(np.int64)
        assert np.array_equal(got_idx, oracle.dsa_topk(sc_row.reshape(1, 1, -1), kk, q_pos=[n - 1])[0, 0]), i
        ow, lw = oracle.dsa_sparse_attention(f64(q[:, i:i + 1]), kc_h, vc_h, got_idx.reshape(1, 1, -1))
        assert max_abs_err(f64(o[:, i:i + 1]), ow) <= BF16_ABS_TOL, i


def test_dsa_decode_1m():
    sa = require_gpu()
    B, S, kk = 4, 1 << 20, 2048
    qi, ki, w, q, k, v = _dsa_inputs(B, 1, S, 1.0, 1600)
    qpos = torch.full((B,), S - 1, dtype=torch.int64, device=DEV)
    sc = sa.dsa_indexer_scores(qi, ki, w, q_pos=qpos)
    idx = sa.dsa_topk(sc, kk, q_pos=qpos)
    o = sa.dsa_sparse_attention_fwd(q, k, v, idx)
    torch.cuda.synchronize()
    for b in range(B):
        sc_row = sc[b, 0].cpu().numpy().astype(np.float64)
        want_sc = oracle.dsa_indexer_scores(f64(qi[b:b + 1]), f64(ki[b:b + 1]), f64(w[b:b + 1]), q_pos=[S - 1])[0, 0]
        assert np.max(np.abs(sc_row - want_sc)) <= 2e-6, b
        got_idx = idx[b, 0].cpu().numpy().astype(np.int64)
        assert np.array_equal(got_idx, oracle.dsa_topk(sc_row.reshape(1, 1, -1), kk, q_pos=[S - 1])[0, 0]), b
        _band_compare(got_idx, want_sc, kk)
        # gather only the selected rows for the oracle (same math, positions renumbered 0..n-1)
        sel = torch.from_numpy(got_idx[got_idx >= 0]).to(DEV)
        local = np.arange(sel.numel()).reshape(1, 1, -1)
        ow, _ = oracle.dsa_sparse_attention(f64(q[b:b + 1]), f64(k[b:b + 1, sel]), f64(v[b:b + 1, sel]), local)
        assert max_abs_err(f64(o[b:b + 1]), ow) <= BF16_ABS_TOL, b

"""GPU parity: HCA compression and attention (HIP library through the C ABI) vs the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import BF16_ABS_TOL, DEV, F32_REL_TOL, f64, max_abs_err, rel_err_normwise, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(shape, dtype, sigma, workload):
    arrs = [synth.np_normal(shape, sigma, dtype, workload, tid) for tid in range(3)]
    return arrs, [synth.to_torch(a, dtype, DEV) for a in arrs]


# ---------------------------------------------------------------------------
# hca_compress
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("dtype,d,T,blk", [("f32", 64, 1024, 128), ("f32", 64, 300, 128), ("bf16", 512, 700, 128),
                                           ("bf16", 512, 37, 4), ("bf16", 256, 260, 128), ("f32", 64, 9, 1),
                                           ("bf16", 576, 300, 128), ("bf16", 576, 50, 3)])
def test_compress(dtype, d, T, blk):
    sa = require_gpu()
    x = synth.np_normal((2, 3, T, d), 1.0, dtype, 101, 0)
    out = sa.hca_compress(synth.to_torch(x, dtype, DEV), blk)
    want = oracle.hca_compress(x, blk)
    got = f64(out)
    assert got.shape == want.shape
    if dtype == "f32":
        assert max_abs_err(got, want) <= 1e-6 * max(1.0, np.max(np.abs(want)))
    else:  # fp32 sum, one RNE rounding to bf16: within one bf16 ulp
        assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-30)


def test_compress_strided_into_cache_slot():
    """Compress a window ring [B,H,128,d] into slot j of a larger cache via strides."""
    sa = require_gpu()
    B, H, d, blk, ncap, slot = 2, 3, 512, 128, 8, 5
    ring = synth.np_normal((B, H, blk, d), 1.0, "bf16", 102, 0)
    cache = torch.zeros((B, H, ncap, d), dtype=torch.bfloat16, device=DEV)
    sa.hca_compress(synth.to_torch(ring, "bf16", DEV), blk, out=cache[:, :, slot:slot + 1])
    got = f64(cache)
    want = oracle.hca_compress(ring, blk)[:, :, 0]
    assert np.all(np.abs(got[:, :, slot] - want) <= 2.0 ** -8 * np.abs(want) + 1e-30)
    others = [j for j in range(ncap) if j != slot]
    assert np.all(got[:, :, others] == 0)


# ---------------------------------------------------------------------------
# HCA prefill
# ---------------------------------------------------------------------------


def _prefill_gpu(sa, tq, tk, tv, blk, window):
    kc = sa.hca_compress(tk, blk)
    vc = sa.hca_compress(tv, blk)
    return sa.hca_attention_fwd(sa.HCA_PREFILL, tq, tk, tv, kc, vc, blk, window, return_lse=True)


def test_prefill_tiny_f32_config():
    """Tiny HCA forward, fp32: [1,4,1024,64], blk = window = 128; normwise rel <= 1e-5 on every row."""
    sa = require_gpu()
    (q, k, v), (tq, tk, tv) = _inputs((1, 4, 1024, 64), "f32", 1.0, 1)
    o, lse = _prefill_gpu(sa, tq, tk, tv, 128, 128)
    ow, lw = oracle.hca_attention_prefill(q, k, v, oracle.hca_compress(k, 128), oracle.hca_compress(v, 128), 128, 128)
    assert rel_err_normwise(f64(o), ow) <= F32_REL_TOL
    assert max_abs_err(f64(lse), lw) <= 1e-5 * max(1.0, np.max(np.abs(lw)))


@pytest.mark.parametrize(
    "T,blk,window,H",
    [(700, 128, 128, 2), (257, 128, 128, 1), (64, 128, 128, 1), (200, 4, 6, 2), (130, 1, 5, 1), (150, 16, 200, 1),
     (1, 128, 128, 1), (333, 32, 1, 1)],
)
def test_prefill_bf16_d512(T, blk, window, H):
    """bf16 head dim 512 on unit-variance inputs: max-abs <= 2e-2 (covers several tiles, ragged tails,
    blk = 1 (dense causal), window >= T (dense causal), window = 1)."""
    sa = require_gpu()
    (q, k, v), (tq, tk, tv) = _inputs((1, H, T, 512), "bf16", 1.0, 2 + T + blk)
    o, lse = _prefill_gpu(sa, tq, tk, tv, blk, window)
    ow, lw = oracle.hca_attention_prefill(q, k, v, oracle.hca_compress(k, blk), oracle.hca_compress(v, blk), blk, window)
    assert max_abs_err(f64(o), ow) <= BF16_ABS_TOL
    assert max_abs_err(f64(lse), lw) <= 1e-2


def test_prefill_same_cache_isolates_attention():
    """Feed both sides the same bf16 compressed cache: attention error alone."""
    sa = require_gpu()
    T, blk, window = 600, 128, 128
    (q, k, v), (tq, tk, tv) = _inputs((2, 2, T, 512), "bf16", 1.0, 7)
    kc = sa.hca_compress(tk, blk)
    vc = sa.hca_compress(tv, blk)
    o = sa.hca_attention_fwd(sa.HCA_PREFILL, tq, tk, tv, kc, vc, blk, window)
    ow, _ = oracle.hca_attention_prefill(q, k, v, f64(kc), f64(vc), blk, window)
    assert max_abs_err(f64(o), ow) <= BF16_ABS_TOL


def test_prefill_deterministic():
    sa = require_gpu()
    (_, _, _), (tq, tk, tv) = _inputs((1, 2, 500, 512), "bf16", 1.0, 8)
    a, la = _prefill_gpu(sa, tq, tk, tv, 128, 128)
    b, lb = _prefill_gpu(sa, tq, tk, tv, 128, 128)
    assert torch.equal(a, b) and torch.equal(la, lb)


# ---------------------------------------------------------------------------
# HCA decode
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("B,H,ncap,positions", [(3, 2, 10, [0, 130, 1407]), (2, 3, 12, [5000, 127]),
                                                 (1, 2, 2000, [256000]), (4, 1, 3, [255, 256, 383, 384])])
def test_decode_bf16(B, H, ncap, positions):
    sa = require_gpu()
    blk, window, d = 128, 128, 512
    q = synth.np_normal((B, H, d), 1.0, "bf16", 20, 0)
    kc = synth.np_normal((B, H, ncap, d), 1.0, "bf16", 20, 1)
    vc = synth.np_normal((B, H, ncap, d), 1.0, "bf16", 20, 2)
    rk = synth.np_normal((B, H, window, d), 1.0, "bf16", 20, 3)
    rv = synth.np_normal((B, H, window, d), 1.0, "bf16", 20, 4)
    pos = torch.tensor(positions, dtype=torch.int64, device=DEV)
    t = [synth.to_torch(a, "bf16", DEV) for a in (q, rk, rv, kc, vc)]
    o, lse = sa.hca_attention_fwd(sa.HCA_DECODE, t[0], t[1], t[2], t[3], t[4], blk, window, pos=pos, return_lse=True)
    ow, lw = oracle.hca_attention_decode(q, kc, vc, rk, rv, positions, blk, window)
    assert max_abs_err(f64(o), ow) <= BF16_ABS_TOL
    assert max_abs_err(f64(lse), lw) <= 1e-2


def test_decode_equals_prefill_row():
    """Cross-mode: decode at position t (ring = last window tokens) equals prefill row t."""
    sa = require_gpu()
    T, blk, window, d = 900, 128, 128, 512
    (q, k, v), (tq, tk, tv) = _inputs((1, 2, T, d), "bf16", 1.0, 21)
    kc = sa.hca_compress(tk, blk)
    vc = sa.hca_compress(tv, blk)
    o_pre = sa.hca_attention_fwd(sa.HCA_PREFILL, tq, tk, tv, kc, vc, blk, window)
    for t in (0, 200, 511, 767, 899):
        ring_k = torch.zeros((1, 2, window, d), dtype=torch.bfloat16, device=DEV)
        ring_v = torch.zeros_like(ring_k)
        for s in range(max(0, t - window + 1), t + 1):
            ring_k[:, :, s % window] = tk[:, :, s]
            ring_v[:, :, s % window] = tv[:, :, s]
        pos = torch.tensor([t], dtype=torch.int64, device=DEV)
        o_dec = sa.hca_attention_fwd(sa.HCA_DECODE, tq[:, :, t].contiguous(), ring_k, ring_v, kc, vc, blk, window, pos=pos)
        assert max_abs_err(f64(o_dec), f64(o_pre[:, :, t])) <= 1e-2, f"t={t}"


def test_streaming_decode_loop_equals_prefill():
    """A serving loop over positions 250..700 of two sequences: each step writes the new token's k, v into
    the window ring (slot pos mod W), decodes, and when the step completes a block (pos + 1 = 128 (j + 1))
    compresses the ring -- which then holds exactly that block -- into cache entry j in place.  Every step's
    output equals prefill row pos (the cache before position 250 comes from hca_compress of the prefix)."""
    sa = require_gpu()
    B, H, T, blk, window, d = 2, 2, 701, 128, 128, 512
    (q, k, v), (tq, tk, tv) = _inputs((B, H, T, d), "bf16", 1.0, 23)
    kc_full, vc_full = sa.hca_compress(tk, blk), sa.hca_compress(tv, blk)
    o_pre = sa.hca_attention_fwd(sa.HCA_PREFILL, tq, tk, tv, kc_full, vc_full, blk, window)
    t0, ncap = 250, T // blk
    kc = torch.zeros((B, H, ncap, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    kc[:, :, :t0 // blk] = sa.hca_compress(tk[:, :, :t0].contiguous(), blk)
    vc[:, :, :t0 // blk] = sa.hca_compress(tv[:, :, :t0].contiguous(), blk)
    ring_k = torch.zeros((B, H, window, d), dtype=torch.bfloat16, device=DEV)
    ring_v = torch.zeros_like(ring_k)
    for s in range(t0 - window, t0):
        ring_k[:, :, s % window] = tk[:, :, s]
        ring_v[:, :, s % window] = tv[:, :, s]
    worst = 0.0
    for t in range(t0, T):
        ring_k[:, :, t % window] = tk[:, :, t]
        ring_v[:, :, t % window] = tv[:, :, t]
        pos = torch.full((B,), t, dtype=torch.int64, device=DEV)
        o_dec = sa.hca_attention_fwd(sa.HCA_DECODE, tq[:, :, t].contiguous(), ring_k, ring_v, kc, vc, blk, window,
                                     pos=pos)
        worst = max(worst, float((o_dec.float() - o_pre[:, :, t].float()).abs().max()))
        if (t + 1) % blk == 0:  # block j = (t + 1) / blk - 1 is complete: the ring holds exactly it
            j = (t + 1) // blk - 1
            sa.hca_compress(ring_k, blk, out=kc[:, :, j:j + 1])
            sa.hca_compress(ring_v, blk, out=vc[:, :, j:j + 1])
            assert torch.equal(kc[:, :, j], kc_full[:, :, j]) and torch.equal(vc[:, :, j], vc_full[:, :, j]), j
    torch.cuda.synchronize()
    print(f"[streaming decode] {T - t0} steps, max |decode - prefill row| {worst:.3e}", flush=True)
    assert worst <= 1e-2


# ---------------------------------------------------------------------------
# Query/key head wider than the value head (qk 576 / v 512)
# ---------------------------------------------------------------------------


def _wide_inputs(B, H, T, workload, dqk=576, dv=512):
    q = synth.np_normal((B, H, T, dqk), 1.0, "bf16", workload, 0)
    k = synth.np_normal((B, H, T, dqk), 1.0, "bf16", workload, 1)
    v = synth.np_normal((B, H, T, dv), 1.0, "bf16", workload, 2)
    return (q, k, v), [synth.to_torch(a, "bf16", DEV) for a in (q, k, v)]


@pytest.mark.parametrize(
    "T,blk,window,H",
    [(700, 128, 128, 2), (1200, 128, 128, 1), (257, 128, 128, 1), (200, 4, 6, 2), (130, 1, 5, 1), (150, 16, 200, 1),
     (1, 128, 128, 1), (333, 32, 1, 1)],
)
def test_prefill_qk576_v512(T, blk, window, H):
    """qk 576 / v 512 on unit-variance inputs: max-abs <= 2e-2 against the oracle (several 128-query
    workgroup tiles, ragged tails, blk = 1 and window >= T (dense causal), window = 1)."""
    sa = require_gpu()
    (q, k, v), (tq, tk, tv) = _wide_inputs(1, H, T, 30 + T + blk)
    o, lse = _prefill_gpu(sa, tq, tk, tv, blk, window)
    assert o.shape == (1, H, T, 512)
    ow, lw = oracle.hca_attention_prefill(q, k, v, oracle.hca_compress(k, blk), oracle.hca_compress(v, blk), blk, window)
    assert max_abs_err(f64(o), ow) <= BF16_ABS_TOL
    assert max_abs_err(f64(lse), lw) <= 1e-2


def test_prefill_qk576_extra_dims_enter_logits():
    """The 64 extra query/key dims change the result; with them zeroed it equals the 512-wide call at the
    same scale (1/24), so they enter only through the logits."""
    sa = require_gpu()
    T, blk, window = 600, 128, 128
    (q, k, v), (tq, tk, tv) = _wide_inputs(1, 2, T, 31)
    o_wide = _prefill_gpu(sa, tq, tk, tv, blk, window)[0]
    tk0 = tk.clone()
    tk0[..., 512:] = 0
    kc0, vc = sa.hca_compress(tk0, blk), sa.hca_compress(tv, blk)
    o_zero = sa.hca_attention_fwd(sa.HCA_PREFILL, tq, tk0, tv, kc0, vc, blk, window)
    o_512 = sa.hca_attention_fwd(sa.HCA_PREFILL, tq[..., :512].contiguous(), tk0[..., :512].contiguous(), tv,
                                 kc0[..., :512].contiguous(), vc, blk, window, scale=1.0 / 24)
    assert max_abs_err(f64(o_zero), f64(o_512)) <= 1e-2
    assert max_abs_err(f64(o_wide), f64(o_zero)) > 1e-2


@pytest.mark.parametrize("B,H,ncap,positions", [(3, 2, 10, [0, 130, 1407]), (2, 3, 12, [5000, 127]),
                                                 (1, 2, 2000, [256000]), (4, 1, 3, [255, 256, 383, 384])])
def test_decode_qk576_v512(B, H, ncap, positions):
    sa = require_gpu()
    blk, window = 128, 128
    q = synth.np_normal((B, H, 576), 1.0, "bf16", 32, 0)
    kc = synth.np_normal((B, H, ncap, 576), 1.0, "bf16", 32, 1)
    vc = synth.np_normal((B, H, ncap, 512), 1.0, "bf16", 32, 2)
    rk = synth.np_normal((B, H, window, 576), 1.0, "bf16", 32, 3)
    rv = synth.np_normal((B, H, window, 512), 1.0, "bf16", 32, 4)
    pos = torch.tensor(positions, dtype=torch.int64, device=DEV)
    t = [synth.to_torch(a, "bf16", DEV) for a in (q, rk, rv, kc, vc)]
    o, lse = sa.hca_attention_fwd(sa.HCA_DECODE, t[0], t[1], t[2], t[3], t[4], blk, window, pos=pos, return_lse=True)
    assert o.shape == (B, H, 512)
    ow, lw = oracle.hca_attention_decode(q, kc, vc, rk, rv, positions, blk, window)
    assert max_abs_err(f64(o), ow) <= BF16_ABS_TOL
    assert max_abs_err(f64(lse), lw) <= 1e-2


def test_decode_equals_prefill_row_qk576():
    sa = require_gpu()
    T, blk, window = 900, 128, 128
    (q, k, v), (tq, tk, tv) = _wide_inputs(1, 2, T, 33)
    kc, vc = sa.hca_compress(tk, blk), sa.hca_compress(tv, blk)
    o_pre = sa.hca_attention_fwd(sa.HCA_PREFILL, tq, tk, tv, kc, vc, blk, window)
    for t in (0, 200, 511, 767, 899):
        ring_k = torch.zeros((1, 2, window, 576), dtype=torch.bfloat16, device=DEV)
        ring_v = torch.zeros((1, 2, window, 512), dtype=torch.bfloat16, device=DEV)
        for s in range(max(0, t - window + 1), t + 1):
            ring_k[:, :, s % window] = tk[:, :, s]
            ring_v[:, :, s % window] = tv[:, :, s]
        pos = torch.tensor([t], dtype=torch.int64, device=DEV)
        o_dec = sa.hca_attention_fwd(sa.HCA_DECODE, tq[:, :, t].contiguous(), ring_k, ring_v, kc, vc, blk, window, pos=pos)
        assert max_abs_err(f64(o_dec), f64(o_pre[:, :, t])) <= 1e-2, f"t={t}"


# ---------------------------------------------------------------------------
# FP8 (E4M3) decode cache
# ---------------------------------------------------------------------------


def _fp8_rows_case():
    """bf16 rows over many magnitudes (subnormal codes included), a zero row, a row with -0.0
    entries, a single-nonzero row and a constant row."""
    x = synth.np_normal((12, 512), 1.0, "bf16", 24, 0).astype(np.float64)
    x *= np.array([1.0, 1e-3, 40.0, 1e-5, 3.0, 0.25, 1.0, 1.0, 1.0, 1.0, 7.0, 1e-2])[:, None]
    x[6, :] = 0.0
    x[7, :] = -0.0
    x[7, 3] = 1.5
    x[8, :] = 0.0
    x[8, 100] = -3.0
    x[9, :] = 0.625
    x[10, :] = np.where(x[10] < 0, -1.0, 1.0) * np.exp2(np.linspace(-25, 3, 512))  # subnormal codes
    return synth.round_to(x, "bf16")


def test_quantize_fp8_bit_exact():
    sa = require_gpu()
    x = _fp8_rows_case()
    codes, scales = sa.hca_quantize_fp8(synth.to_torch(x, "bf16", DEV))
    want_c, want_s = oracle.quantize_fp8_rows(x)
    got_c = codes.cpu().numpy()
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, f"{bad.shape[0]} codes differ, first at {bad[:3]}: {got_c[tuple(bad[0])]:#x} vs {want_c[tuple(bad[0])]:#x}"
    assert np.array_equal(scales.cpu().numpy(), want_s)


def test_quantize_fp8_cache_layout():
    """A [B,H,N,d] cache quantizes row by row (one scale per (b, h, n))."""
    sa = require_gpu()
    x = synth.np_normal((2, 3, 5, 512), 0.5, "bf16", 25, 0)
    codes, scales = sa.hca_quantize_fp8(synth.to_torch(x, "bf16", DEV))
    assert codes.shape == (2, 3, 5, 512) and scales.shape == (2, 3, 5)
    want_c, want_s = oracle.quantize_fp8_rows(x)
    assert np.array_equal(codes.cpu().numpy(), want_c)
    assert np.array_equal(scales.cpu().numpy(), want_s)


@pytest.mark.parametrize("B,H,ncap,positions", [(3, 2, 10, [0, 130, 1407]), (2, 3, 12, [5000, 127]),
                                                 (1, 2, 2000, [256000]), (4, 1, 3, [255, 256, 383, 384])])
def test_decode_fp8(B, H, ncap, positions):
    """GPU-encoded cache (checked bit-exact against the oracle's encoding) -> GPU FP8 decode vs the
    oracle's decode over the dequantized cache."""
    sa = require_gpu()
    blk, window, d = 128, 128, 512
    q = synth.np_normal((B, H, d), 1.0, "bf16", 26, 0)
    rows = {name: synth.np_normal(shape, 1.0, "bf16", 26, tid) for tid, (name, shape) in enumerate(
        (("kc", (B, H, ncap, d)), ("vc", (B, H, ncap, d)), ("rk", (B, H, window, d)), ("rv", (B, H, window, d))),
        start=1)}
    enc = {n: sa.hca_quantize_fp8(synth.to_torch(a, "bf16", DEV)) for n, a in rows.items()}
    deq = {}
    for n, a in rows.items():
        want_c, want_s = oracle.quantize_fp8_rows(a)
        assert np.array_equal(enc[n][0].cpu().numpy(), want_c), n
        assert np.array_equal(enc[n][1].cpu().numpy(), want_s), n
        deq[n] = oracle.dequantize_fp8_rows(want_c, want_s)
    pos = torch.tensor(positions, dtype=torch.int64, device=DEV)
    o, lse = sa.hca_decode_fp8(synth.to_torch(q, "bf16", DEV), *enc["rk"], *enc["rv"], *enc["kc"], *enc["vc"],
                               blk, window, pos, return_lse=True)
    ow, lw = oracle.hca_attention_decode(q, deq["kc"], deq["vc"], deq["rk"], deq["rv"], positions, blk, window)
    assert max_abs_err(f64(o), ow) <= BF16_ABS_TOL
    assert max_abs_err(f64(lse), lw) <= 1e-2

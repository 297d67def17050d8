"""GPU parity: DSA indexer, top-k and sparse attention (HIP library through the C ABI) vs the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import BF16_ABS_TOL, DEV, f64, max_abs_err, require_gpu

pytestmark = pytest.mark.gpu


def _indexer_inputs(B, T, S, workload, grid=False):
    if grid:
        qi = synth.np_int_grid((B, T, 4, 128), [v / 4 for v in range(-3, 4)], workload, 0)
        ki = synth.np_int_grid((B, S, 128), [v / 4 for v in range(-3, 4)], workload, 1)
        w = synth.np_int_grid((B, T, 4), [0, 0.25, 0.5, 0.75, 1.0], workload, 2)
    else:
        qi = synth.np_normal((B, T, 4, 128), 128 ** -0.5, "bf16", workload, 0)
        ki = synth.np_normal((B, S, 128), 128 ** -0.5, "bf16", workload, 1)
        w = synth.np_uniform((B, T, 4), workload, 2)
    return qi, ki, w


def _causal_mask(B, T, S, q_pos):
    m = np.zeros((B, T, S), dtype=bool)
    for b in range(B):
        base = 0 if q_pos is None else q_pos[b]
        for i in range(T):
            m[b, i, : min(S, base + i + 1)] = True
    return m


# ---------------------------------------------------------------------------
# indexer
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("B,T,S,q_pos", [(1, 300, 300, None), (2, 70, 333, [263, 100]), (1, 1, 5000, [4999]),
                                         (2, 1, 4500, [4499, 2047]), (1, 1, 70, None),
                                         (1, 129, 1100, [900]), (2, 3, 2000, [1999, 700]), (1, 4, 300, None),
                                         (3, 2, 129, [128, 0, 64]), (1, 9, 2500, [2400])])
def test_indexer_random(B, T, S, q_pos):
    sa = require_gpu()
    qi, ki, w = _indexer_inputs(B, T, S, 30 + T)
    qp = None if q_pos is None else torch.tensor(q_pos, dtype=torch.int64, device=DEV)
    sc = sa.dsa_indexer_scores(synth.to_torch(qi, "bf16", DEV), synth.to_torch(ki, "bf16", DEV),
                               synth.to_torch(w, "f32", DEV), q_pos=qp)
    want = oracle.dsa_indexer_scores(qi, ki, w, q_pos=q_pos)
    m = _causal_mask(B, T, S, q_pos)
    got = f64(sc)
    # fp32 accumulation of 128 exact bf16 products: |err| <= ~1e-6 on O(1) scores
    assert np.max(np.abs(got[m] - want[m])) <= 2e-6


@pytest.mark.parametrize("B,T,S,q_pos", [(2, 14, 2000, [1500, 1200]), (2, 13, 700, [650, 300]), (2, 30, 1500, [1300, 1000]),
                                         (1, 47, 2100, [2000]), (2, 15, 900, None)])
def test_indexer_partial_wave_rows_stay_in_bounds(B, T, S, q_pos):
    """A wave whose 16 query rows are not all real (13..15 left) stores nothing for the missing rows, also on
    tiles its real rows see in full: a guard region behind the scores keeps its sentinel, entries past each
    row's causal limit are not written, and every visible score matches the oracle (so the next batch's rows
    were not overwritten either)."""
    sa = require_gpu()
    qi, ki, w = _indexer_inputs(B, T, S, 40 + T)
    qp = None if q_pos is None else torch.tensor(q_pos, dtype=torch.int64, device=DEV)
    n = B * T * S
    buf = torch.full((n + 4 * S,), -7.0, dtype=torch.float32, device=DEV)
    out = buf[:n].view(B, T, S)
    sa.dsa_indexer_scores(synth.to_torch(qi, "bf16", DEV), synth.to_torch(ki, "bf16", DEV), synth.to_torch(w, "f32", DEV),
                          q_pos=qp, out=out)
    torch.cuda.synchronize()
    assert bool((buf[n:] == -7.0).all()), "write past the end of the scores"
    m = _causal_mask(B, T, S, q_pos)
    got = f64(out)
    assert np.all(got[~m] == -7.0), "write past a row's causal limit"
    want = oracle.dsa_indexer_scores(qi, ki, w, q_pos=q_pos)
    assert np.max(np.abs(got[m] - want[m])) <= 2e-6


def test_indexer_integer_grid_bit_exact():
    sa = require_gpu()
    B, T, S = 1, 200, 260
    qi, ki, w = _indexer_inputs(B, T, S, 31, grid=True)
    qp = torch.tensor([59], dtype=torch.int64, device=DEV)
    sc = sa.dsa_indexer_scores(synth.to_torch(qi, "bf16", DEV), synth.to_torch(ki, "bf16", DEV),
                               synth.to_torch(w, "f32", DEV), q_pos=qp)
    want = oracle.dsa_indexer_scores(qi, ki, w, q_pos=[59])
    m = _causal_mask(B, T, S, [59])
    assert np.array_equal(f64(sc)[m], want[m])


# ---------------------------------------------------------------------------
# top-k: GPU top-k on the GPU's own scores vs the oracle top-k on the same scores -> bit-exact
# ---------------------------------------------------------------------------


def _topk_check(sa, scores_np, k, q_pos):
    scores = torch.from_numpy(scores_np.astype(np.float32)).to(DEV)
    qp = None if q_pos is None else torch.tensor(q_pos, dtype=torch.int64, device=DEV)
    idx = sa.dsa_topk(scores, k, q_pos=qp)
    want = oracle.dsa_topk(scores_np.astype(np.float32), k, q_pos=q_pos)
    got = idx.cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"first mismatch at {bad[:3]}: got {got[tuple(bad[0][:2])][:8]} want {want[tuple(bad[0][:2])][:8]}"


@pytest.mark.parametrize("T,S,k", [(300, 300, 64), (70, 2100, 2048), (40, 5000, 1)])
def test_topk_random(T, S, k):
    sa = require_gpu()
    g = np.random.default_rng(40 + T)
    sc = g.standard_normal((1, T, S)).astype(np.float32)
    _topk_check(sa, sc, k, [S - T])


def test_topk_heavy_ties_and_signed_zero():
    sa = require_gpu()
    g = np.random.default_rng(41)
    sc = g.integers(-2, 3, size=(2, 50, 3000)).astype(np.float32) * 0.5
    sc[sc == 0] = np.where(g.random(np.count_nonzero(sc == 0)) < 0.5, -0.0, 0.0)
    _topk_check(sa, sc, 700, [2950, 1000])


def test_topk_constant_rows_take_lowest():
    sa = require_gpu()
    sc = np.full((1, 3, 4000), 0.125, dtype=np.float32)
    _topk_check(sa, sc, 2048, [3997])


def test_topk_long_rows_few_distinct_values():
    """32768-wide rows with four distinct scores: the k-th key has thousands of copies, so the
    sampled bracket holds too many candidates and the full-row refinement rounds run."""
    sa = require_gpu()
    g = np.random.default_rng(44)
    S = 32768
    sc = (g.integers(0, 4, size=(1, 4, S)) * 0.25).astype(np.float32)
    _topk_check(sa, sc, 2048, [S - 4])


def test_topk_position_structured_scores():
    """Scores that depend on the position modulo 4 mislead a sample of every 4th position
    (the bracket check fails and the full-row path decides)."""
    sa = require_gpu()
    g = np.random.default_rng(45)
    S = 32768
    pos = np.arange(S)
    sc = np.where(pos % 4 == 0, 10.0 + g.random(S), g.random(S)).astype(np.float32)[None, None, :]
    sc = np.repeat(sc, 3, axis=1)
    sc[0, 1] = np.where(pos % 4 == 2, -g.random(S), g.random(S) * 1e-3)  # mostly tiny values
    _topk_check(sa, sc, 2048, [S - 3])


def test_topk_relu_like_scores_many_zeros():
    """ReLU-like scores with exact zeros at every 4th position (the positions the bracket samples,
    so the full-row path decides); k = 2048 of 32768, and rows just longer than k."""
    sa = require_gpu()
    g = np.random.default_rng(46)
    S = 32768
    sc = np.maximum(g.standard_normal((1, 5, S)), 0).astype(np.float32)
    sc[:, :, ::4] = 0.0
    _topk_check(sa, sc, 2048, [S - 5])
    _topk_check(sa, sc[:, :, :2050].copy(), 2048, [2045])


def test_topk_tie_split_at_threshold():
    """The k-th score has more copies than the selection can take: the lowest positions of
    the tied score are taken (split ties)."""
    sa = require_gpu()
    g = np.random.default_rng(47)
    S = 20000
    sc = g.standard_normal((1, 2, S)).astype(np.float32) - 5.0
    sc[0, :, g.choice(S, 1000, replace=False)] = 3.0        # 1000 clear winners
    tie = g.choice(np.nonzero(sc[0, 0] < 0)[0], 3000, replace=False)
    sc[0, :, tie] = 1.5                                       # 3000 copies straddle k = 2048
    _topk_check(sa, sc, 2048, [S - 2])


def test_topk_causal_row_classes():
    """Causal rows from position 0 are split by length over three workgroup sizes (rows up to
    8192, 16384 and longer positions); rows on both sides of each cut, on normal scores and on
    ReLU-like scores whose zeros straddle the k-th key."""
    sa = require_gpu()
    B, T, k = 2, 17000, 2048
    sc = synth.torch_normal((B, T, T), 1.0, torch.float32, 48, DEV)
    sc[1].clamp_(min=0.0)
    idx = sa.dsa_topk(sc, k)
    torch.cuda.synchronize()
    rows = [0, 1, 2047, 2048, 2049, 3000, 8191, 8192, 8193, 12000, 16383, 16384, 16385, T - 1]
    for b in range(B):
        for i in rows:
            row = sc[b, i, : i + 1].cpu().numpy()
            want = oracle.dsa_topk(row.reshape(1, 1, -1), k, q_pos=[i])[0, 0]
            assert np.array_equal(idx[b, i].cpu().numpy(), want), (b, i)


def test_topk_multi_workgroup_path():
    """Rows longer than the on-chip limit (S > 32768) use the multi-workgroup path."""
    sa = require_gpu()
    g = np.random.default_rng(42)
    S = 70000
    sc = (g.integers(0, 5000, size=(2, 3, S)) / 64.0).astype(np.float32)  # many ties
    _topk_check(sa, sc, 2048, [S - 3, 40000])


def test_topk_multi_workgroup_odd_width_and_short_rows():
    """Long rows of odd width (positions not a multiple of 4 or of the chunk size) with ties
    across chunk boundaries, plus rows no longer than k in the same call."""
    sa = require_gpu()
    g = np.random.default_rng(49)
    S = 50001
    sc = (g.integers(0, 3000, size=(2, 2, S)) / 32.0).astype(np.float32)
    sc[0, 0, 4090:4100] = 200.0  # equal top scores on both sides of a chunk boundary
    _topk_check(sa, sc, 2048, [S - 2, 1000])


def test_topk_on_indexer_scores():
    """The real chain: GPU indexer scores -> GPU top-k vs oracle top-k on those scores."""
    sa = require_gpu()
    T, S, k = 400, 400, 128
    qi, ki, w = _indexer_inputs(1, T, S, 43)
    sc = sa.dsa_indexer_scores(synth.to_torch(qi, "bf16", DEV), synth.to_torch(ki, "bf16", DEV),
                               synth.to_torch(w, "f32", DEV))
    sc_np = sc.cpu().numpy()
    idx = sa.dsa_topk(sc, k).cpu().numpy()
    want = oracle.dsa_topk(np.where(_causal_mask(1, T, S, None), sc_np, np.nan), k)
    assert np.array_equal(idx, want)


# ---------------------------------------------------------------------------
# sparse attention
# ---------------------------------------------------------------------------


def _random_idx(B, T, S, kk, g, q_pos=None):
    idx = np.full((B, T, kk), -1, dtype=np.int64)
    for b in range(B):
        for i in range(T):
            p = min(S - 1, (0 if q_pos is None else q_pos[b]) + i)
            n = min(kk, p + 1)
            sel = np.sort(g.choice(p + 1, size=n, replace=False))
            idx[b, i, :n] = sel
    return idx


@pytest.mark.parametrize("B,T,S,kk", [(1, 40, 400, 128), (2, 9, 3000, 2048), (1, 64, 64, 100), (1, 5, 50, 33),
                                      (1, 600, 700, 64), (2, 300, 2500, 300)])
def test_sparse_attention_unit_variance(B, T, S, kk):
    """Covers the split index-list path (few tokens) and the one-workgroup-per-token path (>= 512 tokens)."""
    sa = require_gpu()
    g = np.random.default_rng(50 + kk)
    q = synth.np_normal((B, T, 64, 256), 1.0, "bf16", 51, 0)
    k = synth.np_normal((B, S, 256), 1.0, "bf16", 51, 1)
    v = synth.np_normal((B, S, 256), 1.0, "bf16", 51, 2)
    idx = _random_idx(B, T, S, kk, g, q_pos=[S - T] * B)
    o, lse = sa.dsa_sparse_attention_fwd(synth.to_torch(q, "bf16", DEV), synth.to_torch(k, "bf16", DEV),
                                         synth.to_torch(v, "bf16", DEV),
                                         torch.from_numpy(idx.astype(np.int32)).to(DEV), return_lse=True)
    ow, lw = oracle.dsa_sparse_attention(q, k, v, idx)
    assert max_abs_err(f64(o), ow) <= BF16_ABS_TOL
    assert max_abs_err(f64(lse), lw) <= 1e-2


def test_sparse_attention_skips_out_of_range_and_empty_rows():
    sa = require_gpu()
    B, T, S, kk = 1, 4, 100, 40
    q = synth.np_normal((B, T, 64, 256), 1.0, "bf16", 52, 0)
    k = synth.np_normal((B, S, 256), 1.0, "bf16", 52, 1)
    v = synth.np_normal((B, S, 256), 1.0, "bf16", 52, 2)
    idx = np.full((B, T, kk), -1, dtype=np.int64)
    idx[0, 0, :5] = [3, 150, 7, -9, 99]  # 150 and -9 are out of range
    idx[0, 1, 10:12] = [42, 43]
    idx[0, 3, :] = np.arange(kk)
    o, lse = sa.dsa_sparse_attention_fwd(synth.to_torch(q, "bf16", DEV), synth.to_torch(k, "bf16", DEV),
                                         synth.to_torch(v, "bf16", DEV),
                                         torch.from_numpy(idx.astype(np.int32)).to(DEV), return_lse=True)
    clean = np.where((idx >= 0) & (idx < S), idx, -1)
    ow, lw = oracle.dsa_sparse_attention(q, k, v, clean)
    assert max_abs_err(f64(o), ow) <= BF16_ABS_TOL
    assert np.all(f64(o)[0, 2] == 0) and np.all(np.isneginf(f64(lse)[0, 2]))
    fin = np.isfinite(lw)
    assert max_abs_err(f64(lse)[fin], lw[fin]) <= 1e-2


def test_dsa_end_to_end_k_ge_context_is_dense():
    """k >= context: the chain reduces to dense causal multi-query attention."""
    sa = require_gpu()
    T = 300
    qi, ki, w = _indexer_inputs(1, T, T, 53)
    q = synth.np_normal((1, T, 64, 256), 1.0, "bf16", 54, 0)
    k = synth.np_normal((1, T, 256), 1.0, "bf16", 54, 1)
    v = synth.np_normal((1, T, 256), 1.0, "bf16", 54, 2)
    sc = sa.dsa_indexer_scores(synth.to_torch(qi, "bf16", DEV), synth.to_torch(ki, "bf16", DEV),
                               synth.to_torch(w, "f32", DEV))
    idx = sa.dsa_topk(sc, 512)
    o = sa.dsa_sparse_attention_fwd(synth.to_torch(q, "bf16", DEV), synth.to_torch(k, "bf16", DEV),
                                    synth.to_torch(v, "bf16", DEV), idx)
    dense = np.full((1, T, 512), -1)
    for i in range(T):
        dense[0, i, : i + 1] = np.arange(i + 1)
    assert np.array_equal(idx.cpu().numpy(), dense)
    ow, _ = oracle.dsa_sparse_attention(q, k, v, dense)
    assert max_abs_err(f64(o), ow) <= BF16_ABS_TOL


# ---------------------------------------------------------------------------
# Fused indexer -> top-k: exactly the separate calls' selection
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("B,T,S,kk,q_pos,grid", [(1, 300, 300, 64, None, False), (2, 70, 333, 32, [263, 100], False),
                                                  (1, 1, 5000, 2048, [4999], False), (1, 2000, 2000, 128, None, False),
                                                  (1, 4096, 4096, 2048, None, False), (2, 17, 3000, 100, [2900, 1500], False),
                                                  (1, 3, 1000, 16, [999], False), (2, 9, 2100, 7, [2000, 30], False),
                                                  (1, 700, 700, 64, None, True), (1, 1500, 1500, 1, None, False),
                                                  (1, 33, 10, 4, None, False), (1, 8320, 8320, 2048, None, False),
                                                  (9, 2, 32768, 2048, [32766 - 3001 * b for b in range(9)], False)])
@pytest.mark.parametrize("force", [False, True])
def test_indexer_topk_equals_separate_calls(B, T, S, kk, q_pos, grid, force):
    """dsa_indexer_topk returns exactly dsa_topk(dsa_indexer_scores(...)): several chunks, ragged sizes,
    per-batch q_pos, decode-sized calls, integer-grid inputs (heavy ties), k = 1, S < 16 (no samples);
    force=True sends every long row through the exact recomputation instead of the candidates.  The
    exact recomputation runs on bounded grids that walk the work: T = S = 8320 gives the 4-wave
    filtered indexer 130 x 9 = 1170 query tile x chunk blocks (more than its 1024 workgroups) and
    the filtered top-k 6272 flagged rows (more than its 512); B = 9, T = 2, S = 32768 gives the
    1-wave filtered indexer 9 x 128 = 1152 blocks."""
    sa = require_gpu()
    qi, ki, w = _indexer_inputs(B, T, S, 50 + T, grid=grid)
    tqi, tki, tw = synth.to_torch(qi, "bf16", DEV), synth.to_torch(ki, "bf16", DEV), synth.to_torch(w, "f32", DEV)
    qp = None if q_pos is None else torch.tensor(q_pos, dtype=torch.int64, device=DEV)
    want = sa.dsa_topk(sa.dsa_indexer_scores(tqi, tki, tw, q_pos=qp), kk, q_pos=qp)
    got = sa.dsa_indexer_topk(tqi, tki, tw, kk, q_pos=qp, force_fallback=force)
    assert torch.equal(got, want)


@pytest.mark.parametrize("B,T,S,kk,q_pos,zero_w", [(2, 64, 1025, 64, [961, 500], True), (2, 64, 1025, 64, [961, 900], False),
                                                    (2, 64, 301, 64, [237, 100], False), (2, 64, 301, 64, [237, 100], True),
                                                    (3, 40, 2049, 32, [2009, 1999, 7], True)])
def test_indexer_topk_odd_width_all_candidate_rows(B, T, S, kk, q_pos, zero_w):
    """Odd S with rows that see every position: the last chunk of a row can be all candidates with an odd
    length (its pad entry then sits at index S of the row), followed by the next row's segments.  w = 0 makes
    every score 0.0, so every visible position is a candidate; S = 301 rows keep every position through a
    zero threshold (too few samples).  The result must equal the separate calls and, for w = 0, the lowest
    positions (ties go to the lower position)."""
    sa = require_gpu()
    qi, ki, w = _indexer_inputs(B, T, S, 70 + S)
    if zero_w:
        w = np.zeros_like(w)
    tqi, tki, tw = synth.to_torch(qi, "bf16", DEV), synth.to_torch(ki, "bf16", DEV), synth.to_torch(w, "f32", DEV)
    qp = torch.tensor(q_pos, dtype=torch.int64, device=DEV)
    want = sa.dsa_topk(sa.dsa_indexer_scores(tqi, tki, tw, q_pos=qp), kk, q_pos=qp)
    got = sa.dsa_indexer_topk(tqi, tki, tw, kk, q_pos=qp)
    assert torch.equal(got, want)
    if zero_w:
        exp = np.full((B, T, kk), -1)
        for b in range(B):
            for i in range(T):
                n = min(S, q_pos[b] + i + 1)
                exp[b, i, : min(n, kk)] = np.arange(min(n, kk))
        assert np.array_equal(got.cpu().numpy(), exp)


@pytest.mark.parametrize("B,T,S,kk,q_pos,zero_w", [(2, 1, 70000, 2048, [69999, 40000], False),
                                                    (1, 3, 100000, 64, [99997], False),
                                                    (2, 2, 40000, 2048, [39998, 100], False),
                                                    (3, 1, 50001, 7, [50000, 33000, 1], False),
                                                    (1, 4, 40000, 300, [39996], True),
                                                    (4, 1, 1 << 20, 2048, [(1 << 20) - 1, 900000, 524287, 40000], False),
                                                    (1, 2, 50000, 2048, [3000], False)])
@pytest.mark.parametrize("force", [False, True])
def test_indexer_topk_long_decode_rows(B, T, S, kk, q_pos, zero_w, force):
    """Decode-shaped calls with rows longer than 32768 positions (up to the 1M context): the candidate path
    of the decode indexer and the per-row select must return exactly the separate calls' indices; rows with
    at most k visible positions keep all; rows with more than k positions but too few samples for a
    threshold (3001 and 3002 positions: 46 samples at stride 64, rank 66) make every position a candidate;
    w = 0 (every score 0.0, more candidates than the select holds) and force=True take the exact
    recomputation from the full scores."""
    sa = require_gpu()
    print(f"[fused long] B={B} T={T} S={S} k={kk} q_pos={q_pos} zero_w={zero_w} force={force}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(90 + T + kk)
    tqi = (torch.randn((B, T, 4, 128), generator=g, device=DEV) * 128 ** -0.5).to(torch.bfloat16)
    tki = (torch.randn((B, S, 128), generator=g, device=DEV) * 128 ** -0.5).to(torch.bfloat16)
    tw = torch.rand((B, T, 4), generator=g, device=DEV)
    if zero_w:
        tw.zero_()
    qp = torch.tensor(q_pos, dtype=torch.int64, device=DEV)
    want = sa.dsa_topk(sa.dsa_indexer_scores(tqi, tki, tw, q_pos=qp), kk, q_pos=qp)
    got = sa.dsa_indexer_topk(tqi, tki, tw, kk, q_pos=qp, force_fallback=force)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    if zero_w:
        n = min(S, q_pos[0] + 1)
        assert torch.equal(got[0, 0, :min(n, kk)].cpu(), torch.arange(min(n, kk), dtype=torch.int32))


def test_indexer_topk_long_decode_max_rows():
    """The largest supported decode rows: S = 2^24 positions, two queries (q_pos near the end): the fused
    call equals the separate indexer + top-k."""
    sa = require_gpu()
    B, T, S, kk = 1, 2, 1 << 24, 2048
    print(f"[fused long max] B={B} T={T} S={S} k={kk}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(98)
    tqi = (torch.randn((B, T, 4, 128), generator=g, device=DEV) * 128 ** -0.5).to(torch.bfloat16)
    tki = torch.empty((B, S, 128), dtype=torch.bfloat16, device=DEV)
    for c in range(0, S, 1 << 22):  # chunks keep the float32 draw small
        tki[:, c:c + (1 << 22)] = (torch.randn((B, 1 << 22, 128), generator=g, device=DEV) * 128 ** -0.5).to(torch.bfloat16)
    tw = torch.rand((B, T, 4), generator=g, device=DEV)
    qp = torch.tensor([S - 2], dtype=torch.int64, device=DEV)
    want = sa.dsa_topk(sa.dsa_indexer_scores(tqi, tki, tw, q_pos=qp), kk, q_pos=qp)
    got = sa.dsa_indexer_topk(tqi, tki, tw, kk, q_pos=qp)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert bool((got[0, :, :-1] < got[0, :, 1:]).all())  # ascending, no padding


def test_indexer_topk_query_blocks_equal_whole_call():
    """A prefill run in query blocks (per-batch q_pos = the block's first position, a workspace sized for the
    block) writes exactly the whole call's indices: rows are independent."""
    sa = require_gpu()
    B, T, S, kk, blk = 2, 4096, 4096, 2048, 1536
    g = torch.Generator(device=DEV)
    g.manual_seed(97)
    qi = (torch.randn((B, T, 4, 128), generator=g, device=DEV) * 128 ** -0.5).to(torch.bfloat16)
    ki = (torch.randn((B, S, 128), generator=g, device=DEV) * 128 ** -0.5).to(torch.bfloat16)
    w = torch.rand((B, T, 4), generator=g, device=DEV)
    whole = sa.dsa_indexer_topk(qi, ki, w, kk)
    for o in range(0, T, blk):
        e = min(T, o + blk)
        qp = torch.full((B,), o, dtype=torch.int64, device=DEV)
        part = sa.dsa_indexer_topk(qi[:, o:e].contiguous(), ki, w[:, o:e].contiguous(), kk, q_pos=qp)
        torch.cuda.synchronize()
        assert torch.equal(part, whole[:, o:e]), o


def test_indexer_topk_32768_top2048():
    """Fused call at the prefill workload's size: identical to the separate calls on every row, and on
    sampled rows equal to the oracle's selection outside the 1e-6 tie band."""
    sa = require_gpu()
    T, kk = 32768, 2048
    qi = synth.torch_normal((1, T, 4, 128), 128 ** -0.5, torch.bfloat16, 1700, DEV)
    ki = synth.torch_normal((1, T, 128), 128 ** -0.5, torch.bfloat16, 1701, DEV)
    w = synth.torch_uniform((1, T, 4), 1702, DEV)
    got = sa.dsa_indexer_topk(qi, ki, w, kk)
    sc = sa.dsa_indexer_scores(qi, ki, w)
    want = sa.dsa_topk(sc, kk)
    assert torch.equal(got, want)
    del sc
    for i in (2047, 2048, 5000, 20000, T - 1):
        n = i + 1
        ws = oracle.dsa_indexer_scores(f64(qi[:, i:i + 1]), f64(ki[:, :n]), f64(w[:, i:i + 1]), q_pos=[i])[0, 0]
        kth = np.sort(ws)[::-1][kk - 1]
        band = np.abs(ws - kth) <= 1e-6
        sel = set(got[0, i].cpu().numpy().tolist()) - {-1}
        want_sel = set(np.argsort(-ws, kind="stable")[:kk].tolist())
        assert {s_ for s_ in sel if not band[s_]} == {s_ for s_ in want_sel if not band[s_]}, i


# ---------------------------------------------------------------------------
# CSA variant: indexer, top-k and sparse attention over block-mean entries
# ---------------------------------------------------------------------------


def _csa_mask(B, T, S, q_pos, ratio):
    m = np.zeros((B, T, S), dtype=bool)
    for b in range(B):
        base = 0 if q_pos is None else q_pos[b]
        for i in range(T):
            m[b, i, : oracle.n_candidates(base + i, ratio, S)] = True
    return m


@pytest.mark.parametrize("B,T,ratio,q_pos,kk", [(1, 700, 4, None, 64), (2, 130, 2, [400, 0], 100),
                                                (1, 300, 16, [2000], 8), (1, 1, 4, [5003], 2048),
                                                (1, 9, 4, None, 4)])
def test_csa_indexer_and_topk(B, T, ratio, q_pos, kk):
    """GPU CSA scores within fp32 rounding of the oracle, only over visible entries; GPU top-k on those
    scores bit-exact against the oracle's selection rule with the same ratio."""
    sa = require_gpu()
    L = T + (0 if q_pos is None else max(q_pos))
    S = L // ratio
    qi, ki_tok, w = _indexer_inputs(B, T, L, 60 + T + ratio)
    ki_tok = ki_tok[:, : S * ratio]
    kc = sa.hca_compress(synth.to_torch(ki_tok, "bf16", DEV)[:, None], ratio)[:, 0]
    qp = None if q_pos is None else torch.tensor(q_pos, dtype=torch.int64, device=DEV)
    sc = sa.csa_indexer_scores(synth.to_torch(qi, "bf16", DEV), kc.contiguous(), synth.to_torch(w, "f32", DEV),
                               ratio, q_pos=qp)
    want = oracle.dsa_indexer_scores(qi, f64(kc), w, q_pos=q_pos, ratio=ratio)
    m = _csa_mask(B, T, S, q_pos, ratio)
    assert np.array_equal(np.isfinite(want), m)
    assert np.max(np.abs(f64(sc)[m] - want[m]), initial=0.0) <= 2e-6
    idx = sa.csa_topk(sc, kk, ratio, q_pos=qp)
    sc_np = np.where(m, sc.cpu().numpy(), np.nan)
    assert np.array_equal(idx.cpu().numpy(), oracle.dsa_topk(sc_np, kk, q_pos=q_pos, ratio=ratio))


def test_csa_layer():
    """Whole CSA layer on the GPU (block-4 means of k_I, K, V; indexer; top-k; sparse attention)
    against the oracle: selection bit-exact on the GPU's scores, attention on the GPU's entries and
    cache within 2e-2, and the rows that see no complete block give o = 0, lse = -inf."""
    sa = require_gpu()
    B, T, ratio, kk = 1, 900, 4, 128
    qi, ki, w = _indexer_inputs(B, T, T, 70)
    q = synth.np_normal((B, T, 64, 256), 1.0, "bf16", 71, 0)
    k = synth.np_normal((B, T, 256), 1.0, "bf16", 71, 1)
    v = synth.np_normal((B, T, 256), 1.0, "bf16", 71, 2)
    t = {n: synth.to_torch(a, "bf16", DEV) for n, a in (("ki", ki), ("q", q), ("k", k), ("v", v))}
    kci = sa.hca_compress(t["ki"][:, None], ratio)[:, 0].contiguous()
    kc = sa.hca_compress(t["k"][:, None], ratio)[:, 0].contiguous()
    vc = sa.hca_compress(t["v"][:, None], ratio)[:, 0].contiguous()
    sc = sa.csa_indexer_scores(synth.to_torch(qi, "bf16", DEV), kci, synth.to_torch(w, "f32", DEV), ratio)
    idx = sa.csa_topk(sc, kk, ratio)
    o, lse = sa.dsa_sparse_attention_fwd(t["q"], kc, vc, idx, return_lse=True)
    S = T // ratio
    m = _csa_mask(B, T, S, None, ratio)
    sc_np = np.where(m, sc.cpu().numpy(), np.nan)
    got_idx = idx.cpu().numpy().astype(np.int64)
    assert np.array_equal(got_idx, oracle.dsa_topk(sc_np, kk, ratio=ratio))
    ow, lw = oracle.dsa_sparse_attention(q, f64(kc), f64(vc), got_idx)
    assert max_abs_err(f64(o), ow) <= BF16_ABS_TOL
    fin = np.isfinite(lw)
    assert np.array_equal(fin, np.isfinite(f64(lse)))
    assert np.max(np.abs(f64(lse)[fin] - lw[fin])) <= 1e-2
    assert not fin[0, : ratio - 1].any() and fin[0, ratio - 1:].all()


def test_csa_topk_causal_row_classes():
    """Long causal CSA rows: with ratio 4 the rows split over the workgroup sizes at entry counts
    8192 and 16384, i.e. token rows 32767 and 65539; rows on both sides of the first cut."""
    sa = require_gpu()
    T, ratio, k = 40000, 4, 2048
    S = T // ratio
    sc = synth.torch_normal((1, T, S), 1.0, torch.float32, 72, DEV)
    idx = sa.csa_topk(sc, k, ratio)
    torch.cuda.synchronize()
    for i in [0, 2, 3, 8194, 8195, 20000, 32766, 32767, 32768, T - 1]:
        n = oracle.n_candidates(i, ratio, S)
        row = sc[0, i, :n].cpu().numpy()
        want = oracle.dsa_topk(row.reshape(1, 1, -1), k, q_pos=[n - 1])[0, 0] if n > 0 else np.full(k, -1)
        assert np.array_equal(idx[0, i].cpu().numpy(), want), i

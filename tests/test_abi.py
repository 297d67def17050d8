"""C ABI on the CPU: the library loads, exports every symbol the header declares, and rejects
invalid arguments with the documented status codes before touching the GPU."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn_hca.h")

SA_OK, SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_UNSUPPORTED, SA_ERR_ALIGN, SA_ERR_WORKSPACE = 0, -1, -2, -3, -4, -5


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def sa():
    import sparse_attention_long_hca_amd as pkg

    if not os.path.exists(pkg.LIB_PATH):
        pytest.fail(f"library not built: {pkg.LIB_PATH}")
    return pkg


def test_header_declares_the_five_calls():
    names = _declared_functions()
    for n in ["hca_compress", "hca_attention_fwd", "dsa_indexer_scores", "dsa_topk", "dsa_sparse_attention_fwd"]:
        assert n in names, names


def test_library_exports_every_declared_symbol(sa):
    lib = ctypes.CDLL(sa.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol(sa):
    from sparse_attention_long_hca_amd import _lib

    missing = [n for n in _declared_functions() if n not in _lib.EXPORTS]
    assert not missing, missing


def test_version(sa):
    assert "gfx950" in sa.version()


def _hca_args(**kw):
    from sparse_attention_long_hca_amd._lib import HcaAttentionArgs

    a = HcaAttentionArgs()
    a.mode, a.dtype = 0, 1
    a.B, a.H, a.d, a.blk, a.window, a.seq_len, a.n_c_cap = 1, 1, 512, 128, 128, 256, 2
    a.q = a.k = a.v = a.k_c = a.v_c = a.o = 4096
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(q=None), SA_ERR_NULL),
        (dict(B=0), SA_ERR_SHAPE),
        (dict(seq_len=0), SA_ERR_SHAPE),
        (dict(d=128), SA_ERR_UNSUPPORTED),
        (dict(dtype=0), SA_ERR_UNSUPPORTED),
        (dict(n_c_cap=3), SA_ERR_SHAPE),
        (dict(q=4100), SA_ERR_ALIGN),
        (dict(mode=1, pos=None), SA_ERR_NULL),
        (dict(mode=1, pos=4096, workspace=None, workspace_bytes=0, B=1, H=1, n_c_cap=100000), SA_ERR_WORKSPACE),
        (dict(mode=7), SA_ERR_SHAPE),
        (dict(d=576, d_v=576), SA_ERR_UNSUPPORTED),
        (dict(d=512, d_v=256), SA_ERR_UNSUPPORTED),
        (dict(d=576, d_v=512, dtype=0), SA_ERR_UNSUPPORTED),
        (dict(d=576, d_v=-1), SA_ERR_SHAPE),
        (dict(mode=1, pos=4096, d=576, d_v=576), SA_ERR_UNSUPPORTED),
        (dict(mode=1, pos=4096, d=64, d_v=64, dtype=0), SA_ERR_UNSUPPORTED),
    ],
)
def test_hca_attention_validation(sa, kw, code):
    a = _hca_args(**kw)
    assert sa.lib().hca_attention_fwd(ctypes.byref(a), None) == code
    assert sa.lib().sa_last_error().decode()


def test_hca_decode_workspace_size_positive(sa):
    a = _hca_args(mode=1, B=4, H=64, n_c_cap=8192)
    n = sa.lib().hca_attention_fwd_workspace_size(ctypes.byref(a))
    assert n > 0
    # the split partials hold value-width rows: qk 576 / v 512 needs the same workspace
    a = _hca_args(mode=1, B=4, H=64, n_c_cap=8192, d=576, d_v=512)
    assert sa.lib().hca_attention_fwd_workspace_size(ctypes.byref(a)) == n
    a = _hca_args(mode=0)
    assert sa.lib().hca_attention_fwd_workspace_size(ctypes.byref(a)) == 0


def test_compress_validation(sa):
    L = sa.lib()
    assert L.hca_compress(None, 4096, 1, 1, 1, 256, 512, 128, 0, 0, 512, 0, 0, 512, None) == SA_ERR_NULL
    assert L.hca_compress(None, None, 1, 1, 1, 100, 512, 128, 0, 0, 512, 0, 0, 512, None) == SA_OK
    assert L.hca_compress(4096, 4096, 1, 1, 1, 256, 500, 128, 0, 0, 500, 0, 0, 500, None) == SA_ERR_UNSUPPORTED
    assert L.hca_compress(4096, 4096, 1, 1, 1, 256, 512, 0, 0, 0, 512, 0, 0, 512, None) == SA_ERR_SHAPE
    assert L.hca_compress(4100, 4096, 1, 1, 1, 256, 512, 128, 0, 0, 512, 0, 0, 512, None) == SA_ERR_ALIGN
    assert L.hca_compress(4096, 4096, 1, 1, 1, 256, 512, 128, 0, 0, 513, 0, 0, 512, None) == SA_ERR_ALIGN
    assert L.hca_compress(4096, 4096, 9, 1, 1, 256, 512, 128, 0, 0, 512, 0, 0, 512, None) == SA_ERR_UNSUPPORTED
    # fewer tokens than one block: nothing to do, OK without touching the GPU
    assert L.hca_compress(4096, 4096, 1, 1, 1, 100, 512, 128, 0, 0, 512, 0, 0, 512, None) == SA_OK


def test_indexer_validation(sa):
    L = sa.lib()
    assert L.dsa_indexer_scores(None, 4096, 4096, None, 4096, 1, 4, 4, 4, 128, None) == SA_ERR_NULL
    assert L.dsa_indexer_scores(4096, 4096, 4096, None, 4096, 1, 4, 4, 8, 128, None) == SA_ERR_UNSUPPORTED
    assert L.dsa_indexer_scores(4096, 4096, 4096, None, 4096, 1, 0, 4, 4, 128, None) == SA_ERR_SHAPE
    assert L.dsa_indexer_scores(4096, 4104, 4096, None, 4096, 1, 4, 4, 4, 128, None) == SA_ERR_ALIGN


def test_topk_validation(sa):
    L = sa.lib()
    assert L.dsa_topk(None, None, 4096, 1, 4, 4, 2, None, 0, None) == SA_ERR_NULL
    assert L.dsa_topk(4096, None, 4096, 1, 4, 4, 4096, None, 0, None) == SA_ERR_UNSUPPORTED
    assert L.dsa_topk(4096, None, 4096, 1, 4, 0, 2, None, 0, None) == SA_ERR_SHAPE
    # long rows need a workspace
    assert L.dsa_topk_workspace_size(4, 1, 1 << 20, 2048) > 0
    assert L.dsa_topk_workspace_size(1, 32768, 32768, 2048) == 0
    assert L.dsa_topk(4096, None, 4096, 4, 1, 1 << 20, 2048, None, 0, None) == SA_ERR_WORKSPACE


def test_sparse_attention_validation(sa):
    L = sa.lib()
    # q, k, v, idx, o, lse, dtype, B, T, S, Hq, D, kk, scale, workspace, workspace_bytes, stream
    # (never called with valid arguments on the CPU)
    args = [4096] * 5 + [None, 1, 1, 4, 16, 64, 256, 32, 0.0, None, 0, None]
    bad = list(args)
    bad[0] = None
    assert L.dsa_sparse_attention_fwd(*bad) == SA_ERR_NULL
    bad = list(args)
    bad[11] = 128  # D
    assert L.dsa_sparse_attention_fwd(*bad) == SA_ERR_UNSUPPORTED
    bad = list(args)
    bad[12] = 4096  # kk
    assert L.dsa_sparse_attention_fwd(*bad) == SA_ERR_UNSUPPORTED
    bad = list(args)
    bad[7] = 0  # T
    assert L.dsa_sparse_attention_fwd(*bad) == SA_ERR_SHAPE
    # decode-sized calls (few tokens) need a workspace for the split partials
    assert L.dsa_sparse_attention_fwd_workspace_size(4, 1, 64, 256, 2048) > 0
    assert L.dsa_sparse_attention_fwd_workspace_size(1, 32768, 64, 256, 2048) == 0
    dec = list(args)
    dec[12] = 2048  # kk: a 4-token call with 2048 indices is split and needs a workspace
    assert L.dsa_sparse_attention_fwd(*dec) == SA_ERR_WORKSPACE


def test_quantize_fp8_validation(sa):
    L = sa.lib()
    assert L.hca_quantize_fp8(None, 4096, 4096, 4, 512, None) == SA_ERR_NULL
    assert L.hca_quantize_fp8(4096, 4096, 4096, 4, 500, None) == SA_ERR_UNSUPPORTED
    assert L.hca_quantize_fp8(4096, 4096, 4096, -1, 512, None) == SA_ERR_SHAPE
    assert L.hca_quantize_fp8(4100, 4096, 4096, 4, 512, None) == SA_ERR_ALIGN
    # no rows: nothing to do, OK without touching the GPU
    assert L.hca_quantize_fp8(None, None, None, 0, 512, None) == SA_OK


def _fp8_args(**kw):
    from sparse_attention_long_hca_amd._lib import HcaDecodeFp8Args

    a = HcaDecodeFp8Args()
    a.B, a.H, a.d, a.blk, a.window, a.n_c_cap = 1, 1, 512, 128, 128, 2
    for f in ("q", "k_c", "k_c_scale", "v_c", "v_c_scale", "k", "k_scale", "v", "v_scale", "pos", "o"):
        setattr(a, f, 4096)
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(q=None), SA_ERR_NULL),
        (dict(k_scale=None), SA_ERR_NULL),
        (dict(pos=None), SA_ERR_NULL),
        (dict(B=0), SA_ERR_SHAPE),
        (dict(n_c_cap=0), SA_ERR_SHAPE),
        (dict(d=256), SA_ERR_UNSUPPORTED),
        (dict(v_c_scale=4100), SA_ERR_ALIGN),
        (dict(B=4, H=64, n_c_cap=8192, workspace=None, workspace_bytes=0), SA_ERR_WORKSPACE),
    ],
)
def test_decode_fp8_validation(sa, kw, code):
    a = _fp8_args(**kw)
    assert sa.lib().hca_decode_fp8(ctypes.byref(a), None) == code
    assert sa.lib().sa_last_error().decode()


def test_decode_fp8_workspace_matches_bf16_decode(sa):
    a = _fp8_args(B=4, H=64, n_c_cap=8192)
    b = _hca_args(mode=1, B=4, H=64, n_c_cap=8192)
    assert sa.lib().hca_decode_fp8_workspace_size(ctypes.byref(a)) == sa.lib().hca_attention_fwd_workspace_size(
        ctypes.byref(b)) > 0


def test_csa_validation(sa):
    L = sa.lib()
    assert L.csa_indexer_scores(4096, 4096, 4096, None, 4096, 1, 4, 4, 4, 128, 0, None) == SA_ERR_SHAPE
    assert L.csa_indexer_scores(None, 4096, 4096, None, 4096, 1, 4, 4, 4, 128, 4, None) == SA_ERR_NULL
    assert L.csa_indexer_scores(4096, 4096, 4096, None, 4096, 1, 4, 4, 8, 128, 4, None) == SA_ERR_UNSUPPORTED
    assert L.csa_topk(4096, None, 4096, 1, 4, 4, 2, 0, None, 0, None) == SA_ERR_SHAPE
    assert L.csa_topk(None, None, 4096, 1, 4, 4, 2, 4, None, 0, None) == SA_ERR_NULL
    assert L.csa_topk(4096, None, 4096, 4, 1, 1 << 20, 2048, 4, None, 0, None) == SA_ERR_WORKSPACE


def test_indexer_topk_validation(sa):
    L = sa.lib()
    ws = 4096
    big = 1 << 40
    # null, shape, unsupported, alignment, workspace
    assert L.dsa_indexer_topk(None, 4096, 4096, None, 4096, 1, 4, 4, 4, 128, 2, 0, ws, big, None) == SA_ERR_NULL
    assert L.dsa_indexer_topk(4096, 4096, 4096, None, 4096, 1, 0, 4, 4, 128, 2, 0, ws, big, None) == SA_ERR_SHAPE
    # rows longer than 32768 positions: decode shapes only (T <= 4), up to 2^24 positions
    assert L.dsa_indexer_topk(4096, 4096, 4096, None, 4096, 1, 5, 40000, 4, 128, 2, 0, ws, big, None) == SA_ERR_UNSUPPORTED
    assert L.dsa_indexer_topk(4096, 4096, 4096, None, 4096, 1, 1, (1 << 24) + 1, 4, 128, 2, 0, ws, big, None) == SA_ERR_UNSUPPORTED
    assert L.dsa_indexer_topk(4096, 4096, 4096, None, 4096, 1, 4, 40000, 4, 128, 2, 0, ws, 1, None) == SA_ERR_WORKSPACE
    assert L.dsa_indexer_topk(4096, 4096, 4096, None, 4096, 1, 4, 4, 4, 128, 4096, 0, ws, big, None) == SA_ERR_UNSUPPORTED
    assert L.dsa_indexer_topk(4096, 4096, 4096, None, 4096, 1, 4, 4, 8, 128, 2, 0, ws, big, None) == SA_ERR_UNSUPPORTED
    assert L.dsa_indexer_topk(4100, 4096, 4096, None, 4096, 1, 4, 4, 4, 128, 2, 0, ws, big, None) == SA_ERR_ALIGN
    assert L.dsa_indexer_topk(4096, 4096, 4096, None, 4096, 1, 4, 4, 4, 128, 2, 0, None, 0, None) == SA_ERR_WORKSPACE
    need = L.dsa_indexer_topk_workspace_size(1, 4, 4, 2)
    assert need > 0
    assert L.dsa_indexer_topk(4096, 4096, 4096, None, 4096, 1, 4, 4, 4, 128, 2, 0, ws, need - 1, None) == SA_ERR_WORKSPACE
    # the workspace holds a candidate slot (8 bytes) per row and position; the
    # recomputed rows' scores reuse that area
    assert L.dsa_indexer_topk_workspace_size(1, 32768, 32768, 2048) >= 32768 * 32768 * 8
    # decode-shaped long rows keep candidates per 128-position chunk and the full scores for recomputed rows
    assert L.dsa_indexer_topk_workspace_size(4, 1, 1 << 20, 2048) >= 4 * (1 << 20) * 4


def test_sparse_attention_bwd_validation(sa):
    L = sa.lib()
    # q, k, v, idx, o, lse, d_o, dq, dk, dv, dtype, B, T, S, Hq, D, kk, scale, workspace, bytes, stream
    # (never called with valid arguments on the CPU: the workspace check comes last)
    args = [4096] * 10 + [1, 1, 4, 16, 64, 256, 32, 0.0, 4096, 0, None]
    for i in range(10):
        bad = list(args)
        bad[i] = None
        assert L.dsa_sparse_attention_bwd(*bad) == SA_ERR_NULL
    for i, val, err in ((15, 128, SA_ERR_UNSUPPORTED), (14, 32, SA_ERR_UNSUPPORTED), (16, 4096, SA_ERR_UNSUPPORTED),
                        (10, 0, SA_ERR_UNSUPPORTED), (12, 0, SA_ERR_SHAPE), (13, 0, SA_ERR_SHAPE),
                        (13, (1 << 23) + 1, SA_ERR_UNSUPPORTED), (7, 4100, SA_ERR_ALIGN)):
        bad = list(args)
        bad[i] = val
        assert L.dsa_sparse_attention_bwd(*bad) == err, (i, val)
    need = L.dsa_sparse_attention_bwd_workspace_size(1, 4, 16, 32)
    assert need > 0
    assert L.dsa_sparse_attention_bwd(*args) == SA_ERR_WORKSPACE
    # at 32768 tokens x top-2048, per chunk of 2048 tokens: bf16 per-entry dk and dv rows (2 x 2 GiB), the
    # P and dS blocks (1 GiB) and the index
    ws = L.dsa_sparse_attention_bwd_workspace_size(1, 32768, 32768, 2048)
    assert 2 * 2048 * 2048 * 256 * 2 + 2048 * 2048 * 64 * 4 <= ws < 5.1 * 2 ** 30

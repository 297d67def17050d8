"""ctypes binding of libsparse_attn_hca.so (argument marshalling only).

Every function here validates nothing beyond what is needed to build the C
call (tensor device/dtype/contiguity), allocates outputs with torch (device
memory is the only thing torch provides), and calls the C entry point of the
same name on the current torch stream.  All computation happens in the HIP
kernels; if the library is missing the call fails loudly.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libsparse_attn_hca.so")

SA_F32, SA_BF16 = 0, 1
HCA_PREFILL, HCA_DECODE = 0, 1

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p


class HcaAttentionArgs(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("B", _c_i64),
        ("H", _c_i64),
        ("d", _c_i64),
        ("blk", _c_i64),
        ("window", _c_i64),
        ("seq_len", _c_i64),
        ("n_c_cap", _c_i64),
        ("scale", ctypes.c_float),
        ("q", _c_p),
        ("k", _c_p),
        ("v", _c_p),
        ("k_c", _c_p),
        ("v_c", _c_p),
        ("pos", _c_p),
        ("o", _c_p),
        ("lse", _c_p),
        ("workspace", _c_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("d_v", _c_i64),
    ]


class HcaDecodeFp8Args(ctypes.Structure):
    _fields_ = [
        ("B", _c_i64),
        ("H", _c_i64),
        ("d", _c_i64),
        ("blk", _c_i64),
        ("window", _c_i64),
        ("n_c_cap", _c_i64),
        ("scale", ctypes.c_float),
        ("q", _c_p),
        ("k_c", _c_p),
        ("k_c_scale", _c_p),
        ("v_c", _c_p),
        ("v_c_scale", _c_p),
        ("k", _c_p),
        ("k_scale", _c_p),
        ("v", _c_p),
        ("v_scale", _c_p),
        ("pos", _c_p),
        ("o", _c_p),
        ("lse", _c_p),
        ("workspace", _c_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class HcaAttentionBwdArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("B", _c_i64),
        ("H", _c_i64),
        ("d", _c_i64),
        ("blk", _c_i64),
        ("window", _c_i64),
        ("seq_len", _c_i64),
        ("n_c", _c_i64),
        ("through_compress", _c_i64),
        ("scale", ctypes.c_float),
        ("q", _c_p),
        ("k", _c_p),
        ("v", _c_p),
        ("k_c", _c_p),
        ("v_c", _c_p),
        ("o", _c_p),
        ("d_o", _c_p),
        ("lse", _c_p),
        ("dq", _c_p),
        ("dk", _c_p),
        ("dv", _c_p),
        ("dk_c", _c_p),
        ("dv_c", _c_p),
        ("workspace", _c_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class SparseAttnError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None

EXPORTS = {
    "sa_last_error": (ctypes.c_char_p, []),
    "sa_version": (ctypes.c_char_p, []),
    "hca_compress": (ctypes.c_int, [_c_p, _c_p, ctypes.c_int] + [_c_i64] * 11 + [_c_p]),
    "hca_attention_fwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(HcaAttentionArgs)]),
    "hca_attention_fwd": (ctypes.c_int, [ctypes.POINTER(HcaAttentionArgs), _c_p]),
    "hca_attention_fwd_noalloc": (ctypes.c_int, [ctypes.POINTER(HcaAttentionArgs), _c_p]),
    "hca_attention_bwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(HcaAttentionBwdArgs)]),
    "hca_attention_bwd": (ctypes.c_int, [ctypes.POINTER(HcaAttentionBwdArgs), _c_p]),
    "hca_quantize_fp8": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_p]),
    "hca_decode_fp8_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(HcaDecodeFp8Args)]),
    "hca_decode_fp8": (ctypes.c_int, [ctypes.POINTER(HcaDecodeFp8Args), _c_p]),
    "dsa_indexer_scores": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p] + [_c_i64] * 5 + [_c_p]),
    "csa_indexer_scores": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p] + [_c_i64] * 6 + [_c_p]),
    "csa_topk": (ctypes.c_int, [_c_p, _c_p, _c_p] + [_c_i64] * 5 + [_c_p, ctypes.c_size_t, _c_p]),
    "dsa_topk_workspace_size": (ctypes.c_size_t, [_c_i64] * 4),
    "dsa_indexer_topk_workspace_size": (ctypes.c_size_t, [_c_i64] * 4),
    "dsa_indexer_topk": (ctypes.c_int, [_c_p] * 5 + [_c_i64] * 7 + [_c_p, ctypes.c_size_t, _c_p]),
    "dsa_topk": (ctypes.c_int, [_c_p, _c_p, _c_p] + [_c_i64] * 4 + [_c_p, ctypes.c_size_t, _c_p]),
    "dsa_sparse_attention_fwd_workspace_size": (ctypes.c_size_t, [_c_i64] * 5),
    "dsa_sparse_attention_fwd": (
        ctypes.c_int,
        [_c_p] * 6 + [ctypes.c_int] + [_c_i64] * 6 + [ctypes.c_float, _c_p, ctypes.c_size_t, _c_p],
    ),
    "dsa_sparse_attention_bwd_workspace_size": (ctypes.c_size_t, [_c_i64] * 4),
    "dsa_sparse_attention_bwd": (
        ctypes.c_int,
        [_c_p] * 10 + [ctypes.c_int] + [_c_i64] * 6 + [ctypes.c_float, _c_p, ctypes.c_size_t, _c_p],
    ),
}


def lib():
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m sparse_attention_long_hca_amd.build`"
            )
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise SparseAttnError(fn, status, lib().sa_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.float32:
        return SA_F32
    if t.dtype == torch.bfloat16:
        return SA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, dtype=None, dim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got {t.dim()}")


def _shape(t, name, shape):
    """The C ABI takes sizes, not shapes: a tensor of the wrong shape would be read or written out of bounds."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def version():
    return lib().sa_version().decode()


# ---------------------------------------------------------------------------
def hca_compress(x, blk, out=None):
    """Block mean of K or V: x [B,H,T,d] -> [B,H,T//blk,d] (same dtype)."""
    _need(x, "x", dim=4)
    B, H, T, d = x.shape
    n = T // blk
    if out is None:
        out = torch.empty((B, H, n, d), dtype=x.dtype, device=x.device)
    if out.dim() != 4 or out.stride(-1) != 1:
        raise ValueError("out must be [B,H,n,d] with a contiguous last dim")
    _shape(out, "out", (B, H, n, d))
    st = _check(
        "hca_compress",
        lib().hca_compress(
            _ptr(x), _ptr(out), _dtype_code(x), B, H, T, d, blk,
            x.stride(0), x.stride(1), x.stride(2), out.stride(0), out.stride(1), out.stride(2),
            _stream(),
        ),
    )
    return out


def _hca_args(mode, q, k, v, k_c, v_c, blk, window, seq_len, n_c_cap, scale, pos, o, lse, ws, ws_bytes):
    a = HcaAttentionArgs()
    a.mode = mode
    a.dtype = _dtype_code(q)
    a.B, a.H, a.d = q.shape[0], q.shape[1], q.shape[-1]
    a.blk, a.window, a.seq_len, a.n_c_cap = blk, window, seq_len, n_c_cap
    a.scale = 0.0 if scale is None else float(scale)
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.k_c = k_c.data_ptr() if k_c is not None else None
    a.v_c = v_c.data_ptr() if v_c is not None else None
    a.pos = pos.data_ptr() if pos is not None else None
    a.o = o.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    a.workspace = ws.data_ptr() if ws is not None else None
    a.workspace_bytes = ws_bytes
    a.d_v = v.shape[-1]
    return a


def hca_attention_fwd(mode, q, k, v, k_c, v_c, blk, window, scale=None, pos=None, return_lse=False, workspace=None,
                      _noalloc=False):
    """HCA attention.

    d is the query/key width (q, k, k_c), dv the value width (v, v_c, o); dv < d
    for the qk 576 / v 512 shape.
    PREFILL: q,k [B,H,T,d], v [B,H,T,dv]; k_c [B,H,Nc,d], v_c [B,H,Nc,dv].
             Returns o [B,H,T,dv] (and lse [B,H,T]).
    DECODE:  q [B,H,d]; k_c [B,H,Ncap,d], v_c [B,H,Ncap,dv]; k,v = window ring
             [B,H,window,d] / [B,H,window,dv]; pos int64 [B] on the device.
             Returns o [B,H,dv] (and lse [B,H]).
    """
    for name, t in (("q", q), ("k", k), ("v", v), ("k_c", k_c), ("v_c", v_c)):
        _need(t, name, dtype=q.dtype)
    d, dv = q.shape[-1], v.shape[-1]
    if mode == HCA_PREFILL:
        B, H, T, _ = q.shape
        seq_len, n_c = T, k_c.shape[2]
        want = {"k": (B, H, T, d), "v": (B, H, T, dv), "k_c": (B, H, n_c, d), "v_c": (B, H, n_c, dv)}
        o_shape = (B, H, T, dv)
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if return_lse else None
    elif mode == HCA_DECODE:
        _need(pos, "pos", dtype=torch.int64, dim=1)
        B, H, _ = q.shape
        seq_len, n_c = 0, k_c.shape[2]
        want = {"k": (B, H, window, d), "v": (B, H, window, dv), "k_c": (B, H, n_c, d), "v_c": (B, H, n_c, dv)}
        if tuple(pos.shape) != (B,):
            raise ValueError(f"pos must have shape ({B},)")
        o_shape = (B, H, dv)
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if return_lse else None
    else:
        raise ValueError("mode must be HCA_PREFILL or HCA_DECODE")
    for name, t in (("k", k), ("v", v), ("k_c", k_c), ("v_c", v_c)):
        if tuple(t.shape) != want[name]:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want[name]}")
    o = torch.empty(o_shape, dtype=q.dtype, device=q.device)
    args = _hca_args(mode, q, k, v, k_c, v_c, blk, window, seq_len, n_c, scale, pos, o, lse, None, 0)
    if _noalloc:
        _check("hca_attention_fwd_noalloc", lib().hca_attention_fwd_noalloc(ctypes.byref(args), _stream()))
        return (o, lse) if return_lse else o
    need = lib().hca_attention_fwd_workspace_size(ctypes.byref(args))
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel() * workspace.element_size()
    _check("hca_attention_fwd", lib().hca_attention_fwd(ctypes.byref(args), _stream()))
    return (o, lse) if return_lse else o


def hca_attention_fwd_noalloc(mode, q, k, v, k_c, v_c, blk, window, scale=None, pos=None, return_lse=False):
    """hca_attention_fwd through the allocation-free entry point: the library's static scratch holds the
    decode split partials (the outputs o and lse are still allocated here, by torch)."""
    return hca_attention_fwd(mode, q, k, v, k_c, v_c, blk, window, scale=scale, pos=pos, return_lse=return_lse,
                             _noalloc=True)


def hca_attention_workspace_size(mode, q, k_c, blk, window):
    a = HcaAttentionArgs()
    a.mode, a.dtype = mode, _dtype_code(q)
    a.B, a.H, a.d = q.shape[0], q.shape[1], q.shape[-1]
    a.blk, a.window, a.n_c_cap = blk, window, k_c.shape[2]
    return lib().hca_attention_fwd_workspace_size(ctypes.byref(a))


def hca_attention_bwd(q, k, v, k_c, v_c, o, lse, do, blk, window, scale=None, through_compress=True, workspace=None):
    """Gradients of HCA prefill: q, k, v, o, do [B,H,T,d] bf16; k_c, v_c [B,H,Nc,d] bf16; lse [B,H,T] fp32
    (o and lse from hca_attention_fwd).  Returns (dq, dk, dv, dk_c, dv_c), fp32; with through_compress dk and
    dv include the block mean's path (dk_c/blk, dv_c/blk on every token of a complete block)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("k_c", k_c), ("v_c", v_c), ("o", o), ("do", do)):
        _need(t, name, dtype=q.dtype)
    _need(lse, "lse", dtype=torch.float32)
    B, H, T, d = q.shape
    n_c = k_c.shape[2]
    for name, t, shp in (("k", k, (B, H, T, d)), ("v", v, (B, H, T, d)), ("o", o, (B, H, T, d)), ("do", do, (B, H, T, d)),
                         ("k_c", k_c, (B, H, n_c, d)), ("v_c", v_c, (B, H, n_c, d)), ("lse", lse, (B, H, T))):
        _shape(t, name, shp)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty((B, H, T, d), **f32), torch.empty((B, H, T, d), **f32), torch.empty((B, H, T, d), **f32)
    dkc, dvc = torch.empty((B, H, n_c, d), **f32), torch.empty((B, H, n_c, d), **f32)
    a = HcaAttentionBwdArgs()
    a.dtype = _dtype_code(q)
    a.B, a.H, a.d, a.blk, a.window, a.seq_len, a.n_c = B, H, d, blk, window, T, n_c
    a.through_compress = 1 if through_compress else 0
    a.scale = 0.0 if scale is None else float(scale)
    a.q, a.k, a.v, a.o, a.d_o, a.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr()
    a.k_c = k_c.data_ptr() if n_c > 0 else None
    a.v_c = v_c.data_ptr() if n_c > 0 else None
    a.dq, a.dk, a.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    a.dk_c = dkc.data_ptr() if n_c > 0 else None
    a.dv_c = dvc.data_ptr() if n_c > 0 else None
    need = lib().hca_attention_bwd_workspace_size(ctypes.byref(a))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    a.workspace = workspace.data_ptr()
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    _check("hca_attention_bwd", lib().hca_attention_bwd(ctypes.byref(a), _stream()))
    return dq, dk, dv, dkc, dvc


def hca_attention_bwd_workspace_size(B, H, T, n_c, window):
    a = HcaAttentionBwdArgs()
    a.dtype, a.B, a.H, a.d, a.blk, a.window, a.seq_len, a.n_c = SA_BF16, B, H, 512, 1, window, T, n_c
    return lib().hca_attention_bwd_workspace_size(ctypes.byref(a))


def hca_quantize_fp8(x, codes=None, scales=None):
    """bf16 rows x [..., d] -> (E4M3 codes uint8 [..., d], fp32 scales [...]), one scale per row."""
    _need(x, "x", torch.bfloat16)
    d = x.shape[-1]
    rows = x.numel() // d if d > 0 else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _need(codes, "codes", torch.uint8)
    _need(scales, "scales", torch.float32)
    _shape(codes, "codes", x.shape)
    _shape(scales, "scales", x.shape[:-1])
    _check("hca_quantize_fp8", lib().hca_quantize_fp8(_ptr(x), _ptr(codes), _ptr(scales), rows, d, _stream()))
    return codes, scales


def _fp8_args(q, k, k_scale, v, v_scale, k_c, k_c_scale, v_c, v_c_scale, blk, window, scale, pos, o, lse):
    a = HcaDecodeFp8Args()
    a.B, a.H, a.d = q.shape
    a.blk, a.window, a.n_c_cap = blk, window, k_c.shape[2]
    a.scale = 0.0 if scale is None else float(scale)
    a.q = q.data_ptr()
    a.k_c, a.k_c_scale, a.v_c, a.v_c_scale = k_c.data_ptr(), k_c_scale.data_ptr(), v_c.data_ptr(), v_c_scale.data_ptr()
    a.k, a.k_scale, a.v, a.v_scale = k.data_ptr(), k_scale.data_ptr(), v.data_ptr(), v_scale.data_ptr()
    a.pos = pos.data_ptr()
    a.o = None if o is None else o.data_ptr()
    a.lse = None if lse is None else lse.data_ptr()
    return a


def hca_decode_fp8(q, k, k_scale, v, v_scale, k_c, k_c_scale, v_c, v_c_scale, blk, window, pos, scale=None,
                   return_lse=False, workspace=None):
    """HCA decode over an E4M3 cache: q [B,H,d] bf16; k,v window-ring codes [B,H,window,d] uint8 with
    scales [B,H,window]; k_c,v_c codes [B,H,Ncap,d] with scales [B,H,Ncap]; pos int64 [B].
    Returns o [B,H,d] bf16 (and lse [B,H])."""
    _need(q, "q", torch.bfloat16, 3)
    for name, t in (("k", k), ("v", v), ("k_c", k_c), ("v_c", v_c)):
        _need(t, name, torch.uint8, 4)
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale), ("k_c_scale", k_c_scale), ("v_c_scale", v_c_scale)):
        _need(t, name, torch.float32, 3)
    _need(pos, "pos", torch.int64, 1)
    B, H, d = q.shape
    ncap = k_c.shape[2]
    for name, t, shape in (("k", k, (B, H, window, d)), ("v", v, (B, H, window, d)), ("k_c", k_c, (B, H, ncap, d)),
                           ("v_c", v_c, (B, H, ncap, d)), ("k_scale", k_scale, (B, H, window)),
                           ("v_scale", v_scale, (B, H, window)), ("k_c_scale", k_c_scale, (B, H, ncap)),
                           ("v_c_scale", v_c_scale, (B, H, ncap)), ("pos", pos, (B,))):
        _shape(t, name, shape)
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if return_lse else None
    args = _fp8_args(q, k, k_scale, v, v_scale, k_c, k_c_scale, v_c, v_c_scale, blk, window, scale, pos, o, lse)
    need = lib().hca_decode_fp8_workspace_size(ctypes.byref(args))
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel() * workspace.element_size()
    _check("hca_decode_fp8", lib().hca_decode_fp8(ctypes.byref(args), _stream()))
    return (o, lse) if return_lse else o


def hca_decode_fp8_workspace_size(q, k_c, blk, window):
    a = HcaDecodeFp8Args()
    a.B, a.H, a.d = q.shape
    a.blk, a.window, a.n_c_cap = blk, window, k_c.shape[2]
    return lib().hca_decode_fp8_workspace_size(ctypes.byref(a))


def dsa_indexer_scores(q_idx, k_idx, w, q_pos=None, out=None):
    """q_idx [B,T,Hi,Di] bf16, k_idx [B,S,Di] bf16, w [B,T,Hi] f32 -> scores [B,T,S] f32."""
    _need(q_idx, "q_idx", torch.bfloat16, 4)
    _need(k_idx, "k_idx", torch.bfloat16, 3)
    _need(w, "w", torch.float32, 3)
    B, T, Hi, Di = q_idx.shape
    S = k_idx.shape[1]
    _shape(k_idx, "k_idx", (B, S, Di))
    _shape(w, "w", (B, T, Hi))
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int64, 1)
        _shape(q_pos, "q_pos", (B,))
    if out is None:
        out = torch.empty((B, T, S), dtype=torch.float32, device=q_idx.device)
    _need(out, "out", torch.float32, 3)
    _shape(out, "out", (B, T, S))
    _check(
        "dsa_indexer_scores",
        lib().dsa_indexer_scores(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(q_pos), _ptr(out), B, T, S, Hi, Di, _stream()),
    )
    return out


def csa_indexer_scores(q_idx, kc_idx, w, ratio, q_pos=None, out=None):
    """CSA indexer: q_idx [B,T,Hi,Di] bf16 (token rows), kc_idx [B,S,Di] bf16 (entries of `ratio` tokens),
    w [B,T,Hi] f32 -> scores [B,T,S] f32 (row i sees entries s < (q_pos + i + 1) // ratio)."""
    _need(q_idx, "q_idx", torch.bfloat16, 4)
    _need(kc_idx, "kc_idx", torch.bfloat16, 3)
    _need(w, "w", torch.float32, 3)
    B, T, Hi, Di = q_idx.shape
    S = kc_idx.shape[1]
    _shape(kc_idx, "kc_idx", (B, S, Di))
    _shape(w, "w", (B, T, Hi))
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int64, 1)
        _shape(q_pos, "q_pos", (B,))
    if out is None:
        out = torch.empty((B, T, S), dtype=torch.float32, device=q_idx.device)
    _need(out, "out", torch.float32, 3)
    _shape(out, "out", (B, T, S))
    _check(
        "csa_indexer_scores",
        lib().csa_indexer_scores(_ptr(q_idx), _ptr(kc_idx), _ptr(w), _ptr(q_pos), _ptr(out), B, T, S, Hi, Di, ratio,
                                 _stream()),
    )
    return out


def csa_topk(scores, k, ratio, q_pos=None, out=None, workspace=None):
    """CSA top-k: scores [B,T,S] f32 over entries of `ratio` tokens -> idx [B,T,k] int32."""
    _need(scores, "scores", torch.float32, 3)
    B, T, S = scores.shape
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int64, 1)
        _shape(q_pos, "q_pos", (B,))
    if out is None:
        out = torch.empty((B, T, k), dtype=torch.int32, device=scores.device)
    _need(out, "out", torch.int32, 3)
    _shape(out, "out", (B, T, k))
    need = lib().dsa_topk_workspace_size(B, T, S, k)
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(
        "csa_topk",
        lib().csa_topk(_ptr(scores), _ptr(q_pos), _ptr(out), B, T, S, k, ratio, _ptr(workspace), wsb, _stream()),
    )
    return out


def dsa_indexer_topk_workspace_size(B, T, S, k):
    return lib().dsa_indexer_topk_workspace_size(B, T, S, k)


def dsa_indexer_topk(q_idx, k_idx, w, k, q_pos=None, out=None, workspace=None, force_fallback=False):
    """Fused indexer and top-k: the idx of dsa_topk(dsa_indexer_scores(q_idx, k_idx, w, q_pos), k, q_pos)
    without the score matrix.  q_idx [B,T,Hi,Di] bf16, k_idx [B,S,Di] bf16, w [B,T,Hi] f32 -> idx [B,T,k] int32."""
    _need(q_idx, "q_idx", torch.bfloat16, 4)
    _need(k_idx, "k_idx", torch.bfloat16, 3)
    _need(w, "w", torch.float32, 3)
    B, T, Hi, Di = q_idx.shape
    S = k_idx.shape[1]
    _shape(k_idx, "k_idx", (B, S, Di))
    _shape(w, "w", (B, T, Hi))
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int64, 1)
        _shape(q_pos, "q_pos", (B,))
    if out is None:
        out = torch.empty((B, T, k), dtype=torch.int32, device=q_idx.device)
    _need(out, "out", torch.int32, 3)
    _shape(out, "out", (B, T, k))
    need = lib().dsa_indexer_topk_workspace_size(B, T, S, k)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_idx.device)
    wsb = workspace.numel() * workspace.element_size()
    _check(
        "dsa_indexer_topk",
        lib().dsa_indexer_topk(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(q_pos), _ptr(out), B, T, S, Hi, Di, k,
                               1 if force_fallback else 0, _ptr(workspace), wsb, _stream()),
    )
    return out


def dsa_topk_workspace_size(B, T, S, k):
    return lib().dsa_topk_workspace_size(B, T, S, k)


def dsa_topk(scores, k, q_pos=None, out=None, workspace=None):
    """scores [B,T,S] f32 -> idx [B,T,k] int32 (ascending positions, -1 padded)."""
    _need(scores, "scores", torch.float32, 3)
    B, T, S = scores.shape
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int64, 1)
        _shape(q_pos, "q_pos", (B,))
    if out is None:
        out = torch.empty((B, T, k), dtype=torch.int32, device=scores.device)
    _need(out, "out", torch.int32, 3)
    _shape(out, "out", (B, T, k))
    need = lib().dsa_topk_workspace_size(B, T, S, k)
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(
        "dsa_topk",
        lib().dsa_topk(_ptr(scores), _ptr(q_pos), _ptr(out), B, T, S, k, _ptr(workspace), wsb, _stream()),
    )
    return out


def dsa_sparse_attention_fwd_workspace_size(B, T, Hq, D, kk):
    return lib().dsa_sparse_attention_fwd_workspace_size(B, T, Hq, D, kk)


def dsa_sparse_attention_fwd(q, k, v, idx, scale=None, return_lse=False, workspace=None):
    """q [B,T,Hq,D], k,v [B,S,D] bf16, idx [B,T,kk] int32 -> o [B,T,Hq,D] (and lse [B,T,Hq])."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(idx, "idx", torch.int32, 3)
    B, T, Hq, D = q.shape
    S = k.shape[1]
    kk = idx.shape[2]
    _shape(k, "k", (B, S, D))
    _shape(v, "v", (B, S, D))
    _shape(idx, "idx", (B, T, kk))
    o = torch.empty_like(q)
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    need = lib().dsa_sparse_attention_fwd_workspace_size(B, T, Hq, D, kk)
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(
        "dsa_sparse_attention_fwd",
        lib().dsa_sparse_attention_fwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(o), _ptr(lse), SA_BF16, B, T, S, Hq, D, kk,
            0.0 if scale is None else float(scale), _ptr(workspace), wsb, _stream(),
        ),
    )
    return (o, lse) if return_lse else o


def dsa_sparse_attention_bwd_workspace_size(B, T, S, kk):
    return lib().dsa_sparse_attention_bwd_workspace_size(B, T, S, kk)


def dsa_sparse_attention_bwd(q, k, v, idx, o, lse, do, scale=None, workspace=None):
    """Gradients of dsa_sparse_attention_fwd for the upstream gradient do of o.

    q, o, do [B,T,Hq,D] bf16; k, v [B,S,D] bf16; idx [B,T,kk] int32; lse [B,T,Hq] fp32 (o and lse
    from the forward call) -> (dq [B,T,Hq,D], dk [B,S,D], dv [B,S,D]) fp32.
    """
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(idx, "idx", torch.int32, 3)
    _need(o, "o", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    _need(do, "do", torch.bfloat16, 4)
    B, T, Hq, D = q.shape
    S = k.shape[1]
    kk = idx.shape[2]
    _shape(k, "k", (B, S, D))
    _shape(v, "v", (B, S, D))
    _shape(idx, "idx", (B, T, kk))
    _shape(o, "o", (B, T, Hq, D))
    _shape(lse, "lse", (B, T, Hq))
    _shape(do, "do", (B, T, Hq, D))
    dq = torch.empty((B, T, Hq, D), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, S, D), dtype=torch.float32, device=q.device)
    dv = torch.empty((B, S, D), dtype=torch.float32, device=q.device)
    need = lib().dsa_sparse_attention_bwd_workspace_size(B, T, S, kk)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(
        "dsa_sparse_attention_bwd",
        lib().dsa_sparse_attention_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
            SA_BF16, B, T, S, Hq, D, kk, 0.0 if scale is None else float(scale), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(),
        ),
    )
    return dq, dk, dv

"""HCA + MLA-DSA forward pass for AMD Instinct MI355X (gfx950).

Python binding of the C ABI in include/sparse_attn_hca.h; every step of the
path runs in the library's HIP kernels.
"""

from ._lib import (
    HCA_DECODE,
    HCA_PREFILL,
    LIB_PATH,
    SparseAttnError,
    csa_indexer_scores,
    csa_topk,
    dsa_indexer_scores,
    dsa_sparse_attention_bwd,
    dsa_sparse_attention_bwd_workspace_size,
    dsa_sparse_attention_fwd,
    dsa_sparse_attention_fwd_workspace_size,
    dsa_topk,
    dsa_topk_workspace_size,
    dsa_indexer_topk,
    dsa_indexer_topk_workspace_size,
    hca_attention_fwd,
    hca_attention_fwd_noalloc,
    hca_attention_workspace_size,
    hca_compress,
    hca_decode_fp8,
    hca_decode_fp8_workspace_size,
    hca_quantize_fp8,
    lib,
    version,
)

__all__ = [
    "HCA_DECODE",
    "HCA_PREFILL",
    "LIB_PATH",
    "SparseAttnError",
    "csa_indexer_scores",
    "csa_topk",
    "dsa_indexer_scores",
    "dsa_sparse_attention_fwd",
    "dsa_sparse_attention_bwd",
    "dsa_sparse_attention_bwd_workspace_size",
    "dsa_sparse_attention_fwd_workspace_size",
    "dsa_topk",
    "dsa_topk_workspace_size",
    "dsa_indexer_topk",
    "dsa_indexer_topk_workspace_size",
    "hca_attention_fwd",
    "hca_attention_fwd_noalloc",
    "hca_attention_workspace_size",
    "hca_compress",
    "hca_decode_fp8",
    "hca_decode_fp8_workspace_size",
    "hca_quantize_fp8",
    "lib",
    "version",
]

"""Float64 CPU oracle for the HCA + MLA-DSA forward pass (and its backward).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library or its Python
binding and imports neither.

Every function is the plain definition of what the method computes, written
in NumPy float64 with no blocking, fusion or reordering beyond what the
definition states.  Inputs are upcast exactly (fp32 and bf16 values are
exactly representable in float64).

Sources (web pages about ERNIE-5.5-Flash-Base, cited by title and section):

  [P1] aitest123.com, "280B总参数、14B激活！百度开源文心5.5 Flash Base，拿下同尺寸SOTA",
       section 二.1 "Latent-Gated Sparse Attention：37层省缓存，6层保精准检索".
  [P2] qunfachuanzhen.com ERNIE-5.5-Flash-Base news page, section
       "◆ 混合稀疏注意力,把 1M 上下文的成本压下来".
  [P3] communeify.com, "百度 ERNIE 5.5 Flash Base 完整解析：280B 混合注意力 MoE 基座模型…",
       section "六大核心架構創新深度解析", item 1 "潛在門控混合稀疏注意力（Hybrid MLA-DSA + HCA）與 VHA".

Where the pages leave a step open, the reading taken is stated in the
docstring of the function that depends on it.

Pins: every function here is pinned by the CPU tests in
tests/test_oracle_pins.py against closed forms, degenerate cases that reduce
to a library routine (torch CPU scaled_dot_product_attention, NumPy matmul),
invariants, hand-derived golden values (tests/golden/) and brute force on tiny
inputs.  Whether the block mean and the ReLU indexer match the real model's
learned layers is "parity unpinned": the pages print no values for them.
"""

from .hca import (
    hca_compress,
    hca_visible_blocks,
    hca_window_range,
    hca_key_set,
    hca_attention_prefill,
    hca_attention_decode,
    hca_attention_bwd,
    hca_compress_bwd,
    hca_layer_bwd,
)
from .dsa import (
    dsa_indexer_scores,
    dsa_topk,
    dsa_sparse_attention,
    dsa_sparse_attention_bwd,
    csa_attention,
    n_candidates,
)
from .fp8 import (
    e4m3_value,
    e4m3_encode,
    quantize_fp8_rows,
    dequantize_fp8_rows,
)

__all__ = [
    "hca_compress",
    "hca_visible_blocks",
    "hca_window_range",
    "hca_key_set",
    "hca_attention_prefill",
    "hca_attention_decode",
    "hca_attention_bwd",
    "hca_compress_bwd",
    "hca_layer_bwd",
    "dsa_indexer_scores",
    "dsa_topk",
    "dsa_sparse_attention",
    "dsa_sparse_attention_bwd",
    "csa_attention",
    "n_candidates",
    "e4m3_value",
    "e4m3_encode",
    "quantize_fp8_rows",
    "dequantize_fp8_rows",
]

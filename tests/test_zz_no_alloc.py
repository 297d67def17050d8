"""GPU: the allocation-free HCA entry point (static scratch) against hca_attention_fwd with a caller workspace.

Both run the same kernels with the same split count, so the outputs must be bit-identical.  Two calls in a
row on the allocation-free entry point, the second with a smaller input (fewer sequences, heads and cache
entries), check that the shared scratch left by the first call does not leak into the second.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV, require_gpu

pytestmark = pytest.mark.gpu


def _decode_inputs(B, H, ncap, win, pos, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    s = 512 ** -0.5

    def rnd(*shape):
        return (torch.randn(shape, generator=g, device=DEV) * s).to(torch.bfloat16)

    q = rnd(B, H, 512)
    kc, vc = rnd(B, H, ncap, 512), rnd(B, H, ncap, 512)
    rk, rv = rnd(B, H, win, 512), rnd(B, H, win, 512)
    p = torch.tensor(pos, dtype=torch.int64, device=DEV)
    return q, kc, vc, rk, rv, p


@pytest.mark.parametrize("first,second", [((4, 64, 8192, [1048575, 1048575, 500000, 130]),
                                           (2, 8, 300, [38399, 1000])),
                                          ((64, 16, 1024, [131071] * 64), (1, 3, 600, [70000]))])
def test_noalloc_decode_matches_workspace_call(first, second):
    sa = require_gpu()
    for n, (B, H, ncap, pos) in enumerate((first, second)):
        print(f"[no_alloc] call {n}: B={B} H={H} n_c_cap={ncap}", flush=True)
        q, kc, vc, rk, rv, p = _decode_inputs(B, H, ncap, 128, pos, 4242 + n)
        want_o, want_l = sa.hca_attention_fwd(sa.HCA_DECODE, q, rk, rv, kc, vc, 128, 128, pos=p, return_lse=True)
        got_o, got_l = sa.hca_attention_fwd_noalloc(sa.HCA_DECODE, q, rk, rv, kc, vc, 128, 128, pos=p, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(got_o, want_o)
        assert torch.equal(got_l, want_l)


def test_noalloc_prefill_matches():
    sa = require_gpu()
    q, k, v = (synth.to_torch(synth.np_normal((1, 2, 300, 512), 1.0, "bf16", 9100, i), "bf16", DEV) for i in range(3))
    kc, vc = sa.hca_compress(k, 128), sa.hca_compress(v, 128)
    want = sa.hca_attention_fwd(sa.HCA_PREFILL, q, k, v, kc, vc, 128, 128)
    got = sa.hca_attention_fwd_noalloc(sa.HCA_PREFILL, q, k, v, kc, vc, 128, 128)
    assert torch.equal(got, want)

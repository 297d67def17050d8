"""Seeded synthetic inputs for the HCA + MLA-DSA workloads.

This module is the only code shared by the HIP path's callers (tests, bench,
smoke) and the float64 oracle.  It draws random numbers and rounds them to
the I/O dtype; it holds none of the attention, compression, indexer or top-k
arithmetic.

Two generators:
  * ``np_*`` functions: NumPy PCG64 streams keyed by
    SeedSequence([workload, tensor id, chunk]), for inputs small enough to
    draw on the host.  Values are float32 arrays already rounded to the
    target dtype (bf16 by round-to-nearest-even), so the device copy and the
    oracle see identical numbers.
  * ``torch_*`` functions: a seeded torch.Generator on the target device,
    for the full-size workloads (billions of elements).  The oracle gets the
    same bits by copying the needed slices back to the host.

Workload recipes (shapes, scales and distributions):
  hca_tiny      q,k,v [1,4,1024,64] f32 N(0,1); block 128, window 128.
  hca_prefill   q,k,v [1,64,32768,512] bf16 N(0,1)/sqrt(512); block 128, window 128.
  hca_decode    q [64,64,512]; compressed K/V [64,64,1024,512]; window ring K/V
                [64,64,128,512]; bf16 N(0,1)/sqrt(512); query position 131071.
  dsa_prefill   indexer q [1,32768,4,128], k [1,32768,128] bf16 N(0,1)/sqrt(128);
                head weights [1,32768,4] f32 U(0,1); attention q [1,32768,64,256],
                k,v [1,32768,256] bf16 N(0,1)/16; top-2048.
  decode_1m     HCA: q [4,64,512], compressed K/V [4,64,8192,512], ring [4,64,128,512];
                DSA: indexer q [4,1,4,128], k [4,1048576,128], w [4,1,4];
                attention q [4,1,64,256], k,v [4,1048576,256]; query position 1048575.
"""

import numpy as np

# ---------------------------------------------------------------------------
# bf16 rounding on the host (round to nearest, ties to even)
# ---------------------------------------------------------------------------


def bf16_round(x):
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def round_to(x, dtype):
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_round(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# NumPy generators
# ---------------------------------------------------------------------------


def np_rng(workload, tensor_id, chunk=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload, tensor_id, chunk])))


def np_normal(shape, sigma, dtype, workload, tensor_id):
    g = np_rng(workload, tensor_id)
    return round_to(g.standard_normal(shape, dtype=np.float32) * np.float32(sigma), dtype)


def np_uniform(shape, workload, tensor_id):
    g = np_rng(workload, tensor_id)
    return g.random(shape, dtype=np.float32)


def np_int_grid(shape, values, workload, tensor_id):
    """Values drawn uniformly from a small finite set (exact in fp32 arithmetic)."""
    g = np_rng(workload, tensor_id)
    vals = np.asarray(values, dtype=np.float32)
    return vals[g.integers(0, len(vals), size=shape)]


# ---------------------------------------------------------------------------
# torch generators (device-side, for full-size workloads)
# ---------------------------------------------------------------------------


def torch_normal(shape, sigma, dtype, seed, device, chunk_elems=1 << 28):
    """N(0, sigma^2) drawn in float32 on ``device`` and cast to ``dtype`` (RNE)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        tmp = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        tmp.mul_(float(sigma))
        flat[s:e].copy_(tmp)
        del tmp
    return out


def torch_uniform(shape, seed, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def to_torch(x, dtype, device):
    """Host float32 array (already representable in ``dtype``) -> torch tensor."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    return t.to(device=device, dtype=tdt)

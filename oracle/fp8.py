"""FP8 decode-cache encoding oracle.  TEST INFRASTRUCTURE ONLY.

The decode step of HCA ([P1] §二.1, [P3] §架構創新 1) reads every visible cache
row once, so its cost is the size of the cache.  The pages name no cache
format; the FP8 cache is an extension of this library, and everything below
is its stated reading, not the pages':

  * format: OCP E4M3, "fn" variant -- sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; the code
    S.1111.111 is NaN; there are no infinities; the largest finite magnitude
    is 448 (S.1111.110);
  * one fp32 scale per row: amax = max_j |x_j|, inv = fl32(448 / amax)
    (0 when amax == 0), code_j = E4M3 nearest to fl32(x_j * inv) with ties to
    the even code, scale = fl32(amax / 448); the row is read back as
    scale * value(code_j).

fl32(.) is one IEEE float32 operation rounded to nearest even, which NumPy
float32 arithmetic performs exactly as written.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code):
    """Float64 value of E4M3 codes (NaN for S.1111.111), straight from the field layout."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x):
    """Nearest E4M3 code to each float64 value, ties to the even code.

    Values spaced 2^(e-3) apart cover [2^e, 2^(e+1)) for e >= -6, and the
    subnormals continue that spacing (2^-9) below 2^-6, so with
    e = max(floor(log2|x|), -6) and n = round_half_even(|x| / 2^(e-3)) the
    code is 8*(e+7) + (n-8) -- n = 16 carries into the next exponent by
    itself, and in the subnormal range the formula gives n directly.  Only
    |x| <= 464 (448 plus half a step) is in range; -0.0 keeps its sign.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)) or np.any(np.abs(x) > 464.0):
        raise ValueError("e4m3_encode: NaN or magnitude beyond 464")
    sign = np.where(np.signbit(x), 0x80, 0)
    a = np.abs(x)
    _, ex = np.frexp(a)                 # a = f * 2^ex with f in [0.5, 1) (ex = 0 for a = 0)
    e = np.where(a > 0, np.maximum(ex - 1, -6), -6)  # floor(log2 a), not below the subnormal exponent
    n = np.rint(np.ldexp(a, -(e - 3)))  # exact scaling by a power of two, then ties to even
    code = 8 * (e + 7) + (n.astype(np.int64) - 8)
    return (sign | code).astype(np.uint8)


def quantize_fp8_rows(x):
    """Per-row E4M3 encoding of cache rows x [..., d] -> (codes uint8 [..., d], scales float32 [...])."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, np.float32(E4M3_MAX) / amax, np.float32(0.0)).astype(np.float32)
    prod = (x32 * inv[..., None]).astype(np.float32)
    codes = e4m3_encode(prod.astype(np.float64))
    scales = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return codes, scales


def dequantize_fp8_rows(codes, scales):
    """scale * value(code) in float64 (both factors are exact in float64, so is the product)."""
    return e4m3_value(codes) * np.asarray(scales, dtype=np.float64)[..., None]

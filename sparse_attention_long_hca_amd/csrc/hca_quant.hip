// FP8 (E4M3) encoding of cache rows for HCA decode (gfx950).
//
// Method: the decode step of [P1] §二.1 / [P3] §架構創新 1 reads every visible
// compressed entry and window token once, so its cost is the bytes of the
// cache.  The pages name no cache format; this library offers, beside bf16,
// OCP E4M3 ("fn": bias 7, largest finite value 448, no infinities) codes with
// one fp32 scale per row:
//   amax = max_j |x[j]|,  inv = 448 / amax (0 when amax == 0),
//   code[j] = E4M3(x[j] * inv) rounded to nearest even,  scale = amax / 448,
// so x[j] ~= scale * value(code[j]).  All arithmetic is fp32; |x[j] * inv|
// never exceeds 448, so no code saturates.
//
// One wave per row: each lane reads 16-byte chunks (8 bf16), the row maximum
// is a wave reduction, and the hardware conversion (round to nearest even)
// packs 8 codes into 8 bytes per chunk.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kQuantThreads = 256;
constexpr int kQuantWaves = kQuantThreads / kWave;

__global__ __launch_bounds__(kQuantThreads) void hca_quantize_fp8_kernel(HcaQuantParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kQuantWaves + wave;
  if (row >= p.rows) return;
  const int chunks = (int)(p.d / 8);  // 8 elements per chunk
  const bf16_t* x = reinterpret_cast<const bf16_t*>(p.x) + row * p.d;
  uint8_t* codes = reinterpret_cast<uint8_t*>(p.codes) + row * p.d;

  float amax = 0.f;
  for (int c = lane; c < chunks; c += kWave) {
    const uint4 u = *reinterpret_cast<const uint4*>(x + 8 * c);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      amax = fmaxf(amax, fabsf(bf16_to_f32(w[e] & 0xffffu)));
      amax = fmaxf(amax, fabsf(__uint_as_float(w[e] & 0xffff0000u)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float inv = amax > 0.f ? 448.f / amax : 0.f;
  for (int c = lane; c < chunks; c += kWave) {
    const uint4 u = *reinterpret_cast<const uint4*>(x + 8 * c);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t a = w[2 * h], b = w[2 * h + 1];
      uint32_t pk = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_to_f32(a & 0xffffu) * inv,
                                                    __uint_as_float(a & 0xffff0000u) * inv, 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_to_f32(b & 0xffffu) * inv, __uint_as_float(b & 0xffff0000u) * inv,
                                           pk, true);
      out[h] = pk;
    }
    *reinterpret_cast<uint2*>(codes + 8 * c) = make_uint2(out[0], out[1]);
  }
  if (lane == 0) p.scales[row] = amax / 448.f;
}

hipError_t launch_hca_quantize_fp8(const HcaQuantParams& p, hipStream_t stream) {
  const int64_t nblocks = (p.rows + kQuantWaves - 1) / kQuantWaves;
  hipLaunchKernelGGL(hca_quantize_fp8_kernel, dim3((uint32_t)nblocks), dim3(kQuantThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa

// HCA block-mean compression (gfx950).
//
// Method: [P1] §二.1, [P2] §混合稀疏注意力 and [P3] §架構創新 1 -- every 128
// consecutive tokens become one cache entry.  The pages do not name the
// operator; the entry is the arithmetic mean of the block's rows.
//
// One workgroup per output row.  With C = chunks (16 bytes) per row and
// R = floor(256 / C) rows per pass, thread t < R*C reads chunk t % C of rows
// t / C, t / C + R, ... so that each wave reads whole rows contiguously (the
// last 256 - R*C threads idle when C does not divide 256, e.g. 72 chunks for
// a 576-wide bf16 row); the partial sums are combined through LDS in a fixed
// order (deterministic), divided by blk and rounded to the I/O dtype.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kCompressThreads = 256;

template <typename T>
__global__ __launch_bounds__(kCompressThreads) void hca_compress_kernel(HcaCompressParams p) {
  constexpr int kEPC = 16 / (int)sizeof(T);
  __shared__ float red[kCompressThreads * kEPC];

  const int64_t id = blockIdx.x;
  const int64_t n = id % p.n_out;
  const int64_t bh = id / p.n_out;
  const int64_t h = bh % p.H, b = bh / p.H;
  const T* src = reinterpret_cast<const T*>(p.x) + b * p.x_sb + h * p.x_sh + n * p.blk * p.x_st;
  T* dst = reinterpret_cast<T*>(p.out) + b * p.o_sb + h * p.o_sh + n * p.o_sn;

  const int chunks = (int)(p.d / kEPC);  // <= 256 (checked on the host)
  const int tid = threadIdx.x;
  const int c = tid % chunks;
  const int rstep = kCompressThreads / chunks;
  const int r0 = tid / chunks < rstep ? tid / chunks : (int)p.blk;  // idle threads read nothing

  float acc[kEPC];
#pragma unroll
  for (int e = 0; e < kEPC; ++e) acc[e] = 0.f;

  const int blk = (int)p.blk;
#pragma unroll 8
  for (int r = r0; r < blk; r += rstep) {
    // Read once: non-temporal loads (a wave reads whole 128-byte lines).
    const uint4 u = load_stream_u4(src + (int64_t)r * p.x_st + c * kEPC);
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_to_f32(w[i] & 0xffffu);
        acc[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
      acc[0] += __uint_as_float(u.x);
      acc[1] += __uint_as_float(u.y);
      acc[2] += __uint_as_float(u.z);
      acc[3] += __uint_as_float(u.w);
    }
  }
#pragma unroll
  for (int e = 0; e < kEPC; ++e) red[tid * kEPC + e] = acc[e];
  __syncthreads();
  if (tid < chunks) {
    float s[kEPC];
#pragma unroll
    for (int e = 0; e < kEPC; ++e) s[e] = 0.f;
    for (int rr = 0; rr < rstep; ++rr) {
#pragma unroll
      for (int e = 0; e < kEPC; ++e) s[e] += red[(rr * chunks + tid) * kEPC + e];
    }
    const float fb = (float)blk;
    if constexpr (sizeof(T) == 2) {
      uint4 out;
      out.x = pack_bf16x2(s[0] / fb, s[1] / fb);
      out.y = pack_bf16x2(s[2] / fb, s[3] / fb);
      out.z = pack_bf16x2(s[4] / fb, s[5] / fb);
      out.w = pack_bf16x2(s[6] / fb, s[7] / fb);
      *reinterpret_cast<uint4*>(dst + tid * kEPC) = out;
    } else {
      *reinterpret_cast<float4*>(dst + tid * kEPC) = make_float4(s[0] / fb, s[1] / fb, s[2] / fb, s[3] / fb);
    }
  }
}

hipError_t launch_hca_compress(const HcaCompressParams& p, int dtype, hipStream_t stream) {
  const int64_t nblocks = p.B * p.H * p.n_out;
  if (dtype == 0)
    hipLaunchKernelGGL(hca_compress_kernel<float>, dim3((uint32_t)nblocks), dim3(kCompressThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(hca_compress_kernel<bf16_t>, dim3((uint32_t)nblocks), dim3(kCompressThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa

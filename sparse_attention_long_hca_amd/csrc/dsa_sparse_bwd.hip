// Backward of the DSA sparse attention over the selected positions (gfx950).
//
// Method: [P1] §二.1, [P3] §架構創新 1 -- core attention runs only on the
// top-K positions; the pages train these layers but print no backward
// formula, so the gradients are the chain rule of the forward's definition
// (one KV head shared by the 64 query heads, 256 wide).  The selection is
// discrete and gets no gradient.  Per token, with P the forward's softmax
// weights over the token's entries (from the saved log-sum-exp) and D_h =
// sum_d dO[h,d] * O[h,d]:
//   dP = dO . v_s,   dS = P * (dP - D_h)
//   dq_h += scale * dS * k_s,  dk[s] += scale * sum_h dS * q_h,
//   dv[s] += sum_h P * dO_h.
//
// One workgroup (256 threads) per token.  Q and dO of the token sit in LDS
// (bf16); the index list is walked in tiles of 16 rows, each tile's K and V
// rows gathered into LDS.  Every thread computes S and dP for one row and four
// heads (bf16 dot2 into fp32), then P and dS go to LDS; dQ accumulates in
// registers (one head, 64 dims per thread); the tile's dK and dV rows are
// summed over the 64 heads in the workgroup and added to the fp32 outputs with
// atomics (several tokens select the same position).  Vector ALU arithmetic:
// a first, plain version of the backward.
#include "common.h"
#include "kernels.h"

namespace sa {

namespace {
constexpr int kBwH = 64;         // query heads
constexpr int kBwD = 256;        // head width
constexpr int kBwTK = 16;        // index-list rows per tile
constexpr int kBwThreads = 256;
constexpr int kBwMaxK = 2048;
constexpr int kBwRowB = kBwD * 2 + 16;  // LDS pitch of a bf16 row: consecutive rows start 4 banks apart
constexpr int kBwPP = kBwH + 1;         // pitch (floats) of the P and dS tiles

__device__ __forceinline__ float bw_dot8(uint4 a, uint4 b, float c) {
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), c, false);
  return c;
}

// acc[0..7] += w * (8 bf16 of u)
__device__ __forceinline__ void bw_axpy8(float* acc, float w, uint4 u) {
  const uint32_t x[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(w, bf16_to_f32(x[i] & 0xffffu), acc[2 * i]);
    acc[2 * i + 1] = fmaf(w, bf16_to_f32(x[i] >> 16), acc[2 * i + 1]);
  }
}
}  // namespace

__global__ __launch_bounds__(256) void dsa_sparse_bwd_zero_kernel(float4* p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ __launch_bounds__(kBwThreads) void dsa_sparse_bwd_kernel(DsaSparseBwdParams p) {
  __shared__ __attribute__((aligned(16))) char qs[kBwH * kBwRowB];
  __shared__ __attribute__((aligned(16))) char dos[kBwH * kBwRowB];
  __shared__ __attribute__((aligned(16))) char ks[kBwTK * kBwRowB];
  __shared__ __attribute__((aligned(16))) char vs[kBwTK * kBwRowB];
  __shared__ float pt[kBwTK * kBwPP];
  __shared__ float dst[kBwTK * kBwPP];
  __shared__ int32_t sidx[kBwMaxK];
  __shared__ float lse2[kBwH];  // log-sum-exp in log2 units
  __shared__ float dsum[kBwH];  // D_h

  const int t = threadIdx.x;
  const int64_t tok = blockIdx.x;  // b*T + i
  const int64_t b = tok / p.T;
  const int kk = (int)p.kk;
  const bf16_t* q = reinterpret_cast<const bf16_t*>(p.q) + tok * kBwH * kBwD;
  const bf16_t* dO = reinterpret_cast<const bf16_t*>(p.dout) + tok * kBwH * kBwD;
  const bf16_t* o = reinterpret_cast<const bf16_t*>(p.o) + tok * kBwH * kBwD;
  const bf16_t* kb = reinterpret_cast<const bf16_t*>(p.k) + b * p.S * kBwD;
  const bf16_t* vb = reinterpret_cast<const bf16_t*>(p.v) + b * p.S * kBwD;

  // Q and dO rows -> LDS (32 chunks of 16 bytes per row); the index list with
  // skipped entries and the tail of the last tile set to -1.
  for (int e = t; e < kBwH * 32; e += kBwThreads) {
    const int r = e >> 5, c = e & 31;
    *reinterpret_cast<uint4*>(qs + r * kBwRowB + c * 16) = reinterpret_cast<const uint4*>(q)[e];
    *reinterpret_cast<uint4*>(dos + r * kBwRowB + c * 16) = reinterpret_cast<const uint4*>(dO)[e];
  }
  const int kk_pad = (kk + kBwTK - 1) / kBwTK * kBwTK;
  for (int n = t; n < kk_pad; n += kBwThreads) {
    const int32_t s = n < kk ? p.idx[tok * kk + n] : -1;
    sidx[n] = (s >= 0 && s < p.S) ? s : -1;
  }
  {
    // D_h from the forward's output (four threads per head, 64 dims each).
    const int h = t >> 2, c = t & 3;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      acc = bw_dot8(reinterpret_cast<const uint4*>(o + h * kBwD + c * 64)[u],
                    reinterpret_cast<const uint4*>(dO + h * kBwD + c * 64)[u], acc);
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (c == 0) {
      dsum[h] = acc;
      lse2[h] = p.lse[tok * kBwH + h] * kLog2e;
    }
  }
  __syncthreads();

  const int hq = t >> 2, cq = t & 3;  // dQ: head, 64-dim chunk
  float dq[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) dq[i] = 0.f;
  const int n_tiles = kk_pad / kBwTK;
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int32_t* trow = sidx + tile * kBwTK;
    // K and V rows of the tile -> LDS (zeros for skipped entries).
    for (int e = t; e < kBwTK * 32; e += kBwThreads) {
      const int r = e >> 5, c = e & 31;
      const int32_t s = trow[r];
      uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = kv;
      if (s >= 0) {
        kv = reinterpret_cast<const uint4*>(kb + (int64_t)s * kBwD)[c];
        vv = reinterpret_cast<const uint4*>(vb + (int64_t)s * kBwD)[c];
      }
      *reinterpret_cast<uint4*>(ks + r * kBwRowB + c * 16) = kv;
      *reinterpret_cast<uint4*>(vs + r * kBwRowB + c * 16) = vv;
    }
    __syncthreads();
    {
      // S and dP of row j for heads 4g .. 4g+3, then P and dS.
      const int j = t & 15, g = t >> 4;
      float sa_[4] = {0.f, 0.f, 0.f, 0.f}, pa[4] = {0.f, 0.f, 0.f, 0.f};
      for (int c = 0; c < 32; ++c) {
        const uint4 kv = *reinterpret_cast<const uint4*>(ks + j * kBwRowB + c * 16);
        const uint4 vv = *reinterpret_cast<const uint4*>(vs + j * kBwRowB + c * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = 4 * g + i;
          sa_[i] = bw_dot8(*reinterpret_cast<const uint4*>(qs + h * kBwRowB + c * 16), kv, sa_[i]);
          pa[i] = bw_dot8(*reinterpret_cast<const uint4*>(dos + h * kBwRowB + c * 16), vv, pa[i]);
        }
      }
      const bool live = trow[j] >= 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * g + i;
        const float pr = live ? fast_exp2(sa_[i] * p.scale_log2 - lse2[h]) : 0.f;
        pt[j * kBwPP + h] = pr;
        dst[j * kBwPP + h] = pr * (pa[i] - dsum[h]);
      }
    }
    __syncthreads();
    // dQ (head hq, dims 64cq .. 64cq+63) += dS * K.
    for (int j = 0; j < kBwTK; ++j) {
      const float w = dst[j * kBwPP + hq];
      const char* kr = ks + j * kBwRowB + cq * 128;
#pragma unroll
      for (int u = 0; u < 8; ++u) bw_axpy8(dq + 8 * u, w, *reinterpret_cast<const uint4*>(kr + u * 16));
    }
    {
      // dK and dV of row j, dims 16c .. 16c+15, summed over the 64 heads.
      const int j = t >> 4, c = t & 15;
      const int32_t s = trow[j];
      if (s >= 0) {
        float ak[16], av[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) ak[i] = av[i] = 0.f;
        for (int h = 0; h < kBwH; ++h) {
          const float wk = dst[j * kBwPP + h], wv = pt[j * kBwPP + h];
          const char* qr = qs + h * kBwRowB + c * 32;
          const char* dr = dos + h * kBwRowB + c * 32;
          bw_axpy8(ak, wk, *reinterpret_cast<const uint4*>(qr));
          bw_axpy8(ak + 8, wk, *reinterpret_cast<const uint4*>(qr + 16));
          bw_axpy8(av, wv, *reinterpret_cast<const uint4*>(dr));
          bw_axpy8(av + 8, wv, *reinterpret_cast<const uint4*>(dr + 16));
        }
        float* dkr = p.dk + (b * p.S + s) * kBwD + c * 16;
        float* dvr = p.dv + (b * p.S + s) * kBwD + c * 16;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          unsafeAtomicAdd(dkr + i, ak[i] * p.scale);
          unsafeAtomicAdd(dvr + i, av[i]);
        }
      }
    }
    __syncthreads();  // the next tile overwrites K, V, P and dS
  }
  float* dqr = p.dq + (tok * kBwH + hq) * kBwD + cq * 64;
#pragma unroll
  for (int u = 0; u < 16; ++u)
    reinterpret_cast<float4*>(dqr)[u] =
        make_float4(dq[4 * u] * p.scale, dq[4 * u + 1] * p.scale, dq[4 * u + 2] * p.scale, dq[4 * u + 3] * p.scale);
}

hipError_t launch_dsa_sparse_bwd(const DsaSparseBwdParams& p, hipStream_t stream) {
  const int64_t n4 = p.B * p.S * kBwD / 4;
  const uint32_t zb = (uint32_t)std::min<int64_t>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(dsa_sparse_bwd_zero_kernel, dim3(zb), dim3(256), 0, stream, reinterpret_cast<float4*>(p.dk), n4);
  hipLaunchKernelGGL(dsa_sparse_bwd_zero_kernel, dim3(zb), dim3(256), 0, stream, reinterpret_cast<float4*>(p.dv), n4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dsa_sparse_bwd_kernel, dim3((uint32_t)(p.B * p.T)), dim3(kBwThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa

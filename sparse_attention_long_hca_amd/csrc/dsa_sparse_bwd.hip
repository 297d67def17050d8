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
// summed over the 64 heads in the workgroup and written, one row per (token,
// entry), to G and H in the workspace.  The dQ, dK and dV sums take two rows
// or two heads per bf16 dot2, with dS and P rounded to bf16 (as the forward
// rounds P for its P*V product).  Several tokens select the same
// position, so dk and dv are then summed per position: tokens are taken in
// chunks; per chunk a counting sort lists each position's (token, entry)
// rows, and one workgroup per position adds them into dk and dv (each output
// row has one owner and chunks run in order, so no floating-point atomics).
// Vector ALU arithmetic: a first, plain version of the backward.
#include "common.h"
#include "kernels.h"
#include "select_util.h"

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

// Two bf16 rows a, b (8 values each) interleaved into pairs (a_e, b_e), then
// acc[e] += a_e * w.x + b_e * w.y for the bf16 pair w: one dot2 per value.
__device__ __forceinline__ void bw_pair8(float* acc, uint32_t w2, uint4 a, uint4 b) {
  const uint32_t xa[4] = {a.x, a.y, a.z, a.w}, xb[4] = {b.x, b.y, b.z, b.w};
  const bf16x2_t w = __builtin_bit_cast(bf16x2_t, w2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (xa[i] & 0xffffu) | (xb[i] << 16);
    const uint32_t hi = (xa[i] >> 16) | (xb[i] & 0xffff0000u);
    acc[2 * i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lo), w, acc[2 * i], false);
    acc[2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, hi), w, acc[2 * i + 1], false);
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
  const int64_t tok = p.tok0 + blockIdx.x;  // b*T + i
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
    // dQ (head hq, dims 64cq .. 64cq+63) += dS * K, two rows per dot2 (dS
    // rounded to bf16, as P is for the forward's P*V product).
    for (int j = 0; j < kBwTK; j += 2) {
      const uint32_t w2 = pack_bf16x2(dst[j * kBwPP + hq], dst[(j + 1) * kBwPP + hq]);
      const char* kr = ks + j * kBwRowB + cq * 128;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        bw_pair8(dq + 8 * u, w2, *reinterpret_cast<const uint4*>(kr + u * 16),
                 *reinterpret_cast<const uint4*>(kr + kBwRowB + u * 16));
    }
    {
      // dK and dV of row j, dims 16c .. 16c+15, summed over the 64 heads.
      const int j = t >> 4, c = t & 15;
      const int32_t s = trow[j];
      if (s >= 0) {
        float ak[16], av[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) ak[i] = av[i] = 0.f;
        // Two heads per dot2 (dS and P rounded to bf16).
        for (int h = 0; h < kBwH; h += 2) {
          const uint32_t wk2 = pack_bf16x2(dst[j * kBwPP + h], dst[j * kBwPP + h + 1]);
          const uint32_t wv2 = pack_bf16x2(pt[j * kBwPP + h], pt[j * kBwPP + h + 1]);
          const char* qr = qs + h * kBwRowB + c * 32;
          const char* dr = dos + h * kBwRowB + c * 32;
          bw_pair8(ak, wk2, *reinterpret_cast<const uint4*>(qr), *reinterpret_cast<const uint4*>(qr + kBwRowB));
          bw_pair8(ak + 8, wk2, *reinterpret_cast<const uint4*>(qr + 16),
                   *reinterpret_cast<const uint4*>(qr + kBwRowB + 16));
          bw_pair8(av, wv2, *reinterpret_cast<const uint4*>(dr), *reinterpret_cast<const uint4*>(dr + kBwRowB));
          bw_pair8(av + 8, wv2, *reinterpret_cast<const uint4*>(dr + 16),
                   *reinterpret_cast<const uint4*>(dr + kBwRowB + 16));
        }
        const int64_t row = ((int64_t)blockIdx.x * kk + tile * kBwTK + j) * kBwD + c * 16;
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          *reinterpret_cast<float4*>(p.g + row + i) =
              make_float4(ak[i] * p.scale, ak[i + 1] * p.scale, ak[i + 2] * p.scale, ak[i + 3] * p.scale);
          *reinterpret_cast<float4*>(p.hh + row + i) = make_float4(av[i], av[i + 1], av[i + 2], av[i + 3]);
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

// Inverse index of one chunk of tokens: entry e = (token - tok0) * kk + j.
__global__ __launch_bounds__(256) void dsa_sparse_bwd_count_kernel(DsaSparseBwdParams p, int64_t ntok, uint32_t* cnt) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= ntok * p.kk) return;
  const int64_t tok = p.tok0 + e / p.kk;
  const int32_t s = p.idx[tok * p.kk + e % p.kk];
  if (s >= 0 && s < p.S) atomicAdd(&cnt[(tok / p.T) * p.S + s], 1u);
}

// Exclusive offsets of the counts (one workgroup): off[0..n], cursor = off.
__global__ __launch_bounds__(1024) void dsa_sparse_bwd_scan_kernel(const uint32_t* cnt, uint32_t* off, uint32_t* cursor,
                                                                   int64_t n) {
  __shared__ uint32_t scratch[32];
  const int64_t per = (n + 1023) / 1024;
  const int64_t i0 = threadIdx.x * per, i1 = min(n, i0 + per);
  uint32_t local = 0;
  for (int64_t i = i0; i < i1; ++i) local += cnt[i];
  uint32_t tot;
  uint32_t run = block_inclusive_scan(local, scratch, tot) - local;
  for (int64_t i = i0; i < i1; ++i) {
    off[i] = run;
    cursor[i] = run;
    run += cnt[i];
  }
  if (threadIdx.x == 0) off[n] = tot;
}

__global__ __launch_bounds__(256) void dsa_sparse_bwd_fill_kernel(DsaSparseBwdParams p, int64_t ntok, uint32_t* cursor,
                                                                  uint32_t* list) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= ntok * p.kk) return;
  const int64_t tok = p.tok0 + e / p.kk;
  const int32_t s = p.idx[tok * p.kk + e % p.kk];
  if (s >= 0 && s < p.S) list[atomicAdd(&cursor[(tok / p.T) * p.S + s], 1u)] = (uint32_t)e;
}

// One workgroup per key row, one thread per dim: dk[r] += sum of the chunk's
// G rows listed for r (dv likewise from H).
__global__ __launch_bounds__(kBwD) void dsa_sparse_bwd_reduce_kernel(DsaSparseBwdParams p, const uint32_t* off,
                                                                     const uint32_t* list) {
  const int64_t r = blockIdx.x;  // b*S + s
  const uint32_t e0 = off[r], e1 = off[r + 1];
  if (e0 == e1) return;
  const int d = threadIdx.x;
  float ak = 0.f, av = 0.f;
  uint32_t e = e0;
  for (; e + 4 <= e1; e += 4) {
    float gk[4], gv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t row = (int64_t)list[e + u] * kBwD + d;
      gk[u] = p.g[row];
      gv[u] = p.hh[row];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ak += gk[u];
      av += gv[u];
    }
  }
  for (; e < e1; ++e) {
    const int64_t row = (int64_t)list[e] * kBwD + d;
    ak += p.g[row];
    av += p.hh[row];
  }
  p.dk[r * kBwD + d] += ak;
  p.dv[r * kBwD + d] += av;
}

int64_t dsa_sparse_bwd_chunk(int64_t BT) { return BT < 1024 ? BT : 1024; }

size_t dsa_sparse_bwd_ws_bytes(int64_t B, int64_t T, int64_t S, int64_t kk) {
  const int64_t tc = dsa_sparse_bwd_chunk(B * T), keys = B * S;
  auto al = [](int64_t x) { return (size_t)((x + 63) & ~(int64_t)63); };  // 256-byte multiples of 4-byte words
  return 4 * (2 * al(tc * kk * kBwD) + al(tc * kk) + 3 * al(keys + 1));
}

hipError_t launch_dsa_sparse_bwd(DsaSparseBwdParams p, hipStream_t stream) {
  const int64_t BT = p.B * p.T, keys = p.B * p.S, tc = dsa_sparse_bwd_chunk(BT);
  auto al = [](int64_t x) { return (x + 63) & ~(int64_t)63; };
  float* w = reinterpret_cast<float*>(p.ws);
  p.g = w;
  p.hh = p.g + al(tc * p.kk * kBwD);
  uint32_t* list = reinterpret_cast<uint32_t*>(p.hh + al(tc * p.kk * kBwD));
  uint32_t* cnt = list + al(tc * p.kk);
  uint32_t* off = cnt + al(keys + 1);
  uint32_t* cursor = off + al(keys + 1);
  const int64_t n4 = keys * kBwD / 4;
  const uint32_t zb = (uint32_t)std::min<int64_t>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(dsa_sparse_bwd_zero_kernel, dim3(zb), dim3(256), 0, stream, reinterpret_cast<float4*>(p.dk), n4);
  hipLaunchKernelGGL(dsa_sparse_bwd_zero_kernel, dim3(zb), dim3(256), 0, stream, reinterpret_cast<float4*>(p.dv), n4);
  const int64_t c4 = al(keys + 1) / 4;  // the counts, zeroed per chunk as float4 words
  const uint32_t cb = (uint32_t)std::min<int64_t>((c4 + 255) / 256, 4096);
  for (int64_t tok0 = 0; tok0 < BT; tok0 += tc) {
    const int64_t ntok = std::min<int64_t>(tc, BT - tok0);
    p.tok0 = tok0;
    const uint32_t eb = (uint32_t)((ntok * p.kk + 255) / 256);
    hipLaunchKernelGGL(dsa_sparse_bwd_zero_kernel, dim3(cb), dim3(256), 0, stream, reinterpret_cast<float4*>(cnt), c4);
    hipLaunchKernelGGL(dsa_sparse_bwd_count_kernel, dim3(eb), dim3(256), 0, stream, p, ntok, cnt);
    hipLaunchKernelGGL(dsa_sparse_bwd_scan_kernel, dim3(1), dim3(1024), 0, stream, cnt, off, cursor, keys);
    hipLaunchKernelGGL(dsa_sparse_bwd_fill_kernel, dim3(eb), dim3(256), 0, stream, p, ntok, cursor, list);
    hipLaunchKernelGGL(dsa_sparse_bwd_kernel, dim3((uint32_t)ntok), dim3(kBwThreads), 0, stream, p);
    hipLaunchKernelGGL(dsa_sparse_bwd_reduce_kernel, dim3((uint32_t)keys), dim3(kBwD), 0, stream, p, off, list);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sa

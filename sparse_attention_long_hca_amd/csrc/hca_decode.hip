// HCA decode attention (gfx950): one query per sequence and head.
//
// Method: [P1] §二.1, [P3] §架構創新 1 -- the query at position t = pos[b]
// attends to the compressed entries j < floor((t - window + 1) / blk)
// (capped at the cache size) and to the window tokens t - window < s <= t,
// which live in a ring of `window` slots (slot = s mod window).
//
// The step is bound by HBM: every visible K and V row is read once.  A
// workgroup (4 waves) handles one (batch, head, key split).  Each wave walks
// its keys 4 at a time, 16 lanes per key: lane (slot, part) reads 16-byte
// chunks part, part+16, ... of its key's K and V rows, so one load
// instruction covers 4 rows x 256 contiguous bytes.  The rows of the next
// group of keys are loaded while the current group is used, so every wave
// keeps two groups (16 KB) in flight.  Dot products use the bf16 dot2
// instruction with fp32 accumulation; the 16-lane reduction uses cross-lane
// shuffles; softmax is online per wave with the running max raised only when
// it grows by more than 2^8.  With more than one split per (batch, head) the
// partial (o, lse) go to the workspace and a second kernel combines them in
// split order.
//
// Wider query/key heads ([P3] §預訓練資料工程 item 3: qk 576 with v 512): the
// DR dims of q and K past the value width D are spread over a key's 16 lanes,
// 4 dims (8 bytes) each, so the extra part of a K row is one 128-byte line.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;

__device__ __forceinline__ int64_t hca_visible_dec(int64_t t, int64_t blk, int64_t window) {
  const int64_t x = t - window + 1;
  return x > 0 ? x / blk : 0;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// kFp8: the K/V rows are E4M3 codes (one byte per dim) with one fp32 scale
// per row; lane `part` of a key's 8 lanes then holds the 16-byte chunks
// (16 dims each) part, part+8, part+16, part+24 of the row, the codes are
// widened with the hardware conversion (exact: every E4M3 value is an fp32
// value), the dot product runs in fp32 and is multiplied by the K row's
// scale, and the V row's scale is folded into the probability.  bf16 rows:
// lane `part` holds the 16-byte chunks part, part+16, ... of the row.  Either
// way one load instruction reads whole 128-byte lines of a key's rows, which
// the non-temporal loads need (they keep nothing in cache for a later
// instruction to reuse).
constexpr int kDecFp8Lanes = 8;  // lanes per key with the FP8 cache (more keys in flight per wave)

template <int D, bool kFp8, int DR>
__global__ __launch_bounds__(kDecThreads) void hca_decode_kernel(HcaDecodeParams p) {
  constexpr int kLanes = kFp8 ? kDecFp8Lanes : 16;  // lanes per key
  static_assert(DR == 0 || (!kFp8 && DR == 4 * 16), "extra query/key dims: 4 per lane of a bf16 key");
  constexpr int kSlots = kWave / kLanes;   // keys per wave step
  constexpr int kPer = D / 8 / kLanes;     // groups of 8 dims per lane
  constexpr int kRowBytes = kFp8 ? D : 2 * D;        // V row; the first D dims of a K row
  constexpr int kKRowBytes = kRowBytes + 2 * DR;     // K row pitch
  constexpr int kLoads = kRowBytes / kLanes / 16;  // 16-byte loads per lane and row
  __shared__ float sh_o[kDecWaves][D];
  __shared__ float sh_m[kDecWaves], sh_l[kDecWaves];

  const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t split = lid % p.nsplit;
  const int64_t bh = lid / p.nsplit;
  const int64_t b = bh / p.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slot = lane / kLanes, part = lane % kLanes;
  // First dim of this lane's group i of 8 dims (FP8: a 16-byte chunk holds
  // groups 2j and 2j + 1).
  auto dim0 = [&](int i) { return kFp8 ? 16 * (part + kLanes * (i >> 1)) + 8 * (i & 1) : 8 * (part + kLanes * i); };
  // Byte offset in a row of this lane's 16-byte load j.
  auto load_off = [&](int j) { return 16 * (part + kLanes * j); };

  int64_t t = p.pos[b];
  if (t < 0) t = 0;
  const int64_t nc = imin64(p.Ncap, hca_visible_dec(t, p.blk, p.window));
  const int64_t nw = imin64(p.window, t + 1);
  const int64_t n_keys = nc + nw;
  const int64_t u_begin = split * p.keys_per_split;
  const int64_t u_end = imin64(n_keys, u_begin + p.keys_per_split);

  const bf16_t* q = reinterpret_cast<const bf16_t*>(p.q) + bh * (D + DR);
  const char* kc = reinterpret_cast<const char*>(p.kc) + bh * p.Ncap * kKRowBytes;
  const char* vc = reinterpret_cast<const char*>(p.vc) + bh * p.Ncap * kRowBytes;
  const char* rk = reinterpret_cast<const char*>(p.rk) + bh * p.window * kKRowBytes;
  const char* rv = reinterpret_cast<const char*>(p.rv) + bh * p.window * kRowBytes;
  const int64_t win_first = t - nw + 1;  // first window position

  // Query: bf16 pairs (bf16 cache) or fp32 (FP8 cache), dims dim0(i) .. +7.
  uint4 qc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) qc[i] = *reinterpret_cast<const uint4*>(q + dim0(i));
  // Extra query/key dims D + 4*part .. +3.
  const uint2 qr = DR ? *reinterpret_cast<const uint2*>(q + D + 4 * part) : make_uint2(0u, 0u);
  float qf[kFp8 ? kPer * 8 : 1];
  if constexpr (kFp8) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const uint32_t w[4] = {qc[i].x, qc[i].y, qc[i].z, qc[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[8 * i + 2 * e] = bf16_to_f32(w[e] & 0xffffu);
        qf[8 * i + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    }
  }

  float acc[kPer * 8];
#pragma unroll
  for (int i = 0; i < kPer * 8; ++i) acc[i] = 0.f;
  float m = -INFINITY, l = 0.f;

  // One group: keys g0 + slot (a group of kSlots consecutive keys).
  struct Rows {
    uint4 k[kLoads], v[kLoads];
    uint2 kr;      // extra K dims (DR > 0)
    float ks, vs;  // row scales (FP8 cache)
  };
  auto load = [&](int64_t g0, Rows& r) __attribute__((always_inline)) {
    const int64_t u = g0 + slot;
    r.ks = 0.f;
    r.vs = 0.f;
    if (u < u_end) {
      const char* krow;
      const char* vrow;
      if (u < nc) {
        krow = kc + u * kKRowBytes;
        vrow = vc + u * kRowBytes;
        if constexpr (kFp8) {
          r.ks = p.kc_scale[bh * p.Ncap + u];
          r.vs = p.vc_scale[bh * p.Ncap + u];
        }
      } else {
        const int64_t sl = (win_first + (u - nc)) % p.window;
        krow = rk + sl * kKRowBytes;
        vrow = rv + sl * kRowBytes;
        if constexpr (kFp8) {
          r.ks = p.rk_scale[bh * p.window + sl];
          r.vs = p.rv_scale[bh * p.window + sl];
        }
      }
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        r.k[j] = load_stream_u4(krow + load_off(j));
        r.v[j] = load_stream_u4(vrow + load_off(j));
      }
      r.kr = DR ? *reinterpret_cast<const uint2*>(krow + kRowBytes + 8 * part) : make_uint2(0u, 0u);
    } else {
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        r.k[j] = make_uint4(0u, 0u, 0u, 0u);
        r.v[j] = make_uint4(0u, 0u, 0u, 0u);
      }
      r.kr = make_uint2(0u, 0u);
    }
  };
  constexpr float kRescaleLog2 = 8.f;
  auto use = [&](int64_t g0, const Rows& r) __attribute__((always_inline)) {
    const bool valid = g0 + slot < u_end;
    float dot = 0.f;
    if constexpr (kFp8) {
      // Load j holds this lane's dims 16*j .. +15 (local order: groups 2j and
      // 2j + 1 of dim0), four codes per word.
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const uint32_t w[4] = {r.k[j].x, r.k[j].y, r.k[j].z, r.k[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[e], false);
          const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[e], true);
          const int d0 = 16 * j + 4 * e;
          dot = fmaf(qf[d0], lo[0], dot);
          dot = fmaf(qf[d0 + 1], lo[1], dot);
          dot = fmaf(qf[d0 + 2], hi[0], dot);
          dot = fmaf(qf[d0 + 3], hi[1], dot);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        dot = dot2_bf16(qc[i].x, r.k[i].x, dot);
        dot = dot2_bf16(qc[i].y, r.k[i].y, dot);
        dot = dot2_bf16(qc[i].z, r.k[i].z, dot);
        dot = dot2_bf16(qc[i].w, r.k[i].w, dot);
      }
      if constexpr (DR > 0) {
        dot = dot2_bf16(qr.x, r.kr.x, dot);
        dot = dot2_bf16(qr.y, r.kr.y, dot);
      }
    }
#pragma unroll
    for (int off = 1; off < kLanes; off <<= 1) dot += __shfl_xor(dot, off);
    if constexpr (kFp8) dot *= r.ks;
    const float x = valid ? dot * p.scale_log2 : -INFINITY;
    float gm = x;
#pragma unroll
    for (int off = kLanes; off < kWave; off <<= 1) gm = fmaxf(gm, __shfl_xor(gm, off));
    // gm is finite: the group has at least one valid key.
    if (gm > m + kRescaleLog2) {  // wave-uniform
      const float alpha = fast_exp2(m - gm);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < kPer * 8; ++i) acc[i] *= alpha;
      m = gm;
    }
    const float pr = fast_exp2(x - m);
    float ps = pr;
#pragma unroll
    for (int off = kLanes; off < kWave; off <<= 1) ps += __shfl_xor(ps, off);
    l += ps;
    if constexpr (kFp8) {
      const float pv = pr * r.vs;
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const uint32_t w[4] = {r.v[j].x, r.v[j].y, r.v[j].z, r.v[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[e], false);
          const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[e], true);
          const int d0 = 16 * j + 4 * e;
          acc[d0] = fmaf(pv, lo[0], acc[d0]);
          acc[d0 + 1] = fmaf(pv, lo[1], acc[d0 + 1]);
          acc[d0 + 2] = fmaf(pv, hi[0], acc[d0 + 2]);
          acc[d0 + 3] = fmaf(pv, hi[1], acc[d0 + 3]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const uint32_t w[4] = {r.v[i].x, r.v[i].y, r.v[i].z, r.v[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[i * 8 + 2 * e] = fmaf(pr, bf16_to_f32(w[e] & 0xffffu), acc[i * 8 + 2 * e]);
          acc[i * 8 + 2 * e + 1] = fmaf(pr, __uint_as_float(w[e] & 0xffff0000u), acc[i * 8 + 2 * e + 1]);
        }
      }
    }
  };

  // Groups of this wave: g0 = u_begin + kSlots*wave + stride*n, two in flight.
  constexpr int64_t kStride = kDecWaves * kSlots;
  Rows ra, rb;
  int64_t g = u_begin + (int64_t)wave * kSlots;
  if (g < u_end) load(g, ra);
  for (; g < u_end; g += 2 * kStride) {
    load(g + kStride, rb);
    use(g, ra);
    if (g + kStride >= u_end) break;
    load(g + 2 * kStride, ra);
    use(g + kStride, rb);
  }

  // Sum the key slots of the wave (lanes with equal part).
#pragma unroll
  for (int i = 0; i < kPer * 8; ++i) {
    float a = acc[i];
#pragma unroll
    for (int off = kLanes; off < kWave; off <<= 1) a += __shfl_xor(a, off);
    acc[i] = a;
  }
  if (slot == 0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) sh_o[wave][dim0(i) + e] = acc[i * 8 + e];
  }
  if (lane == 0) {
    sh_m[wave] = m;
    sh_l[wave] = l;
  }
  __syncthreads();

  // Combine the 4 waves (fixed order).
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, sh_m[w]);
  float scale_w[kDecWaves];
  float Lsum = 0.f;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    scale_w[w] = (M == -INFINITY) ? 0.f : fast_exp2(sh_m[w] - M);
    Lsum += scale_w[w] * sh_l[w];
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  const float lse2 = Lsum > 0.f ? M + __log2f(Lsum) : -INFINITY;
  for (int dd = threadIdx.x * 2; dd < D; dd += kDecThreads * 2) {
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      o0 += scale_w[w] * sh_o[w][dd];
      o1 += scale_w[w] * sh_o[w][dd + 1];
    }
    o0 *= inv;
    o1 *= inv;
    if (p.nsplit == 1) {
      *reinterpret_cast<uint32_t*>(reinterpret_cast<bf16_t*>(p.o) + bh * D + dd) = pack_bf16x2(o0, o1);
    } else {
      *reinterpret_cast<float2*>(p.part_o + (bh * p.nsplit + split) * D + dd) = make_float2(o0, o1);
    }
  }
  if (threadIdx.x == 0) {
    if (p.nsplit == 1) {
      if (p.lse) p.lse[bh] = lse2 * kLn2;
    } else {
      p.part_lse[bh * p.nsplit + split] = lse2;
    }
  }
}

// Combine the splits of one (batch, head) in split order.
template <int D>
__global__ __launch_bounds__(256) void hca_decode_combine_kernel(HcaDecodeParams p) {
  const int64_t bh = blockIdx.x;
  const float* pl = p.part_lse + bh * p.nsplit;
  float M = -INFINITY;
  for (int64_t s = 0; s < p.nsplit; ++s) M = fmaxf(M, pl[s]);
  float Lsum = 0.f;
  for (int64_t s = 0; s < p.nsplit; ++s) Lsum += (M == -INFINITY) ? 0.f : fast_exp2(pl[s] - M);
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  for (int dd = threadIdx.x * 2; dd < D; dd += 512) {
    float o0 = 0.f, o1 = 0.f;
    for (int64_t s = 0; s < p.nsplit; ++s) {
      const float w = (M == -INFINITY) ? 0.f : fast_exp2(pl[s] - M);
      const float2 v = *reinterpret_cast<const float2*>(p.part_o + (bh * p.nsplit + s) * D + dd);
      o0 = fmaf(w, v.x, o0);
      o1 = fmaf(w, v.y, o1);
    }
    *reinterpret_cast<uint32_t*>(reinterpret_cast<bf16_t*>(p.o) + bh * D + dd) = pack_bf16x2(o0 * inv, o1 * inv);
  }
  if (threadIdx.x == 0 && p.lse) p.lse[bh] = Lsum > 0.f ? (M + __log2f(Lsum)) * kLn2 : -INFINITY;
}

int64_t hca_decode_nsplit(int64_t BH, int64_t max_keys) {
  // Enough workgroups to fill 256 CUs several times over (about 1536: at
  // 1M context, B = 4, 6 splits per head measured faster than 8, 9 or 12 with
  // the FP8 cache and equal with bf16), but at least 256 keys per split so
  // the per-split fixed cost stays small.
  int64_t ns = (1536 + BH - 1) / BH;
  const int64_t cap = (max_keys + 255) / 256;
  if (ns > cap) ns = cap;
  if (ns < 1) ns = 1;
  return ns;
}

size_t hca_decode_workspace_bytes(int64_t BH, int64_t nsplit, int64_t d) {
  if (nsplit <= 1) return 0;
  return (size_t)(BH * nsplit * d + BH * nsplit) * sizeof(float);
}

hipError_t launch_hca_decode(const HcaDecodeParams& p, int cache, int d, int dv, hipStream_t stream) {
  if ((cache != 1 && cache != 2) || dv != 512 || (d != 512 && d != 576) || (cache == 2 && d != 512))
    return hipErrorInvalidValue;
  const int64_t BH = p.B * p.H;
  const dim3 grid((uint32_t)(BH * p.nsplit));
  if (cache == 2)
    hipLaunchKernelGGL((hca_decode_kernel<512, true, 0>), grid, dim3(kDecThreads), 0, stream, p);
  else if (d == 576)
    hipLaunchKernelGGL((hca_decode_kernel<512, false, 64>), grid, dim3(kDecThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((hca_decode_kernel<512, false, 0>), grid, dim3(kDecThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  hipLaunchKernelGGL(hca_decode_combine_kernel<512>, dim3((uint32_t)BH), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa

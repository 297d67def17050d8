// 32-row MFMA attention core (v_mfma_f32_32x32x16_bf16) for gfx950, used by
// the multi-query DSA sparse attention: one wave owns 32 query rows (heads),
// so every K/V tile read from LDS serves 32 rows instead of 16 and the LDS
// traffic per FLOP is half that of the 16-row core.
//
// Operand layouts (checked on gfx950), lane l, q = l/32:
//   A (32 x 16): A[l%32][8q + 0..7]     B (16 x 32): B[8q + 0..7][l%32]
//   C (32 x 32): value j (0..15) is C[8*(j/4) + 4q + j%4][l%32]
//
// Per tile of 32 keys and wave:
//   S^T[32 keys x 32 rows] = K . Q^T    (D/16 MFMAs; A = K rows from LDS)
//   lane l then holds the 16 keys {8m + 4q + i : m, i < 4} of row l%32; the
//   row's other 16 keys are in lane l^32 (one cross-lane step per reduction)
//   O^T[D x 32 rows] += V^T . P^T       (D/32 x 2 MFMAs; A = V via
//   transposing LDS reads).  The contraction over the 32 keys is split into
//   two k-steps of 16 whose k-slots map to keys 16s + 4q + {0..3, 8..11}:
//   exactly the values lane l holds, in order, so P needs no shuffles.
#pragma once

#include "attn_core.h"

namespace sa {

template <int D>
struct Attn32Regs {
  i16x8_t q[D / 16];      // Q^T operand: row l%32, dims 8q + 16*kstep .. +7
  f32x16_t o[D / 32];     // O^T accumulators, one 32x32 block per 32 dims
  float m;                // running max (log2 units) of row l%32
  float l;                // running sum
};

template <int D>
__device__ __forceinline__ void load_q32(Attn32Regs<D>& R, const bf16_t* qrow) {
  const int q = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint4 u = *reinterpret_cast<const uint4*>(qrow + ks * 16 + q * 8);
    R.q[ks] = __builtin_bit_cast(i16x8_t, u);
  }
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) R.o[nb][j] = 0.f;
  R.m = -INFINITY;
  R.l = 0.f;
}

// Per-lane LDS byte offsets for attend_tile32, computed once per kernel.
// Tiles use the AttnGeom<bf16_t, D, 1> layout: row r, 16-byte chunk c at
// r*D*2 + 16*(c ^ lds_swizzle32(r)).  The swizzle only flips bits 4..7 of
// the offset, so every operand read is (base ^ constant) + constant:
//   K read, k-step n:   (k ^ 32*(n%8)) + 256*(n/8)
//   V read, dims block nb, key half st, rows +8*hi:
//                       (v[hi] ^ 64*(nb%4)) + 256*(nb/4) + 8192*st
// which needs three base registers instead of sixteen.
struct Tile32Addr {
  uint32_t k, v0, v1;
};

template <int D>
__device__ __forceinline__ Tile32Addr tile32_addr() {
  static_assert(D * 2 == 512, "the V offsets below assume 512-byte rows");
  const int lane = threadIdx.x & 63;
  const int q = lane >> 5, r = lane & 31;
  const int sw = lds_swizzle32(r);
  Tile32Addr a;
  a.k = (uint32_t)r * 512u + 16u * (uint32_t)(q ^ (sw & 1)) + 32u * (uint32_t)(sw >> 1);
  // V: the lane's 16-lane group is (q, h = (l%32)/16), L = l%16; it reads
  // key 16*st + 4q + L/4 + 8*hi, dims 32*nb + 16h + 4*(L%4) .. +3.
  const int h = r >> 4, L = lane & 15;
  uint32_t v[2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const int key = 4 * q + (L >> 2) + 8 * hi;
    v[hi] = (uint32_t)key * 512u + 64u * (uint32_t)(L >> 2) +
            16u * (uint32_t)((2 * h + ((L & 3) >> 1)) ^ (q + 2 * hi)) + 8u * (uint32_t)(L & 1);
  }
  a.v0 = v[0];
  a.v1 = v[1];
  return a;
}

// S^T = K . Q^T for one 32-key tile in LDS (A = K row l%32, chunk q + 2*kstep).
// Returns the raw scores: value j is key 8*(j/4) + 4q + j%4 of row l%32.
// All LDS reads have been issued when this returns; the caller waits for
// them (lgkmcnt) before letting the K buffer be overwritten.
template <int D, int kAhead = 4>  // kAhead: LDS operand reads in flight
__device__ __forceinline__ f32x16_t qk32_ops(const i16x8_t* qb, const char* ks, Tile32Addr ad);

template <int D, int kAhead = 4>  // kAhead: LDS operand reads in flight
__device__ __forceinline__ f32x16_t attend_qk32(const Attn32Regs<D>& R, const char* ks, Tile32Addr ad) {
  return qk32_ops<D, kAhead>(R.q, ks, ad);
}

// The same product with the B operand given as registers: S^T = K . Q^T for
// qb[n] = this lane's Q^T operand of k-step n (row l%32, dims 16n + 8q .. +7).
template <int D, int kAhead>
__device__ __forceinline__ f32x16_t qk32_ops(const i16x8_t* qb, const char* ks, Tile32Addr ad) {
  constexpr int kSteps = D / 16;
  // Opaque copy: the derived offsets are recomputed next to their reads
  // instead of being hoisted out of the key loop into registers.
  asm volatile("" : "+v"(ad.k));
  auto kread = [&](int n) -> i16x8_t {
    return __builtin_bit_cast(i16x8_t, lds_read_b128(ks, (ad.k ^ (32u * (n & 7))) + 256u * (n >> 3)));
  };
  f32x16_t s;
#pragma unroll
  for (int j = 0; j < 16; ++j) s[j] = 0.f;
  i16x8_t ka[kAhead];
#pragma unroll
  for (int n = 0; n < kAhead; ++n) ka[n] = kread(n);
#pragma unroll
  for (int n = 0; n < kSteps; ++n) {
    __builtin_amdgcn_sched_barrier(0);
    s = mfma_bf16_32x32x16(ka[n % kAhead], qb[n], s);
    if (n + kAhead < kSteps) ka[n % kAhead] = kread(n + kAhead);
  }
  __builtin_amdgcn_sched_barrier(0);
  return s;
}

// Probabilities (or any weights) of one tile in the S^T accumulator layout ->
// the B operand of the P.V product.  The contraction over the tile's 32 keys
// is two k-steps of 16 whose k-slots map to keys 16*st + 4q + {0..3, 8..11}:
// exactly the values this lane holds, in order, so no shuffles are needed.
__device__ __forceinline__ void pack_p32(const f32x16_t& s, i16x8_t pf[2]) {
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const uint4 u = make_uint4(pack_bf16x2(s[8 * st + 0], s[8 * st + 1]), pack_bf16x2(s[8 * st + 2], s[8 * st + 3]),
                               pack_bf16x2(s[8 * st + 4], s[8 * st + 5]), pack_bf16x2(s[8 * st + 6], s[8 * st + 7]));
    pf[st] = __builtin_bit_cast(i16x8_t, u);
  }
}

// acc[i] += V^T[dims 32*(nb0+i) .. +31] . P^T for i < NB, with V a 32-row
// tile of 256-dim rows in LDS (read transposed) and pf from pack_p32.
// kOutT: the same product with the MFMA operands swapped, which gives the
// transposed block (acc[i] += P . V[:, dims 32*(nb0+i) ..]): lane l then
// holds dim 32*(nb0+i) + l%32 of rows 8*(j/4) + 4q + j%4.
template <int NB, int kAhead = 2, bool kOutT = false>
__device__ __forceinline__ void pv32_acc(f32x16_t* acc, const i16x8_t pf[2], const char* vs, Tile32Addr ad, int nb0) {
  constexpr int kPairs = NB * 2;  // (dims block, key half)
  asm volatile("" : "+v"(ad.v0), "+v"(ad.v1));
  auto vread = [&](int i) -> i16x8_t {
    const int nb = nb0 + (i >> 1), st = i & 1;
    const uint32_t x = 64u * (uint32_t)(nb & 3), c = 256u * (uint32_t)(nb >> 2) + 8192u * (uint32_t)st;
    const i16x4_t lo = lds_read_tr16_b64(vs + ((ad.v0 ^ x) + c));
    const i16x4_t hi = lds_read_tr16_b64(vs + ((ad.v1 ^ x) + c));
    return i16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  i16x8_t va[kAhead];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) va[i] = vread(i);
#pragma unroll
  for (int i = 0; i < kPairs; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kOutT)
      acc[i >> 1] = mfma_bf16_32x32x16(pf[i & 1], va[i % kAhead], acc[i >> 1]);
    else
      acc[i >> 1] = mfma_bf16_32x32x16(va[i % kAhead], pf[i & 1], acc[i >> 1]);
    if (i + kAhead < kPairs) va[i % kAhead] = vread(i + kAhead);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Online-softmax update and O^T += V^T . P^T for one tile, given its logits
// s (scaled, log2 units, -INFINITY for keys that take no part) and mx, this
// lane's maximum of them.
template <int D>
__device__ __forceinline__ void softmax_pv32(Attn32Regs<D>& R, f32x16_t s, float mx, const char* vs, Tile32Addr ad) {
  constexpr int kAhead = 2;  // pairs of LDS reads in flight (register budget)
  asm volatile("" : "+v"(ad.v0), "+v"(ad.v1));

  mx = max_xor32(mx);
  // Lazy rescale as in the 16-row core: only when the running max grows by
  // more than 2^8.
  constexpr float kRescaleLog2 = 8.f;
  if (__any(mx > R.m + kRescaleLog2)) {
    const float m_new = fmaxf(R.m, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(R.m - m_new);
    R.l *= alpha;
    R.m = m_new;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) R.o[nb] *= alpha;
  }
  const float base = (R.m == -INFINITY) ? 0.f : R.m;
  float rs = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float p = fast_exp2(s[j] - base);
    s[j] = p;
    rs += p;
  }
  rs = sum_xor32(rs);
  R.l += rs;

  i16x8_t pf[2];
  pack_p32(s, pf);
  pv32_acc<D / 32, kAhead>(R.o, pf, vs, ad, 0);
}

// Mask, online-softmax update and O^T += V^T . P^T for the tile whose raw
// scores attend_qk32 returned.  Bit n of key_mask (wave-uniform) says whether
// key n of the tile takes part.
template <int D>
__device__ __forceinline__ void attend_pv32(Attn32Regs<D>& R, f32x16_t s, const char* vs, float scale_log2,
                                            uint32_t key_mask, Tile32Addr ad) {
  const int q = (threadIdx.x & 63) >> 5;
  // Shift the mask by 4q once, then every test is against a compile-time bit.
  const uint32_t kbits = key_mask >> (4 * q);
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float x = (kbits & (1u << (8 * (j >> 2) + (j & 3)))) ? s[j] * scale_log2 : -INFINITY;
    s[j] = x;
    mx = fmaxf(mx, x);
  }
  softmax_pv32<D>(R, s, mx, vs, ad);
}

// As attend_pv32, with a per-row key range instead: key n of the tile takes
// part in row l%32 iff lo <= n <= hi (this lane's bounds).
template <int D>
__device__ __forceinline__ void attend_pv32_range(Attn32Regs<D>& R, f32x16_t s, const char* vs, float scale_log2,
                                                  int lo, int hi, Tile32Addr ad) {
  const int q = (threadIdx.x & 63) >> 5;
  // Key of value j: 8*(j/4) + 4q + j%4; shift the bounds by 4q once.
  const int lo_q = lo - 4 * q, hi_q = hi - 4 * q;
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int kj = 8 * (j >> 2) + (j & 3);
    const float x = (kj >= lo_q && kj <= hi_q) ? s[j] * scale_log2 : -INFINITY;
    s[j] = x;
    mx = fmaxf(mx, x);
  }
  softmax_pv32<D>(R, s, mx, vs, ad);
}

// Normalise and write row l%32 (bf16), and its lse; lane holds dims
// 32*nb + 8*m + 4q + {0..3}.
template <int D>
__device__ __forceinline__ void finish_rows32(const Attn32Regs<D>& R, bf16_t* orow, float* lse_out) {
  const int q = (threadIdx.x & 63) >> 5;
  const float inv = R.l > 0.f ? 1.f / R.l : 0.f;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int dim = 32 * nb + 8 * m + 4 * q;
      const uint2 u = make_uint2(pack_bf16x2(R.o[nb][4 * m] * inv, R.o[nb][4 * m + 1] * inv),
                                 pack_bf16x2(R.o[nb][4 * m + 2] * inv, R.o[nb][4 * m + 3] * inv));
      *reinterpret_cast<uint2*>(orow + dim) = u;
    }
  if (lse_out && q == 0) *lse_out = R.l > 0.f ? (R.m + __log2f(R.l)) * kLn2 : -INFINITY;
}

// Split-K variant: fp32 normalised rows and the log2-domain normaliser.
template <int D>
__device__ __forceinline__ void finish_rows32_partial(const Attn32Regs<D>& R, float* orow, float* lse2_out) {
  const int q = (threadIdx.x & 63) >> 5;
  const float inv = R.l > 0.f ? 1.f / R.l : 0.f;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int dim = 32 * nb + 8 * m + 4 * q;
      *reinterpret_cast<float4*>(orow + dim) = make_float4(R.o[nb][4 * m] * inv, R.o[nb][4 * m + 1] * inv,
                                                           R.o[nb][4 * m + 2] * inv, R.o[nb][4 * m + 3] * inv);
    }
  if (q == 0) *lse2_out = R.l > 0.f ? R.m + __log2f(R.l) : -INFINITY;
}

}  // namespace sa

// Shared pieces of the exact top-k selections (dsa_topk.hip, dsa_fused.hip):
// the order-preserving key of an fp32 score, wave and workgroup scans and
// reductions, and the histogram bin selection.
#pragma once
#include "common.h"

namespace sa {

// Order-preserving 32-bit key of an fp32 score: larger scores give larger
// keys; -0.0 maps as +0.0.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, off));
  return x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, off));
  return x;
}
__device__ __forceinline__ uint32_t uniform_u32(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then the
// row broadcasts 15 and 31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}
// Sum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(x), 63);
}

// Orders this wave's earlier LDS accesses before its later ones for the
// compiler (the hardware executes one wave's LDS instructions in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// hist[bin] += 1 for every lane of the wave with bin < 256.  When the lowest
// active lane's bin is shared by at least 16 lanes (scores near a row's top
// fall in few high-byte bins, where lane-by-lane atomics to one address would
// serialise) the lanes of each distinct bin are counted with one LDS atomic;
// otherwise every lane adds its own.  Call from uniform control flow.
__device__ __forceinline__ void lds_hist_add(uint32_t* hist, uint32_t bin) {
  const int lane = threadIdx.x & 63;
  uint64_t act = __ballot(bin < 256u);
  if (act == 0ull) return;
  {
    const int ld = __builtin_ctzll(act);
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, ld);
    if (__popcll(__ballot(bin == lb)) < 16) {
      if (bin < 256u) atomicAdd(&hist[bin], 1u);
      return;
    }
  }
  while (act) {
    const int ld = __builtin_ctzll(act);
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, ld);
    const uint64_t m = __ballot(bin == lb);
    if (lane == ld) atomicAdd(&hist[lb], (uint32_t)__popcll(m));
    act &= ~m;
  }
}

// One wave, 256 bins in LDS (16-byte aligned): the bin where the count from
// the top reaches need (1 <= need <= total).  *bin, *above (count in higher
// bins) and *count (the bin's count) are uniform over the wave.
__device__ __forceinline__ void wave_top_bin256(const uint32_t* hist, uint32_t need, uint32_t* bin, uint32_t* above,
                                                uint32_t* count) {
  const int lane = threadIdx.x & 63;
  const uint4 v = reinterpret_cast<const uint4*>(hist)[63 - lane];  // lane 0 holds the top four bins
  const uint32_t cs[4] = {v.w, v.z, v.y, v.x};
  const uint32_t s = v.x + v.y + v.z + v.w;
  const uint32_t incl = wave_incl_scan(s);
  const int src = __ffsll((unsigned long long)__ballot(incl >= need)) - 1;
  uint32_t ab = incl - s, b = 0u, a = 0u, c = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (ab < need && ab + cs[j] >= need) {
      b = (uint32_t)(4 * (63 - lane) + 3 - j);
      a = ab;
      c = cs[j];
    }
    ab += cs[j];
  }
  *bin = (uint32_t)__builtin_amdgcn_readlane((int)b, src);
  *above = (uint32_t)__builtin_amdgcn_readlane((int)a, src);
  *count = (uint32_t)__builtin_amdgcn_readlane((int)c, src);
}

// Bin width exponent for 256 bins over an interval of (range + 1) keys.
__device__ __forceinline__ uint32_t bin_shift256(uint32_t range) {
  const int bits = 32 - __clz((int)range);
  return bits > 8 ? (uint32_t)(bits - 8) : 0u;
}

// Bin width exponent for an interval of (range + 1) keys: bins of 2^shift
// keys with range >> shift in [1024, 2047] (or shift 0 for small ranges).
__device__ __forceinline__ uint32_t bin_shift(uint32_t range) {
  const int bits = 32 - __clz((int)range);  // 1..32 for range >= 1
  return bits > 11 ? (uint32_t)(bits - 11) : 0u;
}

// Inclusive scan of one value per thread over the whole workgroup (<= 1024
// threads).  `scratch` holds >= 16 ints.  Returns the inclusive prefix; total
// receives the workgroup sum.
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t x, uint32_t* scratch, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = (blockDim.x + 63) >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const uint32_t v = scratch[w];
    if (w < wave) before += v;
    tot += v;
  }
  __syncthreads();
  total = tot;
  return x + before;
}

// Two targets at once: for each t in {t1, t2} with 1 <= t <= total, the bin
// where the count from the top reaches t (outputs as in select_bin; a target
// above the total leaves its outputs untouched).  Ends with a barrier.
__device__ inline void select_bins2(const uint32_t* hist, int nbins, uint32_t t1, uint32_t t2, uint32_t* scratch,
                             uint32_t* out /* bin1, above1, bin2, above2 */) {
  const int per = (nbins + blockDim.x - 1) / blockDim.x;
  const int hi = nbins - (int)threadIdx.x * per;
  uint32_t local = 0;
  for (int j = 1; j <= per; ++j) {
    const int bin = hi - j;
    if (bin >= 0) local += hist[bin];
  }
  uint32_t tot;
  const uint32_t incl = block_inclusive_scan(local, scratch, tot);
  uint32_t above = incl - local;
  for (int j = 1; j <= per; ++j) {
    const int bin = hi - j;
    if (bin < 0) break;
    const uint32_t c = hist[bin];
    if (above < t1 && above + c >= t1) {
      out[0] = (uint32_t)bin;
      out[1] = above;
    }
    if (above < t2 && above + c >= t2) {
      out[2] = (uint32_t)bin;
      out[3] = above;
    }
    above += c;
  }
  __syncthreads();
}

// Given hist[0..nbins) and need >= 1 (<= total count), find the bin where the
// count from the top reaches need.  Result: *sel_bin, *sel_above (count in
// bins strictly above).  Uses all threads.
__device__ inline void select_bin(const uint32_t* hist, int nbins, uint32_t need, uint32_t* scratch, uint32_t* sel_bin,
                           uint32_t* sel_above) {
  const int per = (nbins + blockDim.x - 1) / blockDim.x;  // 1 or 2
  // Thread t owns bins [hi - per, hi) with hi = nbins - t*per (thread 0 = top bins).
  const int hi = nbins - (int)threadIdx.x * per;
  uint32_t local = 0;
  for (int j = 1; j <= per; ++j) {
    const int bin = hi - j;
    if (bin >= 0) local += hist[bin];
  }
  uint32_t tot;
  const uint32_t incl = block_inclusive_scan(local, scratch, tot);
  uint32_t above = incl - local;  // count in bins above this thread's range
  for (int j = 1; j <= per; ++j) {
    const int bin = hi - j;
    if (bin < 0) break;
    const uint32_t c = hist[bin];
    if (above < need && above + c >= need) {
      *sel_bin = (uint32_t)bin;
      *sel_above = above;
    }
    above += c;
  }
  __syncthreads();
}

}  // namespace sa

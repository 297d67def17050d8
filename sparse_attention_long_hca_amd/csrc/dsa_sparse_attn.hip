// DSA sparse attention over the selected positions (gfx950).
//
// Method: [P1] §二.1, [P3] §架構創新 1 -- core attention runs only on the
// top-K positions chosen by the indexer, so the per-query cost does not
// depend on the context length; MLA heads are 256 wide.  Multi-query layout:
// the query heads of a token share one K row and one V row per position.
//
// One workgroup per query token: its 64 heads are the rows of two 32x32 MFMA
// tiles (2 waves x 32 heads), so every gathered K/V row is read once and used
// by all heads.  The index list is walked in tiles of 32 positions; each
// 512-byte row is gathered with 16-byte loads by 32 consecutive lanes (one
// contiguous row per half-wave).  Indices outside [0, S) are skipped; a tile
// without any valid index is skipped entirely.
#include <type_traits>

#include "attn_core32.h"
#include "kernels.h"

namespace sa {

constexpr int kDsaMaxK = 2048;  // longest index list per query

constexpr int kDsaWaves = 2;                   // 2 waves x 32 heads = 64 heads
constexpr uint32_t kResidentPerXcd = 128;      // workgroups resident on one XCD (32 CUs x 4)
constexpr int kDsaThreads = kDsaWaves * kWave;  // 128

template <int D>
__global__ __launch_bounds__(kDsaThreads) __attribute__((amdgpu_waves_per_eu(2))) void dsa_sparse_kernel(DsaSparseParams p) {
  using T = bf16_t;
  using G = AttnGeom<T, D, 1>;
  // One K tile and one V tile (16 KB each for d = 256) in separate arrays,
  // plus the index list: four workgroups share a CU.  The next K tile is
  // loaded while this tile's softmax and PV run, the next V tile while the
  // next QK runs.
  __shared__ __attribute__((aligned(16))) char kl[G::kTileBytes];
  __shared__ __attribute__((aligned(16))) char vl[G::kTileBytes];
  __shared__ int32_t sidx[kDsaMaxK];

  // Tokens are dealt round-robin over the XCDs (the hardware's own order):
  // early tokens see fewer than k positions, and a contiguous range per XCD
  // would leave the XCD holding them idle at the end.
  const int64_t lid = blockIdx.x;
  const int64_t tok = lid / p.nsplit;  // b*T + i
  const int split = (int)(lid % p.nsplit);
  const int64_t b = tok / p.T;
  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  constexpr int kHq = 64;

  const T* q = reinterpret_cast<const T*>(p.q) + tok * kHq * D;
  const T* kb = reinterpret_cast<const T*>(p.k) + b * p.S * D;
  const T* vb = reinterpret_cast<const T*>(p.v) + b * p.S * D;
  const int32_t* idx = p.idx + tok * p.kk;
  T* o = reinterpret_cast<T*>(p.o) + tok * kHq * D;
  const int h = wave * 32 + (lane & 31);
  const int kk = (int)p.kk;
  const int64_t S = p.S;

  // Index list -> LDS, out-of-range entries and the tail of the last tile
  // replaced by -1.
  const int kk_pad = (kk + kBN - 1) / kBN * kBN;
  for (int n = threadIdx.x; n < kk_pad; n += kDsaThreads) {
    const int32_t s = n < kk ? idx[n] : -1;
    sidx[n] = (s >= 0 && s < S) ? s : -1;
  }
  Attn32Regs<D> R;
  load_q32<D>(R, q + h * D);
  const Tile32Addr ad = tile32_addr<D>();
  __syncthreads();  // the index list is in LDS

  // This workgroup's share of the index list: tiles [t_first, t_first + n_tiles).
  const int t_first = split * (int)p.tiles_per_split;
  const int n_tiles = max(0, min((kk + kBN - 1) / kBN - t_first, (int)p.tiles_per_split));
  // Tile order.  Workgroups on one XCD start one after another, so without
  // care the resident ones sit at every phase of their tile loops and gather
  // from the whole key range at once.  Starting workgroup j of its XCD at
  // tile j * n_tiles / kResidentPerXcd (and wrapping around) lines the
  // resident workgroups up on about the same tile at the same time; since
  // neighbouring tokens' sorted index lists cover the key range at the same
  // rate, their gathers then share a narrow key window in L2.  (The softmax
  // is order-independent up to rounding.)
  int rot = 0;
  if (p.nsplit == 1 && n_tiles > 0) rot = (int)((blockIdx.x / kNumXcd) * (uint32_t)n_tiles / kResidentPerXcd % (uint32_t)n_tiles);
  auto tile_of = [=](int t) {
    const int u = t + rot;
    return u < n_tiles ? u : u - n_tiles;
  };
  // The gather rows of the next tile are read from the index list at the
  // start of a step, a whole step before its K and V loads are sent (both use
  // them): the loads then do not wait on an LDS read (about 3% of the time).
  // The 8 registers they take come from keeping 2 instead of 4 K operand
  // reads in flight in QK, which alone changes nothing measurable.
  constexpr int kPerW = StageGeom<T, D, kDsaWaves>::kPerWave;
  int nrow[kPerW];
  auto fetch_rows = [&](int t) {
    const int32_t* trow = sidx + (t_first + tile_of(t)) * kBN;
#pragma unroll
    for (int j = 0; j < kPerW; ++j) nrow[j] = trow[stage_row_of<T, D, kDsaWaves, 1>(j)];
  };
  auto issue_k = [&]() { stage_rows_pre<T, D, kDsaWaves, 1>(kl, kb, nrow); };
  auto issue_v = [&]() { stage_rows_pre<T, D, kDsaWaves, 1>(vl, vb, nrow); };

  // The last tile is peeled off (more = false) so that every load issue in
  // the loop is unconditional: the compiler's wait tracking then keeps the K
  // and V buffers apart instead of waiting for every load before an LDS
  // read.  Each wait covers only the buffer about to be read (a thread's
  // loads complete in issue order, kLoads per buffer).
  constexpr int kLoads = StageGeom<T, D, kDsaWaves>::kPerWave;
  // Keys of a tile that take part (bit r: entry r is valid).  The next
  // tile's entries are read at the start of this tile's step and its mask is
  // formed after this tile's QK, so a tile's first MFMA does not wait on that
  // LDS read after the barrier (about 1% of the time).
  auto tile_mask = [&](int t) {
    return (uint32_t)(__ballot(sidx[(t_first + tile_of(t)) * kBN + (lane & 31)] >= 0) & 0xffffffffull);
  };
  uint32_t mask_next = 0u;
  auto step = [&](int t, auto more_tag) __attribute__((always_inline)) {
    constexpr bool more = decltype(more_tag)::value;
    const uint32_t mask = mask_next;
    int32_t vnext = -1;
    if constexpr (more) {
      fetch_rows(t + 1);
      vnext = sidx[(t_first + tile_of(t + 1)) * kBN + (lane & 31)];
    }
    wait_loads<kLoads>();  // K of tile t has landed (its V may be in flight)
    lds_barrier();         // ... for both waves
    f32x16_t s;
    if (mask) s = attend_qk32<D, 2>(R, kl, ad);
    if constexpr (more) mask_next = (uint32_t)(__ballot(vnext >= 0) & 0xffffffffull);
    wait_lgkmcnt0();
    lds_barrier();  // both waves are done with the K tile
    if constexpr (more) {
      issue_k();  // tile t + 1
      wait_loads<kLoads>();  // V of tile t has landed (the next K may be in flight)
    } else {
      wait_loads<0>();
    }
    lds_barrier();
    if (mask) attend_pv32<D>(R, s, vl, p.scale_log2, mask, ad);
    if constexpr (more) {
      wait_lgkmcnt0();
      lds_barrier();  // both waves are done with the V tile
      issue_v();  // tile t + 1
    }
  };

  wait_vmcnt<0>();  // Q is in registers before any tile load is in flight
  if (n_tiles > 0) {
    fetch_rows(0);
    mask_next = tile_mask(0);
    issue_k();
    issue_v();
    for (int t = 0; t + 1 < n_tiles; ++t) step(t, std::true_type{});
    step(n_tiles - 1, std::false_type{});
  }
  if (p.nsplit == 1) {
    finish_rows32<D>(R, o + h * D, p.lse ? p.lse + tok * kHq + h : nullptr);
  } else {
    const int64_t ps = tok * p.nsplit + split;
    finish_rows32_partial<D>(R, p.part_o + (ps * kHq + h) * D, p.part_lse + ps * kHq + h);
  }
}

// Merge the splits of one (token, head) in split order: weights
// exp2(lse_s - max).  One workgroup per (token, head), one thread per dim;
// the split weights are computed once into LDS, then every thread sums its
// dim over the splits with independent loads.
template <int D>
__global__ __launch_bounds__(D) void dsa_sparse_combine_kernel(DsaSparseParams p) {
  constexpr int kHq = 64;
  constexpr int kMaxSplit = kDsaMaxK / kBN;  // one tile per split at most
  __shared__ float wgt[kMaxSplit];
  __shared__ float stat[2];
  const int64_t th = blockIdx.x;  // tok * kHq + h
  const int64_t tok = th / kHq;
  const int h = (int)(th % kHq);
  const int ns = (int)p.nsplit;
  const float* pl = p.part_lse + tok * ns * kHq + h;  // stride kHq per split
  if (threadIdx.x < kWave) {
    // Wave 0: max and weights (fixed order of the splits in the sum below).
    float M = -INFINITY;
    for (int s = threadIdx.x; s < ns; s += kWave) M = fmaxf(M, pl[s * kHq]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    for (int s = threadIdx.x; s < ns; s += kWave) wgt[s] = (M == -INFINITY) ? 0.f : fast_exp2(pl[s * kHq] - M);
    if (threadIdx.x == 0) stat[0] = M;
  }
  __syncthreads();
  float wsum = 0.f, acc = 0.f;
  const float* po = p.part_o + (tok * ns * kHq + h) * D + threadIdx.x;  // stride kHq*D per split
  constexpr int kU = 8;
  int s = 0;
  for (; s + kU <= ns; s += kU) {
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = po[(int64_t)(s + u) * kHq * D];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      wsum += wgt[s + u];
      acc = fmaf(wgt[s + u], v[u], acc);
    }
  }
  for (; s < ns; ++s) {
    wsum += wgt[s];
    acc = fmaf(wgt[s], po[(int64_t)s * kHq * D], acc);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  reinterpret_cast<bf16_t*>(p.o)[th * D + threadIdx.x] = (bf16_t)f32_to_bf16_rne(acc * inv);
  if (p.lse && threadIdx.x == 0) p.lse[th] = wsum > 0.f ? (stat[0] + __log2f(wsum)) * kLn2 : -INFINITY;
}

// Decode-sized calls (few tokens) split each token's index list over several
// workgroups so that more CUs gather rows at once.  About 128 workgroups in
// all: more splits cost more in partial results (64 KB per split and token)
// than they gain in parallel gathers.
int64_t dsa_sparse_nsplit(int64_t BT, int64_t kk) {
  const int64_t tiles = (kk + kBN - 1) / kBN;
  if (BT >= 512) return 1;
  int64_t ns = (128 + BT - 1) / BT;
  if (ns > tiles) ns = tiles;
  return ns < 1 ? 1 : ns;
}

size_t dsa_sparse_workspace_bytes(int64_t BT, int64_t nsplit, int64_t hq, int64_t d) {
  if (nsplit <= 1) return 0;
  return (size_t)(BT * nsplit * hq * (d + 1)) * sizeof(float);
}

hipError_t launch_dsa_sparse(const DsaSparseParams& p, int d, int hq, hipStream_t stream) {
  if (d != 256 || hq != 64) return hipErrorInvalidValue;
  const int64_t nblocks = p.B * p.T * p.nsplit;
  hipLaunchKernelGGL(dsa_sparse_kernel<256>, dim3((uint32_t)nblocks), dim3(kDsaThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  hipLaunchKernelGGL(dsa_sparse_combine_kernel<256>, dim3((uint32_t)(p.B * p.T * 64)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa

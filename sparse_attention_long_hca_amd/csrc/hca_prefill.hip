// HCA prefill attention (gfx950).
//
// Method: [P1] §二.1 and [P3] §架構創新 1 -- each query attends to the
// compressed history entries plus a window of recent uncompressed tokens.
// Visibility: compressed entry j is visible to query t iff
// (j+1)*blk - 1 <= t - window; raw token s iff t - window < s <= t.
//
// Work split: one workgroup per (batch*head, 64-query tile).  The key stream
// of a tile is first the compressed entries visible to its last query (in
// tiles of 32), then the raw band [t0-window+1, t_last] (in tiles of 32).  A
// wave skips the MFMA work of a tile that none of its 16 queries can see.
// K and V tiles are staged with direct global->LDS loads.
// Workgroups of one head are kept on one XCD (shared L2 for the compressed
// cache and the overlapping raw band) and the longest tiles start first.
#include <type_traits>

#include "attn_core32.h"
#include "kernels.h"

namespace sa {

// Number of compressed entries visible to the query at position t.
__device__ __forceinline__ int hca_visible(int t, int blk, int window) {
  const int x = t - window + 1;
  return x > 0 ? x / blk : 0;
}

template <typename T, int D>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2))) void hca_prefill_kernel(HcaPrefillParams p) {
  using G = AttnGeom<T, D>;
  __shared__ __attribute__((aligned(16))) char kbuf[G::kTileBytes];
  __shared__ __attribute__((aligned(16))) char vbuf[G::kTileBytes];

  // Positions fit in 32 bits (checked on the host); pointer offsets are 64-bit.
  const int n_qtiles = (int)p.n_qtiles;
  const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = (int)(lid / (uint32_t)n_qtiles);
  const int qt = n_qtiles - 1 - (int)(lid % (uint32_t)n_qtiles);  // longest tiles first
  const int Tn = (int)p.T, blk = (int)p.blk, W = (int)p.window, Nc = (int)p.Nc;
  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const int L = lane & 15;

  const int64_t head_off = (int64_t)bh * Tn * D;
  const T* q = reinterpret_cast<const T*>(p.q) + head_off;
  const T* k = reinterpret_cast<const T*>(p.k) + head_off;
  const T* v = reinterpret_cast<const T*>(p.v) + head_off;
  const T* kc = reinterpret_cast<const T*>(p.kc) + (int64_t)bh * Nc * D;
  const T* vc = reinterpret_cast<const T*>(p.vc) + (int64_t)bh * Nc * D;
  T* o = reinterpret_cast<T*>(p.o) + head_off;

  {
    const int t0 = qt * kBM;
    const int tw = t0 + wave * kRowsPerWave;  // first query of this wave
    const int tq = tw + L;                    // this lane's query
    const bool qvalid = tq < Tn;

    AttnRegs<T, D> R;
    load_q(R, qvalid ? q + (int64_t)tq * D : nullptr);

    // Key stream of the tile.
    const int t_last = min(t0 + kBM - 1, Tn - 1);
    const int nc = min(Nc, hca_visible(t_last, blk, W));
    const int n_ctiles = (nc + kBN - 1) / kBN;
    const int s_lo = max(0, t0 - W + 1);
    const int n_rtiles = (t_last - s_lo + kBN) / kBN;
    const int n_tiles = n_ctiles + n_rtiles;
    // Raw tiles are taken in a rotated order: at step `tile` this workgroup
    // reads the band tile whose global index (s_lo / kBN + r) is congruent to
    // `tile` modulo n_rtiles.  Co-resident tiles of one head overlap in most
    // of their band, and the rotation makes them read the shared rows at the
    // same step, while those rows are still in L2.
    const int rot = n_rtiles > 0 ? ((n_ctiles - s_lo / kBN) % n_rtiles + n_rtiles) % n_rtiles : 0;
    auto band = [&](int tile) {
      const int r = tile - n_ctiles + rot;
      return r >= n_rtiles ? r - n_rtiles : r;
    };

    // This lane's visibility limits.
    const int vis_c = qvalid ? min(Nc, hca_visible(tq, blk, W)) : 0;
    const int win_lo = tq - W + 1;
    // This wave's limits (for skipping whole tiles).
    const bool wvalid = tw < Tn;
    const int tw_last = min(tw + kRowsPerWave - 1, Tn - 1);
    const int wave_nc = wvalid ? min(Nc, hca_visible(tw_last, blk, W)) : 0;
    const int wave_lo = tw - W + 1;

    // Tile t < n_ctiles: compressed entries [32t, 32t+32) of kc/vc; otherwise
    // raw positions from s_lo onwards.  Rows past the segment end are padding.
    auto rows_of = [&](int tile) {
      const bool ct = tile < n_ctiles;
      const int first = ct ? tile * kBN : s_lo + band(tile) * kBN;
      const int last = ct ? nc - 1 : t_last;
      return [=](int r) -> int {
        const int x = first + r;
        return x <= last ? x : -1;
      };
    };
    auto issue_k = [&](int tile) { stage_rows_async<T, D>(kbuf, tile < n_ctiles ? kc : k, rows_of(tile)); };
    auto issue_v = [&](int tile) { stage_rows_async<T, D>(vbuf, tile < n_ctiles ? vc : v, rows_of(tile)); };

    // One K tile and one V tile per workgroup (32 KB each for d = 512), so
    // two workgroups share a CU.  The next K tile streams in while this
    // tile's softmax and PV run, the next V tile while the next QK runs; each
    // wait covers only the buffer about to be read (loads of one thread
    // complete in issue order, kLoads per buffer).  Visibility inside a tile
    // is a per-lane key range [lo, hi]: compressed tile: key < vis_c - j0;
    // raw tile: win_lo <= s0 + key <= tq.
    constexpr int kLoads = StageGeom<T, D>::kPerWave;
    // The last tile is peeled off (more = false) so that every load issue in
    // the loop is unconditional: the compiler's wait tracking then keeps the
    // K and V buffers apart instead of waiting for every load before an LDS
    // read.
    auto step = [&](int tile, auto more_tag) __attribute__((always_inline)) {
      constexpr bool more = decltype(more_tag)::value;
      const bool ctile = tile < n_ctiles;
      const int j0 = tile * kBN;
      const int s0 = s_lo + band(tile) * kBN;
      const bool need = ctile ? (j0 < wave_nc) : (wvalid && s0 <= tw_last && s0 + kBN - 1 >= wave_lo);
      const int lo = ctile ? 0 : win_lo - s0;
      const int hi = ctile ? vis_c - j0 - 1 : tq - s0;

      wait_loads<kLoads>();  // K of this tile has landed (its V may be in flight)
      lds_barrier();         // ... for every wave
      PFrag P;
      if (need) P = attend_qk<T, D>(R, kbuf, p.scale_log2, [=](int key) { return key >= lo && key <= hi; });
      wait_lgkmcnt0();
      lds_barrier();  // every wave is done reading the K tile
      if constexpr (more) {
        issue_k(tile + 1);
        wait_loads<kLoads>();  // V of this tile has landed (the next K may be in flight)
      } else {
        wait_loads<0>();
      }
      lds_barrier();
      if (need) attend_pv<T, D>(R, vbuf, P);
      if constexpr (more) {
        wait_lgkmcnt0();
        lds_barrier();  // every wave is done reading the V tile
        issue_v(tile + 1);
      }
    };
    wait_vmcnt<0>();  // Q is in registers before any tile load is in flight
    if (n_tiles > 0) {
      issue_k(0);
      issue_v(0);
      for (int tile = 0; tile + 1 < n_tiles; ++tile) step(tile, std::true_type{});
      step(n_tiles - 1, std::false_type{});
    }
    finish_rows<T, D>(R, qvalid ? o + (int64_t)tq * D : nullptr,
                      (p.lse && qvalid) ? p.lse + (int64_t)bh * Tn + tq : nullptr);
  }
}

// ---------------------------------------------------------------------------
// bf16, d = 512: wave pairs on the 32-row core.  A workgroup of 4 waves takes
// 64 queries; waves 2p and 2p+1 share queries [32p, 32p + 32) of the tile and
// split the 512 dimensions: wave 2p + h holds Q and O for dims
// [256h, 256h + 256).  Per key tile each wave computes S over its half of the
// dims, the pair adds its two partial S through LDS (both waves then hold
// the same full S and run the same softmax), and each wave accumulates
// O^T += V^T . P^T for its half.  K and V tiles are stored as two half-row
// tiles of 512-byte rows, so every LDS operand read serves 32 queries instead
// of 16 and a wave reads half of each tile.
// ---------------------------------------------------------------------------
constexpr int kHalfD = 256;
constexpr int kPairRows = 32;
constexpr int kH32Waves = 4;  // 2 wave pairs: 64 queries per workgroup

// Wider query/key heads ([P3] §預訓練資料工程 item 3, FlashMask-4's qk 576 /
// v 512): the DR = 64 query/key dims past the value width.  Half h of a wave
// pair takes dims D + 32h .. +31 of them, two more k-steps of its partial S.
// Their 32-key tile is 32 rows x 128 bytes in LDS, 16-byte chunk c of row r
// at r*128 + 16*(c ^ ((r >> 1) & 7)): the operand reads of 16 lanes (rows
// r..r+15, one chunk) then fall in 16 distinct groups of 4 banks.  It is
// staged with 4-byte direct-to-LDS loads so that every wave issues the same
// number of loads per tile (the waits count loads per wave).
template <int DR, int kWaves>
struct RopeTile {
  static_assert(DR == 64, "8 chunks per row");
  static constexpr int kRowBytes = 2 * DR;
  static constexpr int kTileBytes = kBN * kRowBytes;    // 4 KB
  static constexpr int kInstr = kTileBytes / 4 / kWave;  // 4-byte loads of one wave
  static constexpr int kPerWave = kInstr / kWaves;
  static_assert(kInstr % kWaves == 0, "tile must split evenly over the waves");
  __device__ static __forceinline__ uint32_t off(int r, int c) { return (uint32_t)(r * kRowBytes + 16 * (c ^ ((r >> 1) & 7))); }
};

// Stage the extra dims of one 32-key tile: src points at dim D of row 0,
// rowfn(r) as for stage_rows_async, kPitch the K row pitch in bytes.
template <int DR, int kWaves, uint32_t kPitch, typename RowFn>
__device__ __forceinline__ void stage_rope_async(char* buf, const bf16_t* src, RowFn&& rowfn) {
  using RT = RopeTile<DR, kWaves>;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  int row[RT::kPerWave];
#pragma unroll
  for (int j = 0; j < RT::kPerWave; ++j) row[j] = rowfn(((j * kWaves + wave) * kWave + lane) / (RT::kRowBytes / 4));
  __builtin_amdgcn_sched_barrier(0);
  uint32_t off[RT::kPerWave];
#pragma unroll
  for (int j = 0; j < RT::kPerWave; ++j) {
    // Dword P of the tile in LDS: row r, physical chunk pc, dword e of it.
    const int P = (j * kWaves + wave) * kWave + lane;
    const int r = P / (RT::kRowBytes / 4), dw = P % (RT::kRowBytes / 4);
    const int c = (dw >> 2) ^ ((r >> 1) & 7);
    off[j] = (uint32_t)(row[j] < 0 ? 0 : row[j]) * kPitch + (uint32_t)c * 16u + (uint32_t)(dw & 3) * 4u;
  }
  const buffer_rsrc_t rsrc = make_buffer_rsrc(src);
#pragma unroll
  for (int j = 0; j < RT::kPerWave; ++j) buffer_load_lds_4(rsrc, off[j], buf + (j * kWaves + wave) * kWave * 4);
}

// S^T += K_extra . Q_extra^T over this half's 32 extra dims (two k-steps).
template <int DR, int kWaves>
__device__ __forceinline__ f32x16_t rope_qk32(f32x16_t s, const i16x8_t* qr, const char* rbuf, int half) {
  using RT = RopeTile<DR, kWaves>;
  const int lane = threadIdx.x & 63, r = lane & 31, g = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const i16x8_t a = __builtin_bit_cast(i16x8_t, lds_read_b128(rbuf, RT::off(r, 4 * half + 2 * ks + g)));
    s = mfma_bf16_32x32x16(a, qr[ks], s);
  }
  return s;
}

template <int D, int kWaves, int DR>
__global__ __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(2))) void hca_prefill32_kernel(HcaPrefillParams p) {
  static_assert(D == 2 * kHalfD, "two halves of 256 dims");
  static_assert(DR == 0 || DR == 64, "extra query/key dims");
  constexpr int kQK = D + DR;  // query/key row width (elements)
  constexpr int kRows = kWaves / 2 * kPairRows;  // queries per workgroup
  using T = bf16_t;
  using GH = AttnGeom<T, kHalfD, 1>;
  constexpr int kHalfTile = GH::kTileBytes;  // 16 KB: 32 rows x 512 bytes
  constexpr int kRopeBytes = DR > 0 ? RopeTile<(DR > 0 ? DR : 64), kWaves>::kTileBytes : 16;
  __shared__ __attribute__((aligned(16))) char kbuf[2 * kHalfTile];
  __shared__ __attribute__((aligned(16))) char vbuf[2 * kHalfTile];
  __shared__ __attribute__((aligned(16))) char rbuf[kRopeBytes];  // extra K dims (DR > 0)
  __shared__ __attribute__((aligned(16))) char xbuf[kWaves * 16 * kWave * 4];  // partial S, 4 KB per wave

  const int n_qtiles = (int)p.n_qtiles;
  const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = (int)(lid / (uint32_t)n_qtiles);
  const int qt = n_qtiles - 1 - (int)(lid % (uint32_t)n_qtiles);  // longest tiles first
  const int Tn = (int)p.T, blk = (int)p.blk, W = (int)p.window, Nc = (int)p.Nc;
  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const int pair = wave >> 1, half = wave & 1;

  const int64_t head_off = (int64_t)bh * Tn * D, head_qk = (int64_t)bh * Tn * kQK;
  const T* q = reinterpret_cast<const T*>(p.q) + head_qk;
  const T* k = reinterpret_cast<const T*>(p.k) + head_qk;
  const T* v = reinterpret_cast<const T*>(p.v) + head_off;
  const T* kc = reinterpret_cast<const T*>(p.kc) + (int64_t)bh * Nc * kQK;
  const T* vc = reinterpret_cast<const T*>(p.vc) + (int64_t)bh * Nc * D;
  T* o = reinterpret_cast<T*>(p.o) + head_off;

  const int t0 = qt * kRows;
  const int tp = t0 + pair * kPairRows;  // first query of this pair
  const int tq = tp + (lane & 31);       // this lane's query (row l%32)
  const bool qvalid = tq < Tn;

  Attn32Regs<kHalfD> R;
  // Rows past T load the last row (their results are never written).
  const T* qrow = q + (int64_t)min(tq, Tn - 1) * kQK;
  load_q32<kHalfD>(R, qrow + half * kHalfD);
  i16x8_t qr[2];  // extra dims D + 32*half + 16*ks + 8*(lane/32) .. +7
  if constexpr (DR > 0) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      qr[ks] = __builtin_bit_cast(i16x8_t, *reinterpret_cast<const uint4*>(qrow + D + 32 * half + 16 * ks + 8 * (lane >> 5)));
  }
  const Tile32Addr ad = tile32_addr<kHalfD>();

  // Key stream of the tile (as in the 16-row kernel).
  const int t_last = min(t0 + kRows - 1, Tn - 1);
  const int nc = min(Nc, hca_visible(t_last, blk, W));
  const int n_ctiles = (nc + kBN - 1) / kBN;
  const int s_lo = max(0, t0 - W + 1);
  const int n_rtiles = (t_last - s_lo + kBN) / kBN;
  const int n_tiles = n_ctiles + n_rtiles;
  // Raw tiles in a rotated order: at step `tile` the band tile whose global
  // index (s_lo / kBN + r) is congruent to `tile` modulo n_rtiles, so that
  // co-resident tiles of one head read their shared rows at the same step.
  const int rot = n_rtiles > 0 ? ((n_ctiles - s_lo / kBN) % n_rtiles + n_rtiles) % n_rtiles : 0;
  auto band = [&](int tile) {
    const int r = tile - n_ctiles + rot;
    return r >= n_rtiles ? r - n_rtiles : r;
  };

  // This lane's visibility limits, and the pair's (for skipping tiles).
  const int vis_c = qvalid ? min(Nc, hca_visible(tq, blk, W)) : 0;
  const int win_lo = tq - W + 1;
  const bool pvalid = tp < Tn;
  const int tp_last = min(tp + kPairRows - 1, Tn - 1);
  const int pair_nc = pvalid ? min(Nc, hca_visible(tp_last, blk, W)) : 0;
  const int pair_lo = tp - W + 1;

  auto rows_of = [&](int tile) {
    const bool ct = tile < n_ctiles;
    const int first = ct ? tile * kBN : s_lo + band(tile) * kBN;
    const int last = ct ? nc - 1 : t_last;
    return [=](int r) -> int {
      const int x = first + r;
      return x <= last ? x : -1;
    };
  };
  // A K (or V) tile is two half-row tiles: dims [0, 256) at buf, [256, 512)
  // at buf + kHalfTile; K rows also give their extra dims to rbuf.
  auto issue_k = [&](int tile) __attribute__((always_inline)) {
    const auto rf = rows_of(tile);
    const T* src = tile < n_ctiles ? kc : k;
    stage_rows_async<T, kHalfD, kWaves, 1, kQK * 2>(kbuf, src, rf);
    stage_rows_async<T, kHalfD, kWaves, 1, kQK * 2>(kbuf + kHalfTile, src + kHalfD, rf);
    if constexpr (DR > 0) stage_rope_async<DR, kWaves, (uint32_t)(kQK * 2)>(rbuf, src + D, rf);
  };
  auto issue_v = [&](int tile) __attribute__((always_inline)) {
    const auto rf = rows_of(tile);
    const T* src = tile < n_ctiles ? vc : v;
    stage_rows_async<T, kHalfD, kWaves, 1, D * 2>(vbuf, src, rf);
    stage_rows_async<T, kHalfD, kWaves, 1, D * 2>(vbuf + kHalfTile, src + kHalfD, rf);
  };

  // Partial-S exchange: value j of lane l at xbuf + wave*4096 + (j/4)*1024 + l*16.
  float* xs_mine = reinterpret_cast<float*>(xbuf + wave * 4096 + lane * 16);
  const float* xs_other = reinterpret_cast<const float*>(xbuf + (wave ^ 1) * 4096 + lane * 16);

  // Loads per wave of a V tile and of a K tile (the extra dims included).
  constexpr int kLoadsV = 2 * StageGeom<T, kHalfD, kWaves>::kPerWave;
  constexpr int kLoadsK = kLoadsV + (DR > 0 ? RopeTile<(DR > 0 ? DR : 64), kWaves>::kPerWave : 0);
  const char* kh = kbuf + half * kHalfTile;
  const char* vh = vbuf + half * kHalfTile;
  // Same pipeline as the 16-row kernel (last tile peeled off); the partial
  // S is written before the barrier that ends the K tile and read after it.
  auto step = [&](int tile, auto more_tag) __attribute__((always_inline)) {
    constexpr bool more = decltype(more_tag)::value;
    const bool ctile = tile < n_ctiles;
    const int j0 = tile * kBN;
    const int s0 = s_lo + band(tile) * kBN;
    const bool need = ctile ? (j0 < pair_nc) : (pvalid && s0 <= tp_last && s0 + kBN - 1 >= pair_lo);
    const int lo = ctile ? 0 : win_lo - s0;
    const int hi = ctile ? vis_c - j0 - 1 : tq - s0;

    wait_loads<kLoadsV>();  // K of this tile has landed (its V may be in flight)
    lds_barrier();          // ... for every wave
    f32x16_t s;
    if (need) {
      // Two operand reads in flight instead of four leave registers for the
      // extra dims' query part.
      s = attend_qk32<kHalfD, (DR > 0 ? 2 : 4)>(R, kh, ad);
      if constexpr (DR > 0) s = rope_qk32<DR, kWaves>(s, qr, rbuf, half);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<f32x4_t*>(xs_mine + c * 256) = f32x4_t{s[4 * c], s[4 * c + 1], s[4 * c + 2], s[4 * c + 3]};
    }
    wait_lgkmcnt0();
    lds_barrier();  // every wave is done reading the K tile; partial S is visible
    if constexpr (more) {
      issue_k(tile + 1);
      wait_loads<kLoadsK>();  // V of this tile has landed (the next K may be in flight)
    } else {
      wait_loads<0>();
    }
    if (need) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(xs_other + c * 256);
#pragma unroll
        for (int e = 0; e < 4; ++e) s[4 * c + e] += x[e];
      }
    }
    lds_barrier();
    if (need) attend_pv32_range<kHalfD>(R, s, vh, p.scale_log2, lo, hi, ad);
    if constexpr (more) {
      wait_lgkmcnt0();
      lds_barrier();  // every wave is done reading the V tile (and the partner's S)
      issue_v(tile + 1);
    }
  };
  // Q is in registers before any tile load is in flight (otherwise the
  // compiler waits for every load, tile 0's included, before the loop).
  wait_vmcnt<0>();
  if (n_tiles > 0) {
    issue_k(0);
    issue_v(0);
    for (int tile = 0; tile + 1 < n_tiles; ++tile) step(tile, std::true_type{});
    step(n_tiles - 1, std::false_type{});
  }
  if (qvalid)
    finish_rows32<kHalfD>(R, o + (int64_t)tq * D + half * kHalfD,
                          (p.lse && half == 0) ? p.lse + (int64_t)bh * Tn + tq : nullptr);
}

template <typename T, int D>
static hipError_t launch(const HcaPrefillParams& p, hipStream_t stream) {
  const int64_t nblocks = p.B * p.H * p.n_qtiles;
  hipLaunchKernelGGL((hca_prefill_kernel<T, D>), dim3((uint32_t)nblocks), dim3(kAttnThreads), 0, stream, p);
  return hipGetLastError();
}

template <int DR, int kWaves>
static hipError_t launch32(const HcaPrefillParams& p, hipStream_t stream) {
  HcaPrefillParams p32 = p;
  p32.n_qtiles = (p.T + kWaves / 2 * kPairRows - 1) / (kWaves / 2 * kPairRows);
  const int64_t nblocks = p.B * p.H * p32.n_qtiles;
  hipLaunchKernelGGL((hca_prefill32_kernel<512, kWaves, DR>), dim3((uint32_t)nblocks), dim3(kWaves * kWave), 0, stream, p32);
  return hipGetLastError();
}

// qk 576 / v 512 runs 8 waves (4 pairs, 128 queries) per workgroup: with the
// extra-dims tile a 4-wave workgroup needs 84 KB of LDS and two of them no
// longer fit a CU, while one 8-wave workgroup (100 KB) keeps two waves per
// SIMD.
constexpr int kH32WavesQK576 = 8;

hipError_t launch_hca_prefill(const HcaPrefillParams& p, int dtype, int d, int dv, hipStream_t stream) {
  if (dtype == 0 && d == 64 && dv == 64) return launch<float, 64>(p, stream);
  if (dtype == 1 && d == 512 && dv == 512) return launch32<0, kH32Waves>(p, stream);
  if (dtype == 1 && d == 576 && dv == 512) return launch32<64, kH32WavesQK576>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace sa

// DSA lightweight indexer (gfx950).
//
// Method: [P1] §二.1, [P3] §架構創新 1 -- a lightweight indexer scores every
// history position for each query.  The pages give no formula; this library
// computes score[b,i,s] = sum_h w[b,i,h] * max(0, <q_idx[b,i,h,:], k_idx[b,s,:]>)
// for s <= p_i (p_i = q_pos[b] + i, or i when q_pos is NULL).
//
// A GEMM with rows = (query, indexer head) and columns = positions, K = 128.
// With Hi = 4, one 16-row MFMA block is 4 queries x 4 heads and the 16x16x32
// accumulator layout leaves each lane holding the 4 heads of one (query,
// position) pair, so the ReLU, the weighting and the head sum happen in
// registers.  Each wave owns 16 queries (4 M-blocks, Q in registers); the
// workgroup streams 64-position tiles of k_idx into a double-buffered LDS
// ring with direct global->LDS loads and covers a chunk of 1024 positions.
// Workgroups are ordered chunk-major, so the query tiles that read one k_idx
// chunk run together and find it in L2.  Prefill shapes use 4 waves (64
// queries) per workgroup; decode shapes (T <= 16) use 1 wave per workgroup
// and short chunks of positions so that many workgroups stream them in
// parallel (up to 4 queries: the register-operand kernel below).
// The build compiles this file without NaN semantics (scores of finite inputs
// are finite), which makes the ReLU a single max instruction.
#include "common.h"
#include "kernels.h"
#include "select_util.h"

namespace sa {

constexpr int kIdxDi = 128;
constexpr int kIdxHi = 4;
constexpr int kIdxQPerWave = 16;                // queries per wave (4 M-blocks)
constexpr int kIdxKTile = 64;                   // positions per LDS tile
constexpr int kIdxTilesPerChunk = 16;  // prefill: positions per workgroup = 16 tiles
// 1-wave workgroups (T <= 16, except the calls the register-operand decode
// kernel takes): 4 tiles (256 positions) each.  Measured when the
// 1M-position, B = 4 decode still ran this kernel (16384 workgroups): 1, 2,
// 8, 16 and 52 tiles (one resident round) were slower.
constexpr int kIdxDecodeTiles = 4;
constexpr int kIdxRowBytes = kIdxDi * 2;                  // 256
constexpr int kIdxRowChunks = kIdxRowBytes / 16;          // 16
constexpr int kIdxTileBytes = kIdxKTile * kIdxRowBytes;   // 16 KB

__device__ __forceinline__ uint32_t idx_off(int r, int c) {
  return (uint32_t)(r * kIdxRowChunks + (c ^ lds_swizzle(r))) * 16u;
}

// Direct global->LDS load of positions [s0, s0+64) (rows past `stop` load row 0).
template <int kWaves>
__device__ __forceinline__ void idx_stage(char* buf, buffer_rsrc_t rsrc, int s0, int stop) {
  constexpr int kLoads = kIdxTileBytes / 1024 / kWaves;  // wave loads of 1 KB
  const int wave = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int base = (j * kWaves + wave) * 64;  // physical chunk
    const int P = base + lane;
    const int r = P / kIdxRowChunks, cp = P % kIdxRowChunks;
    const int c = cp ^ lds_swizzle(r);
    const int s = s0 + r < stop ? s0 + r : 0;
    const uint32_t off = (uint32_t)s * kIdxRowBytes + (uint32_t)c * 16u;
    buffer_load_lds_16(rsrc, off, buf + base * 16);
  }
}

// kMode: kIdxScores stores the scores; kIdxCand runs candidate mode (see
// DsaIndexerParams); kIdxFiltered stores the scores of the query tiles that
// hold a flagged row only (the row filter); kIdxKeys16 stores the top 16 bits
// of each score's order-preserving key instead of the score.
constexpr int kIdxScores = 0, kIdxCand = 1, kIdxFiltered = 2, kIdxKeys16 = 3;
// One workgroup's query tile x key chunk; lid is its logical id (after the
// XCD renumbering).
template <int kWaves, int kMode>
__device__ __forceinline__ void dsa_indexer_block(DsaIndexerParams p, int n_qtiles, int n_chunks, int chunk,
                                                  const uint32_t lid) {
  constexpr bool kEmit = kMode == kIdxCand;
  __shared__ __attribute__((aligned(16))) char lds0[kIdxTileBytes];
  __shared__ __attribute__((aligned(16))) char lds1[kIdxTileBytes];
  constexpr int kQTile = kWaves * kIdxQPerWave;

  // Chunk-major order: consecutive workgroups (same XCD) share a k_idx chunk.
  // The chunks are taken in folded order 0, n-1, 1, n-2, ...: under the
  // causal limit chunk c has work for the queries past 1024*c only, so a
  // heavy chunk is followed by a light one and every XCD's contiguous range
  // of workgroups gets about the same amount of work.
  const int per_b = n_qtiles * n_chunks;
  const int b = (int)(lid / (uint32_t)per_b);
  const int rem = (int)(lid % (uint32_t)per_b);
  const int kf = rem / n_qtiles;
  const int kc = (kf & 1) ? n_chunks - 1 - (kf >> 1) : (kf >> 1);
  const int qt = n_qtiles - 1 - rem % n_qtiles;

  const int T = (int)p.T, S = (int)p.S;
  const int base = p.q_pos ? (int)p.q_pos[b] : 0;
  // Last key visible to query row qi (token position base + qi): keys are
  // entries of `ratio` tokens (1 = positions) and entry s is visible iff its
  // block ends at or before the query, s < (base + qi + 1) / ratio.  -1 or
  // less: nothing visible.
  const int64_t ratio = p.ratio;
  auto lim = [&](int qi) -> int {
    const int64_t x = ((int64_t)base + qi + 1) / ratio - 1;
    return (int)(x < S - 1 ? x : S - 1);
  };
  const int i0 = qt * kQTile;
  const int i_last = min(i0 + kQTile - 1, T - 1);
  if constexpr (kMode == kIdxFiltered) {  // run only for a tile that holds a flagged row
    __shared__ uint32_t any_row;
    if (threadIdx.x == 0) any_row = 0u;
    __syncthreads();
    if (*p.any_flag != 0u && (int)threadIdx.x < kQTile && i0 + (int)threadIdx.x < T &&
        p.row_flag[(int64_t)b * T + i0 + threadIdx.x] != 0u)
      any_row = 1u;
    __syncthreads();
    if (any_row == 0u) return;
  }
  const int s_end = min(S, lim(i_last) + 1);  // exclusive, whole workgroup
  const int s_begin = kc * chunk;  // chunk: positions per workgroup, a multiple of the tile
  if (s_begin >= s_end) return;
  const int s_stop = min(s_end, s_begin + chunk);
  const int n_tiles = (s_stop - s_begin + kIdxKTile - 1) / kIdxKTile;

  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int L = lane & 15, g = lane >> 4;
  const int iw = i0 + wave * kIdxQPerWave;                   // first query of the wave
  const int n_mb = max(0, min(4, (T - iw + 3) / 4));          // M-blocks with a valid query
  const int wave_plim = n_mb > 0 ? lim(min(iw + kIdxQPerWave - 1, T - 1)) : -1;

  const bf16_t* qI = reinterpret_cast<const bf16_t*>(p.q) + (int64_t)b * T * kIdxHi * kIdxDi;
  const bf16_t* kI = reinterpret_cast<const bf16_t*>(p.k) + (int64_t)b * S * kIdxDi;
  const float* wgt = p.w + (int64_t)b * T * kIdxHi;
  float* out = p.scores + (int64_t)b * T * S;

  // A operand: row (query iw + mb*4 + L/4, head L%4), dims g*8 + 32*ks.
  i16x8_t qa[4][4];
  float wq[4][4];  // weights of this lane's accumulator query (iw + mb*4 + g), heads 0..3
  int plim[4];     // last position visible to that query (-1 if none)
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int qa_i = iw + mb * 4 + (L >> 2);
    const bool va = mb < n_mb && qa_i < T;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (va) {
        const uint4 u = *reinterpret_cast<const uint4*>(qI + ((int64_t)qa_i * kIdxHi + (L & 3)) * kIdxDi + ks * 32 + g * 8);
        qa[mb][ks] = __builtin_bit_cast(i16x8_t, u);
      } else {
        qa[mb][ks] = i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    const int qc_i = iw + mb * 4 + g;
    const bool vc = mb < n_mb && qc_i < T;
#pragma unroll
    for (int h = 0; h < 4; ++h) wq[mb][h] = vc ? wgt[(int64_t)qc_i * kIdxHi + h] : 0.f;
    plim[mb] = vc ? lim(qc_i) : -1;
  }

  // Scores of earlier tiles, held in registers and stored after the next
  // wait: on this GPU a wait for loads also waits for every earlier store
  // of the wave, so stores issued just before a wait would stall it.  Two
  // slots (the prefill pipeline works on pairs of tiles).
  float held[2][4][4];
  int held_s0[2] = {-1, -1};  // first position of the held tile (-1: nothing held)
  // Every position of a tile is visible to every query of the wave when the
  // tile ends at or before the first query's limit and all 16 of the wave's
  // query rows exist (rows past T must not be stored).
  const int wave_full_lim = iw + kIdxQPerWave - 1 < T ? lim(iw) : -1;
  // Candidate mode: the threshold of each of this lane's accumulator rows.
  // Rows that emit nothing (past the end, or keeping every visible position)
  // get 0xffffffff, which no finite or infinite score's key reaches.
  uint32_t thr[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int qi = iw + mb * 4 + g;
    const bool emit_row = kEmit && qi < T && plim[mb] + 1 > (int)p.topk;
    thr[mb] = emit_row ? p.thresh[(int64_t)b * T + qi] : 0xffffffffu;
  }
  // Candidates of this workgroup's chunk go to the rows' segments for the
  // chunk (cand[row][s_begin ..], room for every position of the chunk), so
  // slots come from a running count per row (uniform over the row's 16
  // lanes) and no atomics are needed; the counts are written at the end.
  uint32_t c_run[4] = {0u, 0u, 0u, 0u};
  auto emit_held = [&](int slot) __attribute__((always_inline)) {
    const int h0 = held_s0[slot];
    if (h0 < 0) return;
    // Lanes 16g .. 16g + 15 hold a row's 64 positions of the tile (per M-block).
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      uint32_t fl = 0u;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int s = h0 + nb * 16 + L;
        fl |= (s <= plim[mb] && score_key(held[slot][mb][nb]) >= thr[mb]) ? (1u << nb) : 0u;
      }
      const uint32_t mine = (uint32_t)__popc(fl);
      // Inclusive scan over the row's 16 lanes (one DPP row): row_shr 1, 2, 4, 8,
      // lanes shifted in from outside the row read 0.
      uint32_t x = mine;
      x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, true);
      x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, true);
      x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, true);
      x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, true);
      uint2* seg = p.cand + ((int64_t)b * T + iw + mb * 4 + g) * p.cand_pitch + s_begin;
      uint32_t slot_i = c_run[mb] + x - mine;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        if (fl & (1u << nb)) {
          seg[slot_i] = make_uint2(score_key(held[slot][mb][nb]), (uint32_t)(h0 + nb * 16 + L));
          ++slot_i;
        }
      }
      c_run[mb] += (uint32_t)__shfl(x, 15, 16);
    }
  };
  auto store_held = [&](int slot) __attribute__((always_inline)) {
    if constexpr (kEmit) {
      emit_held(slot);
      return;
    }
    const int h0 = held_s0[slot];
    if (h0 < 0) return;
    if constexpr (kMode == kIdxKeys16) {
      uint16_t* out16 = p.keys16 + (int64_t)b * T * S;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        // Rows past the sequence end have plim = -1: nothing is stored.
        uint16_t* orow = out16 + (int64_t)(iw + mb * 4 + g) * S;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int s = h0 + nb * 16 + L;
          if (s <= plim[mb]) orow[s] = (uint16_t)(score_key(held[slot][mb][nb]) >> 16);
        }
      }
      return;
    }
    if (h0 + kIdxKTile - 1 <= wave_full_lim) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        float* orow = out + (int64_t)(iw + mb * 4 + g) * S + h0 + L;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) orow[nb * 16] = held[slot][mb][nb];
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        // Rows past the sequence end have plim = -1: nothing is stored.
        float* orow = out + (int64_t)(iw + mb * 4 + g) * S;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int s = h0 + nb * 16 + L;
          if (s <= plim[mb]) orow[s] = held[slot][mb][nb];
        }
      }
    }
  };
  auto compute = [&](int tile, const char* buf, int slot) __attribute__((always_inline)) {
    const int s0 = s_begin + tile * kIdxKTile;
    if (s0 > wave_plim) {  // tile entirely after the wave's last query
      held_s0[slot] = -1;
      return;
    }
    // All four M-blocks always run (rows past the sequence end have zero Q
    // and are never stored), so the MFMA stream has no branches.  B operand
    // reads are issued one step ahead of the four MFMAs that use them.
    f32x4_t acc[4][4];
    auto bread = [&](int i) __attribute__((always_inline)) {
      return __builtin_bit_cast(i16x8_t, lds_read_b128(buf, idx_off((i & 3) * 16 + L, g + 4 * (i >> 2))));
    };
    i16x8_t bq[2];
    bq[0] = bread(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // i = 4*ks + nb
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < 16) bq[(i + 1) & 1] = bread(i + 1);
      const int ks = i >> 2, nb = i & 3;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[mb][nb] = mfma_bf16_16x16x32(qa[mb][ks], bq[i & 1], ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[mb][nb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Lane holds heads 0..3 of (query iw + mb*4 + g, position s0 + nb*16 + L).
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        float sc = 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h) sc = fmaf(wq[mb][h], fmaxf(acc[mb][nb][h], 0.f), sc);
        held[slot][mb][nb] = sc;
      }
    held_s0[slot] = s0;
  };

  const buffer_rsrc_t rsrc = make_buffer_rsrc(kI);
  if constexpr (kWaves == 4) {
    // Prefill: a four-stage ring worked in pairs of tiles (lds0/lds1 and
    // lds2/lds3 alternate).  A pair's loads are issued when the previous
    // pair's data is visible and a pair's scores are stored at the start of
    // the next pair, so the wait before a pair -- which also waits for the
    // wave's stores -- covers loads and stores issued a whole pair earlier.
    __shared__ __attribute__((aligned(16))) char lds2[kIdxTileBytes];
    __shared__ __attribute__((aligned(16))) char lds3[kIdxTileBytes];
    auto stage_pair = [&](char* b0, char* b1, int tile) __attribute__((always_inline)) {
      idx_stage<kWaves>(b0, rsrc, s_begin + tile * kIdxKTile, s_stop);
      if (tile + 1 < n_tiles) idx_stage<kWaves>(b1, rsrc, s_begin + (tile + 1) * kIdxKTile, s_stop);
    };
    auto run_pair = [&](int tile, const char* b0, const char* b1) __attribute__((always_inline)) {
      store_held(0);
      store_held(1);
      compute(tile, b0, 0);
      if (tile + 1 < n_tiles) {
        compute(tile + 1, b1, 1);
      } else {
        held_s0[1] = -1;
      }
    };
    stage_pair(lds0, lds1, 0);
    for (int tile = 0; tile < n_tiles; tile += 4) {
      wait_vmcnt<0>();
      lds_barrier();
      if (tile + 2 < n_tiles) stage_pair(lds2, lds3, tile + 2);
      run_pair(tile, lds0, lds1);
      if (tile + 2 >= n_tiles) break;
      wait_lgkmcnt0();
      wait_vmcnt<0>();
      lds_barrier();
      if (tile + 4 < n_tiles) stage_pair(lds0, lds1, tile + 4);
      run_pair(tile + 2, lds2, lds3);
      wait_lgkmcnt0();
    }
    store_held(0);
    store_held(1);
  } else {
    // Decode shapes: two stages, unrolled by two so each buffer has a fixed role.
    idx_stage<kWaves>(lds0, rsrc, s_begin, s_stop);
    for (int tile = 0; tile < n_tiles; tile += 2) {
      wait_vmcnt<0>();
      lds_barrier();
      if (tile + 1 < n_tiles) idx_stage<kWaves>(lds1, rsrc, s_begin + (tile + 1) * kIdxKTile, s_stop);
      store_held(0);
      compute(tile, lds0, 0);
      if (tile + 1 >= n_tiles) break;
      wait_lgkmcnt0();
      wait_vmcnt<0>();
      lds_barrier();
      if (tile + 2 < n_tiles) idx_stage<kWaves>(lds0, rsrc, s_begin + (tile + 2) * kIdxKTile, s_stop);
      store_held(0);
      compute(tile + 1, lds1, 0);
      wait_lgkmcnt0();
    }
    store_held(0);
  }
  if constexpr (kEmit) {
    // Counts, and a pad entry (key 0) after an odd count: segments hold
    // whole pairs.
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int qi = iw + mb * 4 + g;
      if (L == 0 && qi < T) {
        const int64_t row = (int64_t)b * T + qi;
        p.cnt[row * n_chunks + kc] = c_run[mb];
        if (c_run[mb] & 1u) p.cand[row * p.cand_pitch + s_begin + c_run[mb]] = make_uint2(0u, 0u);
      }
    }
  }
}

// The filtered mode (exact fallback of the fused call) runs on a bounded grid
// that walks the logical workgroups: with no row flagged (the usual case) the
// launch costs a few hundred workgroups rather than one per query tile and
// chunk.
constexpr uint32_t kIdxFilterGrid = 1024;

template <int kWaves, int kMode>
__global__ __launch_bounds__(kWaves * 64) void dsa_indexer_kernel(DsaIndexerParams p, int n_qtiles, int n_chunks,
                                                                   int chunk) {
  if constexpr (kMode == kIdxFiltered) {
    if (*p.any_flag == 0u) return;
    const uint32_t n = (uint32_t)(p.B * n_qtiles * n_chunks);
    for (uint32_t v = blockIdx.x; v < n; v += gridDim.x) {
      dsa_indexer_block<kWaves, kMode>(p, n_qtiles, n_chunks, chunk, xcd_remap(v, n));
      __syncthreads();  // LDS is reused by the next workgroup's tiles
    }
  } else {
    dsa_indexer_block<kWaves, kMode>(p, n_qtiles, n_chunks, chunk, xcd_remap(blockIdx.x, gridDim.x));
  }
}

// Decode calls of up to 4 queries: one 16-row M-block (4 queries x 4 heads)
// per wave.  Each lane loads 16 bytes of the tile per load, 16 loads per
// 64-position tile, as whole 128-byte lines with the non-temporal hint
// (a streaming read of this GPU's HBM reaches about 7 TB/s that way, about
// 6 TB/s when each load instruction reads half of every line it touches, as
// loads straight into the MFMA operand layout do); the tile then passes
// through a 16 KB LDS region of the wave into that layout (no barriers: one
// wave per workgroup).  Tiles are double-buffered in registers; a tile's
// scores are stored after the next tile's loads are sent, so the wait before
// a tile (which also covers the wave's earlier stores) finds those stores
// long done.
constexpr int kIdxDecTiles = 2;  // 64-position tiles per workgroup (1, 2, 4, 8, 16 measured: 2 is fastest)

// Modes of the decode kernel.  kDecScores stores the scores.  kDecCand is the
// candidate mode of the fused indexer -> top-k for long decode rows: instead
// of scores, every score whose key reaches the row's threshold is written as
// (key, position) to the row's segment for this workgroup's chunk
// (cand[row * cand_pitch + kc * kChunk ..], room for the whole chunk), in
// ascending position order, and the count to cnt[row * cnt_pitch + kc]
// (cnt_pitch: n_chunks rounded up to a multiple of 8, so that a reader can
// load a row's counts 16 bytes at a time).
// kDecSample scores a strided subset of the keys: position s (of S = the
// sample count) is key row s * ratio + ratio - 1 of a k_idx with k_rows rows
// per batch, visible under the ratio rule, and keys16 (rows pitched at S
// rounded up to a multiple of 8) receives the top 16 bits of the score's key.
constexpr int kDecScores = 0, kDecCand = 1, kDecSample = 2;

template <int kDec>
__device__ __forceinline__ void dsa_indexer_dec_chunk(const DsaIndexerParams& p, int b, int kc, int n_chunks) {
  constexpr bool kCand = kDec == kDecCand;
  const int T = (int)p.T, S = (int)p.S;
  const int base = p.q_pos ? (int)p.q_pos[b] : 0;
  const int64_t ratio = p.ratio;
  auto lim = [&](int qi) -> int {  // last key visible to query row qi (-1 or less: none)
    const int64_t x = ((int64_t)base + qi + 1) / ratio - 1;
    return (int)(x < S - 1 ? x : S - 1);
  };
  constexpr int kChunk = kIdxDecTiles * kIdxKTile;
  const int s_begin = kc * kChunk;
  const int s_end = min(S, lim(T - 1) + 1);  // exclusive
  if (s_begin >= s_end) return;
  const int s_stop = min(s_end, s_begin + kChunk);
  const int n_tiles = (s_stop - s_begin + kIdxKTile - 1) / kIdxKTile;

  const int lane = threadIdx.x & 63;
  const int L = lane & 15, g = lane >> 4;
  const bf16_t* qI = reinterpret_cast<const bf16_t*>(p.q) + (int64_t)b * T * kIdxHi * kIdxDi;
  const int64_t k_rows = kDec == kDecSample ? p.k_rows : (int64_t)S;
  const bf16_t* kI = reinterpret_cast<const bf16_t*>(p.k) + (int64_t)b * k_rows * kIdxDi;
  const float* wgt = p.w + (int64_t)b * T * kIdxHi;

  // A operand: row (query L/4, head L%4), dims g*8 + 32*ks (zero for rows past T).
  i16x8_t qa[4];
  const int qa_i = L >> 2;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (qa_i < T) {
      const uint4 u = *reinterpret_cast<const uint4*>(qI + ((int64_t)qa_i * kIdxHi + (L & 3)) * kIdxDi + ks * 32 + g * 8);
      qa[ks] = __builtin_bit_cast(i16x8_t, u);
    } else {
      qa[ks] = i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  // This lane's accumulator query is g (heads 0..3 in its four values).
  float wq[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) wq[h] = g < T ? wgt[(int64_t)g * kIdxHi + h] : 0.f;
  const int plim = g < T ? lim(g) : -1;
  const int64_t crow = (int64_t)b * T + g;  // this lane's output row
  // Candidate mode: threshold of this lane's query row (0xffffffff, which no
  // key reaches, for rows that keep every visible position or lie past T).
  const uint32_t thr = (kCand && g < T && plim + 1 > (int)p.topk) ? p.thresh[crow] : 0xffffffffu;
  uint32_t c_run = 0u;

  // One tile (64 positions x 256-byte rows) in whole 128-byte lines: load i
  // of a lane is 16-byte chunk lane % 16 of tile row 4i + lane / 16, with the
  // non-temporal hint (each row is read once).  Positions past the chunk's
  // stop load the chunk's first row (finite, never stored).
  const int rr = lane >> 4, cc = lane & 15;
  auto load_tile = [&](int tile, uint4 (&raw)[16]) __attribute__((always_inline)) {
    const int s0 = s_begin + tile * kIdxKTile;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s = s0 + 4 * i + rr;
      const int sv = s < s_stop ? s : s_begin;
      const int64_t kr = kDec == kDecSample ? (int64_t)sv * ratio + (ratio - 1) : (int64_t)sv;
      raw[i] = load_stream_u4(kI + kr * kIdxDi + cc * 8);
    }
  };
  // The loaded tile goes through this wave's LDS region (row r, chunk c at
  // r*256 + 16*(c ^ (r % 16)): conflict-free for both the row-wise writes
  // and the operand reads) into the MFMA B operand layout: for 16-position
  // block nb and 32-dim step ks, lane (L, g) takes chunk 4ks + g of row
  // 16nb + L.
  __shared__ __attribute__((aligned(16))) char stage[kIdxKTile * kIdxDi * 2];
  float sc[4];
  auto compute = [&](const uint4 (&raw)[16]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 4 * i + rr;
      lds_write_b128(stage, (uint32_t)(r * 256 + 16 * (cc ^ (r & 15))), raw[i]);
    }
    // The raw tile's registers are free before the operands are read.
    __builtin_amdgcn_sched_barrier(0);
    uint4 bt[4][4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        bt[nb][ks] = lds_read_b128(stage, (uint32_t)((16 * nb + L) * 256 + 16 * ((4 * ks + g) ^ L)));
    f32x4_t acc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc[nb] = mfma_bf16_16x16x32(qa[ks], __builtin_bit_cast(i16x8_t, bt[nb][ks]), acc[nb]);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      float x = 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h) x = fmaf(wq[h], fmaxf(acc[nb][h], 0.f), x);
      sc[nb] = x;
    }
  };
  auto store = [&](int tile) __attribute__((always_inline)) {
    const int s0 = s_begin + tile * kIdxKTile;
    if constexpr (kCand) {
      // Positions s0 + 16nb + L: for each nb in turn, the 16 lanes of query g
      // take slots in L order (a scan over the 16 lanes), so a segment lists
      // its candidates in ascending position order.
      uint2* seg = p.cand + crow * p.cand_pitch + s_begin;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int s = s0 + nb * 16 + L;
        const uint32_t key = score_key(sc[nb]);
        const uint32_t fl = (s <= plim && s < s_stop && key >= thr) ? 1u : 0u;
        uint32_t x = fl;
        x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, true);
        x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, true);
        x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, true);
        x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, true);
        if (fl) seg[c_run + x - 1u] = make_uint2(key, (uint32_t)s);
        c_run += (uint32_t)__shfl(x, 15, 16);
      }
    } else if constexpr (kDec == kDecSample) {
      uint16_t* o16 = p.keys16 + crow * (((int64_t)S + 7) & ~(int64_t)7);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int s = s0 + nb * 16 + L;
        if (s <= plim && s < s_stop) o16[s] = (uint16_t)(score_key(sc[nb]) >> 16);
      }
    } else {
      float* orow = p.scores + crow * S;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int s = s0 + nb * 16 + L;
        if (s <= plim && s < s_stop) orow[s] = sc[nb];
      }
    }
  };

  uint4 b0[16], b1[16];
  load_tile(0, b0);
  for (int tile = 0; tile < n_tiles; tile += 2) {
    if (tile + 1 < n_tiles) load_tile(tile + 1, b1);
    compute(b0);
    store(tile);
    if (tile + 1 >= n_tiles) break;
    if (tile + 2 < n_tiles) load_tile(tile + 2, b0);
    compute(b1);
    store(tile + 1);
  }
  if constexpr (kCand) {
    if (L == 0 && g < T) p.cnt[crow * (((int64_t)n_chunks + 7) & ~(int64_t)7) + kc] = c_run;
  }
}

// One chunk per workgroup.
template <int kDec>
__global__ __launch_bounds__(64) void dsa_indexer_dec_kernel(DsaIndexerParams p, int n_chunks) {
  dsa_indexer_dec_chunk<kDec>(p, (int)(blockIdx.x / (uint32_t)n_chunks), (int)(blockIdx.x % (uint32_t)n_chunks),
                              n_chunks);
}

// Row filter (scores): nothing runs unless *any_flag != 0; then a bounded grid
// strides over the chunks of the batches holding a flagged row.  A call in
// which no row is flagged costs one small launch, not one workgroup per chunk.
constexpr uint32_t kIdxDecFilterGrid = 2048;
__global__ __launch_bounds__(64) void dsa_indexer_dec_filtered_kernel(DsaIndexerParams p, int n_chunks) {
  if (*p.any_flag == 0u) return;
  const uint32_t nblk = (uint32_t)p.B * (uint32_t)n_chunks;
  for (uint32_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int b = (int)(blk / (uint32_t)n_chunks);
    bool run = false;
    for (int qi = 0; qi < (int)p.T; ++qi) run |= p.row_flag[(int64_t)b * p.T + qi] != 0u;
    if (run) dsa_indexer_dec_chunk<kDecScores>(p, b, (int)(blk % (uint32_t)n_chunks), n_chunks);
  }
}

int64_t dsa_indexer_dec_chunk() { return (int64_t)kIdxDecTiles * kIdxKTile; }

int64_t dsa_indexer_chunk(int64_t T) {
  return T <= kIdxQPerWave ? (int64_t)kIdxDecodeTiles * kIdxKTile : (int64_t)kIdxTilesPerChunk * kIdxKTile;
}

hipError_t launch_dsa_indexer(const DsaIndexerParams& p, hipStream_t stream) {
  if (p.T <= kIdxQPerWave) {
    // Decode: one query tile, short chunks of positions.  (The staged
    // kernel's candidate, filtered and key modes serve the fused indexer ->
    // top-k of rows up to 32768 positions.)
    const int64_t dec_chunks = (p.S + kIdxDecTiles * kIdxKTile - 1) / (kIdxDecTiles * kIdxKTile);
    const dim3 dgrid((uint32_t)(p.B * dec_chunks));
    if (p.T <= 4 && p.dec_cand) {
      hipLaunchKernelGGL(dsa_indexer_dec_kernel<kDecCand>, dgrid, dim3(64), 0, stream, p, (int)dec_chunks);
    } else if (p.T <= 4 && p.dec_sample) {
      hipLaunchKernelGGL(dsa_indexer_dec_kernel<kDecSample>, dgrid, dim3(64), 0, stream, p, (int)dec_chunks);
    } else if (p.T <= 4 && p.dec_filter) {
      const uint32_t n = (uint32_t)(p.B * dec_chunks);
      hipLaunchKernelGGL(dsa_indexer_dec_filtered_kernel, dim3(n < kIdxDecFilterGrid ? n : kIdxDecFilterGrid), dim3(64),
                         0, stream, p, (int)dec_chunks);
    } else if (p.T <= 4 && !p.cand && !p.row_flag && !p.keys16) {
      hipLaunchKernelGGL(dsa_indexer_dec_kernel<kDecScores>, dgrid, dim3(64), 0, stream, p, (int)dec_chunks);
    } else {
      const int chunk = kIdxDecodeTiles * kIdxKTile;
      const int64_t n_chunks = (p.S + chunk - 1) / chunk;
      const dim3 grid((uint32_t)(p.B * n_chunks));
      if (p.cand)
        hipLaunchKernelGGL((dsa_indexer_kernel<1, kIdxCand>), grid, dim3(64), 0, stream, p, 1, (int)n_chunks, chunk);
      else if (p.row_flag)
        hipLaunchKernelGGL((dsa_indexer_kernel<1, kIdxFiltered>), dim3(std::min(grid.x, kIdxFilterGrid)), dim3(64), 0,
                           stream, p, 1, (int)n_chunks, chunk);
      else if (p.keys16)
        hipLaunchKernelGGL((dsa_indexer_kernel<1, kIdxKeys16>), grid, dim3(64), 0, stream, p, 1, (int)n_chunks, chunk);
      else
        hipLaunchKernelGGL((dsa_indexer_kernel<1, kIdxScores>), grid, dim3(64), 0, stream, p, 1, (int)n_chunks, chunk);
    }
  } else {
    const int chunk = kIdxTilesPerChunk * kIdxKTile;
    const int64_t n_chunks = (p.S + chunk - 1) / chunk;
    const int64_t n_qtiles = (p.T + 4 * kIdxQPerWave - 1) / (4 * kIdxQPerWave);
    const int64_t nblocks = p.B * n_qtiles * n_chunks;
    const dim3 grid((uint32_t)nblocks);
    if (p.cand)
      hipLaunchKernelGGL((dsa_indexer_kernel<4, kIdxCand>), grid, dim3(256), 0, stream, p, (int)n_qtiles, (int)n_chunks,
                         chunk);
    else if (p.row_flag)
      hipLaunchKernelGGL((dsa_indexer_kernel<4, kIdxFiltered>), dim3(std::min(grid.x, kIdxFilterGrid)), dim3(256), 0,
                         stream, p, (int)n_qtiles, (int)n_chunks, chunk);
    else if (p.keys16)
      hipLaunchKernelGGL((dsa_indexer_kernel<4, kIdxKeys16>), grid, dim3(256), 0, stream, p, (int)n_qtiles,
                         (int)n_chunks, chunk);
    else
      hipLaunchKernelGGL((dsa_indexer_kernel<4, kIdxScores>), grid, dim3(256), 0, stream, p, (int)n_qtiles,
                         (int)n_chunks, chunk);
  }
  return hipGetLastError();
}

}  // namespace sa

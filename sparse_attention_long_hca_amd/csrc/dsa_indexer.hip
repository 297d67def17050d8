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
// queries) per workgroup; decode shapes (T <= 16) use 1 wave per workgroup so
// that many workgroups stream the positions in parallel.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kIdxDi = 128;
constexpr int kIdxHi = 4;
constexpr int kIdxQPerWave = 16;                // queries per wave (4 M-blocks)
constexpr int kIdxKTile = 64;                   // positions per LDS tile
constexpr int kIdxTilesPerChunk = 16;
constexpr int kIdxChunk = kIdxTilesPerChunk * kIdxKTile;  // positions per workgroup
constexpr int kIdxRowBytes = kIdxDi * 2;                  // 256
constexpr int kIdxRowChunks = kIdxRowBytes / 16;          // 16
constexpr int kIdxTileBytes = kIdxKTile * kIdxRowBytes;   // 16 KB

__device__ __forceinline__ uint32_t idx_off(int r, int c) {
  return (uint32_t)(r * kIdxRowChunks + (c ^ lds_swizzle(r))) * 16u;
}

// Direct global->LDS load of positions [s0, s0+64) (rows past `stop` load row 0).
template <int kWaves>
__device__ __forceinline__ void idx_stage(char* buf, const bf16_t* kI, int s0, int stop) {
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
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(kI) + off, (lds_void_t*)(buf + base * 16), 16, 0,
                                     0);
  }
}

template <int kWaves>
__global__ __launch_bounds__(kWaves * 64) void dsa_indexer_kernel(DsaIndexerParams p, int n_qtiles, int n_chunks) {
  __shared__ __attribute__((aligned(16))) char lds0[kIdxTileBytes];
  __shared__ __attribute__((aligned(16))) char lds1[kIdxTileBytes];
  constexpr int kQTile = kWaves * kIdxQPerWave;

  // Chunk-major order: consecutive workgroups (same XCD) share a k_idx chunk.
  const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_b = n_qtiles * n_chunks;
  const int b = (int)(lid / (uint32_t)per_b);
  const int rem = (int)(lid % (uint32_t)per_b);
  const int kc = rem / n_qtiles;
  const int qt = n_qtiles - 1 - rem % n_qtiles;

  const int T = (int)p.T, S = (int)p.S;
  const int base = p.q_pos ? (int)p.q_pos[b] : 0;
  const int i0 = qt * kQTile;
  const int i_last = min(i0 + kQTile - 1, T - 1);
  const int s_end = min(S, base + i_last + 1);  // exclusive, whole workgroup
  const int s_begin = kc * kIdxChunk;
  if (s_begin >= s_end) return;
  const int s_stop = min(s_end, s_begin + kIdxChunk);
  const int n_tiles = (s_stop - s_begin + kIdxKTile - 1) / kIdxKTile;

  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int L = lane & 15, g = lane >> 4;
  const int iw = i0 + wave * kIdxQPerWave;                  // first query of the wave
  const int n_mb = max(0, min(4, (T - iw + 3) / 4));          // M-blocks with a valid query
  const int wave_plim = n_mb > 0 ? min(base + min(iw + kIdxQPerWave - 1, T - 1), S - 1) : -1;

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
    plim[mb] = vc ? min(base + qc_i, S - 1) : -1;
  }

  auto compute = [&](int tile, const char* buf) {
    const int s0 = s_begin + tile * kIdxKTile;
    if (s0 > wave_plim) return;  // tile entirely after the wave's last query
    f32x4_t acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const uint4 bu = lds_read_b128(buf, idx_off(nb * 16 + L, g + 4 * ks));
        const i16x8_t bb = __builtin_bit_cast(i16x8_t, bu);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          if (mb < n_mb) acc[mb][nb] = mfma_bf16_16x16x32(qa[mb][ks], bb, acc[mb][nb]);
      }
    }
    // Lane holds heads 0..3 of (query iw + mb*4 + g, position s0 + nb*16 + L).
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb >= n_mb) continue;
      float* orow = out + (int64_t)(iw + mb * 4 + g) * S;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int s = s0 + nb * 16 + L;
        float sc = 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h) sc = fmaf(wq[mb][h], fmaxf(acc[mb][nb][h], 0.f), sc);
        if (s <= plim[mb]) orow[s] = sc;
      }
    }
  };

  // Two-stage pipeline, unrolled by two so each buffer has a fixed role.
  idx_stage<kWaves>(lds0, kI, s_begin, s_stop);
  for (int tile = 0; tile < n_tiles; tile += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tile + 1 < n_tiles) idx_stage<kWaves>(lds1, kI, s_begin + (tile + 1) * kIdxKTile, s_stop);
    compute(tile, lds0);
    if (tile + 1 >= n_tiles) break;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tile + 2 < n_tiles) idx_stage<kWaves>(lds0, kI, s_begin + (tile + 2) * kIdxKTile, s_stop);
    compute(tile + 1, lds1);
  }
}

hipError_t launch_dsa_indexer(const DsaIndexerParams& p, hipStream_t stream) {
  const int64_t n_chunks = (p.S + kIdxChunk - 1) / kIdxChunk;
  if (p.T <= kIdxQPerWave) {
    const int64_t n_qtiles = 1;
    const int64_t nblocks = p.B * n_qtiles * n_chunks;
    hipLaunchKernelGGL(dsa_indexer_kernel<1>, dim3((uint32_t)nblocks), dim3(64), 0, stream, p, (int)n_qtiles,
                       (int)n_chunks);
  } else {
    const int64_t n_qtiles = (p.T + 4 * kIdxQPerWave - 1) / (4 * kIdxQPerWave);
    const int64_t nblocks = p.B * n_qtiles * n_chunks;
    hipLaunchKernelGGL(dsa_indexer_kernel<4>, dim3((uint32_t)nblocks), dim3(256), 0, stream, p, (int)n_qtiles,
                       (int)n_chunks);
  }
  return hipGetLastError();
}

}  // namespace sa

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
// registers.  A workgroup (4 waves x 16 queries) stages 64-position tiles of
// k_idx into LDS once for all its waves and covers a chunk of 1024 positions;
// chunks entirely after the workgroup's last query are skipped.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kIdxThreads = 256;
constexpr int kIdxDi = 128;
constexpr int kIdxHi = 4;
constexpr int kIdxQPerWave = 16;                    // queries per wave (4 M-blocks)
constexpr int kIdxQTile = 4 * kIdxQPerWave;         // queries per workgroup
constexpr int kIdxKTile = 64;                       // positions per LDS tile
constexpr int kIdxChunk = 16 * kIdxKTile;           // positions per workgroup
constexpr int kIdxRowChunks = kIdxDi * 2 / 16;      // 16-byte chunks per k row (16)
constexpr int kIdxCPT = kIdxKTile * kIdxRowChunks / kIdxThreads;  // 4

__device__ __forceinline__ uint32_t idx_off(int r, int c) {
  return (uint32_t)(r * kIdxRowChunks + (c ^ (r & 7))) * 16u;
}

__global__ __launch_bounds__(kIdxThreads) void dsa_indexer_kernel(DsaIndexerParams p, int64_t n_qtiles,
                                                                  int64_t n_chunks) {
  __shared__ __attribute__((aligned(16))) char lds[kIdxKTile * kIdxRowChunks * 16];

  const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t per_b = n_qtiles * n_chunks;
  const int64_t b = lid / per_b;
  const int64_t rem = lid % per_b;
  const int64_t qt = n_qtiles - 1 - rem / n_chunks;  // longest rows first
  const int64_t kc = rem % n_chunks;

  const int64_t base = p.q_pos ? p.q_pos[b] : 0;
  const int64_t i0 = qt * kIdxQTile;
  const int64_t i_last = imin64(i0 + kIdxQTile - 1, p.T - 1);
  const int64_t s_end = imin64(p.S, base + i_last + 1);  // exclusive, whole workgroup
  const int64_t s_begin = kc * kIdxChunk;
  if (s_begin >= s_end) return;
  const int64_t s_stop = imin64(s_end, s_begin + kIdxChunk);
  const int n_tiles = (int)((s_stop - s_begin + kIdxKTile - 1) / kIdxKTile);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int L = lane & 15, g = lane >> 4;
  const int64_t iw = i0 + wave * kIdxQPerWave;  // first query of the wave
  const int n_mb = (int)imax64(0, imin64(4, (p.T - iw + 3) / 4));  // M-blocks with a valid query

  const bf16_t* qI = reinterpret_cast<const bf16_t*>(p.q) + b * p.T * kIdxHi * kIdxDi;
  const bf16_t* kI = reinterpret_cast<const bf16_t*>(p.k) + b * p.S * kIdxDi;
  const float* wgt = p.w + b * p.T * kIdxHi;
  float* out = p.scores + b * p.T * p.S;

  // A operand: row (query iw + mb*4 + L/4, head L%4), dims g*8 + 32*ks.
  i16x8_t qa[4][4];
  float wq[4][4];  // weights of this lane's accumulator query (iw + mb*4 + g), heads 0..3
  int64_t plim[4];  // last position visible to that query (or -1)
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int64_t qa_i = iw + mb * 4 + (L >> 2);
    const bool va = mb < n_mb && qa_i < p.T;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (va) {
        const uint4 u = *reinterpret_cast<const uint4*>(qI + (qa_i * kIdxHi + (L & 3)) * kIdxDi + ks * 32 + g * 8);
        qa[mb][ks] = __builtin_bit_cast(i16x8_t, u);
      } else {
        qa[mb][ks] = i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    const int64_t qc_i = iw + mb * 4 + g;
    const bool vc = mb < n_mb && qc_i < p.T;
#pragma unroll
    for (int h = 0; h < 4; ++h) wq[mb][h] = vc ? wgt[qc_i * kIdxHi + h] : 0.f;
    plim[mb] = vc ? imin64(base + qc_i, p.S - 1) : -1;
  }

  // Staging: thread handles chunks id = pass*256 + tid -> row id/16, chunk id%16.
  uint4 st[kIdxCPT];
  auto load_tile = [&](int tile) {
    const int64_t s0 = s_begin + (int64_t)tile * kIdxKTile;
#pragma unroll
    for (int pp = 0; pp < kIdxCPT; ++pp) {
      const int id = pp * kIdxThreads + threadIdx.x;
      const int r = id / kIdxRowChunks, c = id % kIdxRowChunks;
      const int64_t s = s0 + r;
      st[pp] = (s < s_stop) ? *reinterpret_cast<const uint4*>(kI + s * kIdxDi + c * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  load_tile(0);
  for (int tile = 0; tile < n_tiles; ++tile) {
    __syncthreads();
#pragma unroll
    for (int pp = 0; pp < kIdxCPT; ++pp) {
      const int id = pp * kIdxThreads + threadIdx.x;
      lds_write_b128(lds, idx_off(id / kIdxRowChunks, id % kIdxRowChunks), st[pp]);
    }
    __syncthreads();
    if (tile + 1 < n_tiles) load_tile(tile + 1);
    const int64_t s0 = s_begin + (int64_t)tile * kIdxKTile;
    if (n_mb == 0) continue;
    // Skip the tile if it lies entirely after the wave's last query.
    const int64_t wave_plim = imin64(base + imin64(iw + kIdxQPerWave - 1, p.T - 1), p.S - 1);
    if (s0 > wave_plim) continue;

    f32x4_t acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const uint4 bu = lds_read_b128(lds, idx_off(nb * 16 + L, g + 4 * ks));
        const i16x8_t bb = __builtin_bit_cast(i16x8_t, bu);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          if (mb < n_mb) acc[mb][nb] = mfma_bf16_16x16x32(qa[mb][ks], bb, acc[mb][nb]);
        }
      }
    }
    // Epilogue: lane holds heads 0..3 of (query iw + mb*4 + g, position s0 + nb*16 + L).
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb >= n_mb) continue;
      const int64_t qi = iw + mb * 4 + g;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int64_t s = s0 + nb * 16 + L;
        float sc = 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h) sc = fmaf(wq[mb][h], fmaxf(acc[mb][nb][h], 0.f), sc);
        if (s <= plim[mb]) out[qi * p.S + s] = sc;
      }
    }
  }
}

hipError_t launch_dsa_indexer(const DsaIndexerParams& p, hipStream_t stream) {
  const int64_t n_qtiles = (p.T + kIdxQTile - 1) / kIdxQTile;
  const int64_t n_chunks = (p.S + kIdxChunk - 1) / kIdxChunk;
  const int64_t nblocks = p.B * n_qtiles * n_chunks;
  hipLaunchKernelGGL(dsa_indexer_kernel, dim3((uint32_t)nblocks), dim3(kIdxThreads), 0, stream, p, n_qtiles,
                     n_chunks);
  return hipGetLastError();
}

}  // namespace sa

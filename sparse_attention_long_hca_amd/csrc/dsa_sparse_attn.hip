// DSA sparse attention over the selected positions (gfx950).
//
// Method: [P1] §二.1, [P3] §架構創新 1 -- core attention runs only on the
// top-K positions chosen by the indexer, so the per-query cost does not
// depend on the context length; MLA heads are 256 wide.  Multi-query layout:
// the query heads of a token share one K row and one V row per position.
//
// One workgroup per query token: its 64 heads are the 64 rows of the MFMA
// tile (4 waves x 16 heads), so every gathered K/V row is read once and used
// by all heads.  The index list is walked in tiles of 32 positions; each
// 512-byte row is gathered with 16-byte loads by 32 consecutive lanes (one
// contiguous row per half-wave).  Indices outside [0, S) are skipped; a tile
// without any valid index is skipped entirely.
#include "attn_core.h"
#include "kernels.h"

namespace sa {

constexpr int kDsaMaxK = 2048;  // longest index list per query

template <int D>
__global__ __launch_bounds__(kAttnThreads) void dsa_sparse_kernel(DsaSparseParams p) {
  using T = bf16_t;
  using G = AttnGeom<T, D>;
  // Two pipeline stages as separate LDS objects (see hca_prefill.hip).
  __shared__ __attribute__((aligned(16))) char lds0[G::kStageBytes];
  __shared__ __attribute__((aligned(16))) char lds1[G::kStageBytes];
  __shared__ int32_t sidx[kDsaMaxK];

  const int64_t tok = xcd_remap(blockIdx.x, gridDim.x);  // b*T + i
  const int64_t b = tok / p.T;
  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const int L = lane & 15;
  constexpr int kHq = kBM;  // 64 heads

  const T* q = reinterpret_cast<const T*>(p.q) + tok * kHq * D;
  const T* kb = reinterpret_cast<const T*>(p.k) + b * p.S * D;
  const T* vb = reinterpret_cast<const T*>(p.v) + b * p.S * D;
  const int32_t* idx = p.idx + tok * p.kk;
  T* o = reinterpret_cast<T*>(p.o) + tok * kHq * D;
  const int h = wave * kRowsPerWave + L;
  const int kk = (int)p.kk;
  const int64_t S = p.S;

  // Index list -> LDS, out-of-range entries replaced by -1.
  for (int n = threadIdx.x; n < kk; n += kAttnThreads) {
    const int32_t s = idx[n];
    sidx[n] = (s >= 0 && s < S) ? s : -1;
  }
  AttnRegs<T, D> R;
  load_q(R, q + h * D);
  __syncthreads();

  const int n_tiles = (kk + kBN - 1) / kBN;
  auto issue = [&](int tile, char* buf) {
    stage_async<T, D>(buf, buf + G::kTileBytes, kb, vb, [=](int r) -> int {
      const int n = tile * kBN + r;
      return n < kk ? sidx[n] : -1;
    });
  };
  auto compute = [&](int tile, const char* buf) {
    const int n = tile * kBN + (lane & 31);
    const uint32_t mask = (uint32_t)(__ballot(n < kk && sidx[n] >= 0) & 0xffffffffull);
    if (mask) attend_tile<T, D>(R, buf, buf + G::kTileBytes, p.scale_log2, [&](int key) { return (mask >> key) & 1u; });
  };

  if (n_tiles > 0) issue(0, lds0);
  for (int tile = 0; tile < n_tiles; tile += 2) {
    wait_loads<0>();
    __syncthreads();
    if (tile + 1 < n_tiles) issue(tile + 1, lds1);
    compute(tile, lds0);
    if (tile + 1 >= n_tiles) break;
    wait_loads<0>();
    __syncthreads();
    if (tile + 2 < n_tiles) issue(tile + 2, lds0);
    compute(tile + 1, lds1);
  }
  finish_rows<T, D>(R, o + h * D, p.lse ? p.lse + tok * kHq + h : nullptr);
}

hipError_t launch_dsa_sparse(const DsaSparseParams& p, int d, int hq, hipStream_t stream) {
  if (d != 256 || hq != kBM) return hipErrorInvalidValue;
  const int64_t nblocks = p.B * p.T;
  hipLaunchKernelGGL(dsa_sparse_kernel<256>, dim3((uint32_t)nblocks), dim3(kAttnThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa

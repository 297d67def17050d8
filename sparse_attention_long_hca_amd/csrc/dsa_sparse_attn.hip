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
  // One stage of K and V (32 KB for d = 256); several workgroups share a CU
  // and cover each other's load latency (see hca_prefill.hip).
  __shared__ __attribute__((aligned(16))) char lds0[G::kStageBytes];
  __shared__ int32_t sidx[kDsaMaxK];

  const int64_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t tok = lid / p.nsplit;  // b*T + i
  const int split = (int)(lid % p.nsplit);
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
  __syncthreads();  // the index list is in LDS

  // This workgroup's share of the index list: tiles [t_first, t_first + n_tiles).
  const int t_first = split * (int)p.tiles_per_split;
  const int n_tiles = max(0, min((kk + kBN - 1) / kBN - t_first, (int)p.tiles_per_split));
  auto issue = [&](int t, char* buf) {
    const int tile = t_first + t;
    stage_async<T, D>(buf, buf + G::kTileBytes, kb, vb, [=](int r) -> int {
      const int n = tile * kBN + r;
      return n < kk ? sidx[n] : -1;
    });
  };
  auto compute = [&](int t, const char* buf) {
    const int n = (t_first + t) * kBN + (lane & 31);
    const uint32_t mask = (uint32_t)(__ballot(n < kk && sidx[n] >= 0) & 0xffffffffull);
    if (mask) attend_tile<T, D>(R, buf, buf + G::kTileBytes, p.scale_log2, [&](int key) { return (mask >> key) & 1u; });
  };

  wait_vmcnt<0>();  // Q is in registers before any tile load is in flight
  if (n_tiles > 0) issue(0, lds0);
  for (int tile = 0; tile < n_tiles; ++tile) {
    wait_loads<0>();
    lds_barrier();
    compute(tile, lds0);
    wait_lgkmcnt0();
    lds_barrier();
    if (tile + 1 < n_tiles) issue(tile + 1, lds0);
  }
  if (p.nsplit == 1) {
    finish_rows<T, D>(R, o + h * D, p.lse ? p.lse + tok * kHq + h : nullptr);
  } else {
    const int64_t ps = tok * p.nsplit + split;
    finish_rows_partial<T, D>(R, p.part_o + (ps * kHq + h) * D, p.part_lse + ps * kHq + h);
  }
}

// Merge the splits of one (token, head) in split order: weights
// exp2(lse_s - max).  One workgroup per (token, head), one thread per dim.
template <int D>
__global__ __launch_bounds__(D) void dsa_sparse_combine_kernel(DsaSparseParams p) {
  constexpr int kHq = kBM;
  const int64_t th = blockIdx.x;  // tok * kHq + h
  const int64_t tok = th / kHq;
  const int h = (int)(th % kHq);
  const int ns = (int)p.nsplit;
  const float* pl = p.part_lse + tok * ns * kHq + h;  // stride kHq per split
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, pl[s * kHq]);
  float wsum = 0.f, acc = 0.f;
  const float* po = p.part_o + (tok * ns * kHq + h) * D + threadIdx.x;  // stride kHq*D per split
  for (int s = 0; s < ns; ++s) {
    const float w = (M == -INFINITY) ? 0.f : fast_exp2(pl[s * kHq] - M);
    wsum += w;
    acc = fmaf(w, po[(int64_t)s * kHq * D], acc);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  reinterpret_cast<bf16_t*>(p.o)[th * D + threadIdx.x] = (bf16_t)f32_to_bf16_rne(acc * inv);
  if (p.lse && threadIdx.x == 0) p.lse[th] = wsum > 0.f ? (M + __log2f(wsum)) * kLn2 : -INFINITY;
}

// Decode-sized calls (few tokens) split each token's index list over several
// workgroups so that the whole chip streams the gathered rows.
int64_t dsa_sparse_nsplit(int64_t BT, int64_t kk) {
  const int64_t tiles = (kk + kBN - 1) / kBN;
  if (BT >= 512) return 1;
  int64_t ns = (1024 + BT - 1) / BT;
  if (ns > tiles) ns = tiles;
  return ns < 1 ? 1 : ns;
}

size_t dsa_sparse_workspace_bytes(int64_t BT, int64_t nsplit, int64_t hq, int64_t d) {
  if (nsplit <= 1) return 0;
  return (size_t)(BT * nsplit * hq * (d + 1)) * sizeof(float);
}

hipError_t launch_dsa_sparse(const DsaSparseParams& p, int d, int hq, hipStream_t stream) {
  if (d != 256 || hq != kBM) return hipErrorInvalidValue;
  const int64_t nblocks = p.B * p.T * p.nsplit;
  hipLaunchKernelGGL(dsa_sparse_kernel<256>, dim3((uint32_t)nblocks), dim3(kAttnThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  hipLaunchKernelGGL(dsa_sparse_combine_kernel<256>, dim3((uint32_t)(p.B * p.T * kBM)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa

// Fused DSA indexer -> top-k (gfx950).
//
// Method: [P1] §二.1, [P3] §架構創新 1 -- a lightweight indexer scores every
// history position and only the top-k positions are kept.  This call returns
// exactly what dsa_indexer_scores followed by dsa_topk returns (same fp32
// scores, same selection rule: score descending, then position ascending;
// ascending output) without writing or reading back the T x S score matrix.
//
//   1. Sample: the k_idx rows at positions 16j + 15 are scored with the
//      indexer in its ratio-16 mode, whose visibility rule (entry j visible
//      to position p iff 16j + 15 <= p) is exactly "sampled position <= p".
//   2. Threshold: per row, the r-th largest sampled key (r = k/16 plus a
//      margin of six standard deviations), or 0 when the row has at most r
//      samples.
//   3. Candidates: the indexer runs in candidate mode and appends (key,
//      position) of every score whose key is >= the row's threshold; its
//      scores are the same fp32 values as in dsa_indexer_scores (same code,
//      same order of accumulation).
//   4. Select: if a row has at least k and at most kCap candidates, the k-th
//      largest key K over them is the k-th largest of the row (at least k
//      keys lie above the threshold, so every key of the top k, ties of K
//      included, is a candidate).  Rounds of key histograms find K exactly;
//      positions with key > K and the lowest `need` positions with key == K
//      are marked in an LDS bitmap and written in ascending order.
//   5. Exact fallback: rows with fewer than k or more than kCap candidates
//      (the sample misjudged them) are flagged; the plain indexer and top-k
//      then run for the flagged rows only (every workgroup of those launches
//      exits at once when no row is flagged).
#include "common.h"
#include "kernels.h"
#include "select_util.h"

namespace sa {

constexpr int kSample = 16;     // sample stride (positions)
constexpr int64_t kCap = 8192;  // candidates kept per row
constexpr int kSelThreads = 256;
constexpr int kSelPer = (int)(kCap / kSelThreads);  // candidates per thread
constexpr int kMaxS = 32768;                        // bitmap of the select step
constexpr int kThrPer = 2048 / 64;                  // sampled keys per lane (S / 16 <= 2048)

// Sample rank for k: k/16 rounded up, plus six standard deviations of a
// binomial count of that mean, plus a constant.
__host__ __device__ inline int fused_rank(int64_t k) {
  const int m = (int)((k + kSample - 1) / kSample);
  int sd = 1;
  while (sd * sd < m) ++sd;
  return m + 6 * sd + 8;
}

struct FusedLayout {
  size_t ks, sscore, thresh, cnt, fail, anyf, cand, fb, total;
};

static FusedLayout fused_layout(int64_t B, int64_t T, int64_t S) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t Ss = S / kSample, rows = B * T;
  FusedLayout L;
  size_t off = 0;
  L.ks = off;
  off += al((size_t)(B * Ss) * 256);
  L.sscore = off;
  off += al((size_t)(rows * Ss) * 4);
  L.thresh = off;
  off += al((size_t)rows * 4);
  L.cnt = off;
  off += al((size_t)rows * 4);
  L.fail = off;
  off += al((size_t)rows * 4);
  L.anyf = off;
  off += 256;
  L.cand = off;
  off += al((size_t)(rows * kCap) * 8);
  L.fb = off;
  off += al((size_t)(rows * S) * 4);
  L.total = off;
  return L;
}

size_t dsa_indexer_topk_ws_bytes(int64_t B, int64_t T, int64_t S, int64_t k) {
  (void)k;
  return fused_layout(B, T, S).total;
}

struct FusedPtrs {
  const bf16_t* ks;
  const float* sscore;
  uint32_t* thresh;
  uint32_t* cnt;
  uint32_t* fail;
  uint32_t* anyf;
  const uint2* cand;
  int64_t Ss;
};

// ks[b, j] = k[b, 16j + 15]: 16 threads per 256-byte row.
__global__ __launch_bounds__(256) void fused_sample_kernel(const bf16_t* k, bf16_t* ks, int64_t B, int64_t S,
                                                           int64_t Ss) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= B * Ss * 16) return;
  const int64_t c = t & 15, r = t >> 4, b = r / Ss, j = r % Ss;
  const uint4* src = reinterpret_cast<const uint4*>(k + (b * S + j * kSample + kSample - 1) * 128) + c;
  reinterpret_cast<uint4*>(ks + r * 128)[c] = *src;
}

// One wave per row: clears the row's count and flag, and writes the
// threshold key (0: every visible position is a candidate).
__global__ __launch_bounds__(256) void fused_thresh_kernel(DsaIndexerTopkParams p, FusedPtrs f) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blockIdx.x == 0 && threadIdx.x == 0) *f.anyf = 0u;
  if (row >= p.B * p.T) return;
  const int64_t b = row / p.T, i = row % p.T;
  const int64_t base = p.q_pos ? p.q_pos[b] : 0;
  if (lane == 0) {
    f.cnt[row] = 0u;
    f.fail[row] = 0u;
  }
  int64_t n = base + i + 1;
  n = n < p.S ? n : p.S;
  uint32_t V = 0u;
  if (p.force_fallback) {
    V = 0xffffffffu;  // no finite score reaches it: every long row takes the exact fallback
  } else if (n > p.topk) {
    int64_t ns = (base + i + 1) / kSample;
    ns = ns < f.Ss ? ns : f.Ss;
    const uint32_t r = (uint32_t)fused_rank(p.topk);
    if (ns > (int64_t)r) {
      const float* ss = f.sscore + row * f.Ss;
      uint32_t kv[kThrPer];
#pragma unroll
      for (int t = 0; t < kThrPer; ++t) {
        const int64_t j = lane + 64 * t;
        kv[t] = j < ns ? score_key(ss[j]) : 0u;  // 0: absent (below every threshold tried)
      }
      // Largest V with at least r keys >= V, bit by bit from the top.
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t tv = V | (1u << bit);
        uint32_t c = 0;
#pragma unroll
        for (int t = 0; t < kThrPer; ++t) c += kv[t] >= tv ? 1u : 0u;
        if (wave_sum_u32(c) >= r) V = tv;
      }
    }
  }
  if (lane == 0) f.thresh[row] = V;
}

// One workgroup per row: the exact k-th largest candidate key K by rounds of
// histograms over the key interval [lo, hi] (first [threshold, max]; 2048
// bins of 2^shift keys, each round at least 1024 times narrower, one-key
// bins end it), then the kept positions in an LDS bitmap, written in order.
__global__ __launch_bounds__(kSelThreads) void fused_select_kernel(DsaIndexerTopkParams p, FusedPtrs f) {
  constexpr int kBinsSel = 2048;
  __shared__ uint32_t hist[kBinsSel];
  __shared__ uint32_t sel[kMaxS / 32];
  __shared__ uint32_t tie[kMaxS / 32];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t res[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t b = row / p.T, i = row % p.T;
  const int64_t base = p.q_pos ? p.q_pos[b] : 0;
  int64_t n = base + i + 1;
  n = n < p.S ? n : p.S;
  const int k = (int)p.topk;
  int32_t* out = p.idx + row * p.topk;
  if (n <= k) {  // every visible position
    for (int j = tid; j < k; j += kSelThreads) out[j] = j < n ? j : -1;
    return;
  }
  const uint32_t c = f.cnt[row];
  if (c < (uint32_t)k || c > (uint32_t)kCap) {  // the exact fallback writes this row
    if (tid == 0) {
      f.fail[row] = 1u;
      atomicOr(f.anyf, 1u);
    }
    return;
  }
  const uint2* cr = f.cand + row * kCap;
  uint32_t kv[kSelPer], ps[kSelPer];
  uint32_t mx = 0u;
#pragma unroll
  for (int t = 0; t < kSelPer; ++t) {
    const uint32_t j = (uint32_t)(tid + kSelThreads * t);
    const uint2 e = j < c ? cr[j] : make_uint2(0u, 0u);
    kv[t] = e.x;
    ps[t] = e.y;
    mx = max(mx, e.x);
  }
  mx = wave_max_u32(mx);
  if ((tid & 63) == 0) scratch[tid >> 6] = mx;
  __syncthreads();
  uint32_t hi = 0u;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) hi = max(hi, scratch[w]);
  __syncthreads();
  // Every candidate key is >= the row's threshold; absent slots hold 0 and
  // fall outside [lo, hi] (lo >= 1 whenever a real key is 0 never occurs).
  uint32_t lo = f.thresh[row];
  uint32_t need = (uint32_t)k;  // keys still to take from [lo, hi]
  while (lo < hi) {
    const uint32_t range = hi - lo, sh = bin_shift(range);
    for (int j = tid; j < kBinsSel; j += kSelThreads) hist[j] = 0u;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kSelPer; ++t) {
      const uint32_t d = kv[t] - lo;  // wraps for keys below lo (and absent slots when lo > 0)
      if (tid + kSelThreads * t < (int)c && d <= range) atomicAdd(&hist[d >> sh], 1u);
    }
    __syncthreads();
    select_bin(hist, kBinsSel, need, scratch, &res[0], &res[1]);
    const uint32_t bsel = uniform_u32(res[0]);
    need -= uniform_u32(res[1]);
    hi = lo + min(range, (bsel << sh) | ((1u << sh) - 1u));
    lo = lo + (bsel << sh);
    __syncthreads();
  }
  const uint32_t K = lo;  // k-th largest key; `need` copies of it are taken
  for (int w = tid; w < kMaxS / 32; w += kSelThreads) {
    sel[w] = 0u;
    tie[w] = 0u;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kSelPer; ++t) {
    if (tid + kSelThreads * t < (int)c) {
      const uint32_t bit = 1u << (ps[t] & 31u);
      if (kv[t] > K) atomicOr(&sel[ps[t] >> 5], bit);
      else if (kv[t] == K) atomicOr(&tie[ps[t] >> 5], bit);
    }
  }
  __syncthreads();
  // Thread t owns bitmap words 4t .. 4t+3 (positions 128t .. 128t+127, in order).
  constexpr int kWords = kMaxS / 32 / kSelThreads;
  uint32_t tc = 0;
#pragma unroll
  for (int u = 0; u < kWords; ++u) tc += (uint32_t)__popc(tie[kWords * tid + u]);
  uint32_t tot;
  uint32_t rank = block_inclusive_scan(tc, scratch, tot) - tc;  // copies of K at lower positions
#pragma unroll
  for (int u = 0; u < kWords; ++u) {
    uint32_t w = tie[kWords * tid + u], add = 0u;
    while (w != 0u && rank < need) {
      const uint32_t low = w & (~w + 1u);
      add |= low;
      w ^= low;
      ++rank;
    }
    sel[kWords * tid + u] |= add;
  }
  __syncthreads();
  uint32_t sc = 0;
#pragma unroll
  for (int u = 0; u < kWords; ++u) sc += (uint32_t)__popc(sel[kWords * tid + u]);
  uint32_t o = block_inclusive_scan(sc, scratch, tot) - sc;
#pragma unroll
  for (int u = 0; u < kWords; ++u) {
    uint32_t w = sel[kWords * tid + u];
    while (w != 0u) {
      const int bpos = __ffs((int)w) - 1;
      out[o++] = (kWords * tid + u) * 32 + bpos;
      w &= w - 1u;
    }
  }
}

hipError_t launch_dsa_indexer_topk(const DsaIndexerTopkParams& p, hipStream_t stream) {
  const FusedLayout L = fused_layout(p.B, p.T, p.S);
  char* ws = reinterpret_cast<char*>(p.ws);
  const int64_t Ss = p.S / kSample, rows = p.B * p.T;
  FusedPtrs f;
  f.ks = reinterpret_cast<const bf16_t*>(ws + L.ks);
  f.sscore = reinterpret_cast<const float*>(ws + L.sscore);
  f.thresh = reinterpret_cast<uint32_t*>(ws + L.thresh);
  f.cnt = reinterpret_cast<uint32_t*>(ws + L.cnt);
  f.fail = reinterpret_cast<uint32_t*>(ws + L.fail);
  f.anyf = reinterpret_cast<uint32_t*>(ws + L.anyf);
  f.cand = reinterpret_cast<const uint2*>(ws + L.cand);
  f.Ss = Ss;
  float* fb = reinterpret_cast<float*>(ws + L.fb);
  hipError_t e;

  // 1. Sampled scores (ratio-16 visibility).
  if (Ss > 0) {
    const int64_t nthr = p.B * Ss * 16;
    hipLaunchKernelGGL(fused_sample_kernel, dim3((uint32_t)((nthr + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<const bf16_t*>(p.k), const_cast<bf16_t*>(f.ks), p.B, p.S, Ss);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    DsaIndexerParams sp{};
    sp.q = p.q;
    sp.k = f.ks;
    sp.w = p.w;
    sp.q_pos = p.q_pos;
    sp.scores = const_cast<float*>(f.sscore);
    sp.B = p.B;
    sp.T = p.T;
    sp.S = Ss;
    sp.ratio = kSample;
    if ((e = launch_dsa_indexer(sp, stream)) != hipSuccess) return e;
  }
  // 2. Thresholds (also clears counts and flags).
  hipLaunchKernelGGL(fused_thresh_kernel, dim3((uint32_t)((rows + 3) / 4)), dim3(256), 0, stream, p, f);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 3. Candidates.
  DsaIndexerParams ep{};
  ep.q = p.q;
  ep.k = p.k;
  ep.w = p.w;
  ep.q_pos = p.q_pos;
  ep.scores = fb;
  ep.B = p.B;
  ep.T = p.T;
  ep.S = p.S;
  ep.ratio = 1;
  ep.thresh = f.thresh;
  ep.cnt = f.cnt;
  ep.cand = const_cast<uint2*>(f.cand);
  ep.cap = kCap;
  ep.topk = p.topk;
  if ((e = launch_dsa_indexer(ep, stream)) != hipSuccess) return e;
  // 4. Exact selection over the candidates.
  hipLaunchKernelGGL(fused_select_kernel, dim3((uint32_t)rows), dim3(kSelThreads), 0, stream, p, f);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 5. Exact fallback for flagged rows (every workgroup returns at once when none is).
  DsaIndexerParams fp{};
  fp.q = p.q;
  fp.k = p.k;
  fp.w = p.w;
  fp.q_pos = p.q_pos;
  fp.scores = fb;
  fp.B = p.B;
  fp.T = p.T;
  fp.S = p.S;
  fp.ratio = 1;
  fp.row_flag = f.fail;
  fp.any_flag = f.anyf;
  if ((e = launch_dsa_indexer(fp, stream)) != hipSuccess) return e;
  DsaTopkParams tp{};
  tp.scores = fb;
  tp.q_pos = p.q_pos;
  tp.idx = p.idx;
  tp.B = p.B;
  tp.T = p.T;
  tp.S = p.S;
  tp.k = p.topk;
  tp.ws = nullptr;
  tp.ratio = 1;
  tp.row_flag = f.fail;
  tp.any_flag = f.anyf;
  return launch_dsa_topk(tp, stream);
}

}  // namespace sa

// DSA exact top-k selection (gfx950).
//
// Method: [P1] §二.1, [P3] §架構創新 1 -- keep only the top-K scoring history
// positions per query.  Order: score descending, then position ascending
// (ties go to the lower position); -0.0 ranks equal to +0.0.  The selected
// positions are written in ascending order, padded with -1.
//
// Radix select on order-preserving 32-bit keys (3 digits: 11 + 11 + 10 bits).
// Each pass histograms the digit of the keys that still match the selected
// prefix and picks the bin where the count from the top reaches k.  After
// the last pass the k-th key K is exact, with `above` keys strictly greater
// and need = k - above copies of K to take (the lowest positions first).
// The output is then an ordered compaction: position s is kept iff
// key > K, or key == K and fewer than `need` copies of K precede it; its
// output slot is #(key > K before s) + min(#(key == K before s), need).
//
// Rows up to 32768 positions: one workgroup per row keeps the whole row of
// keys in registers.  Longer rows: a multi-workgroup pipeline with
// histograms and per-chunk counts in the workspace.  All counts are integers,
// so both paths give bit-identical, run-to-run stable results.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kTopkThreads = 1024;
constexpr int kBins = 2048;
// Digit layout of the 32-bit key: bits 31..21, 20..10, 9..0.
__device__ __forceinline__ int digit_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t digit_mask(int pass) { return pass == 2 ? 0x3ffu : 0x7ffu; }
constexpr int kMwThreads = 256;
constexpr int kMwChunk = 16384;  // positions per workgroup in the multi-workgroup path

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int64_t row_len(const DsaTopkParams& p, int64_t b, int64_t i) {
  const int64_t base = p.q_pos ? p.q_pos[b] : 0;
  int64_t n = base + i + 1;
  if (n > p.S) n = p.S;
  if (n < 0) n = 0;
  return n;
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

// Given hist[0..nbins) and need >= 1 (<= total count), find the bin where the
// count from the top reaches need.  Result: *sel_bin, *sel_above (count in
// bins strictly above).  Uses all threads; nbins <= 2 * blockDim.x.
__device__ void select_bin(const uint32_t* hist, int nbins, uint32_t need, uint32_t* scratch, uint32_t* sel_bin,
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

// ---------------------------------------------------------------------------
// Rows up to kRegRow positions: one 512-thread workgroup per row holds the
// whole row of keys in registers.  Thread t owns positions 4*(t + 512*j) + e
// (j < 16, e < 4), read with 16-byte loads that are all in flight at once.
// The ordered compaction scans packed (greater, equal) counts per 4-element
// group: lane prefix inside the wave, then a table of per-(group, wave)
// totals in LDS.
// ---------------------------------------------------------------------------
constexpr int kRegThreads = 512;
constexpr int kRegWaves = kRegThreads / kWave;
constexpr int kRegVec = 16;                            // 4-element groups per thread
constexpr int kRegRow = kRegThreads * kRegVec * 4;     // 32768

__global__ __launch_bounds__(kRegThreads) void dsa_topk_reg_kernel(DsaTopkParams p) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t res[2];
  __shared__ uint32_t wtot[kRegVec][kRegWaves];  // packed counts per (group j, wave)

  const int64_t row = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t b = row / p.T, i = row % p.T;
  const int n = (int)row_len(p, b, i);
  const int k = (int)p.k;
  int32_t* out = p.idx + row * p.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (n <= k) {
    for (int j = tid; j < k; j += kRegThreads) out[j] = j < n ? j : -1;
    return;
  }
  const float* sc = p.scores + row * p.S;

  // Keys (0 marks a position past the row end; only an all-ones NaN also maps
  // to 0).  Every load is unconditional (clamped into the row) so that all
  // of them are in flight together; positions >= n are masked afterwards.
  uint32_t key[kRegVec][4];
  if ((p.S & 3) == 0) {  // 16-byte aligned rows
    float4 f[kRegVec];
#pragma unroll
    for (int j = 0; j < kRegVec; ++j) {
      const int pos0 = min(4 * (tid + kRegThreads * j), (int)p.S - 4);
      f[j] = *reinterpret_cast<const float4*>(sc + pos0);
    }
#pragma unroll
    for (int j = 0; j < kRegVec; ++j) {
      const int pos0 = 4 * (tid + kRegThreads * j);
      key[j][0] = pos0 + 0 < n ? score_key(f[j].x) : 0u;
      key[j][1] = pos0 + 1 < n ? score_key(f[j].y) : 0u;
      key[j][2] = pos0 + 2 < n ? score_key(f[j].z) : 0u;
      key[j][3] = pos0 + 3 < n ? score_key(f[j].w) : 0u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kRegVec; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = 4 * (tid + kRegThreads * j) + e;
        const float f = sc[min(pos, (int)p.S - 1)];
        key[j][e] = pos < n ? score_key(f) : 0u;
      }
  }

  uint32_t prefix = 0, need = (uint32_t)k;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    for (int j = tid; j < kBins; j += kRegThreads) hist[j] = 0;
    __syncthreads();
    const int sh = digit_shift(pass);
    const uint32_t dm = digit_mask(pass);
    const int sh_prev = pass > 0 ? digit_shift(pass - 1) : 0;
#pragma unroll
    for (int j = 0; j < kRegVec; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kv = key[j][e];
        const bool match = kv != 0u && (pass == 0 || (kv >> sh_prev) == prefix);
        if (match) atomicAdd(&hist[(kv >> sh) & dm], 1u);
      }
    __syncthreads();
    select_bin(hist, (int)dm + 1, need, scratch, &res[0], &res[1]);
    prefix = (prefix << (pass == 0 ? 0 : (sh_prev - sh))) | res[0];
    need -= res[1];
    __syncthreads();
  }
  const uint32_t K = prefix;  // the k-th largest key; need = copies of K to take

  // Packed counts: low 16 bits = keys > K, high 16 bits = keys == K.
  uint32_t incl[kRegVec];
#pragma unroll
  for (int j = 0; j < kRegVec; ++j) {
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) c += (key[j][e] > K ? 1u : 0u) + (key[j][e] == K ? 0x10000u : 0u);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(c, off);
      if (lane >= off) c += y;
    }
    incl[j] = c;
    if (lane == 63) wtot[j][wave] = c;
  }
  __syncthreads();
  // Exclusive prefix of the (group, wave) totals in position order (group-major).
  if (tid == 0) {
    uint32_t run = 0;
    for (int j = 0; j < kRegVec; ++j)
      for (int w = 0; w < kRegWaves; ++w) {
        const uint32_t t = wtot[j][w];
        wtot[j][w] = run;
        run += t;
      }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kRegVec; ++j) {
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) c += (key[j][e] > K ? 1u : 0u) + (key[j][e] == K ? 0x10000u : 0u);
    uint32_t before = wtot[j][wave] + incl[j] - c;
    const int pos0 = 4 * (tid + kRegThreads * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t kv = key[j][e];
      const uint32_t g_b = before & 0xffffu, e_b = before >> 16;
      const bool take = kv > K || (kv == K && e_b < need);
      const uint32_t slot = g_b + (e_b < need ? e_b : need);
      if (take && slot < (uint32_t)k) out[slot] = pos0 + e;
      before += (kv > K ? 1u : 0u) + (kv == K ? 0x10000u : 0u);
    }
  }
}

// ---------------------------------------------------------------------------
// Long rows: multi-workgroup pipeline.
// Workspace layout (uint32): hist[rows][kBins] | state[rows][4] | cnt[rows][nchunk][2]
// state: 0 = prefix, 1 = need, 2 = above_total, 3 = unused
// ---------------------------------------------------------------------------
struct MwLayout {
  uint32_t* hist;
  uint32_t* state;
  uint32_t* cnt;
  int64_t nchunk;
};

__device__ __forceinline__ MwLayout mw_layout(const DsaTopkParams& p) {
  const int64_t rows = p.B * p.T;
  MwLayout m;
  m.hist = reinterpret_cast<uint32_t*>(p.ws);
  m.state = m.hist + rows * kBins;
  m.cnt = m.state + rows * 4;
  m.nchunk = (p.S + kMwChunk - 1) / kMwChunk;
  return m;
}

__global__ __launch_bounds__(kMwThreads) void topk_mw_init(DsaTopkParams p) {
  const MwLayout m = mw_layout(p);
  const int64_t row = blockIdx.x;
  for (int j = threadIdx.x; j < kBins; j += kMwThreads) m.hist[row * kBins + j] = 0;
  if (threadIdx.x == 0) {
    m.state[row * 4 + 0] = 0;
    m.state[row * 4 + 1] = (uint32_t)p.k;
    m.state[row * 4 + 2] = 0;
    m.state[row * 4 + 3] = 0;
  }
}

__global__ __launch_bounds__(kMwThreads) void topk_mw_hist(DsaTopkParams p, int pass) {
  __shared__ uint32_t lh[kBins];
  const MwLayout m = mw_layout(p);
  const int64_t row = blockIdx.x / m.nchunk, chunk = blockIdx.x % m.nchunk;
  const int64_t b = row / p.T, i = row % p.T;
  const int64_t n = row_len(p, b, i);
  if (n <= p.k) return;
  const int64_t s_beg = chunk * kMwChunk, s_fin = imin64(n, s_beg + kMwChunk);
  if (s_beg >= s_fin) return;
  for (int j = threadIdx.x; j < kBins; j += kMwThreads) lh[j] = 0;
  __syncthreads();
  const uint32_t prefix = m.state[row * 4 + 0];
  const float* sc = p.scores + row * p.S;
  const int sh = digit_shift(pass);
  const uint32_t dm = digit_mask(pass);
  const int sh_prev = pass > 0 ? digit_shift(pass - 1) : 32;
  for (int64_t s = s_beg + threadIdx.x; s < s_fin; s += kMwThreads) {
    const uint32_t key = score_key(sc[s]);
    const bool match = pass == 0 || (key >> sh_prev) == prefix;
    if (match) atomicAdd(&lh[(key >> sh) & dm], 1u);
  }
  __syncthreads();
  for (int j = threadIdx.x; j <= (int)dm; j += kMwThreads) {
    const uint32_t c = lh[j];
    if (c) atomicAdd(&m.hist[row * kBins + j], c);
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_mw_select(DsaTopkParams p, int pass) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t res[2];
  const MwLayout m = mw_layout(p);
  const int64_t row = blockIdx.x;
  const int64_t b = row / p.T, i = row % p.T;
  const int64_t n = row_len(p, b, i);
  if (n <= p.k) return;
  const int nb = (int)digit_mask(pass) + 1;
  for (int j = threadIdx.x; j < kBins; j += kTopkThreads) {
    h[j] = m.hist[row * kBins + j];
    m.hist[row * kBins + j] = 0;  // ready for the next pass
  }
  __syncthreads();
  const uint32_t need = m.state[row * 4 + 1];
  select_bin(h, nb, need, scratch, &res[0], &res[1]);
  if (threadIdx.x == 0) {
    const uint32_t prefix = m.state[row * 4 + 0];
    const int widen = pass == 0 ? 0 : (digit_shift(pass - 1) - digit_shift(pass));
    m.state[row * 4 + 0] = (prefix << widen) | res[0];
    m.state[row * 4 + 1] = need - res[1];
    m.state[row * 4 + 2] += res[1];
  }
}

__global__ __launch_bounds__(kMwThreads) void topk_mw_count(DsaTopkParams p) {
  __shared__ uint32_t part[2][kMwThreads / kWave];
  const MwLayout m = mw_layout(p);
  const int64_t row = blockIdx.x / m.nchunk, chunk = blockIdx.x % m.nchunk;
  const int64_t b = row / p.T, i = row % p.T;
  const int64_t n = row_len(p, b, i);
  if (n <= p.k) return;
  const int64_t s_beg = chunk * kMwChunk, s_fin = imin64(n, s_beg + kMwChunk);
  const uint32_t K = m.state[row * 4 + 0];
  const float* sc = p.scores + row * p.S;
  uint32_t gt = 0, eq = 0;
  for (int64_t s = s_beg + threadIdx.x; s < s_fin; s += kMwThreads) {
    const uint32_t key = score_key(sc[s]);
    gt += key > K;
    eq += key == K;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    gt += __shfl_xor(gt, off);
    eq += __shfl_xor(eq, off);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    part[0][wave] = gt;
    part[1][wave] = eq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t g = 0, e = 0;
    for (int w = 0; w < kMwThreads / kWave; ++w) {
      g += part[0][w];
      e += part[1][w];
    }
    m.cnt[(row * m.nchunk + chunk) * 2 + 0] = g;
    m.cnt[(row * m.nchunk + chunk) * 2 + 1] = e;
  }
}

__global__ __launch_bounds__(kMwThreads) void topk_mw_write(DsaTopkParams p) {
  __shared__ uint32_t wcnt[2][kMwThreads / kWave];
  const MwLayout m = mw_layout(p);
  const int64_t row = blockIdx.x / m.nchunk, chunk = blockIdx.x % m.nchunk;
  const int64_t b = row / p.T, i = row % p.T;
  const int64_t n = row_len(p, b, i);
  int32_t* out = p.idx + row * p.k;
  if (n <= p.k) {  // keep every candidate
    for (int64_t j = chunk * kMwChunk + threadIdx.x; j < imin64(p.k, (chunk + 1) * kMwChunk); j += kMwThreads)
      out[j] = j < n ? (int32_t)j : -1;
    return;
  }
  const int64_t s_beg = chunk * kMwChunk, s_fin = imin64(n, s_beg + kMwChunk);
  if (s_beg >= s_fin) return;
  const uint32_t K = m.state[row * 4 + 0];
  const uint32_t need = m.state[row * 4 + 1];
  uint32_t gt_before = 0, eq_before = 0;
  for (int64_t c = 0; c < chunk; ++c) {
    gt_before += m.cnt[(row * m.nchunk + c) * 2 + 0];
    eq_before += m.cnt[(row * m.nchunk + c) * 2 + 1];
  }
  // Wave w of this chunk owns positions [s_beg + w*seg, ...).
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kW = kMwThreads / kWave;
  const int64_t seg = kMwChunk / kW;
  const int64_t w_beg = s_beg + wave * seg, w_fin = imin64(s_fin, w_beg + seg);
  const float* sc = p.scores + row * p.S;
  uint32_t g = 0, e = 0;
  for (int64_t s0 = w_beg; s0 < w_fin; s0 += 64) {
    const int64_t s = s0 + lane;
    const bool in = s < w_fin;
    const uint32_t key = in ? score_key(sc[s]) : 0u;
    g += __popcll(__ballot(in && key > K));
    e += __popcll(__ballot(in && key == K));
  }
  if (lane == 0) {
    wcnt[0][wave] = g;
    wcnt[1][wave] = e;
  }
  __syncthreads();
  for (int w = 0; w < wave; ++w) {
    gt_before += wcnt[0][w];
    eq_before += wcnt[1][w];
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t s0 = w_beg; s0 < w_fin; s0 += 64) {
    const int64_t s = s0 + lane;
    const bool in = s < w_fin;
    const uint32_t key = in ? score_key(sc[s]) : 0u;
    const uint64_t mgt = __ballot(in && key > K);
    const uint64_t meq = __ballot(in && key == K);
    const uint32_t g_b = gt_before + __popcll(mgt & below);
    const uint32_t e_b = eq_before + __popcll(meq & below);
    const uint32_t slot = g_b + (e_b < need ? e_b : need);
    if (in && (key > K || (key == K && e_b < need)) && slot < (uint32_t)p.k) out[slot] = (int32_t)s;
    gt_before += __popcll(mgt);
    eq_before += __popcll(meq);
  }
}

size_t dsa_topk_ws_bytes(int64_t B, int64_t T, int64_t S, int64_t k) {
  (void)k;
  if (S <= kRegRow) return 0;
  const int64_t rows = B * T;
  const int64_t nchunk = (S + kMwChunk - 1) / kMwChunk;
  return (size_t)(rows * kBins + rows * 4 + rows * nchunk * 2) * sizeof(uint32_t);
}

hipError_t launch_dsa_topk(const DsaTopkParams& p, hipStream_t stream) {
  const int64_t rows = p.B * p.T;
  if (p.S <= kRegRow) {
    hipLaunchKernelGGL(dsa_topk_reg_kernel, dim3((uint32_t)rows), dim3(kRegThreads), 0, stream, p);
    return hipGetLastError();
  }
  const int64_t nchunk = (p.S + kMwChunk - 1) / kMwChunk;
  hipLaunchKernelGGL(topk_mw_init, dim3((uint32_t)rows), dim3(kMwThreads), 0, stream, p);
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(topk_mw_hist, dim3((uint32_t)(rows * nchunk)), dim3(kMwThreads), 0, stream, p, pass);
    hipLaunchKernelGGL(topk_mw_select, dim3((uint32_t)rows), dim3(kTopkThreads), 0, stream, p, pass);
  }
  hipLaunchKernelGGL(topk_mw_count, dim3((uint32_t)(rows * nchunk)), dim3(kMwThreads), 0, stream, p);
  hipLaunchKernelGGL(topk_mw_write, dim3((uint32_t)(rows * nchunk)), dim3(kMwThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa

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
//      margin of 4.5 standard deviations) cut to its top 16 bits, or 0 when
//      the row has at most r samples.
//   3. Candidates: the indexer runs in candidate mode and writes (key,
//      position) of every score whose key is >= the row's threshold, per
//      chunk of positions into the row's segment for that chunk; its scores
//      are the same fp32 values as in dsa_indexer_scores (same code, same
//      order of accumulation).
//   4. Select: if a row has at least k and at most kCap candidates, the k-th
//      largest key K over them is the k-th largest of the row (at least k
//      keys lie above the threshold, so every key of the top k, ties of K
//      included, is a candidate).  Rounds of key histograms narrow the key
//      interval holding K; positions with larger keys and the lowest `need`
//      positions with key K are marked in an LDS bitmap and written in
//      ascending order.
//   5. Exact fallback: rows with fewer than k or more than kCap candidates
//      (the sample misjudged them) are flagged; the plain indexer and top-k
//      then run for the flagged rows only (every workgroup of those launches
//      exits at once when no row is flagged).
#include "common.h"
#include "kernels.h"
#include "select_util.h"

namespace sa {

constexpr int kSample = 16;     // sample stride (positions)
constexpr int64_t kCap = 4096;  // most candidates the select step holds per row
constexpr int kSelPer = (int)(kCap / 64);           // candidates per lane (one wave per row)
constexpr int kMaxS = 32768;                        // bitmap of the select step
constexpr int kThrPer = 2048 / 64;                  // sampled keys per lane (S / 16 <= 2048)

// Sample rank for k: k/16 rounded up, plus four and a half standard
// deviations of a binomial count of that mean, plus a constant.  At k = 2048
// (rank 190) a row has about 3040 candidates; with scores independent of
// position, fewer than k or (pads included) more than kCap of them take
// about 4.5 standard deviations of the sample either way.
__host__ __device__ inline int fused_rank(int64_t k) {
  const int m = (int)((k + kSample - 1) / kSample);
  int sd = 1;
  while (sd * sd < m) ++sd;
  return m + (9 * sd + 1) / 2 + 8;
}

constexpr int kMaxSeg = 128;  // chunks of the candidate launch per row (S / 256 at most)

struct FusedLayout {
  size_t ks, sscore, thresh, cnt, fail, anyf, cand, total;
};

// Candidate rows are pitched at Sp = S rounded up to even: a row whose last
// chunk is all candidates with an odd length puts its pad entry at index S,
// which then stays in the row, and every row starts 16-byte aligned (the
// select step loads entry pairs as 16 bytes).  The exact fallback's scores
// ([rows, S] fp32) reuse the candidate area ([rows, Sp] pairs): they are
// written after the select step has read it.
static int64_t cand_pitch(int64_t S) { return (S + 1) & ~(int64_t)1; }
static FusedLayout fused_layout(int64_t B, int64_t T, int64_t S) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t Ss = S / kSample, rows = B * T;
  const int64_t nseg = (S + dsa_indexer_chunk(T) - 1) / dsa_indexer_chunk(T);
  FusedLayout L;
  size_t off = 0;
  L.ks = off;
  off += al((size_t)(B * Ss) * 256);
  L.sscore = off;
  off += al((size_t)(rows * Ss) * 2);
  L.thresh = off;
  off += al((size_t)rows * 4);
  L.cnt = off;
  off += al((size_t)(rows * nseg) * 4);
  L.fail = off;
  off += al((size_t)rows * 4);
  L.anyf = off;
  off += 256;
  L.cand = off;
  off += al((size_t)(rows * cand_pitch(S)) * 8);
  L.total = off;
  return L;
}

size_t dsa_indexer_topk_ws_bytes(int64_t B, int64_t T, int64_t S, int64_t k) {
  (void)k;
  return fused_layout(B, T, S).total;
}

struct FusedPtrs {
  const bf16_t* ks;
  const uint16_t* skey;  // [rows, Ss]: top 16 bits of the sampled scores' keys
  uint32_t* thresh;
  const uint32_t* cnt;  // [rows, nseg]
  uint32_t* fail;
  uint32_t* anyf;
  const uint2* cand;  // [rows, Sp]: segment c at c * chunk
  int64_t Ss, chunk, nseg, pitch;
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

// One wave per row: clears the row's fallback flag, and writes the
// threshold key (0: every visible position is a candidate).  The threshold is
// the r-th largest sampled key cut to its top 16 bits (two rounds of 256-bin
// histograms over the key's top two bytes), so at least r sampled keys reach
// it; exactness never depends on it (the select step checks the counts).
__global__ __launch_bounds__(256) void fused_thresh_kernel(DsaIndexerTopkParams p, FusedPtrs f) {
  __shared__ __attribute__((aligned(16))) uint32_t hist_all[4][256];
  const int lane = threadIdx.x & 63;
  uint32_t* hist = hist_all[threadIdx.x >> 6];
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blockIdx.x == 0 && threadIdx.x == 0) *f.anyf = 0u;
  if (row >= p.B * p.T) return;
  const int64_t b = row / p.T, i = row % p.T;
  const int64_t base = p.q_pos ? p.q_pos[b] : 0;
  if (lane == 0) f.fail[row] = 0u;
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
      const uint16_t* ss = f.skey + row * f.Ss;
      uint32_t kv[kThrPer];
#pragma unroll
      for (int t = 0; t < kThrPer; ++t) {
        const int64_t j = lane + 64 * t;
        kv[t] = j < ns ? (uint32_t)ss[j] << 16 : 0u;  // the key's top 16 bits: all the threshold uses
      }
      reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
      wave_lds_sync();
#pragma unroll
      for (int t = 0; t < kThrPer; ++t)
        if (lane + 64 * t < ns) atomicAdd(&hist[kv[t] >> 24], 1u);
      wave_lds_sync();
      uint32_t d1, above, cnt;
      wave_top_bin256(hist, r, &d1, &above, &cnt);
      wave_lds_sync();
      reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
      wave_lds_sync();
#pragma unroll
      for (int t = 0; t < kThrPer; ++t)
        if (lane + 64 * t < ns && (kv[t] >> 24) == d1) atomicAdd(&hist[(kv[t] >> 16) & 255u], 1u);
      wave_lds_sync();
      uint32_t d2;
      wave_top_bin256(hist, r - above, &d2, &above, &cnt);
      V = (d1 << 24) | (d2 << 16);
    }
  }
  if (lane == 0) f.thresh[row] = V;
}

// One wave per row.  The row's candidates stay in registers (keys, and
// positions packed two per register).  Rounds of 256-bin histograms over the
// key interval [lo, hi] (first [threshold, max]) narrow it to the bin where
// the count from the top reaches k, until the interval holds exactly the
// keys still needed or a single key.  Keys above the interval are kept; of
// the keys in it, all when their count is what is needed, else (one key,
// tied) the lowest positions.  Kept positions are marked in an LDS bitmap
// and written in ascending order.
__global__ __launch_bounds__(64) void fused_select_kernel(DsaIndexerTopkParams p, FusedPtrs f) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[256];
  __shared__ __attribute__((aligned(16))) uint32_t bm[kMaxS / 32];
  __shared__ uint32_t pre[kMaxSeg + 1];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t b = row / p.T, i = row % p.T;
  const int64_t base = p.q_pos ? p.q_pos[b] : 0;
  int64_t n = base + i + 1;
  n = n < p.S ? n : p.S;
  const int k = (int)p.topk;
  int32_t* out = p.idx + row * p.topk;
  if (n <= k) {  // every visible position
    for (int j = lane; j < k; j += 64) out[j] = j < n ? j : -1;
    return;
  }
  // The row's candidates: segments 0 .. nseg-1 (one per chunk holding a
  // visible position), each padded to an even length, concatenated;
  // pre[s] = entries before segment s.
  const int nseg = (int)((n + f.chunk - 1) / f.chunk);
  uint32_t c = 0u, cp = 0u;  // candidates; entries with pads
  for (int s0 = 0; s0 < nseg; s0 += 64) {
    const int si = s0 + lane;
    const uint32_t v = si < nseg ? f.cnt[row * f.nseg + si] : 0u;
    const uint32_t incl = wave_incl_scan((v + 1u) & ~1u) + cp;
    if (si < nseg) pre[si + 1] = incl;
    cp = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    c += wave_sum_u32(v);
  }
  if (lane == 0) pre[0] = 0u;
  if (c < (uint32_t)k || cp > (uint32_t)kCap) {  // the exact fallback writes this row
    if (lane == 0) {
      f.fail[row] = 1u;
      atomicOr(f.anyf, 1u);
    }
    return;
  }
  wave_lds_sync();
  // Lane l takes entry pairs m = l + 64u (entries 2m, 2m + 1; a pair never
  // straddles segments) with one 16-byte load: keys to kv[2u], kv[2u + 1],
  // positions to ps[2u], ps[2u + 1].  Nothing loaded is used before the loop
  // ends, so the loads are all in flight together.  Lanes past the end load
  // the last pair again; `valid` excludes them, and the pads.
  const uint2* cr = f.cand + row * f.pitch;
  uint32_t kv[kSelPer], ps[kSelPer];
  int seg = 0;  // this lane's segment; entries j of it lie in [seg_lo, seg_hi)
  uint32_t seg_lo = 0u, seg_hi = pre[1];
#pragma unroll
  for (int u = 0; u < kSelPer / 2; ++u) {
    kv[2 * u] = kv[2 * u + 1] = ps[2 * u] = ps[2 * u + 1] = 0u;
    if (128 * u < (int)cp) {
      const uint32_t j = min((uint32_t)(2 * (lane + 64 * u)), cp - 2u);
      while (j >= seg_hi) {
        ++seg;
        seg_lo = seg_hi;
        seg_hi = pre[seg + 1];
      }
      const uint4 e = *reinterpret_cast<const uint4*>(cr + (int64_t)seg * f.chunk + (j - seg_lo));
      kv[2 * u] = e.x;
      ps[2 * u] = e.y;
      kv[2 * u + 1] = e.z;
      ps[2 * u + 1] = e.w;
    }
  }
  auto valid = [&](int t) __attribute__((always_inline)) {
    return 2 * (lane + 64 * (t >> 1)) < (int)cp && kv[t] != 0u;
  };
  auto pos = [&](int t) __attribute__((always_inline)) { return ps[t]; };
  uint32_t mx = 0u;
#pragma unroll
  for (int t = 0; t < kSelPer; ++t) mx = max(mx, valid(t) ? kv[t] : 0u);
  uint32_t hi = wave_max_u32(mx);
  uint32_t lo = f.thresh[row];  // every candidate key is in [lo, hi]
  uint32_t need = (uint32_t)k;  // keys still to take from [lo, hi]
  uint32_t in_range = c;        // candidate keys in [lo, hi]
  while (lo < hi && in_range != need) {
    const uint32_t range = hi - lo, sh = bin_shift256(range);
    reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < kSelPer; ++t) {
      if (128 * (t >> 1) < (int)cp) {
        const uint32_t d = kv[t] - lo;  // wraps for keys below lo
        if (valid(t) && d <= range) atomicAdd(&hist[d >> sh], 1u);
      }
    }
    wave_lds_sync();
    uint32_t bsel, above;
    wave_top_bin256(hist, need, &bsel, &above, &in_range);
    wave_lds_sync();
    need -= above;
    hi = lo + min(range, (bsel << sh) | ((1u << sh) - 1u));
    lo = lo + (bsel << sh);
  }
  const bool take_range = in_range == need;
#pragma unroll
  for (int q = 0; q < kMaxS / 32 / 256; ++q) reinterpret_cast<uint4*>(bm)[lane + 64 * q] = make_uint4(0u, 0u, 0u, 0u);
  wave_lds_sync();
  if (!take_range) {
    // A single key K = lo = hi with more copies than needed: mark them, then
    // keep the `need` lowest.  Lane l owns words 16l .. 16l + 15.
#pragma unroll
    for (int t = 0; t < kSelPer; ++t) {
      if (128 * (t >> 1) < (int)cp) {
        if (valid(t) && kv[t] == lo) atomicOr(&bm[pos(t) >> 5], 1u << (pos(t) & 31u));
      }
    }
    wave_lds_sync();
    constexpr int kOwn = kMaxS / 32 / 64;
    uint32_t w[kOwn], tc = 0u;
#pragma unroll
    for (int u = 0; u < kOwn; ++u) {
      w[u] = bm[kOwn * lane + u];
      tc += (uint32_t)__popc(w[u]);
    }
    uint32_t rank = wave_incl_scan(tc) - tc;  // copies at lower positions
#pragma unroll
    for (int u = 0; u < kOwn; ++u) {
      const uint32_t pc = (uint32_t)__popc(w[u]);
      if (rank >= need) {
        w[u] = 0u;
      } else if (rank + pc > need) {
        uint32_t keep = 0u, x = w[u];
        for (uint32_t m = need - rank; m > 0u; --m) {
          const uint32_t low = x & (~x + 1u);
          keep |= low;
          x ^= low;
        }
        w[u] = keep;
      }
      rank += pc;
      bm[kOwn * lane + u] = w[u];
    }
    wave_lds_sync();
  }
#pragma unroll
  for (int t = 0; t < kSelPer; ++t) {
    if (128 * (t >> 1) < (int)cp) {
      if (valid(t) && (kv[t] > hi || (take_range && kv[t] >= lo))) atomicOr(&bm[pos(t) >> 5], 1u << (pos(t) & 31u));
    }
  }
  wave_lds_sync();
  // Output: 64 words (2048 positions) per step, one word per lane.
  const int nw = (int)((n + 31) / 32);
  uint32_t o_base = 0u;
  for (int cw = 0; cw < nw; cw += 64) {
    uint32_t w = cw + lane < nw ? bm[cw + lane] : 0u;
    const uint32_t pc = (uint32_t)__popc(w);
    const uint32_t incl = wave_incl_scan(pc);
    uint32_t o = o_base + incl - pc;
    while (w != 0u) {
      out[o++] = (cw + lane) * 32 + (__ffs((int)w) - 1);
      w &= w - 1u;
    }
    o_base += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  }
}

hipError_t launch_dsa_indexer_topk(const DsaIndexerTopkParams& p, hipStream_t stream) {
  const FusedLayout L = fused_layout(p.B, p.T, p.S);
  char* ws = reinterpret_cast<char*>(p.ws);
  const int64_t Ss = p.S / kSample, rows = p.B * p.T;
  FusedPtrs f;
  f.ks = reinterpret_cast<const bf16_t*>(ws + L.ks);
  f.skey = reinterpret_cast<const uint16_t*>(ws + L.sscore);
  f.thresh = reinterpret_cast<uint32_t*>(ws + L.thresh);
  f.cnt = reinterpret_cast<const uint32_t*>(ws + L.cnt);
  f.fail = reinterpret_cast<uint32_t*>(ws + L.fail);
  f.anyf = reinterpret_cast<uint32_t*>(ws + L.anyf);
  f.cand = reinterpret_cast<const uint2*>(ws + L.cand);
  f.Ss = Ss;
  f.chunk = dsa_indexer_chunk(p.T);
  f.nseg = (p.S + f.chunk - 1) / f.chunk;
  f.pitch = cand_pitch(p.S);
  float* fb = reinterpret_cast<float*>(ws + L.cand);
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
    sp.keys16 = const_cast<uint16_t*>(f.skey);
    sp.B = p.B;
    sp.T = p.T;
    sp.S = Ss;
    sp.ratio = kSample;
    if ((e = launch_dsa_indexer(sp, stream)) != hipSuccess) return e;
  }
  // 2. Thresholds (also clears the fallback flags).
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
  ep.cnt = const_cast<uint32_t*>(f.cnt);
  ep.cand = const_cast<uint2*>(f.cand);
  ep.cand_pitch = f.pitch;
  ep.topk = p.topk;
  if ((e = launch_dsa_indexer(ep, stream)) != hipSuccess) return e;
  // 4. Exact selection over the candidates.
  hipLaunchKernelGGL(fused_select_kernel, dim3((uint32_t)rows), dim3(64), 0, stream, p, f);
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

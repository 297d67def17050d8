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
constexpr int kSelStage = 1024;  // kept positions the select stages in LDS per output step
constexpr int kThrPer = 2048 / 64;                  // sampled keys per lane (S / 16 <= 2048)

// Sample rank for k at sample stride st: k/st rounded up, plus four and a
// half standard deviations of a binomial count of that mean, plus a
// constant.  At k = 2048 and stride 16 (rank 190) a row has about 3040
// candidates; with scores independent of position, fewer than k or (pads
// included) more than kCap of them take about 4.5 standard deviations of the
// sample either way, whatever the stride.
__host__ __device__ inline int fused_rank(int64_t k, int st = kSample) {
  const int m = (int)((k + st - 1) / st);
  int sd = 1;
  while (sd * sd < m) ++sd;
  return m + (9 * sd + 1) / 2 + 8;
}

// Long decode rows sample every kSampleL-th key: a 1M-position row still has
// 16384 samples, and the sampling pass and the threshold read a quarter of
// what stride 16 reads.  At k = 2048 the rank is 66 and a row has about 4200
// candidates (the sample's 4.5 standard deviations: about 2000 above k).
constexpr int kSampleL = 64;

constexpr int kCapL = 8192;  // candidates the long-row select holds per row
constexpr int kMaxSeg = 128;  // chunks of the candidate launch per row (S / 256 at most)

struct FusedLayout {
  size_t ks, sscore, thresh, cnt, fail, anyf, cand, total;
  size_t comp, ctot;  // long rows only
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
  FusedLayout L{};
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

// Long decode rows (T <= 4, S > 32768): candidates per chunk of the decode
// indexer (dsa_indexer_dec_chunk() positions), rows pitched at the chunks'
// total; the exact fallback's scores ([rows, S] fp32) reuse the area.  The
// compacted candidates take kCapL entries per row, and their count a word.
static bool fused_long(int64_t T, int64_t S) { return T <= 4 && S > kMaxS; }

__host__ __device__ inline int64_t pad8(int64_t x) { return (x + 7) & ~(int64_t)7; }
static FusedLayout fused_layout_long(int64_t B, int64_t T, int64_t S) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t rows = B * T, ch = dsa_indexer_dec_chunk();
  const int64_t nch = (S + ch - 1) / ch;
  FusedLayout L{};
  size_t off = 0;
  L.ks = off;  // unused: the sampled keys are scored in place
  L.sscore = off;  // rows pitched at a multiple of 8 keys
  off += al((size_t)(rows * pad8(S / kSampleL)) * 2);
  L.thresh = off;
  off += al((size_t)rows * 4);
  L.cnt = off;  // rows pitched at a multiple of 8 counts
  off += al((size_t)(rows * pad8(nch)) * 4);
  L.fail = off;
  off += al((size_t)rows * 4);
  L.anyf = off;
  off += 256;
  L.comp = off;
  off += al((size_t)(rows * kCapL) * 8);
  L.ctot = off;
  off += al((size_t)rows * 4);
  L.cand = off;
  off += al((size_t)(rows * nch * ch) * 8);
  L.total = off;
  return L;
}

size_t dsa_indexer_topk_ws_bytes(int64_t B, int64_t T, int64_t S, int64_t k) {
  (void)k;
  return fused_long(T, S) ? fused_layout_long(B, T, S).total : fused_layout(B, T, S).total;
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
  int64_t spitch, cpitch;  // long rows: row pitches of skey and cnt (multiples of 8)
  uint2* comp;              // long rows: [rows, kCapL] candidates in position order
  uint32_t* ctot;           // long rows: [rows] candidate count
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

// One wave per row.  The row's candidates stay in registers (keys and
// positions, one register each).  Rounds of 256-bin histograms over the
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
  __shared__ uint32_t ostage[kSelStage];
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
  // Output: 64 words (2048 positions) per step, one word per lane.  A step's
  // kept positions go to an LDS stage in order and then out with full-wave
  // stores (a lane's own positions, stored one by one, would take a store
  // instruction per position with few lanes active); a step keeping more
  // than the stage holds (short, dense rows) stores directly.
  const int nw = (int)((n + 31) / 32);
  uint32_t o_base = 0u;
  for (int cw = 0; cw < nw; cw += 64) {
    uint32_t w = cw + lane < nw ? bm[cw + lane] : 0u;
    const uint32_t pc = (uint32_t)__popc(w);
    const uint32_t incl = wave_incl_scan(pc);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (total <= (uint32_t)kSelStage) {
      uint32_t o = incl - pc;
      while (w != 0u) {
        ostage[o++] = (cw + lane) * 32 + (__ffs((int)w) - 1);
        w &= w - 1u;
      }
      wave_lds_sync();
      for (uint32_t j = lane; j < total; j += 64) out[o_base + j] = (int32_t)ostage[j];
      wave_lds_sync();  // the stage's reads are done before the next step writes it
    } else {
      uint32_t o = o_base + incl - pc;
      while (w != 0u) {
        out[o++] = (cw + lane) * 32 + (__ffs((int)w) - 1);
        w &= w - 1u;
      }
    }
    o_base += total;
  }
}

// ---------------------------------------------------------------------------
// Long decode rows.  Sampled keys: the decode indexer scores every
// kSampleL-th key in place (no copy of the sampled keys) and stores the top
// 16 bits of their keys.  Threshold: one 256-thread workgroup per row, the r-th largest
// sampled key from LDS histograms.
// Compaction: the rows' candidates, scattered over per-chunk segments, are
// packed in position order by many workgroups.  Select: one workgroup per row
// over the row's packed candidates, loaded into LDS with one round of
// coalesced loads (kFromScores: over the row's full scores, for the
// rows flagged for the exact fallback): the k-th largest key K by four rounds
// of 8-bit histograms, then every key above K and the lowest-position `need`
// copies of K, written in position order.
// ---------------------------------------------------------------------------

// The r-th largest of the row's sampled keys above zero (top 16 bits), in
// two rounds: a 4096-bin histogram of their top 12 bits, then a 16-bin one of
// the low 4 bits of the keys in the chosen bin.  (Bins of 12 bits split the
// keys finely enough that a wave's lanes rarely add to one bin together,
// where 8-bit bins put most of a row in a handful of bins.  A score is
// exactly zero wherever every head's product is negative, about one position
// in sixteen: zero and negative scores are left out, and a row with fewer
// than r samples above zero gets threshold 0.)
// Threads of the long-row threshold workgroup: a 1M-position row has 16384
// samples, 64 per thread in one round of loads.
constexpr int kThrL = 256;
__global__ __launch_bounds__(kThrL) void fused_thresh_long_kernel(DsaIndexerTopkParams p, FusedPtrs f) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[4096];
  __shared__ uint32_t scr[32];
  __shared__ uint32_t res[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t b = row / p.T, i = row % p.T;
  const int64_t base = p.q_pos ? p.q_pos[b] : 0;
  if (blockIdx.x == 0 && tid == 0) *f.anyf = 0u;
  if (tid == 0) f.fail[row] = 0u;
  int64_t n = base + i + 1;
  n = n < p.S ? n : p.S;
  if (p.force_fallback) {  // no finite score reaches it: every long row takes the exact fallback
    if (tid == 0) f.thresh[row] = 0xffffffffu;
    return;
  }
  int64_t ns = (base + i + 1) / kSampleL;  // the row's sampled positions
  ns = ns < f.Ss ? ns : f.Ss;
  const uint32_t r = (uint32_t)fused_rank(p.topk, kSampleL);
  if (n <= p.topk || ns <= (int64_t)r) {  // every visible position is a candidate
    if (tid == 0) f.thresh[row] = 0u;
    return;
  }
  // The row's keys, 8 per 16-byte load (the row is pitched at a multiple of
  // 8): each pass issues 8 loads per thread together, 64 * kThrL keys.
  const uint4* ss = reinterpret_cast<const uint4*>(f.skey + row * f.spitch);
  const int64_t nv = (ns + 7) / 8;
  auto key_of = [&](const uint4& v, int e, int64_t j) -> uint32_t {  // key e of the group at vector j (0: none)
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    const uint32_t k16 = (e & 1) ? w >> 16 : w & 0xffffu;
    return 8 * j + e < ns ? k16 : 0u;
  };
  uint32_t V = 0u;
  // Round 1: top 12 bits.  (Rows of up to 64 * kThrL samples keep their keys
  // in registers for round 2.)
  for (int j = tid; j < 4096; j += kThrL) hist[j] = 0u;
  __syncthreads();
  uint4 v[8];
  for (int64_t j0 = 0; j0 < nv; j0 += 8 * kThrL) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = j0 + u * kThrL + tid;
      v[u] = j < nv ? ss[j] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t k16 = key_of(v[u], e, j0 + u * kThrL + tid);
        if (k16 > 0x8000u) atomicAdd(&hist[k16 >> 4], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t tot;
  {
    // Thread t owns bins [4096 - kPer(t+1), 4096 - kPer t) (thread 0: the top
    // bins), read as kPer/4 16-byte words.
    constexpr int kPer = 4096 / kThrL;
    uint32_t c[kPer];  // c[e]: bin 4096 - kPer t - 1 - e
#pragma unroll
    for (int w = 0; w < kPer / 4; ++w) {
      const uint4 h = reinterpret_cast<const uint4*>(hist)[(4096 - kPer * (tid + 1)) / 4 + (kPer / 4 - 1 - w)];
      c[4 * w] = h.w;
      c[4 * w + 1] = h.z;
      c[4 * w + 2] = h.y;
      c[4 * w + 3] = h.x;
    }
    uint32_t local = 0u;
#pragma unroll
    for (int e = 0; e < kPer; ++e) local += c[e];
    const uint32_t incl = block_inclusive_scan(local, scr, tot);
    uint32_t above = incl - local;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (above < r && above + c[e] >= r) {
        res[0] = (uint32_t)(4096 - kPer * tid - 1 - e);
        res[1] = above;
      }
      above += c[e];
    }
  }
  if (tot >= r) {  // uniform: tot comes from the block scan
    __syncthreads();
    const uint32_t b12 = res[0], need = r - res[1];
    // Round 2: low 4 bits of the keys in bin b12.
    if (tid < 16) hist[tid] = 0u;
    __syncthreads();
    for (int64_t j0 = 0; j0 < nv; j0 += 8 * kThrL) {
      if (nv > 8 * kThrL) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t j = j0 + u * kThrL + tid;
          v[u] = j < nv ? ss[j] : make_uint4(0u, 0u, 0u, 0u);
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t k16 = key_of(v[u], e, j0 + u * kThrL + tid);
          if (k16 > 0x8000u && (k16 >> 4) == b12) atomicAdd(&hist[k16 & 15u], 1u);
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t above = 0u;
      for (int e = 15; e >= 0; --e) {
        if (above < need && above + hist[e] >= need) V = ((b12 << 4) | (uint32_t)e) << 16;
        above += hist[e];
      }
    }
  }
  if (tid == 0) f.thresh[row] = V;
}

// Compaction: workgroup (row, c) takes segments [256c, 256c + 256) of the
// row, one per thread; its offset is the count of the segments before them,
// and its entries go to comp[row * kCapL + offset ..] in position order (the
// entries past kCapL are dropped: the select step sends such rows to the
// exact fallback).  The workgroup holding the row's last segment writes the
// row's total.  Spread over many CUs, the scattered segment reads overlap.
constexpr int kCompSeg = 256;
__global__ __launch_bounds__(kCompSeg) void fused_compact_long_kernel(DsaIndexerTopkParams p, FusedPtrs f) {
  __shared__ uint32_t scr[32];
  const int tid = threadIdx.x;
  const int64_t nblk = (f.nseg + kCompSeg - 1) / kCompSeg;
  const int64_t row = blockIdx.x / nblk, bk = blockIdx.x % nblk;
  const int64_t b = row / p.T, i = row % p.T;
  const int64_t base = p.q_pos ? p.q_pos[b] : 0;
  int64_t n = base + i + 1;
  n = n < p.S ? n : p.S;
  if (n <= p.topk) return;  // the select step writes such rows directly
  const int64_t nseg = (n + f.chunk - 1) / f.chunk;
  const int64_t sg0 = bk * kCompSeg;
  if (sg0 >= nseg) return;
  const uint32_t* cnt = f.cnt + row * f.cpitch;
  const uint2* cr = f.cand + row * f.pitch;
  const int64_t sg = sg0 + tid;
  // This thread's segment: count and first two entries, loaded together.
  const uint32_t c = sg < nseg ? cnt[sg] : 0u;
  const uint4 x = sg < nseg ? *reinterpret_cast<const uint4*>(cr + sg * f.chunk) : make_uint4(0u, 0u, 0u, 0u);
  // Counts of the earlier segments (sg0 is a multiple of 8: 16-byte loads).
  uint32_t before = 0u;
  for (int64_t j = 8 * tid; j < sg0; j += 8 * kCompSeg) {
    const uint4 a = *reinterpret_cast<const uint4*>(cnt + j), d = *reinterpret_cast<const uint4*>(cnt + j + 4);
    before += a.x + a.y + a.z + a.w + d.x + d.y + d.z + d.w;
  }
  uint32_t off0;
  block_inclusive_scan(before, scr, off0);
  uint32_t tb;
  const uint32_t o = off0 + block_inclusive_scan(c, scr, tb) - c;
  uint2* dst = f.comp + row * kCapL;
  if (c > 0u && o < (uint32_t)kCapL) dst[o] = make_uint2(x.x, x.y);
  if (c > 1u && o + 1u < (uint32_t)kCapL) dst[o + 1u] = make_uint2(x.z, x.w);
  for (uint32_t e = 2; e < c && o + e < (uint32_t)kCapL; ++e) dst[o + e] = cr[sg * f.chunk + e];
  if (sg0 + kCompSeg >= nseg && tid == 0) f.ctot[row] = off0 + tb;
}

template <bool kFromScores>
__global__ __launch_bounds__(1024) void fused_select_long_kernel(DsaIndexerTopkParams p, FusedPtrs f, const float* scores) {
  __shared__ uint32_t ckey[kFromScores ? 1 : kCapL];
  __shared__ uint32_t cpos[kFromScores ? 1 : kCapL];
  __shared__ __attribute__((aligned(16))) uint32_t hist[256];
  __shared__ uint32_t scr[32];
  __shared__ uint32_t bc[2];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t b = row / p.T, i = row % p.T;
  const int64_t base = p.q_pos ? p.q_pos[b] : 0;
  int64_t n = base + i + 1;
  n = n < p.S ? n : p.S;
  const int k = (int)p.topk;
  int32_t* out = p.idx + row * p.topk;
  uint32_t m;  // elements: candidates, or the row's visible positions
  if constexpr (kFromScores) {
    if (*f.anyf == 0u || f.fail[row] == 0u) return;
    m = (uint32_t)n;
  } else {
    if (n <= k) {  // every visible position
      for (int j = tid; j < k; j += 1024) out[j] = j < n ? j : -1;
      return;
    }
    // The row's candidates, compacted in position order.
    const uint32_t tot = f.ctot[row];
    if (tot < (uint32_t)k || tot > (uint32_t)kCapL) {  // the exact fallback writes this row
      if (tid == 0) {
        f.fail[row] = 1u;
        atomicOr(f.anyf, 1u);
      }
      return;
    }
    const uint2* src = f.comp + row * kCapL;
    uint2 x[kCapL / 1024];
#pragma unroll
    for (int u = 0; u < kCapL / 1024; ++u) {
      const uint32_t j = (uint32_t)(u * 1024 + tid);
      x[u] = j < tot ? src[j] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kCapL / 1024; ++u) {
      const uint32_t j = (uint32_t)(u * 1024 + tid);
      if (j < tot) {
        ckey[j] = x[u].x;
        cpos[j] = x[u].y;
      }
    }
    __syncthreads();
    m = tot;
  }
  auto key_at = [&](uint32_t j) -> uint32_t {
    if constexpr (kFromScores)
      return score_key(scores[row * p.S + j]);
    else
      return ckey[j];
  };
  uint32_t prefix = 0u, mask = 0u, need = (uint32_t)k;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int sh = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (uint32_t j0 = 0; j0 < m; j0 += 1024) {
      const uint32_t j = j0 + tid;
      const uint32_t key = j < m ? key_at(j) : 0u;
      lds_hist_add(hist, (j < m && (key & mask) == prefix) ? (key >> sh) & 255u : 256u);
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t bin, above, cnt;
      wave_top_bin256(hist, need, &bin, &above, &cnt);
      if (tid == 0) {
        bc[0] = bin;
        bc[1] = above;
      }
    }
    __syncthreads();
    prefix |= bc[0] << sh;
    mask |= 0xffu << sh;
    need -= bc[1];
    __syncthreads();
  }
  // prefix is the k-th largest key K; keep every key above it and the
  // `need` lowest-position copies of it.  Each thread walks a contiguous
  // range of elements (position order).
  const uint32_t K = prefix;
  const uint32_t per = (m + 1023u) / 1024u, j0 = tid * per, j1 = j0 + per < m ? j0 + per : m;
  uint32_t ties = 0u;
  for (uint32_t j = j0; j < j1; ++j) ties += key_at(j) == K ? 1u : 0u;
  uint32_t tt;
  const uint32_t tie0 = block_inclusive_scan(ties, scr, tt) - ties;
  uint32_t kept = 0u, tr = tie0;
  for (uint32_t j = j0; j < j1; ++j) {
    const uint32_t key = key_at(j);
    if (key > K) {
      ++kept;
    } else if (key == K) {
      if (tr < need) ++kept;
      ++tr;
    }
  }
  uint32_t kt;
  uint32_t ob = block_inclusive_scan(kept, scr, kt) - kept;
  tr = tie0;
  for (uint32_t j = j0; j < j1; ++j) {
    const uint32_t key = key_at(j);
    bool keep = key > K;
    if (key == K) {
      keep = tr < need;
      ++tr;
    }
    if (keep) {
      if constexpr (kFromScores)
        out[ob] = (int32_t)j;
      else
        out[ob] = (int32_t)cpos[j];
      ++ob;
    }
  }
}

static hipError_t launch_fused_long(const DsaIndexerTopkParams& p, hipStream_t stream) {
  const FusedLayout L = fused_layout_long(p.B, p.T, p.S);
  char* ws = reinterpret_cast<char*>(p.ws);
  const int64_t Ss = p.S / kSampleL, rows = p.B * p.T, ch = dsa_indexer_dec_chunk();
  FusedPtrs f{};
  f.ks = nullptr;
  f.skey = reinterpret_cast<const uint16_t*>(ws + L.sscore);
  f.thresh = reinterpret_cast<uint32_t*>(ws + L.thresh);
  f.cnt = reinterpret_cast<const uint32_t*>(ws + L.cnt);
  f.fail = reinterpret_cast<uint32_t*>(ws + L.fail);
  f.anyf = reinterpret_cast<uint32_t*>(ws + L.anyf);
  f.cand = reinterpret_cast<const uint2*>(ws + L.cand);
  f.Ss = Ss;
  f.chunk = ch;
  f.nseg = (p.S + ch - 1) / ch;
  f.pitch = f.nseg * ch;
  f.spitch = pad8(Ss);
  f.cpitch = pad8(f.nseg);
  f.comp = reinterpret_cast<uint2*>(ws + L.comp);
  f.ctot = reinterpret_cast<uint32_t*>(ws + L.ctot);
  float* fb = reinterpret_cast<float*>(ws + L.cand);
  hipError_t e;
  // 1. Sampled keys: every kSampleL-th key scored in place (ratio-kSampleL
  // visibility), top 16 bits of the score keys.
  if (Ss > 0) {
    DsaIndexerParams sp{};
    sp.q = p.q;
    sp.k = p.k;
    sp.w = p.w;
    sp.q_pos = p.q_pos;
    sp.keys16 = const_cast<uint16_t*>(f.skey);
    sp.B = p.B;
    sp.T = p.T;
    sp.S = Ss;
    sp.ratio = kSampleL;
    sp.dec_sample = 1;
    sp.k_rows = p.S;
    if ((e = launch_dsa_indexer(sp, stream)) != hipSuccess) return e;
  }
  // 2. Thresholds (also clears the fallback flags).
  hipLaunchKernelGGL(fused_thresh_long_kernel, dim3((uint32_t)rows), dim3(kThrL), 0, stream, p, f);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 3. Candidates, per chunk in position order.
  DsaIndexerParams ep{};
  ep.q = p.q;
  ep.k = p.k;
  ep.w = p.w;
  ep.q_pos = p.q_pos;
  ep.B = p.B;
  ep.T = p.T;
  ep.S = p.S;
  ep.ratio = 1;
  ep.thresh = f.thresh;
  ep.cnt = const_cast<uint32_t*>(f.cnt);
  ep.cand = const_cast<uint2*>(f.cand);
  ep.cand_pitch = f.pitch;
  ep.topk = p.topk;
  ep.dec_cand = 1;
  if ((e = launch_dsa_indexer(ep, stream)) != hipSuccess) return e;
  // 4. Compaction, then the exact selection over the candidates.
  hipLaunchKernelGGL(fused_compact_long_kernel, dim3((uint32_t)(rows * ((f.nseg + kCompSeg - 1) / kCompSeg))),
                     dim3(kCompSeg), 0, stream, p, f);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(fused_select_long_kernel<false>, dim3((uint32_t)rows), dim3(1024), 0, stream, p, f, fb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 5. Exact fallback for flagged rows: their full scores, then the selection
  // over them (both return at once when no row is flagged).
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
  fp.dec_filter = 1;
  if ((e = launch_dsa_indexer(fp, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(fused_select_long_kernel<true>, dim3((uint32_t)rows), dim3(1024), 0, stream, p, f, fb);
  return hipGetLastError();
}

hipError_t launch_dsa_indexer_topk(const DsaIndexerTopkParams& p, hipStream_t stream) {
  if (fused_long(p.T, p.S)) return launch_fused_long(p, stream);
  const FusedLayout L = fused_layout(p.B, p.T, p.S);
  char* ws = reinterpret_cast<char*>(p.ws);
  const int64_t Ss = p.S / kSample, rows = p.B * p.T;
  FusedPtrs f{};
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

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
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "select_util.h"

namespace sa {

constexpr int kBins = 2048;
// Digit layout of the 32-bit key: bits 31..21, 20..10, 9..0.
__device__ __forceinline__ int digit_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t digit_mask(int pass) { return pass == 2 ? 0x3ffu : 0x7ffu; }
constexpr int kMwThreads = 256;
constexpr int kMwChunk = 4096;   // positions per workgroup in the multi-workgroup path


// Candidates of row i: keys s < (base + i + 1) / ratio (positions s <= base + i
// for ratio 1), at most S.
__device__ __forceinline__ int64_t row_len(const DsaTopkParams& p, int64_t b, int64_t i) {
  const int64_t base = p.q_pos ? p.q_pos[b] : 0;
  int64_t n = (base + i + 1) / p.ratio;
  if (n > p.S) n = p.S;
  if (n < 0) n = 0;
  return n;
}




// ---------------------------------------------------------------------------
// Rows up to kRegRow positions: one workgroup per row holds the whole row
// of keys in registers.  Thread t of kThreads owns positions
// 4*(t + kThreads*j) + e (j < 16, e < 4), read with 16-byte loads that are
// all in flight at once.  The workgroup is sized to the row: 128, 256 or 512
// threads for rows of up to 8192, 16384 or 32768 positions, so that short
// (causal) rows take fewer lanes and more of them run on a CU at once.
// The work is bound by vector ALU instructions per key, so every sweep over
// the 64 keys of a thread is kept short:
//
//  1. Find the k-th largest key K* exactly.  Candidates are the keys in an
//     interval [lo, hi] of key values, first the row's extremes.  A round
//     histograms the candidates by (key - lo) >> shift, with shift chosen so
//     that the bins are 2^shift keys wide and (hi - lo) lands in bins
//     1024..2047; the bin where the count from the top reaches the number of
//     keys still needed gives the next, exact interval (at least 1024 times
//     narrower; one-key bins end it).  Once at most kCandLds candidates are
//     left they move to LDS with their positions and further rounds run over
//     those; at most kCandCap are finally ranked pairwise by one wave.
//  2. With K* and need_eq (copies of K* to take, lowest positions first),
//     an ordered compaction emits position s iff key > K*, or key == K* and
//     fewer than need_eq copies precede s.  Packed (greater, equal) counts
//     are scanned inside each wave with DPP, then across (group, wave).
// ---------------------------------------------------------------------------
constexpr int kRegVec = 16;                  // 4-element groups per thread
constexpr int kRegRow = 512 * kRegVec * 4;   // 32768: longest row of the largest workgroup
constexpr int64_t kFilterGrid = 512;  // workgroups of the flagged-rows launch (one per CU at a time: two rounds)
constexpr int kCandPer = 4;                  // LDS candidates per thread
constexpr int kCandCap = kWave;              // ranked pairwise by one wave


// Rows i0 .. i0 + ni - 1 of every batch entry, one workgroup each.
// kFilter: only rows with row_flag[row] != 0 run (and none unless *any_flag),
// on a bounded grid whose workgroups walk the rows.
template <int kThreads, bool kFilter>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kFilter ? 2 : 4))) void dsa_topk_reg_kernel(
    DsaTopkParams p, int64_t i0, int64_t ni) {
  constexpr int kRegThreads = kThreads;
  constexpr int kRegWaves = kRegThreads / kWave;
  constexpr int kCandLds = kCandPer * kRegThreads;  // candidates moved to LDS
  __shared__ uint32_t hist[kBins];  // also the staging buffer of the output row
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t res[8];
  __shared__ uint32_t wtot[kRegVec * kRegWaves];
  __shared__ uint32_t red[3][kRegWaves];
  __shared__ uint32_t ckey[kCandLds];
  __shared__ uint32_t cpos[kCandLds];
  __shared__ int32_t sink[kWave];

  // Rows are dealt round-robin over the XCDs (the hardware's own order):
  // causal rows grow with i, and a contiguous range per XCD would give the
  // last XCD the longest loads.
  // One row (lid: its index among the launch's rows).
  auto run_row = [&](const int64_t lid) __attribute__((always_inline)) {
  const int64_t b = lid / ni, i = i0 + lid % ni;
  const int64_t row = b * p.T + i;
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
  // to 0 and is never selected).  Every load is unconditional so that all of
  // them are in flight together; loads past the row end are clamped onto its
  // last 16 bytes (a cache hit) and masked afterwards.
  uint32_t key[kRegVec][4];
  if ((p.S & 3) == 0) {  // 16-byte aligned rows
    const int last4 = (n - 1) & ~3;
    float4 f[kRegVec];
#pragma unroll
    for (int j = 0; j < kRegVec; ++j) {
      const int pos0 = min(4 * (tid + kRegThreads * j), last4);
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
        const float f = sc[min(pos, n - 1)];
        key[j][e] = pos < n ? score_key(f) : 0u;
      }
  }
  // A re-read of the key registers that the compiler cannot see through, so
  // that a sweep recomputes its per-key predicates instead of keeping 64 of
  // them alive (in scalar registers) from an earlier sweep.  Only used where
  // every control path has merged: a refresh inside a branch would make the
  // compiler keep both versions of the keys.
  auto refresh_keys = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kRegVec; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(key[j][e]));
  };
  // Workgroup-wide (min, max, sum) of per-thread values; uniform results.
  auto reduce3 = [&](uint32_t a, uint32_t z, uint32_t c, uint32_t& mn, uint32_t& mx, uint32_t& sum) __attribute__((always_inline)) {
    a = wave_min_u32(a);
    z = wave_max_u32(z);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += (uint32_t)__shfl_xor((int)c, off);
    if (lane == 0) {
      red[0][wave] = a;
      red[1][wave] = z;
      red[2][wave] = c;
    }
    __syncthreads();
    mn = 0xffffffffu;
    mx = 0u;
    sum = 0u;
#pragma unroll
    for (int w = 0; w < kRegWaves; ++w) {
      mn = min(mn, red[0][w]);
      mx = max(mx, red[1][w]);
      sum += red[2][w];
    }
    mn = uniform_u32(mn);
    mx = uniform_u32(mx);
    sum = uniform_u32(sum);
    __syncthreads();  // red may be reused
  };
  // One refinement round over nk keys per thread: histogram of the keys in
  // [lo, hi], select the bin where the count from the top reaches need, and
  // narrow [lo, hi], need and cand to it.
  auto round = [&](auto nk_tag, auto&& keys_of, uint32_t& lo, uint32_t& hi, uint32_t& need, uint32_t& cand) __attribute__((always_inline)) {
    constexpr int nk = decltype(nk_tag)::value;
    const uint32_t range = hi - lo, sh = bin_shift(range);
    for (int j = tid; j < kBins; j += kRegThreads) hist[j] = 0;
    if (tid == 0) {
      res[0] = 0;
      res[1] = 0;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < nk; ++m) {
      const uint32_t d = keys_of(m) - lo;  // wraps for keys below lo
      if (d <= range) atomicAdd(&hist[d >> sh], 1u);
    }
    __syncthreads();
    select_bin(hist, kBins, need, scratch, &res[0], &res[1]);
    const uint32_t bsel = uniform_u32(res[0]);
    need -= uniform_u32(res[1]);
    cand = uniform_u32(hist[bsel]);
    // Keys of bin bsel: lo + [bsel << sh, (bsel << sh) | (2^sh - 1)], clipped
    // to the old range (no overflow: the upper offset never passes range's
    // top bits).
    hi = lo + min(range, (bsel << sh) | ((1u << sh) - 1u));
    lo = lo + (bsel << sh);
    __syncthreads();  // hist and res may be rewritten
  };

  // Candidates (keys in [lo, hi]) to LDS with their positions, thread t's at
  // slots base_t, base_t + 1, ... (base_t from a scan of per-thread counts).
  auto gather = [&](uint32_t glo, uint32_t ghi, uint32_t base) __attribute__((always_inline)) {
    // Opaque copies of the bounds: the membership tests are recomputed here
    // rather than kept (64 masks) from the counting sweep before the scan.
    glo = uniform_u32(glo);
    ghi = uniform_u32(ghi);
    asm volatile("" : "+s"(glo), "+s"(ghi));
    uint32_t pb = 4u * (uint32_t)tid;
    asm volatile("" : "+v"(pb));
    uint32_t r = base;
#pragma unroll
    for (int j = 0; j < kRegVec; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kv = key[j][e];
        const bool in = kv - glo <= ghi - glo;
        if (in) {
          ckey[r] = kv;
          cpos[r] = pb + (uint32_t)(4 * kRegThreads * j + e);
        }
        r += in ? 1u : 0u;
      }
  };

  // ---- 1. the k-th largest key K* and the copies of it to take -------------
  uint32_t lo, hi, nsel;
  {
    uint32_t a = 0xffffffffu, z = 0u, c = 0u;
#pragma unroll
    for (int j = 0; j < kRegVec; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kv = key[j][e];
        a = min(a, kv - 1u);  // an absent key (0) wraps to the top
        z = max(z, kv);
        c += kv != 0u ? 1u : 0u;
      }
    reduce3(a, z, c, lo, hi, nsel);
    lo += 1u;
  }
  uint32_t need = (uint32_t)k;  // keys still to take from [lo, hi]
  uint32_t Kt = 1u, need_eq = 0u, eq_total = 0u;  // defaults: take every selectable key
  if (nsel > need) {
    uint32_t cand = nsel;
    bool in_lds = false;  // the cand candidates are in ckey/cpos[0, cand)
    if (cand > (uint32_t)kCandLds && lo < hi) {
      // Sampled bracket: histogram the keys at every 4th position, take the
      // bins where the sample count from the top passes need/4 minus and
      // plus a margin of about four standard deviations, then count the row
      // exactly against the bracket [L, H].  If the k-th key lies inside and
      // at most kCandLds keys do, those keys go straight to LDS and no
      // full-row refinement round is needed.
      const uint32_t range = hi - lo, sh = bin_shift(range);
      for (int j = tid; j < kBins; j += kRegThreads) hist[j] = 0;
      if (tid == 0) {
        res[0] = 0;
        res[1] = 0;
        res[2] = 0;
        res[3] = 0;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kRegVec; ++j) {
        const uint32_t d = key[j][0] - lo;
        if (d <= range) atomicAdd(&hist[d >> sh], 1u);
      }
      __syncthreads();
      const float ns = (float)((n + 3) >> 2);  // sampled positions
      const float mu = (float)need * ns / (float)nsel;
      const float margin = 4.f * sqrtf(mu) + 8.f;
      const uint32_t t_hi = mu - margin >= 1.f ? (uint32_t)(mu - margin) : 0u;  // 0: no upper cut
      const uint32_t t_lo = (uint32_t)fminf(mu + margin, ns);
      select_bins2(hist, kBins, t_hi > 0u ? t_hi : 1u, max(t_lo, 1u), scratch, res);
      const uint32_t b_hi = uniform_u32(res[0]), b_lo = uniform_u32(res[2]);
      const uint32_t L = lo + (b_lo << sh);
      // Top key of bin b_hi; (b << sh) | (2^sh - 1) cannot pass range's top bits.
      const uint32_t H = t_hi > 0u ? lo + min(range, (b_hi << sh) | ((1u << sh) - 1u)) : hi;
      // Exact counts: keys above H, keys in [L, H] (packed, each <= 32768),
      // scanned so that every thread also gets its gather slot.
      uint32_t g = 0, w = 0;
#pragma unroll
      for (int j = 0; j < kRegVec; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t kv = key[j][e];
          g += kv > H ? 1u : 0u;
          w += kv - L <= H - L ? 1u : 0u;
        }
      const uint32_t mine = g | (w << 16);
      uint32_t tot;
      const uint32_t incl = block_inclusive_scan(mine, scratch, tot);
      const uint32_t c_above = uniform_u32(tot & 0xffffu), c_in = uniform_u32(tot >> 16);
      if (c_above < need && need <= c_above + c_in && c_in <= (uint32_t)kCandLds) {
        need -= c_above;
        cand = c_in;
        lo = L;
        hi = H;
        if (lo < hi) {
          gather(L, H, (incl - mine) >> 16);
          in_lds = true;
        }
      }
    }
    if (!in_lds) {
      while (cand > (uint32_t)kCandLds && lo < hi)
        round(std::integral_constant<int, kRegVec * 4>{}, [&](int m) { return key[m >> 2][m & 3]; }, lo, hi, need,
              cand);
      if (lo < hi) {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < kRegVec; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) w += key[j][e] - lo <= hi - lo ? 1u : 0u;
        uint32_t tot;
        const uint32_t incl = block_inclusive_scan(w, scratch, tot);
        gather(lo, hi, incl - w);
        in_lds = true;
      }
    }
    __syncthreads();  // candidates are in LDS
    if (lo < hi && cand > (uint32_t)kCandCap) {
      // Further rounds over the LDS candidates (kCandPer per thread).
      uint32_t ck[kCandPer], cp[kCandPer];
#pragma unroll
      for (int m = 0; m < kCandPer; ++m) {
        const uint32_t c = (uint32_t)(tid + kRegThreads * m);
        ck[m] = c < cand ? ckey[c] : 0u;
        cp[m] = c < cand ? cpos[c] : 0u;
      }
      while (cand > (uint32_t)kCandCap && lo < hi)
        round(std::integral_constant<int, kCandPer>{}, [&](int m) { return ck[m]; }, lo, hi, need, cand);
      if (lo < hi) {
        // At most kCandCap candidates left: gather them into the front of
        // the LDS arrays for the ranking wave.
        if (tid == 0) res[2] = 0;
        __syncthreads();  // every thread has its candidates out of LDS
#pragma unroll
        for (int m = 0; m < kCandPer; ++m)
          if ((ck[m] != 0u) & (ck[m] - lo <= hi - lo)) {
            const uint32_t slot = atomicAdd(&res[2], 1u);
            ckey[slot] = ck[m];
            cpos[slot] = cp[m];
          }
        __syncthreads();
      }
    }
    if (lo == hi) {
      Kt = lo;  // every candidate is a copy of K*
      need_eq = need;
      eq_total = cand;
    } else {
      // Rank the <= kCandCap candidates (score descending, then position
      // ascending); the one of rank need-1 is the k-th overall.
      if (wave == 0) {
        const bool act = (uint32_t)lane < cand;
        const uint32_t kc = act ? ckey[lane] : 0u, pc = act ? cpos[lane] : 0u;
        uint32_t rank = 0, gtc = 0, eqc = 0;
        for (uint32_t o = 0; o < cand; ++o) {
          const uint32_t ko = (uint32_t)__builtin_amdgcn_readlane((int)kc, (int)o);
          const uint32_t po = (uint32_t)__builtin_amdgcn_readlane((int)pc, (int)o);
          const uint32_t gt = (uint32_t)(ko > kc), eq = (uint32_t)(ko == kc);
          gtc += gt;
          eqc += eq;
          rank += gt | (eq & (uint32_t)(po < pc));
        }
        if (act && rank == need - 1) {
          res[3] = kc;
          res[4] = need - gtc;
          res[5] = eqc;  // copies of K* among the candidates (all of them)
        }
      }
      __syncthreads();
      Kt = uniform_u32(res[3]);
      need_eq = uniform_u32(res[4]);
      eq_total = uniform_u32(res[5]);
    }
  }

  // ---- 2. ordered compaction -----------------------------------------------
  // Usually every copy of K* is taken: the rule is key >= K* and two groups'
  // counts share one scan (16-bit fields; a wave holds at most 256 per
  // group).  Otherwise each group scans packed counts: keys > K* in the low
  // 16 bits, copies of K* in the high 16 bits (each at most 32768).
  const bool split_ties = need_eq < eq_total;
  const uint32_t kt_lo = split_ties ? Kt + 1u : Kt;  // taken outright: key >= kt_lo
  refresh_keys();
  auto count4 = [&](int j) __attribute__((always_inline)) {
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) c += key[j][e] >= kt_lo ? 1u : 0u;
    return c;
  };
  auto count4_split = [&](int j) __attribute__((always_inline)) {
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) c += (key[j][e] >= kt_lo ? 1u : 0u) + (key[j][e] == Kt ? 0x10000u : 0u);
    return c;
  };
  if (!split_ties) {
#pragma unroll
    for (int jj = 0; jj < kRegVec; jj += 2) {
      const uint32_t incl = wave_incl_scan(count4(jj) | (count4(jj + 1) << 16));
      if (lane == 63) {
        wtot[jj * kRegWaves + wave] = incl & 0xffffu;
        wtot[(jj + 1) * kRegWaves + wave] = incl >> 16;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kRegVec; ++j) {
      const uint32_t incl = wave_incl_scan(count4_split(j));
      if (lane == 63) wtot[j * kRegWaves + wave] = incl;
    }
  }
  __syncthreads();
  constexpr int kTot = kRegVec * kRegWaves;  // (group, wave) totals, lane l holds 2l and 2l + 1
  static_assert(kTot <= 2 * kWave, "one wave scans the (group, wave) totals");
  if (wave == 0) {
    const bool has_a = 2 * lane < kTot, has_z = 2 * lane + 1 < kTot;
    const uint32_t a = has_a ? wtot[2 * lane] : 0u, z = has_z ? wtot[2 * lane + 1] : 0u;
    const uint32_t ex = wave_incl_scan(a + z) - a - z;
    if (has_a) wtot[2 * lane] = ex;
    if (has_z) wtot[2 * lane + 1] = ex + a;
  }
  __syncthreads();
  // Selected positions are staged in LDS (reusing the histogram), then
  // written out with coalesced stores.  Every key stores: unselected ones
  // into a per-lane sink, so the loop has no branches.
  int32_t* sel = reinterpret_cast<int32_t*>(hist);
  int32_t* my_sink = sink + lane;
  refresh_keys();
  uint32_t pb = 4u * (uint32_t)tid;
  asm volatile("" : "+v"(pb));
  if (!split_ties) {
#pragma unroll
    for (int jj = 0; jj < kRegVec; jj += 2) {
      const uint32_t c = count4(jj) | (count4(jj + 1) << 16);
      const uint32_t ex = wave_incl_scan(c) - c;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = jj + h;
        uint32_t r = wtot[j * kRegWaves + wave] + (h ? ex >> 16 : ex & 0xffffu);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool t = key[j][e] >= kt_lo;
          *(t ? sel + r : my_sink) = (int32_t)(pb + (uint32_t)(4 * kRegThreads * j + e));
          r += t ? 1u : 0u;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kRegVec; ++j) {
      const uint32_t c = count4_split(j);
      uint32_t r = wtot[j * kRegWaves + wave] + wave_incl_scan(c) - c;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kv = key[j][e];
        const uint32_t gb = r & 0xffffu, eb = r >> 16;
        const bool g = kv >= kt_lo, q = kv == Kt;
        const bool t = g || (q && eb < need_eq);
        const uint32_t slot = gb + min(eb, need_eq);
        *(t ? sel + slot : my_sink) = (int32_t)(pb + (uint32_t)(4 * kRegThreads * j + e));
        r += g ? 1u : (q ? 0x10000u : 0u);
      }
    }
  }
  __syncthreads();
  // Slots past the selected count (only rows with fewer than k selectable
  // keys) are padded with -1.
  const uint32_t taken = nsel > (uint32_t)k ? (uint32_t)k : nsel;
  for (uint32_t j = tid; j < (uint32_t)k; j += kRegThreads) out[j] = j < taken ? sel[j] : -1;
  };
  if constexpr (kFilter) {
    // A bounded grid walks the rows and runs the flagged ones, so a launch
    // with no row flagged (the usual case) costs a few hundred workgroups
    // rather than one per row.
    if (*p.any_flag == 0u) return;
    const int64_t total = p.B * ni;
    for (int64_t lid = blockIdx.x; lid < total; lid += gridDim.x) {
      if (p.row_flag[(lid / ni) * p.T + i0 + lid % ni] != 0u) {
        run_row(lid);
        __syncthreads();  // LDS is reused by the next row
      }
    }
  } else {
    run_row((int64_t)blockIdx.x);
  }
}

// ---------------------------------------------------------------------------
// Long rows: multi-workgroup pipeline over chunks of kMwChunk positions.
// Three digit passes (11 + 11 + 10 bits): every chunk histograms the digit of
// its keys that match the prefix chosen so far and adds its histogram to one
// of the row's sub-histograms; one workgroup per row then picks the bin where
// the count from the top reaches `need` and extends the prefix.  After the
// third pass the prefix is the k-th key K; each chunk then counts its keys
// > K and == K, and an ordered write places every kept position at its slot.
// Workspace (uint32): hist[rows][kMwSub][kBins] | state[rows][4] | cnt[rows][nchunk][2]
// state: 0 = prefix, 1 = need, 2 = above_total, 3 = unused
// ---------------------------------------------------------------------------
constexpr int kMwPer = kMwChunk / kMwThreads;  // positions per thread
constexpr int kMwSub = 8;                       // sub-histograms per row

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
  m.state = m.hist + rows * kMwSub * kBins;
  m.cnt = m.state + rows * 4;
  m.nchunk = (p.S + kMwChunk - 1) / kMwChunk;
  return m;
}

// Keys of this thread's positions of a chunk: wave w, lane l holds positions
// s_beg + 1024*w + 64*i + l (i < kMwPer), so that a wave's positions are
// contiguous and in order.  Every load is issued (positions past s_fin read
// the chunk's first position); valid(i) says whether position i exists.
struct MwKeys {
  uint32_t key[kMwPer];
};
__device__ __forceinline__ MwKeys mw_load(const float* sc, int64_t s_beg, int64_t s_fin) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t base = s_beg + (int64_t)wave * (kWave * kMwPer) + lane;
  float f[kMwPer];
#pragma unroll
  for (int i = 0; i < kMwPer; ++i) {
    const int64_t s = base + kWave * i;
    f[i] = sc[s < s_fin ? s : s_beg];
  }
  MwKeys k;
#pragma unroll
  for (int i = 0; i < kMwPer; ++i) k.key[i] = score_key(f[i]);
  return k;
}
__device__ __forceinline__ bool mw_valid(int64_t s_beg, int64_t s_fin, int i) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return s_beg + (int64_t)wave * (kWave * kMwPer) + kWave * i + lane < s_fin;
}

__global__ __launch_bounds__(kMwThreads) void topk_mw_init(DsaTopkParams p) {
  const MwLayout m = mw_layout(p);
  const int64_t row = blockIdx.x;
  for (int j = threadIdx.x; j < kMwSub * kBins; j += kMwThreads) m.hist[row * kMwSub * kBins + j] = 0;
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
  const MwKeys k = mw_load(p.scores + row * p.S, s_beg, s_fin);
  for (int j = threadIdx.x; j < kBins; j += kMwThreads) lh[j] = 0;
  __syncthreads();
  const uint32_t prefix = m.state[row * 4 + 0];
  const int sh = digit_shift(pass);
  const uint32_t dm = digit_mask(pass);
  const int sh_prev = pass > 0 ? digit_shift(pass - 1) : 32;
#pragma unroll
  for (int e = 0; e < kMwPer; ++e) {
    const uint32_t key = k.key[e];
    const bool match = pass == 0 || (key >> sh_prev) == prefix;
    if (mw_valid(s_beg, s_fin, e) && match) atomicAdd(&lh[(key >> sh) & dm], 1u);
  }
  __syncthreads();
  // Chunks add their histograms into sub-histogram chunk % kMwSub, which
  // spreads the atomics on the few busy bins over kMwSub addresses.
  uint32_t* gh = m.hist + (row * kMwSub + chunk % kMwSub) * kBins;
  for (int j = threadIdx.x; j <= (int)dm; j += kMwThreads) {
    const uint32_t c = lh[j];
    if (c) atomicAdd(&gh[j], c);
  }
}

// One workgroup per row: sum the sub-histograms (and clear them for the next
// pass), pick the bin where the count from the top reaches `need`.
__global__ __launch_bounds__(kMwThreads) void topk_mw_select(DsaTopkParams p, int pass) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t res[2];
  const MwLayout m = mw_layout(p);
  const int64_t row = blockIdx.x;
  const int64_t b = row / p.T, i = row % p.T;
  const int64_t n = row_len(p, b, i);
  if (n <= p.k) return;
  const int nb = (int)digit_mask(pass) + 1;
  for (int j = threadIdx.x; j < kBins; j += kMwThreads) {
    uint32_t c = 0;
#pragma unroll
    for (int u = 0; u < kMwSub; ++u) {
      uint32_t* gh = m.hist + (row * kMwSub + u) * kBins + j;
      c += *gh;
      *gh = 0;  // ready for the next pass
    }
    h[j] = j < nb ? c : 0u;
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

// Per chunk: keys > K and keys == K.
__global__ __launch_bounds__(kMwThreads) void topk_mw_count(DsaTopkParams p) {
  __shared__ uint32_t part[2][kMwThreads / kWave];
  const MwLayout m = mw_layout(p);
  const int64_t row = blockIdx.x / m.nchunk, chunk = blockIdx.x % m.nchunk;
  const int64_t b = row / p.T, i = row % p.T;
  const int64_t n = row_len(p, b, i);
  if (n <= p.k) return;
  const int64_t s_beg = chunk * kMwChunk, s_fin = imin64(n, s_beg + kMwChunk);
  uint32_t gt = 0, eq = 0;
  if (s_beg < s_fin) {
    const uint32_t K = m.state[row * 4 + 0];
    const MwKeys k = mw_load(p.scores + row * p.S, s_beg, s_fin);
#pragma unroll
    for (int e = 0; e < kMwPer; ++e) {
      const bool v = mw_valid(s_beg, s_fin, e);
      gt += (v && k.key[e] > K) ? 1u : 0u;
      eq += (v && k.key[e] == K) ? 1u : 0u;
    }
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

// Ordered write: position s is kept iff key > K, or key == K and fewer than
// `need` copies of K precede it; its slot is #(key > K before s) +
// #(key == K before s).
__global__ __launch_bounds__(kMwThreads) void topk_mw_write(DsaTopkParams p) {
  __shared__ uint32_t wcnt[2][kMwThreads / kWave];
  __shared__ uint32_t before[2][kMwThreads / kWave];
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
  const MwKeys k = mw_load(p.scores + row * p.S, s_beg, s_fin);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Counts of the earlier chunks, summed by all threads.
  uint32_t gb = 0, eb = 0;
  for (int64_t c = threadIdx.x; c < chunk; c += kMwThreads) {
    gb += m.cnt[(row * m.nchunk + c) * 2 + 0];
    eb += m.cnt[(row * m.nchunk + c) * 2 + 1];
  }
  uint32_t g = 0, e = 0;
#pragma unroll
  for (int j = 0; j < kMwPer; ++j) {
    const bool v = mw_valid(s_beg, s_fin, j);
    g += (v && k.key[j] > K) ? 1u : 0u;
    e += (v && k.key[j] == K) ? 1u : 0u;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    gb += __shfl_xor(gb, off);
    eb += __shfl_xor(eb, off);
    g += __shfl_xor(g, off);
    e += __shfl_xor(e, off);
  }
  if (lane == 0) {
    before[0][wave] = gb;
    before[1][wave] = eb;
    wcnt[0][wave] = g;
    wcnt[1][wave] = e;
  }
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
  for (int w = 0; w < kMwThreads / kWave; ++w) {
    gt_before += before[0][w];
    eq_before += before[1][w];
    if (w < wave) {
      gt_before += wcnt[0][w];
      eq_before += wcnt[1][w];
    }
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t base = s_beg + (int64_t)wave * (kWave * kMwPer) + lane;
#pragma unroll
  for (int j = 0; j < kMwPer; ++j) {
    const bool v = mw_valid(s_beg, s_fin, j);
    const uint32_t key = k.key[j];
    const uint64_t mgt = __ballot(v && key > K);
    const uint64_t meq = __ballot(v && key == K);
    const uint32_t g_b = gt_before + __popcll(mgt & below);
    const uint32_t e_b = eq_before + __popcll(meq & below);
    const uint32_t slot = g_b + (e_b < need ? e_b : need);
    if (v && (key > K || (key == K && e_b < need)) && slot < (uint32_t)p.k) out[slot] = (int32_t)(base + kWave * j);
    gt_before += __popcll(mgt);
    eq_before += __popcll(meq);
  }
}

size_t dsa_topk_ws_bytes(int64_t B, int64_t T, int64_t S, int64_t k) {
  (void)k;
  if (S <= kRegRow) return 0;
  const int64_t rows = B * T;
  const int64_t nchunk = (S + kMwChunk - 1) / kMwChunk;
  return (size_t)(rows * kMwSub * kBins + rows * 4 + rows * nchunk * 2) * sizeof(uint32_t);
}

hipError_t launch_dsa_topk(const DsaTopkParams& p, hipStream_t stream) {
  const int64_t rows = p.B * p.T;
  if (p.S <= kRegRow) {
    if (p.row_flag) {  // the flagged rows only, any length: one bounded launch
      const uint32_t grid = (uint32_t)std::min<int64_t>(rows, kFilterGrid);
      hipLaunchKernelGGL((dsa_topk_reg_kernel<512, true>), dim3(grid), dim3(512), 0, stream, p, (int64_t)0, p.T);
      return hipGetLastError();
    }
    if (p.q_pos) {  // row lengths are on the device: one size fits all
      hipLaunchKernelGGL((dsa_topk_reg_kernel<512, false>), dim3((uint32_t)rows), dim3(512), 0, stream, p, (int64_t)0, p.T);
      return hipGetLastError();
    }
    // Causal rows from position 0: row i holds min((i + 1) / ratio, S)
    // candidates, so the rows that fit a smaller workgroup (cap = kThreads * 64
    // candidates, i.e. i < (cap + 1) * ratio - 1) form contiguous ranges, one
    // launch each.
    auto run = [&](auto threads_tag, int64_t& i0) {
      constexpr int kThreads = decltype(threads_tag)::value;
      const int64_t cap = (int64_t)kThreads * kRegVec * 4;
      const int64_t i1 = kThreads == 512 ? p.T : std::min<int64_t>(p.T, (cap + 1) * p.ratio - 1);
      if (i1 > i0) {
        const dim3 grid((uint32_t)(p.B * (i1 - i0)));
        hipLaunchKernelGGL((dsa_topk_reg_kernel<kThreads, false>), grid, dim3(kThreads), 0, stream, p, i0, i1 - i0);
        i0 = i1;
      }
    };
    int64_t i0 = 0;
    run(std::integral_constant<int, 128>{}, i0);
    run(std::integral_constant<int, 256>{}, i0);
    run(std::integral_constant<int, 512>{}, i0);
    return hipGetLastError();
  }
  const int64_t nchunk = (p.S + kMwChunk - 1) / kMwChunk;
  hipLaunchKernelGGL(topk_mw_init, dim3((uint32_t)rows), dim3(kMwThreads), 0, stream, p);
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(topk_mw_hist, dim3((uint32_t)(rows * nchunk)), dim3(kMwThreads), 0, stream, p, pass);
    hipLaunchKernelGGL(topk_mw_select, dim3((uint32_t)rows), dim3(kMwThreads), 0, stream, p, pass);
  }
  hipLaunchKernelGGL(topk_mw_count, dim3((uint32_t)(rows * nchunk)), dim3(kMwThreads), 0, stream, p);
  hipLaunchKernelGGL(topk_mw_write, dim3((uint32_t)(rows * nchunk)), dim3(kMwThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa

// Backward of the DSA sparse attention over the selected positions (gfx950).
//
// Method: [P1] §二.1, [P3] §架構創新 1 -- core attention runs only on the
// top-K positions; the pages train these layers but print no backward
// formula, so the gradients are the chain rule of the forward's definition
// (one KV head shared by the 64 query heads, 256 wide).  The selection is
// discrete and gets no gradient.  Per token, with P the forward's softmax
// weights over the token's entries (from the saved log-sum-exp) and D_h =
// sum_d dO[h,d] * O[h,d]:
//   dP = dO . v_s,   dS = P * (dP - D_h)
//   dq_h += scale * dS * k_s,  dk[s] += scale * sum_h dS * q_h,
//   dv[s] += sum_h P * dO_h.
//
// Tokens are taken in chunks; per chunk, every contraction on 32x32x16 bf16
// MFMA and no floating-point atomics:
//  1. dsa_bwd_ds_kernel, one workgroup (2 waves x 32 heads) per token, the
//     forward's tiling: entry tiles of 32 gathered K/V rows, S^T = K Q^T and
//     dP^T = V dO^T, P and dS, dQ^T += K^T dS^T; each tile's P and dS (bf16)
//     are stored as 32x32 blocks (entries x heads of one wave).
//  2. dsa_bwd_contrib_kernel, one workgroup (4 waves x 64 dims) per token:
//     for each entry tile, dK^T = Q^T dS and dV^T = dO^T P over the 64 heads
//     (Q and dO staged in LDS and read transposed, the blocks as the B
//     operand): one dK row and one dV row per entry (bf16).
//  3. The inverse index of the chunk's entries (integer counts, a scan, a
//     fill in arbitrary order), then dsa_bwd_reduce_kernel: one workgroup per
//     key row sorts its segment's entry ids in LDS and adds the entries' rows
//     in ascending (token, entry) order into dk and dv.  Chunks run in order,
//     so every output element is summed in a fixed order and the result is
//     bit-identical from run to run.
// The inverse index depends only on the selection, so it is built on a
// second stream into one of two buffers, ahead of the chunks' MFMA passes;
// events order each chunk's reduce after its index and each buffer's reuse
// after the reduce that read it.
#include <type_traits>
#include <vector>

#include "attn_core32.h"
#include "kernels.h"
#include "select_util.h"

namespace sa {

namespace {
constexpr int kBwH = 64;         // query heads
constexpr int kBwD = 256;        // head width
constexpr int kBwMaxK = 2048;
constexpr int kBlkE = 32 * 32;   // one stored block (P or dS of 32 entries x 32 heads)
constexpr int kSortCap = 4096;   // segment length sorted in LDS; longer ones take the ordered scan
constexpr int64_t kChunkTokens = 2048;

// Column of head x (0..31) within a stored block: bits 2 and 3 swapped, so
// that the 8 heads a lane needs for one k-step of the contribution product
// (16st + 4q + {0..3, 8..11}, the k-slot order of the transposing LDS read)
// are 16 contiguous bytes of the entry's row.
__device__ __forceinline__ int bw_col(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

__host__ __device__ __forceinline__ int64_t bw_ntile(int64_t kk) { return (kk + 31) / 32; }
}  // namespace

__global__ __launch_bounds__(256) void dsa_sparse_bwd_zero_kernel(float4* p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---------------------------------------------------------------------------
// Pass 1: dq and the P / dS blocks.  One workgroup per token: wave w holds Q,
// dO (B operands, 256 dims) and dQ^T of heads 32w .. 32w + 31.  K tiles are
// double buffered, V single (the next one is sent once dP has read it).  Every
// tile issues the same loads and stores on every wave, so the waits count
// exactly (the prologue's stores go to a discard block).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1))) void dsa_bwd_ds_kernel(DsaSparseBwdParams p) {
  using T = bf16_t;
  using G = AttnGeom<T, kBwD, 1>;
  constexpr int kWaves = 2;
  // Two K buffers as separate arrays, and a tile loop unrolled by two so that
  // every load and read names its buffer at compile time (with a computed
  // index the compiler would wait for every load before any LDS read).
  __shared__ __attribute__((aligned(16))) char kl0[G::kTileBytes];
  __shared__ __attribute__((aligned(16))) char kl1[G::kTileBytes];
  __shared__ __attribute__((aligned(16))) char vl[G::kTileBytes];
  __shared__ int32_t sidx[kBwMaxK];

  const int64_t tl = blockIdx.x;  // token within the chunk
  const int64_t tok = p.tok0 + tl;
  const int64_t b = tok / p.T;
  const int wave = wave_id(), lane = threadIdx.x & 63, qh = lane >> 5;
  const int h = wave * 32 + (lane & 31);
  const int kk = (int)p.kk;
  const int ntile = (int)bw_ntile(p.kk);
  const int64_t S = p.S;
  const T* kb = reinterpret_cast<const T*>(p.k) + b * S * kBwD;
  const T* vb = reinterpret_cast<const T*>(p.v) + b * S * kBwD;

  for (int n = threadIdx.x; n < 32 * ntile; n += 128) {
    const int32_t s = n < kk ? p.idx[tok * kk + n] : -1;
    sidx[n] = (s >= 0 && s < S) ? s : -1;
  }
  // Q, dO of head h as B operands (k-step n: dims 16n + 8q .. +7), D_h.
  i16x8_t qb[16], db[16];
  float dpart = 0.f;
  {
    const int64_t row = (tok * kBwH + h) * kBwD + 8 * qh;
    const T* qr = reinterpret_cast<const T*>(p.q) + row;
    const T* dr = reinterpret_cast<const T*>(p.dout) + row;
    const T* orr = reinterpret_cast<const T*>(p.o) + row;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      qb[n] = __builtin_bit_cast(i16x8_t, *reinterpret_cast<const uint4*>(qr + 16 * n));
      const uint4 du = *reinterpret_cast<const uint4*>(dr + 16 * n);
      db[n] = __builtin_bit_cast(i16x8_t, du);
      const uint4 ou = *reinterpret_cast<const uint4*>(orr + 16 * n);
      const uint32_t a[4] = {du.x, du.y, du.z, du.w}, c[4] = {ou.x, ou.y, ou.z, ou.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dpart = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a[e]), __builtin_bit_cast(bf16x2_t, c[e]),
                                                dpart, false);
    }
  }
  const float Dh = sum_xor32(dpart);
  const float lse2 = p.lse[tok * kBwH + h] * kLog2e;
  const Tile32Addr ad = tile32_addr<kBwD>();

  auto rows_of = [&](int t) {
    const int32_t* trow = sidx + 32 * t;
    return [=](int r) -> int { return trow[r]; };
  };
  auto issue_k = [&](int t, char* buf) { stage_rows_async<T, kBwD, kWaves, 1>(buf, kb, rows_of(t)); };
  auto issue_v = [&](int t) { stage_rows_async<T, kBwD, kWaves, 1>(vl, vb, rows_of(t)); };
  constexpr int kLd = StageGeom<T, kBwD, kWaves>::kPerWave;  // loads per wave of a K (or V) tile
  constexpr int kSt = 32;                                    // block stores per wave and tile

  uint16_t* const blk_tok = p.blocks + tl * ntile * 4 * kBlkE;
  uint16_t* const discard = p.blocks + p.ntok * ntile * 4 * kBlkE;
  const int col = bw_col(lane & 31);
  auto store_block = [&](uint16_t* base, const f32x16_t& x) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = 8 * (j >> 2) + 4 * qh + (j & 3);
      base[e * 32 + col] = (uint16_t)(pack_bf16x2(x[j], 0.f) & 0xffffu);
    }
  };
  f32x16_t dqa[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) dqa[nb][j] = 0.f;
  f32x16_t zero16;
#pragma unroll
  for (int j = 0; j < 16; ++j) zero16[j] = 0.f;

  wait_vmcnt<0>();  // Q, dO, O, lse and the index list are in
  __syncthreads();  // sidx
  issue_k(0, kl0);
  issue_v(0);
  // Two blocks' worth of stores to distinct addresses (identical stores to one
  // address could be merged, and the waits would then miscount).
  store_block(discard, zero16);
  store_block(discard + 2 * kBlkE, zero16);

  auto step = [&](int t, auto more_tag, auto buf_tag) __attribute__((always_inline)) {
    constexpr bool more = decltype(more_tag)::value;
    constexpr int buf = decltype(buf_tag)::value;  // t & 1
    const char* kt = buf == 0 ? kl0 : kl1;
    if constexpr (more) {
      issue_k(t + 1, buf == 0 ? kl1 : kl0);
      wait_vmcnt<kLd + kSt + kLd>();  // K(t) landed: V(t), stores(t - 1), K(t + 1) may be in flight
    } else {
      wait_vmcnt<kLd + kSt>();
    }
    lds_barrier();
    f32x16_t s = qk32_ops<kBwD, 4>(qb, kt, ad);
    if constexpr (more) {
      wait_vmcnt<kSt + kLd>();  // V(t) landed
    } else {
      wait_vmcnt<kSt>();
    }
    lds_barrier();
    f32x16_t dp = qk32_ops<kBwD, 4>(db, vl, ad);
    const uint32_t mask = (uint32_t)(__ballot(sidx[32 * t + (lane & 31)] >= 0) & 0xffffffffull);
    wait_lgkmcnt0();
    lds_barrier();  // both waves are done reading V(t)
    if constexpr (more) issue_v(t + 1);
    const uint32_t kbits = mask >> (4 * qh);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float pr = (kbits & (1u << (8 * (j >> 2) + (j & 3)))) ? fast_exp2(s[j] * p.scale_log2 - lse2) : 0.f;
      s[j] = pr;
      dp[j] = pr * (dp[j] - Dh);
    }
    i16x8_t pf[2];
    pack_p32(dp, pf);
    pv32_acc<8, 2>(dqa, pf, kt, ad, 0);
    wait_lgkmcnt0();
    uint16_t* bt = blk_tok + (int64_t)t * 4 * kBlkE + wave * kBlkE;
    store_block(bt, s);              // P:  tensor 0
    store_block(bt + 2 * kBlkE, dp); // dS: tensor 1
    lds_barrier();  // both waves are done with K(t)
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int t = 0;
  for (; t + 2 < ntile; t += 2) {
    step(t, std::true_type{}, B0{});
    step(t + 1, std::true_type{}, B1{});
  }
  if (t + 1 < ntile) {
    step(t, std::true_type{}, B0{});
    step(t + 1, std::false_type{}, B1{});
  } else {
    step(t, std::false_type{}, B0{});
  }

  float* dqr = p.dq + (tok * kBwH + h) * kBwD;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *reinterpret_cast<float4*>(dqr + 32 * nb + 8 * m + 4 * qh) =
          make_float4(dqa[nb][4 * m] * p.scale, dqa[nb][4 * m + 1] * p.scale, dqa[nb][4 * m + 2] * p.scale,
                      dqa[nb][4 * m + 3] * p.scale);
}

// ---------------------------------------------------------------------------
// Pass 2: each entry's dK and dV rows.  One workgroup of 4 waves per token:
// Q and dO (64 heads x 256 dims, as two 32-head tiles each) are staged once;
// the blocks of each entry tile are staged double buffered; wave w computes
// dims [64w, 64w + 64) of dK^T = Q^T dS and dV^T = dO^T P (contraction over
// the 64 heads: two tiles x two k-steps) and stores them as bf16 rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void dsa_bwd_contrib_kernel(DsaSparseBwdParams p) {
  using T = bf16_t;
  using G = AttnGeom<T, kBwD, 1>;
  constexpr int kWaves = 4;
  constexpr int kTile = G::kTileBytes;  // 16 KB
  __shared__ __attribute__((aligned(16))) char qs[2][kTile];
  __shared__ __attribute__((aligned(16))) char dos[2][kTile];
  __shared__ __attribute__((aligned(16))) char bl[2][4 * 2 * kBlkE];  // 4 blocks of 2 KB per stage

  const int64_t tl = blockIdx.x;
  const int64_t tok = p.tok0 + tl;
  const int wave = wave_id(), lane = threadIdx.x & 63, qh = lane >> 5;
  const int kk = (int)p.kk;
  const int ntile = (int)bw_ntile(p.kk);
  const T* qt = reinterpret_cast<const T*>(p.q) + tok * kBwH * kBwD;
  const T* dt = reinterpret_cast<const T*>(p.dout) + tok * kBwH * kBwD;
  auto ident = [](int r) -> int { return r; };
#pragma unroll
  for (int hw = 0; hw < 2; ++hw) {
    stage_rows_async<T, kBwD, kWaves, 1>(qs[hw], qt + hw * 32 * kBwD, ident);
    stage_rows_async<T, kBwD, kWaves, 1>(dos[hw], dt + hw * 32 * kBwD, ident);
  }
  // Blocks of tile t: four 2 KB blocks (tensor e, head half hw) at (2e + hw) * 2 KB;
  // 16-byte chunk c of block row r at chunk c ^ ((r >> 2) & 3).  Wave w loads
  // the 1 KB halves 2w and 2w + 1.
  const buffer_rsrc_t brs = make_buffer_rsrc(p.blocks + tl * ntile * 4 * kBlkE);
  auto stage_blocks = [&](int st, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = 2 * wave + i, blk4 = u >> 1, hb = u & 1;
      const int r = 16 * hb + (lane >> 2), c = (lane & 3) ^ ((r >> 2) & 3);
      const uint32_t off = (uint32_t)(((int64_t)t * 4 + blk4) * kBlkE * 2) + (uint32_t)(r * 64 + c * 16);
      buffer_load_lds_16(brs, off, bl[st] + blk4 * 2 * kBlkE + hb * 1024);
    }
  };
  const Tile32Addr ad = tile32_addr<kBwD>();
  const int br = lane & 31;
  uint32_t boff[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) boff[st] = (uint32_t)(br * 64 + 16 * ((2 * st + qh) ^ ((br >> 2) & 3)));
  const int nb0 = 2 * wave;
  uint16_t* const discard_k = p.gk + p.ntok * p.kk * kBwD;
  uint16_t* const discard_v = p.gv + p.ntok * p.kk * kBwD;
  constexpr int kLd = 2, kSt = 32;

  stage_blocks(0, 0);
  // Discard stores so that every tile sees the same outstanding operations,
  // each to its own address (identical stores to one address could be merged,
  // and the waits would then miscount).
#pragma unroll
  for (int i = 0; i < kSt / 2; ++i) {
    *reinterpret_cast<uint32_t*>(discard_k + 2 * i * kBwD + 2 * lane) = 0u;
    *reinterpret_cast<uint32_t*>(discard_v + 2 * i * kBwD + 2 * lane) = 0u;
  }

  for (int t = 0; t < ntile; ++t) {
    if (t + 1 < ntile) {
      stage_blocks((t + 1) & 1, t + 1);
      wait_vmcnt<kSt + kLd>();
    } else {
      wait_vmcnt<kSt>();
    }
    lds_barrier();
    f32x16_t ak[2], av[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) ak[nb][j] = av[nb][j] = 0.f;
    const char* b0 = bl[t & 1];
#pragma unroll
    for (int hw = 0; hw < 2; ++hw) {
      i16x8_t bp[2], bd[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bp[st] = __builtin_bit_cast(i16x8_t, lds_read_b128(b0 + hw * 2 * kBlkE, boff[st]));
        bd[st] = __builtin_bit_cast(i16x8_t, lds_read_b128(b0 + (2 + hw) * 2 * kBlkE, boff[st]));
      }
      pv32_acc<2, 2, true>(ak, bd, qs[hw], ad, nb0);
      pv32_acc<2, 2, true>(av, bp, dos[hw], ad, nb0);
    }
    wait_lgkmcnt0();
    // Lane l holds dims 64w + l%32 (ak[0]) and 64w + 32 + l%32 (ak[1]) of
    // entries 32t + 8(j/4) + 4q + j%4.  Lanes l, l^1 trade one value per j:
    // the even lane then stores dims (l, l+1) and the odd lane dims
    // (32 + l - 1, 32 + l) of the same entry, so each half-wave writes the 128
    // contiguous bytes (one cache line) of its entry's 64 dims per store.
    const bool odd = lane & 1;
    const int dcol = 64 * wave + (lane & 30) + (odd ? 32 : 0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int jj = 32 * t + 8 * (j >> 2) + 4 * qh + (j & 3);
      const int64_t e = tl * kk + jj;
      const bool live = jj < kk;
      const float k0 = ak[0][j] * p.scale, k1 = ak[1][j] * p.scale;
      const float kx = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(odd ? k0 : k1), 0xb1, 0xf, 0xf, false));
      const float v0 = av[0][j], v1 = av[1][j];
      const float vx = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(odd ? v0 : v1), 0xb1, 0xf, 0xf, false));
      uint16_t* rk = (live ? p.gk + e * kBwD : discard_k) + dcol;
      uint16_t* rv = (live ? p.gv + e * kBwD : discard_v) + dcol;
      // Streamed out (read once, by the reduction): non-temporal stores.
      __builtin_nontemporal_store(odd ? pack_bf16x2(kx, k1) : pack_bf16x2(k0, kx), reinterpret_cast<uint32_t*>(rk));
      __builtin_nontemporal_store(odd ? pack_bf16x2(vx, v1) : pack_bf16x2(v0, vx), reinterpret_cast<uint32_t*>(rv));
    }
    lds_barrier();  // the stage's buffer is free for the load two tiles on
  }
}

// ---------------------------------------------------------------------------
// Inverse index of one chunk of tokens: entry e = (token - tok0) * kk + j.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t bw_key(const DsaSparseBwdParams& p, int64_t e) {
  const int64_t tok = p.tok0 + e / p.kk;
  const int32_t s = p.idx[tok * p.kk + e % p.kk];
  return (s >= 0 && s < p.S) ? (tok / p.T) * p.S + s : -1;
}

__global__ __launch_bounds__(256) void dsa_sparse_bwd_count_kernel(DsaSparseBwdParams p, uint32_t* cnt) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= p.ntok * p.kk) return;
  const int64_t key = bw_key(p, e);
  if (key >= 0) atomicAdd(&cnt[key], 1u);
}

// Exclusive offsets of the counts (one workgroup): off[0..n], cursor = off.
// Each thread takes a run of a multiple of 32 counts, loaded 32 at a time
// (eight 16-byte loads in flight together; cnt, off and cursor are 16-byte
// aligned) and written back the same way.
__global__ __launch_bounds__(1024) void dsa_sparse_bwd_scan_kernel(const uint32_t* cnt, uint32_t* off, uint32_t* cursor,
                                                                   int64_t n) {
  __shared__ uint32_t scratch[32];
  const int64_t per = ((n + 1023) / 1024 + 31) & ~(int64_t)31;
  const int64_t i0 = threadIdx.x * per, i1 = min(n, i0 + per);
  auto load32 = [&](int64_t i, uint32_t (&c)[32]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = i + 4 * u;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (j + 4 <= i1) {
        x = *reinterpret_cast<const uint4*>(cnt + j);
      } else {
        if (j < i1) x.x = cnt[j];
        if (j + 1 < i1) x.y = cnt[j + 1];
        if (j + 2 < i1) x.z = cnt[j + 2];
      }
      c[4 * u] = x.x;
      c[4 * u + 1] = x.y;
      c[4 * u + 2] = x.z;
      c[4 * u + 3] = x.w;
    }
  };
  uint32_t local = 0;
  for (int64_t i = i0; i < i1; i += 32) {
    uint32_t c[32];
    load32(i, c);
#pragma unroll
    for (int u = 0; u < 32; ++u) local += c[u];
  }
  uint32_t tot;
  uint32_t run = block_inclusive_scan(local, scratch, tot) - local;
  for (int64_t i = i0; i < i1; i += 32) {
    uint32_t c[32];
    load32(i, c);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = i + 4 * u;
      uint4 o;
      o.x = run;
      o.y = o.x + c[4 * u];
      o.z = o.y + c[4 * u + 1];
      o.w = o.z + c[4 * u + 2];
      run = o.w + c[4 * u + 3];
      if (j + 4 <= i1) {
        *reinterpret_cast<uint4*>(off + j) = o;
        *reinterpret_cast<uint4*>(cursor + j) = o;
      } else {
        const uint32_t ov[4] = {o.x, o.y, o.z, o.w};
        for (int e = 0; e < 4 && j + e < i1; ++e) {
          off[j + e] = ov[e];
          cursor[j + e] = ov[e];
        }
      }
    }
  }
  if (threadIdx.x == 0) off[n] = tot;
}

// Segment slots in arbitrary order: the reduce step orders each segment.
__global__ __launch_bounds__(256) void dsa_sparse_bwd_fill_kernel(DsaSparseBwdParams p, uint32_t* cursor) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= p.ntok * p.kk) return;
  const int64_t key = bw_key(p, e);
  if (key >= 0) p.list[atomicAdd(&cursor[key], 1u)] = (uint32_t)e;
}

// ---------------------------------------------------------------------------
// dk[key] += the chunk's dK rows of the key's entries, in ascending entry
// order (dv likewise).  One workgroup per key row (grid-stride), one thread
// per dim.  Segments of up to kSortCap entries are sorted in LDS (bitonic);
// a longer segment (an index list with many repeated positions) is ordered
// by scanning the chunk's entries in order instead.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dsa_sparse_bwd_reduce_kernel(DsaSparseBwdParams p, int64_t nkeys) {
  __shared__ uint32_t ids[kSortCap];
  __shared__ uint32_t wtot[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = tid;
  // The rows are read once: non-temporal loads (each wave reads a whole
  // 128-byte line per load).
  auto ld = [](const uint16_t* q) -> float { return bf16_to_f32(__builtin_nontemporal_load(q)); };
  auto row_sum = [&](int m, float& ak, float& av) __attribute__((always_inline)) {
    int r = 0;
    for (; r + 8 <= m; r += 8) {
      float xk[8], xv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t row = (int64_t)ids[r + u] * kBwD + d;
        xk[u] = ld(p.gk + row);
        xv[u] = ld(p.gv + row);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ak += xk[u];
        av += xv[u];
      }
    }
    for (; r < m; ++r) {
      const int64_t row = (int64_t)ids[r] * kBwD + d;
      ak += ld(p.gk + row);
      av += ld(p.gv + row);
    }
  };
  for (int64_t key = blockIdx.x; key < nkeys; key += gridDim.x) {
    const uint32_t e0 = p.off[key], n = p.off[key + 1] - e0;
    if (n == 0) continue;
    float ak = 0.f, av = 0.f;
    if (n <= (uint32_t)kSortCap) {
      uint32_t np2 = 1;
      while (np2 < n) np2 <<= 1;
      for (uint32_t i = tid; i < np2; i += 256) ids[i] = i < n ? p.list[e0 + i] : 0xffffffffu;
      __syncthreads();
      for (uint32_t k2 = 2; k2 <= np2; k2 <<= 1) {
        for (uint32_t j = k2 >> 1; j > 0; j >>= 1) {
          for (uint32_t i = tid; i < np2; i += 256) {
            const uint32_t ixj = i ^ j;
            if (ixj > i) {
              const uint32_t a = ids[i], c = ids[ixj];
              if ((a > c) == ((i & k2) == 0)) {
                ids[i] = c;
                ids[ixj] = a;
              }
            }
          }
          __syncthreads();
        }
      }
      row_sum((int)n, ak, av);
    } else {
      // Ordered scan: the chunk's entries 256 at a time, matches appended in order.
      const int64_t ne = p.ntok * p.kk;
      for (int64_t base = 0; base < ne; base += 256) {
        const int64_t e = base + tid;
        const bool match = e < ne && bw_key(p, e) == key;
        const uint64_t bal = __ballot(match);
        const uint32_t rank = (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wtot[wave] = (uint32_t)__popcll(bal);
        __syncthreads();
        uint32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          before += w < wave ? wtot[w] : 0u;
          total += wtot[w];
        }
        if (match) ids[before + rank] = (uint32_t)e;
        __syncthreads();
        row_sum((int)total, ak, av);
        __syncthreads();
      }
    }
    p.dk[key * kBwD + d] += ak;
    p.dv[key * kBwD + d] += av;
    __syncthreads();  // ids is reused by the next key
  }
}

int64_t dsa_sparse_bwd_chunk(int64_t BT) { return BT < kChunkTokens ? BT : kChunkTokens; }

namespace {
struct BwdLayout {
  size_t blocks, gk, gv, list[2], cnt[2], off[2], cursor[2], total;  // two inverse-index buffers
};
BwdLayout bwd_layout(int64_t B, int64_t T, int64_t S, int64_t kk) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t tc = dsa_sparse_bwd_chunk(B * T), keys = B * S;
  BwdLayout L;
  size_t off = 0;
  L.blocks = off;
  off += al((size_t)(tc * bw_ntile(kk) + 1) * 4 * kBlkE * 2);  // + a discard tile
  L.gk = off;
  off += al((size_t)(tc * kk + 32) * kBwD * 2);  // + 32 discard rows
  L.gv = off;
  off += al((size_t)(tc * kk + 32) * kBwD * 2);
  for (int b = 0; b < 2; ++b) {
    L.list[b] = off;
    off += al((size_t)(tc * kk) * 4);
    L.cnt[b] = off;
    off += al((size_t)(keys + 1) * 4);
    L.off[b] = off;
    off += al((size_t)(keys + 1) * 4);
    L.cursor[b] = off;
    off += al((size_t)(keys + 1) * 4);
  }
  L.total = off;
  return L;
}

// The inverse-index stream of this host thread for `dev` (default priority,
// non-blocking), and a pool of this thread's events.  Both are created on
// first use and kept for the life of the process: one stream per (thread,
// device) is what a caller's threads need, and tearing streams down from a
// thread-exit destructor could run after the runtime has shut down.
constexpr int kMaxDevices = 64;
hipError_t index_stream(int dev, hipStream_t* out) {
  thread_local hipStream_t streams[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!streams[dev]) {
    hipStream_t s = nullptr;
    const hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e != hipSuccess) return e;
    streams[dev] = s;
  }
  *out = streams[dev];
  return hipSuccess;
}
struct EventPool {
  std::vector<hipEvent_t> ev;
};
// n events of device dev (the current device), reused from call to call:
// a wait enqueued before an event is recorded again still waits for the
// record it was enqueued after.
hipError_t thread_events(int dev, size_t n, hipEvent_t** out) {
  thread_local EventPool pools[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  EventPool& pool = pools[dev];
  while (pool.ev.size() < n) {
    hipEvent_t e = nullptr;
    const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (r != hipSuccess) return r;
    pool.ev.push_back(e);
  }
  *out = pool.ev.data();
  return hipSuccess;
}
}  // namespace

size_t dsa_sparse_bwd_ws_bytes(int64_t B, int64_t T, int64_t S, int64_t kk) { return bwd_layout(B, T, S, kk).total; }

hipError_t launch_dsa_sparse_bwd(DsaSparseBwdParams p, hipStream_t stream) {
  const int64_t BT = p.B * p.T, keys = p.B * p.S, tc = dsa_sparse_bwd_chunk(BT);
  const int64_t nch = (BT + tc - 1) / tc;
  const BwdLayout L = bwd_layout(p.B, p.T, p.S, p.kk);
  char* w = reinterpret_cast<char*>(p.ws);
  p.blocks = reinterpret_cast<uint16_t*>(w + L.blocks);
  p.gk = reinterpret_cast<uint16_t*>(w + L.gk);
  p.gv = reinterpret_cast<uint16_t*>(w + L.gv);
  const int64_t n4 = keys * kBwD / 4;
  const uint32_t zb = (uint32_t)std::min<int64_t>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(dsa_sparse_bwd_zero_kernel, dim3(zb), dim3(256), 0, stream, reinterpret_cast<float4*>(p.dk), n4);
  hipLaunchKernelGGL(dsa_sparse_bwd_zero_kernel, dim3(zb), dim3(256), 0, stream, reinterpret_cast<float4*>(p.dv), n4);
  const int64_t c4 = ((keys + 1 + 63) & ~(int64_t)63) / 4;  // the counts, zeroed per chunk as float4 words
  const uint32_t cb = (uint32_t)std::min<int64_t>((c4 + 255) / 256, 4096);
  const uint32_t rb = (uint32_t)std::min<int64_t>(keys, 65536);

  // The index stream and events (ev[0]: start; ev[1 + c]: chunk c's index
  // built; ev[1 + nch + c]: chunk c's reduce done), on the caller stream's
  // device.  Without them (another device current, or a creation failure)
  // everything runs on the caller's stream in the same order.
  hipStream_t aux = nullptr;
  hipEvent_t* ev = nullptr;
  {
    int sdev = -1, cdev = -1;
    if (hipStreamGetDevice(stream, &sdev) == hipSuccess && hipGetDevice(&cdev) == hipSuccess && sdev == cdev &&
        index_stream(cdev, &aux) == hipSuccess && thread_events(cdev, (size_t)(1 + 2 * nch), &ev) == hipSuccess) {
    } else {
      (void)hipGetLastError();  // a failed lookup leaves nothing to report: the single-stream order is used
      aux = nullptr;
    }
  }
  hipError_t e = hipSuccess;
  if (aux) {
    if ((e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(aux, ev[0], 0)) != hipSuccess) return e;
  }
  hipStream_t is = aux ? aux : stream;  // the index kernels' stream
  for (int64_t c = 0; c < nch; ++c) {
    const int b = (int)(c & 1);
    p.tok0 = c * tc;
    p.ntok = std::min<int64_t>(tc, BT - p.tok0);
    p.list = reinterpret_cast<uint32_t*>(w + L.list[b]);
    p.off = reinterpret_cast<const uint32_t*>(w + L.off[b]);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(w + L.cnt[b]);
    uint32_t* off = reinterpret_cast<uint32_t*>(w + L.off[b]);
    uint32_t* cursor = reinterpret_cast<uint32_t*>(w + L.cursor[b]);
    const uint32_t eb = (uint32_t)((p.ntok * p.kk + 255) / 256);
    // Buffer b was last read by chunk c - 2's reduce.
    if (aux && c >= 2 && (e = hipStreamWaitEvent(aux, ev[1 + nch + c - 2], 0)) != hipSuccess) return e;
    hipLaunchKernelGGL(dsa_sparse_bwd_zero_kernel, dim3(cb), dim3(256), 0, is, reinterpret_cast<float4*>(cnt), c4);
    hipLaunchKernelGGL(dsa_sparse_bwd_count_kernel, dim3(eb), dim3(256), 0, is, p, cnt);
    hipLaunchKernelGGL(dsa_sparse_bwd_scan_kernel, dim3(1), dim3(1024), 0, is, cnt, off, cursor, keys);
    hipLaunchKernelGGL(dsa_sparse_bwd_fill_kernel, dim3(eb), dim3(256), 0, is, p, cursor);
    if (aux && (e = hipEventRecord(ev[1 + c], aux)) != hipSuccess) return e;
    hipLaunchKernelGGL(dsa_bwd_ds_kernel, dim3((uint32_t)p.ntok), dim3(128), 0, stream, p);
    hipLaunchKernelGGL(dsa_bwd_contrib_kernel, dim3((uint32_t)p.ntok), dim3(256), 0, stream, p);
    if (aux && (e = hipStreamWaitEvent(stream, ev[1 + c], 0)) != hipSuccess) return e;
    hipLaunchKernelGGL(dsa_sparse_bwd_reduce_kernel, dim3(rb), dim3(256), 0, stream, p, keys);
    if (aux && (e = hipEventRecord(ev[1 + nch + c], stream)) != hipSuccess) return e;
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sa

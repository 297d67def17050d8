// HCA prefill backward (gfx950): dq, dk, dv and the compressed entries' dkc, dvc.
//
// Method: [P1] §二.1 and [P3] §架構創新 1 define the forward (one softmax over
// the visible compressed entries and the recent window); [P3] §預訓練資料工程
// item 3 (FlashMask-4) trains these layers with a backward pass but prints no
// formula, so the gradients are the chain rule of the forward's definition.
// Per query t with keys (entries j < visible(t), window t-W < s <= t), P the
// forward's weights (from its log-sum-exp) and D_t = sum_d dO[t,d] O[t,d]:
//   dP = dO_t . value,  dS = P (dP - D_t)
//   dq_t   = scale sum dS key,   d(key) += scale dS q_t,   d(value) += P dO_t
// and through the block mean every token of a complete block j < Nc gets
// dkc[j] / blk and dvc[j] / blk on top of its window-path gradient.
//
// Three passes, every contraction on 32x32x16 bf16 MFMA, no atomics:
//  1. hca_bwd_dq_kernel, query-centric (the forward's tiling): per 32-query
//     tile the key stream (compressed entry tiles, then 32-aligned raw tiles
//     of the band), S^T and dP^T over the 512 dims split across a wave pair
//     (partials added through LDS), P and dS, dQ^T += K^T dS^T; the tile's P
//     and dS (bf16) are stored as 32x32 blocks for pass 2.
//  2. hca_bwd_kv_kernel, key-centric: per pair of 32-key tiles, the query
//     tiles that saw them; dK^T += Q^T dS and dV^T += dO^T P with Q and dO
//     staged in LDS (read transposed) and the stored blocks as the B operand.
//     Compressed entry tiles run first in chunks of query tiles, each chunk
//     writing its partial sums; hca_bwd_reduce_kernel adds them in chunk
//     order into dkc, dvc.  Raw tiles run last and write dk, dv with the
//     compression path (dkc/blk, dvc/blk) added.
#include <type_traits>

#include "attn_core32.h"
#include "kernels.h"

namespace sa {

namespace {

constexpr int kBwdD = 512;                 // head width (query/key = value)
constexpr int kBwdHD = 256;                // half of it: one wave of a pair
constexpr int kChunkTiles = 128;           // query tiles per workgroup of the compressed pass
constexpr int kBlkElems = 32 * 32;         // one stored block (P or dS)
constexpr int kPairElems = 2 * kBlkElems;  // P then dS

__device__ __forceinline__ int bwd_visible(int t, int blk, int window) {
  const int x = t - window + 1;
  return x > 0 ? x / blk : 0;
}

// Column of local query x (0..31) in a stored block: bits 2 and 3 swapped, so
// that the 8 queries a lane needs for one k-step of the key-centric product
// (16st + 4q + {0..3, 8..11}, the k-slot order of the transposing LDS read)
// are 16 contiguous bytes.
__device__ __forceinline__ int bwd_col(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// First 32-query tile whose stream holds compressed entry tile jt (some query
// of the tile sees entry 32*jt), or ntq if none.
__device__ __forceinline__ int64_t bwd_tq_min(int64_t jt, int64_t blk, int64_t W, int64_t T, int64_t Nc, int64_t ntq) {
  if (32 * jt >= Nc) return ntq;
  const int64_t t_min = (32 * jt + 1) * blk + W - 1;
  return t_min <= T - 1 ? t_min / 32 : ntq;
}

// First raw key tile of query tile tq's stream.
__device__ __forceinline__ int bwd_raw_first(int tq, int W) {
  const int x = 32 * tq - W + 1;
  return x > 0 ? x / 32 : 0;
}

}  // namespace

// ---------------------------------------------------------------------------
// Pass 1: dq, and the P / dS blocks.  One workgroup of 4 waves per 64
// queries: waves 2p, 2p+1 share 32 queries and split the dims (wave 2p + h
// holds Q, dO and dQ^T for dims [256h, 256h + 256)).  K tiles are double
// buffered (the next one streams in during the whole tile), V single (the
// next one is sent once dP has read it).  Every tile of the workgroup's
// stream issues the same loads and stores on every wave (a pair's stores go
// to a discard block when its queries do not use the tile), so the waits
// count exactly.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void hca_bwd_dq_kernel(HcaBwdParams p) {
  using T = bf16_t;
  using GH = AttnGeom<T, kBwdHD, 1>;
  constexpr int kWaves = 4;
  constexpr int kHalfTile = GH::kTileBytes;  // 16 KB: 32 rows x 512 bytes
  // Two K buffers as separate arrays, and a tile loop unrolled by two so that
  // every load and read names its buffer at compile time (with a computed
  // index the compiler would wait for every load before any LDS read).
  __shared__ __attribute__((aligned(16))) char kbuf0[2 * kHalfTile];
  __shared__ __attribute__((aligned(16))) char kbuf1[2 * kHalfTile];
  __shared__ __attribute__((aligned(16))) char vbuf[2 * kHalfTile];
  __shared__ __attribute__((aligned(16))) char xbuf[kWaves * 8192];  // partial S^T, dP^T per wave
  __shared__ float dsh[kWaves][32];

  const int ntq = (int)p.ntq;
  const int nwt = (ntq + 1) / 2;
  const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = (int)(lid / (uint32_t)nwt);
  const int wt = nwt - 1 - (int)(lid % (uint32_t)nwt);  // longest streams first
  const int Tn = (int)p.T, blk = (int)p.blk, W = (int)p.window, Nc = (int)p.Nc;
  const int nct = (int)p.nct, nr = (int)p.nr, nslot = (int)p.nslot;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int pair = wave >> 1, half = wave & 1, qh = lane >> 5;

  const int64_t head = (int64_t)bh * Tn * kBwdD;
  const T* q = reinterpret_cast<const T*>(p.q) + head;
  const T* k = reinterpret_cast<const T*>(p.k) + head;
  const T* v = reinterpret_cast<const T*>(p.v) + head;
  const T* o = reinterpret_cast<const T*>(p.o) + head;
  const T* dO = reinterpret_cast<const T*>(p.dout) + head;
  const T* kc = reinterpret_cast<const T*>(p.kc) + (int64_t)bh * Nc * kBwdD;
  const T* vc = reinterpret_cast<const T*>(p.vc) + (int64_t)bh * Nc * kBwdD;

  const int tqi = 2 * wt + pair;  // this pair's query tile
  const int tp = 32 * tqi;
  const int tq = tp + (lane & 31);
  const bool qvalid = tq < Tn, pvalid = tp < Tn;
  const int trow = min(tq, Tn - 1);

  // Q and dO of this lane's query and half as B operands (k-step n: dims
  // 256*half + 16n + 8q .. +7), and the partial D over the same dims.
  i16x8_t qb[16], db[16];
  float dpart = 0.f;
  {
    const T* qr = q + (int64_t)trow * kBwdD + half * kBwdHD + 8 * qh;
    const T* dr = dO + (int64_t)trow * kBwdD + half * kBwdHD + 8 * qh;
    const T* orr = o + (int64_t)trow * kBwdD + half * kBwdHD + 8 * qh;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      qb[n] = __builtin_bit_cast(i16x8_t, *reinterpret_cast<const uint4*>(qr + 16 * n));
      const uint4 du = *reinterpret_cast<const uint4*>(dr + 16 * n);
      db[n] = __builtin_bit_cast(i16x8_t, du);
      const uint4 ou = *reinterpret_cast<const uint4*>(orr + 16 * n);
      const uint32_t a[4] = {du.x, du.y, du.z, du.w}, b[4] = {ou.x, ou.y, ou.z, ou.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dpart = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a[e]), __builtin_bit_cast(bf16x2_t, b[e]),
                                                dpart, false);
    }
  }
  dpart = sum_xor32(dpart);
  if (lane < 32) dsh[wave][lane] = dpart;
  const float lse2 = p.lse[(int64_t)bh * Tn + trow] * kLog2e;
  const Tile32Addr ad = tile32_addr<kBwdHD>();

  // The workgroup's key stream: compressed entry tiles, then raw tiles.
  const int t0 = 64 * wt;
  const int t_last = min(t0 + 63, Tn - 1);
  const int nc_w = min(Nc, bwd_visible(t_last, blk, W));
  const int n_ct = (nc_w + 31) / 32;
  const int r_lo = bwd_raw_first(2 * wt, W);
  const int n_rt = t_last / 32 - r_lo + 1;
  const int n_tiles = n_ct + n_rt;
  // The pair's own tiles.
  const int tp_last = min(tp + 31, Tn - 1);
  const int n_ct_p = pvalid ? (min(Nc, bwd_visible(tp_last, blk, W)) + 31) / 32 : 0;
  const int r_lo_p = bwd_raw_first(tqi, W);
  // This lane's visibility.
  const int vis_c = qvalid ? min(Nc, bwd_visible(tq, blk, W)) : 0;
  const int win_lo = tq - W + 1;

  auto rows_of = [=](int tile) {
    const bool ct = tile < n_ct;
    const int first = ct ? 32 * tile : 32 * (r_lo + tile - n_ct);
    const int last = ct ? nc_w - 1 : t_last;
    return [=](int r) -> int {
      const int x = first + r;
      return x <= last ? x : -1;
    };
  };
  auto issue_k = [&](int tile, char* dst) __attribute__((always_inline)) {
    const auto rf = rows_of(tile);
    const T* src = tile < n_ct ? kc : k;
    stage_rows_async<T, kBwdHD, kWaves, 1, kBwdD * 2>(dst, src, rf);
    stage_rows_async<T, kBwdHD, kWaves, 1, kBwdD * 2>(dst + kHalfTile, src + kBwdHD, rf);
  };
  auto issue_v = [&](int tile) __attribute__((always_inline)) {
    const auto rf = rows_of(tile);
    const T* src = tile < n_ct ? vc : v;
    stage_rows_async<T, kBwdHD, kWaves, 1, kBwdD * 2>(vbuf, src, rf);
    stage_rows_async<T, kBwdHD, kWaves, 1, kBwdD * 2>(vbuf + kHalfTile, src + kBwdHD, rf);
  };
  constexpr int kLd = 2 * StageGeom<T, kBwdHD, kWaves>::kPerWave;  // loads per wave of a K (or V) tile
  constexpr int kSt = 16;                                          // block stores per wave and tile

  // Stored blocks: this lane writes (key 8m + 4q + i, column bwd_col(l%32)).
  uint16_t* const blk_head = p.blocks + ((int64_t)bh * ntq + tqi) * nslot * kPairElems;
  uint16_t* const discard = p.blocks + p.B * p.H * (int64_t)ntq * nslot * kPairElems;
  const int col = bwd_col(lane & 31);
  auto store_block = [&](uint16_t* base, const f32x16_t& x) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = 8 * (j >> 2) + 4 * qh + (j & 3);
      base[key * 32 + col] = (uint16_t)(pack_bf16x2(x[j], 0.f) & 0xffffu);
    }
  };

  float* xs_mine = reinterpret_cast<float*>(xbuf + wave * 8192 + lane * 16);
  const float* xs_other = reinterpret_cast<const float*>(xbuf + (wave ^ 1) * 8192 + lane * 16);

  f32x16_t dqa[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) dqa[nb][j] = 0.f;

  // Prologue: tile 0's K and V, and one tile's worth of stores to the discard
  // block so that every tile sees the same pattern of outstanding operations.
  wait_vmcnt<0>();  // Q, dO, O and lse are in registers
  __syncthreads();  // dsh
  const float Dq = dsh[2 * pair][lane & 31] + dsh[2 * pair + 1][lane & 31];
  f32x16_t zero16;
#pragma unroll
  for (int j = 0; j < 16; ++j) zero16[j] = 0.f;
  if (n_tiles > 0) {
    issue_k(0, kbuf0);
    issue_v(0);
    store_block(discard + half * kBlkElems, zero16);
  }

  auto step = [&](int tile, auto more_tag, auto buf_tag) __attribute__((always_inline)) {
    constexpr bool more = decltype(more_tag)::value;
    constexpr int buf = decltype(buf_tag)::value;  // tile & 1
    const bool ct = tile < n_ct;
    const int jt = tile, r = r_lo + tile - n_ct;
    const bool need = pvalid && (ct ? jt < n_ct_p : (r >= r_lo_p && r <= tqi));
    const int slot = ct ? jt : nct + (r - tqi + nr - 1);
    const char* kt = (buf == 0 ? kbuf0 : kbuf1) + half * kHalfTile;
    if constexpr (more) {
      issue_k(tile + 1, buf == 0 ? kbuf1 : kbuf0);
      wait_vmcnt<kLd + kSt + kLd>();  // K(tile) landed: V(tile), stores(tile - 1), K(tile + 1) may be in flight
    } else {
      wait_vmcnt<kLd + kSt>();
    }
    lds_barrier();
    f32x16_t s = qk32_ops<kBwdHD, 4>(qb, kt, ad);
    if constexpr (more) {
      wait_vmcnt<kSt + kLd>();  // V(tile) landed
    } else {
      wait_vmcnt<kSt>();
    }
    lds_barrier();
    f32x16_t dp = qk32_ops<kBwdHD, 4>(db, vbuf + half * kHalfTile, ad);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      *reinterpret_cast<f32x4_t*>(xs_mine + c * 256) = f32x4_t{s[4 * c], s[4 * c + 1], s[4 * c + 2], s[4 * c + 3]};
      *reinterpret_cast<f32x4_t*>(xs_mine + 1024 + c * 256) =
          f32x4_t{dp[4 * c], dp[4 * c + 1], dp[4 * c + 2], dp[4 * c + 3]};
    }
    wait_lgkmcnt0();
    lds_barrier();  // partials visible; every wave is done reading V(tile)
    if constexpr (more) issue_v(tile + 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4_t xs = *reinterpret_cast<const f32x4_t*>(xs_other + c * 256);
      const f32x4_t xd = *reinterpret_cast<const f32x4_t*>(xs_other + 1024 + c * 256);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[4 * c + e] += xs[e];
        dp[4 * c + e] += xd[e];
      }
    }
    // P and dS of the tile (zero where the key is not visible to the query).
    const int lo = ct ? 0 : win_lo - 32 * r;
    const int hi = ct ? vis_c - 32 * jt - 1 : (qvalid ? tq - 32 * r : -1);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = 8 * (j >> 2) + 4 * qh + (j & 3);
      const float pr = (key >= lo && key <= hi) ? fast_exp2(s[j] * p.scale_log2 - lse2) : 0.f;
      s[j] = pr;
      dp[j] = pr * (dp[j] - Dq);
    }
    i16x8_t pf[2];
    pack_p32(dp, pf);
    pv32_acc<8, 2>(dqa, pf, kt, ad, 0);
    wait_lgkmcnt0();
    uint16_t* dst = (need ? blk_head + slot * kPairElems : discard) + half * kBlkElems;
    store_block(dst, half == 0 ? s : dp);
    lds_barrier();  // every wave is done with K(tile) and the partials
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  if (n_tiles > 0) {
    int tile = 0;
    for (; tile + 2 < n_tiles; tile += 2) {
      step(tile, std::true_type{}, B0{});
      step(tile + 1, std::true_type{}, B1{});
    }
    if (tile + 1 < n_tiles) {
      step(tile, std::true_type{}, B0{});
      step(tile + 1, std::false_type{}, B1{});
    } else {
      step(tile, std::false_type{}, B0{});
    }
  }
  if (qvalid) {
    float* dqr = p.dq + head + (int64_t)tq * kBwdD + half * kBwdHD;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        *reinterpret_cast<float4*>(dqr + 32 * nb + 8 * m + 4 * qh) =
            make_float4(dqa[nb][4 * m] * p.scale, dqa[nb][4 * m + 1] * p.scale, dqa[nb][4 * m + 2] * p.scale,
                        dqa[nb][4 * m + 3] * p.scale);
  }
}

// ---------------------------------------------------------------------------
// Pass 2: dK, dV of a pair of 32-key tiles (8 waves: wave w takes key tile
// w / 4 and dims [128 (w % 4), +128)).  Per query tile: Q and dO (32 rows x
// 512 dims, as two 256-dim half tiles each) and the four stored blocks (P and
// dS of both key tiles) go to LDS with direct loads, double buffered; then
// dK^T += Q^T dS and dV^T += dO^T P.  kComp: compressed entry tiles over one
// chunk of query tiles (partial sums out); otherwise raw tiles over their
// band (dk, dv out, with dkc/blk and dvc/blk added).
// ---------------------------------------------------------------------------
template <bool kComp>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void hca_bwd_kv_kernel(HcaBwdParams p) {
  using T = bf16_t;
  using GH = AttnGeom<T, kBwdHD, 1>;
  constexpr int kWaves = 8;
  constexpr int kHalfTile = GH::kTileBytes;                  // 16 KB
  constexpr int kStage = 4 * kHalfTile + 4 * 2 * kBlkElems;  // Q, dO, 4 blocks: 72 KB
  __shared__ __attribute__((aligned(16))) char lds[2 * kStage];

  const int ntq = (int)p.ntq, nct = (int)p.nct, nr = (int)p.nr, nslot = (int)p.nslot;
  const int Tn = (int)p.T, Nc = (int)p.Nc;
  const int nkp = kComp ? (nct + 1) / 2 : (ntq + 1) / 2;  // key-tile pairs per head
  const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  int bh, kp, chunk = 0;
  if constexpr (kComp) {
    const int per_bh = (int)p.nchunk * nkp;
    bh = (int)(lid / (uint32_t)per_bh);
    const int rem = (int)(lid % (uint32_t)per_bh);
    chunk = rem / nkp;
    kp = rem % nkp;
  } else {
    bh = (int)(lid / (uint32_t)nkp);
    kp = (int)(lid % (uint32_t)nkp);
  }
  const int wave = wave_id(), lane = threadIdx.x & 63, qh = lane >> 5;
  const int kt = wave >> 2, quarter = wave & 3, hsel = quarter >> 1, nb0 = 4 * (quarter & 1);
  const int n_keyt = kComp ? nct : ntq;
  const int ktile[2] = {2 * kp, 2 * kp + 1};  // entry tiles (kComp) or raw tiles

  // Query tiles [tq_begin, tq_end) of this workgroup, and of each key tile.
  int tq_begin, tq_end, kt_lo[2], kt_hi[2];  // key tile i is used by query tiles [kt_lo, kt_hi]
  if constexpr (kComp) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      kt_lo[i] = ktile[i] < n_keyt ? (int)bwd_tq_min(ktile[i], p.blk, p.window, p.T, p.Nc, ntq) : ntq;
      kt_hi[i] = ntq - 1;
    }
    tq_begin = max(kt_lo[0], chunk * kChunkTiles);
    tq_end = min(ntq, (chunk + 1) * kChunkTiles);
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      kt_lo[i] = ktile[i] < n_keyt ? ktile[i] : ntq;
      kt_hi[i] = min(ntq - 1, ktile[i] + nr - 1);
    }
    tq_begin = kt_lo[0];
    tq_end = min(ntq, max(kt_hi[0], kt_hi[1]) + 1);
  }
  const int n = tq_end - tq_begin;
  if (n <= 0) return;

  const int64_t head = (int64_t)bh * Tn * kBwdD;
  const T* q = reinterpret_cast<const T*>(p.q) + head;
  const T* dO = reinterpret_cast<const T*>(p.dout) + head;
  const uint16_t* blk_head = p.blocks + (int64_t)bh * ntq * nslot * kPairElems;
  const buffer_rsrc_t brs = make_buffer_rsrc(blk_head);

  auto slot_of = [&](int i, int tqx) { return kComp ? ktile[i] : nct + (ktile[i] - tqx + nr - 1); };
  auto valid = [&](int i, int tqx) { return tqx >= kt_lo[i] && tqx <= kt_hi[i]; };

  // LDS of stage st: Q halves at 0, 16K; dO halves at 32K, 48K; blocks at 64K
  // (key tile i, tensor e: 2 KB at 64K + (2i + e) * 2K).  Block rows are 64
  // bytes; 16-byte chunk c of row r sits at chunk c ^ ((r >> 2) & 3).
  auto stage = [&](int st, int tqx) __attribute__((always_inline)) {
    char* base = lds + st * kStage;
    auto rf = [=](int r) -> int {
      const int t = 32 * tqx + r;
      return t < Tn ? t : -1;
    };
    stage_rows_async<T, kBwdHD, kWaves, 1, kBwdD * 2>(base, q, rf);
    stage_rows_async<T, kBwdHD, kWaves, 1, kBwdD * 2>(base + kHalfTile, q + kBwdHD, rf);
    stage_rows_async<T, kBwdHD, kWaves, 1, kBwdD * 2>(base + 2 * kHalfTile, dO, rf);
    stage_rows_async<T, kBwdHD, kWaves, 1, kBwdD * 2>(base + 3 * kHalfTile, dO + kBwdHD, rf);
    // One 1 KB load per wave: key tile wave/4, tensor (wave/2)%2, rows 16*(wave%2) ..
    const int i = wave >> 2, e = (wave >> 1) & 1, hb = wave & 1;
    const int r = 16 * hb + (lane >> 2), c = (lane & 3) ^ ((r >> 2) & 3);
    const int sl = valid(i, tqx) ? slot_of(i, tqx) : 0;  // unused data from a valid slot otherwise
    const uint32_t off = (uint32_t)((((int64_t)tqx * nslot + sl) * kPairElems + e * kBlkElems) * 2) + (uint32_t)(r * 64 + c * 16);
    buffer_load_lds_16(brs, off, base + 4 * kHalfTile + (2 * i + e) * 2 * kBlkElems + hb * 1024);
  };
  constexpr int kLd = 4 * StageGeom<T, kBwdHD, kWaves>::kPerWave + 1;  // loads per wave and stage

  const Tile32Addr ad = tile32_addr<kBwdHD>();
  f32x16_t ak[4], av[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) ak[nb][j] = av[nb][j] = 0.f;
  // This lane's B operand reads: row l%32, chunk 2st + q of the block.
  const int br = lane & 31;
  uint32_t boff[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) boff[st] = (uint32_t)(br * 64 + 16 * ((2 * st + qh) ^ ((br >> 2) & 3)));

  stage(0, tq_begin);
  for (int it = 0; it < n; ++it) {
    const int tqx = tq_begin + it;
    if (it + 1 < n) {
      stage((it + 1) & 1, tqx + 1);
      wait_vmcnt<kLd>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    if (valid(kt, tqx)) {
      const char* base = lds + (it & 1) * kStage;
      const char* bl = base + 4 * kHalfTile + 2 * kt * 2 * kBlkElems;
      i16x8_t bp[2], bd[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bp[st] = __builtin_bit_cast(i16x8_t, lds_read_b128(bl, boff[st]));
        bd[st] = __builtin_bit_cast(i16x8_t, lds_read_b128(bl + 2 * kBlkElems, boff[st]));
      }
      pv32_acc<4, 2>(ak, bd, base + hsel * kHalfTile, ad, nb0);
      pv32_acc<4, 2>(av, bp, base + (2 + hsel) * kHalfTile, ad, nb0);
    }
    wait_lgkmcnt0();
    lds_barrier();  // the stage's buffer is free for the load two steps on
  }

  // Lane holds key l%32 of key tile kt, dims 256*hsel + 32*(nb0 + nb) + 8m + 4q .. +3.
  if (ktile[kt] >= n_keyt) return;
  const int key = 32 * ktile[kt] + (lane & 31);
  if constexpr (kComp) {
    if (key >= Nc || chunk < kt_lo[kt] / kChunkTiles) return;
    float* pk = p.part + ((((int64_t)chunk * p.B * p.H + bh) * Nc + key) * 2) * kBwdD + hsel * kBwdHD;
    float* pv = pk + kBwdD;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d = 32 * (nb0 + nb) + 8 * m + 4 * qh;
        *reinterpret_cast<float4*>(pk + d) = make_float4(ak[nb][4 * m] * p.scale, ak[nb][4 * m + 1] * p.scale,
                                                         ak[nb][4 * m + 2] * p.scale, ak[nb][4 * m + 3] * p.scale);
        *reinterpret_cast<float4*>(pv + d) = make_float4(av[nb][4 * m], av[nb][4 * m + 1], av[nb][4 * m + 2], av[nb][4 * m + 3]);
      }
  } else {
    if (key >= Tn) return;
    const int64_t row = (int64_t)bh * Tn + key;
    float* pk = p.dk + row * kBwdD + hsel * kBwdHD;
    float* pv = p.dv + row * kBwdD + hsel * kBwdHD;
    const int j = key / (int)p.blk;
    const bool in_c = p.spread != 0 && j < Nc;
    const float inv_blk = 1.0f / (float)p.blk;
    const float* ck = p.dkc + ((int64_t)bh * Nc + (in_c ? j : 0)) * kBwdD + hsel * kBwdHD;
    const float* cv = p.dvc + ((int64_t)bh * Nc + (in_c ? j : 0)) * kBwdD + hsel * kBwdHD;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d = 32 * (nb0 + nb) + 8 * m + 4 * qh;
        float4 xk = make_float4(ak[nb][4 * m] * p.scale, ak[nb][4 * m + 1] * p.scale, ak[nb][4 * m + 2] * p.scale,
                                ak[nb][4 * m + 3] * p.scale);
        float4 xv = make_float4(av[nb][4 * m], av[nb][4 * m + 1], av[nb][4 * m + 2], av[nb][4 * m + 3]);
        if (in_c) {
          const float4 gk = *reinterpret_cast<const float4*>(ck + d);
          const float4 gv = *reinterpret_cast<const float4*>(cv + d);
          xk.x += gk.x * inv_blk; xk.y += gk.y * inv_blk; xk.z += gk.z * inv_blk; xk.w += gk.w * inv_blk;
          xv.x += gv.x * inv_blk; xv.y += gv.y * inv_blk; xv.z += gv.z * inv_blk; xv.w += gv.w * inv_blk;
        }
        *reinterpret_cast<float4*>(pk + d) = xk;
        *reinterpret_cast<float4*>(pv + d) = xv;
      }
  }
}

// dkc, dvc of one compressed entry: the chunks' partial sums added in chunk
// order (the chunks before the first query tile that sees the entry's tile
// wrote nothing).  One workgroup of 128 threads per (batch*head, entry).
__global__ __launch_bounds__(128) void hca_bwd_reduce_kernel(HcaBwdParams p) {
  const int64_t bh = blockIdx.x / p.Nc, j = blockIdx.x % p.Nc;
  const int64_t tq0 = bwd_tq_min(j / 32, p.blk, p.window, p.T, p.Nc, p.ntq);
  const int64_t c0 = tq0 < p.ntq ? tq0 / kChunkTiles : p.nchunk;
  const int d = 4 * threadIdx.x;
  float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
  for (int64_t c = c0; c < p.nchunk; ++c) {
    const float* pk = p.part + (((c * p.B * p.H + bh) * p.Nc + j) * 2) * kBwdD + d;
    const float4 a = *reinterpret_cast<const float4*>(pk);
    const float4 b = *reinterpret_cast<const float4*>(pk + kBwdD);
    sk.x += a.x; sk.y += a.y; sk.z += a.z; sk.w += a.w;
    sv.x += b.x; sv.y += b.y; sv.z += b.z; sv.w += b.w;
  }
  *reinterpret_cast<float4*>(p.dkc + (bh * p.Nc + j) * kBwdD + d) = sk;
  *reinterpret_cast<float4*>(p.dvc + (bh * p.Nc + j) * kBwdD + d) = sv;
}

static void hca_bwd_geometry(int64_t T, int64_t Nc, int64_t window, int64_t* ntq, int64_t* nct, int64_t* nr,
                             int64_t* nslot, int64_t* nchunk) {
  *ntq = (T + 31) / 32;
  *nct = (Nc + 31) / 32;
  *nr = (window + 30) / 32 + 1;
  *nslot = *nct + *nr;
  *nchunk = (*ntq + kChunkTiles - 1) / kChunkTiles;
}

size_t hca_bwd_ws_bytes(int64_t B, int64_t H, int64_t T, int64_t Nc, int64_t window) {
  int64_t ntq, nct, nr, nslot, nchunk;
  hca_bwd_geometry(T, Nc, window, &ntq, &nct, &nr, &nslot, &nchunk);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t blocks = al((size_t)(B * H * ntq * nslot + 1) * kPairElems * 2);
  const size_t part = al((size_t)(nchunk * B * H * Nc) * 2 * kBwdD * 4);
  return blocks + part;
}

hipError_t launch_hca_bwd(HcaBwdParams p, hipStream_t stream) {
  hca_bwd_geometry(p.T, p.Nc, p.window, &p.ntq, &p.nct, &p.nr, &p.nslot, &p.nchunk);
  const int64_t BH = p.B * p.H;
  p.part = reinterpret_cast<float*>(reinterpret_cast<char*>(p.blocks) +
                                    (((size_t)(BH * p.ntq * p.nslot + 1) * kPairElems * 2 + 255) & ~(size_t)255));
  hipLaunchKernelGGL(hca_bwd_dq_kernel, dim3((uint32_t)(BH * ((p.ntq + 1) / 2))), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.Nc > 0) {
    hipLaunchKernelGGL(hca_bwd_kv_kernel<true>, dim3((uint32_t)(BH * p.nchunk * ((p.nct + 1) / 2))), dim3(512), 0,
                       stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(hca_bwd_reduce_kernel, dim3((uint32_t)(BH * p.Nc)), dim3(128), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(hca_bwd_kv_kernel<false>, dim3((uint32_t)(BH * ((p.ntq + 1) / 2))), dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa

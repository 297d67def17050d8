// MFMA attention core for gfx950, shared by HCA prefill and DSA sparse
// attention.  One workgroup = 4 waves; each wave owns 16 query rows (queries
// for HCA, heads of one token for the multi-query DSA layout) and keeps its Q
// operand and O accumulator in registers.  Keys arrive in tiles of 32 rows
// that the whole workgroup stages into LDS; the per-tile key rows come from a
// policy object (compressed entries + raw window for HCA, gathered positions
// for DSA).
//
// Per tile and wave (transposed formulation, so no register shuffles are
// needed between the two products):
//   S^T[32 keys x 16 rows] = K_tile . Q^T          (A = K from LDS, B = Q regs)
//   online softmax over the key axis (state per query row, fp32, exp2)
//   O^T[D x 16 rows]     += V_tile^T . P^T        (A = V via transposing
//                                                   LDS reads, B = P regs)
// S^T's accumulator layout leaves lane l holding keys {4g..4g+3, 16+4g..16+4g+3}
// (g = l/16) of query row l%16.  The contraction over keys is order-free, so
// those eight values are used directly as the B operand of the P.V product
// and the transposing V reads fetch the same eight keys.
#pragma once

#include <type_traits>

#include "common.h"

namespace sa {

constexpr int kAttnWaves = 4;
constexpr int kAttnThreads = kAttnWaves * kWave;  // 256
constexpr int kRowsPerWave = 16;
constexpr int kBM = kAttnWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBN = 32;                         // keys per tile

// kSwz selects the LDS row swizzle: 0 = lds_swizzle (16-row core),
// 1 = lds_swizzle32 (32-row core).
template <typename T, int D, int kSwz = 0>
struct AttnGeom {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int kEPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int kChunks = D / kEPC;          // 16-byte chunks per row
  static constexpr int kRowBytes = D * (int)sizeof(T);
  static constexpr int kTileBytes = kBN * kRowBytes;
  static constexpr int kQRegs = kBf16 ? D / 32 : D / 4;
  static constexpr int kONb = D / 16;
  static constexpr int kStageBytes = 2 * kTileBytes;  // one pipeline stage: K tile + V tile
  static_assert(kChunks >= 16, "the LDS swizzle needs at least 16 chunks per row");
  __device__ static __forceinline__ int swz(int r) { return kSwz == 0 ? lds_swizzle(r) : lds_swizzle32(r); }
  // Row r, 16-byte chunk c -> byte offset in a tile.
  __device__ static __forceinline__ uint32_t chunk_off(int r, int c) {
    return (uint32_t)(r * kChunks + (c ^ swz(r))) * 16u;
  }
};

template <typename T, int D>
struct AttnRegs {
  using G = AttnGeom<T, D>;
  using QReg = typename std::conditional<G::kBf16, i16x8_t, float>::type;
  QReg q[G::kQRegs];
  f32x4_t o[G::kONb];
  float m;  // running max of scaled logits, log2 units
  float l;  // running sum of exp2(logit - m)
};

// ---------------------------------------------------------------------------
// Q operand: row pointer of this lane's query row (lane%16), or nullptr.
// ---------------------------------------------------------------------------
template <typename T, int D>
__device__ __forceinline__ void load_q(AttnRegs<T, D>& R, const T* qrow) {
  using G = AttnGeom<T, D>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < G::kQRegs; ++ks) {
    if constexpr (G::kBf16) {
      if (qrow) {
        uint4 u = *reinterpret_cast<const uint4*>(qrow + ks * 32 + g * 8);
        R.q[ks] = __builtin_bit_cast(i16x8_t, u);
      } else {
        R.q[ks] = i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      }
    } else {
      R.q[ks] = qrow ? qrow[ks * 4 + g] : 0.f;
    }
  }
#pragma unroll
  for (int nb = 0; nb < G::kONb; ++nb) R.o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  R.m = -INFINITY;
  R.l = 0.f;
}

// ---------------------------------------------------------------------------
// Global -> LDS staging of one K/V tile with gfx950's direct LDS loads
// (global_load_lds_dwordx4: lane i of the wave writes 16 bytes at
// lds_base + 16*i).  Wave w, step j fills the 64 physical chunks starting at
// chunk (j*4 + w)*64; the lane picks the logical chunk that belongs at its
// physical slot under the XOR swizzle, so reads stay contiguous within a row.
// Every tile issues the same number of loads per wave (padding rows load the
// fallback row, which is finite and masked), so a fixed vmcnt wait is exact.
// ---------------------------------------------------------------------------
template <typename T, int D, int kWaves = kAttnWaves>
struct StageGeom {
  using G = AttnGeom<T, D>;
  static constexpr int kInstr = kBN * G::kChunks / kWave;  // wave loads per K (or V) tile
  static constexpr int kPerWave = kInstr / kWaves;
  static_assert(kInstr % kWaves == 0, "tile must split evenly over the waves");
  static constexpr int kLoadsPerTile = 2 * kPerWave;  // K and V
};


// Tile source: uniform base pointers of the K and V rows; rowfn(r) gives the
// row index of tile row r relative to them, or -1 for a padding row (which
// loads row 0 of the same tensor: finite, and masked by the caller).  The
// tile holds D elements of each row; kSrcRowBytes is the row pitch in memory
// when that differs from the tile's row (a tile of half rows), else 0.
template <typename T, int D, int kWaves = kAttnWaves, int kSwz = 0, int kSrcRowBytes = 0, typename RowFn>
__device__ __forceinline__ void stage_rows_async(char* buf, const T* base_ptr, RowFn&& rowfn) {
  using G = AttnGeom<T, D, kSwz>;
  using SG = StageGeom<T, D, kWaves>;
  constexpr uint32_t kPitch = kSrcRowBytes > 0 ? (uint32_t)kSrcRowBytes : (uint32_t)G::kRowBytes;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  // All row lookups first: rowfn may read LDS, and such a read cannot be
  // moved past a direct-to-LDS load, so interleaving them would serialise
  // every load behind an LDS round trip.
  int row[SG::kPerWave];
#pragma unroll
  for (int j = 0; j < SG::kPerWave; ++j) row[j] = rowfn((int)(((unsigned)(j * kWaves + wave) * kWave + lane) / G::kChunks));
  // Keep the lookups together, ahead of every use.
  __builtin_amdgcn_sched_barrier(0);
  uint32_t off[SG::kPerWave];
#pragma unroll
  for (int j = 0; j < SG::kPerWave; ++j) {
    const unsigned P = (unsigned)(j * kWaves + wave) * kWave + lane;
    const int r = (int)(P / G::kChunks), cp = (int)(P % G::kChunks);
    const int c = cp ^ G::swz(r);
    off[j] = (uint32_t)(row[j] < 0 ? 0 : row[j]) * kPitch + (uint32_t)c * 16u;
  }
  const buffer_rsrc_t rsrc = make_buffer_rsrc(base_ptr);
#pragma unroll
  for (int j = 0; j < SG::kPerWave; ++j) {
    const int base = (j * kWaves + wave) * kWave;  // first physical chunk of this load
    buffer_load_lds_16(rsrc, off[j], buf + base * 16);
  }
}

// The same loads with the rows looked up beforehand: row[j] is the row of
// this lane's load j, i.e. of tile row stage_row_of(j).  A caller whose rows
// come from LDS can read them well ahead of the loads, so that sending the
// loads does not wait on that read.
template <typename T, int D, int kWaves, int kSwz>
__device__ __forceinline__ int stage_row_of(int j) {
  using G = AttnGeom<T, D, kSwz>;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  return (int)(((unsigned)(j * kWaves + wave) * kWave + lane) / G::kChunks);
}

template <typename T, int D, int kWaves, int kSwz>
__device__ __forceinline__ void stage_rows_pre(char* buf, const T* base_ptr, const int* row) {
  using G = AttnGeom<T, D, kSwz>;
  using SG = StageGeom<T, D, kWaves>;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const buffer_rsrc_t rsrc = make_buffer_rsrc(base_ptr);
#pragma unroll
  for (int j = 0; j < SG::kPerWave; ++j) {
    const unsigned P = (unsigned)(j * kWaves + wave) * kWave + lane;
    const int r = (int)(P / G::kChunks), cp = (int)(P % G::kChunks);
    const int c = cp ^ G::swz(r);
    const uint32_t off = (uint32_t)(row[j] < 0 ? 0 : row[j]) * (uint32_t)G::kRowBytes + (uint32_t)c * 16u;
    buffer_load_lds_16(rsrc, off, buf + (j * kWaves + wave) * kWave * 16);
  }
}

template <typename T, int D, typename RowFn>
__device__ __forceinline__ void stage_async(char* kbuf, char* vbuf, const T* kbase, const T* vbase,
                                            RowFn&& rowfn) {
  stage_rows_async<T, D>(kbuf, kbase, rowfn);
  stage_rows_async<T, D>(vbuf, vbase, rowfn);
}

// Wait until this wave's direct LDS loads, except the newest kPendingLoads,
// have landed.
template <int kPendingLoads>
__device__ __forceinline__ void wait_loads() {
  wait_vmcnt<kPendingLoads>();
}

// ---------------------------------------------------------------------------
// One key tile for one wave, in two stages so that callers can stream the V
// tile while the first stage runs:
//   attend_qk: S^T = K . Q^T, mask, online-softmax update -> probabilities
//   attend_pv: O^T += V^T . P^T
// visible(key_in_tile) is evaluated for this lane's query row (lane%16) and
// the 8 keys the lane holds.  scale_log2 = softmax scale * log2(e).
// ---------------------------------------------------------------------------
struct PFrag {
  f32x4_t s[2];  // probabilities of keys {4g..4g+3} (s[0]) and {16+4g..16+4g+3} (s[1])
};

// Raw scores of one key tile: S^T = K . Q^T (no mask, no softmax).
// kValuSlots > 0 interleaves that many independent VALU instructions per MFMA
// pair into the MFMA stream (for callers that overlap other work with it).
template <typename T, int D, int kValuSlots = 0>
__device__ __forceinline__ PFrag qk_raw(const AttnRegs<T, D>& R, const char* ks) {
  using G = AttnGeom<T, D>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, L = lane & 15;

  // ---- S^T = K . Q^T -------------------------------------------------------
  f32x4_t s[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  if constexpr (G::kBf16) {
    // Row r = kb*16 + L, logical chunk g + 4*kstep.  With s = lds_swizzle(L)
    // the physical chunk is (g ^ s%4) + 4*((kstep%4) ^ s/4) + 16*(kstep/4):
    // four per-lane bases plus compile-time offsets.
    // Bits 6..7 of rb are zero, so kbase ^ 64*(kstep%4) gives the swizzled
    // chunk with one base register; the opaque copy keeps the compiler from
    // hoisting the four variants out of the caller's key loop.
    const int sw = lds_swizzle(L);
    uint32_t kb0 = (uint32_t)L * G::kRowBytes + 16u * (uint32_t)(g ^ (sw & 3)) + 64u * (uint32_t)(sw >> 2);
    asm volatile("" : "+v"(kb0));
    // Four independent accumulator chains (key block x kstep parity) so that
    // dependent MFMAs are never back to back; operand reads are software
    // pipelined against the MFMAs (see the schedule groups below).
    f32x4_t acc[2][2] = {{f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}},
                         {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
    for (int kstep = 0; kstep < G::kQRegs; ++kstep) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t off = (kb0 ^ (64u * (kstep & 3))) + 256u * (kstep >> 2) + kb * 16 * G::kRowBytes;
        const uint4 a = lds_read_b128(ks, off);
        acc[kb][kstep & 1] = mfma_bf16_16x16x32(__builtin_bit_cast(i16x8_t, a), R.q[kstep], acc[kb][kstep & 1]);
      }
    }
    // Schedule: 6 operand reads ahead, then alternate 2 MFMAs / 2 reads,
    // with room for up to kValuSlots independent VALU instructions (the
    // previous tile's softmax, when the caller overlaps it) after each MFMA
    // pair.
    constexpr int kReads = 2 * G::kQRegs;
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < (kReads - 6) / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      if constexpr (kValuSlots > 0) __builtin_amdgcn_sched_group_barrier(0x002, kValuSlots, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    s[0] = acc[0][0] + acc[0][1];
    s[1] = acc[1][0] + acc[1][1];
  } else {
#pragma unroll
    for (int kstep = 0; kstep < G::kQRegs; ++kstep) {
      const int e = kstep * 4 + g;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r = kb * 16 + L;
        const float a = *reinterpret_cast<const float*>(ks + G::chunk_off(r, e >> 2) + (e & 3) * 4);
        s[kb] = mfma_f32_16x16x4(a, R.q[kstep], s[kb]);
      }
    }
  }
  return PFrag{{s[0], s[1]}};
}

// Mask and online-softmax update of one tile's raw scores, in place: on
// return P holds the tile's probabilities (against R.m) and R.l, R.m and the
// O accumulators are updated.
template <typename T, int D, typename VisFn>
__device__ __forceinline__ void softmax_update(AttnRegs<T, D>& R, PFrag& P, float scale_log2, VisFn&& visible) {
  using G = AttnGeom<T, D>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  f32x4_t* s = P.s;
  // ---- mask, online softmax ------------------------------------------------
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = kb * 16 + g * 4 + j;
      const float x = visible(key) ? s[kb][j] * scale_log2 : -INFINITY;
      s[kb][j] = x;
      mx = fmaxf(mx, x);
    }
  }
  mx = max_across_groups(mx);
  // Lazy rescaling: the reference max only moves when the tile's max exceeds
  // it by more than 2^kRescaleLog2.  Until then probabilities are computed
  // against the stale max (values up to 2^kRescaleLog2, exact in fp32 and
  // fine for bf16), and since l uses the same reference the result is
  // unchanged.  This skips the O-accumulator rescale on almost every tile.
  constexpr float kRescaleLog2 = 8.f;
  if (__any(mx > R.m + kRescaleLog2)) {
    const float m_new = fmaxf(R.m, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(R.m - m_new);
    R.l *= alpha;
    R.m = m_new;
#pragma unroll
    for (int nb = 0; nb < G::kONb; ++nb) {
      R.o[nb] *= alpha;
      if ((nb & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
  }
  const float base = (R.m == -INFINITY) ? 0.f : R.m;
  float rs = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p = fast_exp2(s[kb][j] - base);
      s[kb][j] = p;
      rs += p;
    }
  }
  rs = sum_across_groups(rs);
  R.l += rs;
}

template <typename T, int D, typename VisFn>
__device__ __forceinline__ PFrag attend_qk(AttnRegs<T, D>& R, const char* ks, float scale_log2, VisFn&& visible) {
  PFrag P = qk_raw<T, D>(R, ks);
  softmax_update<T, D>(R, P, scale_log2, visible);
  return P;
}

template <typename T, int D>
__device__ __forceinline__ void attend_pv(AttnRegs<T, D>& R, const char* vs, const PFrag& P) {
  using G = AttnGeom<T, D>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, L = lane & 15;
  const f32x4_t* s = P.s;

  // ---- O^T += V^T . P^T ----------------------------------------------------
  if constexpr (G::kBf16) {
    const uint32_t p01 = pack_bf16x2(s[0][0], s[0][1]), p23 = pack_bf16x2(s[0][2], s[0][3]);
    const uint32_t p45 = pack_bf16x2(s[1][0], s[1][1]), p67 = pack_bf16x2(s[1][2], s[1][3]);
    const i16x8_t pf = __builtin_bit_cast(i16x8_t, make_uint4(p01, p23, p45, p67));
    // Transposing reads: group g's lane L points at row key1 = 4g + L/4 (and
    // key1 + 16), dims nb*16 + 4*(L%4) .. +3, i.e. logical chunk 2*nb + h with
    // h = (L%4)/2, byte 8*(L%2) within it.  With s = lds_swizzle(key1) the
    // physical byte offset is 256*(nb/8) + 32*((nb%8) ^ s/2) + 16*(h ^ s%2)
    // + 8*(L%2): eight per-lane bases plus compile-time offsets.
    // Bits 5..7 of the row offset are zero: one base register, XOR-ed with
    // 32*(nb%8) (opaque copy: recomputed here, not hoisted by the caller).
    const int key1 = 4 * g + (L >> 2);
    const int sw = lds_swizzle(key1);
    uint32_t vb0 = (uint32_t)key1 * G::kRowBytes + 16u * (uint32_t)(((L & 3) >> 1) ^ (sw & 1)) + 8u * (L & 1) +
                   32u * (uint32_t)(sw >> 1);
    asm volatile("" : "+v"(vb0));
#pragma unroll
    for (int nb = 0; nb < G::kONb; ++nb) {
      const uint32_t off = (vb0 ^ (32u * (nb & 7))) + 256u * (nb >> 3);
      const i16x4_t lo = lds_read_tr16_b64(vs + off);
      const i16x4_t hi = lds_read_tr16_b64(vs + off + 16 * G::kRowBytes);
      const i16x8_t a = i16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      R.o[nb] = mfma_bf16_16x16x32(a, pf, R.o[nb]);
    }
    // Schedule: 8 transposing reads (4 blocks) ahead, then 1 MFMA / 2 reads.
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
    for (int i = 0; i < G::kONb - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
  } else {
#pragma unroll
    for (int nb = 0; nb < G::kONb; ++nb) {
      const int dim = nb * 16 + L;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = 16 * kb + 4 * g + j;
          const float a = *reinterpret_cast<const float*>(vs + G::chunk_off(key, dim >> 2) + (dim & 3) * 4);
          R.o[nb] = mfma_f32_16x16x4(a, s[kb][j], R.o[nb]);
        }
      }
    }
  }
}

// Both stages on one tile whose K and V are already in LDS.
template <typename T, int D, typename VisFn>
__device__ __forceinline__ void attend_tile(AttnRegs<T, D>& R, const char* ks, const char* vs, float scale_log2,
                                            VisFn&& visible) {
  const PFrag P = attend_qk<T, D>(R, ks, scale_log2, visible);
  attend_pv<T, D>(R, vs, P);
}

// ---------------------------------------------------------------------------
// Normalise and write this wave's 16 output rows.  orow: row pointer for the
// lane's query row (lane%16) or nullptr; lse_out: pointer for that row's lse
// or nullptr.
// ---------------------------------------------------------------------------
template <typename T, int D>
__device__ __forceinline__ void finish_rows(const AttnRegs<T, D>& R, T* orow, float* lse_out) {
  using G = AttnGeom<T, D>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const float inv = R.l > 0.f ? 1.f / R.l : 0.f;
  if (orow) {
#pragma unroll
    for (int nb = 0; nb < G::kONb; ++nb) {
      const int dim = nb * 16 + g * 4;
      const f32x4_t v = R.o[nb] * inv;
      if constexpr (G::kBf16) {
        uint2 u = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        *reinterpret_cast<uint2*>(orow + dim) = u;
      } else {
        *reinterpret_cast<float4*>(orow + dim) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
  if (lse_out && g == 0) {
    *lse_out = R.l > 0.f ? (R.m + __log2f(R.l)) * kLn2 : -INFINITY;
  }
}

// Split-K variant: write this wave's rows normalised in fp32 plus the
// log2-domain normaliser (m + log2 l) of this split; a combine kernel merges
// the splits.  Rows without any visible key get o = 0 and -inf.
template <typename T, int D>
__device__ __forceinline__ void finish_rows_partial(const AttnRegs<T, D>& R, float* orow, float* lse2_out) {
  using G = AttnGeom<T, D>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const float inv = R.l > 0.f ? 1.f / R.l : 0.f;
#pragma unroll
  for (int nb = 0; nb < G::kONb; ++nb) {
    const f32x4_t v = R.o[nb] * inv;
    *reinterpret_cast<float4*>(orow + nb * 16 + g * 4) = make_float4(v[0], v[1], v[2], v[3]);
  }
  if (g == 0) *lse2_out = R.l > 0.f ? R.m + __log2f(R.l) : -INFINITY;
}

}  // namespace sa

// Device helpers shared by the gfx950 kernels: bf16 conversion, MFMA
// wrappers, LDS addressing, XCD-aware block numbering and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t bf16_t;  // storage type of a bfloat16 value

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// bfloat16 <-> float
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round to nearest, ties to even (the usual bias-and-truncate construction);
// NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even,
// with gfx950's v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// ---------------------------------------------------------------------------
// MFMA (operand layouts checked on gfx950):
//  16x16x32 bf16: A lane l holds A[l%16][(l/16)*8 + 0..7], B lane l holds
//    B[(l/16)*8 + 0..7][l%16], C lane l holds C[(l/16)*4 + 0..3][l%16].
//  32x32x16 bf16: A lane l holds A[l%32][(l/32)*8 + 0..7], B lane l holds
//    B[(l/32)*8 + 0..7][l%32], C value j holds C[8*(j/4) + (l/32)*4 + j%4][l%32].
//  16x16x4 f32:   A lane l holds A[l%16][l/16], B lane l holds B[l/16][l%16],
//    C as above.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4_t mfma_bf16_16x16x32(i16x8_t a, i16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma_bf16_32x32x16(i16x8_t a, i16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f32_16x16x4(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Streaming global loads: 16 bytes with the non-temporal hint, for data read
// once (decode caches, compression inputs).  A plain streaming read of 8 GiB
// measures 7.05-7.15 TB/s with the hint against 6.0-6.3 TB/s without it.
// ---------------------------------------------------------------------------
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream_u4(const void* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// ---------------------------------------------------------------------------
// LDS access
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint4 lds_read_b128(const char* lds_base, uint32_t byte_off) {
  return *reinterpret_cast<const uint4*>(lds_base + byte_off);
}
__device__ __forceinline__ void lds_write_b128(char* lds_base, uint32_t byte_off, uint4 v) {
  *reinterpret_cast<uint4*>(lds_base + byte_off) = v;
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane L supplies the address of 4 consecutive 16-bit values M[L][0..3];
// lane i receives {M[i/4 + 4c][i%4] : c = 0..3}.
__device__ __forceinline__ i16x4_t lds_read_tr16_b64(const char* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
}

// ---------------------------------------------------------------------------
// Direct global -> LDS loads go through a buffer descriptor (MUBUF with the
// LDS bit) rather than the FLAT-encoded global form: the compiler then counts
// them on vmcnt alone, and LDS reads issued while they are in flight keep
// exact lgkmcnt waits.  The descriptor covers [base, base + 4 GiB); callers
// pass byte offsets below 2^32 (bounds are checked before the offsets are
// formed).
typedef __amdgpu_buffer_rsrc_t buffer_rsrc_t;
__device__ __forceinline__ buffer_rsrc_t make_buffer_rsrc(const void* base) {
  // Word 3 of a gfx9 raw buffer descriptor: 32-bit data format, no swizzle.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0xffffffff, 0x00020000);
}
// Lane i's 16 bytes at byte offset voff land at lds_wave_base + 16*i.
__device__ __forceinline__ void buffer_load_lds_16(buffer_rsrc_t rsrc, uint32_t voff, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds_wave_base, 16, voff, 0, 0, 0);
}
// Lane i's 4 bytes at byte offset voff land at lds_wave_base + 4*i.
__device__ __forceinline__ void buffer_load_lds_4(buffer_rsrc_t rsrc, uint32_t voff, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds_wave_base, 4, voff, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Cross-lane pairs without LDS: v_permlane16_swap / v_permlane32_swap with
// both operands equal leave, in every lane, the values of the lane pair
// (l, l^16) or (l, l^32), always in the same order, so the reductions below
// give bit-identical results in both lanes of a pair.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave reductions over lanes that share lane%16 (xor 16 and xor 32).
__device__ __forceinline__ float max_across_groups(float x) { return max_xor32(max_xor16(x)); }
__device__ __forceinline__ float sum_across_groups(float x) { return sum_xor32(sum_xor16(x)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Workgroups are dispatched to the XCDs round-robin (block b runs on XCD
// b % 8).  Renumber so that consecutive logical ids run on the same XCD and
// share its L2: XCD x gets a contiguous range of logical ids.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t n) {
  const uint32_t q = n / kNumXcd, r = n % kNumXcd;
  const uint32_t x = b % kNumXcd, local = b / kNumXcd;
  return x * q + (x < r ? x : r) + local;
}

// LDS row swizzle for tiles stored as rows of >= 16 chunks of 16 bytes:
// chunk c of row r lives at physical chunk c ^ lds_swizzle(r).  With 64 LDS
// banks (256 bytes per cycle) this is conflict-free both for 16 lanes reading
// the same chunk of 16 consecutive rows (an MFMA operand fetch) and for 8
// consecutive rows read as 32-byte pieces (the transposing V reads).
__device__ __forceinline__ int lds_swizzle(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
// Variant for the 32-row core, whose transposing reads take 64 bytes from
// each of 4 consecutive rows per LDS cycle: distinct over any 16 consecutive
// rows, and distinct in bits 2..3 over 4 aligned rows.
__device__ __forceinline__ int lds_swizzle32(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// ---------------------------------------------------------------------------
// Wait counters and barriers for pipelines fed by direct global->LDS loads.
// The builtin s_waitcnt is visible to the compiler's own wait insertion (an
// asm one is not), so it does not add a full vmcnt(0) wait of its own before
// LDS reads.  A plain __syncthreads() is a release fence and would wait for
// every outstanding LDS load; lds_barrier() is the bare s_barrier with
// compiler-only fences, for use after the caller's explicit waits.
// s_waitcnt immediate (gfx9): vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4]<<14.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wave index within the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }
__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

}  // namespace sa

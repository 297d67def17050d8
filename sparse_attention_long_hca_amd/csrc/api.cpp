// C ABI of the HCA + MLA-DSA forward library: argument validation, workspace
// sizing and dispatch to the gfx950 kernels.  Every check runs on the host
// before anything is enqueued and touches no HIP state, so invalid calls are
// rejected (with a status code and a message) even without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "sparse_attn_hca.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elem_size(sa_dtype dt) { return dt == SA_BF16 ? 2 : 4; }

float resolve_scale_log2(float scale, int64_t d) {
  const float s = scale > 0.f ? scale : 1.0f / std::sqrt((float)d);
  return s * 1.4426950408889634f;
}

}  // namespace

extern "C" {

const char* sa_last_error(void) { return g_err; }

const char* sa_version(void) { return "sparse_attn_hca 0.1.0 (gfx950)"; }

// ---------------------------------------------------------------------------
int hca_compress(const void* x, void* out, sa_dtype dtype, int64_t B, int64_t H, int64_t n_tokens, int64_t d,
                 int64_t blk, int64_t x_sb, int64_t x_sh, int64_t x_st, int64_t o_sb, int64_t o_sh, int64_t o_sn,
                 hipStream_t stream) {
  if (dtype != SA_F32 && dtype != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "hca_compress: unknown dtype %d", (int)dtype);
  if (B <= 0 || H <= 0 || d <= 0 || blk <= 0 || n_tokens < 0)
    return fail(SA_ERR_SHAPE, "hca_compress: B, H, d, blk must be > 0 and n_tokens >= 0");
  if (n_tokens / blk == 0) return ok();  // no complete block: nothing to write (pointers may be NULL)
  if (!x || !out) return fail(SA_ERR_NULL, "hca_compress: x and out must be non-NULL");
  const int64_t es = (int64_t)elem_size(dtype);
  const int64_t chunks = d * es / 16;
  if ((d * es) % 16 != 0 || chunks > 256)
    return fail(SA_ERR_UNSUPPORTED, "hca_compress: d*sizeof(elem) must be a multiple of 16 bytes, at most 4096 (d=%lld)",
                (long long)d);
  if (blk > (1 << 20)) return fail(SA_ERR_SHAPE, "hca_compress: blk too large");
  if (!aligned16(x) || !aligned16(out)) return fail(SA_ERR_ALIGN, "hca_compress: pointers must be 16-byte aligned");
  const int64_t epc = 16 / es;
  if (x_sb % epc || x_sh % epc || x_st % epc || o_sb % epc || o_sh % epc || o_sn % epc)
    return fail(SA_ERR_ALIGN, "hca_compress: strides must be multiples of 16 bytes");
  const int64_t n_out = n_tokens / blk;
  if (B * H * n_out > 0x7fffffffLL) return fail(SA_ERR_SHAPE, "hca_compress: too many output rows");
  sa::HcaCompressParams p{x, out, B, H, n_out, d, blk, x_sb, x_sh, x_st, o_sb, o_sh, o_sn};
  return hip_status(sa::launch_hca_compress(p, dtype == SA_BF16 ? 1 : 0, stream), "hca_compress launch");
}

// ---------------------------------------------------------------------------
static int64_t hca_dv(const hca_attention_args* a) { return a->d_v == 0 ? a->d : a->d_v; }

static int hca_check(const hca_attention_args* a) {
  if (!a) return fail(SA_ERR_NULL, "hca_attention_fwd: args is NULL");
  if (a->mode != HCA_PREFILL && a->mode != HCA_DECODE) return fail(SA_ERR_SHAPE, "hca_attention_fwd: unknown mode");
  if (!a->q || !a->k || !a->v || !a->o) return fail(SA_ERR_NULL, "hca_attention_fwd: q, k, v, o must be non-NULL");
  if (a->B <= 0 || a->H <= 0 || a->d <= 0 || a->d_v < 0 || a->blk <= 0 || a->window <= 0 || a->n_c_cap < 0)
    return fail(SA_ERR_SHAPE, "hca_attention_fwd: B, H, d, blk, window must be > 0, d_v, n_c_cap >= 0");
  const int64_t dv = hca_dv(a);
  const bool bf16_512 = a->dtype == SA_BF16 && a->d == 512 && dv == 512;
  const bool bf16_576 = a->dtype == SA_BF16 && a->d == 576 && dv == 512;
  if (a->n_c_cap > 0 && (!a->k_c || !a->v_c))
    return fail(SA_ERR_NULL, "hca_attention_fwd: k_c, v_c must be non-NULL when n_c_cap > 0");
  if (a->mode == HCA_PREFILL) {
    if (a->seq_len <= 0) return fail(SA_ERR_SHAPE, "hca_attention_fwd: seq_len must be > 0 for PREFILL");
    const bool sup = (a->dtype == SA_F32 && a->d == 64 && dv == 64) || bf16_512 || bf16_576;
    if (!sup)
      return fail(SA_ERR_UNSUPPORTED,
                  "hca_attention_fwd PREFILL: supported (dtype, d, d_v) are (f32, 64, 64), (bf16, 512, 512), (bf16, 576, 512)");
    if (a->n_c_cap > a->seq_len / a->blk)
      return fail(SA_ERR_SHAPE, "hca_attention_fwd PREFILL: n_c_cap (%lld) exceeds seq_len/blk (%lld)",
                  (long long)a->n_c_cap, (long long)(a->seq_len / a->blk));
    if (a->seq_len >= ((int64_t)1 << 30) || a->blk >= ((int64_t)1 << 30) || a->window >= ((int64_t)1 << 30))
      return fail(SA_ERR_SHAPE, "hca_attention_fwd PREFILL: seq_len, blk and window must be < 2^30");
    const int64_t n_qt = (a->seq_len + 63) / 64;
    if (a->B * a->H * n_qt > 0x7fffffffLL) return fail(SA_ERR_SHAPE, "hca_attention_fwd: grid too large");
  } else {
    if (!a->pos) return fail(SA_ERR_NULL, "hca_attention_fwd DECODE: pos must be non-NULL");
    if (!bf16_512 && !bf16_576)
      return fail(SA_ERR_UNSUPPORTED, "hca_attention_fwd DECODE: supported (dtype, d, d_v) are (bf16, 512, 512), (bf16, 576, 512)");
    if (a->n_c_cap < 1) return fail(SA_ERR_SHAPE, "hca_attention_fwd DECODE: n_c_cap must be >= 1");
  }
  const void* ptrs[] = {a->q, a->k, a->v, a->k_c, a->v_c, a->o, a->lse};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SA_ERR_ALIGN, "hca_attention_fwd: pointers must be 16-byte aligned");
  return SA_OK;
}

static int64_t hca_dec_nsplit(const hca_attention_args* a) {
  return sa::hca_decode_nsplit(a->B * a->H, a->n_c_cap + a->window);
}

size_t hca_attention_fwd_workspace_size(const hca_attention_args* a) {
  if (!a || a->mode != HCA_DECODE || a->B <= 0 || a->H <= 0 || a->d <= 0 || a->d_v < 0) return 0;
  return sa::hca_decode_workspace_bytes(a->B * a->H, hca_dec_nsplit(a), hca_dv(a));
}

int hca_attention_fwd(const hca_attention_args* a, hipStream_t stream) {
  const int c = hca_check(a);
  if (c != SA_OK) return c;
  const float sl2 = resolve_scale_log2(a->scale, a->d);
  if (a->mode == HCA_PREFILL) {
    sa::HcaPrefillParams p{a->q, a->k, a->v, a->k_c, a->v_c, a->o, a->lse, a->B, a->H, a->seq_len,
                           a->n_c_cap, a->blk, a->window, sl2, (a->seq_len + 63) / 64};
    return hip_status(sa::launch_hca_prefill(p, a->dtype == SA_BF16 ? 1 : 0, (int)a->d, (int)hca_dv(a), stream),
                      "hca_attention_fwd prefill launch");
  }
  const int64_t BH = a->B * a->H;
  const int64_t ns = hca_dec_nsplit(a);
  const int64_t dv = hca_dv(a);
  const size_t need = sa::hca_decode_workspace_bytes(BH, ns, dv);
  if (need > 0) {
    if (!a->workspace || a->workspace_bytes < need)
      return fail(SA_ERR_WORKSPACE, "hca_attention_fwd DECODE: needs %zu workspace bytes, got %zu", need,
                  a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned16(a->workspace)) return fail(SA_ERR_ALIGN, "hca_attention_fwd: workspace must be 16-byte aligned");
  }
  if (BH * ns > 0x7fffffffLL) return fail(SA_ERR_SHAPE, "hca_attention_fwd: grid too large");
  const int64_t max_keys = a->n_c_cap + a->window;
  float* part_o = reinterpret_cast<float*>(a->workspace);
  float* part_lse = part_o ? part_o + BH * ns * dv : nullptr;
  sa::HcaDecodeParams p{a->q, a->k_c, a->v_c, a->k, a->v, nullptr, nullptr, nullptr, nullptr,
                        a->pos, a->o, a->lse, part_o, part_lse,
                        a->B, a->H, a->n_c_cap, a->blk, a->window, sl2, ns, (max_keys + ns - 1) / ns};
  return hip_status(sa::launch_hca_decode(p, 1, (int)a->d, (int)dv, stream), "hca_attention_fwd decode launch");
}

// ---------------------------------------------------------------------------
static int hca_bwd_check(const hca_attention_bwd_args* a) {
  if (!a) return fail(SA_ERR_NULL, "hca_attention_bwd: args is NULL");
  if (a->B <= 0 || a->H <= 0 || a->d <= 0 || a->blk <= 0 || a->window <= 0 || a->seq_len <= 0 || a->n_c < 0)
    return fail(SA_ERR_SHAPE, "hca_attention_bwd: B, H, d, blk, window, seq_len must be > 0 and n_c >= 0");
  if (a->dtype != SA_BF16 || a->d != 512)
    return fail(SA_ERR_UNSUPPORTED, "hca_attention_bwd: supported is (bf16, d = 512)");
  if (a->n_c > a->seq_len / a->blk)
    return fail(SA_ERR_SHAPE, "hca_attention_bwd: n_c (%lld) exceeds seq_len/blk (%lld)", (long long)a->n_c,
                (long long)(a->seq_len / a->blk));
  if (a->seq_len >= ((int64_t)1 << 24) || a->window >= ((int64_t)1 << 24))
    return fail(SA_ERR_SHAPE, "hca_attention_bwd: seq_len and window must be < 2^24");
  if (!a->q || !a->k || !a->v || !a->o || !a->d_o || !a->lse || !a->dq || !a->dk || !a->dv)
    return fail(SA_ERR_NULL, "hca_attention_bwd: q, k, v, o, d_o, lse, dq, dk, dv must be non-NULL");
  if (a->n_c > 0 && (!a->k_c || !a->v_c || !a->dk_c || !a->dv_c))
    return fail(SA_ERR_NULL, "hca_attention_bwd: k_c, v_c, dk_c, dv_c must be non-NULL when n_c > 0");
  const int64_t ntq = (a->seq_len + 31) / 32, nslot = (a->n_c + 31) / 32 + (a->window + 30) / 32 + 1;
  if (ntq * nslot * 4096 >= ((int64_t)1 << 32))
    return fail(SA_ERR_SHAPE, "hca_attention_bwd: (seq_len/32) * (n_c/32 + window/32) too large (per-head weight blocks "
                              "must stay below 4 GiB)");
  const int64_t BH = a->B * a->H;
  if (BH * ((ntq + 1) / 2) > 0x7fffffffLL || BH * a->n_c > 0x7fffffffLL)
    return fail(SA_ERR_SHAPE, "hca_attention_bwd: grid too large");
  const void* ptrs[] = {a->q, a->k, a->v, a->k_c, a->v_c, a->o, a->d_o, a->lse, a->dq, a->dk, a->dv, a->dk_c, a->dv_c};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SA_ERR_ALIGN, "hca_attention_bwd: pointers must be 16-byte aligned");
  return SA_OK;
}

size_t hca_attention_bwd_workspace_size(const hca_attention_bwd_args* a) {
  if (!a || a->B <= 0 || a->H <= 0 || a->seq_len <= 0 || a->n_c < 0 || a->window <= 0) return 0;
  return sa::hca_bwd_ws_bytes(a->B, a->H, a->seq_len, a->n_c, a->window);
}

int hca_attention_bwd(const hca_attention_bwd_args* a, hipStream_t stream) {
  const int c = hca_bwd_check(a);
  if (c != SA_OK) return c;
  const size_t need = sa::hca_bwd_ws_bytes(a->B, a->H, a->seq_len, a->n_c, a->window);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(SA_ERR_WORKSPACE, "hca_attention_bwd: needs %zu workspace bytes, got %zu", need,
                a->workspace ? a->workspace_bytes : (size_t)0);
  if (!aligned16(a->workspace)) return fail(SA_ERR_ALIGN, "hca_attention_bwd: workspace must be 16-byte aligned");
  sa::HcaBwdParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.kc = a->k_c;
  p.vc = a->v_c;
  p.o = a->o;
  p.dout = a->d_o;
  p.lse = a->lse;
  p.dq = a->dq;
  p.dk = a->dk;
  p.dv = a->dv;
  p.dkc = a->dk_c;
  p.dvc = a->dv_c;
  p.B = a->B;
  p.H = a->H;
  p.T = a->seq_len;
  p.Nc = a->n_c;
  p.blk = a->blk;
  p.window = a->window;
  p.spread = a->through_compress != 0 ? 1 : 0;
  p.scale = a->scale > 0.f ? a->scale : 1.0f / std::sqrt((float)a->d);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  p.blocks = reinterpret_cast<uint16_t*>(a->workspace);
  return hip_status(sa::launch_hca_bwd(p, stream), "hca_attention_bwd launch");
}

// ---------------------------------------------------------------------------
// Allocation-free HCA attention: the decode split partials go to `scratch`, a
// file-scope device array (each GPU the library runs on holds its own copy
// until the process ends) instead of a caller workspace.  Host code never
// passes the array's name to a kernel: the device address is looked up once
// per device with hipGetSymbolAddress and kept in g_scratch_ptr.
}  // extern "C"

static constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on device dev, looked up on the first call for
// that device with dev current.
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(SA_ERR_HIP, "hca_attention_fwd_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess || !p)
      return fail(SA_ERR_HIP, "hca_attention_fwd_noalloc: scratch address on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}
}  // namespace

extern "C" {

int hca_attention_fwd_noalloc(const hca_attention_args* a, hipStream_t stream) {
  const int c = hca_check(a);
  if (c != SA_OK) return c;
  hca_attention_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (a->mode == HCA_DECODE) {
    const size_t need = sa::hca_decode_workspace_bytes(a->B * a->H, hca_dec_nsplit(a), hca_dv(a));
    if (need > kScratchBytes)
      return fail(SA_ERR_WORKSPACE, "hca_attention_fwd_noalloc: needs %zu scratch bytes, the static limit is %zu", need,
                  kScratchBytes);
    if (need > 0) {
      int dev = 0;
      const hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
      if (e != hipSuccess) return hip_status(e, "hca_attention_fwd_noalloc: stream device");
      void* ptr = nullptr;
      const int r = scratch_on(dev, &ptr);
      if (r != SA_OK) return r;
      b.workspace = ptr;
      b.workspace_bytes = kScratchBytes;
    }
  }
  return hca_attention_fwd(&b, stream);
}

// ---------------------------------------------------------------------------
int hca_quantize_fp8(const void* x, void* codes, float* scales, int64_t rows, int64_t d, hipStream_t stream) {
  if (rows < 0 || d <= 0) return fail(SA_ERR_SHAPE, "hca_quantize_fp8: rows must be >= 0 and d > 0");
  if (rows == 0) return ok();
  if (!x || !codes || !scales) return fail(SA_ERR_NULL, "hca_quantize_fp8: x, codes, scales must be non-NULL");
  if (d % 16 != 0 || d > 4096) return fail(SA_ERR_UNSUPPORTED, "hca_quantize_fp8: d must be a multiple of 16, <= 4096");
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales))
    return fail(SA_ERR_ALIGN, "hca_quantize_fp8: pointers must be 16-byte aligned");
  if ((rows + 3) / 4 > 0x7fffffffLL) return fail(SA_ERR_SHAPE, "hca_quantize_fp8: too many rows");
  sa::HcaQuantParams p{x, codes, scales, rows, d};
  return hip_status(sa::launch_hca_quantize_fp8(p, stream), "hca_quantize_fp8 launch");
}

static int hca_fp8_check(const hca_decode_fp8_args* a) {
  if (!a) return fail(SA_ERR_NULL, "hca_decode_fp8: args is NULL");
  if (!a->q || !a->k_c || !a->k_c_scale || !a->v_c || !a->v_c_scale || !a->k || !a->k_scale || !a->v ||
      !a->v_scale || !a->pos || !a->o)
    return fail(SA_ERR_NULL, "hca_decode_fp8: q, codes, scales, pos and o must be non-NULL");
  if (a->B <= 0 || a->H <= 0 || a->d <= 0 || a->blk <= 0 || a->window <= 0 || a->n_c_cap < 1)
    return fail(SA_ERR_SHAPE, "hca_decode_fp8: B, H, d, blk, window and n_c_cap must be > 0");
  if (a->d != 512) return fail(SA_ERR_UNSUPPORTED, "hca_decode_fp8: d must be 512");
  const void* ptrs[] = {a->q, a->k_c, a->k_c_scale, a->v_c, a->v_c_scale, a->k, a->k_scale, a->v, a->v_scale, a->o, a->lse};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SA_ERR_ALIGN, "hca_decode_fp8: pointers must be 16-byte aligned");
  return SA_OK;
}

size_t hca_decode_fp8_workspace_size(const hca_decode_fp8_args* a) {
  if (!a || a->B <= 0 || a->H <= 0 || a->d <= 0) return 0;
  const int64_t ns = sa::hca_decode_nsplit(a->B * a->H, a->n_c_cap + a->window);
  return sa::hca_decode_workspace_bytes(a->B * a->H, ns, a->d);
}

int hca_decode_fp8(const hca_decode_fp8_args* a, hipStream_t stream) {
  const int c = hca_fp8_check(a);
  if (c != SA_OK) return c;
  const float sl2 = resolve_scale_log2(a->scale, a->d);
  const int64_t BH = a->B * a->H;
  const int64_t max_keys = a->n_c_cap + a->window;
  const int64_t ns = sa::hca_decode_nsplit(BH, max_keys);
  const size_t need = sa::hca_decode_workspace_bytes(BH, ns, a->d);
  if (need > 0) {
    if (!a->workspace || a->workspace_bytes < need)
      return fail(SA_ERR_WORKSPACE, "hca_decode_fp8: needs %zu workspace bytes, got %zu", need,
                  a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned16(a->workspace)) return fail(SA_ERR_ALIGN, "hca_decode_fp8: workspace must be 16-byte aligned");
  }
  if (BH * ns > 0x7fffffffLL) return fail(SA_ERR_SHAPE, "hca_decode_fp8: grid too large");
  float* part_o = reinterpret_cast<float*>(a->workspace);
  float* part_lse = part_o ? part_o + BH * ns * a->d : nullptr;
  sa::HcaDecodeParams p{a->q, a->k_c, a->v_c, a->k, a->v, a->k_c_scale, a->v_c_scale, a->k_scale, a->v_scale,
                        a->pos, a->o, a->lse, part_o, part_lse,
                        a->B, a->H, a->n_c_cap, a->blk, a->window, sl2, ns, (max_keys + ns - 1) / ns};
  return hip_status(sa::launch_hca_decode(p, 2, (int)a->d, (int)a->d, stream), "hca_decode_fp8 launch");
}

// ---------------------------------------------------------------------------
static int indexer_impl(const char* fn, const void* q_idx, const void* k_idx, const float* w, const int64_t* q_pos,
                        float* scores, int64_t B, int64_t T, int64_t S, int64_t Hi, int64_t Di, int64_t ratio,
                        hipStream_t stream) {
  if (!q_idx || !k_idx || !w || !scores) return fail(SA_ERR_NULL, "%s: q_idx, k_idx, w, scores must be non-NULL", fn);
  if (B <= 0 || T <= 0 || S <= 0 || Hi <= 0 || Di <= 0) return fail(SA_ERR_SHAPE, "%s: sizes must be > 0", fn);
  if (ratio < 1 || ratio > ((int64_t)1 << 20)) return fail(SA_ERR_SHAPE, "%s: ratio must be in [1, 2^20]", fn);
  if (Hi != 4 || Di != 128) return fail(SA_ERR_UNSUPPORTED, "%s: supported Hi = 4, Di = 128", fn);
  if (S > ((int64_t)1 << 24) || T >= ((int64_t)1 << 31))
    return fail(SA_ERR_UNSUPPORTED, "%s: S must be <= 2^24 and T < 2^31", fn);
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w) || !aligned16(scores))
    return fail(SA_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  // Grid of the launch: decode shapes take 128 (T <= 4) or 256 (T <= 16)
  // positions per workgroup, prefill shapes 64 queries x 1024 positions.
  const int64_t nblocks = T <= 4    ? B * ((S + 127) / 128)
                          : T <= 16 ? B * ((S + 255) / 256)
                                    : B * ((T + 63) / 64) * ((S + 1023) / 1024);
  if (nblocks > 0x7fffffffLL) return fail(SA_ERR_SHAPE, "%s: grid too large", fn);
  sa::DsaIndexerParams p{q_idx, k_idx, w, q_pos, scores, B, T, S, ratio};
  return hip_status(sa::launch_dsa_indexer(p, stream), fn);
}

int dsa_indexer_scores(const void* q_idx, const void* k_idx, const float* w, const int64_t* q_pos, float* scores,
                       int64_t B, int64_t T, int64_t S, int64_t Hi, int64_t Di, hipStream_t stream) {
  return indexer_impl("dsa_indexer_scores", q_idx, k_idx, w, q_pos, scores, B, T, S, Hi, Di, 1, stream);
}

int csa_indexer_scores(const void* q_idx, const void* k_idx, const float* w, const int64_t* q_pos, float* scores,
                       int64_t B, int64_t T, int64_t S, int64_t Hi, int64_t Di, int64_t ratio, hipStream_t stream) {
  return indexer_impl("csa_indexer_scores", q_idx, k_idx, w, q_pos, scores, B, T, S, Hi, Di, ratio, stream);
}

// ---------------------------------------------------------------------------
size_t dsa_topk_workspace_size(int64_t B, int64_t T, int64_t S, int64_t k) {
  if (B <= 0 || T <= 0 || S <= 0 || k <= 0) return 0;
  return sa::dsa_topk_ws_bytes(B, T, S, k);
}

static int topk_impl(const char* fn, const float* scores, const int64_t* q_pos, int32_t* idx, int64_t B, int64_t T,
                     int64_t S, int64_t k, int64_t ratio, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!scores || !idx) return fail(SA_ERR_NULL, "%s: scores and idx must be non-NULL", fn);
  if (B <= 0 || T <= 0 || S <= 0 || k <= 0) return fail(SA_ERR_SHAPE, "%s: sizes must be > 0", fn);
  if (ratio < 1 || ratio > ((int64_t)1 << 20)) return fail(SA_ERR_SHAPE, "%s: ratio must be in [1, 2^20]", fn);
  if (k > 2048) return fail(SA_ERR_UNSUPPORTED, "%s: k must be <= 2048", fn);
  if (S >= (int64_t)1 << 31) return fail(SA_ERR_UNSUPPORTED, "%s: S must be < 2^31", fn);
  if (!aligned16(scores) || !aligned16(idx)) return fail(SA_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  if (B * T > 0x7fffffffLL) return fail(SA_ERR_SHAPE, "%s: too many rows", fn);
  const size_t need = sa::dsa_topk_ws_bytes(B, T, S, k);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(SA_ERR_WORKSPACE, "%s: needs %zu workspace bytes, got %zu", fn, need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(SA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
    const int64_t nchunk = (S + 4095) / 4096;  // chunk size of the multi-workgroup path
    if (B * T * nchunk > 0x7fffffffLL) return fail(SA_ERR_SHAPE, "%s: grid too large", fn);
  }
  sa::DsaTopkParams p{scores, q_pos, idx, B, T, S, k, workspace, ratio};
  return hip_status(sa::launch_dsa_topk(p, stream), fn);
}

int dsa_topk(const float* scores, const int64_t* q_pos, int32_t* idx, int64_t B, int64_t T, int64_t S, int64_t k,
             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return topk_impl("dsa_topk", scores, q_pos, idx, B, T, S, k, 1, workspace, workspace_bytes, stream);
}

int csa_topk(const float* scores, const int64_t* q_pos, int32_t* idx, int64_t B, int64_t T, int64_t S, int64_t k,
             int64_t ratio, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return topk_impl("csa_topk", scores, q_pos, idx, B, T, S, k, ratio, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
size_t dsa_indexer_topk_workspace_size(int64_t B, int64_t T, int64_t S, int64_t k) {
  if (B <= 0 || T <= 0 || S <= 0 || k <= 0) return 0;
  return sa::dsa_indexer_topk_ws_bytes(B, T, S, k);
}

int dsa_indexer_topk(const void* q_idx, const void* k_idx, const float* w, const int64_t* q_pos, int32_t* idx,
                     int64_t B, int64_t T, int64_t S, int64_t Hi, int64_t Di, int64_t k, int64_t force_fallback,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "dsa_indexer_topk";
  if (!q_idx || !k_idx || !w || !idx) return fail(SA_ERR_NULL, "%s: q_idx, k_idx, w, idx must be non-NULL", fn);
  if (B <= 0 || T <= 0 || S <= 0 || Hi <= 0 || Di <= 0 || k <= 0) return fail(SA_ERR_SHAPE, "%s: sizes must be > 0", fn);
  if (Hi != 4 || Di != 128) return fail(SA_ERR_UNSUPPORTED, "%s: supported Hi = 4, Di = 128", fn);
  if (S > 32768 && (T > 4 || S > ((int64_t)1 << 24)))
    return fail(SA_ERR_UNSUPPORTED, "%s: S must be <= 32768, or <= 2^24 with T <= 4", fn);
  if (k > 2048) return fail(SA_ERR_UNSUPPORTED, "%s: k must be <= 2048", fn);
  if (B * T > 0x7fffffffLL || B * ((T + 63) / 64) * ((S + 127) / 128) > 0x7fffffffLL)
    return fail(SA_ERR_SHAPE, "%s: too many rows", fn);
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w) || !aligned16(idx))
    return fail(SA_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  const size_t need = sa::dsa_indexer_topk_ws_bytes(B, T, S, k);
  if (!workspace || workspace_bytes < need)
    return fail(SA_ERR_WORKSPACE, "%s: needs %zu workspace bytes, got %zu", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(SA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  sa::DsaIndexerTopkParams p{q_idx, k_idx, w, q_pos, idx, B, T, S, k, workspace, force_fallback != 0 ? 1 : 0};
  return hip_status(sa::launch_dsa_indexer_topk(p, stream), fn);
}

// ---------------------------------------------------------------------------
size_t dsa_sparse_attention_fwd_workspace_size(int64_t B, int64_t T, int64_t Hq, int64_t D, int64_t kk) {
  if (B <= 0 || T <= 0 || Hq <= 0 || D <= 0 || kk <= 0) return 0;
  return sa::dsa_sparse_workspace_bytes(B * T, sa::dsa_sparse_nsplit(B * T, kk), Hq, D);
}

int dsa_sparse_attention_fwd(const void* q, const void* k, const void* v, const int32_t* idx, void* o, float* lse,
                             sa_dtype dtype, int64_t B, int64_t T, int64_t S, int64_t Hq, int64_t D, int64_t kk,
                             float scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !idx || !o) return fail(SA_ERR_NULL, "dsa_sparse_attention_fwd: q, k, v, idx, o must be non-NULL");
  if (B <= 0 || T <= 0 || S <= 0 || Hq <= 0 || D <= 0 || kk <= 0)
    return fail(SA_ERR_SHAPE, "dsa_sparse_attention_fwd: sizes must be > 0");
  if (dtype != SA_BF16 || D != 256 || Hq != 64)
    return fail(SA_ERR_UNSUPPORTED, "dsa_sparse_attention_fwd: supported dtype bf16, D = 256, Hq = 64");
  if (kk > 2048) return fail(SA_ERR_UNSUPPORTED, "dsa_sparse_attention_fwd: kk must be <= 2048");
  if (S > ((int64_t)1 << 23)) return fail(SA_ERR_UNSUPPORTED, "dsa_sparse_attention_fwd: S must be <= 2^23");
  const void* ptrs[] = {q, k, v, idx, o, lse};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SA_ERR_ALIGN, "dsa_sparse_attention_fwd: pointers must be 16-byte aligned");
  const int64_t BT = B * T;
  const int64_t ns = sa::dsa_sparse_nsplit(BT, kk);
  if (BT * ns > 0x7fffffffLL) return fail(SA_ERR_SHAPE, "dsa_sparse_attention_fwd: too many tokens");
  const size_t need = sa::dsa_sparse_workspace_bytes(BT, ns, Hq, D);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(SA_ERR_WORKSPACE, "dsa_sparse_attention_fwd: needs %zu workspace bytes, got %zu", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(SA_ERR_ALIGN, "dsa_sparse_attention_fwd: workspace must be 16-byte aligned");
  }
  const int64_t tiles = (kk + 31) / 32;
  float* part_o = reinterpret_cast<float*>(workspace);
  float* part_lse = part_o ? part_o + BT * ns * Hq * D : nullptr;
  sa::DsaSparseParams p{q, k, v, idx, o, lse, part_o, part_lse, B, T, S, kk, resolve_scale_log2(scale, D),
                        ns, (tiles + ns - 1) / ns};
  return hip_status(sa::launch_dsa_sparse(p, (int)D, (int)Hq, stream), "dsa_sparse_attention_fwd launch");
}

size_t dsa_sparse_attention_bwd_workspace_size(int64_t B, int64_t T, int64_t S, int64_t kk) {
  if (B <= 0 || T <= 0 || S <= 0 || kk <= 0) return 0;
  return sa::dsa_sparse_bwd_ws_bytes(B, T, S, kk);
}

int dsa_sparse_attention_bwd(const void* q, const void* k, const void* v, const int32_t* idx, const void* o,
                             const float* lse, const void* d_o, float* dq, float* dk, float* dv, sa_dtype dtype,
                             int64_t B, int64_t T, int64_t S, int64_t Hq, int64_t D, int64_t kk, float scale,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !idx || !o || !lse || !d_o || !dq || !dk || !dv)
    return fail(SA_ERR_NULL, "dsa_sparse_attention_bwd: every pointer must be non-NULL");
  if (B <= 0 || T <= 0 || S <= 0 || Hq <= 0 || D <= 0 || kk <= 0)
    return fail(SA_ERR_SHAPE, "dsa_sparse_attention_bwd: sizes must be > 0");
  if (dtype != SA_BF16 || D != 256 || Hq != 64)
    return fail(SA_ERR_UNSUPPORTED, "dsa_sparse_attention_bwd: supported dtype bf16, D = 256, Hq = 64");
  if (kk > 2048) return fail(SA_ERR_UNSUPPORTED, "dsa_sparse_attention_bwd: kk must be <= 2048");
  if (S > ((int64_t)1 << 23)) return fail(SA_ERR_UNSUPPORTED, "dsa_sparse_attention_bwd: S must be <= 2^23");
  if (B * T > 0x7fffffffLL) return fail(SA_ERR_SHAPE, "dsa_sparse_attention_bwd: too many tokens");
  const void* ptrs[] = {q, k, v, idx, o, lse, d_o, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(SA_ERR_ALIGN, "dsa_sparse_attention_bwd: pointers must be 16-byte aligned");
  if (B * S >= 0xffffffffLL) return fail(SA_ERR_SHAPE, "dsa_sparse_attention_bwd: B*S must be < 2^32 - 1");
  const size_t need = sa::dsa_sparse_bwd_ws_bytes(B, T, S, kk);
  if (!workspace || workspace_bytes < need)
    return fail(SA_ERR_WORKSPACE, "dsa_sparse_attention_bwd: needs %zu workspace bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(SA_ERR_ALIGN, "dsa_sparse_attention_bwd: workspace must be 16-byte aligned");
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)D);
  sa::DsaSparseBwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.idx = idx;
  p.o = o;
  p.lse = lse;
  p.dout = d_o;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.B = B;
  p.T = T;
  p.S = S;
  p.kk = kk;
  p.scale = sc;
  p.scale_log2 = resolve_scale_log2(scale, D);
  p.ws = workspace;
  return hip_status(sa::launch_dsa_sparse_bwd(p, stream), "dsa_sparse_attention_bwd launch");
}

}  // extern "C"

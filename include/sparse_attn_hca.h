/*
 * sparse_attn_hca.h -- C ABI of the HCA + MLA-DSA forward library for AMD
 * Instinct MI355X (gfx950).
 *
 * The method is the hybrid sparse attention described for ERNIE-5.5-Flash-Base:
 *
 *   [P1] aitest123.com, "280B总参数、14B激活！百度开源文心5.5 Flash Base，拿下同尺寸SOTA",
 *        section 二.1 "Latent-Gated Sparse Attention：37层省缓存，6层保精准检索".
 *   [P2] qunfachuanzhen.com ERNIE-5.5-Flash-Base news page,
 *        section "◆ 混合稀疏注意力,把 1M 上下文的成本压下来".
 *   [P3] communeify.com, "百度 ERNIE 5.5 Flash Base 完整解析：280B 混合注意力 MoE 基座模型…",
 *        section "六大核心架構創新深度解析", item 1
 *        "潛在門控混合稀疏注意力（Hybrid MLA-DSA + HCA）與 VHA".
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates device memory (its one static array, the scratch
 *    of hca_attention_fwd_noalloc, is part of the loaded code object) and
 *    keeps no pointer after a call returns.  Buffers must stay alive until
 *    the enqueued work has finished.
 *  - Every call only enqueues work on the given stream (NULL = the default
 *    stream) and never synchronises (dsa_sparse_attention_bwd also forks
 *    part of its work to a stream of its own and joins it back with events,
 *    so it orders on the given stream like any other work).  Results are
 *    deterministic: the same inputs give bit-identical outputs on every run.
 *  - Inputs are read-only.  Outputs must not alias inputs.
 *  - Tensors are dense and row-major in the shapes given below, with the last
 *    (feature) dimension contiguous, unless strides are passed explicitly.
 *    Every tensor base address must be 16-byte aligned.
 *  - Arguments are validated on the host before anything is enqueued.  A
 *    non-OK status means nothing was enqueued; sa_last_error() then returns a
 *    human-readable reason (thread-local, valid until the next call on the
 *    same thread).
 *  - Device-side CONTENTS (positions, indices) are not validated.  Values
 *    outside their contract give unspecified results but never out-of-bounds
 *    memory accesses: positions are clamped and indices outside [0, S) are
 *    skipped.
 */
#ifndef SPARSE_ATTN_HCA_H
#define SPARSE_ATTN_HCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's own hipStream_t (a typedef may be repeated). */
typedef struct ihipStream_t* hipStream_t;

typedef enum { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;

typedef enum {
  SA_OK = 0,
  SA_ERR_NULL = -1,        /* a required pointer is NULL                        */
  SA_ERR_SHAPE = -2,       /* a size is non-positive or sizes are inconsistent  */
  SA_ERR_UNSUPPORTED = -3, /* (dtype, head dim, ...) combination not compiled   */
  SA_ERR_ALIGN = -4,       /* a pointer or stride breaks the 16-byte rule       */
  SA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required        */
  SA_ERR_HIP = -6          /* the HIP runtime rejected a launch                 */
} sa_status;

/* Detail for the last non-OK return on this thread ("" if none). */
const char* sa_last_error(void);
/* Library version string. */
const char* sa_version(void);

/* ------------------------------------------------------------------------
 * hca_compress -- block-mean compression of K or V.
 *
 * [P1] §二.1, [P2] §混合稀疏注意力, [P3] §架構創新 1: every 128 consecutive
 * tokens are pressed into one cache entry.  The pages do not name the
 * operator; this library uses the arithmetic mean of the block's rows:
 *
 *   out[b,h,j,:] = (1/blk) * sum_{i<blk} x[b,h,j*blk+i,:],  j < floor(n_tokens/blk)
 *
 * Trailing tokens that do not fill a block produce no entry; with no complete
 * block the call does nothing and x/out may be NULL.
 * x:   [B,H,n_tokens,d] with element strides (x_sb, x_sh, x_st), d contiguous.
 * out: [B,H,n_tokens/blk,d] with element strides (o_sb, o_sh, o_sn).
 * Arithmetic: fp32 sum, one division by blk, rounded (RNE) to the I/O dtype.
 * Supported: SA_F32 and SA_BF16 with d*sizeof(element) a multiple of 16
 * bytes, at most 4096 bytes (e.g. f32 d = 64, bf16 d = 256, 512 or 576).
 * Strides must be multiples of 16 bytes.
 * ------------------------------------------------------------------------ */
int hca_compress(const void* x, void* out, sa_dtype dtype,
                 int64_t B, int64_t H, int64_t n_tokens, int64_t d, int64_t blk,
                 int64_t x_sb, int64_t x_sh, int64_t x_st,
                 int64_t o_sb, int64_t o_sh, int64_t o_sn,
                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * hca_attention_fwd -- HCA attention, prefill or decode.
 *
 * [P1] §二.1: attention runs only over the compressed entries plus a window of
 * the most recent uncompressed tokens.  [P3] §架構創新 1: each query attends to
 * all compressed history entries and the short recent window; heads are 512
 * wide.  Readings where the pages are silent:
 *   - compressed entry j (tokens j*blk .. j*blk+blk-1) is visible to the query
 *     at position t iff (j+1)*blk - 1 <= t - window, i.e. the first
 *     max(0, floor((t-window+1)/blk)) entries (capped at the cache size);
 *   - raw tokens t-window < s <= t (s >= 0) form the window;
 *   - one softmax over both sets with logits scale*<q,k>; no sink/bias/gate.
 *
 * Head widths: d is the query/key width, d_v the value/output width (d_v = 0
 * means d_v = d).  [P3] §預訓練資料工程 item 3 (FlashMask-4) names a query/key
 * head of 576 with a value head of 512; that shape is supported beside the
 * plain 512/512 one.
 * PREFILL (mode = HCA_PREFILL), T = seq_len:
 *   q, k: [B,H,T,d];  v, o: [B,H,T,d_v];  k_c: [B,H,n_c,d], v_c: [B,H,n_c,d_v]
 *   with n_c = n_c_cap (normally T/blk, as written by hca_compress);  query
 *   row t sits at position t.
 * DECODE (mode = HCA_DECODE), one query per sequence:
 *   q: [B,H,d], o: [B,H,d_v];  k_c: [B,H,n_c_cap,d], v_c: [B,H,n_c_cap,d_v];
 *   k, v: the window ring [B,H,window,d] and [B,H,window,d_v] where position
 *   s lives in slot s mod window;  pos: device int64[B], the query's
 *   position (its own K/V is already in the ring).  pos values < 0 are
 *   treated as 0.
 * lse: optional (NULL to skip) fp32 [B,H,T] (prefill) or [B,H] (decode):
 *   natural-log normaliser of the scaled logits.
 * scale <= 0 selects 1/sqrt(d) (the query/key width).
 * Arithmetic: bf16 inputs, fp32 accumulation and softmax, probabilities
 * rounded to bf16 for the P*V product, output rounded (RNE) to the I/O dtype.
 * Supported (dtype, d, d_v): prefill (SA_F32, 64, 64), (SA_BF16, 512, 512),
 * (SA_BF16, 576, 512); decode (SA_BF16, 512, 512), (SA_BF16, 576, 512).
 * Workspace: DECODE may need split-K partials; query
 *   hca_attention_fwd_workspace_size() (0 for PREFILL).
 * ------------------------------------------------------------------------ */
typedef enum { HCA_PREFILL = 0, HCA_DECODE = 1 } hca_mode;

typedef struct {
  hca_mode mode;
  sa_dtype dtype;
  int64_t B, H, d;
  int64_t blk;      /* compression block (128 in the model)               */
  int64_t window;   /* uncompressed recent window (128)                   */
  int64_t seq_len;  /* PREFILL: T.  DECODE: ignored                       */
  int64_t n_c_cap;  /* number of entries in k_c / v_c                     */
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const void* k_c;
  const void* v_c;
  const int64_t* pos; /* DECODE only */
  void* o;
  float* lse;
  void* workspace;
  size_t workspace_bytes;
  int64_t d_v;      /* value/output width; 0 = d                          */
} hca_attention_args;

size_t hca_attention_fwd_workspace_size(const hca_attention_args* args);
int hca_attention_fwd(const hca_attention_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * hca_attention_bwd -- gradients of HCA prefill (an extension: the pages
 * train the HCA layers -- [P3] §預訓練資料工程 item 3, FlashMask-4 has a
 * backward pass -- but print no backward formula).
 *
 * The chain rule of hca_attention_fwd's definition (PREFILL, every row).  Per
 * query t with its keys (visible compressed entries, then the window), P the
 * forward's weights rebuilt from lse and D_t = sum_d d_o[t,d] * o[t,d]:
 *   dS = P * (d_o[t] . value - D_t)
 *   dq[t]      = scale * sum dS * key
 *   d(key)    += scale * dS * q[t]      (entry j -> dk_c[j], window s -> dk[s])
 *   d(value)  += P * d_o[t]             (dv_c, dv likewise)
 * When through_compress != 0, k_c and v_c are taken to be hca_compress(k)
 * and hca_compress(v) with the same blk, and dk, dv also receive the
 * compression path: every token s of a complete block j < n_c gets
 * dk_c[j] / blk and dv_c[j] / blk (the gradient of the whole layer with
 * respect to the raw k, v).  dk_c, dv_c are always the gradients with
 * respect to the compressed entries as inputs of their own.
 * q, k, v, o, d_o: [B,H,T,d] bf16 (o and lse as written by hca_attention_fwd
 * for the same inputs); k_c, v_c: [B,H,n_c,d] bf16; lse: fp32 [B,H,T]
 * (natural log), required.  Outputs, fp32, every element written: dq, dk,
 * dv [B,H,T,d]; dk_c, dv_c [B,H,n_c,d] (may be NULL when n_c == 0).
 * scale <= 0 selects 1/sqrt(d).  Arithmetic: bf16 inputs, fp32 products and
 * sums; P and dS rounded to bf16 for the dq, dk, dv products (as the forward
 * rounds P for its P*V product).  Results are deterministic (fixed-order
 * sums, no atomics).
 * Supported: SA_BF16, d = 512, n_c <= T / blk, T < 2^24.
 * Workspace: hca_attention_bwd_workspace_size() bytes, 16-byte aligned (the
 * P and dS blocks of every (32 queries, 32 keys) tile pair -- about 3.4 GB
 * at T = 32768, 64 heads -- and partial sums of the compressed entries).
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_UNSUPPORTED, SA_ERR_ALIGN,
 * SA_ERR_WORKSPACE, SA_ERR_HIP.
 * ------------------------------------------------------------------------ */
typedef struct {
  sa_dtype dtype;
  int64_t B, H, d;
  int64_t blk;       /* compression block                                   */
  int64_t window;    /* uncompressed recent window                          */
  int64_t seq_len;   /* T                                                   */
  int64_t n_c;       /* entries in k_c / v_c                                */
  int64_t through_compress; /* nonzero: add dk_c/blk, dv_c/blk into dk, dv */
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const void* k_c;
  const void* v_c;
  const void* o;
  const void* d_o;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* dk_c;
  float* dv_c;
  void* workspace;
  size_t workspace_bytes;
} hca_attention_bwd_args;

size_t hca_attention_bwd_workspace_size(const hca_attention_bwd_args* args);
int hca_attention_bwd(const hca_attention_bwd_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * hca_attention_fwd_noalloc -- hca_attention_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Same arguments, validation, kernels and results as hca_attention_fwd;
 * args->workspace and args->workspace_bytes are ignored.  DECODE calls keep
 * their split-K partials in a static device array of the library (8 MiB per
 * GPU, held until the process ends; every supported decode shape needs at
 * most about 6.3 MB of it); a call needing more returns SA_ERR_WORKSPACE.
 * PREFILL needs no scratch.  The call allocates nothing; its first call on a
 * device looks up the array's address there (hipGetSymbolAddress) and keeps
 * it.  Every call on one GPU shares that array and every decode call writes
 * all of the partials it reads, so nothing needs clearing between calls, but
 * calls that overlap on one GPU (concurrent streams or threads) race on it and
 * must be serialised by the caller.
 * ------------------------------------------------------------------------ */
int hca_attention_fwd_noalloc(const hca_attention_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * FP8 decode cache (an extension: the pages fix no cache format).
 *
 * [P1] §二.1 / [P3] §架構創新 1: HCA decode reads every visible compressed
 * entry and window token once, so its cost is the size of the cache.  Beside
 * bf16 the library offers OCP E4M3 codes ("fn" variant: exponent bias 7,
 * largest finite value 448, no infinities) with one fp32 scale per row.
 *
 * hca_quantize_fp8 -- encode bf16 rows.  For each row r of x [rows, d]:
 *   amax = max_j |x[r,j]|;  inv = 448 / amax (fp32; 0 when amax == 0);
 *   codes[r,j] = E4M3(x[r,j] * inv)   (fp32 product, round to nearest even);
 *   scales[r] = amax / 448            (fp32)
 * so that x[r,j] ~= scales[r] * value(codes[r,j]).  |x * inv| <= 448 holds,
 * so no code saturates.  NaN or infinite inputs give unspecified codes.
 * x: bf16 [rows, d]; codes: uint8 [rows, d]; scales: fp32 [rows].
 * Supported: d a multiple of 16, at most 4096.  rows == 0 does nothing.
 * ------------------------------------------------------------------------ */
int hca_quantize_fp8(const void* x, void* codes, float* scales, int64_t rows, int64_t d, hipStream_t stream);

/* ------------------------------------------------------------------------
 * hca_decode_fp8 -- HCA decode (one query per sequence, as HCA_DECODE of
 * hca_attention_fwd) over an FP8 cache: every K/V row is scale * E4M3 codes
 * as written by hca_quantize_fp8.
 *   q, o: bf16 [B,H,d];  k_c, v_c: codes [B,H,n_c_cap,d] with scales
 *   k_c_scale, v_c_scale: fp32 [B,H,n_c_cap];  k, v: the window ring, codes
 *   [B,H,window,d] (position s in slot s mod window) with scales k_scale,
 *   v_scale: fp32 [B,H,window];  pos: device int64[B];  lse: optional fp32
 *   [B,H] (natural log).  Visibility, scale and softmax as in HCA_DECODE.
 * Arithmetic: codes widened exactly to fp32; fp32 dot products multiplied by
 * the K row's scale, fp32 softmax, the V row's scale folded into the
 * probability, fp32 accumulation, output rounded (RNE) to bf16.
 * Supported: d = 512, n_c_cap >= 1.  Workspace as for hca_attention_fwd
 * DECODE: hca_decode_fp8_workspace_size() bytes.
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t B, H, d;
  int64_t blk;      /* compression block (128)                            */
  int64_t window;   /* window ring size (128)                             */
  int64_t n_c_cap;  /* number of entries in k_c / v_c                     */
  float scale;      /* <= 0 selects 1/sqrt(d)                             */
  const void* q;
  const void* k_c;
  const float* k_c_scale;
  const void* v_c;
  const float* v_c_scale;
  const void* k;
  const float* k_scale;
  const void* v;
  const float* v_scale;
  const int64_t* pos;
  void* o;
  float* lse;
  void* workspace;
  size_t workspace_bytes;
} hca_decode_fp8_args;

size_t hca_decode_fp8_workspace_size(const hca_decode_fp8_args* args);
int hca_decode_fp8(const hca_decode_fp8_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dsa_indexer_scores -- lightweight indexer of MLA-DSA.
 *
 * [P1] §二.1 and [P3] §架構創新 1: a lightweight indexer scores every history
 * position for each query.  The pages give no formula; this library computes
 *
 *   scores[b,i,s] = sum_h w[b,i,h] * max(0, <q_idx[b,i,h,:], k_idx[b,s,:]>)
 *
 * for every s <= p_i, p_i = q_pos[b] + i (q_pos == NULL: p_i = i).  Entries
 * with s > p_i are unspecified (they may or may not be written).
 * q_idx: [B,T,Hi,Di] bf16; k_idx: [B,S,Di] bf16 (one key per position, shared
 * by the indexer heads); w: [B,T,Hi] fp32; scores: [B,T,S] fp32.
 * Arithmetic: exact bf16 products accumulated in fp32, then fp32 ReLU,
 * weighting and head sum.
 * Supported: Di = 128, Hi = 4, S <= 2^24.
 * ------------------------------------------------------------------------ */
int dsa_indexer_scores(const void* q_idx, const void* k_idx, const float* w,
                       const int64_t* q_pos, float* scores,
                       int64_t B, int64_t T, int64_t S, int64_t Hi, int64_t Di,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * dsa_topk -- exact top-k selection per query row.
 *
 * [P1] §二.1 / [P3] §架構創新 1: only the top-K scoring positions are kept.
 * For row i of batch b the candidates are s <= p_i (p_i as above, capped at
 * S-1).  The selected set is the first min(k, p_i+1) candidates in the order
 * (score descending, position ascending): ties go to the lower position and
 * -0.0 ranks equal to +0.0.  idx[b,i,:] lists the selected positions in
 * ascending order, padded with -1.  NaN scores are unspecified.
 * scores: [B,T,S] fp32; idx: [B,T,k] int32.
 * Integer-exact: comparisons are on order-preserving 32-bit keys.
 * Supported: 1 <= k <= 2048; S < 2^31.
 * Workspace: dsa_topk_workspace_size() bytes (rows longer than the on-chip
 * limit use a multi-workgroup path that needs histograms in global memory).
 * ------------------------------------------------------------------------ */
size_t dsa_topk_workspace_size(int64_t B, int64_t T, int64_t S, int64_t k);
int dsa_topk(const float* scores, const int64_t* q_pos, int32_t* idx,
             int64_t B, int64_t T, int64_t S, int64_t k,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * CSA variant: indexer and top-k over compressed entries.
 *
 * The pages contrast DSA with CSA, which compresses the history by 4x and
 * keeps the top-k of the compressed entries.  Library reading: indexer keys,
 * K and V are block means over `ratio` consecutive tokens (hca_compress with
 * blk = ratio), and the query at token position p_i = q_pos[b] + i (or i) sees
 * the entries s < floor((p_i + 1) / ratio) -- the blocks that end at or
 * before the query.  csa_indexer_scores and csa_topk are dsa_indexer_scores
 * and dsa_topk with that rule (S = number of entries; ratio = 1 is DSA); the
 * selected entries go to dsa_sparse_attention_fwd with the compressed K, V.
 * Supported: as the DSA calls, 1 <= ratio <= 2^20.
 * ------------------------------------------------------------------------ */
int csa_indexer_scores(const void* q_idx, const void* k_idx, const float* w,
                       const int64_t* q_pos, float* scores,
                       int64_t B, int64_t T, int64_t S, int64_t Hi, int64_t Di, int64_t ratio,
                       hipStream_t stream);
int csa_topk(const float* scores, const int64_t* q_pos, int32_t* idx,
             int64_t B, int64_t T, int64_t S, int64_t k, int64_t ratio,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dsa_indexer_topk -- fused indexer and top-k (an extra export beside the two
 * separate calls, which define its result).
 *
 * [P1] §二.1, [P3] §架構創新 1: the indexer scores every history position and
 * only the top-k positions are kept.  This call writes exactly the idx that
 * dsa_indexer_scores followed by dsa_topk would write for the same inputs
 * (the same fp32 scores, score descending then position ascending, ascending
 * output padded with -1) without writing the [B,T,S] score matrix: a sample
 * of every 16th position sets a per-row threshold, the indexer keeps only the
 * (key, position) pairs at or above it, and an exact selection runs over
 * those.  Rows where the sample misjudges the threshold (fewer than k or more
 * than 4096 candidates) are recomputed exactly by the separate kernels inside
 * the call, so the result never depends on the sample.
 * q_idx: [B,T,Hi,Di] bf16; k_idx: [B,S,Di] bf16; w: [B,T,Hi] fp32;
 * q_pos: device int64[B] or NULL (as for dsa_indexer_scores);
 * idx: [B,T,k] int32.
 * Decode-shaped calls with long rows (T <= 4, S > 32768) take the register-
 * operand decode indexer: it scores every 64th key in place for the
 * threshold (rank k/64 plus the same margin), then writes the candidates of
 * each chunk of 128 positions in position order; a compaction packs them
 * and one workgroup per row selects over them (at most 8192 candidates;
 * otherwise the row is recomputed exactly from its full scores inside the
 * call).
 * force_fallback: 0 normally; nonzero sends every row with more than k
 * candidates through the exact recomputation (a test of that path).
 * Supported: Hi = 4, Di = 128, 1 <= k <= 2048, and S <= 32768 or (T <= 4 and
 * S <= 2^24).
 * Workspace: dsa_indexer_topk_workspace_size() bytes (it includes room for
 * the candidates and for the recomputed rows' scores).
 * ------------------------------------------------------------------------ */
size_t dsa_indexer_topk_workspace_size(int64_t B, int64_t T, int64_t S, int64_t k);
int dsa_indexer_topk(const void* q_idx, const void* k_idx, const float* w, const int64_t* q_pos, int32_t* idx,
                     int64_t B, int64_t T, int64_t S, int64_t Hi, int64_t Di, int64_t k,
                     int64_t force_fallback, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dsa_sparse_attention_fwd -- exact attention over the selected positions.
 *
 * [P1] §二.1 / [P3] §架構創新 1: core attention runs only on the top-K
 * positions, so its per-query cost is constant in the context length; MLA
 * heads are 256 wide.  Multi-query layout: all Hq query heads share one K and
 * one V row per position.
 *
 *   o[b,i,h,:] = sum_{s in idx[b,i]} softmax_s(scale*<q[b,i,h], k[b,s]>) * v[b,s,:]
 *
 * Entries of idx that are negative or >= S are skipped.  A row with no valid
 * entry yields o = 0 and lse = -inf.
 * q, o: [B,T,Hq,D] bf16; k, v: [B,S,D] bf16 (v == k is allowed);
 * idx: [B,T,kk] int32; lse: optional fp32 [B,T,Hq].  scale <= 0 -> 1/sqrt(D).
 * Arithmetic: bf16 inputs, fp32 accumulation and softmax, probabilities
 * rounded to bf16 for the P*V product, output rounded (RNE) to bf16.
 * Supported: SA_BF16, D = 256, Hq = 64, 1 <= kk <= 2048, S <= 2^23.
 * Workspace: calls with few tokens (decode) split each token's index list
 * over several workgroups and need dsa_sparse_attention_fwd_workspace_size()
 * bytes of scratch for the partial results (0 for prefill-sized calls).
 * ------------------------------------------------------------------------ */
size_t dsa_sparse_attention_fwd_workspace_size(int64_t B, int64_t T, int64_t Hq, int64_t D, int64_t kk);
int dsa_sparse_attention_fwd(const void* q, const void* k, const void* v,
                             const int32_t* idx, void* o, float* lse, sa_dtype dtype,
                             int64_t B, int64_t T, int64_t S, int64_t Hq, int64_t D,
                             int64_t kk, float scale, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * dsa_sparse_attention_bwd -- gradients of dsa_sparse_attention_fwd.
 *
 * [P1] §二.1 / [P3] §架構創新 1 define the forward (exact attention over the
 * selected positions); the pages train these layers but print no backward
 * formula, so this is the chain rule of the forward's definition, entry by
 * entry of idx (an entry listed twice counts twice; skipped entries and the
 * selection itself get no gradient).  With P the forward's weights over the
 * row's entries, rebuilt from lse, and D_h = sum_d d_o[h,d] * o[h,d]:
 *   dq[b,i,h]   = scale * sum_j P_hj (d_o[h].v[s_j] - D_h) k[s_j]
 *   dk[b,s_j]  += scale * sum_h P_hj (d_o[h].v[s_j] - D_h) q[b,i,h]
 *   dv[b,s_j]  += sum_h P_hj d_o[b,i,h]
 * q, o, d_o: [B,T,Hq,D] bf16 (o and lse as written by the forward call with
 * the same q, k, v, idx, scale); k, v: [B,S,D] bf16; idx: [B,T,kk] int32;
 * lse: fp32 [B,T,Hq], required.  Outputs (fp32, every element written): dq
 * [B,T,Hq,D]; dk, dv [B,S,D].  scale <= 0 -> 1/sqrt(D).
 * Arithmetic: bf16 inputs, fp32 products and sums; P and dS rounded to bf16
 * for the dq, dk, dv products (as the forward rounds P for its P*V
 * product), and each entry's dk and dv rows (sums over the heads) rounded to
 * bf16 before they are added per position in fp32.  Deterministic: the
 * entries of a position are added in ascending (token, entry) order, chunk
 * after chunk, with no floating-point atomics.
 * Supported: SA_BF16, D = 256, Hq = 64, 1 <= kk <= 2048, S <= 2^23,
 * B*S < 2^32 - 1.
 * Workspace: dsa_sparse_attention_bwd_workspace_size(B, T, S, kk) bytes,
 * 16-byte aligned (for chunks of up to 2048 tokens: the P and dS blocks,
 * each entry's dk / dv rows and two inverse-index buffers: about 5.4 GB at
 * kk = 2048).
 * Streams: each chunk's inverse index (integer work that depends only on
 * idx) is built on a second stream of the calling thread and device
 * (created on first use, default priority, kept for the process), forked
 * from `stream` after the work enqueued before the call and joined back
 * before the reduction that reads it, so that it overlaps the previous
 * chunks' attention passes.  If the current device is not `stream`'s, or
 * the stream or its events cannot be created, everything runs on `stream`.
 * Errors: SA_ERR_NULL (any pointer NULL), SA_ERR_SHAPE, SA_ERR_UNSUPPORTED,
 * SA_ERR_ALIGN (every pointer 16-byte aligned), SA_ERR_WORKSPACE, SA_ERR_HIP.
 * ------------------------------------------------------------------------ */
size_t dsa_sparse_attention_bwd_workspace_size(int64_t B, int64_t T, int64_t S, int64_t kk);
int dsa_sparse_attention_bwd(const void* q, const void* k, const void* v, const int32_t* idx,
                             const void* o, const float* lse, const void* d_o,
                             float* dq, float* dk, float* dv, sa_dtype dtype,
                             int64_t B, int64_t T, int64_t S, int64_t Hq, int64_t D, int64_t kk,
                             float scale, void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_HCA_H */

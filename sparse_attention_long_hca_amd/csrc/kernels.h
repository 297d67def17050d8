// Kernel parameter blocks and host launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

// ---- hca_compress ----------------------------------------------------------
struct HcaCompressParams {
  const void* x;
  void* out;
  int64_t B, H, n_out, d, blk;
  int64_t x_sb, x_sh, x_st;
  int64_t o_sb, o_sh, o_sn;
};
hipError_t launch_hca_compress(const HcaCompressParams& p, int dtype, hipStream_t stream);

// ---- hca_attention_fwd, prefill ---------------------------------------------
struct HcaPrefillParams {
  const void* q;
  const void* k;
  const void* v;
  const void* kc;
  const void* vc;
  void* o;
  float* lse;
  int64_t B, H, T, Nc, blk, window;
  float scale_log2;
  int64_t n_qtiles;
};
// d: query/key width, dv: value/output width.
hipError_t launch_hca_prefill(const HcaPrefillParams& p, int dtype, int d, int dv, hipStream_t stream);

// ---- hca_attention_fwd, decode ----------------------------------------------
struct HcaDecodeParams {
  const void* q;
  const void* kc;
  const void* vc;
  const void* rk;  // window ring [B,H,window,d]
  const void* rv;
  // FP8 cache only: one fp32 scale per row of kc, vc ([B,H,Ncap]), rk, rv ([B,H,window]).
  const float* kc_scale;
  const float* vc_scale;
  const float* rk_scale;
  const float* rv_scale;
  const int64_t* pos;
  void* o;
  float* lse;
  float* part_o;    // [B*H*nsplit, d]  (nsplit > 1)
  float* part_lse;  // [B*H*nsplit]     log2 units
  int64_t B, H, Ncap, blk, window;
  float scale_log2;
  int64_t nsplit, keys_per_split;
};
int64_t hca_decode_nsplit(int64_t BH, int64_t max_keys);
size_t hca_decode_workspace_bytes(int64_t BH, int64_t nsplit, int64_t d);
// cache: 1 = bf16 rows, 2 = E4M3 codes with per-row scales.
// d: query/key width (512 or 576), dv: value/output width (512).
hipError_t launch_hca_decode(const HcaDecodeParams& p, int cache, int d, int dv, hipStream_t stream);

// ---- hca_attention_bwd (prefill) --------------------------------------------
// Stored weights: for every (32-query tile tq, key tile) pair of the forward's
// key stream, the 32 x 32 blocks of P and dS (bf16, [key][query] with the
// query columns permuted as hca_bwd_col()), slot jt < nct for compressed
// entry tile jt, slot nct + u for raw tile tq - nr + 1 + u.
struct HcaBwdParams {
  const void* q;   // [B,H,T,512] bf16
  const void* k;
  const void* v;
  const void* kc;  // [B,H,Nc,512]
  const void* vc;
  const void* o;   // forward output
  const void* dout;
  const float* lse;  // [B,H,T] natural log
  float* dq;   // [B,H,T,512]
  float* dk;
  float* dv;
  float* dkc;  // [B,H,Nc,512]
  float* dvc;
  int64_t B, H, T, Nc, blk, window;
  int64_t spread;  // nonzero: dk, dv also get dkc/blk, dvc/blk (the block mean's gradient)
  float scale, scale_log2;
  uint16_t* blocks;  // [B*H, ntq, nslot, 2, 32, 32] + one trash block pair
  float* part;       // [nchunk, B*H, Nc, 2, 512] compressed partial dK, dV
  int64_t ntq, nct, nr, nslot, nchunk;
};
size_t hca_bwd_ws_bytes(int64_t B, int64_t H, int64_t T, int64_t Nc, int64_t window);
hipError_t launch_hca_bwd(HcaBwdParams p, hipStream_t stream);

// ---- hca_quantize_fp8 -------------------------------------------------------
struct HcaQuantParams {
  const void* x;  // [rows, d] bf16
  void* codes;    // [rows, d] E4M3
  float* scales;  // [rows]
  int64_t rows, d;
};
hipError_t launch_hca_quantize_fp8(const HcaQuantParams& p, hipStream_t stream);

// ---- dsa_indexer_scores -----------------------------------------------------
struct DsaIndexerParams {
  const void* q;   // [B,T,Hi,Di] bf16
  const void* k;   // [B,S,Di] bf16
  const float* w;  // [B,T,Hi]
  const int64_t* q_pos;
  float* scores;  // [B,T,S]
  int64_t B, T, S;
  int64_t ratio;  // keys are entries of `ratio` tokens: row i sees keys s < (q_pos + i + 1) / ratio
  // Candidate mode (cand != NULL; ratio 1): no scores are stored.  Positions
  // are worked in chunks of dsa_indexer_chunk(T); for every row with more
  // than topk visible positions, the workgroup of chunk c writes (order-
  // preserving key, position) of each score whose key is >= thresh[row] to
  // cand[row*cand_pitch + c*chunk ..] (room for the whole chunk), their
  // number to cnt[row*n_chunks + c] (n_chunks = ceil(S / chunk)), and after
  // an odd number a pad entry (0, 0) (no score has key 0).  cand_pitch is S
  // rounded up to even, so the pad after an all-candidate last chunk of odd
  // length stays inside the row.  Rows keeping every visible position write
  // count 0.  Every chunk holding a visible position of a row writes that
  // row's count.
  const uint32_t* thresh;
  uint32_t* cnt;
  uint2* cand;
  int64_t cand_pitch;
  // Decode candidate mode (dec_cand != 0, T <= 4): the register-operand decode
  // kernel writes each row's candidates per chunk of dsa_indexer_dec_chunk()
  // positions in ascending position order (cand, cand_pitch, thresh, topk as
  // above, no pad entries); the count of chunk c goes to
  // cnt[row * cnt_pitch + c], cnt_pitch = n_chunks rounded up to a multiple
  // of 8 (n_chunks = ceil(S / dsa_indexer_dec_chunk())).
  int dec_cand;
  int64_t topk;
  // Decode sampled-key mode (dec_sample != 0, T <= 4, keys16 set): position
  // s of S (the sample count) is key row s*ratio + ratio - 1 of a k with
  // k_rows rows per batch, visible under the ratio rule; keys16 as below but
  // with rows pitched at S rounded up to a multiple of 8.
  int dec_sample;
  int64_t k_rows;
  // Decode row filter (dec_filter != 0, T <= 4, row_flag and any_flag set):
  // the scores of the batches holding a flagged row, from a bounded grid.
  int dec_filter;
  // Key mode (keys16 != NULL): instead of scores, keys16[b,i,s] (same layout)
  // receives the top 16 bits of the score's order-preserving key.
  uint16_t* keys16;
  // Row filter (row_flag != NULL): nothing runs unless *any_flag != 0, and a
  // workgroup runs only if one of its rows has row_flag[row] != 0.
  const uint32_t* row_flag;
  const uint32_t* any_flag;
};
hipError_t launch_dsa_indexer(const DsaIndexerParams& p, hipStream_t stream);
int64_t dsa_indexer_chunk(int64_t T);  // positions per workgroup for T queries
int64_t dsa_indexer_dec_chunk();       // positions per workgroup of the decode kernel

// ---- dsa_topk ---------------------------------------------------------------
struct DsaTopkParams {
  const float* scores;
  const int64_t* q_pos;
  int32_t* idx;
  int64_t B, T, S, k;
  void* ws;
  int64_t ratio;  // as in DsaIndexerParams
  // Row filter as in DsaIndexerParams (rows of at most 32768 positions).
  const uint32_t* row_flag;
  const uint32_t* any_flag;
};
size_t dsa_topk_ws_bytes(int64_t B, int64_t T, int64_t S, int64_t k);
hipError_t launch_dsa_topk(const DsaTopkParams& p, hipStream_t stream);

// ---- dsa_indexer_topk (fused) -------------------------------------------------
struct DsaIndexerTopkParams {
  const void* q;   // [B,T,4,128] bf16
  const void* k;   // [B,S,128] bf16
  const float* w;  // [B,T,4]
  const int64_t* q_pos;
  int32_t* idx;    // [B,T,topk]
  int64_t B, T, S, topk;
  void* ws;
  int force_fallback;
};
size_t dsa_indexer_topk_ws_bytes(int64_t B, int64_t T, int64_t S, int64_t k);
hipError_t launch_dsa_indexer_topk(const DsaIndexerTopkParams& p, hipStream_t stream);

// ---- dsa_sparse_attention_fwd -----------------------------------------------
struct DsaSparseParams {
  const void* q;  // [B,T,Hq,D]
  const void* k;  // [B,S,D]
  const void* v;
  const int32_t* idx;  // [B,T,kk]
  void* o;
  float* lse;
  float* part_o;    // [B*T*nsplit, Hq, D] fp32 (nsplit > 1)
  float* part_lse;  // [B*T*nsplit, Hq]    log2 units
  int64_t B, T, S, kk;
  float scale_log2;
  int64_t nsplit, tiles_per_split;
};
int64_t dsa_sparse_nsplit(int64_t BT, int64_t kk);
size_t dsa_sparse_workspace_bytes(int64_t BT, int64_t nsplit, int64_t hq, int64_t d);
hipError_t launch_dsa_sparse(const DsaSparseParams& p, int d, int hq, hipStream_t stream);

// ---- dsa_sparse_bwd -----------------------------------------------------------
struct DsaSparseBwdParams {
  const void* q;  // [B,T,64,256] bf16
  const void* k;  // [B,S,256]
  const void* v;
  const int32_t* idx;  // [B,T,kk]
  const void* o;       // forward output [B,T,64,256] bf16
  const float* lse;    // forward log-sum-exp [B,T,64] (natural log)
  const void* dout;    // [B,T,64,256] bf16
  float* dq;           // [B,T,64,256]
  float* dk;           // [B,S,256] (zeroed, then accumulated chunk by chunk)
  float* dv;
  int64_t B, T, S, kk;
  float scale, scale_log2;
  void* ws;            // dsa_sparse_bwd_ws_bytes()
  // Set by the launcher per chunk of tokens [tok0, tok0 + ntok): the chunk's
  // P / dS blocks, per-entry dK / dV rows (bf16, entry e = (token - tok0) * kk
  // + j), and the inverse index (segment of key b*S + s: list[off[key] ..
  // off[key + 1]), entry ids in arbitrary order).
  int64_t tok0, ntok;
  uint16_t* blocks;  // [ntok, kk/32 tiles, 2 tensors, 2 head halves, 32, 32]
  uint16_t* gk;      // [ntok * kk, 256]
  uint16_t* gv;
  uint32_t* list;
  const uint32_t* off;
};
size_t dsa_sparse_bwd_ws_bytes(int64_t B, int64_t T, int64_t S, int64_t kk);
hipError_t launch_dsa_sparse_bwd(DsaSparseBwdParams p, hipStream_t stream);

}  // namespace sa

/*
 * libmla -- Multi-Head Latent Attention (MLA) decode with weight absorption on
 * AMD Instinct MI355X (gfx950).  Plain C ABI: host or device pointers and sizes,
 * no framework types.
 *
 * What the library computes (sources are web pages, cited by page and section):
 *
 *   [MLA explainer]    xxmr.cn/news/206254, sections "MLA的计算过程" (stage 2A:
 *                      explicit decompression; stage 2B: absorbed inference) and
 *                      "MLA的实现" (RoPE module, forward_inference_absorbed).
 *   [MLA architecture] intelliparadigm.com, "MLA架构：低秩注意力机制优化LLM显存与计算效率",
 *                      section 1 (128 heads; qk head = 128 no-RoPE + 64 RoPE;
 *                      576 cached values per token), 3.1 (absorption),
 *                      3.2 (latent cache + shared RoPE key cache), 4.2 (pre-allocated
 *                      cache; RoPE fused with the cache update).
 *   [MLA deep dive]    mlqm.cn/news/500296, 2.3 (weight absorption), 5.1 (paged cache).
 *
 * One decode/prefill step for a batch of sequences is four calls on one stream:
 *
 *   mla_absorb_q      q_lat[:, :, 0:d_c]  = W_UK^T q_nope            (per head)
 *   mla_append_cache  pool rows <- [c_kv | RoPE(k_pe)];  q_lat[:, :, d_c:] = RoPE(q_pe)
 *   mla_decode        o_lat = softmax(scale * q_lat . rows^T) . c_kv  (paged, split-KV)
 *   mla_out_proj      out = W_UV o_lat                                 (per head)
 *
 * Full per-head K and V are never formed.  The result equals explicit-decompression
 * attention with scale 1/sqrt(d_nope + d_rope) up to rounding ([MLA architecture]
 * 3.1: absorption is associativity of the matrix products).
 *
 * Supported shapes (anything else returns MLA_ERR_UNSUPPORTED):
 *   bf16: num_heads=128, d_latent=512, d_rope=64, d_nope=128, d_v=128, block_size=64
 *         (DeepSeek-V3 shapes; bf16 storage, fp32 accumulation)
 *   f32 : num_heads in [1, 128], d_latent in {64, 128, 256, 512}, d_rope in {16, 32, 64},
 *         d_nope, d_v in [1, 256], block_size=64 (all-fp32 test mode)
 *
 * Layouts: row-major, last index contiguous.  T = number of query (new) tokens.
 *   q_nope [T][H][d_nope]      q_pe  [T][H][d_rope]     q_lat [T][H][d_latent + d_rope]
 *   c_kv   [T][d_latent]       k_pe  [T][d_rope]
 *   w_uk   [H][d_nope][d_latent]     w_uv [H][d_v][d_latent]
 *   kv_pool [num_blocks][block_size][d_latent + d_rope]   row = [c_kv | RoPE(k_pe)]
 *   o_lat  [T][H][d_latent]    out   [T][H][d_v]  (always fp32)
 *   block_table [num_seqs][max_blocks_per_seq] int32, physical block ids, -1 = unused
 * Element type of every "void*" tensor is the config dtype (bf16 or fp32).
 * Device tensors must be 16-byte aligned.
 *
 * Ownership and execution: every buffer is owned by the caller.  The library never
 * allocates device memory and keeps no device state.  Calls enqueue kernels on the
 * given stream (a hipStream_t; NULL = the default stream), return without waiting,
 * and never synchronise the device.  Calls are reentrant.
 *
 * Errors: a call validates everything it can see on the host and returns a status
 * without launching anything when a check fails.  Device-resident indices
 * (positions, sequence ids, block ids) are checked inside the kernels: an entry that
 * is out of range is skipped (nothing is written for it) and, if the caller passes
 * an error word, bit flags are OR-ed into it (see MLA_DEVERR_*).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer, bad length */
  MLA_ERR_UNSUPPORTED = 2, /* dims / dtype combination not built */
  MLA_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  MLA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Bits OR-ed into the optional device error word by the kernels. */
#define MLA_DEVERR_POSITION 1u /* position < 0 or >= max_pos */
#define MLA_DEVERR_SEQ 2u      /* sequence id < 0 or >= num_seqs */
#define MLA_DEVERR_BLOCK 4u    /* block-table entry < 0 or >= num_pool_blocks */
#define MLA_DEVERR_LENGTH 8u   /* device lengths disagree with the host copies */

/* Largest token count one mla_absorb_q / mla_out_proj call accepts. */
#define MLA_MAX_PROJ_TOKENS 262144

typedef struct {
  int32_t num_heads;   /* H */
  int32_t d_latent;    /* d_c: latent (compressed KV) width, 512 for V3 */
  int32_t d_rope;      /* d_r: decoupled RoPE width, 64 for V3 (even) */
  int32_t d_nope;      /* d_n: no-RoPE query/key width per head, 128 for V3 */
  int32_t d_v;         /* value width per head, 128 for V3 */
  int32_t block_size;  /* tokens per cache block, 64 */
  float softmax_scale; /* 1/sqrt(d_nope + d_rope) ([MLA explainer] "MLA的实现") */
  int32_t dtype;       /* mla_dtype */
} mla_config;

/* Human-readable name of a status code (static string). */
const char* mla_status_string(mla_status s);

/* Host helper.  RoPE tables ([MLA explainer] "MLA的实现", RoPE module: inverse
 * frequency theta^(-2i/d_rope), rotate-half pairing): for p < max_pos and
 * i < d_rope/2, cos_host[p*(d_rope/2)+i] = cos(p * theta^(-2i/d_rope)) and likewise
 * sin, evaluated in double precision and rounded once to float.  Host memory of
 * max_pos*d_rope/2 floats each, owned by the caller; upload it for
 * mla_append_cache.  INVALID_ARG for null pointers, max_pos < 1 or odd d_rope. */
mla_status mla_rope_table(float* cos_host, float* sin_host, int32_t max_pos,
                          int32_t d_rope, double theta);

/* Query absorption ([MLA explainer] stage 2B / forward_inference_absorbed: the
 * no-RoPE query is mapped through W_UK into the latent space; [MLA deep dive] 2.3):
 *   q_lat[t][h][c] = round( sum_d q_nope[t][h][d] * w_uk[h][d][c] ),  c < d_latent
 * fp32 accumulation, rounded to the storage dtype (nearest-even for bf16).  Writes
 * columns [0, d_latent) of q_lat only; the RoPE columns are written by
 * mla_append_cache.  T = 0 is a no-op; T > MLA_MAX_PROJ_TOKENS is INVALID_ARG.
 * Device pointers. */
mla_status mla_absorb_q(const mla_config* cfg, int32_t T, const void* q_nope,
                        const void* w_uk, void* q_lat, void* stream);

/* Fused RoPE + latent-cache append ([MLA architecture] 4.2: RoPE fused with the
 * cache update; 3.2: cache = latent part + shared RoPE key).  For each token t
 * (sequence s = token_seq[t], position p = positions[t]):
 *   row = block_table[s][p / block_size] * block_size + p % block_size
 *   kv_pool[row][0:d_c]    = c_kv[t]                         (copied bit for bit)
 *   kv_pool[row][d_c:d_c+d_r] = RoPE_p(k_pe[t])
 *   q_lat[t][h][d_c:d_c+d_r]  = RoPE_p(q_pe[t][h])  for every head (if q_pe != NULL)
 * RoPE_p(x): with half = d_r/2, c = rope_cos[p][i], s = rope_sin[p][i], i < half,
 *   y[i] = x[i]*c - x[i+half]*s,  y[i+half] = x[i+half]*c + x[i]*s,
 * computed in fp32 with every product and sum rounded to fp32 (no fused
 * multiply-add), then rounded to the storage dtype (nearest-even).  The pool row
 * is therefore bit-exact and independent of the device.
 * rope_cos / rope_sin: device [max_pos][d_r/2] fp32 (e.g. from mla_rope_table).
 * q_pe / q_lat may both be NULL (cache-only append, e.g. filling history).
 * Entries with an out-of-range position, sequence id or block id are skipped and
 * flagged in *dev_error (optional, device uint32, may be NULL).  Tokens that map
 * to the same row race; the caller must not do that.  Device pointers. */
mla_status mla_append_cache(const mla_config* cfg, int32_t T, const void* c_kv,
                            const void* k_pe, const void* q_pe, const int32_t* token_seq,
                            const int32_t* positions, const int32_t* block_table,
                            int32_t num_seqs, int32_t max_blocks_per_seq,
                            int64_t num_pool_blocks, const float* rope_cos,
                            const float* rope_sin, int32_t max_pos, void* kv_pool,
                            void* q_lat, uint32_t* dev_error, void* stream);

/* Workspace bytes that mla_decode needs for this batch (split-KV partial results).
 * Query tokens of sequence b are q_start[b] .. q_start[b+1]-1; the last of them is
 * the token at position kv_lens[b]-1.  num_workgroups = 0 lets the library choose
 * the split plan; a positive value forces that many KV ranges (used to check
 * that results do not depend on the split).  Host arrays.  INVALID_ARG when a
 * length is < 1, a sequence has more query tokens than kv_len, or q_start is not
 * non-decreasing from 0. */
mla_status mla_decode_workspace_size(const mla_config* cfg, int32_t num_seqs,
                                     const int32_t* q_start_host,
                                     const int32_t* kv_lens_host, int32_t causal,
                                     int32_t num_workgroups, size_t* bytes);

/* Absorbed latent attention over the paged cache ([MLA explainer] stage 2B and
 * forward_inference_absorbed: latent score plus RoPE score, scaled, softmax,
 * weighted sum of the cached latents; "MLA的常见问题" Q4: 512 + 64 asymmetric
 * contraction).  For query token t of sequence b at position P = kv_lens[b] -
 * (q_start[b+1]-q_start[b]) + j (j = t - q_start[b]) and every head h:
 *   s_u = softmax_scale * sum_{k < d_c+d_r} q_lat[t][h][k] * row_u[k]
 *   for cached positions u < kv_lens[b] (u <= P when causal != 0)
 *   o_lat[t][h][c] = round( sum_u softmax(s)_u * row_u[c] ),  c < d_c
 * Exact max-subtracted softmax, fp32 arithmetic, one rounding of o_lat to the
 * storage dtype (split-KV partials are stored normalised in the storage dtype
 * with an fp32 log-sum-exp and merged in fp32, in a fixed order: results are
 * run-to-run bitwise deterministic for a given split plan).
 * q_start, kv_lens, block_table: device; q_start_host, kv_lens_host: the same
 * values on the host (used to plan the split without a device sync).
 * workspace: device, at least mla_decode_workspace_size() bytes (may be NULL if
 * that is 0).  dev_error: optional device word for MLA_DEVERR_* flags (a bad block
 * id is skipped; the affected outputs are then undefined but no memory outside the
 * given buffers is touched).  UNSUPPORTED when the split plan has 2^31 or more
 * (token, block) units or the block table has 2^31 or more entries. */
mla_status mla_decode(const mla_config* cfg, int32_t num_seqs, const int32_t* q_start,
                      const int32_t* kv_lens, const int32_t* q_start_host,
                      const int32_t* kv_lens_host, const int32_t* block_table,
                      int32_t max_blocks_per_seq, int64_t num_pool_blocks,
                      const void* q_lat, const void* kv_pool, int32_t causal,
                      int32_t num_workgroups, void* workspace, size_t workspace_bytes,
                      void* o_lat, uint32_t* dev_error, void* stream);

/* Bytes of device scratch that mla_decode_noalloc owns on each device: enough
 * for the default split plan of the DeepSeek-V3 bf16 shapes on a 256-CU MI355X
 * (2 x 256 partial slots of [128][512] bf16 plus their fp32 log-sum-exp). */
#define MLA_DECODE_SCRATCH_BYTES ((size_t)65 << 20)

/* mla_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, math, plan, kernels and results as
 * mla_decode (bitwise, for the same num_workgroups); the split partials go to a
 * library-owned device array of MLA_DECODE_SCRATCH_BYTES per device (held until
 * the process ends) instead of a workspace.  Allocates nothing: no hipMalloc,
 * hipFree or allocating library call.  MLA_ERR_WORKSPACE when the plan needs
 * more than MLA_DECODE_SCRATCH_BYTES (mla_decode_workspace_size tells; force a
 * smaller num_workgroups).  Every call on one device shares that device's array:
 * calls that overlap on one device (other streams, other host threads) race and
 * must be serialised by the caller.  Nothing in the array needs to start at
 * zero: each partial the merge reads is written earlier in the same call. */
mla_status mla_decode_noalloc(const mla_config* cfg, int32_t num_seqs, const int32_t* q_start,
                              const int32_t* kv_lens, const int32_t* q_start_host,
                              const int32_t* kv_lens_host, const int32_t* block_table,
                              int32_t max_blocks_per_seq, int64_t num_pool_blocks,
                              const void* q_lat, const void* kv_pool, int32_t causal,
                              int32_t num_workgroups, void* o_lat, uint32_t* dev_error,
                              void* stream);

/* Per-head value up-projection ([MLA explainer] forward_inference_absorbed: the
 * attended latent is mapped through W_UV per head, V is never formed):
 *   out[t][h][v] = sum_c o_lat[t][h][c] * w_uv[h][v][c]   (fp32 accumulate, fp32 out)
 * T = 0 is a no-op; T > MLA_MAX_PROJ_TOKENS is INVALID_ARG.  Device pointers. */
mla_status mla_out_proj(const mla_config* cfg, int32_t T, const void* o_lat,
                        const void* w_uv, float* out, void* stream);

/* ---------------------------------------------------------------------------
 * Weight-level absorption: the query-side and output-side fused weights.
 * --------------------------------------------------------------------------- */

/* Largest model width (and compressed-query width) the fused-weight calls and
 * mla_kv_down_append accept. */
#define MLA_MAX_D_MODEL 65536

/* Query absorption with the fused weight ([MLA explainer]
 * forward_inference_absorbed, w_q_absorbed = W_UQ^T W_UK per head: the
 * compressed query c_q goes straight into the latent space):
 *   q_lat[t][h][c] = round( sum_j c_q[t][j] * w_kq[h][j][c] ),  c < d_latent
 * c_q [T][d_cq], w_kq [H][d_cq][d_latent] (W_KQ[h][j][c] = sum_d W_UQ[h][d][j] *
 * W_UK[h][d][c], prepared by the caller), q_lat as mla_absorb_q (columns
 * [0, d_latent) written).  fp32 accumulation, one rounding (nearest even).
 * Only the DeepSeek-V3 bf16 configuration (UNSUPPORTED otherwise); d_cq a
 * positive multiple of 128, at most MLA_MAX_D_MODEL; T as mla_absorb_q
 * (INVALID_ARG otherwise).  Device pointers, 16-byte aligned. */
mla_status mla_absorb_q_fused(const mla_config* cfg, int32_t T, int32_t d_cq, const void* c_q,
                              const void* w_kq, void* q_lat, void* stream);

/* Workspace bytes for mla_out_proj_fused: fp32 partial sums of 16 ranges of
 * the contraction, 16 * T * d_model * 4.  Same argument checks as the call. */
mla_status mla_out_proj_fused_workspace_size(const mla_config* cfg, int32_t T,
                                             int32_t d_model, size_t* bytes);

/* Output projection with the fused weight ([MLA explainer]
 * forward_inference_absorbed, w_o_absorbed = W_UV^T W_O per head: the attended
 * latent goes straight to the model width, summed over the heads):
 *   out[t][m] = sum_h sum_c o_lat[t][h][c] * w_ov[h][c][m]     (fp32 out)
 * o_lat [T][H][d_latent], w_ov [H][d_latent][d_model] (W_OV[h][c][m] =
 * sum_v W_UV[h][v][c] * W_O[m][h][v], prepared by the caller), out [T][d_model].
 * The contraction over (h, c) is split into 16 ranges whose fp32 partial sums
 * go to the workspace and are added in a fixed order (results are run-to-run
 * bitwise deterministic).  workspace: device, at least
 * mla_out_proj_fused_workspace_size() bytes (WORKSPACE otherwise).  Only the
 * DeepSeek-V3 bf16 configuration; d_model a positive multiple of 256, at most
 * MLA_MAX_D_MODEL; T as mla_out_proj.  Device pointers, 16-byte aligned. */
mla_status mla_out_proj_fused(const mla_config* cfg, int32_t T, int32_t d_model,
                              const void* o_lat, const void* w_ov, float* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Non-absorbed (explicit-decompression) attention, for prefill.
 * --------------------------------------------------------------------------- */

/* Workspace bytes for mla_prefill_decompressed: the per-head decompressed keys
 * and values of every cached row of the batch (each sequence's rows rounded up
 * to a multiple of 64): 2 * H * R * 128 * 2 bytes for R rounded rows, plus a
 * small header.  Host arrays; the same length checks as the call. */
mla_status mla_prefill_workspace_size(const mla_config* cfg, int32_t num_seqs,
                                      const int32_t* q_start_host,
                                      const int32_t* kv_lens_host, size_t* bytes);

/* Attention with explicitly decompressed keys and values ([MLA explainer]
 * forward_training: K_h = [W_UK_h c_kv | RoPE key], V_h = W_UV_h c_kv;
 * [MLA architecture] 5.2: the form that suits prefill-heavy batches).  For query
 * token t of sequence b at position P (as mla_decode) and every head h:
 *   s_u = softmax_scale * ( sum_d q_nope[t][h][d] * K_h[u][d]
 *                         + sum_i q_lat[t][h][d_latent + i] * row_u[d_latent + i] )
 *   K_h[u][d] = round( sum_c w_uk[h][d][c] * row_u[c] ),  V_h[u][v] likewise with w_uv
 *   out[t][h][v] = sum_u softmax(s)_u * V_h[u][v]    (fp32 out [T][H][d_v])
 * over cached positions u < kv_lens[b] (u <= P when causal != 0).  The RoPE
 * query columns come from q_lat (written by mla_append_cache); the same output
 * as mla_absorb_q + mla_decode + mla_out_proj, up to rounding.  K_h and V_h are
 * rounded to bf16 in the workspace (overwritten).  Other arguments as mla_decode.
 * Only the DeepSeek-V3 bf16 configuration (UNSUPPORTED otherwise).  Device
 * pointers, 16-byte aligned; WORKSPACE if the workspace is too small. */
mla_status mla_prefill_decompressed(const mla_config* cfg, int32_t num_seqs,
                                    const int32_t* q_start, const int32_t* kv_lens,
                                    const int32_t* q_start_host, const int32_t* kv_lens_host,
                                    const int32_t* block_table, int32_t max_blocks_per_seq,
                                    int64_t num_pool_blocks, const void* q_nope,
                                    const void* q_lat, const void* kv_pool, const void* w_uk,
                                    const void* w_uv, int32_t causal, void* workspace,
                                    size_t workspace_bytes, float* out, uint32_t* dev_error,
                                    void* stream);

/* ---------------------------------------------------------------------------
 * Upstream of the cache: the joint KV down-projection fused with the append.
 * --------------------------------------------------------------------------- */

/* Workspace bytes that mla_kv_down_append needs: fp32 partial sums over
 * 512-deep slices of the hidden state, (d_model / 512) * T * (d_latent + d_rope)
 * * 4.  Same argument checks as mla_kv_down_append. */
mla_status mla_kv_down_workspace_size(const mla_config* cfg, int32_t T, int32_t d_model,
                                      size_t* bytes);

/* Joint KV down-projection and latent RMSNorm fused with the cache append
 * ([MLA architecture] 2.2: kv_a_proj_with_mqa maps the hidden state to the
 * 512-d latent and the 64-d shared RoPE key in one linear layer, and
 * kv_a_layernorm RMS-normalises the latent; 4.2: RoPE fused with the cache
 * update).  For each new token t (sequence token_seq[t], position positions[t]):
 *   y[n]   = round( sum_k x[t][k] * w_dkv[n][k] + b_dkv[n] ),  n < d_latent + d_rope
 *            (fp32 accumulation, one rounding to bf16; b_dkv may be NULL = 0)
 *   c[i]   = round( rms_gamma[i] * y[i] / sqrt(mean_{j<d_latent} y[j]^2 + rms_eps) )
 *   kv_pool row = [c | RoPE_p(y[d_latent:])]  with the RoPE of mla_append_cache
 *   q_lat[t][h][d_latent:] = RoPE_p(q_pe[t][h])  as mla_append_cache (if q_pe != NULL)
 * The normalisation is computed in fp32 (rounding may differ from an exact
 * evaluation by one bf16 unit in the last place).
 * x [T][d_model], w_dkv [d_latent + d_rope][d_model] (a linear layer's weight),
 * b_dkv [d_latent + d_rope], rms_gamma [d_latent]: bf16, device, 16-byte aligned.
 * Other arguments as mla_append_cache.  workspace: device, at least
 * mla_kv_down_workspace_size() bytes (WORKSPACE otherwise), overwritten.
 * Only the DeepSeek-V3 bf16 configuration is supported (UNSUPPORTED otherwise);
 * d_model must be a positive multiple of 512, at most MLA_MAX_D_MODEL, and
 * rms_eps finite and >= 0 (INVALID_ARG otherwise).  Entries with an
 * out-of-range position, sequence id or block id are skipped and flagged in
 * *dev_error. */
mla_status mla_kv_down_append(const mla_config* cfg, int32_t T, int32_t d_model, const void* x,
                              const void* w_dkv, const void* b_dkv, const void* rms_gamma,
                              float rms_eps, const void* q_pe, const int32_t* token_seq,
                              const int32_t* positions, const int32_t* block_table,
                              int32_t num_seqs, int32_t max_blocks_per_seq,
                              int64_t num_pool_blocks, const float* rope_cos,
                              const float* rope_sin, int32_t max_pos, void* workspace,
                              size_t workspace_bytes, void* kv_pool, void* q_lat,
                              uint32_t* dev_error, void* stream);

/* ---------------------------------------------------------------------------
 * e4m3 (fp8) latent cache ([MLA architecture] 4.2, "量化的影响": a quantised
 * cache halves the bytes per cached token; the page cautions that the absorbed
 * matrices are sensitive to precision).  DeepSeek-V3 bf16 configuration only
 * (UNSUPPORTED otherwise): the cache holds 576 bytes per token, every other
 * tensor keeps its bf16 / fp32 type.
 *
 * Format and scale convention: OCP e4m3 (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits; subnormals down to 2^-9; largest finite 448; 0x7F and 0xFF are
 * NaN), one scale per cache, a power of two kv_scale in [2^-60, 2^60]
 * (INVALID_ARG otherwise):  code = e4m3(x / kv_scale),  value = kv_scale * code.
 * Encoding rounds to nearest, ties to even, and saturates finite magnitudes at
 * 448.  Layout: kv_pool_fp8 [num_blocks][block_size][576] bytes, 16-byte aligned.
 * ------------------------------------------------------------------------- */

/* mla_append_cache for an e4m3 cache.  The row holds e4m3(c_kv[t] / kv_scale)
 * and e4m3(RoPE_p(k_pe[t]) / kv_scale), where RoPE_p is computed in fp32 with
 * the op order of mla_append_cache and rounded once (straight from fp32 to
 * e4m3, no bf16 step): the row is bit-exact and independent of the device.
 * q_lat's RoPE columns are written in bf16 exactly as mla_append_cache does.
 * Other arguments, errors and device-side checks as mla_append_cache; rope_cos
 * and rope_sin must be 16-byte aligned. */
mla_status mla_append_cache_fp8(const mla_config* cfg, int32_t T, const void* c_kv,
                                const void* k_pe, const void* q_pe, const int32_t* token_seq,
                                const int32_t* positions, const int32_t* block_table,
                                int32_t num_seqs, int32_t max_blocks_per_seq,
                                int64_t num_pool_blocks, const float* rope_cos,
                                const float* rope_sin, int32_t max_pos, float kv_scale,
                                void* kv_pool_fp8, void* q_lat, uint32_t* dev_error,
                                void* stream);

/* mla_decode over an e4m3 cache: the same attention over the dequantised rows
 * kv_scale * code, with the same split plan and workspace
 * (mla_decode_workspace_size), o_lat in bf16.  The scores run on fp8 MFMA: each
 * query head's 576 values are scaled by a power of two 2^(7-e), where 2^e <=
 * max|q| < 2^(e+1) over the head's values, and split into two e4m3 terms (hi =
 * e4m3(q), lo = e4m3(q - hi)), both multiplied against the stored codes, so the
 * query keeps about bf16's precision.  The weighted sum of the latents runs on
 * bf16 MFMA: the stored codes are widened to bf16 (exact) and the softmax
 * weights are bf16, as in mla_decode.  Accumulation and the softmax are fp32.
 * Results are run-to-run bitwise deterministic for a given split plan.
 * Arguments and errors as mla_decode, plus kv_scale. */
mla_status mla_decode_fp8(const mla_config* cfg, int32_t num_seqs, const int32_t* q_start,
                          const int32_t* kv_lens, const int32_t* q_start_host,
                          const int32_t* kv_lens_host, const int32_t* block_table,
                          int32_t max_blocks_per_seq, int64_t num_pool_blocks,
                          const void* q_lat, const void* kv_pool_fp8, float kv_scale,
                          int32_t causal, int32_t num_workgroups, void* workspace,
                          size_t workspace_bytes, void* o_lat, uint32_t* dev_error,
                          void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H_ */

// libmla C ABI: argument checks, split planning and kernel launches.
// The public contract (math, layouts, errors) is documented in include/mla.h.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "mla_internal.h"

namespace mla {
hipError_t launch_absorb_generic(const mla_config& c, int T, const void* q_nope,
                                 const void* w_uk, void* q_lat, hipStream_t st);
hipError_t launch_out_proj_generic(const mla_config& c, int T, const void* o_lat,
                                   const void* w_uv, float* out, hipStream_t st);
bool v3_kernels_available();

namespace {

bool is_v3_bf16(const mla_config& c) {
  return c.dtype == MLA_BF16 && c.num_heads == 128 && c.d_latent == 512 && c.d_rope == 64 &&
         c.d_nope == 128 && c.d_v == 128 && c.block_size == 64;
}

bool is_f32_supported(const mla_config& c) {
  const bool dc_ok = c.d_latent == 64 || c.d_latent == 128 || c.d_latent == 256 ||
                     c.d_latent == 512;
  const bool dr_ok = c.d_rope == 16 || c.d_rope == 32 || c.d_rope == 64;
  return c.dtype == MLA_F32 && c.num_heads >= 1 && c.num_heads <= 128 && dc_ok && dr_ok &&
         c.d_nope >= 1 && c.d_nope <= 256 && c.d_v >= 1 && c.d_v <= 256 && c.block_size == 64;
}

// kv_scale of an e4m3 cache: a power of two in [2^-60, 2^60]
bool kv_scale_ok(float s) {
  if (!(s > 0.f) || !isfinite(s)) return false;
  int e = 0;
  const float m = frexpf(s, &e);
  return m == 0.5f && e >= -59 && e <= 61;
}

mla_status check_cfg(const mla_config* c) {
  if (!c) return MLA_ERR_INVALID_ARG;
  if (c->num_heads < 1 || c->d_latent < 1 || c->d_rope < 2 || (c->d_rope & 1) ||
      c->d_nope < 1 || c->d_v < 1 || c->block_size < 1 || !(c->softmax_scale > 0.f) ||
      !isfinite(c->softmax_scale))
    return MLA_ERR_INVALID_ARG;
  if (c->dtype != MLA_F32 && c->dtype != MLA_BF16) return MLA_ERR_INVALID_ARG;
  if (!is_v3_bf16(*c) && !is_f32_supported(*c)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t elt(const mla_config& c) { return c.dtype == MLA_BF16 ? 2 : 4; }

mla_status from_hip(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Compute units of the current device (cached per device id).
mla_status device_cus(int* out) {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  std::lock_guard<std::mutex> g(mu);
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *out = cache[dev];
    return MLA_OK;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return MLA_ERR_HIP;
  if (dev >= 0 && dev < 64) cache[dev] = n;
  *out = n;
  return MLA_OK;
}

struct HostPlan {
  int32_t T = 0;
  int64_t U = 0;
  int32_t G = 0;
  size_t ws_bytes = 0;
  size_t lse_bytes = 0;
};

mla_status plan_decode(const mla_config& c, int32_t B, const int32_t* qs, const int32_t* kl,
                       int32_t causal, int32_t num_wg, HostPlan* hp) {
  if (B < 1 || !qs || !kl || num_wg < 0) return MLA_ERR_INVALID_ARG;
  if (qs[0] != 0) return MLA_ERR_INVALID_ARG;
  int64_t U = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t q = (int64_t)qs[b + 1] - qs[b];
    const int64_t L = kl[b];
    if (q < 0 || L < 1 || q > L) return MLA_ERR_INVALID_ARG;
    U += seq_units_before(L, q, q, c.block_size, causal ? 1 : 0);
  }
  if (U >= ((int64_t)1 << 31)) return MLA_ERR_UNSUPPORTED;  // unit indices are 32-bit
  hp->T = qs[B];
  hp->U = U;
  if (U == 0) {
    hp->G = 0;
    hp->ws_bytes = 0;
    return MLA_OK;
  }
  int64_t G = num_wg;
  if (G == 0) {
    int cus = 0;
    mla_status s = device_cus(&cus);
    if (s != MLA_OK) return s;
    // one KV range per compute unit, all resident at once: the V3 kernel runs
    // one workgroup per range and (by its LDS footprint) one per compute unit
    G = cus;
  }
  if (G > U) G = U;
  if (G > (1 << 30)) G = 1 << 30;
  hp->G = (int32_t)G;
  if (G == 1) {
    hp->ws_bytes = 0;
    hp->lse_bytes = 0;
  } else {
    hp->lse_bytes = ws_align(ws_lse_bytes(G, c.num_heads));
    hp->ws_bytes = hp->lse_bytes + (size_t)(2 * G) * c.num_heads * c.d_latent * elt(c);
  }
  return MLA_OK;
}

// Scratch of mla_decode_noalloc: the split partials live in this array instead
// of a caller-provided workspace.  The HIP runtime gives every device its own
// copy when it loads the code object; host code must use the per-device address
// from hipGetSymbolAddress, never the array's name (a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[MLA_DECODE_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per device.
mla_status scratch_ptr(void** out) {
  static std::mutex mu;
  static void* cache[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= 64) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> g(mu);
  if (!cache[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MLA_ERR_HIP;
    cache[dev] = ptr;
  }
  *out = cache[dev];
  return MLA_OK;
}

// Everything of mla_decode after planning.  `workspace` holds at least
// hp.ws_bytes bytes (checked by the caller), or is null with use_scratch set:
// then the library's scratch is used, looked up after the argument checks.
mla_status decode_planned(const mla_config* cfg, const HostPlan& hp, int32_t num_seqs,
                          const int32_t* q_start, const int32_t* kv_lens,
                          const int32_t* kv_lens_host, const int32_t* block_table,
                          int32_t max_blocks_per_seq, int64_t num_pool_blocks,
                          const void* q_lat, const void* kv_pool, int32_t causal,
                          void* workspace, bool use_scratch, void* o_lat, uint32_t* dev_error,
                          void* stream, const float* kv_scale_fp8 = nullptr) {
  if (!q_start || !kv_lens || !block_table || !q_lat || !kv_pool || !o_lat)
    return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_lat) || !aligned16(kv_pool) || !aligned16(o_lat)) return MLA_ERR_INVALID_ARG;
  if (num_pool_blocks < 1) return MLA_ERR_INVALID_ARG;
  int64_t maxL = 0;
  for (int b = 0; b < num_seqs; ++b) maxL = kv_lens_host[b] > maxL ? kv_lens_host[b] : maxL;
  if (max_blocks_per_seq < (maxL + cfg->block_size - 1) / cfg->block_size)
    return MLA_ERR_INVALID_ARG;
  // block-table entries are addressed with 32-bit indices on the device
  if ((int64_t)num_seqs * max_blocks_per_seq >= ((int64_t)1 << 31)) return MLA_ERR_UNSUPPORTED;
  if (use_scratch && hp.ws_bytes > 0) {
    mla_status s = scratch_ptr(&workspace);
    if (s != MLA_OK) return s;
  }
  DecodeArgs a;
  a.plan.q_start = q_start;
  a.plan.kv_lens = kv_lens;
  a.plan.B = num_seqs;
  a.plan.T = hp.T;
  a.plan.block_size = cfg->block_size;
  a.plan.causal = causal ? 1 : 0;
  a.plan.G = hp.G;
  a.plan.U = hp.U;
  a.block_table = block_table;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_pool_blocks;
  a.q_lat = q_lat;
  a.pool = kv_pool;
  a.o_lat = o_lat;
  a.ws_lse = hp.ws_bytes ? (float*)workspace : nullptr;
  a.ws_o = hp.ws_bytes ? (void*)((char*)workspace + hp.lse_bytes) : nullptr;
  a.err = dev_error;
  a.scale_log2 = cfg->softmax_scale * kLog2e;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (kv_scale_fp8)
    e = launch_decode_fp8(a, *kv_scale_fp8, st);
  else if (is_v3_bf16(*cfg) && v3_kernels_available())
    e = launch_decode_v3(a, st);
  else
    e = launch_decode_generic(*cfg, a, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (hp.G > 1) e = is_v3_bf16(*cfg) ? launch_merge_v3(a, st) : launch_merge(*cfg, a, st);
  return from_hip(e);
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported dims/dtype";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

mla_status mla_rope_table(float* cos_host, float* sin_host, int32_t max_pos, int32_t d_rope,
                          double theta) {
  if (!cos_host || !sin_host || max_pos < 1 || d_rope < 2 || (d_rope & 1) || !(theta > 0))
    return MLA_ERR_INVALID_ARG;
  const int half = d_rope / 2;
  for (int i = 0; i < half; ++i) {
    const double inv = 1.0 / pow(theta, 2.0 * i / (double)d_rope);
    for (int64_t p = 0; p < max_pos; ++p) {
      const double a = (double)p * inv;
      cos_host[p * half + i] = (float)cos(a);
      sin_host[p * half + i] = (float)sin(a);
    }
  }
  return MLA_OK;
}

mla_status mla_absorb_q(const mla_config* cfg, int32_t T, const void* q_nope, const void* w_uk,
                        void* q_lat, void* stream) {
  mla_status s = check_cfg(cfg);
  if (s != MLA_OK) return s;
  if (T < 0 || T > MLA_MAX_PROJ_TOKENS) return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!q_nope || !w_uk || !q_lat) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_lat)) return MLA_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (is_v3_bf16(*cfg)) return from_hip(launch_absorb_q(*cfg, T, q_nope, w_uk, q_lat, st));
  return from_hip(launch_absorb_generic(*cfg, T, q_nope, w_uk, q_lat, st));
}

mla_status mla_append_cache(const mla_config* cfg, int32_t T, const void* c_kv, const void* k_pe,
                            const void* q_pe, const int32_t* token_seq, const int32_t* positions,
                            const int32_t* block_table, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int64_t num_pool_blocks,
                            const float* rope_cos, const float* rope_sin, int32_t max_pos,
                            void* kv_pool, void* q_lat, uint32_t* dev_error, void* stream) {
  mla_status s = check_cfg(cfg);
  if (s != MLA_OK) return s;
  if (T < 0) return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!c_kv || !k_pe || !token_seq || !positions || !block_table || !rope_cos || !rope_sin ||
      !kv_pool)
    return MLA_ERR_INVALID_ARG;
  if ((q_pe == nullptr) != (q_lat == nullptr)) return MLA_ERR_INVALID_ARG;
  if (num_seqs < 1 || max_blocks_per_seq < 1 || num_pool_blocks < 1 || max_pos < 1)
    return MLA_ERR_INVALID_ARG;
  if (!aligned16(c_kv) || !aligned16(k_pe) || !aligned16(kv_pool) ||
      (q_pe && (!aligned16(q_pe) || !aligned16(q_lat))))
    return MLA_ERR_INVALID_ARG;
  return from_hip(launch_append(*cfg, T, c_kv, k_pe, q_pe, token_seq, positions, block_table,
                                num_seqs, max_blocks_per_seq, num_pool_blocks, rope_cos,
                                rope_sin, max_pos, kv_pool, q_lat, dev_error,
                                (hipStream_t)stream));
}

mla_status mla_decode_workspace_size(const mla_config* cfg, int32_t num_seqs,
                                     const int32_t* q_start_host, const int32_t* kv_lens_host,
                                     int32_t causal, int32_t num_workgroups, size_t* bytes) {
  mla_status s = check_cfg(cfg);
  if (s != MLA_OK) return s;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  HostPlan hp;
  s = plan_decode(*cfg, num_seqs, q_start_host, kv_lens_host, causal, num_workgroups, &hp);
  if (s != MLA_OK) return s;
  *bytes = hp.ws_bytes;
  return MLA_OK;
}

mla_status mla_decode(const mla_config* cfg, int32_t num_seqs, const int32_t* q_start,
                      const int32_t* kv_lens, const int32_t* q_start_host,
                      const int32_t* kv_lens_host, const int32_t* block_table,
                      int32_t max_blocks_per_seq, int64_t num_pool_blocks, const void* q_lat,
                      const void* kv_pool, int32_t causal, int32_t num_workgroups,
                      void* workspace, size_t workspace_bytes, void* o_lat, uint32_t* dev_error,
                      void* stream) {
  mla_status s = check_cfg(cfg);
  if (s != MLA_OK) return s;
  HostPlan hp;
  s = plan_decode(*cfg, num_seqs, q_start_host, kv_lens_host, causal, num_workgroups, &hp);
  if (s != MLA_OK) return s;
  if (hp.T == 0) return MLA_OK;
  if (hp.ws_bytes > 0) {
    if (!workspace || workspace_bytes < hp.ws_bytes || !aligned16(workspace))
      return MLA_ERR_WORKSPACE;
  }
  return decode_planned(cfg, hp, num_seqs, q_start, kv_lens, kv_lens_host, block_table,
                        max_blocks_per_seq, num_pool_blocks, q_lat, kv_pool, causal, workspace,
                        false, o_lat, dev_error, stream);
}

mla_status mla_decode_noalloc(const mla_config* cfg, int32_t num_seqs, const int32_t* q_start,
                              const int32_t* kv_lens, const int32_t* q_start_host,
                              const int32_t* kv_lens_host, const int32_t* block_table,
                              int32_t max_blocks_per_seq, int64_t num_pool_blocks,
                              const void* q_lat, const void* kv_pool, int32_t causal,
                              int32_t num_workgroups, void* o_lat, uint32_t* dev_error,
                              void* stream) {
  mla_status s = check_cfg(cfg);
  if (s != MLA_OK) return s;
  HostPlan hp;
  s = plan_decode(*cfg, num_seqs, q_start_host, kv_lens_host, causal, num_workgroups, &hp);
  if (s != MLA_OK) return s;
  if (hp.T == 0) return MLA_OK;
  if (hp.ws_bytes > MLA_DECODE_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  return decode_planned(cfg, hp, num_seqs, q_start, kv_lens, kv_lens_host, block_table,
                        max_blocks_per_seq, num_pool_blocks, q_lat, kv_pool, causal, nullptr,
                        true, o_lat, dev_error, stream);
}

mla_status mla_out_proj(const mla_config* cfg, int32_t T, const void* o_lat, const void* w_uv,
                        float* out, void* stream) {
  mla_status s = check_cfg(cfg);
  if (s != MLA_OK) return s;
  if (T < 0 || T > MLA_MAX_PROJ_TOKENS) return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!o_lat || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (is_v3_bf16(*cfg)) return from_hip(launch_out_proj(*cfg, T, o_lat, w_uv, out, st));
  return from_hip(launch_out_proj_generic(*cfg, T, o_lat, w_uv, out, st));
}

static mla_status check_fused(const mla_config* cfg, int32_t T, int32_t width, int32_t mult) {
  mla_status s = check_cfg(cfg);
  if (s != MLA_OK) return s;
  if (!is_v3_bf16(*cfg)) return MLA_ERR_UNSUPPORTED;
  if (T < 0 || T > MLA_MAX_PROJ_TOKENS) return MLA_ERR_INVALID_ARG;
  if (width < mult || width > MLA_MAX_D_MODEL || width % mult != 0) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

mla_status mla_absorb_q_fused(const mla_config* cfg, int32_t T, int32_t d_cq, const void* c_q,
                              const void* w_kq, void* q_lat, void* stream) {
  mla_status s = check_fused(cfg, T, d_cq, 128);
  if (s != MLA_OK) return s;
  if (T == 0) return MLA_OK;
  if (!c_q || !w_kq || !q_lat) return MLA_ERR_INVALID_ARG;
  if (!aligned16(c_q) || !aligned16(w_kq) || !aligned16(q_lat)) return MLA_ERR_INVALID_ARG;
  return from_hip(launch_absorb_q_fused(T, d_cq, c_q, w_kq, q_lat, (hipStream_t)stream));
}

mla_status mla_out_proj_fused_workspace_size(const mla_config* cfg, int32_t T,
                                             int32_t d_model, size_t* bytes) {
  mla_status s = check_fused(cfg, T, d_model, 256);
  if (s != MLA_OK) return s;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  *bytes = out_fused_workspace_bytes(T, d_model);
  return MLA_OK;
}

mla_status mla_out_proj_fused(const mla_config* cfg, int32_t T, int32_t d_model,
                              const void* o_lat, const void* w_ov, float* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  mla_status s = check_fused(cfg, T, d_model, 256);
  if (s != MLA_OK) return s;
  if (T == 0) return MLA_OK;
  if (!o_lat || !w_ov || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned16(o_lat) || !aligned16(w_ov) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < out_fused_workspace_bytes(T, d_model) ||
      !aligned16(workspace))
    return MLA_ERR_WORKSPACE;
  return from_hip(
      launch_out_proj_fused(T, d_model, o_lat, w_ov, out, workspace, (hipStream_t)stream));
}

struct PrefillPlan {
  int32_t T = 0;
  int64_t R = 0;
  int32_t max_qt = 0;
};

static mla_status plan_prefill(const mla_config* cfg, int32_t B, const int32_t* qs,
                               const int32_t* kl, int32_t max_blocks, PrefillPlan* pp) {
  mla_status s = check_cfg(cfg);
  if (s != MLA_OK) return s;
  if (!is_v3_bf16(*cfg)) return MLA_ERR_UNSUPPORTED;
  if (B < 1 || !qs || !kl || qs[0] != 0) return MLA_ERR_INVALID_ARG;
  int64_t R = 0;
  int32_t max_qt = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t q = (int64_t)qs[b + 1] - qs[b];
    const int64_t L = kl[b];
    if (q < 0 || L < 1 || q > L) return MLA_ERR_INVALID_ARG;
    const int64_t nblk = (L + 63) / 64;
    if (max_blocks > 0 && nblk > max_blocks) return MLA_ERR_INVALID_ARG;
    R += 64 * nblk;
    max_qt = std::max<int32_t>(max_qt, (int32_t)((q + 127) / 128));  // 128-query tiles
  }
  if (R >= ((int64_t)1 << 31) || (int64_t)B * max_qt >= ((int64_t)1 << 31))
    return MLA_ERR_UNSUPPORTED;
  pp->T = qs[B];
  pp->R = R;
  pp->max_qt = max_qt;
  return MLA_OK;
}

mla_status mla_prefill_workspace_size(const mla_config* cfg, int32_t num_seqs,
                                      const int32_t* q_start_host,
                                      const int32_t* kv_lens_host, size_t* bytes) {
  PrefillPlan pp;
  mla_status s = plan_prefill(cfg, num_seqs, q_start_host, kv_lens_host, 0, &pp);
  if (s != MLA_OK) return s;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  *bytes = prefill_workspace_bytes(num_seqs, pp.R);
  return MLA_OK;
}

mla_status mla_prefill_decompressed(const mla_config* cfg, int32_t num_seqs,
                                    const int32_t* q_start, const int32_t* kv_lens,
                                    const int32_t* q_start_host, const int32_t* kv_lens_host,
                                    const int32_t* block_table, int32_t max_blocks_per_seq,
                                    int64_t num_pool_blocks, const void* q_nope,
                                    const void* q_lat, const void* kv_pool, const void* w_uk,
                                    const void* w_uv, int32_t causal, void* workspace,
                                    size_t workspace_bytes, float* out, uint32_t* dev_error,
                                    void* stream) {
  if (max_blocks_per_seq < 1 || num_pool_blocks < 1) return MLA_ERR_INVALID_ARG;
  PrefillPlan pp;
  mla_status s = plan_prefill(cfg, num_seqs, q_start_host, kv_lens_host, max_blocks_per_seq, &pp);
  if (s != MLA_OK) return s;
  if (pp.T == 0) return MLA_OK;
  if (!q_start || !kv_lens || !block_table || !q_nope || !q_lat || !kv_pool || !w_uk || !w_uv ||
      !out)
    return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(q_lat) || !aligned16(kv_pool) || !aligned16(w_uk) ||
      !aligned16(w_uv) || !aligned16(out))
    return MLA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < prefill_workspace_bytes(num_seqs, pp.R) ||
      !aligned16(workspace))
    return MLA_ERR_WORKSPACE;
  return from_hip(launch_prefill(num_seqs, pp.T, pp.R, pp.max_qt, q_start, kv_lens, block_table,
                                 max_blocks_per_seq, num_pool_blocks, q_nope, q_lat, kv_pool,
                                 w_uk, w_uv, causal ? 1 : 0, cfg->softmax_scale, workspace, out,
                                 dev_error, (hipStream_t)stream));
}

static mla_status check_kv_down(const mla_config* cfg, int32_t T, int32_t d_model) {
  mla_status s = check_cfg(cfg);
  if (s != MLA_OK) return s;
  if (!is_v3_bf16(*cfg)) return MLA_ERR_UNSUPPORTED;
  if (T < 0 || T > MLA_MAX_PROJ_TOKENS) return MLA_ERR_INVALID_ARG;
  if (d_model < 512 || d_model > MLA_MAX_D_MODEL || d_model % 512 != 0) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

mla_status mla_kv_down_workspace_size(const mla_config* cfg, int32_t T, int32_t d_model,
                                      size_t* bytes) {
  mla_status s = check_kv_down(cfg, T, d_model);
  if (s != MLA_OK) return s;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  *bytes = kv_down_workspace_bytes(T, d_model);
  return MLA_OK;
}

mla_status mla_kv_down_append(const mla_config* cfg, int32_t T, int32_t d_model, const void* x,
                              const void* w_dkv, const void* b_dkv, const void* rms_gamma,
                              float rms_eps, const void* q_pe, const int32_t* token_seq,
                              const int32_t* positions, const int32_t* block_table,
                              int32_t num_seqs, int32_t max_blocks_per_seq,
                              int64_t num_pool_blocks, const float* rope_cos,
                              const float* rope_sin, int32_t max_pos, void* workspace,
                              size_t workspace_bytes, void* kv_pool, void* q_lat,
                              uint32_t* dev_error, void* stream) {
  mla_status s = check_kv_down(cfg, T, d_model);
  if (s != MLA_OK) return s;
  if (!(rms_eps >= 0.f) || rms_eps > 3.0e38f) return MLA_ERR_INVALID_ARG;  // also NaN, inf
  if (T == 0) return MLA_OK;
  if (!x || !w_dkv || !rms_gamma || !token_seq || !positions || !block_table || !rope_cos ||
      !rope_sin || !kv_pool)
    return MLA_ERR_INVALID_ARG;
  if ((q_pe == nullptr) != (q_lat == nullptr)) return MLA_ERR_INVALID_ARG;
  if (num_seqs < 1 || max_blocks_per_seq < 1 || num_pool_blocks < 1 || max_pos < 1)
    return MLA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_dkv) || !aligned16(rms_gamma) || !aligned16(kv_pool) ||
      !aligned16(rope_cos) || !aligned16(rope_sin) || (b_dkv && !aligned16(b_dkv)) ||
      (q_pe && (!aligned16(q_pe) || !aligned16(q_lat))))
    return MLA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < kv_down_workspace_bytes(T, d_model) ||
      !aligned16(workspace))
    return MLA_ERR_WORKSPACE;
  return from_hip(launch_kv_down_append(T, d_model, x, w_dkv, b_dkv, rms_gamma, rms_eps, q_pe,
                                        token_seq, positions, block_table, num_seqs,
                                        max_blocks_per_seq, num_pool_blocks, rope_cos, rope_sin,
                                        max_pos, workspace, kv_pool, q_lat, dev_error,
                                        (hipStream_t)stream));
}

mla_status mla_append_cache_fp8(const mla_config* cfg, int32_t T, const void* c_kv,
                                const void* k_pe, const void* q_pe, const int32_t* token_seq,
                                const int32_t* positions, const int32_t* block_table,
                                int32_t num_seqs, int32_t max_blocks_per_seq,
                                int64_t num_pool_blocks, const float* rope_cos,
                                const float* rope_sin, int32_t max_pos, float kv_scale,
                                void* kv_pool, void* q_lat, uint32_t* dev_error, void* stream) {
  mla_status s = check_cfg(cfg);
  if (s != MLA_OK) return s;
  if (!is_v3_bf16(*cfg)) return MLA_ERR_UNSUPPORTED;
  if (!kv_scale_ok(kv_scale)) return MLA_ERR_INVALID_ARG;
  if (T < 0) return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!c_kv || !k_pe || !token_seq || !positions || !block_table || !rope_cos || !rope_sin ||
      !kv_pool)
    return MLA_ERR_INVALID_ARG;
  if ((q_pe == nullptr) != (q_lat == nullptr)) return MLA_ERR_INVALID_ARG;
  if (num_seqs < 1 || max_blocks_per_seq < 1 || num_pool_blocks < 1 || max_pos < 1)
    return MLA_ERR_INVALID_ARG;
  if (!aligned16(c_kv) || !aligned16(k_pe) || !aligned16(kv_pool) || !aligned16(rope_cos) ||
      !aligned16(rope_sin) || (q_pe && (!aligned16(q_pe) || !aligned16(q_lat))))
    return MLA_ERR_INVALID_ARG;
  return from_hip(launch_append_fp8(T, c_kv, k_pe, q_pe, token_seq, positions, block_table,
                                    num_seqs, max_blocks_per_seq, num_pool_blocks, rope_cos,
                                    rope_sin, max_pos, 1.0f / kv_scale, kv_pool, q_lat,
                                    dev_error, (hipStream_t)stream));
}

mla_status mla_decode_fp8(const mla_config* cfg, int32_t num_seqs, const int32_t* q_start,
                          const int32_t* kv_lens, const int32_t* q_start_host,
                          const int32_t* kv_lens_host, const int32_t* block_table,
                          int32_t max_blocks_per_seq, int64_t num_pool_blocks, const void* q_lat,
                          const void* kv_pool, float kv_scale, int32_t causal,
                          int32_t num_workgroups, void* workspace, size_t workspace_bytes,
                          void* o_lat, uint32_t* dev_error, void* stream) {
  mla_status s = check_cfg(cfg);
  if (s != MLA_OK) return s;
  if (!is_v3_bf16(*cfg)) return MLA_ERR_UNSUPPORTED;
  if (!kv_scale_ok(kv_scale)) return MLA_ERR_INVALID_ARG;
  HostPlan hp;
  s = plan_decode(*cfg, num_seqs, q_start_host, kv_lens_host, causal, num_workgroups, &hp);
  if (s != MLA_OK) return s;
  if (hp.T == 0) return MLA_OK;
  if (hp.ws_bytes > 0) {
    if (!workspace || workspace_bytes < hp.ws_bytes || !aligned16(workspace))
      return MLA_ERR_WORKSPACE;
  }
  return decode_planned(cfg, hp, num_seqs, q_start, kv_lens, kv_lens_host, block_table,
                        max_blocks_per_seq, num_pool_blocks, q_lat, kv_pool, causal, workspace,
                        false, o_lat, dev_error, stream, &kv_scale);
}

}  // extern "C"

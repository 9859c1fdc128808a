// Non-absorbed (explicit-decompression) attention for prefill, DeepSeek-V3
// shapes (128 heads, d_c 512, d_r 64, d_nope = d_v = 128), bf16, on gfx950 MFMA.
//
// [MLA explainer] forward_training: K and V are decompressed from the cached
// latent per head, K_h = [W_UK_h c_kv | RoPE key] (192 wide), V_h = W_UV_h c_kv
// (128 wide), and attention runs at those widths.  [MLA architecture] 5.2: for
// prefill-heavy batches the absorbed form is the wrong trade; per (query, key)
// pair the decompressed form costs 2*128*(192 + 128) operations against
// 2*128*(576 + 512) absorbed, for a one-time decompression of the keys.
// For query token t (sequence b, position p) and head h:
//   out[t][h][v] = sum_u softmax_u(scale * ([q_nope | RoPE(q_pe)][t][h] . K_h[u])) V_h[u][v]
// over u < kv_len[b] (u <= p when causal).  The RoPE query columns are read
// from q_lat (written by mla_append_cache), the RoPE key from the cache rows.
//
// Workspace: row_base [B+1] int32 (first packed key row of each sequence; each
// sequence's rows are padded to a multiple of 64, so a 64-row tile is one
// cache block), then K_nope [H][R][128] and V [H][R][128] bf16 for R packed
// rows.  Padding rows repeat the sequence's last row (finite values, masked
// out of the softmax).
//
// row_base_kernel: one wave scans the device lengths.
// decompress_kernel: workgroup = (4096 packed rows, head, K or V).  The head's
//   W_UK (or W_UV) [128 x 512] is staged in LDS; each wave takes 16-row blocks
//   and loads their latent rows from the paged pool straight into the MFMA
//   B operand (16 bytes per lane per 32-deep step), two blocks ahead of the
//   one it multiplies: C^T[d][row] =
//   W[d][.] . c_kv[row][.] on v_mfma_f32_16x16x32_bf16, 4 d-values per lane
//   stored as 8 bytes.
// attn_kernel: workgroup = (128 queries of one sequence, head), 8 waves x 16
//   queries (two per SIMD, sharing every staged tile).  Key tiles of 64 rows ([K_nope | RoPE key] 400-byte LDS rows, V
//   288-byte rows) are loaded into registers one tile ahead and staged in LDS.
//   Per tile and wave: S^T[64 keys x 16 queries] = K . Q^T (24 MFMAs, Q^T in
//   registers), online softmax per query (a lane owns one query and 16 keys,
//   max and sum across the 4 lanes of a query), O^T[128 x 16] += V^T . P^T
//   (16 MFMAs): V^T comes from the transposing LDS read ds_read_b64_tr_b16,
//   whose k-slot order (keys 4g..4g+3, then 16+4g..) is exactly the order of
//   the probabilities a lane holds, so P never leaves the registers.
//
// MFMA operand layout (lane l = 16g + i): A[i][k], B[k][i] with the 8 k-slots
// of group g; D[4g + r][i], r = 0..3.
#include <math.h>

#include "plan_device.h"

namespace mla {
namespace {

constexpr int kH = 128;
constexpr int kDC = 512;
constexpr int kRow = 576;
constexpr int kDN = 128;              // no-RoPE query / key width (and value width)
constexpr int kBS = 64;
constexpr int kQT = 128;              // queries per attention workgroup (8 waves x 16)
constexpr int kChunk = 4096;          // packed rows per decompression workgroup
constexpr int kAhead = 2;             // 16-row blocks in flight ahead of the one multiplied
constexpr int kWRowB = kDC * 2 + 16;  // W row in LDS (bytes, padded)
constexpr int kKRowB = 192 * 2 + 16;  // key row in LDS: 128 no-RoPE + 64 RoPE (padded)
constexpr int kVRowB = kDN * 2 + 32;  // value row in LDS (padded)

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

__global__ __launch_bounds__(64) void row_base_kernel(int B, const int32_t* __restrict__ kv_lens,
                                                      int32_t* __restrict__ row_base) {
  const int lane = threadIdx.x;
  int acc = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    int v = b < B ? ((max(kv_lens[b], 1) + kBS - 1) / kBS) * kBS : 0;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (b < B) row_base[b] = acc + incl - v;
    acc += __shfl(incl, 63, 64);
  }
  if (lane == 0) row_base[B] = acc;
}

// Cache row of position u of sequence b (u < the sequence's padded length);
// positions past the last cached one repeat it.  Out-of-range block ids are
// flagged and replaced by block 0 so that every access stays in bounds.
__device__ __forceinline__ int64_t key_row(const int32_t* bt, int b, int max_blocks,
                                           int64_t num_blocks, int L, int u, uint32_t& bad) {
  u = min(u, L - 1);
  if (u < 0 || u / kBS >= max_blocks) {
    bad |= MLA_DEVERR_LENGTH;
    u = 0;
  }
  int64_t blk = bt[(int64_t)b * max_blocks + u / kBS];
  if (blk < 0 || blk >= num_blocks) {
    bad |= MLA_DEVERR_BLOCK;
    blk = 0;
  }
  return blk * kBS + u % kBS;
}

__global__ __launch_bounds__(256) void decompress_kernel(
    int B, int64_t R, const int32_t* __restrict__ row_base, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ bt, int max_blocks, int64_t num_blocks,
    const uint16_t* __restrict__ pool, const uint16_t* __restrict__ w_uk,
    const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ kd, uint16_t* __restrict__ vd,
    uint32_t* err) {
  __shared__ __attribute__((aligned(16))) char wt[kDN * kWRowB];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int h = blockIdx.y, half = blockIdx.z;
  const uint16_t* w = (half ? w_uv : w_uk) + (int64_t)h * kDN * kDC;
  uint16_t* dst = (half ? vd : kd) + (int64_t)h * R * kDN;
#pragma unroll 8
  for (int i = 0; i < kDN * kDC / 8 / 256; ++i) {
    const int k = tid + 256 * i, r = k >> 6, c = k & 63;
    *(u32x4*)(wt + r * kWRowB + 16 * c) = *(const u32x4*)(w + r * kDC + 8 * c);
  }
  __syncthreads();

  // wave w owns the 16-row blocks r0 + 16w + 64i, i < kChunk / 64; blocks past
  // R (or past the chunk, in the loop's last round) are computed on a valid
  // row and not stored.  The latent rows of block
  // i + kAhead are requested while block i is multiplied (a ring of kAhead + 1
  // register sets, unconditional loads so that the waits stay precise).
  const int64_t r0 = (int64_t)blockIdx.x * kChunk + 16 * uni(wave);  // uniform: scalar walk
  uint32_t bad = 0;
  int b = 0;
  // The 16 rows of a block lie in one 64-row cache block (positions past the
  // last cached one, which repeat it, included), so the block-table entry is
  // uniform and comes through the scalar cache: the address of the next loads
  // never waits on a vector load.
  auto source = [&](int64_t rb) -> const uint16_t* {
    // the sequence of rows rb .. rb+15 (rows only grow: walk forward)
    rb = min(rb, R - 16);
    while (b + 1 < B && ldc(row_base, b + 1) <= rb) ++b;
    int L = ldc(kv_lens, b);
    const int rb0 = ldc(row_base, b), rb1 = ldc(row_base, b + 1);
    int u0 = (int)(rb - rb0);
    if (L < 1 || rb1 - rb0 != ((L + kBS - 1) / kBS) * kBS || u0 / kBS >= max_blocks) {
      bad |= MLA_DEVERR_LENGTH;  // device lengths disagree with the host's
      L = 1;
      u0 = 0;
    }
    int64_t blk = ldc(bt, (int64_t)b * max_blocks + u0 / kBS);
    if (blk < 0 || blk >= num_blocks) {
      bad |= MLA_DEVERR_BLOCK;
      blk = 0;
    }
    return pool + (blk * kBS + min(u0 + i16, L - 1) % kBS) * kRow + 8 * g;
  };
  u32x4 x[kAhead + 1][kDC / 32];
  auto load = [&](int slot, int64_t rb) {
    const uint16_t* src = source(rb);
#pragma unroll
    for (int kk = 0; kk < kDC / 32; ++kk) x[slot][kk] = *(const u32x4*)(src + 32 * kk);
  };
#pragma unroll
  for (int i = 0; i < kAhead; ++i) load(i, r0 + 64 * i);
  // blocks this wave owns in the chunk, rounded up to whole rounds of the ring
  const int64_t left = R - (int64_t)blockIdx.x * kChunk;
  const int nblk = (int)min<int64_t>(kChunk / 64, (left + 63) / 64);
  for (int i0 = 0; i0 < nblk; i0 += kAhead + 1) {
#pragma unroll
    for (int d = 0; d < kAhead + 1; ++d) {
      const int64_t rb = r0 + 64 * (i0 + d);
      load((d + kAhead) % (kAhead + 1), rb + 64 * kAhead);
      f32x4 acc[kDN / 16];
#pragma unroll
      for (int nb = 0; nb < kDN / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      // the weight operands are the same for every block: an opaque offset keeps
      // the compiler from hoisting all 128 of their LDS reads out of the loop
      int wofs = (16 * 0 + i16) * kWRowB + 16 * g;
      asm volatile("" : "+v"(wofs));
#pragma unroll
      for (int kk = 0; kk < kDC / 32; ++kk) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, x[d][kk]);
#pragma unroll
        for (int nb = 0; nb < kDN / 16; ++nb) {
          const bf16x8 av = __builtin_bit_cast(
              bf16x8, *(const u32x4*)(wt + wofs + 16 * nb * kWRowB + 64 * kk));
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[nb], 0, 0, 0);
        }
      }
      if (rb < R && i0 + d < kChunk / 64) {
        // lane holds C^T[d = 16nb + 4g + r][row rb + i16]
        uint16_t* o = dst + (rb + i16) * kDN + 4 * g;
#pragma unroll
        for (int nb = 0; nb < kDN / 16; ++nb) {
          u32x2 v;
          v.x = pack_bf16x2(acc[nb][0], acc[nb][1]);
          v.y = pack_bf16x2(acc[nb][2], acc[nb][3]);
          *(u32x2*)(o + 16 * nb) = v;
        }
      }
    }
  }
  if (bad && err) atomicOr(err, bad);
}

__global__ __launch_bounds__(512) void attn_kernel(
    int B, int T, int max_qt, int64_t R, const int32_t* __restrict__ row_base,
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ bt, int max_blocks, int64_t num_blocks,
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_lat,
    const uint16_t* __restrict__ pool, const uint16_t* __restrict__ kd,
    const uint16_t* __restrict__ vd, int causal, float scale_log2, float* __restrict__ out,
    uint32_t* err) {
  __shared__ __attribute__((aligned(16))) char kt[kBS * kKRowB];
  __shared__ __attribute__((aligned(16))) char vt[kBS * kVRowB];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int h = blockIdx.y, b = blockIdx.x / max_qt, qt = blockIdx.x % max_qt;
  const int qs0 = q_start[b], qlen = q_start[b + 1] - qs0, L = kv_lens[b];
  const int j0 = kQT * qt;
  if (j0 >= qlen) return;
  const int nq = min(kQT, qlen - j0);
  const int P0 = L - qlen;  // position of the sequence's first query token
  const int64_t rbase = row_base[b];
  uint32_t bad = 0;
  if (qs0 < 0 || qs0 + qlen > T || L < 1 || qlen > L || rbase < 0 ||
      rbase + ((L + kBS - 1) / kBS) * kBS > R) {
    // device lengths disagree with the host's (the grid and workspace came from those)
    if (tid == 0 && err) atomicOr(err, MLA_DEVERR_LENGTH);
    return;
  }

  // this lane's query (lanes past the tile's last query repeat it, unstored)
  const int jq = j0 + min(16 * wave + i16, nq - 1);
  const int t = qs0 + jq;
  const int pos_q = P0 + jq;
  u32x4 q[6];  // Q^T operand: k-steps 0..3 no-RoPE, 4..5 RoPE
  {
    const uint16_t* qn = q_nope + ((int64_t)t * kH + h) * kDN + 8 * g;
    const uint16_t* qr = q_lat + ((int64_t)t * kH + h) * kRow + kDC + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) q[ks] = *(const u32x4*)(qn + 32 * ks);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) q[4 + ks] = *(const u32x4*)(qr + 32 * ks);
  }
  // keys of the tile: u < u_end
  const int u_end = causal ? P0 + j0 + nq : L;
  const int ntiles = (u_end + kBS - 1) / kBS;

  // tile loads per thread: 2 no-RoPE key, 1 RoPE key, 2 value pieces of 16 B
  u32x4 kn[2], kr, vv[2];
  const uint16_t* kd_h = kd + ((int64_t)h * R + rbase) * kDN;
  const uint16_t* vd_h = vd + ((int64_t)h * R + rbase) * kDN;
  auto load = [&](int k_t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = tid + 512 * i, r = k >> 4, c = k & 15;
      kn[i] = *(const u32x4*)(kd_h + (int64_t)(kBS * k_t + r) * kDN + 8 * c);
      vv[i] = *(const u32x4*)(vd_h + (int64_t)(kBS * k_t + r) * kDN + 8 * c);
    }
    const int r = tid >> 3, c = tid & 7;
    const int64_t row = key_row(bt, b, max_blocks, num_blocks, L, kBS * k_t + r, bad);
    kr = *(const u32x4*)(pool + row * kRow + kDC + 8 * c);
  };

  float m_run = -INFINITY, l_part = 0.f;
  f32x4 acc[kDN / 16];
#pragma unroll
  for (int vb = 0; vb < kDN / 16; ++vb) acc[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
  load(0);
  for (int k_t = 0; k_t < ntiles; ++k_t) {
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = tid + 512 * i, r = k >> 4, c = k & 15;
      *(u32x4*)(kt + r * kKRowB + 16 * c) = kn[i];
      *(u32x4*)(vt + r * kVRowB + 16 * c) = vv[i];
    }
    *(u32x4*)(kt + (tid >> 3) * kKRowB + 2 * kDN + 16 * (tid & 7)) = kr;
    __syncthreads();
    if (k_t + 1 < ntiles) load(k_t + 1);

    // scores S^T[key 16kb + 4g + r][query i16]
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) {
        const bf16x8 av = __builtin_bit_cast(
            bf16x8, *(const u32x4*)(kt + (16 * kb + i16) * kKRowB + 64 * ks + 16 * g));
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, q[ks]),
                                                        s[kb], 0, 0, 0);
      }
    }
    // scale, mask, online softmax for this lane's query over the tile
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = kBS * k_t + 16 * kb + 4 * g + r;
        const bool ok = u < L && (!causal || u <= pos_q);
        s[kb][r] = ok ? s[kb][r] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[kb][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);  // finite: key 0 is never masked
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_part *= alpha;
#pragma unroll
    for (int vb = 0; vb < kDN / 16; ++vb) acc[vb] *= alpha;
    float p[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kb][r] = exp2f(s[kb][r] - m_new);
        l_part += p[kb][r];
      }
    // P^T operand per 32-key step: slots 0..3 keys 4g.., slots 4..7 keys 16+4g..
    bf16x8 pb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      pb[ks] = __builtin_bit_cast(
          bf16x8, u32x4{pack_bf16x2(p[2 * ks][0], p[2 * ks][1]),
                        pack_bf16x2(p[2 * ks][2], p[2 * ks][3]),
                        pack_bf16x2(p[2 * ks + 1][0], p[2 * ks + 1][1]),
                        pack_bf16x2(p[2 * ks + 1][2], p[2 * ks + 1][3])});
    // O^T[v][query] += V^T . P^T; V^T through the transposing read: lane i16
    // points at row (key) 32ks + 4g + i16/4, columns 16vb + 4(i16 & 3)
#pragma unroll
    for (int vb = 0; vb < kDN / 16; ++vb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const char* pv = vt + (32 * ks + 4 * g + (i16 >> 2)) * kVRowB + (16 * vb + 4 * (i16 & 3)) * 2;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)pv);
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(pv + 16 * kVRowB));
        const bf16x8 av =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[ks], acc[vb], 0, 0, 0);
      }
  }
  float l_tot = l_part + __shfl_xor(l_part, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = 1.f / l_tot;
  if (16 * wave + i16 < nq) {
    // lane holds O^T[v = 16vb + 4g + r][query i16]
    float* o = out + ((int64_t)t * kH + h) * kDN + 4 * g;
#pragma unroll
    for (int vb = 0; vb < kDN / 16; ++vb) *(f32x4*)(o + 16 * vb) = acc[vb] * inv;
  }
  if (bad && err && tid == 0) atomicOr(err, bad);
}

}  // namespace

size_t prefill_workspace_bytes(int B, int64_t R) {
  return ws_align((size_t)(B + 1) * sizeof(int32_t)) + 2 * (size_t)kH * R * kDN * 2;
}

hipError_t launch_prefill(int B, int T, int64_t R, int max_qt, const int32_t* q_start,
                          const int32_t* kv_lens, const int32_t* bt, int max_blocks,
                          int64_t num_blocks, const void* q_nope, const void* q_lat,
                          const void* pool, const void* w_uk, const void* w_uv, int causal,
                          float scale, void* workspace, float* out, uint32_t* err,
                          hipStream_t st) {
  int32_t* row_base = (int32_t*)workspace;
  uint16_t* kd = (uint16_t*)((char*)workspace + ws_align((size_t)(B + 1) * sizeof(int32_t)));
  uint16_t* vd = kd + (size_t)kH * R * kDN;
  hipLaunchKernelGGL(row_base_kernel, dim3(1), dim3(64), 0, st, B, kv_lens, row_base);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decompress_kernel, dim3((unsigned)((R + kChunk - 1) / kChunk), kH, 2),
                     dim3(256), 0, st, B, R, row_base, kv_lens, bt, max_blocks, num_blocks,
                     (const uint16_t*)pool, (const uint16_t*)w_uk, (const uint16_t*)w_uv, kd, vd,
                     err);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_kernel, dim3(B * max_qt, kH), dim3(512), 0, st, B, T, max_qt, R, row_base,
                     q_start, kv_lens, bt, max_blocks, num_blocks, (const uint16_t*)q_nope,
                     (const uint16_t*)q_lat, (const uint16_t*)pool, kd, vd, causal,
                     scale * kLog2e, out, err);
  return hipGetLastError();
}

}  // namespace mla

// Split-KV absorbed latent attention over an e4m3 (fp8) latent cache, DeepSeek-V3
// shapes, on gfx950 fp8 MFMA.
//
// [MLA architecture] 4.2 ("量化的影响"): a quantised cache halves the bytes of
// every cached token; the page warns that the absorbed matrices are sensitive
// to precision.  Here the cache rows are 576 e4m3 values (576 bytes) under one
// power-of-two scale per cache, value = kv_scale * e4m3.  The method is the
// same as the bf16 kernel's ([MLA explainer] stage 2B: score = scale *
// q_lat . row over the 576 columns, softmax over the attended rows, o_lat =
// sum p * c_kv).
//   - Scores on v_mfma_scale_f32_16x16x128_f8f6f4 (e4m3 operands, unit
//     scales; twice the rate per column of the 16x16x32 fp8 form) for the 512
//     latent columns and on v_mfma_f32_16x16x32_fp8_fp8 for the 64 RoPE
//     columns.  The cached operand is the stored
//     e4m3 value itself; the query is split into two e4m3 terms, q = hi + lo
//     with hi = e4m3(q) and lo = e4m3(q - hi), both multiplied against the same
//     cache operand and summed in fp32, which keeps about as many significant
//     bits as bf16 (one e4m3 term keeps four, and costs the attention output
//     about ten times the error of the bf16 path).  Each query head's 576
//     values are first scaled by the power of two 2^(7-e), 2^e <= max|q| <
//     2^(e+1) over the head (scaled magnitudes stay below 256, inside the
//     format's 448), when its token's Q is loaded.
//   - Values on v_mfma_f32_16x16x32_bf16: each V^T operand (8 e4m3 values) is
//     widened to bf16 right after its LDS read, which is exact, and the softmax
//     weights P are bf16 as in the bf16 kernel.  A V^T operand serves four
//     MFMAs (the team's four head blocks), so the widening costs 4 VALU
//     instructions per 4 MFMAs; the score's K operand is read by all eight
//     waves for only 2 MFMAs each, which is why the scores stay on fp8 MFMA.
// The result is normalised in fp32 and rounded to bf16 (o_lat and the split
// partials), so the merge kernel of the bf16 cache serves this kernel too.
//
// Structure as in the bf16 kernel: one 8-wave workgroup per KV range, all 128
// heads; two teams of four waves in a score / value ping-pong half a tile apart;
// 32-row tiles streamed HBM -> LDS with direct-to-LDS loads into four buffers.
// Per tile and wave: 16 fp8 score MFMAs of 128 columns and 8 of 32 (2 row
// blocks x 2 query terms x (4 latent chunks + 2 RoPE k-steps); K rows from LDS,
// Q^T's hi term in 36 registers, its lo term in this wave's LDS area, read with
// the K operands) and 32 bf16 value MFMAs (V^T from LDS with the 8-bit
// transposing read ds_read_b64_tr_b8, P^T from LDS).
//
// Score operands: in latent chunk v (128 columns) the lanes of group g4 hold the
// 32 columns 128v + 32g4 .. +31 of their row (K) or head (Q), the same columns
// for both operands; two 16-byte LDS reads per row block and chunk.  In the
// two RoPE k-steps e = 0, 1 group g4 holds columns 512 + 16 g4 + 8 e .. +7, one
// 16-byte read per row block for both steps.
//
// LDS tile layout (18 KiB): 32 latent rows of 512 B, then 32 RoPE rows of 64 B.
// Latent row t keeps its 16-byte chunk c at c ^ F(t), F(t) = (t & 15) ^ 12*((t >> 4) & 1):
// a score read of one lane group (16 rows, one chunk each) and a transposing read of
// any two lane groups (rows {4a..4a+3, 4b..4b+3} and the same plus 16, a ^ b = 1 or
// 2) both touch distinct chunk positions, i.e. every LDS bank at most once.  RoPE
// row t keeps chunk c at c ^ ((t >> 2) & 3).
#include <math.h>

#include "gfx950_asm.h"
#include "plan_device.h"
#include "tile_walk.h"

namespace mla {
namespace {

using namespace tiles;

constexpr int kH = 128;
constexpr int kDC = 512;
constexpr int kRow = 576;
constexpr int kRowBytes = kRow;                    // 576: one byte per value
constexpr int kLatBytes = kDC;                     // 512: latent part of a row
constexpr int kRopeBytes = kRowBytes - kLatBytes;  // 64: RoPE part of a row
constexpr int kTileBytes = kTile * kRowBytes;      // 18432
constexpr int kRegionB = kTile * kLatBytes;        // 16384: start of the RoPE region
constexpr int kNBuf = 4;
constexpr int kWaves = 8;
constexpr float kRescale = 8.0f;  // lazy rescale threshold (log2 units): P <= 2^8

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int F(int t) { return (t & 15) ^ (((t >> 4) & 1) * 12); }
__device__ __forceinline__ int Fr(int t) { return (t >> 2) & 3; }

// This wave's direct-to-LDS loads of one tile.  Latent: loads d = w and w + 8,
// each 1 KiB = LDS rows 2d and 2d+1 (lane L: row 2d + L/32, physical chunk
// L % 32, so it fetches logical chunk (L % 32) ^ F(row)).  RoPE (waves 0 and 1):
// load w = RoPE rows 16w .. 16w+15 (lane L: row 16w + L/4, physical chunk L % 4).
// Rows past the end of a partial tile repeat its last valid row.
__device__ __forceinline__ void issue_rows(int wave, const char* blk, int last, char* buf,
                                           uint32_t lane) {
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = 2 * wave + 16 * r + (int)(lane >> 5);
    const uint32_t voff =
        (uint32_t)(min(t, last) * kRowBytes) + (((lane & 31) ^ (uint32_t)F(t)) << 4);
    dma16(blk, voff, buf + (wave + 8 * r) * 1024);
  }
  if (wave < 2) {
    const int t = 16 * wave + (int)(lane >> 2);
    const uint32_t voff = (uint32_t)(min(t, last) * kRowBytes + kLatBytes) +
                          (((lane & 3) ^ (uint32_t)Fr(t)) << 4);
    dma16(blk, voff, buf + kRegionB + wave * 1024);
  }
}

// Per-lane geometry (lane = 16 g4 + l16; tile buffers 1 KiB aligned):
//   score reads, column chunk v < 4, half e: row l16, logical 16-byte chunk
//     8v + 2g4 + e -> lat ^ 128 v ^ 16 e; row l16 + 16 (F differs by 12) at
//     ((lat ^ 192) + 8192) ^ 128 v ^ 16 e;
//   score reads, RoPE: RoPE row l16 (+16), logical chunk g4 -> rope; rows
//     l16 + 16 at + 1024;
//   transposing reads of feature block 8wk + f: the 16 lanes of group g4 read
//     rows R(g4, l16/2) = 4 g4 + l16/2 (l16 < 8) or 16 + 4 g4 + l16/2 - 4,
//     bytes 8 (l16 % 2) of the block's chunk -> val(wk) ^ 16 f; lane l16 then
//     holds feature l16 of rows R(g4, 0..7): tokens 4g4..4g4+3, 16+4g4..+3,
//     the order in which the score lanes hold their weights.
struct LaneGeom {
  int lane, l16, g4;
  __device__ __forceinline__ explicit LaneGeom(uint32_t tid)
      : lane((int)(tid & 63)), l16((int)(tid & 15)), g4((int)((tid >> 4) & 3)) {}
  __device__ __forceinline__ uint32_t lat() const {
    return l16 * kLatBytes + (((2 * g4) ^ l16) << 4);
  }
  __device__ __forceinline__ uint32_t rope() const {
    return kRegionB + l16 * kRopeBytes + ((g4 ^ Fr(l16)) << 4);
  }
  __device__ __forceinline__ uint32_t val(int wk) const {
    const int r = l16 >> 1;
    const int t = r < 4 ? 4 * g4 + r : 12 + 4 * g4 + r;
    return t * kLatBytes + (((8 * wk) ^ F(t)) << 4) + 8 * (l16 & 1);
  }
};

struct Shared {
  char tiles[kNBuf][kTileBytes];
  u32x4 pbuf[2][4][64];     // P^T fragments (bf16) [team][head block][lane]
  float alpha[2][4][16];    // rescale factor [team][head block][head % 16]
  float invl[2][4][16];     // kv_scale / softmax denominator, same layout
  int desc[kWaves][kNBuf][2];  // per wave: [tile % 4] = {flags | valid rows, token}
  u32x4 qlo[kWaves][4][2][64];  // Q^T lo term of each wave's heads [wave][latent chunk][half][lane]
  u32x4 qlo_r[kWaves][64];     // ... and of the two RoPE k-steps [wave][lane]
};

// four fp32 -> four e4m3 (nearest even) packed in one word, a first
__device__ __forceinline__ int pk_fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// eight fp32 -> two e4m3 terms: hi = e4m3(x), lo = e4m3(x - hi) (the
// subtraction is exact: hi is x's nearest e4m3 value)
__device__ __forceinline__ void split_fp8x8(const float* x, i32x2& hi, i32x2& lo) {
  hi = i32x2{pk_fp8x4(x[0], x[1], x[2], x[3]), pk_fp8x4(x[4], x[5], x[6], x[7])};
  float r[8];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(hi[w], false);  // bytes 0, 1
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(hi[w], true);   // bytes 2, 3
    r[4 * w] = x[4 * w] - a[0];
    r[4 * w + 1] = x[4 * w + 1] - a[1];
    r[4 * w + 2] = x[4 * w + 2] - b[0];
    r[4 * w + 3] = x[4 * w + 3] - b[1];
  }
  lo = i32x2{pk_fp8x4(r[0], r[1], r[2], r[3]), pk_fp8x4(r[4], r[5], r[6], r[7])};
}

// eight e4m3 values -> eight bf16 (exact: e4m3 values have 4 significant bits
// and an exponent range inside bf16's), two per v_cvt_scalef32_pk_bf16_fp8
// with unit scale
__device__ __forceinline__ bf16x8 widen_fp8x8(i32x2 v) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  u32x4 o;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[w], 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[w], 1.0f, true);
    o[2 * w] = __builtin_bit_cast(uint32_t, a);      // bytes 0, 1
    o[2 * w + 1] = __builtin_bit_cast(uint32_t, b);  // bytes 2, 3
  }
  return __builtin_bit_cast(bf16x8, o);
}

__global__ __launch_bounds__(512, 1) void decode_fp8_kernel(
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ block_table, const uint8_t* __restrict__ pool,
    const uint16_t* __restrict__ qlat, uint16_t* __restrict__ o_lat, uint16_t* __restrict__ ws_o,
    float* __restrict__ ws_lse, uint32_t* __restrict__ err, int B, int T, int causal, int G,
    int64_t U, int max_blocks, int64_t num_blocks, float sl2, float kv_scale) {
  __shared__ __attribute__((aligned(1024))) Shared sh;
  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);
  const int team = wave >> 2, wk = wave & 3;
  PlanArgs p;
  p.q_start = q_start;
  p.kv_lens = kv_lens;
  p.B = B;
  p.T = T;
  p.block_size = kBS;
  p.causal = causal;
  p.G = G;
  p.U = U;
  if (!plan_consistent(p, max_blocks)) {
    if (blockIdx.x == 0 && threadIdx.x == 0 && err) atomicOr(err, MLA_DEVERR_LENGTH);
    return;
  }
  // consecutive ranges (which share a split token) go to one XCD
  int w = blockIdx.x;
  if ((G & 7) == 0) w = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int u0 = (int)range_start(w, U, G), u1 = (int)range_start(w + 1, U, G);
  if (u0 >= u1) return;

  const char* lds0 = (const char*)&sh;
  const char* pool_b = (const char*)pool;
  const int nmine = wave < 2 ? 3 : 2;  // direct-to-LDS loads per tile of this wave
  Loader lg;
  lg.init(p, block_table, max_blocks, u0, u1);
  int issued = 0;
  bool pending_adv = false;

  i32x8 qh[4];   // Q^T (e4m3 hi term) of this lane's head, chunk v: columns 128 v + 32 g4 ..
  i32x2 qhr[2];  // ... and RoPE k-step e: columns 512 + 16 g4 + 8 e ..
  float qs2 = 0.f;  // log2(e) * softmax scale * kv_scale * Q scale of this lane's head
  f32x4 acc[8][4];  // [feature block][head block]
  float m_run = -INFINITY, l_part = 0.f;

  auto issue = [&]() {
    const int k_ = issued % kNBuf;
    const int bad_ = uni(lg.blk_raw < 0 || lg.blk_raw >= num_blocks);
    const int phys_ = uni(bad_ ? 0 : lg.blk_raw);
    const char* blk_ = pool_b + ((int64_t)phys_ * kBS + lg.half * kTile) * kRowBytes;
    issue_rows(wave, blk_, bad_ ? 0 : lg.nvalid - 1, sh.tiles[k_], opaque(threadIdx.x) & 63);
    if (lane == 0) {
      sh.desc[wave][k_][0] = (bad_ ? 0 : lg.nvalid) | (lg.first ? kFirstOfSeg : 0) |
                             (lg.last_of_segment() ? kLastOfSeg : 0) |
                             (lg.whole_token() ? kWhole : 0) | (bad_ ? kBad : 0) |
                             (lg.nseg > 0 ? kSecondSlot : 0);
      sh.desc[wave][k_][1] = lg.c.t;
    }
    ++issued;
    pending_adv = true;
  };
  auto advance = [&]() {
    if (pending_adv) {
      lg.next(p, block_table, max_blocks);
      pending_adv = false;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  };
  auto desc_of = [&](int i) { return uni(sh.desc[wave][i % kNBuf][0]); };
  auto tok_of = [&](int i) { return uni(sh.desc[wave][i % kNBuf][1]); };
  // Q^T of head 64team + 16wk + l16 as two e4m3 terms: the head's largest
  // magnitude max|q| (over the 4 lanes of the head) fixes the power of two
  // 2^(e-7), 2^e <= max|q| < 2^(e+1); the lane's 144 values are multiplied by
  // 2^(7-e) (exact) and split into hi + lo.
  auto load_q = [&](int tok) {
    const LaneGeom lg_(opaque(threadIdx.x));
    const uint32_t head = 64 * team + 16 * wk + lg_.l16;
    const char* qb = (const char*)qlat + (int64_t)tok * (kH * kRow * 2) + head * (kRow * 2);
    // raw[4v + j]: columns 128 v + 32 g4 + 8 j; raw[16 + e]: 512 + 16 g4 + 8 e
    u32x4 raw[18];
#pragma unroll
    for (int k = 0; k < 18; ++k) {
      const uint32_t col =
          k < 16 ? 128 * (k >> 2) + 32 * lg_.g4 + 8 * (k & 3) : 512 + 16 * lg_.g4 + 8 * (k - 16);
      raw[k] = *(const u32x4*)(qb + 2 * col);
    }
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
    uint32_t mx = 0;  // bf16 magnitudes compare as integers
#pragma unroll
    for (int k = 0; k < 18; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t v = raw[k][j];
        mx = max(mx, max(v & 0x7fffu, (v >> 16) & 0x7fffu));
      }
    const float amax = head_max(__uint_as_float(mx << 16));
    int e = (int)((__float_as_uint(amax) >> 23) & 0xff) - 127;
    e = min(max(e, -119), 127);
    const float up = __uint_as_float((uint32_t)(127 + 7 - e) << 23);    // 2^(7-e)
    qs2 = sl2 * kv_scale * __uint_as_float((uint32_t)(127 - 7 + e) << 23);  // * 2^(e-7)
    auto split8 = [&](const u32x4& r, i32x2& hi, i32x2& lo) {
      float f[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[2 * q] = __uint_as_float(r[q] << 16) * up;
        f[2 * q + 1] = __uint_as_float(r[q] & 0xffff0000u) * up;
      }
      split_fp8x8(f, hi, lo);
    };
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      i32x2 hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) split8(raw[4 * v + j], hi[j], lo[j]);
      qh[v] = i32x8{hi[0][0], hi[0][1], hi[1][0], hi[1][1], hi[2][0], hi[2][1], hi[3][0], hi[3][1]};
      sh.qlo[wave][v][0][lg_.lane] =
          u32x4{(uint32_t)lo[0][0], (uint32_t)lo[0][1], (uint32_t)lo[1][0], (uint32_t)lo[1][1]};
      sh.qlo[wave][v][1][lg_.lane] =
          u32x4{(uint32_t)lo[2][0], (uint32_t)lo[2][1], (uint32_t)lo[3][0], (uint32_t)lo[3][1]};
    }
    i32x2 lr[2];
    split8(raw[16], qhr[0], lr[0]);
    split8(raw[17], qhr[1], lr[1]);
    sh.qlo_r[wave][lg_.lane] =
        u32x4{(uint32_t)lr[0][0], (uint32_t)lr[0][1], (uint32_t)lr[1][0], (uint32_t)lr[1][1]};
  };

  // ---------------------------------------------------------------- S phase
  auto score_phase = [&](int i, int d) {
    const char* tb = sh.tiles[i % kNBuf];
    const LaneGeom lgm(opaque(threadIdx.x));
    const int lane = lgm.lane, l16 = lgm.l16, g4 = lgm.g4;
    if (d & kFirstOfSeg) {
      m_run = -INFINITY;
      l_part = 0.f;
    }
    f32x4 s0 = {}, s1 = {}, t0 = {}, t1 = {};  // rows 0..15 / 16..31 x Q hi / Q lo
    const uint32_t la = (uint32_t)(tb - lds0) + lgm.lat();
    const uint32_t ra = (uint32_t)(tb - lds0) + lgm.rope();
    auto cat = [](const u32x4& x, const u32x4& y) {
      return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                   (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
    };
    auto rd32 = [&](uint32_t a0) {  // two 16-byte LDS reads (a0, a0 ^ 16) -> 32 bytes
      return cat(*(const u32x4*)(lds0 + a0), *(const u32x4*)(lds0 + (a0 ^ 16)));
    };
    // Q lo of chunk v: two lane-contiguous 16-byte reads
    auto ldl = [&](int v) { return cat(sh.qlo[wave][v][0][lane], sh.qlo[wave][v][1][lane]); };
    // K operand of latent step st = 2v + b: chunk v, row block b
    auto ldk = [&](int st) {
      const int v = st >> 1, b = st & 1;
      return rd32(b ? ((la ^ 192) + 16 * kLatBytes) ^ (128 * v) : la ^ (128 * v));
    };
    // eight latent steps (chunk, row block); the next step's K, and at even steps
    // the next chunk's Q lo, are read one step ahead; the RoPE operands are read
    // during the last two steps
    i32x8 kc = ldk(0), ql = ldl(0), qn = {};
    u32x4 kr0 = {}, kr1 = {}, qr = {};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int v = st >> 1;
      i32x8 kn = {};
      if (st + 1 < 8) kn = ldk(st + 1);
      if ((st & 1) == 0 && v + 1 < 4) qn = ldl(v + 1);
      if (st == 6) {
        kr0 = *(const u32x4*)(lds0 + ra);
        kr1 = *(const u32x4*)(lds0 + ra + 16 * kRopeBytes);
        qr = sh.qlo_r[wave][lane];
      }
      if (st & 1) {
        s1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kc, qh[v], s1, 0, 0, 0, 127, 0, 127);
        t1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kc, ql, t1, 0, 0, 0, 127, 0, 127);
        ql = qn;
      } else {
        s0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kc, qh[v], s0, 0, 0, 0, 127, 0, 127);
        t0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kc, ql, t0, 0, 0, 0, 127, 0, 127);
      }
      kc = kn;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const long k0 = __builtin_bit_cast(long, u32x2{kr0[2 * e], kr0[2 * e + 1]});
      const long k1 = __builtin_bit_cast(long, u32x2{kr1[2 * e], kr1[2 * e + 1]});
      const long qa = __builtin_bit_cast(long, qhr[e]);
      const long qb = __builtin_bit_cast(long, u32x2{qr[2 * e], qr[2 * e + 1]});
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(k0, qa, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(k1, qa, s1, 0, 0, 0);
      t0 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(k0, qb, t0, 0, 0, 0);
      t1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(k1, qb, t1, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // K and Q lo of step 0
#pragma unroll
    for (int v = 0; v < 3; ++v) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // K of step 2v+1, Q lo of chunk v+1
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMAs (step 2v)
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // K of step 2v+2
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMAs (step 2v+1)
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);  // K of step 7, RoPE K and Q lo
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMAs (step 6)
    __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);  // step 7 and the RoPE steps
    __builtin_amdgcn_sched_barrier(0);
    s0 += t0;
    s1 += t1;
    // online softmax: lane holds head l16, tokens 4g4+r (s0) and 16+4g4+r (s1)
    const int nvalid = d & 0xff;
    if ((d & kBad) && lane == 0 && err) atomicOr(err, MLA_DEVERR_BLOCK);
    if (nvalid < kTile) {
      const int lim = nvalid - 4 * g4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r >= lim) s0[r] = -INFINITY;
        if (r >= lim - 16) s1[r] = -INFINITY;
      }
    }
    const float mx = head_max(fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                                    fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3]))));
    const float mt = mx * qs2;
    float alpha = 1.f;
    if (mt > m_run + kRescale) {
      alpha = __builtin_amdgcn_exp2f(m_run - mt);
      m_run = mt;
      l_part *= alpha;
    }
    float pr[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], qs2, -m_run));
      pr[4 + r] = __builtin_amdgcn_exp2f(fmaf(s1[r], qs2, -m_run));
    }
    l_part += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
    // P^T fragment of head block wk: k slots 0..3 = tokens 4g4+r, 4..7 = 16+4g4+r
    sh.pbuf[team][wk][lane] = u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                                    pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
    if (g4 == 0) sh.alpha[team][wk][l16] = alpha;
    if (d & kLastOfSeg) {
      const float l_tot = head_sum(l_part);
      if (g4 == 0) sh.invl[team][wk][l16] = kv_scale * __builtin_amdgcn_rcpf(l_tot);
      if (!(d & kWhole)) {
        const int slot = 2 * w + ((d & kSecondSlot) ? 1 : 0);
        const buf_t lse = buf_rsrc((char*)ws_lse + (int64_t)uni(slot) * (kH * 4), kH * 4);
        const uint32_t tid = opaque(threadIdx.x);
        const uint32_t hd = ((tid >> 8) << 6) + (((tid >> 6) & 3) << 4) + (tid & 15);
        if (g4 == 0)
          buf_store_b32(__float_as_uint(m_run + __builtin_amdgcn_logf(l_tot)), lse, 4 * hd, 0);
      }
    }
  };

  // ---------------------------------------------------------------- P phase
  auto value_phase = [&](int i, int d, int tok) {
    const char* tb = sh.tiles[i % kNBuf];
    const LaneGeom lgm(opaque(threadIdx.x));
    const int lane = lgm.lane, l16 = lgm.l16, g4 = lgm.g4;
    const f32x4 al = {sh.alpha[team][0][l16], sh.alpha[team][1][l16], sh.alpha[team][2][l16],
                      sh.alpha[team][3][l16]};
    bf16x8 pb[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) pb[h] = __builtin_bit_cast(bf16x8, sh.pbuf[team][h][lane]);
    const bool first = (d & kFirstOfSeg) != 0;
    const bool resc =
        !first && __ballot((al[0] != 1.f) | (al[1] != 1.f) | (al[2] != 1.f) | (al[3] != 1.f)) != 0;
    const uint32_t va0 = (uint32_t)(tb - lds0) + lgm.val(wk);
    i32x2 vr[4];
    auto ldv = [&](int f) {
      return __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(lds0 + (va0 ^ (f << 4))));
    };
    vr[0] = ldv(0);
    vr[1] = ldv(1);
    vr[2] = ldv(2);
    if (first) {
#pragma unroll
      for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int h = 0; h < 4; ++h) acc[f][h] = f32x4{};
    } else if (resc) {
#pragma unroll
      for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int h = 0; h < 4; ++h) acc[f][h] *= al[h];
    }
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f + 3 < 8) vr[(f + 3) & 3] = ldv(f + 3);
      const bf16x8 va = widen_fp8x8(vr[f & 3]);
#pragma unroll
      for (int h = 0; h < 4; ++h)
        acc[f][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[h], acc[f][h], 0, 0, 0);
    }
#pragma unroll
    for (int f = 0; f < 5; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read (block f+3)
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // 4 MFMAs (block f)
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
    if (d & kLastOfSeg) {
      const f32x4 inv = {sh.invl[team][0][l16], sh.invl[team][1][l16], sh.invl[team][2][l16],
                         sh.invl[team][3][l16]};
      uint16_t* base;
      if (d & kWhole) {
        base = o_lat + (int64_t)tok * kH * kDC;
      } else {
        const int slot = 2 * w + ((d & kSecondSlot) ? 1 : 0);
        base = ws_o + (int64_t)uni(slot) * kH * kDC;
      }
      // lane holds features 16(8wk+f) + 4g4 + r of head 64team + 16h + l16
      const buf_t out = buf_rsrc(base, kH * kDC * 2);
      const uint32_t voff = ((64 * team + l16) * kDC + 128 * wk + 4 * g4) * 2;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
#pragma unroll
        for (int f = 0; f < 8; ++f)
          buf_store_b64(pack_bf16x2(acc[f][h][0] * inv[h], acc[f][h][1] * inv[h]),
                        pack_bf16x2(acc[f][h][2] * inv[h], acc[f][h][3] * inv[h]), out, voff,
                        16 * h * kDC * 2 + 32 * f);
      }
    }
  };

  // ---------------------------------------------------------------- schedule
  // As in the bf16 kernel: phase 2i, team 0 scores tile i while team 1 runs the
  // values of tile i-1; phase 2i+1, team 0 runs the values of tile i while team
  // 1 scores it.  Team 0 keeps three tiles ahead, team 1 two.
  {
    const int t0 = uni(lg.c.t);
    const int pro = team == 0 ? kNBuf - 1 : kNBuf - 2;
    for (int k = 0; k < pro && lg.valid; ++k) {
      issue();
      advance();
    }
    load_q(t0);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  }
  int d_prev = 0, t_prev = 0;
  for (int i = 0;; ++i) {
    const bool has = i < issued;
    const int d_i = has ? desc_of(i) : 0, t_i = has ? tok_of(i) : 0;
    if (has) wait_vm(nmine * (issued - i - 1));
    barrier();
    if (team == 1) {
      if (has && i > 0 && (d_i & kFirstOfSeg)) load_q(t_i);
      if (lg.valid) issue();  // tile i+2
      if (i > 0) value_phase(i - 1, d_prev, t_prev);
    } else if (has) {
      __builtin_amdgcn_s_setprio(2);
      score_phase(i, d_i);
      advance();
      __builtin_amdgcn_s_setprio(0);
    }
    const int d_next = i + 1 < issued ? desc_of(i + 1) : 0;
    barrier();
    if (!has) break;
    if (team == 0) {
      if (i + 1 < issued && (d_next & kFirstOfSeg)) load_q(tok_of(i + 1));
      if (lg.valid) issue();  // tile i+3
      value_phase(i, d_i, t_i);
    } else {
      __builtin_amdgcn_s_setprio(2);
      score_phase(i, d_i);
      advance();
      __builtin_amdgcn_s_setprio(0);
    }
    d_prev = d_i;
    t_prev = t_i;
  }
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeArgs& a, float kv_scale, hipStream_t st) {
  hipLaunchKernelGGL(decode_fp8_kernel, dim3(a.plan.G), dim3(512), 0, st, a.plan.q_start,
                     a.plan.kv_lens, a.block_table, (const uint8_t*)a.pool,
                     (const uint16_t*)a.q_lat, (uint16_t*)a.o_lat, (uint16_t*)a.ws_o, a.ws_lse,
                     a.err, a.plan.B, a.plan.T, a.plan.causal, a.plan.G, a.plan.U, a.max_blocks,
                     a.num_blocks, a.scale_log2, kv_scale);
  return hipGetLastError();
}

}  // namespace mla

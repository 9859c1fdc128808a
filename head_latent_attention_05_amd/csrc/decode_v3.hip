// Split-KV absorbed latent attention for DeepSeek-V3 shapes on gfx950 MFMA.
//
// [MLA explainer] stage 2B / forward_inference_absorbed: per head, score =
// (q_lat . c_kv + q_pe . k_pe) * scale, softmax, o_lat = sum p * c_kv; all 128
// heads share one cached row of 576 values ([MLA architecture] section 1, 3.2).
// "MLA的常见问题" Q4 notes the 512 + 64 contraction does not fit square
// attention tiles; here the row is one 576-deep contraction for the scores and
// its first 512 columns are the values.
//
// Two workgroups (4 waves each) per KV range of the split plan, one per half of
// the 128 heads; both run on the same XCD, so each cache tile comes from HBM
// once and from L2 the second time.  Per 32-token tile, wave w:
//   scores for heads 16w..16w+15 of its half:
//     S^T[32 tok x 16 heads] = K[32 x 576] . Q^T[576 x 16]  (36 MFMA 16x16x32 bf16);
//     K rows come from LDS (16-byte reads), Q^T stays in registers for the
//     whole segment of a query token;
//   online softmax: a lane owns one head (4 lanes per head, 8 tokens each);
//     the tile max and the sums reduce with cross-lane swaps; rescaling is lazy
//     (only when the running max grows by more than 2^8), which leaves the
//     result unchanged;  P^T (bf16) and the rescale factors go to LDS;
//   values for features 128w..128w+127 of all 64 heads:
//     O^T[128 x 64] += V^T[128 x 32 tok] . P^T[32 tok x 64 heads]  (32 MFMA);
//     V^T operands come from the same LDS tile through the gfx950 transposing
//     read (ds_read_b64_tr_b16); splitting this product by feature makes every
//     V element leave LDS once per workgroup instead of once per wave.
//   The token (k) index of the value product is permuted so that P^T is the
//   score accumulator converted to bf16 in place.
// Tiles stream HBM -> LDS with direct-to-LDS loads (global_load_lds_dwordx4),
// four 36 KiB buffers, three tiles in flight.  In LDS a tile is split in two
// regions: the 32 latent rows (1 KiB each, one load instruction per row) and the
// 32 RoPE rows (128 B each, 8 rows per instruction); 16-byte chunks are
// XOR-swizzled per row so that the row reads (16 lanes per LDS cycle) and the
// transposing reads (32 lanes per cycle) hit 64 distinct banks.
#include <math.h>

#include "gfx950_asm.h"
#include "plan_device.h"

namespace mla {
namespace {

constexpr int kH = 128;
constexpr int kDC = 512;
constexpr int kRow = 576;
constexpr int kBS = 64;
constexpr int kTile = 32;
constexpr int kRowBytes = kRow * 2;                      // 1152
constexpr int kChunksPerRow = kRowBytes / 16;            // 72
constexpr int kTileChunks = kTile * kChunksPerRow;       // 2304
constexpr int kTileBytes = kTileChunks * 16;             // 36864
constexpr int kNBuf = 4;
constexpr float kRescale = 8.0f;                         // lazy rescale threshold (log2)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

static_assert(kTileChunks % 256 == 0, "tile must split evenly over 4 waves");

constexpr int kLatBytes = kDC * 2;                       // 1024: latent part of a row
constexpr int kRopeBytes = kRowBytes - kLatBytes;        // 128: RoPE part of a row
constexpr int kRegionB = kTile * kLatBytes;              // 32768: start of the RoPE region

// Chunk swizzles (chosen by measuring LDS throughput of both read patterns on
// gfx950).  Latent region: chunk c of row t sits at c ^ fa(t), which spreads the
// 16 rows of a score read and the 8 rows of a transposing read over distinct
// banks.  RoPE region: chunk c of row t sits at c ^ fb(t).
__device__ __forceinline__ int fa(int t) { return (t & 7) << 1; }
__device__ __forceinline__ int fb(int t) { return (t >> 1) & 7; }

// Wait until at most 9*ahead of this wave's vector-memory operations are
// outstanding (they complete in order), i.e. the tile that is `ahead` tiles
// older than the newest issued one has landed in LDS.
__device__ __forceinline__ void wait_tiles(int ahead) {
  if (ahead >= 2)
    __builtin_amdgcn_s_waitcnt((0x3f70 & ~0xf) | (18 & 0xf) | ((18 >> 4) << 14));
  else if (ahead == 1)
    __builtin_amdgcn_s_waitcnt((0x3f70 & ~0xf) | 9);
  else
    __builtin_amdgcn_s_waitcnt(0x3f70);
}

// Per-tile descriptor handed from the loader walk to the compute loop.
enum : int { kFirstOfSeg = 1 << 8, kLastOfSeg = 1 << 9, kWhole = 1 << 10, kBad = 1 << 11 };

// Walks the tiles (half cache blocks) of one workgroup's unit range in order.
// All fields are wave-uniform.  The block-table entry of the tile to issue next
// is loaded one step ahead (blk_raw), so its latency hides behind a tile of work.
struct Loader {
  TokenCursor c;
  int u1;
  int ub, ub_beg, ub_end;  // block range of the current segment (within the token)
  int half;
  int rows;     // valid rows of the current block
  int nvalid;   // valid rows of the current tile (1..32)
  int blk_raw;  // block-table entry of the current block
  int valid;
  int first;    // first tile of a segment

  __device__ __forceinline__ void fill(const PlanArgs& p, const int32_t* bt, int stride,
                                       bool new_block) {
    const int A = p.causal ? c.L - c.q + c.j + 1 : c.L;
    rows = uni(min(kBS, A - ub * kBS));
    nvalid = min(kTile, rows - kTile * half);
    if (new_block) blk_raw = ldc(bt, c.b * stride + ub);  // host keeps B*stride < 2^31
  }
  __device__ __forceinline__ void init(const PlanArgs& p, const int32_t* bt, int stride, int u0,
                                       int u1_) {
    u1 = u1_;
    c = locate_unit(p, u0);
    ub = ub_beg = u0 - c.ts;
    ub_end = uni(min(u1, c.ts + c.nu) - c.ts);
    half = 0;
    valid = 1;
    first = 1;
    fill(p, bt, stride, true);
  }
  __device__ __forceinline__ bool last_of_segment() const {
    return ub == ub_end - 1 && (half == 1 || rows <= kTile);
  }
  __device__ __forceinline__ bool whole_token() const { return ub_beg == 0 && ub_end == c.nu; }
  __device__ __forceinline__ void next(const PlanArgs& p, const int32_t* bt, int stride) {
    first = 0;
    if (half == 0 && rows > kTile) {
      half = 1;
      fill(p, bt, stride, false);
      return;
    }
    half = 0;
    ++ub;
    if (ub == ub_end) {
      if (c.ts + c.nu >= u1) {
        valid = 0;
        return;
      }
      cursor_next(p, c);
      ub = ub_beg = 0;
      ub_end = uni(min(u1, c.ts + c.nu) - c.ts);
      first = 1;
    }
    fill(p, bt, stride, true);
  }
};

// Issue this wave's 9 direct-to-LDS loads of one tile.  Load i (0..35) moves the
// latent part of row i (i < 32) or the RoPE parts of rows 8(i-32)..8(i-32)+7;
// waves 0-2 issue latent rows 9w..9w+8, wave 3 rows 27..31 and the 4 RoPE loads.
// Rows past the end of a partial tile repeat its last valid row (their scores
// are masked).
template <int W>
__device__ __forceinline__ void issue_tile_w(const char* blk, int last, char* lds_buf, int lane) {
  // rows are compile-time constants here, which keeps the address arithmetic
  // out of long-lived scalar registers
  constexpr int kFirst = 9 * W, kEnd = W < 3 ? 9 * W + 9 : kTile;
#pragma unroll
  for (int i = kFirst; i < kEnd; ++i)
    dma16(blk + min(i, last) * kRowBytes, (uint32_t)((lane ^ fa(i)) << 4), lds_buf + i * 1024);
  if (W == 3) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 8 * j + (lane >> 3);
      const uint32_t voff = min(t, last) * kRowBytes + kLatBytes + (((lane & 7) ^ fb(t)) << 4);
      dma16(blk, voff, lds_buf + (32 + j) * 1024);
    }
  }
}

__device__ __forceinline__ void issue_tile(const char* blk, int last, char* lds_buf, int wave,
                                           int lane) {
  switch (wave) {
    case 0: issue_tile_w<0>(blk, last, lds_buf, lane); break;
    case 1: issue_tile_w<1>(blk, last, lds_buf, lane); break;
    case 2: issue_tile_w<2>(blk, last, lds_buf, lane); break;
    default: issue_tile_w<3>(blk, last, lds_buf, lane); break;
  }
}

// max / sum over the 4 lanes that share a head (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float head_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float head_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__global__ __launch_bounds__(256, 1) void decode_v3_kernel(
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ block_table, const uint16_t* __restrict__ pool,
    const uint16_t* __restrict__ qlat, uint16_t* __restrict__ o_lat, uint16_t* __restrict__ ws_o,
    float* __restrict__ ws_lse, uint32_t* __restrict__ err, int B, int T, int causal, int G,
    int64_t U, int max_blocks, int64_t num_blocks, float sl2) {
  __shared__ __attribute__((aligned(1024))) char lds[kNBuf * kTileBytes];
  __shared__ __attribute__((aligned(16))) u32x4 pbuf[4][64];  // P^T fragments [wave][lane]
  __shared__ __attribute__((aligned(16))) float alpha_s[16][4];  // [head % 16][head / 16]
  __shared__ __attribute__((aligned(16))) float invl_s[16][4];
  __shared__ int descs[4][kNBuf][2];  // [wave][tile % 4] = {descriptor, token}
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  PlanArgs p;
  p.q_start = q_start;
  p.kv_lens = kv_lens;
  p.B = B;
  p.T = T;
  p.block_size = kBS;
  p.causal = causal;
  p.G = G;
  p.U = U;
  // Two workgroups per KV range, one per half of the heads.  Block ids are dealt
  // round-robin over the 8 XCDs; the mapping keeps both halves of a range, and
  // consecutive ranges, on one XCD so they share its L2 (tiles, query, partials).
  int w, hh;
  if ((G & 7) == 0) {
    const int x = blockIdx.x & 7, r = blockIdx.x >> 3;
    hh = r & 1;
    w = x * (G >> 3) + (r >> 1);
  } else {
    hh = blockIdx.x & 1;
    w = blockIdx.x >> 1;
  }
  const int u0 = (int)range_start(w, U, G), u1 = (int)range_start(w + 1, U, G);
  if (u0 >= u1) return;

  const int l16 = lane & 15;  // head within a 16-head block (MFMA column)
  const int g4 = lane >> 4;   // 16-lane group
  const int shead = hh * 64 + wave * 16 + l16;  // head this lane scores

  // score reads (A operand = K rows): row l16 (+16 for the second token block),
  // latent chunk 4kk + g4 (kk < 16) or RoPE chunk 4(kk-16) + g4 (kk = 16, 17);
  // fa only touches chunk bits 1..3, so chunk 4kk + g4 sits at
  // 16*(kk >> 2) + ((4*(kk & 3) + g4) ^ fa).
  int offA[4], offB[2];
#pragma unroll
  for (int r = 0; r < 4; ++r) offA[r] = l16 * kLatBytes + (((4 * r + g4) ^ fa(l16)) * 16);
#pragma unroll
  for (int r = 0; r < 2; ++r)
    offB[r] = kRegionB + l16 * kRopeBytes + (((4 * r + g4) ^ fb(l16)) * 16);
  // transposing reads (A operand = V^T) for feature block f = 8*wave + f7: group
  // g4 reads rows 4*g4 + (l16>>2) (+16 for the second read) at features
  // 16f + 4(l16&3), i.e. chunk 2f + ((l16>>1)&1), swizzled to
  // 2((f & 7) ^ (fa >> 1)) + c1 + 16(f >> 3).
  const int trow = 4 * g4 + (l16 >> 2);
  const int c1 = (l16 >> 1) & 1;
  int offV[8];  // [f7]; + 16 KiB for the second read as an immediate
#pragma unroll
  for (int f7 = 0; f7 < 8; ++f7)
    offV[f7] = trow * kLatBytes + (((2 * f7 + c1) ^ fa(trow)) * 16) + 8 * (l16 & 1) + wave * 256;

  const char* pool_b = (const char*)pool;
  Loader lg;
  lg.init(p, block_table, max_blocks, u0, u1);
  int issued = 0;
#define ISSUE_NEXT()                                                                        \
  do {                                                                                      \
    const int k_ = issued % kNBuf;                                                          \
    const int bad_ = uni(lg.blk_raw < 0 || lg.blk_raw >= num_blocks);                       \
    const int phys_ = uni(bad_ ? 0 : lg.blk_raw);                                           \
    const char* blk_ = pool_b + ((int64_t)phys_ * kBS + lg.half * kTile) * kRowBytes;       \
    issue_tile(blk_, bad_ ? 0 : lg.nvalid - 1, lds + k_ * kTileBytes, wave, lane);          \
    if (lane == 0) {                                                                        \
      descs[wave][k_][0] = (bad_ ? 0 : lg.nvalid) | (lg.first ? kFirstOfSeg : 0) |          \
                           (lg.last_of_segment() ? kLastOfSeg : 0) |                        \
                           (lg.whole_token() ? kWhole : 0) | (bad_ ? kBad : 0);             \
      descs[wave][k_][1] = lg.c.t;                                                          \
    }                                                                                       \
    lg.next(p, block_table, max_blocks);                                                    \
    ++issued;                                                                               \
  } while (0)
#pragma unroll
  for (int k = 0; k < kNBuf - 1; ++k)
    if (lg.valid) ISSUE_NEXT();

  u32x4 qreg[18];
  f32x4 acc[8][4];  // [feature block][head block]
  float m_run = -INFINITY, l_part = 0.f;
  int slot_first = 1;

  for (int tile = 0; tile < issued; ++tile) {
    const int d = uni(descs[wave][tile % kNBuf][0]);
    const int tok = uni(descs[wave][tile % kNBuf][1]);
    if (d & kFirstOfSeg) {
      const u32x4* qp = (const u32x4*)(qlat + ((int64_t)tok * kH + shead) * kRow + 8 * g4);
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) qreg[kk] = qp[4 * kk];
      // wait here for the query (this also drains the tiles in flight, once per
      // segment) so no wait on it is needed inside the tile loop
      __builtin_amdgcn_s_waitcnt(0x3f70);
#pragma unroll
      for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int h = 0; h < 4; ++h) acc[f][h] = f32x4{};
      m_run = -INFINITY;
      l_part = 0.f;
    }
    wait_tiles(issued - tile - 1);
    barrier();
    if (lg.valid) ISSUE_NEXT();
    const char* tb = lds + (tile % kNBuf) * kTileBytes;

    // ---- scores S^T = K . Q^T, two 16-token blocks.  The 36 K operands are read
    // in 3 groups of 6 k-steps, the next group in flight while the current one
    // feeds the MFMAs (the LDS read latency is far longer than one MFMA).
    f32x4 s0 = {}, s1 = {}, s2 = {}, s3 = {};
    u32x4 kb[2][12];
    auto load_group = [&](int g, u32x4* dst) {
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        const int kk = 6 * g + i;
        if (kk < 16) {
          dst[2 * i] = *(const u32x4*)(tb + offA[kk & 3] + (kk >> 2) * 256);
          dst[2 * i + 1] = *(const u32x4*)(tb + offA[kk & 3] + (kk >> 2) * 256 + 16 * kLatBytes);
        } else {
          dst[2 * i] = *(const u32x4*)(tb + offB[kk - 16]);
          dst[2 * i + 1] = *(const u32x4*)(tb + offB[kk - 16] + 16 * kRopeBytes);
        }
      }
    };
    load_group(0, kb[0]);
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      if (g < 2) load_group(g + 1, kb[(g + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        const int kk = 6 * g + i;
        const bf16x8 qb = __builtin_bit_cast(bf16x8, qreg[kk]);
        const bf16x8 a0 = __builtin_bit_cast(bf16x8, kb[g & 1][2 * i]);
        const bf16x8 a1 = __builtin_bit_cast(bf16x8, kb[g & 1][2 * i + 1]);
        if (i & 1) {
          s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qb, s2, 0, 0, 0);
          s3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qb, s3, 0, 0, 0);
        } else {
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qb, s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qb, s1, 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    s0 += s2;
    s1 += s3;

    // ---- online softmax: lane holds head l16, tokens 4*g4+i (s0) and 16+4*g4+i (s1)
    const int nvalid = d & 0xff;
    if ((d & kBad) && threadIdx.x == 0 && err) atomicOr(err, MLA_DEVERR_BLOCK);
    if (nvalid < kTile) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * g4 + i >= nvalid) s0[i] = -INFINITY;
        if (16 + 4 * g4 + i >= nvalid) s1[i] = -INFINITY;
      }
    }
    const float mx = head_max(fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                                    fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3]))));
    const float mt = mx * sl2;
    float alpha = 1.f;
    if (mt > m_run + kRescale) {
      alpha = exp2f(m_run - mt);
      m_run = mt;
      l_part *= alpha;
    }
    float pr[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = exp2f(fmaf(s0[i], sl2, -m_run));
      pr[4 + i] = exp2f(fmaf(s1[i], sl2, -m_run));
    }
    l_part += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
    // P^T fragment for head block `wave`: k slots 0..3 = tokens 4*g4+i, 4..7 = 16+4*g4+i
    pbuf[wave][lane] = u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                             pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
    if (g4 == 0) alpha_s[l16][wave] = alpha;
    if (d & kLastOfSeg) {
      const float l_tot = head_sum(l_part);
      if (g4 == 0) {
        invl_s[l16][wave] = 1.f / l_tot;
        if (!(d & kWhole)) {
          const int64_t slot = slot_first ? 2 * (int64_t)w : 2 * (int64_t)w + 1;
          ws_lse[slot * kH + shead] = m_run + log2f(l_tot);
        }
      }
    }
    barrier();  // P^T fragments and rescale factors of all 64 heads are in LDS

    // ---- O^T[128w.., 64 heads] += V^T . P^T
    const f32x4 al = *(const f32x4*)&alpha_s[l16][0];
    const bool resc = (al[0] != 1.f) | (al[1] != 1.f) | (al[2] != 1.f) | (al[3] != 1.f);
    if (__ballot(resc) != 0) {
#pragma unroll
      for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int h = 0; h < 4; ++h) acc[f][h] *= al[h];
    }
    bf16x8 pb[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) pb[h] = __builtin_bit_cast(bf16x8, pbuf[h][lane]);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(tb + offV[f]));
      const i16x4 v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(tb + offV[f] + 16 * kLatBytes));
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4,
                                                                           5, 6, 7));
#pragma unroll
      for (int h = 0; h < 4; ++h)
        acc[f][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[h], acc[f][h], 0, 0, 0);
    }

    // ---- end of a segment: normalise and write the output or a partial
    if (d & kLastOfSeg) {
      const f32x4 inv = *(const f32x4*)&invl_s[l16][0];
      uint16_t* base;
      if (d & kWhole) {
        base = o_lat + ((int64_t)tok * kH + hh * 64) * kDC;
      } else {
        const int64_t slot = slot_first ? 2 * (int64_t)w : 2 * (int64_t)w + 1;
        base = ws_o + (slot * kH + hh * 64) * kDC;
      }
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        uint16_t* row = base + (16 * h + l16) * kDC + 128 * wave + 4 * g4;
#pragma unroll
        for (int f = 0; f < 8; ++f) {
          u32x2 v;
          v.x = pack_bf16x2(acc[f][h][0] * inv[h], acc[f][h][1] * inv[h]);
          v.y = pack_bf16x2(acc[f][h][2] * inv[h], acc[f][h][3] * inv[h]);
          *(u32x2*)(row + 16 * f) = v;
        }
      }
      slot_first = 0;
    }
  }
}

}  // namespace

bool v3_kernels_available() { return true; }

hipError_t launch_decode_v3(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(decode_v3_kernel, dim3(2 * a.plan.G), dim3(256), 0, st,
      a.plan.q_start, a.plan.kv_lens, a.block_table, (const uint16_t*)a.pool,
      (const uint16_t*)a.q_lat, (uint16_t*)a.o_lat, (uint16_t*)a.ws_o, a.ws_lse, a.err, a.plan.B,
      a.plan.T, a.plan.causal, a.plan.G, a.plan.U, a.max_blocks, a.num_blocks, a.scale_log2);
  return hipGetLastError();
}

}  // namespace mla

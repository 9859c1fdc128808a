// Split-KV absorbed latent attention for DeepSeek-V3 shapes on gfx950 MFMA.
//
// [MLA explainer] stage 2B / forward_inference_absorbed: per head, score =
// (q_lat . c_kv + q_pe . k_pe) * scale, softmax, o_lat = sum p * c_kv; all 128
// heads share one cached row of 576 values ([MLA architecture] section 1, 3.2).
// "MLA的常见问题" Q4 notes the 512 + 64 contraction does not fit square
// attention tiles; here the row is one 576-deep contraction for the scores and
// its first 512 columns are the values.
//
// One workgroup (4 waves) per KV range of the split plan; it owns all 128 heads
// of a query token (wave w: heads 32w..32w+31), so the cache is read from HBM
// exactly once per query token.  Per 32-token tile:
//   S^T[32 tok x 32 heads] = K[32 x 576] . Q^T[576 x 32]   (36 MFMA 32x32x16 bf16)
//       K rows come from LDS (16-byte reads); Q^T stays in registers for the
//       whole segment of a query token.
//   online softmax on S^T: every lane owns one head; the per-tile max needs one
//       cross-lane exchange (lanes l, l^32); rescaling is lazy (only when the
//       running max grows by more than 2^8), which leaves the result unchanged.
//   O^T[512 x 32 heads] += V^T[512 x 32 tok] . P^T[32 tok x 32 heads]
//       (32 MFMA); V^T operands come from the same LDS tile through the gfx950
//       transposing LDS read (ds_read_b64_tr_b16), and P^T is the S^T
//       accumulator converted to bf16 in place (no data movement) thanks to a
//       matching permutation of the token (k) index.
// Tiles stream HBM -> LDS with direct-to-LDS loads (global_load_lds_dwordx4),
// four 36 KiB buffers, three tiles in flight.  In LDS a tile is split in two
// regions: the 32 latent rows (1 KiB each, one load instruction per row) and the
// 32 RoPE rows (128 B each, 8 rows per instruction); 16-byte chunks are
// XOR-swizzled per row so that the row reads (16 lanes per LDS cycle) and the
// transposing reads (32 lanes per cycle) hit 64 distinct banks.
#include <math.h>

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
constexpr int kLoadsPerWave = kTileChunks / 256;         // 9 x 1 KiB per wave
constexpr float kRescale = 8.0f;                         // lazy rescale threshold (log2)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
#define LDS_AS __attribute__((address_space(3)))

static_assert(kTileChunks % 256 == 0, "tile must split evenly over 4 waves");

constexpr int kLatBytes = kDC * 2;                       // 1024: latent part of a row
constexpr int kRopeBytes = kRowBytes - kLatBytes;        // 128: RoPE part of a row
constexpr int kRegionB = kTile * kLatBytes;              // 32768: start of the RoPE region

// Chunk swizzles.  Latent region: chunk c of row t sits at c ^ fa(t); fa is a
// bijection on 16 consecutive rows (row reads) and fa >> 1 = t & 7 separates the
// 8 rows that one 32-lane transposing read touches.  RoPE region: chunk c of row
// t sits at c ^ fb(t).
__device__ __forceinline__ int fa(int t) { return 2 * (t & 7) + ((t >> 3) & 1); }
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

// Workgroup barrier without the memory fence that __syncthreads implies (that
// fence waits for every outstanding load, which would drain the tile pipeline);
// the explicit wait_tiles() before it orders the LDS data.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Per-tile descriptor handed from the loader walk to the compute loop.
enum : int { kFirstOfSeg = 1 << 8, kLastOfSeg = 1 << 9, kWhole = 1 << 10, kBad = 1 << 11 };

// Walks the tiles (half cache blocks) of one workgroup's unit range in order.
// All fields are wave-uniform.
struct TileGen {
  TokenCursor c;
  int u1;
  int ub, ub_beg, ub_end;  // block range of the current segment (within the token)
  int half;
  int rows;    // valid rows of the current block
  int nvalid;  // valid rows of the current tile (1..32)
  int phys;    // physical block id (0 if out of range)
  int bad;     // block id out of range: tile is fully masked
  int valid;
  int first;   // first tile of a segment

  __device__ __forceinline__ void fill(const PlanArgs& p, const int32_t* __restrict__ bt, int stride,
                       int64_t num_blocks) {
    const int A = p.causal ? c.L - c.q + c.j + 1 : c.L;
    rows = uni(min(kBS, A - ub * kBS));
    nvalid = min(kTile, rows - kTile * half);
    const int blk = uni(ldc(bt, c.b * stride + ub));  // the host keeps B*stride < 2^31
    bad = blk < 0 || blk >= num_blocks;
    phys = bad ? 0 : blk;
  }
  __device__ __forceinline__ void init(const PlanArgs& p, const int32_t* __restrict__ bt, int stride,
                       int64_t num_blocks, int u0, int u1_) {
    u1 = u1_;
    c = locate_unit(p, u0);
    ub = ub_beg = u0 - c.ts;
    ub_end = min(u1, c.ts + c.nu) - c.ts;
    half = 0;
    valid = 1;
    first = 1;
    fill(p, bt, stride, num_blocks);
  }
  __device__ __forceinline__ bool last_of_segment() const {
    return ub == ub_end - 1 && (half == 1 || rows <= kTile);
  }
  __device__ __forceinline__ bool whole_token() const { return ub_beg == 0 && ub_end == c.nu; }
  __device__ __forceinline__ int desc() const {
    return (bad ? 0 : nvalid) | (first ? kFirstOfSeg : 0) | (last_of_segment() ? kLastOfSeg : 0) |
           (whole_token() ? kWhole : 0) | (bad ? kBad : 0);
  }
  __device__ __forceinline__ void next(const PlanArgs& p, const int32_t* __restrict__ bt,
                                       int stride, int64_t num_blocks) {
    first = 0;
    if (half == 0 && rows > kTile) {
      half = 1;
    } else {
      half = 0;
      ++ub;
      if (ub == ub_end) {
        if (c.ts + c.nu >= u1) {
          valid = 0;
        } else {
          cursor_next(p, c);
          ub = ub_beg = 0;
          ub_end = uni(min(u1, c.ts + c.nu) - c.ts);
          first = 1;
        }
      }
    }
    if (valid) fill(p, bt, stride, num_blocks);
  }
};

// One 16-byte-per-lane direct-to-LDS load: lane l's 16 bytes from `src` land at
// lds_dst + 16*l.  Written as inline asm so the compiler does not treat every
// later LDS read as a possible reader of the in-flight data (it would then wait
// for all outstanding loads before each tile); ordering is explicit instead:
// wait_tiles() + barrier() before a tile is read.  The instruction has no
// destination register, only the address operand, which is read at issue.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is set here and used by nothing else
__device__ __forceinline__ void dma16(const char* src, char* lds_dst) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(LDS_AS char*)lds_dst;
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(m0v)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Issue this wave's 9 direct-to-LDS loads of one tile into `lds_buf`.  Load i
// (0..35, wave w issues 9w..9w+8): i < 32 moves the latent part of row i, i >= 32
// the RoPE parts of rows 8(i-32)..8(i-32)+7.  Rows past the end of a partial tile
// repeat its last valid row (their scores are masked).
__device__ __forceinline__ void issue_tile(const TileGen& g, const uint16_t* __restrict__ pool,
                                           char* lds_buf, int wave, int lane) {
  const char* blk = (const char*)(pool + ((int64_t)g.phys * kBS + g.half * kTile) * kRow);
  const int last = g.bad ? 0 : g.nvalid - 1;
#pragma unroll
  for (int k = 0; k < kLoadsPerWave; ++k) {
    const int i = wave * kLoadsPerWave + k;  // wave-uniform
    const char* src;
    if (i < kTile) {
      const int t = min(i, last);
      src = blk + t * kRowBytes + ((lane ^ fa(i)) * 16);
    } else {
      const int t = 8 * (i - kTile) + (lane >> 3);
      src = blk + min(t, last) * kRowBytes + kLatBytes + (((lane & 7) ^ fb(t)) * 16);
    }
    dma16(src, lds_buf + i * 1024);
  }
}

__global__ __launch_bounds__(256, 1) void decode_v3_kernel(
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ block_table, const uint16_t* __restrict__ pool,
    const uint16_t* __restrict__ qlat, uint16_t* __restrict__ o_lat, uint16_t* __restrict__ ws_o,
    float* __restrict__ ws_lse, uint32_t* __restrict__ err, int B, int T, int causal, int G,
    int64_t U, int max_blocks, int64_t num_blocks, float sl2) {
  __shared__ __attribute__((aligned(1024))) char lds[kNBuf * kTileBytes];
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

  const int l16 = lane & 15;  // head within the wave (MFMA column)
  const int g4 = lane >> 4;   // 16-lane group
  const int head = hh * 64 + wave * 16 + l16;

  // score reads (A operand = K rows): row l16 (+16 for the second token block),
  // latent chunk 4kk + g4 (kk < 16) or RoPE chunk 4(kk-16) + g4 (kk = 16, 17).
  int offA[4], offB[2];
#pragma unroll
  for (int r = 0; r < 4; ++r) offA[r] = l16 * kLatBytes + (((4 * r + g4) ^ fa(l16)) * 16);
#pragma unroll
  for (int r = 0; r < 2; ++r)
    offB[r] = kRegionB + l16 * kRopeBytes + (((4 * r + g4) ^ fb(l16)) * 16);
  // transposing reads (A operand = V^T): group g4 reads rows 4*g4 + (l16>>2)
  // (+16 for the second read) at features 16f + 4(l16&3): chunk 2f + ((l16>>1)&1),
  // swizzled to 2(f ^ tau) + (((l16>>1)&1) ^ beta).
  const int tau = (4 * (g4 & 1) + (l16 >> 2)) & 7;
  const int beta = g4 >> 1;
  const int trow = 4 * g4 + (l16 >> 2);
  int offV[8];  // [f & 7]; + 16 KiB (second read) + (f >> 3) * 256 as immediates
#pragma unroll
  for (int f7 = 0; f7 < 8; ++f7)
    offV[f7] = trow * kLatBytes + 32 * (f7 ^ tau) + 16 * (((l16 >> 1) & 1) ^ beta) + 8 * (l16 & 1);

  TileGen lg;
  lg.init(p, block_table, max_blocks, num_blocks, u0, u1);
  int issued = 0;
#pragma unroll
  for (int k = 0; k < kNBuf - 1; ++k) {
    if (lg.valid) {
      issue_tile(lg, pool, lds + k * kTileBytes, wave, lane);
      if (lane == 0) {
        descs[wave][k][0] = lg.desc();
        descs[wave][k][1] = lg.c.t;
      }
      lg.next(p, block_table, max_blocks, num_blocks);
      ++issued;
    }
  }

  u32x4 qreg[18];
  f32x4 acc[32];
  float m_run = -INFINITY, l_part = 0.f;
  int slot_first = 1;

  for (int tile = 0; tile < issued; ++tile) {
    const int d = uni(descs[wave][tile % kNBuf][0]);
    const int tok = uni(descs[wave][tile % kNBuf][1]);
    if (d & kFirstOfSeg) {
      const u32x4* qp = (const u32x4*)(qlat + ((int64_t)tok * kH + head) * kRow + 8 * g4);
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) qreg[kk] = qp[4 * kk];
      // wait here for the query (this also drains the tiles in flight, once per
      // segment) so no wait on it is needed inside the tile loop
      __builtin_amdgcn_s_waitcnt(0x3f70);
#pragma unroll
      for (int f = 0; f < 32; ++f) acc[f] = f32x4{};
      m_run = -INFINITY;
      l_part = 0.f;
    }
    wait_tiles(issued - tile - 1);
    barrier();
    if (lg.valid) {
      const int k = issued % kNBuf;
      issue_tile(lg, pool, lds + k * kTileBytes, wave, lane);
      if (lane == 0) {
        descs[wave][k][0] = lg.desc();
        descs[wave][k][1] = lg.c.t;
      }
      lg.next(p, block_table, max_blocks, num_blocks);
      ++issued;
    }
    const char* tb = lds + (tile % kNBuf) * kTileBytes;

    // ---- scores S^T = K . Q^T, two 16-token blocks
    f32x4 s0 = {}, s1 = {};
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) {
      u32x4 k0, k1;
      if (kk < 16) {
        k0 = *(const u32x4*)(tb + offA[kk & 3] + (kk >> 2) * 256);
        k1 = *(const u32x4*)(tb + offA[kk & 3] + (kk >> 2) * 256 + 16 * kLatBytes);
      } else {
        k0 = *(const u32x4*)(tb + offB[kk - 16]);
        k1 = *(const u32x4*)(tb + offB[kk - 16] + 16 * kRopeBytes);
      }
      const bf16x8 qb = __builtin_bit_cast(bf16x8, qreg[kk]);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k0), qb, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k1), qb, s1, 0, 0, 0);
    }
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
    float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                     fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mt = mx * sl2;
    const bool grow = mt > m_run + kRescale;
    if (__ballot(grow) != 0) {
      const float m_new = grow ? mt : m_run;
      const float alpha = exp2f(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int f = 0; f < 32; ++f) acc[f] *= alpha;
      m_run = m_new;
    }
    float pr[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = exp2f(fmaf(s0[i], sl2, -m_run));
      pr[4 + i] = exp2f(fmaf(s1[i], sl2, -m_run));
    }
    l_part += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
    // P^T as the B operand: k slots 0..3 = tokens 4*g4+i, 4..7 = 16+4*g4+i
    const u32x4 pb = {pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                      pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
    const bf16x8 pbb = __builtin_bit_cast(bf16x8, pb);

    // ---- O^T += V^T . P^T: 32 blocks of 16 features, k = the 32 tokens
#pragma unroll
    for (int f = 0; f < 32; ++f) {
      const int imm = (f >> 3) * 256;
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4*)(tb + offV[f & 7] + imm));
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4*)(tb + offV[f & 7] + imm + 16 * kLatBytes));
      const i16x8 va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), pbb,
                                                       acc[f], 0, 0, 0);
    }

    // ---- end of a segment: normalise and write the output or a partial
    if (d & kLastOfSeg) {
      float l_tot = l_part + __shfl_xor(l_part, 16, 64);
      l_tot += __shfl_xor(l_tot, 32, 64);
      const float inv = 1.f / l_tot;
      uint16_t* dst;
      if (d & kWhole) {
        dst = o_lat + ((int64_t)tok * kH + head) * kDC;
      } else {
        const int64_t slot = slot_first ? 2 * (int64_t)w : 2 * (int64_t)w + 1;
        dst = ws_o + (slot * kH + head) * kDC;
        if (g4 == 0) ws_lse[slot * kH + head] = m_run + log2f(l_tot);
      }
#pragma unroll
      for (int f = 0; f < 32; ++f) {
        u32x2 v;
        v.x = pack_bf16x2(acc[f][0] * inv, acc[f][1] * inv);
        v.y = pack_bf16x2(acc[f][2] * inv, acc[f][3] * inv);
        *(u32x2*)(dst + 16 * f + 4 * g4) = v;
      }
      slot_first = 0;
    }
  }
}

}  // namespace

bool v3_kernels_available() { return true; }

hipError_t launch_decode_v3(const DecodeArgs& a, hipStream_t st) {
  decode_v3_kernel<<<dim3(2 * a.plan.G), dim3(256), 0, st>>>(
      a.plan.q_start, a.plan.kv_lens, a.block_table, (const uint16_t*)a.pool,
      (const uint16_t*)a.q_lat, (uint16_t*)a.o_lat, (uint16_t*)a.ws_o, a.ws_lse, a.err, a.plan.B,
      a.plan.T, a.plan.causal, a.plan.G, a.plan.U, a.max_blocks, a.num_blocks, a.scale_log2);
  return hipGetLastError();
}

}  // namespace mla

// Split-KV absorbed latent attention for DeepSeek-V3 shapes on gfx950 MFMA.
//
// [MLA explainer] stage 2B / forward_inference_absorbed: per head, score =
// (q_lat . c_kv + q_pe . k_pe) * scale, softmax over the cached rows, o_lat =
// sum p * c_kv.  All 128 heads read the same cached row of 576 values
// ([MLA architecture] section 1, 3.2).  "MLA的常见问题" Q4: the contraction is
// 512 + 64 deep and does not fit square attention tiles; here a row is one
// 576-deep contraction for the scores, and its first 512 columns are the values.
//
// One workgroup per KV range of the split plan, all 128 heads, 8 waves: every
// cache tile goes from HBM into this CU's LDS exactly once.  The waves form two
// teams of four; team T owns heads 64T..64T+63.  Per 32-token tile a team runs
// two phases:
//   S: wave k scores heads 64T+16k..+15:
//        S^T[32 tok x 16 heads] = K[32 x 576] . Q^T[576 x 16] (36 MFMA 16x16x32),
//        K rows read from LDS, Q^T held in registers for the query token;
//      online softmax (a lane owns one head and 8 tokens, max / sum across the
//      4 lanes of a head with permlane swaps, lazy rescaling);
//      P^T (bf16) and the rescale factors of the team's heads go to LDS.
//   P: wave k multiplies the values of features 128k..128k+127 for the team's
//      64 heads: O^T[128 x 64] += V^T[128 x 32 tok] . P^T[32 tok x 64] (32 MFMA),
//      V^T from the same LDS tile through the transposing read ds_read_b64_tr_b16.
// The teams are half a tile apart: while team 0 scores tile i, team 1 runs the
// value product of tile i-1, and the other way round in the next phase.  Each
// SIMD holds one wave of each team, so one wave's MFMAs overlap the other's
// LDS reads and softmax, and the K reads of the score phase are spread over
// both phases.  A workgroup barrier separates phases.  The scoring wave runs at
// a raised issue priority: its chain of LDS reads and MFMAs is the longer one,
// and without it the SIMD favours the older wave, so team 1's score phases ran
// longest.
//
// Tiles (half cache blocks, 32 rows, 36 KiB) stream HBM -> LDS with
// direct-to-LDS loads (global_load_lds_dwordx4) into four buffers; every wave
// loads its own rows.  Team 0 issues its share of tile i+3 in phase 2i+1, team 1
// its share of tile i+2 in phase 2i, so two to two-and-a-half tiles are in
// flight.  A wave whose next score phase starts a new query token loads that
// token's Q during its value phase (its Q registers are idle then).
//
// LDS tile layout: the 32 latent rows (1 KiB each) then the 32 RoPE rows (128 B
// each); 16-byte chunks are XOR-swizzled per row so that the score reads (16
// rows x one chunk per LDS cycle) and the transposing reads hit distinct banks.
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
constexpr int kRowBytes = kRow * 2;                // 1152
constexpr int kLatBytes = kDC * 2;                 // 1024: latent part of a row
constexpr int kRopeBytes = kRowBytes - kLatBytes;  // 128: RoPE part of a row
constexpr int kTileBytes = kTile * kRowBytes;      // 36864
constexpr int kRegionB = kTile * kLatBytes;        // 32768: start of the RoPE region
constexpr int kNBuf = 4;
constexpr int kWaves = 8;
constexpr float kRescale = 8.0f;  // lazy rescale threshold (log2 units)

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Chunk swizzles.  Latent region: chunk c of row t sits at c ^ fa(t); RoPE
// region: chunk c of row t sits at c ^ fb(t).  fa only touches chunk bits 1..3.
__device__ __forceinline__ int fa(int t) { return (t & 7) << 1; }
__device__ __forceinline__ int fb(int t) { return (t >> 1) & 7; }

// This wave's direct-to-LDS loads of one tile: latent rows w, w+8, w+16, w+24
// (one 1 KiB load each) and, for waves 0-3, the RoPE parts of rows 8w..8w+7.
// Rows past the end of a partial tile repeat its last valid row (their scores
// are masked; repeating keeps every value finite).  All latent rows of a wave
// share one chunk swizzle (fa(w + 8r) = fa(w)), so one lane offset serves them;
// the RoPE offset is formed here from the lane id, at issue time, rather than
// kept in a register.
__device__ __forceinline__ void issue_rows(int wave, const char* blk, int last, char* buf,
                                           uint32_t lane) {
  const uint32_t lat_off = (lane ^ (uint32_t)fa(wave)) << 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = wave + 8 * r;
    dma16(blk + min(i, last) * kRowBytes, lat_off, buf + i * kLatBytes);
  }
  if (wave < 4) {
    const int t = 8 * wave + (int)(lane >> 3);
    const uint32_t voff =
        (uint32_t)(min(t, last) * kRowBytes + kLatBytes) + (((lane & 7) ^ (uint32_t)fb(t)) << 4);
    dma16(blk, voff, buf + kRegionB + wave * 1024);
  }
}

// Per-lane geometry of the MFMA operands (lane = 16 g4 + l16).  Tile buffers
// are 4 KiB aligned in the shared block and the chunk swizzles only touch
// offset bits 4..7, so every operand address is (tile base + lane part) ^ (a
// constant selecting the chunk):
//   score reads (A operand = K rows): row l16 (+16 rows for the second token
//   block), latent chunk 4kk + g4 -> (lat ^ ((kk & 3) << 6)) + 256 (kk >> 2),
//   RoPE chunk 4r + g4 (kk = 16 + r) -> rope ^ (r << 6);
//   transposing reads (A operand = V^T) of feature block 8wk + f: rows
//   4g4 + (l16 >> 2) (+16), features 16(8wk + f) + 4(l16 & 3), i.e. chunk
//   16wk + 2f + ((l16 >> 1) & 1) -> val ^ (f << 5).
struct LaneGeom {
  int lane, l16, g4;
  __device__ __forceinline__ explicit LaneGeom(uint32_t tid)
      : lane((int)(tid & 63)), l16((int)(tid & 15)), g4((int)((tid >> 4) & 3)) {}
  __device__ __forceinline__ uint32_t lat() const {
    const int f = fa(l16);
    return l16 * kLatBytes + (((f >> 2) & 3) << 6) + ((g4 ^ (f & 2)) << 4);
  }
  __device__ __forceinline__ uint32_t rope() const {
    return kRegionB + l16 * kRopeBytes + ((g4 ^ fb(l16)) << 4);
  }
  __device__ __forceinline__ uint32_t val(int wk) const {
    const int trow = 4 * g4 + (l16 >> 2);
    return trow * kLatBytes + ((fa(trow) >> 1) << 5) + (((l16 >> 1) & 1) << 4) + 8 * (l16 & 1) +
           wk * 256;
  }
};

struct Shared {
  char tiles[kNBuf][kTileBytes];
  u32x4 pbuf[2][4][64];     // P^T fragments [team][head block][lane]
  float alpha[2][4][16];    // rescale factor [team][head block][head % 16]
  float invl[2][4][16];     // 1 / softmax denominator, same layout
  int desc[kWaves][kNBuf][2];  // per wave: [tile % 4] = {flags | valid rows, token}
};

__global__ __launch_bounds__(512, 1) void decode_v4_kernel(
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ block_table, const uint16_t* __restrict__ pool,
    const uint16_t* __restrict__ qlat, uint16_t* __restrict__ o_lat, uint16_t* __restrict__ ws_o,
    float* __restrict__ ws_lse, uint32_t* __restrict__ err, int B, int T, int causal, int G,
    int64_t U, int max_blocks, int64_t num_blocks, float sl2) {
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
  // Block ids are dealt round-robin over the 8 XCDs; consecutive ranges (which
  // share a split token, its query and its partials) go to one XCD.
  int w = blockIdx.x;
  if ((G & 7) == 0) w = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int u0 = (int)range_start(w, U, G), u1 = (int)range_start(w + 1, U, G);
  if (u0 >= u1) return;

  // LDS addresses are byte offsets from the start of the shared block (see
  // LaneGeom); the lane-dependent parts are rebuilt inside each phase from the
  // lane id instead of being held in registers across the tile loop.
  const char* lds0 = (const char*)&sh;

  const char* pool_b = (const char*)pool;
  const int nmine = wave < 4 ? 5 : 4;  // direct-to-LDS loads per tile of this wave
  Loader lg;
  lg.init(p, block_table, max_blocks, u0, u1);
  int issued = 0;  // tiles this wave has issued
  bool pending_adv = false;  // the walk still describes the tile last issued

  u32x4 qreg[18];
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
  // Moves the walk to the next tile.  Its scalar loads (block table, lengths)
  // share a wait counter with LDS reads and may return out of order, so while
  // one is outstanding every LDS wait the compiler emits must be a full one;
  // waiting for them here, at the end of the short score phase, keeps the LDS
  // reads of the other phases pipelined.
  auto advance = [&]() {
    if (pending_adv) {
      lg.next(p, block_table, max_blocks);
      pending_adv = false;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  };
  auto desc_of = [&](int i) { return uni(sh.desc[wave][i % kNBuf][0]); };
  auto tok_of = [&](int i) { return uni(sh.desc[wave][i % kNBuf][1]); };
  // Q^T operand of this lane: head shead, columns 32kk + 8g4 .. +7.  The wait
  // for it drains this wave's tiles in flight as well (loads complete in
  // order); it sits right here so the compiler knows no load into qreg is
  // pending anywhere else and adds no waits of its own inside the tile loop.
  auto load_q = [&](int tok) {
    const LaneGeom lg_(opaque(threadIdx.x));
    const uint32_t q_lane = ((64 * team + 16 * wk + lg_.l16) * kRow + 8 * lg_.g4) * 2;
    const char* qb = (const char*)qlat + (int64_t)tok * (kH * kRow * 2) + q_lane;
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) qreg[kk] = *(const u32x4*)(qb + 64 * kk);
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
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
    f32x4 s0 = {}, s1 = {};
    u32x4 ka[3][2];  // K operands of k-steps kk .. kk+2
    const uint32_t la = (uint32_t)(tb - lds0) + lgm.lat();
    const uint32_t ra = (uint32_t)(tb - lds0) + lgm.rope();
    auto ld = [&](int kk, u32x4* dst) {
      const uint32_t a = kk < 16 ? (la ^ ((kk & 3) << 6)) + (kk >> 2) * 256 : ra ^ ((kk - 16) << 6);
      const int second = kk < 16 ? 16 * kLatBytes : 16 * kRopeBytes;
      dst[0] = *(const u32x4*)(lds0 + a);
      dst[1] = *(const u32x4*)(lds0 + a + second);
    };
    ld(0, ka[0]);
    ld(1, ka[1]);
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) {
      if (kk + 2 < 18) ld(kk + 2, ka[(kk + 2) % 3]);
      const bf16x8 qb = __builtin_bit_cast(bf16x8, qreg[kk]);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[kk % 3][0]), qb,
                                                   s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[kk % 3][1]), qb,
                                                   s1, 0, 0, 0);
    }
    // keep the K reads two k-steps ahead of the MFMAs that consume them
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads (k-steps 0, 1)
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMAs (k-step kk)
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads (k-step kk+2)
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
    // online softmax: lane holds head l16, tokens 4g4+r (s0) and 16+4g4+r (s1).
    // Weights are 2^(s*scale*log2(e) - m) on the hardware exp2 (v_exp_f32, ~1 ulp;
    // arguments below -126 flush to 0, which is below bf16 resolution of P anyway).
    const int nvalid = d & 0xff;
    if ((d & kBad) && lane == 0 && err) atomicOr(err, MLA_DEVERR_BLOCK);
    if (nvalid < kTile) {
      const int lim = nvalid - 4 * g4;  // rows 4g4 + r of s0 are valid for r < lim
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r >= lim) s0[r] = -INFINITY;
        if (r >= lim - 16) s1[r] = -INFINITY;
      }
    }
    const float mx = head_max(fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                                    fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3]))));
    const float mt = mx * sl2;
    float alpha = 1.f;
    if (mt > m_run + kRescale) {
      alpha = __builtin_amdgcn_exp2f(m_run - mt);
      m_run = mt;
      l_part *= alpha;
    }
    float pr[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], sl2, -m_run));
      pr[4 + r] = __builtin_amdgcn_exp2f(fmaf(s1[r], sl2, -m_run));
    }
    l_part += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
    // P^T fragment of head block wk: k slots 0..3 = tokens 4g4+r, 4..7 = 16+4g4+r
    sh.pbuf[team][wk][lane] = u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                                    pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
    if (g4 == 0) sh.alpha[team][wk][l16] = alpha;
    if (d & kLastOfSeg) {
      const float l_tot = head_sum(l_part);
      if (g4 == 0) sh.invl[team][wk][l16] = __builtin_amdgcn_rcpf(l_tot);
      if (!(d & kWhole)) {
        const int slot = 2 * w + ((d & kSecondSlot) ? 1 : 0);
        const buf_t lse = buf_rsrc((char*)ws_lse + (int64_t)uni(slot) * (kH * 4), kH * 4);
        // the lane offset is rebuilt here rather than kept live for this rare store
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
    // LDS reads first: the rescale factors of the team's heads (the decision
    // to rescale waits for them alone), the P^T fragments, and the V^T operands
    // of feature blocks 0..2, all in flight together; the loop below keeps
    // three feature blocks ahead (the transposing read's latency is several
    // MFMAs long).
    const f32x4 al = {sh.alpha[team][0][l16], sh.alpha[team][1][l16], sh.alpha[team][2][l16],
                      sh.alpha[team][3][l16]};
    bf16x8 pb[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) pb[h] = __builtin_bit_cast(bf16x8, sh.pbuf[team][h][lane]);
    const bool first = (d & kFirstOfSeg) != 0;
    const bool resc =
        !first && __ballot((al[0] != 1.f) | (al[1] != 1.f) | (al[2] != 1.f) | (al[3] != 1.f)) != 0;
    const uint32_t va0 = (uint32_t)(tb - lds0) + lgm.val(wk);
    i16x4 vr[4][2];
    auto ldv = [&](int f, i16x4* dst) {
      const char* vp = lds0 + (va0 ^ (f << 5));
      dst[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)vp);
      dst[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vp + 16 * kLatBytes));
    };
    ldv(0, vr[0]);
    ldv(1, vr[1]);
    ldv(2, vr[2]);
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
      if (f + 3 < 8) ldv(f + 3, vr[(f + 3) & 3]);
      const bf16x8 va = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(vr[f & 3][0], vr[f & 3][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int h = 0; h < 4; ++h)
        acc[f][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[h], acc[f][h], 0, 0, 0);
    }
    // keep the reads three blocks ahead of the MFMAs that consume them
#pragma unroll
    for (int f = 0; f < 5; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads (block f+3)
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
  // Phase 2i: team 0 scores tile i, team 1 multiplies the values of tile i-1;
  // phase 2i+1: team 0 multiplies the values of tile i, team 1 scores it.
  // Tile j is first read in phase 2j; every wave waits for its own loads of it
  // before the barrier that opens that phase.  A wave issues its share of its
  // next tile in each of its value phases (team 0 tile i+3 in phase 2i+1, team 1
  // tile i+2 in phase 2i, each into the buffer of a tile finished by then), and
  // when its next score phase starts a new query token it loads that token's Q
  // there first.  Prologue: team 0 issues tiles 0..2, team 1 tiles 0..1.
  {
    const int t0 = uni(lg.c.t);
    const int pro = team == 0 ? kNBuf - 1 : kNBuf - 2;
    for (int k = 0; k < pro && lg.valid; ++k) {
      issue();
      advance();
    }
    load_q(t0);
    // no scalar load may look outstanding at the loop entry (the compiler
    // would otherwise make every LDS wait in the loop a full one)
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  }
  // Tile descriptors are read before the barrier that opens a phase (the wave
  // waits there anyway), so no LDS read is outstanding when a phase starts.
  int d_prev = 0, t_prev = 0;  // descriptor and token of tile i-1
  for (int i = 0;; ++i) {
    const bool has = i < issued;
    const int d_i = has ? desc_of(i) : 0, t_i = has ? tok_of(i) : 0;
    // ---- phase 2i.  Loads complete in issue order: tile i has landed once at
    // most the loads of the tiles issued after it are outstanding.
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
    // ---- phase 2i+1
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

bool v3_kernels_available() { return true; }

hipError_t launch_decode_v3(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(decode_v4_kernel, dim3(a.plan.G), dim3(512), 0, st, a.plan.q_start,
                     a.plan.kv_lens, a.block_table, (const uint16_t*)a.pool,
                     (const uint16_t*)a.q_lat, (uint16_t*)a.o_lat, (uint16_t*)a.ws_o, a.ws_lse,
                     a.err, a.plan.B, a.plan.T, a.plan.causal, a.plan.G, a.plan.U, a.max_blocks,
                     a.num_blocks, a.scale_log2);
  return hipGetLastError();
}

}  // namespace mla

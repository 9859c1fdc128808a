// Host emulation of the HIP execution model, for compiling the library's kernel
// sources as ordinary C++ and running them on the CPU in tests.
//
// Every work-item runs as a fiber on one OS thread.  A fiber runs until it
// reaches a point where it must meet other work-items:
//   - a wavefront collective (MFMA, cross-lane shuffles, ballot,
//     readfirstlane, the transposing LDS read): all live lanes of the
//     64-lane wave must arrive at the same collective, which is then computed
//     for the whole wave at once;
//   - a workgroup barrier: all live work-items of the group must arrive.
// Between those points fibers run in a seeded random order, so a missing
// barrier shows up as results that change with the seed.  Workgroups of a grid
// run one after the other; `__shared__` variables become function statics
// (one workgroup is live at a time).  Loads and stores are plain host memory
// accesses, except the direct-to-LDS loads: those are queued per wave and land
// in issue order, mostly only when an s_waitcnt vmcnt requires them, so a wait
// count that is too weak leaves stale LDS data behind.  Timing itself is not
// modelled.
//
// Cross-lane layouts (gfx950, wave64):
//   v_mfma_f32_16x16x32_bf16: lane l = 16g + i holds A[i][8g..8g+7] and
//     B[8g..8g+7][i] (8 bf16 each) and D[4g..4g+3][i] (4 fp32);
//   ds_read_b64_tr_b16: in each 16-lane group, lane j supplies 4 consecutive
//     16-bit values src[j][0..3]; lane i receives src[4r + i/4][i%4], r = 0..3.
//   v_mfma_f32_16x16x32_fp8_fp8: as the bf16 form with 8 OCP e4m3 bytes per
//     lane (A[i][8g..8g+7], B[8g..8g+7][i]);
//   v_mfma_scale_f32_16x16x128_f8f6f4 (e4m3 operands, unit scales): lane
//     16g + i holds 32 bytes, A[i][32g..32g+31] and B[32g..32g+31][i] (the probe
//     on MI355X showed the A and B column orders agree), D as above;
//   ds_read_b64_tr_b8: in each 16-lane group, lane j supplies 8 consecutive
//     bytes src[j][0..7]; lane i receives src[2r + i/8][i%8], r = 0..7.
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <functional>
#include <tuple>
#include <type_traits>
#include <utility>

struct dim3 {
  uint32_t x, y, z;
  constexpr dim3(uint32_t x_ = 1, uint32_t y_ = 1, uint32_t z_ = 1) : x(x_), y(y_), z(z_) {}
};

namespace emu {

constexpr int kWave = 64;

struct LaneIO {
  alignas(16) unsigned char in[96];
  alignas(16) unsigned char out[64];
};
// A wave collective: io[l] is lane l's in/out block (null when lane l is not
// live); `live` has bit l set for every live lane.
typedef void (*WaveFn)(uint64_t live, LaneIO* const* io);

extern dim3* g_tid;
extern dim3 g_bid, g_bdim, g_gdim;

int lane_id();
void wave_op(WaveFn fn, const void* in, size_t nin, void* out, size_t nout);
void block_barrier();
void fail(const char* msg);
void run_grid(dim3 grid, dim3 block, const std::function<void()>& body);

void op_mfma_16x16x32_bf16(uint64_t live, LaneIO* const* io);
void op_tr16_b64(uint64_t live, LaneIO* const* io);
void op_mfma_16x16x32_fp8(uint64_t live, LaneIO* const* io);
void op_tr8_b64(uint64_t live, LaneIO* const* io);
void op_mfma_16x16x128_f8(uint64_t live, LaneIO* const* io);
unsigned char f32_to_e4m3_rne(float x);
void op_gather(uint64_t live, LaneIO* const* io);
void op_ballot(uint64_t live, LaneIO* const* io);
void op_first(uint64_t live, LaneIO* const* io);
void op_dma16(uint64_t live, LaneIO* const* io);
void op_waitcnt(uint64_t live, LaneIO* const* io);

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

inline f32x4_t mfma_16x16x32_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  unsigned char in[48];
  memcpy(in, &a, 16);
  memcpy(in + 16, &b, 16);
  memcpy(in + 32, &c, 16);
  f32x4_t d;
  wave_op(op_mfma_16x16x32_bf16, in, sizeof in, &d, sizeof d);
  return d;
}

typedef int i32x2_t __attribute__((ext_vector_type(2)));

inline f32x4_t mfma_16x16x32_fp8(long a, long b, f32x4_t c) {
  unsigned char in[32];
  memcpy(in, &a, 8);
  memcpy(in + 8, &b, 8);
  memcpy(in + 16, &c, 16);
  f32x4_t d;
  wave_op(op_mfma_16x16x32_fp8, in, sizeof in, &d, sizeof d);
  return d;
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

inline f32x4_t mfma_16x16x128_f8(i32x8_t a, i32x8_t b, f32x4_t c, int fmt_a, int fmt_b,
                                 int scale_a, int scale_b) {
  if (fmt_a != 0 || fmt_b != 0 || scale_a != 127 || scale_b != 127)
    fail("16x16x128 f8f6f4: only e4m3 operands with unit scales are emulated");
  unsigned char in[80];
  memcpy(in, &a, 32);
  memcpy(in + 32, &b, 32);
  memcpy(in + 64, &c, 16);
  f32x4_t d;
  wave_op(op_mfma_16x16x128_f8, in, sizeof in, &d, sizeof d);
  return d;
}

inline i32x2_t tr8_b64(const void* p) {
  i32x2_t r;
  wave_op(op_tr8_b64, &p, sizeof p, &r, sizeof r);
  return r;
}

// v_cvt_pk_fp8_f32: a, b -> two e4m3 (nearest even) in the low (hi = false) or
// high 16 bits of old
inline int cvt_pk_fp8(float a, float b, int old, bool hi) {
  const unsigned v = (unsigned)f32_to_e4m3_rne(a) | ((unsigned)f32_to_e4m3_rne(b) << 8);
  const unsigned o = (unsigned)old;
  return (int)(hi ? ((o & 0xffffu) | (v << 16)) : ((o & 0xffff0000u) | v));
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
double e4m3_to_double(unsigned char c);

// v_cvt_pk_f32_fp8: bytes 0, 1 (hi = false) or 2, 3 of v -> two fp32 (exact)
inline f32x2_t cvt_pk_f32_fp8(int v, bool hi) {
  const unsigned u = (unsigned)v >> (hi ? 16 : 0);
  f32x2_t r;
  r[0] = (float)e4m3_to_double((unsigned char)(u & 0xff));
  r[1] = (float)e4m3_to_double((unsigned char)((u >> 8) & 0xff));
  return r;
}

// v_cvt_scalef32_pk_bf16_fp8: bytes 0, 1 (hi = false) or 2, 3 of v -> two bf16,
// times scale (only a unit scale is emulated; the conversion is then exact)
inline unsigned cvt_scalef32_pk_bf16_fp8(unsigned v, float scale, bool hi) {
  if (scale != 1.0f) fail("cvt_scalef32_pk_bf16_fp8: only a unit scale is emulated");
  const unsigned u = v >> (hi ? 16 : 0);
  unsigned r = 0;
  for (int k = 0; k < 2; ++k) {
    const float f = (float)e4m3_to_double((unsigned char)((u >> (8 * k)) & 0xff));
    unsigned b;
    memcpy(&b, &f, 4);
    r |= (b >> 16) << (16 * k);
  }
  return r;
}

inline i16x4_t tr16_b64(const void* p) {
  i16x4_t r;
  wave_op(op_tr16_b64, &p, sizeof p, &r, sizeof r);
  return r;
}

template <typename T>
inline T gather(T v, int src) {
  static_assert(sizeof(T) <= 8, "shuffle of at most 8 bytes");
  unsigned char in[12] = {};
  memcpy(in, &v, sizeof(T));
  memcpy(in + 8, &src, 4);
  unsigned char out[8];
  wave_op(op_gather, in, sizeof in, out, sizeof out);
  T r;
  memcpy(&r, out, sizeof(T));
  return r;
}

inline int readfirstlane(int v) {
  int r;
  wave_op(op_first, &v, sizeof v, &r, sizeof r);
  return r;
}
inline int readfirstlane(unsigned v) { return readfirstlane((int)v); }

// {own value, value of lane l ^ 16} / {own value, value of lane l ^ 32}
inline u32x2_t permlane_swap(unsigned v, int mask) {
  u32x2_t r;
  r[0] = v;
  r[1] = gather(v, lane_id() ^ mask);
  return r;
}

// Direct-to-LDS load of 16 bytes per lane (lane l's bytes land at
// lds_base + 16*l): asynchronous, see op_dma16.
inline void dma16(const char* src, char* lds_base) {
  unsigned char in[16], out[1];
  memcpy(in, &src, 8);
  memcpy(in + 8, &lds_base, 8);
  wave_op(op_dma16, in, sizeof in, out, 0);
}

// s_waitcnt: waits until at most vmcnt of the wave's direct-to-LDS loads are
// in flight (the other counters have nothing to wait for here).
inline void s_waitcnt(int imm) {
  const int vm = (imm & 0xf) | (((imm >> 14) & 3) << 4);
  unsigned char out[1];
  wave_op(op_waitcnt, &vm, sizeof vm, out, 0);
}

template <typename... P, typename... A>
void launch(void (*k)(P...), dim3 grid, dim3 block, A&&... args) {
  // convert the arguments to the kernel's parameter types once, as a launch does
  std::tuple<std::decay_t<P>...> packed(std::forward<A>(args)...);
  run_grid(grid, block, [&]() { std::apply(k, packed); });
}

}  // namespace emu

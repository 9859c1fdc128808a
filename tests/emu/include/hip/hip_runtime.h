// Stand-in for <hip/hip_runtime.h> when the library's kernel sources are built
// as host C++ for the emulator (see emu_runtime.h).  Provides the subset of the
// HIP device API that those sources use.
#pragma once

#include "emu_runtime.h"

#define __global__
#define __device__
#define __host__
#define __shared__ static
#define __forceinline__ inline __attribute__((always_inline))
#define __launch_bounds__(...)
#define __align__(n) __attribute__((aligned(n)))

#define threadIdx (*::emu::g_tid)
#define blockIdx (::emu::g_bid)
#define blockDim (::emu::g_bdim)
#define gridDim (::emu::g_gdim)

typedef enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorNotSupported = 801,
} hipError_t;
typedef struct ihipStream_t* hipStream_t;
typedef enum hipDeviceAttribute_t {
  hipDeviceAttributeMultiprocessorCount = 1,
} hipDeviceAttribute_t;

hipError_t hipGetLastError();
// a file-scope __device__ array is an ordinary host array here: its address is
// the "device" address
#define HIP_SYMBOL(x) ((const void*)&(x))
inline hipError_t hipGetSymbolAddress(void** p, const void* sym) {
  *p = const_cast<void*>(sym);
  return hipSuccess;
}
hipError_t hipGetDevice(int* dev);
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int dev);

#define hipLaunchKernelGGL(kernel, grid, block, shmem, stream, ...) \
  ::emu::launch(kernel, dim3(grid), dim3(block), ##__VA_ARGS__)

// a full barrier also waits for every outstanding load of the wave
inline void __syncthreads() {
  ::emu::s_waitcnt(0);
  ::emu::block_barrier();
}

template <typename A, typename B>
inline typename std::common_type<A, B>::type min(A a, B b) {
  typedef typename std::common_type<A, B>::type C;
  return (C)a < (C)b ? (C)a : (C)b;
}
template <typename A, typename B>
inline typename std::common_type<A, B>::type max(A a, B b) {
  typedef typename std::common_type<A, B>::type C;
  return (C)a > (C)b ? (C)a : (C)b;
}

inline unsigned __float_as_uint(float x) {
  unsigned u;
  memcpy(&u, &x, 4);
  return u;
}
inline float __uint_as_float(unsigned u) {
  float x;
  memcpy(&x, &u, 4);
  return x;
}
inline int __float_as_int(float x) { return (int)__float_as_uint(x); }
inline float __int_as_float(int i) { return __uint_as_float((unsigned)i); }
inline int __ffsll(long long x) { return __builtin_ffsll(x); }
inline int __popcll(unsigned long long x) { return __builtin_popcountll(x); }

inline unsigned atomicOr(unsigned* p, unsigned v) {
  unsigned o = *p;
  *p = o | v;
  return o;
}
inline unsigned atomicAdd(unsigned* p, unsigned v) {
  unsigned o = *p;
  *p = o + v;
  return o;
}
inline int atomicAdd(int* p, int v) {
  int o = *p;
  *p = o + v;
  return o;
}
inline float atomicAdd(float* p, float v) {
  float o = *p;
  *p = o + v;
  return o;
}

template <typename T>
inline T __shfl(T v, int src, int width = 64) {
  const int l = ::emu::lane_id();
  return ::emu::gather(v, (l & ~(width - 1)) + (src & (width - 1)));
}
template <typename T>
inline T __shfl_xor(T v, int mask, int width = 64) {
  const int l = ::emu::lane_id();
  int s = l ^ mask;
  if ((s & ~(width - 1)) != (l & ~(width - 1))) s = l;
  return ::emu::gather(v, s);
}
template <typename T>
inline T __shfl_up(T v, unsigned d, int width = 64) {
  const int l = ::emu::lane_id();
  return ::emu::gather(v, (l & (width - 1)) >= (int)d ? l - (int)d : l);
}
template <typename T>
inline T __shfl_down(T v, unsigned d, int width = 64) {
  const int l = ::emu::lane_id();
  return ::emu::gather(v, (l & (width - 1)) + (int)d < width ? l + (int)d : l);
}
inline unsigned long long __ballot(int pred) {
  unsigned long long m;
  ::emu::wave_op(::emu::op_ballot, &pred, sizeof pred, &m, sizeof m);
  return m;
}

#define __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, cbsz, abid, blgp) \
  ::emu::mfma_16x16x32_bf16((a), (b), (c))
#define __builtin_amdgcn_ds_read_tr16_b64_v4i16(p) ::emu::tr16_b64((const void*)(p))
#define __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, cbsz, abid, blgp) \
  ::emu::mfma_16x16x32_fp8((a), (b), (c))
#define __builtin_amdgcn_ds_read_tr8_b64_v2i32(p) ::emu::tr8_b64((const void*)(p))
#define __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, fa, fb, oa, sa, ob, sb) \
  ::emu::mfma_16x16x128_f8((a), (b), (c), (fa), (fb), (sa), (sb))
#define __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, hi) ::emu::cvt_pk_fp8((a), (b), (old), (hi))
#define __builtin_amdgcn_cvt_pk_f32_fp8(v, hi) ::emu::cvt_pk_f32_fp8((v), (hi))
#define __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, s, hi) \
  __builtin_bit_cast(__bf16 __attribute__((ext_vector_type(2))),                 \
                     ::emu::cvt_scalef32_pk_bf16_fp8((v), (s), (hi)))
#define __builtin_amdgcn_readfirstlane(x) ::emu::readfirstlane(x)
#define __builtin_amdgcn_permlane16_swap(a, b, fi, bc) ::emu::permlane_swap((a), 16)
#define __builtin_amdgcn_permlane32_swap(a, b, fi, bc) ::emu::permlane_swap((a), 32)
#define __builtin_amdgcn_s_waitcnt(x) ::emu::s_waitcnt(x)
#define __builtin_amdgcn_sched_barrier(x) ((void)0)
#define __builtin_amdgcn_sched_group_barrier(m, n, id) ((void)0)
#define __builtin_amdgcn_s_setprio(x) ((void)0)
// hardware transcendentals: the emulator uses the libm functions (the GPU's are
// within about 1 ulp of them)
#define __builtin_amdgcn_exp2f(x) exp2f(x)
#define __builtin_amdgcn_logf(x) log2f(x)
#define __builtin_amdgcn_rcpf(x) (1.0f / (x))
#define __builtin_amdgcn_s_setprio(x) ((void)0)
// shader clock: a counter that only moves forward
inline unsigned long long emu_clock_() {
  static unsigned long long t = 0;
  return t += 4;
}
#define __builtin_amdgcn_s_memtime() emu_clock_()

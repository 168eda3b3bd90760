// Small gfx950 building blocks shared by the window-scan kernels: buffer
// descriptors, the hardware exponential, the transposed LDS read, buffer
// loads straight into LDS, and the binary32 dt softplus of the window scans.
#pragma once
#include "common.h"

namespace m2 {

typedef short s4 __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kSc1 = 16;   // buffer cache policy: device-coherent access

// Buffer descriptor over [p, p + bytes).  p and bytes must be wave-uniform;
// they are read from the first lane so that the descriptor is built in SGPRs
// (a descriptor the compiler cannot prove uniform turns every access through
// it into a loop over lanes).  Loads past the range return zero; stores past
// it are dropped.
__device__ __forceinline__ rsrc_t mkr(const void* p, unsigned bytes) {
  const unsigned long long v = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  void* const pu = (void*)(((unsigned long long)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(pu, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// 2^x with the hardware exponential (arguments here are <= 0; results below
// the binary32 normal range are negligible against the terms they scale)
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ h8 cat(h4 lo, h4 hi) { return h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}; }

// Transposed 64-bit LDS read: within each 16-lane group, lane i receives the
// 16-bit elements at column (i % 4) of the 8-byte chunks addressed by lanes
// 4k + i / 4, k = 0..3.
__device__ __forceinline__ h4 tr4(const _Float16* p) {
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4*)(__attribute__((address_space(3))) void*)(p));
  return __builtin_bit_cast(h4, v);
}

// The dt softplus of a raw dt in binary32 with the hardware exponential and
// logarithm: v above 20, e (1 - e/2) for e = exp(v) below 1e-3 (the series of
// log1p, error below e^3/3), else log(1 + e) (relative error below about
// 6e-5, from rounding 1 + e).  The window scans only need dt within their
// tolerance; the double-precision form of the decode contract would keep its
// constants in registers across the whole scan.
__device__ __forceinline__ float dt_softplus_fast(float raw, float bias) {
  const float v = raw + bias;
  const float e = __expf(v);
  const float sp = e < 1e-3f ? e * (1.f - 0.5f * e) : __logf(1.f + e);
  return v > 20.f ? v : sp;
}

}  // namespace m2

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

// ---- streaming operands into LDS (the window scans) ----------------------------

// Buffer descriptor words in scalar registers (wave-uniform p and bytes) for
// the loads below; loads past `bytes` return zero.
__device__ __forceinline__ u4 rsrc_words(const void* p, unsigned bytes) {
  const unsigned long long v = (unsigned long long)p;
  return u4{(unsigned)__builtin_amdgcn_readfirstlane((unsigned)v),
            (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(v >> 32)),
            (unsigned)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

// LDS byte address of a workgroup-shared location
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)__builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(const __attribute__((address_space(3))) void*)p);
}

// 16 bytes per lane from the buffer at byte offset voff straight into LDS:
// lane l's bytes land at lds + 16 l.  Written as an asm statement so that the
// compiler does not track these loads: it would otherwise make some LDS reads
// wait for every LDS-writing load in flight, draining the prefetch.  The
// waits for them are explicit (vm_wait, before the barrier that publishes a
// slot); the load has no register result, so nothing is written to a
// register while it is in flight.
__device__ __forceinline__ void dma16(u4 r, unsigned lds, unsigned voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}

// 4 bytes per lane into LDS (lane l's bytes land at lds + 4 l); as dma16.
__device__ __forceinline__ void dma4(u4 r, unsigned lds, unsigned voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}

// Wait until at most n of this wave's vector memory operations are
// outstanding (they complete in issue order); n outside 0..15 waits for all.
__device__ __forceinline__ void vm_wait(int n) {
#define M2_VMW(k) \
  case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
  switch (n) {
    M2_VMW(1) M2_VMW(2) M2_VMW(3) M2_VMW(4) M2_VMW(5) M2_VMW(6) M2_VMW(7) M2_VMW(8) M2_VMW(9) M2_VMW(10)
    M2_VMW(11) M2_VMW(12) M2_VMW(13) M2_VMW(14) M2_VMW(15)
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
#undef M2_VMW
}

// Workgroup barrier for the slots.  No fence: a workgroup release fence would
// make the compiler wait for every LDS-writing buffer load in flight.  The
// empty asm statements keep the compiler from moving LDS accesses across it;
// the caller has already waited for what must be visible.
__device__ __forceinline__ void slot_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS reads and writes are done
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace m2

// Resident decode state (B, H, P, N) in binary16 or binary32: 8 consecutive
// elements per access, widened to or narrowed from binary32.
#pragma once
#include "common.h"

namespace m2 {

// The resident state is streamed once per step and not reused before the
// next step touches the rest of the batch: its loads and stores are marked
// non-temporal so that they do not evict the other operands from the caches.
template <int N> struct StateF16 {
  using T = _Float16;
  // the 8 elements as loaded, widened only where they are used (a load kept
  // raw does not make the code after it wait)
  using Raw = h8;
  static __device__ __forceinline__ Raw load_raw(const T* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const h8*>(p));
  }
  static __device__ __forceinline__ void widen(const Raw& h, float* v) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
  }
  static __device__ __forceinline__ void load(const T* p, float* v) {
    const h8 h = __builtin_nontemporal_load(reinterpret_cast<const h8*>(p));
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
  }
  static __device__ __forceinline__ void store(T* p, const float* v) {
    h8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // The value is rounded to binary32 first and then to binary16 (RNE,
      // subnormals kept).  The empty asm pins the binary32 value in a register:
      // without it the compiler fuses the producing fma with this conversion
      // into one mixed-precision fma that rounds only once, which differs at
      // binary32 values lying exactly on a binary16 tie.
      float t = v[i];
      asm volatile("" : "+v"(t));
      h[i] = (_Float16)t;
    }
    __builtin_nontemporal_store(h, reinterpret_cast<h8*>(p));
  }
};
template <int N> struct StateF32 {
  using T = float;
  struct Raw {
    f4 lo, hi;
  };
  static __device__ __forceinline__ Raw load_raw(const T* p) {
    return Raw{*reinterpret_cast<const f4*>(p), *reinterpret_cast<const f4*>(p + 4)};
  }
  static __device__ __forceinline__ void widen(const Raw& r, float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = r.lo[i];
      v[4 + i] = r.hi[i];
    }
  }
  static __device__ __forceinline__ void load(const T* p, float* v) { io<float>::load8(p, v); }
  static __device__ __forceinline__ void store(T* p, const float* v) {
    *reinterpret_cast<f4*>(p) = f4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f4*>(p + 4) = f4{v[4], v[5], v[6], v[7]};
  }
};

}  // namespace m2

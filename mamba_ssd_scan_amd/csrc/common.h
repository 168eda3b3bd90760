// Shared device-side definitions for the gfx950 Mamba-2 mixer-core kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2 {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// 16x16x32 f16 MFMA with fp32 accumulate.  Lane l holds A[l%16][k-slots of
// group l/16], B[k-slots of group l/16][l%16]; D reg i is D[4*(l/16)+i][l%16].
// The k-slot -> k mapping only has to agree between A and B.
__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Widen 8 consecutive I/O elements to float.
template <typename T> struct io;
template <> struct io<_Float16> {
  static __device__ __forceinline__ void load8(const _Float16* p, float* v) {
    h8 h = *reinterpret_cast<const h8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
  }
  static __device__ __forceinline__ h8 load8h(const _Float16* p) { return *reinterpret_cast<const h8*>(p); }
  static __device__ __forceinline__ float load1(const _Float16* p) { return (float)*p; }
  static __device__ __forceinline__ void store1(_Float16* p, float v) { *p = (_Float16)v; }
  static __device__ __forceinline__ void store4(_Float16* p, f4 v) {
    h4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<h4*>(p) = h;
  }
};
template <> struct io<float> {
  static __device__ __forceinline__ void load8(const float* p, float* v) {
    f4 a = *reinterpret_cast<const f4*>(p), b = *reinterpret_cast<const f4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  static __device__ __forceinline__ h8 load8h(const float* p) {
    f4 a = *reinterpret_cast<const f4*>(p), b = *reinterpret_cast<const f4*>(p + 4);
    h8 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) { h[i] = (_Float16)a[i]; h[4 + i] = (_Float16)b[i]; }
    return h;
  }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
  static __device__ __forceinline__ void store1(float* p, float v) { *p = v; }
  static __device__ __forceinline__ void store4(float* p, f4 v) { *reinterpret_cast<f4*>(p) = v; }
};

// dt from its raw pre-activation (dims.dt_softplus): sp(raw + bias) in
// double precision, rounded once to binary32; sp(v) = v above 20, else
// log1p(exp(v)).
__device__ __forceinline__ float dt_softplus(float raw, float bias) {
  const double v = (double)raw + (double)bias;
  return (float)(v > 20.0 ? v : log1p(exp(v)));
}

// First row and length of sequence b in the caller's per-token tensors.
// Packed (cu != nullptr): rows cu[b] .. cu[b+1]-1 of T rows.  Otherwise rows
// b*L .., length seqlens[b] (or L).  Lengths are clamped to [0, L] and packed
// rows to [0, T), so no access leaves the tensors whatever the offsets hold.
struct SeqRows {
  long long base;
  int len;
};
__device__ __forceinline__ SeqRows seq_rows(const int* seqlens, const int* cu, int b, int L, int T) {
  if (cu) {
    const int s = min(max(cu[b], 0), T);
    const int e = min(max(cu[b + 1], s), T);
    return SeqRows{(long long)s, min(e - s, L)};
  }
  const int len = seqlens ? seqlens[b] : L;
  return SeqRows{(long long)b * L, len < 0 ? 0 : (len > L ? L : len)};
}

}  // namespace m2


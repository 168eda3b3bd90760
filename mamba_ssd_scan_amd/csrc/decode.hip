// One-token recurrent step and resident-state load/store.
//
// The step is the Mamba-2 selective state-space update for one token (method
// listed under "References" on page "Mamb2_8B_FP4_Recall_SQ3.25"):
//   S <- exp(dt*A_h) S + dt x (outer) B,   y = S.C + D_h x.
// With a binary16 resident state the state is stored back to binary16 after
// the token, as the page's decode requantizes the recurrent row every token
// (section "Representation", paragraph "State").
//
// Work split: one 256-thread workgroup per (sequence, head) P x N tile.  Each
// thread owns 8 consecutive n of some rows p, so every state load/store is a
// 16-byte (f16) or 32-byte (f32) vector and each wave instruction touches a
// contiguous span of the row-major (P, N) tile.  y[p] is an N-reduction over
// the N/8 lanes of a row (cross-lane shuffles inside one wave).
// The kernel is HBM-bound: per (b,h) it moves 2*P*N state elements and
// ~(2P + 2N) I/O elements, with ~6 flops per state element.
#include "state_io.h"

namespace m2 {

// N in {16, 64, 128}; P % (256 / (N/8)) == 0 handled by the row loop.
template <typename IO, typename ST, int N>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const IO* __restrict__ x, const IO* __restrict__ dt, const IO* __restrict__ Bm,
    const IO* __restrict__ Cm, const float* __restrict__ A, const float* __restrict__ D,
    typename ST::T* __restrict__ state, IO* __restrict__ y, int H, int P, int G, int dt_sp,
    const float* __restrict__ dt_bias) {
  constexpr int LPR = N / 8;          // lanes per state row
  constexpr int RPP = 256 / LPR;      // rows per pass
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh - b * H;
  const int g = h / (H / G);
  const int tid = threadIdx.x;
  const int nc = (tid % LPR) * 8;     // first n of this thread
  const int r0 = tid / LPR;

  float d = io<IO>::load1(dt + bh);
  if (dt_sp) d = dt_softplus(d, dt_bias ? dt_bias[h] : 0.f);
  const float Ah = A[h];
  // Decay rounded once from a double-precision exponential (binary32 contract).
  const float a = (float)exp((double)d * (double)Ah);
  float bv[8], cv[8];
  io<IO>::load8(Bm + ((size_t)b * G + g) * N + nc, bv);
  io<IO>::load8(Cm + ((size_t)b * G + g) * N + nc, cv);
  const float Dh = D[h];
  typename ST::T* S = state + (size_t)bh * P * N;
  const IO* xb = x + (size_t)bh * P;
  IO* yb = y + (size_t)bh * P;

  for (int p0 = 0; p0 < P; p0 += RPP * 4) {
    float s[4][8];
    float xp[4];
    bool ok[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = p0 + r0 + k * RPP;
      ok[k] = p < P;
      if (ok[k]) {
        ST::load(S + (size_t)p * N + nc, s[k]);
        xp[k] = io<IO>::load1(xb + p);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!ok[k]) continue;
      const int p = p0 + r0 + k * RPP;
      float acc = 0.f;
      {
#pragma clang fp contract(off)
        const float u = d * xp[k];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float v = u * bv[i];
          const float sn = __builtin_fmaf(a, s[k][i], v);
          s[k][i] = sn;
          acc = __builtin_fmaf(sn, cv[i], acc);
        }
      }
      ST::store(S + (size_t)p * N + nc, s[k]);
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
      if ((tid % LPR) == 0) io<IO>::store1(yb + p, acc + Dh * xp[k]);
    }
  }
}

// f32 <-> resident state conversion (elementwise, 8 elements per thread).
template <typename ST>
__global__ __launch_bounds__(256) void state_load_kernel(const float* __restrict__ src,
                                                          typename ST::T* __restrict__ dst, size_t n8) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float v[8];
  io<float>::load8(src + i * 8, v);
  ST::store(dst + i * 8, v);
}
template <typename ST>
__global__ __launch_bounds__(256) void state_store_kernel(const typename ST::T* __restrict__ src,
                                                           float* __restrict__ dst, size_t n8) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float v[8];
  ST::load(src + i * 8, v);
  StateF32<8>::store(dst + i * 8, v);
}

// ---------------------------------------------------------------------------
// Host launchers (called by the ABI after validation).
template <typename IO, typename ST>
static hipError_t launch_decode_T(int N, const void* x, const void* dt, const void* Bm, const void* Cm,
                                  const float* A, const float* D, void* state, void* y, int Bsz, int H,
                                  int P, int G, int dt_sp, const float* dt_bias, hipStream_t st) {
  dim3 grid(Bsz * H), block(256);
  using S = typename ST::T;
  switch (N) {
    case 16:
      decode_step_kernel<IO, ST, 16><<<grid, block, 0, st>>>((const IO*)x, (const IO*)dt, (const IO*)Bm,
                                                             (const IO*)Cm, A, D, (S*)state, (IO*)y, H, P, G, dt_sp, dt_bias);
      break;
    case 64:
      decode_step_kernel<IO, ST, 64><<<grid, block, 0, st>>>((const IO*)x, (const IO*)dt, (const IO*)Bm,
                                                             (const IO*)Cm, A, D, (S*)state, (IO*)y, H, P, G, dt_sp, dt_bias);
      break;
    default:
      decode_step_kernel<IO, ST, 128><<<grid, block, 0, st>>>((const IO*)x, (const IO*)dt, (const IO*)Bm,
                                                              (const IO*)Cm, A, D, (S*)state, (IO*)y, H, P, G, dt_sp, dt_bias);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_decode(int io_f16, int state_f16, int N, const void* x, const void* dt, const void* Bm,
                         const void* Cm, const float* A, const float* D, void* state, void* y, int Bsz,
                         int H, int P, int G, int dt_sp, const float* dt_bias, hipStream_t st) {
  if (io_f16 && state_f16)
    return launch_decode_T<_Float16, StateF16<8>>(N, x, dt, Bm, Cm, A, D, state, y, Bsz, H, P, G, dt_sp, dt_bias,
                                                  st);
  if (io_f16)
    return launch_decode_T<_Float16, StateF32<8>>(N, x, dt, Bm, Cm, A, D, state, y, Bsz, H, P, G, dt_sp, dt_bias,
                                                  st);
  if (state_f16)
    return launch_decode_T<float, StateF16<8>>(N, x, dt, Bm, Cm, A, D, state, y, Bsz, H, P, G, dt_sp, dt_bias, st);
  return launch_decode_T<float, StateF32<8>>(N, x, dt, Bm, Cm, A, D, state, y, Bsz, H, P, G, dt_sp, dt_bias, st);
}

hipError_t launch_state_convert(int to_resident, int state_f16, const void* src, void* dst, size_t n,
                                hipStream_t st) {
  const size_t n8 = n / 8;
  dim3 grid((unsigned)((n8 + 255) / 256)), block(256);
  if (n8 == 0) return hipSuccess;
  if (to_resident) {
    if (state_f16)
      state_load_kernel<StateF16<8>><<<grid, block, 0, st>>>((const float*)src, (_Float16*)dst, n8);
    else
      state_load_kernel<StateF32<8>><<<grid, block, 0, st>>>((const float*)src, (float*)dst, n8);
  } else {
    if (state_f16)
      state_store_kernel<StateF16<8>><<<grid, block, 0, st>>>((const _Float16*)src, (float*)dst, n8);
    else
      state_store_kernel<StateF32<8>><<<grid, block, 0, st>>>((const float*)src, (float*)dst, n8);
  }
  return hipGetLastError();
}

}  // namespace m2

// Whole-window Mamba-2 scan in its chunked state-space-dual form, with an
// optional fused causal conv1d(4)+SiLU prologue and a gated-RMSNorm epilogue.
//
// The method is Mamba-2 / structured state-space duality (Dao and Gu 2024,
// listed under "References" on page "Mamb2_8B_FP4_Recall_SQ3.25").  For one
// head, with log-decays la_t = dt_t * A_h and their running sum S_t inside a
// chunk, the recurrence S <- e^{la_t} S + dt_t x_t B_t^T, y_t = S C_t + D x_t
// is evaluated per chunk of Q tokens as
//   y_t   = sum_{s<=t in chunk} (C_t.B_s) e^{S_t-S_s} dt_s x_s        (diagonal)
//         + e^{S_t} C_t . H_in                                          (carry-in)
//         + D x_t
//   H_out = e^{S_end} H_in + sum_s e^{S_end-S_s} dt_s x_s B_s^T          (hand-off)
// Only differences S_t - S_s with s <= t are exponentiated, so every factor is
// <= 1 and nothing overflows however long the chunk decays.
//
// Design for gfx950:
//  * one 256-thread workgroup (4 waves) per (chunk, sequence, head) item, taken
//    in chunk-major order from an atomic ticket, so that an item only ever
//    waits for an item that started before it (no deadlock whatever the
//    dispatch order);
//  * inside a chunk the quadratic (attention-like) part is restricted to
//    64-token sub-chunks, and sub-chunks are linked by running fp32 states kept
//    in registers, which cuts the MFMA work of a 256-token chunk by ~40%;
//  * all contractions (C.B^T, the decay-masked product with dt*x, chunk states
//    x^T B, and the C.H readout) are 16x16x32 f16 MFMAs with fp32 accumulate,
//    operands staged through LDS (x and B transposed on the way in so that the
//    token index is the contiguous k index);
//  * the only cross-workgroup traffic is the fp32 P x N hand-off state of each
//    (chunk, head), published through a flag tagged with a per-call generation
//    number (so the workspace never needs clearing between calls).  The state
//    and the flag move with device-coherent (sc1) accesses -- relaxed
//    agent-scope atomics -- ordered by waiting for the stores to complete.
//    An agent-scope release/acquire fence would instead write back or
//    invalidate the whole L2 of the XCD, once per workgroup.
#include "common.h"
#include "../../include/mamba2ssd.h"

namespace m2 {

constexpr int kP = 64;          // head dim
constexpr int kTS = 64;         // tokens per sub-chunk
constexpr int kXP = kTS + 8;    // pitch (halfs) of [p][s] tiles
constexpr int kXN = kP + 8;     // pitch (halfs) of [s][p] tiles
constexpr unsigned kSpinLimit = 1u << 22;

template <int N> struct Lay {
  static constexpr int NT = N / 16;          // n-tiles of the state
  static constexpr int KN = (N + 31) / 32;   // k-steps over n
  static constexpr int NP = N + 8;           // pitch of [s][n] and [p][n] tiles (halfs)
  static constexpr int BTP = kTS + 8;        // pitch of the [n][s] tile
  // state tiles (n-tile x p-tile) owned by each wave in the chunk-state phase
  static constexpr int NTW = N == 128 ? 2 : 1;
  static constexpr int PTW = N == 16 ? 1 : 4;
  static constexpr int TILES = NTW * PTW;
};

template <int N, bool CONV> struct alignas(16) Smem {
  alignas(16) _Float16 xt[kP * kXP];                 // [p][s]: x (post-conv when fused), transposed
  alignas(16) _Float16 bt[N * Lay<N>::BTP];          // [n][s]: dt- and decay-weighted B, transposed
  alignas(16) _Float16 bn[kTS * Lay<N>::NP];         // [s][n]: B as read
  alignas(16) _Float16 cn[kTS * Lay<N>::NP];         // [t][n]: C as read
  alignas(16) _Float16 r[kP * Lay<N>::NP];           // [p][n]: state entering the sub-chunk
  float S[256];                                      // running log2-decay from the chunk start (inclusive)
  _Float16 dts[256];                                 // dt per token (0 past the sequence end)
  float wsum[4];
  unsigned ticket, gen;
};

template <typename IO> struct WinArgs {
  int B, L, H, G, Q, nchunks, norm;
  int Cd;  // conv channels
  const IO* x;
  const IO* Bm;
  const IO* Cm;
  const IO* xBC;
  const float* conv_w;
  const float* conv_b;
  const IO* conv_in;
  IO* conv_out;
  const IO* dt;
  const float* A;
  const float* D;
  const float* state_in;
  float* state_out;
  const int* seqlens;
  const IO* z;
  float* normsum;   // (B, L, H) per-head sum of g^2 (norm epilogue)
  IO* y;
  unsigned* ctrl;   // [0] ticket [1] done [2] generation [3] error
  unsigned* flags;  // per item
  float* states;    // per item hand-off state (private layout)
};

// ---- input access: plain tensors, or conv1d(4)+SiLU over raw xBC ----------
template <typename IO, bool CONV> struct Src {
  // 8 consecutive raw channels at token tau (< 0: history or zeros)
  static __device__ __forceinline__ void raw8(const WinArgs<IO>& a, int b, int tau, int ch0, float* r) {
    if (tau >= 0) {
      io<IO>::load8(a.xBC + ((size_t)b * a.L + tau) * a.Cd + ch0, r);
    } else if (a.conv_in) {
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = io<IO>::load1(a.conv_in + ((size_t)b * a.Cd + ch0 + e) * 3 + 3 + tau);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = 0.f;
    }
  }
  static __device__ __forceinline__ h8 conv8(const WinArgs<IO>& a, int b, int t, int ch0) {
    float v[8];
    conv8f(a, b, t, ch0, v);
    h8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (_Float16)v[e];
    return r;
  }
  static __device__ __forceinline__ void conv8f(const WinArgs<IO>& a, int b, int t, int ch0, float* v) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = a.conv_b ? a.conv_b[ch0 + e] : 0.f;
    float w[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f4 ww = *reinterpret_cast<const f4*>(a.conv_w + (size_t)(ch0 + e) * 4);
      w[e][0] = ww[0]; w[e][1] = ww[1]; w[e][2] = ww[2]; w[e][3] = ww[3];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float r[8];
      raw8(a, b, t - 3 + k, ch0, r);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(w[e][k], r[e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = acc[e] / (1.f + __expf(-acc[e]));
  }
  static __device__ __forceinline__ h8 x8(const WinArgs<IO>& a, int b, int t, int h, int p0) {
    if (CONV) return conv8(a, b, t, h * kP + p0);
    return io<IO>::load8h(a.x + (((size_t)b * a.L + t) * a.H + h) * kP + p0);
  }
  template <int N>
  static __device__ __forceinline__ h8 b8(const WinArgs<IO>& a, int b, int t, int g, int n0) {
    if (CONV) return conv8(a, b, t, a.H * kP + g * N + n0);
    return io<IO>::load8h(a.Bm + (((size_t)b * a.L + t) * a.G + g) * N + n0);
  }
  template <int N>
  static __device__ __forceinline__ h8 c8(const WinArgs<IO>& a, int b, int t, int g, int n0) {
    if (CONV) return conv8(a, b, t, a.H * kP + a.G * N + g * N + n0);
    return io<IO>::load8h(a.Cm + (((size_t)b * a.L + t) * a.G + g) * N + n0);
  }
};

// Workgroup barrier that orders LDS only.  __syncthreads() would also wait for
// every outstanding global load, which would drain the loads prefetched for
// the next sub-chunk at each barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ h8 cat(h4 lo, h4 hi) { return h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}; }

// One thread's share of a 64-token sub-chunk, fetched ahead of its use.
//   x: tokens sx, sx+1 at channels 8*px..8*px+7 of the head
//   B, C: tokens sb..sb+TPT-1 at state columns 8*nb..8*nb+7 of the group
//   bs (fused conv only): B weighted for the state contraction, formed from the
//   fp32 conv output so that the weighted B is rounded to binary16 once
template <int N, bool CONV> struct Pref {
  static constexpr int NCH = N / 8;
  static constexpr int TPT = (kTS * NCH) / 256 > 0 ? (kTS * NCH) / 256 : 1;
  h8 x[2];
  h8 b[TPT];
  h8 c[TPT];
  h8 bs[CONV ? TPT : 1];
};

template <typename IO, int N, bool CONV, bool NORM>
__global__ __launch_bounds__(256, 2) void ssd_window_kernel(WinArgs<IO> a) {
  using Ly = Lay<N>;
  using SRC = Src<IO, CONV>;
  using PF = Pref<N, CONV>;
  __shared__ Smem<N, CONV> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, q = lane >> 4;

  // ---- take a ticket: item = (chunk, sequence, head), chunk-major ----------
  if (tid == 0) {
    sm.gen = __hip_atomic_load(&a.ctrl[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.ticket = __hip_atomic_fetch_add(&a.ctrl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const unsigned item = sm.ticket, gen = sm.gen;
  const int BH = a.B * a.H;
  const int c = item / BH, bh = item - c * BH;
  const int b = bh / a.H, h = bh - b * a.H;
  const int g = h / (a.H / a.G);
  int len = a.seqlens ? a.seqlens[b] : a.L;
  len = len < 0 ? 0 : (len > a.L ? a.L : len);
  const int t0 = c * a.Q;                      // first token of the chunk
  const int nvalid = min(max(len - t0, 0), a.Q);
  const int Jv = (nvalid + kTS - 1) / kTS;     // sub-chunks holding real tokens
  const float Ah = a.A[h] * kLog2e;
  const float Dh = a.D[h];

  // per-thread staging coordinates
  const int px = tid & 7, sx = 2 * (tid >> 3);
  const int nb = tid % PF::NCH, sb = (tid / PF::NCH) * PF::TPT;
  const bool bact = sb < kTS;

  // issue the global loads of sub-chunk j (tokens past the end are fetched
  // from a valid token and zeroed when written to LDS)
  // Sref: reference of the state weights (fused conv only, which forms the
  // weighted B here; it needs the phase-0 decays)
  auto fetch = [&](PF& f, int j, bool withC, float Sref) {
    const int i0 = j * kTS;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int s = i0 + sx + k;
      f.x[k] = SRC::x8(a, b, t0 + (s < nvalid ? s : i0), h, px * 8);
    }
    if (bact) {
#pragma unroll
      for (int k = 0; k < PF::TPT; ++k) {
        const int s = i0 + sb + k;
        const int t = t0 + (s < nvalid ? s : i0);
        if constexpr (CONV) {
          float v[8];
          SRC::conv8f(a, b, t, a.H * kP + g * N + nb * 8, v);
          const float wgt = s < nvalid ? (float)sm.dts[s] * exp2f(Sref - sm.S[s]) : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            f.b[k][e] = (_Float16)v[e];
            f.bs[k][e] = (_Float16)(v[e] * wgt);
          }
        } else {
          f.b[k] = SRC::template b8<N>(a, b, t, g, nb * 8);
        }
        if (withC) f.c[k] = SRC::template c8<N>(a, b, t, g, nb * 8);
      }
    }
  };

  // ---- phase 0: dt and the inclusive running log2-decay over the chunk -----
  PF pf;
  if (!CONV && Jv > 0) fetch(pf, 0, false, 0.f);
  {
    float d = 0.f;
    if (tid < nvalid) d = io<IO>::load1(a.dt + ((size_t)b * a.L + t0 + tid) * a.H + h);
    float v = d * Ah;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      float u = __shfl_up(v, off, 64);
      if (lane >= off) v += u;
    }
    if (lane == 63) sm.wsum[w] = v;
    __syncthreads();
    float pre = 0.f;
    for (int k = 0; k < w; ++k) pre += sm.wsum[k];
    if (tid < a.Q) {
      sm.S[tid] = v + pre;
      sm.dts[tid] = (_Float16)d;
    }
    __syncthreads();
  }
  const float Send = sm.S[a.Q - 1];
  if (CONV && Jv > 0) fetch(pf, 0, false, Send);

  // state tiles of this wave: n-tile nt0+i, p-tile pt0+jj
  const int nt0 = (N == 16) ? 0 : w * Ly::NTW;
  const int pt0 = (N == 16) ? w : 0;

  // write x (transposed, as read: no rounding for f16 inputs) and the
  // transposed B weighted by dt_s e^{Sref - S_s} of sub-chunk j
  auto stage_state_operands = [&](const PF& f, int j, float Sref) {
    const int i0 = j * kTS;
    {
      const bool ok0 = i0 + sx < nvalid, ok1 = i0 + sx + 1 < nvalid;
      const _Float16 zero = (_Float16)0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<h2*>(&sm.xt[(px * 8 + e) * kXP + sx]) = h2{ok0 ? f.x[0][e] : zero, ok1 ? f.x[1][e] : zero};
    }
    if (CONV && bact) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        _Float16* dst = &sm.bt[(nb * 8 + e) * Ly::BTP + sb];
#pragma unroll
        for (int k = 0; k < PF::TPT; ++k) dst[k] = f.bs[k][e];
      }
    } else if (bact) {
      float wk[PF::TPT];
#pragma unroll
      for (int k = 0; k < PF::TPT; ++k) {
        const int s = i0 + sb + k;
        wk[k] = s < nvalid ? (float)sm.dts[s] * exp2f(Sref - sm.S[s]) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        _Float16* dst = &sm.bt[(nb * 8 + e) * Ly::BTP + sb];
        if constexpr (PF::TPT == 4) {
          *reinterpret_cast<h4*>(dst) = h4{(_Float16)((float)f.b[0][e] * wk[0]), (_Float16)((float)f.b[1][e] * wk[1]),
                                           (_Float16)((float)f.b[2][e] * wk[2]), (_Float16)((float)f.b[3][e] * wk[3])};
        } else if constexpr (PF::TPT == 2) {
          *reinterpret_cast<h2*>(dst) = h2{(_Float16)((float)f.b[0][e] * wk[0]), (_Float16)((float)f.b[1][e] * wk[1])};
        } else {
          dst[0] = (_Float16)((float)f.b[0][e] * wk[0]);
        }
      }
    }
  };
  // acc[i][jj] += (weighted B)^T . x  for this wave's state tiles
  auto state_mfma = [&](f4 (&acc)[Ly::NTW][Ly::PTW]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      h8 bf[Ly::PTW];
#pragma unroll
      for (int jj = 0; jj < Ly::PTW; ++jj)
        bf[jj] = *reinterpret_cast<const h8*>(&sm.xt[(16 * (pt0 + jj) + lr) * kXP + 32 * kk + 8 * q]);
#pragma unroll
      for (int i = 0; i < Ly::NTW; ++i) {
        h8 af = *reinterpret_cast<const h8*>(&sm.bt[(16 * (nt0 + i) + lr) * Ly::BTP + 32 * kk + 8 * q]);
#pragma unroll
        for (int jj = 0; jj < Ly::PTW; ++jj) acc[i][jj] = mfma16(af, bf[jj], acc[i][jj]);
      }
    }
  };

  // ---- phase 1: local chunk state  s_c = sum_s e^{S_end-S_s} dt_s x_s B_s^T --
  f4 acc[Ly::NTW][Ly::PTW];
#pragma unroll
  for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
    for (int jj = 0; jj < Ly::PTW; ++jj) acc[i][jj] = f4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < Jv; ++j) {
    stage_state_operands(pf, j, Send);
    lds_barrier();
    if (j + 1 < Jv) fetch(pf, j + 1, false, Send);
    else fetch(pf, 0, true, sm.S[kTS - 1]);   // first sub-chunk of the output phase
    state_mfma(acc);
    lds_barrier();
  }

  // ---- phase 2: carry-in state, hand-off to the next chunk -----------------
  f4 R[Ly::NTW][Ly::PTW];   // state entering the current sub-chunk (fp32)
  {
    if (c == 0) {
#pragma unroll
      for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
        for (int jj = 0; jj < Ly::PTW; ++jj) {
          if (a.state_in) {
            const int p = 16 * (pt0 + jj) + lr, n = 16 * (nt0 + i) + 4 * q;
            R[i][jj] = *reinterpret_cast<const f4*>(a.state_in + ((size_t)bh * kP + p) * N + n);
          } else {
            R[i][jj] = f4{0.f, 0.f, 0.f, 0.f};
          }
        }
    } else {
      const unsigned pred = item - BH;
      if (tid == 0) {
        unsigned spins = 0;
        while (__hip_atomic_load(&a.flags[pred], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != gen + 1u) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > kSpinLimit) {
            __hip_atomic_fetch_or(&a.ctrl[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
      }
      __syncthreads();
      // device-coherent loads: they never hit a stale line of this XCD's L2
      const uint64_t* src = reinterpret_cast<const uint64_t*>(a.states + ((size_t)pred * 4 + w) * Ly::TILES * 256);
#pragma unroll
      for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
        for (int jj = 0; jj < Ly::PTW; ++jj) {
          const uint64_t* q2 = src + ((i * Ly::PTW + jj) * 256 + lane * 4) / 2;
          const uint64_t lo = __hip_atomic_load(q2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint64_t hi = __hip_atomic_load(q2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          R[i][jj] = f4{__uint_as_float((unsigned)lo), __uint_as_float((unsigned)(lo >> 32)),
                        __uint_as_float((unsigned)hi), __uint_as_float((unsigned)(hi >> 32))};
        }
    }
    const float dec = exp2f(Send);
    if (c + 1 < a.nchunks) {
      // device-coherent (write-through) stores, then wait until every wave's
      // stores have completed before the flag is raised
      uint64_t* dst = reinterpret_cast<uint64_t*>(a.states + ((size_t)item * 4 + w) * Ly::TILES * 256);
#pragma unroll
      for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
        for (int jj = 0; jj < Ly::PTW; ++jj) {
          const f4 v = R[i][jj] * dec + acc[i][jj];
          uint64_t* q2 = dst + ((i * Ly::PTW + jj) * 256 + lane * 4) / 2;
          __hip_atomic_store(q2, (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(q2 + 1, (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) __hip_atomic_store(&a.flags[item], gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (a.state_out) {
#pragma unroll
      for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
        for (int jj = 0; jj < Ly::PTW; ++jj) {
          const int p = 16 * (pt0 + jj) + lr, n = 16 * (nt0 + i) + 4 * q;
          *reinterpret_cast<f4*>(a.state_out + ((size_t)bh * kP + p) * N + n) = R[i][jj] * dec + acc[i][jj];
        }
    }
  }

  // ---- phase 3: outputs, sub-chunk by sub-chunk ----------------------------
  for (int j = 0; j < Jv; ++j) {
    const int i0 = j * kTS;
    const float Sj_start = j ? sm.S[i0 - 1] : 0.f;
    const float Sj_end = sm.S[i0 + kTS - 1];
    // stage: R (f16), dt*x, weighted B^T for the running state, B, C as read
    stage_state_operands(pf, j, Sj_end);
#pragma unroll
    for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
      for (int jj = 0; jj < Ly::PTW; ++jj) {
        const f4 v = R[i][jj];
        const int p = 16 * (pt0 + jj) + lr, n = 16 * (nt0 + i) + 4 * q;
        *reinterpret_cast<h4*>(&sm.r[p * Ly::NP + n]) = h4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
      }
    if (bact) {
#pragma unroll
      for (int k = 0; k < PF::TPT; ++k) {
        const bool ok = i0 + sb + k < nvalid;
        const h8 z8 = {};
        *reinterpret_cast<h8*>(&sm.bn[(sb + k) * Ly::NP + nb * 8]) = ok ? pf.b[k] : z8;
        *reinterpret_cast<h8*>(&sm.cn[(sb + k) * Ly::NP + nb * 8]) = ok ? pf.c[k] : z8;
      }
    }
    lds_barrier();
    if (j + 1 < Jv) fetch(pf, j + 1, true, sm.S[i0 + 2 * kTS - 1]);
    // running state for the next sub-chunk: R <- e^{S_end_j - S_start_j} R + s_j
    if (j + 1 < Jv) {
      const float dec = exp2f(Sj_end - Sj_start);
#pragma unroll
      for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
        for (int jj = 0; jj < Ly::PTW; ++jj) R[i][jj] *= dec;
      state_mfma(R);
    }
    {
      const int T = w;                       // this wave's 16 tokens: i0 + 16T + lr
      const int ti = i0 + 16 * T + lr;       // chunk-relative token of this lane's column
      const float St = sm.S[ti];
      // C.B^T for s-tiles 0..T, masked and decayed
      f4 m[4];
#pragma unroll
      for (int S = 0; S < 4; ++S) {
        m[S] = f4{0.f, 0.f, 0.f, 0.f};
        if (S <= T) {
#pragma unroll
          for (int kk = 0; kk < Ly::KN; ++kk) {
            const int n0 = 32 * kk + 8 * q;
            h8 af = {}, bf = {};
            if (n0 < N) {
              af = *reinterpret_cast<const h8*>(&sm.bn[(16 * S + lr) * Ly::NP + n0]);
              bf = *reinterpret_cast<const h8*>(&sm.cn[(16 * T + lr) * Ly::NP + n0]);
            }
            m[S] = mfma16(af, bf, m[S]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int si = i0 + 16 * S + 4 * q + i;
            m[S][i] = (si <= ti) ? m[S][i] * (float)sm.dts[si] * exp2f(St - sm.S[si]) : 0.f;
          }
        }
      }
      f4 yacc[4], racc[4];
#pragma unroll
      for (int tp = 0; tp < 4; ++tp) { yacc[tp] = f4{0.f, 0.f, 0.f, 0.f}; racc[tp] = f4{0.f, 0.f, 0.f, 0.f}; }
      // diagonal: Y^T[p, t] += sum_s x^T[p, s] M^T[s, t],  M = (C.B^T) dt_s e^{S_t-S_s} masked
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        if (2 * pr <= T) {
          const int S0 = 2 * pr, S1 = 2 * pr + 1;
          h8 bf = {(_Float16)m[S0][0], (_Float16)m[S0][1], (_Float16)m[S0][2], (_Float16)m[S0][3],
                   (_Float16)m[S1][0], (_Float16)m[S1][1], (_Float16)m[S1][2], (_Float16)m[S1][3]};
#pragma unroll
          for (int tp = 0; tp < 4; ++tp) {
            const _Float16* row = &sm.xt[(16 * tp + lr) * kXP];
            h8 af = cat(*reinterpret_cast<const h4*>(row + 16 * S0 + 4 * q),
                        *reinterpret_cast<const h4*>(row + 16 * S1 + 4 * q));
            yacc[tp] = mfma16(af, bf, yacc[tp]);
          }
        }
      }
      // carry-in readout: R[p, n] C[t, n]
#pragma unroll
      for (int kk = 0; kk < Ly::KN; ++kk) {
        const int n0 = 32 * kk + 8 * q;
        h8 bf = {};
        if (n0 < N) bf = *reinterpret_cast<const h8*>(&sm.cn[(16 * T + lr) * Ly::NP + n0]);
#pragma unroll
        for (int tp = 0; tp < 4; ++tp) {
          h8 af = {};
          if (n0 < N) af = *reinterpret_cast<const h8*>(&sm.r[(16 * tp + lr) * Ly::NP + n0]);
          racc[tp] = mfma16(af, bf, racc[tp]);
        }
      }
      const float sc = exp2f(St - Sj_start);
      if (ti < nvalid) {
        const size_t tok = (size_t)b * a.L + t0 + ti;
        IO* yrow = a.y + (tok * a.H + h) * kP;
        float gsq = 0.f;
#pragma unroll
        for (int tp = 0; tp < 4; ++tp) {
          const int p0 = 16 * tp + 4 * q;
          float xv[4];
          if constexpr (CONV || sizeof(IO) == 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[i] = (float)sm.xt[(p0 + i) * kXP + 16 * T + lr];
          } else {
            const IO* xrow = a.x + (tok * a.H + h) * kP + p0;
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[i] = io<IO>::load1(xrow + i);
          }
          f4 out;
#pragma unroll
          for (int i = 0; i < 4; ++i) out[i] = yacc[tp][i] + sc * racc[tp][i] + Dh * xv[i];
          if (NORM) {
            const IO* zrow = a.z + (tok * a.H + h) * kP + p0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float zz = io<IO>::load1(zrow + i);
              out[i] = out[i] * (zz / (1.f + __expf(-zz)));
              gsq += out[i] * out[i];
            }
          }
          io<IO>::store4(yrow + p0, out);
        }
        if (NORM) {
          gsq += __shfl_xor(gsq, 16, 64);
          gsq += __shfl_xor(gsq, 32, 64);
          if (q == 0) a.normsum[tok * a.H + h] = gsq;
        }
      }
    }
    lds_barrier();
  }

  // ---- conv state out: the 3 raw tokens before the sequence end -------------
  if (CONV && a.conv_out) {
    const int clast = len > 0 ? (len - 1) / a.Q : 0;
    if (c == clast) {
      const int hpg = a.H / a.G;
      const int nch = kP + ((h % hpg) == 0 ? 2 * N : 0);
      for (int k = tid; k < nch * 3; k += 256) {
        const int ci = k / 3, kk = k % 3;
        const int ch = ci < kP ? h * kP + ci : (ci - kP < N ? a.H * kP + g * N + (ci - kP)
                                                             : a.H * kP + a.G * N + g * N + (ci - kP - N));
        const int tau = len - 3 + kk;
        float v;
        if (tau >= 0) v = io<IO>::load1(a.xBC + ((size_t)b * a.L + tau) * a.Cd + ch);
        else v = a.conv_in ? io<IO>::load1(a.conv_in + ((size_t)b * a.Cd + ch) * 3 + 3 + tau) : 0.f;
        io<IO>::store1(a.conv_out + ((size_t)b * a.Cd + ch) * 3 + kk, v);
      }
    }
  }

  // ---- retire: the last item resets the ticket and bumps the generation -----
  __syncthreads();
  if (tid == 0) {
    const unsigned total = (unsigned)(a.nchunks * BH);
    // Relaxed: the next call reads these only after this kernel has ended.
    const unsigned done = __hip_atomic_fetch_add(&a.ctrl[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == total - 1) {
      __hip_atomic_store(&a.ctrl[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctrl[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctrl[2], gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Gated RMSNorm finish: out = g * rsqrt(mean_group(g^2) + eps) * w, with the
// per-head sums of g^2 produced by the scan's epilogue.  One block per token.
template <typename IO>
__global__ __launch_bounds__(256) void gated_norm_kernel(IO* __restrict__ y, const float* __restrict__ normsum,
                                                         const float* __restrict__ nw, const int* __restrict__ seqlens,
                                                         int L, int H, int group, float eps) {
  __shared__ float rs[256];
  const int tok = blockIdx.x, b = tok / L, t = tok - b * L;
  int len = seqlens ? seqlens[b] : L;
  len = len < 0 ? 0 : (len > L ? L : len);
  if (t >= len) return;
  const int C = H * kP, ngr = C / group, hpgr = group / kP;
  for (int gi = threadIdx.x; gi < ngr; gi += 256) {
    float s = 0.f;
    for (int k = 0; k < hpgr; ++k) s += normsum[(size_t)tok * H + gi * hpgr + k];
    rs[gi] = rsqrtf(s / (float)group + eps);
  }
  __syncthreads();
  IO* row = y + (size_t)tok * C;
  for (int c0 = threadIdx.x * 8; c0 < C; c0 += 256 * 8) {
    float v[8];
    io<IO>::load8(row + c0, v);
    const float r = rs[c0 / group];
    f4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) { lo[e] = v[e] * r * nw[c0 + e]; hi[e] = v[4 + e] * r * nw[c0 + 4 + e]; }
    io<IO>::store4(row + c0, lo);
    io<IO>::store4(row + c0 + 4, hi);
  }
}

// ---------------------------------------------------------------------------
struct WsLayout {
  size_t ctrl, flags, states, normsum, total;
};
static WsLayout ws_layout(const mamba2_dims& d) {
  const size_t nchunks = ((size_t)d.seqlen + d.chunk - 1) / d.chunk;
  const size_t items = nchunks * d.batch * d.nheads;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  WsLayout w;
  w.ctrl = 0;
  w.flags = 256;
  w.states = up(w.flags + items * 4);
  w.normsum = up(w.states + items * (size_t)kP * d.dstate * 4);
  w.total = up(w.normsum + (d.norm_group > 0 ? (size_t)d.batch * d.seqlen * d.nheads * 4 : 0));
  return w;
}

size_t window_workspace_bytes(const mamba2_dims& d) { return ws_layout(d).total; }

template <typename IO, int N, bool CONV, bool NORM>
static hipError_t launch_T(const WinArgs<IO>& a, hipStream_t st) {
  const unsigned items = (unsigned)(a.nchunks * a.B * a.H);
  ssd_window_kernel<IO, N, CONV, NORM><<<items, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <typename IO, int N>
static hipError_t launch_N(const WinArgs<IO>& a, bool conv, bool norm, hipStream_t st) {
  if (conv && norm) return launch_T<IO, N, true, true>(a, st);
  if (conv) return launch_T<IO, N, true, false>(a, st);
  if (norm) return launch_T<IO, N, false, true>(a, st);
  return launch_T<IO, N, false, false>(a, st);
}

template <typename IO>
static hipError_t launch_IO(const mamba2_dims& d, const mamba2_window_io& io_, void* ws, hipStream_t st) {
  const WsLayout wl = ws_layout(d);
  WinArgs<IO> a;
  a.B = d.batch; a.L = d.seqlen; a.H = d.nheads; a.G = d.ngroups; a.Q = d.chunk;
  a.nchunks = (d.seqlen + d.chunk - 1) / d.chunk;
  a.norm = d.norm_group;
  a.Cd = d.nheads * kP + 2 * d.ngroups * d.dstate;
  a.x = (const IO*)io_.x; a.Bm = (const IO*)io_.B; a.Cm = (const IO*)io_.C;
  a.xBC = (const IO*)io_.xBC; a.conv_w = io_.conv_w; a.conv_b = io_.conv_b;
  a.conv_in = (const IO*)io_.conv_state_in; a.conv_out = (IO*)io_.conv_state_out;
  a.dt = (const IO*)io_.dt; a.A = io_.A; a.D = io_.D;
  a.state_in = io_.state_in; a.state_out = io_.state_out; a.seqlens = io_.seqlens;
  a.z = (const IO*)io_.z; a.y = (IO*)io_.y;
  char* base = (char*)ws;
  a.ctrl = (unsigned*)(base + wl.ctrl);
  a.flags = (unsigned*)(base + wl.flags);
  a.states = (float*)(base + wl.states);
  a.normsum = (float*)(base + wl.normsum);
  const bool conv = d.conv_width == 4, norm = d.norm_group > 0;
  hipError_t e;
  switch (d.dstate) {
    case 16: e = launch_N<IO, 16>(a, conv, norm, st); break;
    case 64: e = launch_N<IO, 64>(a, conv, norm, st); break;
    default: e = launch_N<IO, 128>(a, conv, norm, st); break;
  }
  if (e != hipSuccess || !norm) return e;
  gated_norm_kernel<IO><<<(unsigned)(d.batch * d.seqlen), 256, 0, st>>>(
      (IO*)io_.y, a.normsum, io_.norm_w, io_.seqlens, d.seqlen, d.nheads, d.norm_group, d.norm_eps);
  return hipGetLastError();
}

hipError_t launch_window(const mamba2_dims& d, const mamba2_window_io& io_, void* ws, hipStream_t st) {
  if (d.io_dtype == MAMBA2_F16) return launch_IO<_Float16>(d, io_, ws, st);
  return launch_IO<float>(d, io_, ws, st);
}

}  // namespace m2

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
//  * one 512-thread workgroup (8 waves) per (chunk, sequence, head) item, taken
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
#ifndef M2_WAVES
#define M2_WAVES 8
#endif
#ifndef M2_DEPTH
#define M2_DEPTH 1
#endif
constexpr int kDepth = M2_DEPTH;  // sub-chunk steps the global loads run ahead (1 or 2)
constexpr int kWaves = M2_WAVES;  // waves per workgroup (4 or 8)
constexpr int kThreads = 64 * kWaves;
constexpr int kNormParts = kWaves / 4;   // partial sums of g^2 per (token, head)

template <int N> struct Lay {
  static constexpr int NT = N / 16;          // n-tiles of the state
  static constexpr int KN = (N + 31) / 32;   // k-steps over n
  static constexpr int NP = N + 8;           // pitch of [s][n] and [p][n] tiles (halfs)
  static constexpr int BTP = kTS + 8;        // pitch of the [n][s] tile
  // state tiles (n-tile x p-tile) owned by each wave: whole n-tiles x all four
  // p-tiles when there are at least as many n-tiles as waves, else one n-tile
  // x a share of the p-tiles (N=16 with 8 waves: one tile on waves 0..3)
  static constexpr bool WIDE = NT >= kWaves;
  static constexpr int NTW = WIDE ? NT / kWaves : 1;
  static constexpr int PTW = WIDE ? 4 : (4 * NT >= kWaves ? 4 * NT / kWaves : 1);
  static constexpr int TILES = NTW * PTW;
  static constexpr int STATE_FLOATS = kWaves * TILES * 256;   // private hand-off layout
  static __device__ __forceinline__ int nt0(int w) { return WIDE ? w * NTW : w % NT; }
  static __device__ __forceinline__ int pt0(int w) { return WIDE ? 0 : (w / NT) * PTW; }
  static __device__ __forceinline__ bool owns(int w) { return WIDE || w < 4 * NT; }
};

template <int N, bool CONV> struct alignas(16) Smem {
  alignas(16) _Float16 xt[kP * kXP];                 // [p][s]: x (post-conv when fused), transposed
  union alignas(16) {
    alignas(16) _Float16 bt[N * Lay<N>::BTP];        // [n][s]: dt- and decay-weighted B, transposed
    alignas(16) _Float16 mt[kTS * kXN];              // [t][s]: decay-masked C.B^T (after the state update)
  };
  alignas(16) _Float16 bn[kTS * Lay<N>::NP];         // [s][n]: B as read
  alignas(16) _Float16 cn[kTS * Lay<N>::NP];         // [t][n]: C as read
  union alignas(16) {
    alignas(16) _Float16 r[kP * Lay<N>::NP];         // [p][n]: state entering the sub-chunk
    struct {                                         // look-back list (carry-in phase only)
      unsigned lb_item[65];
      float lb_coef[65];
      int lb_kind[65];   // 0 aggregate, 1 inclusive, 2 initial state
      int lb_n;
    };
  };
  alignas(16) float u[kTS];                          // dt_s e^{S_r - S_s}, r = last token of s's 16-token tile
  float S[256];                                      // running log2-decay from the chunk start (inclusive)
  _Float16 dts[256];                                 // dt per token (0 past the sequence end)
  float wsum[kWaves];
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
  unsigned* ctrl;     // per-partition claim counters, done counter, generation, error
  unsigned* flags;    // per item: generation tag | 1 (aggregate) | 2 (inclusive)
  float* agg;         // per item local chunk state (private layout)
  float* incl;        // per item inclusive state after the chunk (private layout)
  unsigned* aggdec;   // per item chunk decay e^{S_end} (float bits)
  int tree_lg;        // log2 of the radix of the chunk tree (plain-input scan)
};

// control block: eight claim counters and the done counter / generation /
// error word, each on its own 128-byte line
constexpr int kCtrlStride = 32;
constexpr int kCtrlDone = 8 * kCtrlStride;
constexpr int kCtrlGen = 9 * kCtrlStride;
constexpr int kCtrlErr = 10 * kCtrlStride;
constexpr int kCtrlBytes = 11 * kCtrlStride * 4;

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
  // NE (4 or 8) consecutive raw channels at token tau (< 0: history or zeros)
  template <int NE>
  static __device__ __forceinline__ void rawn(const WinArgs<IO>& a, int b, int tau, int ch0, float* r) {
    if (tau >= 0) {
      const IO* src = a.xBC + ((size_t)b * a.L + tau) * a.Cd + ch0;
      if constexpr (NE == 8) io<IO>::load8(src, r);
      else {
#pragma unroll
        for (int e = 0; e < NE; ++e) r[e] = io<IO>::load1(src + e);
      }
    } else if (a.conv_in) {
#pragma unroll
      for (int e = 0; e < NE; ++e) r[e] = io<IO>::load1(a.conv_in + ((size_t)b * a.Cd + ch0 + e) * 3 + 3 + tau);
    } else {
#pragma unroll
      for (int e = 0; e < NE; ++e) r[e] = 0.f;
    }
  }
  template <int NE = 8>
  static __device__ __forceinline__ void conv8f(const WinArgs<IO>& a, int b, int t, int ch0, float* v) {
    float acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = a.conv_b ? a.conv_b[ch0 + e] : 0.f;
    float w[NE][4];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      f4 ww = *reinterpret_cast<const f4*>(a.conv_w + (size_t)(ch0 + e) * 4);
      w[e][0] = ww[0]; w[e][1] = ww[1]; w[e][2] = ww[2]; w[e][3] = ww[3];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float r[NE];
      rawn<NE>(a, b, t - 3 + k, ch0, r);
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[e] = __builtin_fmaf(w[e][k], r[e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) v[e] = acc[e] / (1.f + __expf(-acc[e]));
  }
  // NE (4 or 8) consecutive channels of x as binary16
  template <int NE, typename HV>
  static __device__ __forceinline__ HV xv(const WinArgs<IO>& a, int b, int t, int h, int p0) {
    HV r;
    if constexpr (CONV) {
      float v[NE];
      conv8f<NE>(a, b, t, h * kP + p0, v);
#pragma unroll
      for (int e = 0; e < NE; ++e) r[e] = (_Float16)v[e];
    } else {
      const IO* src = a.x + (((size_t)b * a.L + t) * a.H + h) * kP + p0;
      if constexpr (sizeof(IO) == 2) {
        r = *reinterpret_cast<const HV*>(src);
      } else {
#pragma unroll
        for (int e = 0; e < NE; e += 4) {
          const f4 v = *reinterpret_cast<const f4*>(src + e);
#pragma unroll
          for (int k = 0; k < 4; ++k) r[e + k] = (_Float16)v[k];
        }
      }
    }
    return r;
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

// x channels per thread per token (two tokens per thread)
constexpr int kXE = (kTS * kP) / (2 * kThreads);
typedef _Float16 hx __attribute__((ext_vector_type(kXE)));

// One thread's share of a 64-token sub-chunk, fetched ahead of its use.
//   x: tokens sx, sx+1 at channels kXE*px .. kXE*px+kXE-1 of the head
//   B, C: tokens sb..sb+TPT-1 at state columns 8*nb..8*nb+7 of the group
//   bs (fused conv only): B weighted for the state contraction, formed from the
//   fp32 conv output so that the weighted B is rounded to binary16 once
template <int N, bool CONV> struct Pref {
  static constexpr int NCH = N / 8;
  static constexpr int TPT = (kTS * NCH) / kThreads > 0 ? (kTS * NCH) / kThreads : 1;
  hx x[2];
  h8 b[TPT];
  h8 c[TPT];
  h8 bs[CONV ? TPT : 1];
};

template <typename IO, int N, bool CONV, bool NORM>
__global__ __launch_bounds__(kThreads, 2) void ssd_window_kernel(WinArgs<IO> a) {
  using Ly = Lay<N>;
  using SRC = Src<IO, CONV>;
  using PF = Pref<N, CONV>;
  __shared__ Smem<N, CONV> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, q = lane >> 4;
  const int BH = a.B * a.H;
  const int hpg = a.H / a.G;

  // ---- claim an item ------------------------------------------------------
  // Items are split into 8 partitions by (sequence, group) so that the heads
  // sharing B/C, and the chunks of one head, run on one XCD and meet in its
  // L2.  A workgroup claims from the partition of the XCD it runs on, and from
  // the others once that one is used up.  Inside a partition items are handed
  // out chunk-major, so an item only ever waits for an item claimed before it.
  if (tid == 0) {
    sm.gen = __hip_atomic_load(&a.ctrl[kCtrlGen], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned x0 = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 7u;   // HW_REG_XCC_ID
    const int BG = a.B * a.G;
    unsigned px = 0, t = 0;
    for (int k = 0; k < 8; ++k) {
      px = (x0 + k) & 7u;
      const int npairs = BG > (int)px ? (BG - (int)px + 7) / 8 : 0;
      const unsigned n = (unsigned)(npairs * hpg * a.nchunks);
      if (n == 0) continue;
      unsigned* cnt = &a.ctrl[px * kCtrlStride];
      if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) continue;
      t = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t < n) {
        const int per_c = npairs * hpg;
        const int cc = (int)t / per_c, rem = (int)t - cc * per_c;
        const int gid = (int)px + 8 * (rem / hpg);
        const int bb = gid / a.G, gg = gid - bb * a.G;
        sm.ticket = (unsigned)(cc * BH + bb * a.H + gg * hpg + rem % hpg);
        break;
      }
    }
  }
  __syncthreads();
  const unsigned item = sm.ticket, gen = sm.gen;
  const unsigned tag = (gen & 0x3fffffffu) << 2;   // flag = tag | 1 (aggregate) or tag | 2 (inclusive)
  const int c = item / BH, bh = item - c * BH;
  const int b = bh / a.H, h = bh - b * a.H;
  const int g = h / hpg;
  int len = a.seqlens ? a.seqlens[b] : a.L;
  len = len < 0 ? 0 : (len > a.L ? a.L : len);
  const int t0 = c * a.Q;                      // first token of the chunk
  const int nvalid = min(max(len - t0, 0), a.Q);
  const int Jv = (nvalid + kTS - 1) / kTS;     // sub-chunks holding real tokens
  const float Ah = a.A[h] * kLog2e;
  const float Dh = a.D[h];

  // per-thread staging coordinates
  const int px = tid % (kP / kXE), sx = 2 * (tid / (kP / kXE));
  const int nb = tid % PF::NCH, sb = (tid / PF::NCH) * PF::TPT;
  const bool bact = sb < kTS;

  // The work of an item is a sequence of 2*Jv steps over its 64-token
  // sub-chunks: steps [0, Jv) accumulate the chunk state, steps [Jv, 2Jv)
  // produce the outputs.  Global loads run two steps ahead of their use.
  const int NS = 2 * Jv;
  // issue the global loads of step k (tokens past the end are fetched from a
  // valid token and zeroed when written to LDS)
  auto fetch = [&](PF& f, int k) {
    const bool out = k >= Jv;
    const int j = out ? k - Jv : k;
    const int i0 = j * kTS;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int s = i0 + sx + kk;
      f.x[kk] = SRC::template xv<kXE, hx>(a, b, t0 + (s < nvalid ? s : i0), h, px * kXE);
    }
    if (bact) {
      // fused conv only: weight reference of this step (chunk end, or sub-chunk end)
      const float Sref = CONV ? (out ? sm.S[i0 + kTS - 1] : sm.S[a.Q - 1]) : 0.f;
#pragma unroll
      for (int kk = 0; kk < PF::TPT; ++kk) {
        const int s = i0 + sb + kk;
        const int t = t0 + (s < nvalid ? s : i0);
        if constexpr (CONV) {
          float v[8];
          SRC::conv8f(a, b, t, a.H * kP + g * N + nb * 8, v);
          const float wgt = s < nvalid ? (float)sm.dts[s] * exp2f(Sref - sm.S[s]) : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            f.b[kk][e] = (_Float16)v[e];
            f.bs[kk][e] = (_Float16)(v[e] * wgt);
          }
        } else {
          f.b[kk] = SRC::template b8<N>(a, b, t, g, nb * 8);
        }
        if (out) f.c[kk] = SRC::template c8<N>(a, b, t, g, nb * 8);
      }
    }
  };

  PF pa, pb;
  if (!CONV) {
    if (NS > 0) fetch(pa, 0);
    if (kDepth == 2 && NS > 1) fetch(pb, 1);
  }

  // ---- phase 0: dt and the inclusive running log2-decay over the chunk -----
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
  if (CONV) {
    if (NS > 0) fetch(pa, 0);
    if (kDepth == 2 && NS > 1) fetch(pb, 1);
  }

  // state tiles of this wave: n-tile nt0+i, p-tile pt0+jj
  const int nt0 = Ly::nt0(w), pt0 = Ly::pt0(w);
  const bool owner = Ly::owns(w);

  // write x (transposed, as read: no rounding for f16 inputs) and the
  // transposed B weighted by dt_s e^{Sref - S_s} of sub-chunk j
  auto stage_state_operands = [&](const PF& f, int j, float Sref) {
    const int i0 = j * kTS;
    {
      const bool ok0 = i0 + sx < nvalid, ok1 = i0 + sx + 1 < nvalid;
      const _Float16 zero = (_Float16)0.f;
#pragma unroll
      for (int e = 0; e < kXE; ++e)
        *reinterpret_cast<h2*>(&sm.xt[(px * kXE + e) * kXP + sx]) = h2{ok0 ? f.x[0][e] : zero, ok1 ? f.x[1][e] : zero};
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
    if (!owner) return;
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
  // private layout of a hand-off state: [wave][tile][lane][4] floats
  auto st_off = [&](unsigned it, int i, int jj) -> size_t {
    return (size_t)it * Ly::STATE_FLOATS + ((size_t)w * Ly::TILES + (i * Ly::PTW + jj)) * 256 + lane * 4;
  };
  // device-coherent (write-through) store / load of this thread's state values
  auto put_state = [&](float* base, unsigned it, const f4 (&v)[Ly::NTW][Ly::PTW]) {
    if (!owner) return;
#pragma unroll
    for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
      for (int jj = 0; jj < Ly::PTW; ++jj) {
        uint64_t* q2 = reinterpret_cast<uint64_t*>(base + st_off(it, i, jj));
        const f4 x4 = v[i][jj];
        __hip_atomic_store(q2, (uint64_t)__float_as_uint(x4[0]) | ((uint64_t)__float_as_uint(x4[1]) << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(q2 + 1, (uint64_t)__float_as_uint(x4[2]) | ((uint64_t)__float_as_uint(x4[3]) << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  };
  auto add_state = [&](const float* base, unsigned it, float coef, f4 (&v)[Ly::NTW][Ly::PTW]) {
    if (!owner) return;
#pragma unroll
    for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
      for (int jj = 0; jj < Ly::PTW; ++jj) {
        const uint64_t* q2 = reinterpret_cast<const uint64_t*>(base + st_off(it, i, jj));
        const uint64_t lo = __hip_atomic_load(q2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t hi = __hip_atomic_load(q2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v[i][jj] += coef * f4{__uint_as_float((unsigned)lo), __uint_as_float((unsigned)(lo >> 32)),
                              __uint_as_float((unsigned)hi), __uint_as_float((unsigned)(hi >> 32))};
      }
  };
  // raise this item's flag once every wave's stores have completed
  auto raise_flag = [&](unsigned status) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(&a.flags[item], tag | status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  f4 acc[Ly::NTW][Ly::PTW];   // local chunk state, from zero at the chunk start
#pragma unroll
  for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
    for (int jj = 0; jj < Ly::PTW; ++jj) acc[i][jj] = f4{0.f, 0.f, 0.f, 0.f};
  f4 R[Ly::NTW][Ly::PTW];     // state entering the current sub-chunk (fp32)
  const float dec_chunk = exp2f(Send);

  // ---- phase 2: carry-in state and hand-off to later chunks -----------------
  // Decoupled look-back: a chunk first publishes its local (aggregate) state,
  // then starts from the nearest published inclusive state of an earlier chunk,
  // applies the aggregates in between, and publishes its own inclusive state.
  // No chunk waits for a chain of hand-offs to ripple through.
  auto carry_in = [&]() {
    const bool publish = c + 1 < a.nchunks;
    if (c > 0 && publish) {
      put_state(a.agg, item, acc);
      if (tid == 0) __hip_atomic_store(&a.aggdec[item], __float_as_uint(dec_chunk), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
      raise_flag(1u);
    }
#pragma unroll
    for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
      for (int jj = 0; jj < Ly::PTW; ++jj) R[i][jj] = f4{0.f, 0.f, 0.f, 0.f};
    if (c > 0) {
      if (w == 0) {
        const int W = c < 64 ? c : 64;      // predecessors c-1 .. c-W, one per lane
        const unsigned pred = (unsigned)((c - 1 - lane) * BH + bh);
        unsigned spins = 0;
        int need = 0, lstar = W;
        while (true) {
          unsigned st = 0;
          if (lane < W) {
            const unsigned f = __hip_atomic_load(&a.flags[pred], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            st = (f & ~3u) == tag ? (f & 3u) : 0u;
          }
          const unsigned long long incl = __ballot(st == 2u), ready = __ballot(st >= 1u);
          lstar = incl ? (int)__builtin_ctzll(incl) : W;            // nearest inclusive
          need = lstar;                                               // aggregates before it
          const unsigned long long m = need >= 64 ? ~0ull : ((1ull << need) - 1ull);
          bool ok = (ready & m) == m;
          if (lstar == W && c > W) ok = false;                        // window too short: wait
          if (ok) break;
          __builtin_amdgcn_s_sleep(1);
          if (++spins > kSpinLimit) {
            if (lane == 0) __hip_atomic_fetch_or(&a.ctrl[kCtrlErr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            need = 0; lstar = W;
            break;
          }
        }
        // The carry-in state is rebuilt from the nearest inclusive state (or the
        // initial state) by applying the later chunks' hand-offs in order,
        // H <- a_k H + s_k, with the same fused multiply-add the chain itself
        // uses -- so the result is bitwise the same whichever predecessor
        // happened to be published first.  List order: base, then aggregates
        // of chunks c-need .. c-1.
        if (lane < need) {
          const int e = need - lane;                         // chunk c-1-lane at position e
          sm.lb_item[e] = pred;
          sm.lb_coef[e] = __uint_as_float(__hip_atomic_load(&a.aggdec[pred], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          sm.lb_kind[e] = 0;
        }
        if (lane == 0) {
          if (lstar < W) {                       // an inclusive state of an earlier chunk
            sm.lb_item[0] = (unsigned)((c - 1 - lstar) * BH + bh);
            sm.lb_kind[0] = 1;
          } else {
            sm.lb_kind[0] = a.state_in ? 2 : 3;  // the initial state, or zeros
          }
          sm.lb_n = need + 1;
        }
      }
      __syncthreads();
      const int n = sm.lb_n;
      {
        const int kind = sm.lb_kind[0];
        if (owner) {
          if (kind == 1) {
            add_state(a.incl, sm.lb_item[0], 1.f, R);
          } else if (kind == 2) {
#pragma unroll
            for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
              for (int jj = 0; jj < Ly::PTW; ++jj) {
                const int p = 16 * (pt0 + jj) + lr, nn = 16 * (nt0 + i) + 4 * q;
                R[i][jj] = *reinterpret_cast<const f4*>(a.state_in + ((size_t)bh * kP + p) * N + nn);
              }
          }
        }
      }
      for (int e = 1; e < n; ++e) {
        if (owner) {
          f4 Ae[Ly::NTW][Ly::PTW];
#pragma unroll
          for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
            for (int jj = 0; jj < Ly::PTW; ++jj) Ae[i][jj] = f4{0.f, 0.f, 0.f, 0.f};
          add_state(a.agg, sm.lb_item[e], 1.f, Ae);
          const float ae = sm.lb_coef[e];
#pragma unroll
          for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
            for (int jj = 0; jj < Ly::PTW; ++jj)
#pragma unroll
              for (int k = 0; k < 4; ++k) R[i][jj][k] = __builtin_fmaf(ae, R[i][jj][k], Ae[i][jj][k]);
        }
      }
    } else if (a.state_in && owner) {
#pragma unroll
      for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
        for (int jj = 0; jj < Ly::PTW; ++jj) {
          const int p = 16 * (pt0 + jj) + lr, nn = 16 * (nt0 + i) + 4 * q;
          R[i][jj] = *reinterpret_cast<const f4*>(a.state_in + ((size_t)bh * kP + p) * N + nn);
        }
    }
    // inclusive state after this chunk, H_c = a_c H_{c-1} + s_c (in place: the
    // local state is no longer needed)
    f4 (&Hout)[Ly::NTW][Ly::PTW] = acc;
#pragma unroll
    for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
      for (int jj = 0; jj < Ly::PTW; ++jj)
#pragma unroll
        for (int k = 0; k < 4; ++k) Hout[i][jj][k] = __builtin_fmaf(dec_chunk, R[i][jj][k], acc[i][jj][k]);
    if (publish) {
      put_state(a.incl, item, Hout);
      raise_flag(2u);
    } else if (a.state_out && owner) {
#pragma unroll
      for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
        for (int jj = 0; jj < Ly::PTW; ++jj) {
          const int p = 16 * (pt0 + jj) + lr, nn = 16 * (nt0 + i) + 4 * q;
          *reinterpret_cast<f4*>(a.state_out + ((size_t)bh * kP + p) * N + nn) = Hout[i][jj];
        }
    }
    // the look-back list shares LDS with the carried-state tile written next
    lds_barrier();
  };

  // ---- output step for sub-chunk j ------------------------------------------
  auto output_step = [&](PF& f, int j, int knext) {
    const int i0 = j * kTS;
    const float Sj_start = j ? sm.S[i0 - 1] : 0.f;
    const float Sj_end = sm.S[i0 + kTS - 1];
    // stage: R (f16), x, weighted B^T for the running state, B, C as read
    stage_state_operands(f, j, Sj_end);
    if (tid < kTS) {
      const int s = i0 + tid;
      sm.u[tid] = s < nvalid ? (float)sm.dts[s] * exp2f(sm.S[i0 + (tid | 15)] - sm.S[s]) : 0.f;
    }
    if (owner)
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
        *reinterpret_cast<h8*>(&sm.bn[(sb + k) * Ly::NP + nb * 8]) = ok ? f.b[k] : z8;
        *reinterpret_cast<h8*>(&sm.cn[(sb + k) * Ly::NP + nb * 8]) = ok ? f.c[k] : z8;
      }
    }
    lds_barrier();
    if (knext < NS) fetch(f, knext);
    // running state for the next sub-chunk: R <- e^{S_end_j - S_start_j} R + s_j
    if (j + 1 < Jv) {
      const float dec = exp2f(Sj_end - Sj_start);
#pragma unroll
      for (int i = 0; i < Ly::NTW; ++i)
#pragma unroll
        for (int jj = 0; jj < Ly::PTW; ++jj) R[i][jj] *= dec;
      state_mfma(R);
    }
    lds_barrier();   // the weighted B^T tile is dead: its space takes the masked C.B^T
    {
      // Decay-masked C.B^T, one causal 16x16 block (s-tile S <= t-tile T) per
      // job; the 10 jobs of a sub-chunk are spread over the 8 waves and the
      // blocks meet in LDS as M[t][s] = (C_t.B_s) dt_s e^{S_t - S_s}.  Off the
      // diagonal the decay is split at the last token r of the s-tile,
      // e^{S_t-S_r} e^{S_r-S_s}, both factors <= 1, so a lane needs one
      // exponential per block.
#pragma unroll
      for (int jb = 0; jb < (10 + kWaves - 1) / kWaves; ++jb) {
        const int job = w + kWaves * jb;
        if (job < 10) {
          // job -> (S, T): (0,0) (0,1) (1,1) (0,2) (1,2) (2,2) (0,3) (1,3) (2,3) (3,3)
          const int T = job < 1 ? 0 : (job < 3 ? 1 : (job < 6 ? 2 : 3));
          const int S = job - (T * (T + 1)) / 2;
          f4 cb = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < Ly::KN; ++kk) {
            const int n0 = 32 * kk + 8 * q;
            h8 af = {}, bf = {};
            if (n0 < N) {
              af = *reinterpret_cast<const h8*>(&sm.bn[(16 * S + lr) * Ly::NP + n0]);
              bf = *reinterpret_cast<const h8*>(&sm.cn[(16 * T + lr) * Ly::NP + n0]);
            }
            cb = mfma16(af, bf, cb);
          }
          const int tl = 16 * T + lr;                 // token of this lane's column
          const float St = sm.S[i0 + tl];
          const int s0 = 16 * S + 4 * q;              // first of this lane's four s
          f4 mv;
          if (S < T) {
            const float vt = exp2f(St - sm.S[i0 + 16 * S + 15]);
            const f4 uu = *reinterpret_cast<const f4*>(&sm.u[s0]);
#pragma unroll
            for (int i = 0; i < 4; ++i) mv[i] = cb[i] * uu[i] * vt;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int si = s0 + i;
              mv[i] = si <= tl ? cb[i] * (float)sm.dts[i0 + si] * exp2f(St - sm.S[i0 + si]) : 0.f;
            }
          }
          *reinterpret_cast<h4*>(&sm.mt[tl * kXN + s0]) = h4{(_Float16)mv[0], (_Float16)mv[1], (_Float16)mv[2], (_Float16)mv[3]};
        }
      }
      lds_barrier();
      constexpr int PTO = 16 / kWaves;       // p-tiles per wave in the output
      const int T = w & 3;                   // this wave's 16 tokens: i0 + 16T + lr
      const int tpb = PTO * (w >> 2);        // and its p-tiles tpb .. tpb+PTO-1
      const int ti = i0 + 16 * T + lr;       // chunk-relative token of this lane's column
      const float St = sm.S[ti];
      f4 yacc[PTO], racc[PTO];
#pragma unroll
      for (int u = 0; u < PTO; ++u) { yacc[u] = f4{0.f, 0.f, 0.f, 0.f}; racc[u] = f4{0.f, 0.f, 0.f, 0.f}; }
      // diagonal: Y^T[p, t] += sum_s x^T[p, s] M[t, s]
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        if (2 * pr <= T) {
          const int S0 = 2 * pr, S1 = 2 * pr + 1;
          const _Float16* mrow = &sm.mt[(16 * T + lr) * kXN];
          const h4 lo = *reinterpret_cast<const h4*>(mrow + 16 * S0 + 4 * q);
          const h4 hi = S1 <= T ? *reinterpret_cast<const h4*>(mrow + 16 * S1 + 4 * q) : h4{};
          const h8 bf = cat(lo, hi);
#pragma unroll
          for (int u = 0; u < PTO; ++u) {
            const _Float16* row = &sm.xt[(16 * (tpb + u) + lr) * kXP];
            h8 af = cat(*reinterpret_cast<const h4*>(row + 16 * S0 + 4 * q),
                        *reinterpret_cast<const h4*>(row + 16 * S1 + 4 * q));
            yacc[u] = mfma16(af, bf, yacc[u]);
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
        for (int u = 0; u < PTO; ++u) {
          h8 af = {};
          if (n0 < N) af = *reinterpret_cast<const h8*>(&sm.r[(16 * (tpb + u) + lr) * Ly::NP + n0]);
          racc[u] = mfma16(af, bf, racc[u]);
        }
      }
      const float sc = exp2f(St - Sj_start);
      if (ti < nvalid) {
        const size_t tok = (size_t)b * a.L + t0 + ti;
        IO* yrow = a.y + (tok * a.H + h) * kP;
        float gsq = 0.f;
#pragma unroll
        for (int u = 0; u < PTO; ++u) {
          const int p0 = 16 * (tpb + u) + 4 * q;
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
          for (int i = 0; i < 4; ++i) out[i] = yacc[u][i] + sc * racc[u][i] + Dh * xv[i];
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
          if (q == 0) a.normsum[(tok * a.H + h) * kNormParts + (w >> 2)] = gsq;   // this wave's share of the head
        }
      }
    }
    lds_barrier();
  };
  // chunk-state step for sub-chunk j (weights to the chunk end)
  auto state_step = [&](PF& f, int j, int knext) {
    stage_state_operands(f, j, Send);
    lds_barrier();
    if (knext < NS) fetch(f, knext);
    state_mfma(acc);
    lds_barrier();
  };
  auto run_step = [&](PF& f, int k) {
    if (k < Jv) state_step(f, k, k + kDepth);
    else output_step(f, k - Jv, k + kDepth);
  };

  // one inlined step body: pa always holds the data of step k; after the step
  // it is refilled with step k+kDepth (and with depth 2 the buffers trade places)
  for (int k = 0; k <= NS; ++k) {
    if (k == Jv) carry_in();
    if (k == NS) break;
    run_step(pa, k);
    if constexpr (kDepth == 2) {
      const PF t = pa;
      pa = pb;
      pb = t;
    }
  }

  // ---- conv state out: the 3 raw tokens before the sequence end -------------
  if (CONV && a.conv_out) {
    const int clast = len > 0 ? (len - 1) / a.Q : 0;
    if (c == clast) {
      const int nch = kP + ((h % hpg) == 0 ? 2 * N : 0);
      for (int k = tid; k < nch * 3; k += kThreads) {
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

  // ---- retire: the last item resets the counters and bumps the generation ---
  __syncthreads();
  if (tid == 0) {
    const unsigned total = (unsigned)(a.nchunks * BH);
    // Relaxed: the next call reads these only after this kernel has ended.
    const unsigned done = __hip_atomic_fetch_add(&a.ctrl[kCtrlDone], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == total - 1) {
      for (int k = 0; k < 8; ++k) __hip_atomic_store(&a.ctrl[k * kCtrlStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctrl[kCtrlDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctrl[kCtrlGen], gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ===========================================================================
// Chunked scan for plain x, B, C inputs: one workgroup per (chunk, sequence,
// group, block of KH heads of the group), one wave per (head, half of the
// head dim).
//
// Each half of a head is an independent scan (the recurrence is separable
// over p).  A wave keeps its 32 x N share of the fp32 state in registers as
// MFMA tiles of s^T[n, p], so the carry-in readout takes its A operand
// straight from those registers, and the wave stays within 256 registers so
// that two waves share each SIMD.  The KH heads of a workgroup read the same
// B and C rows: each 32-token step of B and C is loaded once per workgroup
// into LDS tiles (as read, [token][n]) and every wave takes its operands from
// there; x of a step goes into a per-wave LDS tile, once as read and once
// scaled by the per-token state weight, and is read back transposed
// (ds_read_b64_tr_b16) where tokens are the contraction index.
//
// State columns are kept in a permuted order so that the n-slots a lane owns
// in the state tiles are the slots it needs for the readout's contraction
// over n, so that a C fragment is one contiguous 16-byte read, and so that
// the four column groups of a transposed read of the B tile fall N/4 columns
// apart (in different LDS banks):
//   tile nt, row 4j + e  <->  n = (N/4) j + 8 (nt / 2) + 4 (nt % 2) + e   (N >= 32)
//   tile 0,  row 4j + e  <->  n = 4 j + e                                 (N = 16)
//
// Inputs are read through buffer descriptors whose range ends at the
// sequence's last token, so tokens at or past the sequence length read as
// zero (dt = 0 keeps the state) and their outputs are dropped by the store.
namespace wv {
constexpr int TS = 32;                 // tokens per step
constexpr int PH = 32;                 // head-dim columns per item
constexpr int PT = PH / 16;            // p-tiles per item
constexpr int XP = PH + 8;             // pitch (halfs) of the [s][p] x tiles
constexpr int kSc1 = 16;               // cache policy: device-coherent access

typedef short s4 __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Buffer descriptor over [p, p + bytes).  p and bytes must be wave-uniform;
// they are read from the first lane so that the descriptor is built in SGPRs
// (a descriptor the compiler cannot prove uniform turns every access through
// it into a loop over lanes).
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

// Transposed 64-bit LDS read: within each 16-lane group, lane i receives the
// 16-bit elements at column (i % 4) of the 8-byte chunks addressed by lanes
// 4k + i / 4, k = 0..3.
__device__ __forceinline__ h4 tr4(const _Float16* p) {
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4*)(__attribute__((address_space(3))) void*)(p));
  return __builtin_bit_cast(h4, v);
}

// NV (4 or 8) consecutive elements at byte offset off, as binary16, zero-padded to 8
template <typename IO, int NV> __device__ __forceinline__ h8 ldh(rsrc_t r, unsigned off) {
  if constexpr (sizeof(IO) == 2) {
    if constexpr (NV == 8) {
      return __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    } else {
      const h4 v = __builtin_bit_cast(h4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
      return h8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
    }
  } else {
    const f4 lo = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    f4 hi = f4{0.f, 0.f, 0.f, 0.f};
    if constexpr (NV == 8) hi = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
    return h8{(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
              (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]};
  }
}
template <typename IO> __device__ __forceinline__ float ld1(rsrc_t r, unsigned off) {
  if constexpr (sizeof(IO) == 2)
    return (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
  else
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
template <typename IO> __device__ __forceinline__ f4 ld4f(rsrc_t r, unsigned off) {
  if constexpr (sizeof(IO) == 2) {
    const h4 v = __builtin_bit_cast(h4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    return f4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  } else {
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
}
template <typename IO> __device__ __forceinline__ void st4(rsrc_t r, unsigned off, f4 v) {
  if constexpr (sizeof(IO) == 2) {
    const h4 hv = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, hv), r, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, 0);
  }
}

constexpr int KH = 4;                  // heads per workgroup
constexpr int NWV = 2 * KH;            // waves per workgroup

template <int N> struct SmG {
  static constexpr int NP = N + 8;     // pitch (halfs) of the [s][n] B and C tiles
  alignas(16) _Float16 b[TS * NP];     // [s][n] B as read
  alignas(16) _Float16 c[TS * NP];     // [t][n] C as read
  alignas(16) _Float16 x[NWV][TS * XP];   // per wave: [s][p] x as read
  alignas(16) _Float16 xw[NWV][TS * XP];  // per wave: x times the state weight of token s
  alignas(16) float S[NWV][256];       // per wave: running log2-decay from the chunk start (inclusive)
  alignas(16) _Float16 dts[NWV][256];
  unsigned ticket, gen;
};

// first state column of the 4-row group j of state tile nt
template <int N> __device__ __forceinline__ int ncol(int nt, int j) {
  if constexpr (N >= 32) return (N / 4) * j + 8 * (nt >> 1) + 4 * (nt & 1);
  else return 4 * j;
}
}  // namespace wv

static_assert(kNormParts >= 2, "one g^2 partial per head half");

template <typename IO, int N, bool NORM>
__global__ __launch_bounds__(64 * wv::NWV) void ssd_window_group_kernel(WinArgs<IO> a) {
  using namespace wv;
  constexpr unsigned ES = sizeof(IO);
  constexpr int NT = N / 16;                    // state tiles along n
  constexpr int KM = N >= 32 ? N / 32 : 1;      // 32-wide k-steps over n
  constexpr int NV = N >= 32 ? 8 : 4;           // real n per lane in a k-step
  constexpr int NCH = N / 8;                    // 8-element chunks per B or C row
  constexpr int NTH = 64 * NWV;
  constexpr int BK = (TS * NCH + NTH - 1) / NTH;   // B (and C) chunks per thread per step
  constexpr int XPL = TS * (PH / 8) / 64;       // x chunks per lane per step
  constexpr int NP = SmG<N>::NP;
  __shared__ SmG<N> sm;
  // wave-uniform values are pinned to scalar registers (readfirstlane): the
  // buffer descriptors built from them must live in SGPRs
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, q = lane >> 4;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hpg = a.H / a.G;
  const int nhb = (hpg + KH - 1) / KH;          // head blocks per group
  const int BG = a.B * a.G;
  // hand-off items run over virtual heads hv = 2 h + half
  const int HV = 2 * a.H;
  const int BHV = a.B * HV;

  // ---- claim a workgroup item: the XCD's own group pairs first, chunk-major --
  if (tid == 0) {
    sm.gen = __hip_atomic_load(&a.ctrl[kCtrlGen], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned x0 = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 7u;   // HW_REG_XCC_ID
    for (int k = 0; k < 8; ++k) {
      const unsigned px = (x0 + k) & 7u;
      const int npairs = BG > (int)px ? (BG - (int)px + 7) / 8 : 0;
      const unsigned n = (unsigned)(npairs * nhb * a.nchunks);
      if (n == 0) continue;
      unsigned* cnt = &a.ctrl[px * kCtrlStride];
      if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) continue;
      const unsigned t = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t < n) {
        const int per_c = npairs * nhb;
        const int cc = (int)t / per_c, rem = (int)t - cc * per_c;
        const int gid = (int)px + 8 * (rem / nhb);
        sm.ticket = (unsigned)((cc * BG + gid) * nhb + rem % nhb);
        break;
      }
    }
  }
  __syncthreads();
  const unsigned ticket = __builtin_amdgcn_readfirstlane(sm.ticket);
  const unsigned gen = __builtin_amdgcn_readfirstlane(sm.gen);
  const unsigned tag = (gen & 0x3fffffffu) << 2;
  const int hblk = (int)(ticket % (unsigned)nhb);
  const int c = (int)(ticket / (unsigned)nhb) / BG;
  const int gid = (int)(ticket / (unsigned)nhb) - c * BG;
  const int b = gid / a.G, g = gid - b * a.G;
  const int hin = hblk * KH + (wid >> 1);       // head within the group
  const bool live = hin < hpg;                  // waves past the group's last head only help load B, C
  const int h = g * hpg + (live ? hin : 0);
  const int half = wid & 1;
  const int hb = b * a.H + h;                   // (sequence, head) index
  const int bhv = b * HV + 2 * h + half;
  const unsigned item = (unsigned)(c * BHV + bhv);
  int len = a.seqlens ? __builtin_amdgcn_readfirstlane(a.seqlens[b]) : a.L;
  len = len < 0 ? 0 : (len > a.L ? a.L : len);
  const int t0 = c * a.Q;
  const int nvalid = min(max(len - t0, 0), a.Q);
  const int Jv = (nvalid + TS - 1) / TS;        // steps holding real tokens
  const float Ah = a.A[h] * kLog2e;
  const float Dh = a.D[h];

  // buffer views of this sequence (range ends at its last token)
  const unsigned xrow = (unsigned)(a.H * kP) * ES;     // bytes between tokens in x, z, y
  const unsigned grow = (unsigned)(a.G * N) * ES;      // in B, C
  const unsigned xspan = len > 0 && live ? (unsigned)(len - 1) * xrow + PH * ES : 0u;
  const unsigned gspan = len > 0 ? (unsigned)(len - 1) * grow + N * ES : 0u;
  const size_t seq_x = ((size_t)b * a.L * a.H + h) * kP + PH * half;
  const size_t seq_g = ((size_t)b * a.L * a.G + g) * N;
  const rsrc_t rx = mkr(a.x + seq_x, xspan);
  const rsrc_t rb = mkr(a.Bm + seq_g, gspan);
  const rsrc_t rc = mkr(a.Cm + seq_g, gspan);
  const rsrc_t ry = mkr(a.y + seq_x, xspan);
  const rsrc_t rdt = mkr(a.dt + (size_t)b * a.L * a.H + h, len > 0 && live ? (unsigned)((len - 1) * a.H + 1) * ES : 0u);
  float* const Sw = sm.S[wid];
  _Float16* const dtw = sm.dts[wid];
  _Float16* const xs = sm.x[wid];
  _Float16* const xws = sm.xw[wid];

  // ---- phase 0: dt and the running log2-decay over the chunk (4 tokens/lane) --
  {
    float d[4], v[4];
    float run = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * lane + e;
      d[e] = i < a.Q ? ld1<IO>(rdt, (unsigned)((t0 + i) * a.H) * ES) : 0.f;
      run += d[e] * Ah;
      v[e] = run;
    }
    float pre = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float u = __shfl_up(pre, off, 64);
      if (lane >= off) pre += u;
    }
    pre -= run;                                   // exclusive prefix of the lane totals
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * lane + e;
      if (i < a.Q) {
        Sw[i] = v[e] + pre;
        dtw[i] = (_Float16)d[e];
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  const float Send = Sw[a.Q - 1];
  const float dec_chunk = ex2(Send);

  // ---- per-step operands ---------------------------------------------------
  struct XB { h8 x[XPL]; h8 b[BK]; h8 c[BK]; };
  auto fetch = [&](XB& r, int j, bool with_c) {
    const unsigned tok = (unsigned)(t0 + j * TS);
#pragma unroll
    for (int k = 0; k < XPL; ++k) {
      const int c8 = lane + 64 * k, s = c8 / (PH / 8), pc = c8 % (PH / 8);
      r.x[k] = ldh<IO, 8>(rx, (tok + s) * xrow + (unsigned)(pc * 8) * ES);
    }
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      const int id = tid + NTH * k, s = id / NCH, nc = id % NCH;
      if (id < TS * NCH) {
        const unsigned off = (tok + s) * grow + (unsigned)(nc * 8) * ES;
        r.b[k] = ldh<IO, 8>(rb, off);
        if (with_c) r.c[k] = ldh<IO, 8>(rc, off);
      }
    }
  };
  // stage step j: B (and C) as read, x as read (phase 3 only) and x weighted
  // by dt_s e^{Sref - S_s} for the state contraction
  auto stage = [&](const XB& r, int j, float Sref, bool with_c) {
    const int i0 = j * TS;
#pragma unroll
    for (int k = 0; k < XPL; ++k) {
      const int c8 = lane + 64 * k, s = c8 / (PH / 8), pc = c8 % (PH / 8);
      const float w = (float)dtw[i0 + s] * ex2(Sref - Sw[i0 + s]);
      h8 xw;
#pragma unroll
      for (int e = 0; e < 8; ++e) xw[e] = (_Float16)((float)r.x[k][e] * w);
      *reinterpret_cast<h8*>(&xws[s * XP + pc * 8]) = xw;
      if (with_c) *reinterpret_cast<h8*>(&xs[s * XP + pc * 8]) = r.x[k];
    }
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      const int id = tid + NTH * k, s = id / NCH, nc = id % NCH;
      if (id < TS * NCH) {
        *reinterpret_cast<h8*>(&sm.b[s * NP + nc * 8]) = r.b[k];
        if (with_c) *reinterpret_cast<h8*>(&sm.c[s * NP + nc * 8]) = r.c[k];
      }
    }
  };
  // acc[nt][pt] += sum_s B[s, n] (w_s x[s, p]) over the staged step (K = 32 tokens)
  auto state_mfma = [&](f4 (&acc)[NT][PT]) {
    h8 xf[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      const int col = 16 * pt + 4 * (lr & 3);
      xf[pt] = cat(tr4(&xws[(8 * q + (lr >> 2)) * XP + col]), tr4(&xws[(8 * q + 4 + (lr >> 2)) * XP + col]));
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = ncol<N>(nt, lr & 3);
      const h8 af = cat(tr4(&sm.b[(8 * q + (lr >> 2)) * NP + col]), tr4(&sm.b[(8 * q + 4 + (lr >> 2)) * NP + col]));
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) acc[nt][pt] = mfma16(af, xf[pt], acc[nt][pt]);
    }
  };
  // 8 (or 4) n of row r of an LDS [s][n] tile at the n-slots of k-step m
  auto row8 = [&](const _Float16* tile, int r, int m) -> h8 {
    const _Float16* row = tile + r * NP;
    if constexpr (NV == 8) return *reinterpret_cast<const h8*>(row + (N / 4) * q + 8 * m);
    else {
      const h4 v = *reinterpret_cast<const h4*>(row + 4 * q);
      return h8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
    }
  };

  f4 acc[NT][PT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) acc[nt][pt] = f4{0.f, 0.f, 0.f, 0.f};

  // ---- phase 1: local chunk state ------------------------------------------
  XB xb;
  if (Jv > 0) fetch(xb, 0, false);
  for (int j = 0; j < Jv; ++j) {
    stage(xb, j, Send, false);
    lds_barrier();
    fetch(xb, j + 1 < Jv ? j + 1 : 0, j + 1 == Jv);   // the last fetch is the output phase's first step
    if (live) state_mfma(acc);
    lds_barrier();
  }

  // ---- phase 2: carry-in state over an indexed tree of chunks (radix r = 2^lg)
  // With i = c + 1 and block(i) = r^(number of trailing zero base-r digits of i),
  // chunk c publishes the aggregate of chunks (i - block(i), i] (1-based), and
  // its carry-in is the initial state advanced through the aggregates that
  // tile [1, i-1].  Those aggregates are taken newest first,
  // n_1 = i-1, n_{k+1} = n_k - block(n_k):
  //   carry = F(n_1) + D(n_1) F(n_2) + D(n_1) D(n_2) F(n_3) + ... + (prod D) h0
  // (F: aggregate state, D: its decay), so the aggregates that are ready first
  // are folded in first.  The first (r-1) log_r(block(i)) of them cover
  // (i - block(i), i-1]: once they are folded in, the running sum combined
  // with the local state is this chunk's own aggregate, published for later
  // chunks.  A chunk waits only on earlier chunks (claimed before it), and the
  // order of the sums is fixed, so results do not depend on timing.  A larger
  // radix means fewer dependent publishes (shorter latency chain) and more
  // aggregate loads (more traffic).
  // hand-off states: per item N*PH floats, tile-major, 16 contiguous bytes per lane
  constexpr unsigned kStBytes = (unsigned)(N * PH) * 4u;
  auto st_off = [&](int nt, int pt) -> unsigned { return (unsigned)((nt * PT + pt) * 256 + lane * 4) * 4u; };
  auto node_item = [&](int j) -> unsigned { return (unsigned)((j - 1) * BHV + bhv); };   // j: 1-based chunk

  f4 R[NT][PT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) R[nt][pt] = f4{0.f, 0.f, 0.f, 0.f};
  if (live) {
    const int i = c + 1;
    const bool last = c + 1 == a.nchunks;
    const int lg = a.tree_lg;                             // tree radix 2^lg
    const int t = ((1 << lg) - 1) * (__builtin_ctz((unsigned)i) / lg);   // aggregates inside this chunk's block
    float scale = 1.f;                                     // product of the decays folded in so far
    auto publish = [&]() {                                 // own aggregate: (dec_chunk R + local, dec_chunk scale)
      const rsrc_t r = mkr(a.agg + (size_t)item * (N * PH), kStBytes);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          f4 v = acc[nt][pt];
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = __builtin_fmaf(dec_chunk, R[nt][pt][k], v[k]);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, st_off(nt, pt), 0, kSc1);
        }
      if (lane == 0) __hip_atomic_store(&a.aggdec[item], __float_as_uint(dec_chunk * scale), __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      if (lane == 0) __hip_atomic_store(&a.flags[item], tag | 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // the aggregates to fold, newest first: lane k holds the k-th (1-based chunk)
    int nodes = 0, my_node = 0;
    for (int n = i - 1; n > 0; n -= 1 << (lg * (__builtin_ctz((unsigned)n) / lg)), ++nodes)
      if (lane == nodes) my_node = n;
    // wait until aggregates k0 .. k1-1 are published (one flag per lane, all
    // polled together), then read their decays
    float my_dec = 1.f;
    auto wait_group = [&](int k0, int k1) {
      const bool mine = lane >= k0 && lane < k1;
      const unsigned it = mine ? node_item(my_node) : 0u;
      unsigned spins = 0;
      while (true) {
        bool ready = true;
        if (mine) ready = __hip_atomic_load(&a.flags[it], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (tag | 1u);
        if (__ballot(!ready) == 0) break;
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
          if (lane == 0) __hip_atomic_fetch_or(&a.ctrl[kCtrlErr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
      if (mine) my_dec = __uint_as_float(__hip_atomic_load(&a.aggdec[it], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    };
    auto fold = [&](int k) {
      const int n = __builtin_amdgcn_readlane(my_node, k);
      const float Dn = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_dec), k));
      const rsrc_t r = mkr(a.agg + (size_t)node_item(n) * (N * PH), kStBytes);
      f4 F[NT][PT];                                        // all loads in flight at once
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
          F[nt][pt] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, st_off(nt, pt), 0, kSc1));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
          for (int e = 0; e < 4; ++e) R[nt][pt][e] = __builtin_fmaf(scale, F[nt][pt][e], R[nt][pt][e]);
      scale *= Dn;
    };
    // the first t aggregates are this chunk's block: fold them, publish, then the rest
    const int tb = t < nodes ? t : nodes;
    if (tb > 0) {
      wait_group(0, tb);
      for (int k = 0; k < tb; ++k) fold(k);
    }
    if (!last) publish();
    if (nodes > tb) {
      wait_group(tb, nodes);
      for (int k = tb; k < nodes; ++k) fold(k);
    }
    if (a.state_in) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          const int p = PH * half + 16 * pt + lr, n = ncol<N>(nt, q);
          const f4 h0 = *reinterpret_cast<const f4*>(a.state_in + ((size_t)hb * kP + p) * N + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) R[nt][pt][e] = __builtin_fmaf(scale, h0[e], R[nt][pt][e]);
        }
    }
    if (last && a.state_out) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          const int p = PH * half + 16 * pt + lr, n = ncol<N>(nt, q);
          f4 v = acc[nt][pt];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(dec_chunk, R[nt][pt][e], v[e]);
          *reinterpret_cast<f4*>(a.state_out + ((size_t)hb * kP + p) * N + n) = v;
        }
    }
  }

  // ---- phase 3: outputs ------------------------------------------------------
  rsrc_t rz = ry;
  if constexpr (NORM) rz = mkr(a.z + seq_x, xspan);
  for (int j = 0; j < Jv; ++j) {
    const int i0 = j * TS;
    const float Sj_start = j ? Sw[i0 - 1] : 0.f;
    const float Sj_end = Sw[i0 + TS - 1];
    stage(xb, j, Sj_end, true);
    lds_barrier();
    if (j + 1 < Jv) fetch(xb, j + 1, true);
    if (live) {
      // C fragments: rows t = 16T + lr, n-slots of k-step m
      h8 cf[2][KM];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int m = 0; m < KM; ++m) cf[T][m] = row8(sm.c, 16 * T + lr, m);
      // decay-masked C.B^T, rows s (4 per lane) x column t (one per lane), per t-tile
      h8 mf[2];
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        const int tl = 16 * T + lr;
        const float St = Sw[i0 + tl];
        f4 mb[2];
#pragma unroll
        for (int S = 0; S < 2; ++S) {
          mb[S] = f4{0.f, 0.f, 0.f, 0.f};
          if (S <= T) {
#pragma unroll
            for (int m = 0; m < KM; ++m) mb[S] = mfma16(row8(sm.b, 16 * S + lr, m), cf[T][m], mb[S]);
            const f4 Ss = *reinterpret_cast<const f4*>(&Sw[i0 + 16 * S + 4 * q]);
            const h4 ds = *reinterpret_cast<const h4*>(&dtw[i0 + 16 * S + 4 * q]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int si = 16 * S + 4 * q + i;
              mb[S][i] = si <= tl ? mb[S][i] * (float)ds[i] * ex2(St - Ss[i]) : 0.f;
            }
          }
        }
        mf[T] = h8{(_Float16)mb[0][0], (_Float16)mb[0][1], (_Float16)mb[0][2], (_Float16)mb[0][3],
                   (_Float16)mb[1][0], (_Float16)mb[1][1], (_Float16)mb[1][2], (_Float16)mb[1][3]};
      }
      float sc[2];
#pragma unroll
      for (int T = 0; T < 2; ++T) sc[T] = ex2(Sw[i0 + 16 * T + lr] - Sj_start);
      float gsq[2] = {0.f, 0.f};
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        // diagonal: sum_s x[s, p] M[s, t]; x rows s = 4q..4q+3 and 16+4q..16+4q+3
        const int col = 16 * pt + 4 * (lr & 3);
        const h8 xa = cat(tr4(&xs[(4 * q + (lr >> 2)) * XP + col]), tr4(&xs[(16 + 4 * q + (lr >> 2)) * XP + col]));
        // carry-in readout operand: the state rows p of this p-tile as binary16
        h8 ra[KM];
#pragma unroll
        for (int m = 0; m < KM; ++m) {
          const f4 r0 = R[N >= 32 ? 2 * m : 0][pt];
          const f4 r1 = N >= 32 ? R[N >= 32 ? 2 * m + 1 : 0][pt] : f4{0.f, 0.f, 0.f, 0.f};
          ra[m] = h8{(_Float16)r0[0], (_Float16)r0[1], (_Float16)r0[2], (_Float16)r0[3],
                     (_Float16)r1[0], (_Float16)r1[1], (_Float16)r1[2], (_Float16)r1[3]};
        }
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          const int tl = 16 * T + lr;
          const f4 yd = mfma16(xa, mf[T], f4{0.f, 0.f, 0.f, 0.f});
          f4 yr = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < KM; ++m) yr = mfma16(ra[m], cf[T][m], yr);
          const int p0 = 16 * pt + 4 * q;
          const h4 xr = *reinterpret_cast<const h4*>(&xs[tl * XP + p0]);
          const unsigned off = (unsigned)(t0 + i0 + tl) * xrow + (unsigned)p0 * ES;
          f4 out;
#pragma unroll
          for (int i = 0; i < 4; ++i) out[i] = __builtin_fmaf(sc[T], yr[i], yd[i]) + Dh * (float)xr[i];
          if constexpr (NORM) {
            const f4 zz = ld4f<IO>(rz, off);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              out[i] = out[i] * (zz[i] / (1.f + __expf(-zz[i])));
              gsq[T] += out[i] * out[i];
            }
          }
          st4<IO>(ry, off, out);
        }
      }
      if constexpr (NORM) {
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          float v = gsq[T];
          v += __shfl_xor(v, 16, 64);
          v += __shfl_xor(v, 32, 64);
          const int tl = 16 * T + lr;
          if (q == 0 && t0 + i0 + tl < len) {
            const size_t tok = (size_t)b * a.L + t0 + i0 + tl;
            a.normsum[(tok * a.H + h) * kNormParts + half] = v;
            if (half == 0) {
#pragma unroll
              for (int k = 2; k < kNormParts; ++k) a.normsum[(tok * a.H + h) * kNormParts + k] = 0.f;
            }
          }
        }
      }
      // running state for the next step: R <- e^{S_end_j - S_start_j} R + sum_s w_s B_s x_s
      if (j + 1 < Jv) {
        const float dec = ex2(Sj_end - Sj_start);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) R[nt][pt] *= dec;
        state_mfma(R);
      }
    }
    lds_barrier();
  }

  // ---- retire -------------------------------------------------------------------
  if (tid == 0) {
    const unsigned total = (unsigned)(a.nchunks * BG * nhb);
    const unsigned done = __hip_atomic_fetch_add(&a.ctrl[kCtrlDone], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == total - 1) {
      for (int k = 0; k < 8; ++k) __hip_atomic_store(&a.ctrl[k * kCtrlStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctrl[kCtrlDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctrl[kCtrlGen], gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    for (int k = 0; k < kNormParts * hpgr; ++k) s += normsum[((size_t)tok * H + gi * hpgr) * kNormParts + k];
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
  size_t ctrl, flags, aggdec, agg, incl, normsum, total;
};
static WsLayout ws_layout(const mamba2_dims& d) {
  const size_t nchunks = ((size_t)d.seqlen + d.chunk - 1) / d.chunk;
  const size_t items = nchunks * d.batch * d.nheads;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  WsLayout w;
  w.ctrl = 0;
  // flags and decays for up to two items per (chunk, sequence, head): the
  // plain-input scan splits each head into two independent halves
  w.flags = up(kCtrlBytes);
  w.aggdec = up(w.flags + 2 * items * 4);
  w.agg = up(w.aggdec + 2 * items * 4);
  const size_t sf = d.dstate == 128 ? Lay<128>::STATE_FLOATS : (d.dstate == 64 ? Lay<64>::STATE_FLOATS
                                                                                 : Lay<16>::STATE_FLOATS);
  w.incl = up(w.agg + items * sf * 4);
  w.normsum = up(w.incl + items * sf * 4);
  w.total = up(w.normsum + (d.norm_group > 0 ? (size_t)d.batch * d.seqlen * d.nheads * kNormParts * 4 : 0));
  return w;
}

size_t window_workspace_bytes(const mamba2_dims& d) { return ws_layout(d).total; }

// compute units of the current device (cached per device)
static int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev] = n;
  return n;
}

template <typename IO, int N, bool CONV, bool NORM>
static hipError_t launch_T(const WinArgs<IO>& a, hipStream_t st) {
  const unsigned items = (unsigned)(a.nchunks * a.B * a.H);
  if constexpr (CONV) ssd_window_kernel<IO, N, CONV, NORM><<<items, kThreads, 0, st>>>(a);
  else {
    const int hpg = a.H / a.G;
    const unsigned wgs = (unsigned)(a.nchunks * a.B * a.G * ((hpg + wv::KH - 1) / wv::KH));
    // When every workgroup is resident at once (one per CU), all chunks reach
    // the hand-off together and the chain of dependent publishes is the
    // critical path: a radix-8 tree.  Otherwise chunk levels are staggered in
    // time and aggregate traffic matters more: radix 4.
    WinArgs<IO> b = a;
    b.tree_lg = wgs <= (unsigned)device_cus() ? 3 : 2;
    ssd_window_group_kernel<IO, N, NORM><<<wgs, 64 * wv::NWV, 0, st>>>(b);
  }
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
  a.aggdec = (unsigned*)(base + wl.aggdec);
  a.agg = (float*)(base + wl.agg);
  a.incl = (float*)(base + wl.incl);
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

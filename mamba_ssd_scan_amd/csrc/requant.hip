// Whole window with the recurrent state requantized to binary16 after every
// token: the one-token step of the decode path, run token by token over a
// window with the state kept on chip.
//
// Page "Mamb2_8B_FP4_Recall_SQ3.25" scores each 2048-token window with the
// recurrent row requantized every token (section "Representation", paragraph
// "State"; reset per window, section "Measured quality").  Per token and head
// the step is the decode step's binary32 contract:
//   a  = (float) exp((double) dt * A_h)         (rounded once)
//   u  = dt * x_p,  v = u * B_n                 (one rounding each)
//   s  = fma(a, S, v)                           (binary32)
//   y_p = sum_n s C_n  (binary32 fma chain) + D_h x_p
//   S  <- binary16_rne(s)
// so the stored state after any number of tokens is reproducible bit for bit.
//
// The same kernel without the binary16 rounding (state kept in binary32) is
// the window scan for binary32 I/O: the recurrence itself, token by token,
// with every operand binary32 (a = (float) exp((double) dt A), s = fma(a, S,
// dt x B), y = sum_n s C_n + D x), so no input is rounded to binary16.
//
// Work split: a workgroup owns one (sequence, head, block of ROWS state rows
// p) for the whole window; each thread keeps RPT rows x 8 consecutive n of
// the state in registers (binary16 values held as binary32).  Tokens are
// staged 32 at a time into LDS (B and C rows, x of the block's rows, the
// decays), double-buffered so that the next block's loads are in flight while
// the current block runs; y of a block is gathered in LDS and stored as 64
// contiguous bytes per token.  The work is fp32 VALU-bound: per state element
// and token one multiply, two fmas and a binary16 rounding.
#include <type_traits>

#include "common.h"
#include "../../include/mamba2ssd.h"

namespace m2 {

template <int N> struct RqShape;
template <> struct RqShape<128> { static constexpr int ROWS = 16, RPT = 1, NTH = 256; };
template <> struct RqShape<64> { static constexpr int ROWS = 32, RPT = 1, NTH = 256; };
template <> struct RqShape<16> { static constexpr int ROWS = 64, RPT = 1, NTH = 128; };

constexpr int kRqTB = 32;   // tokens per staged block

// Sum over groups of W consecutive lanes (W = 2, 8 or 16), left in every lane
// of the group: cross-lane DPP moves inside a row (swap neighbours, swap
// pairs, mirror within 8, mirror within 16) instead of LDS permutes.
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  // old value 0 with bound control on: the compiler folds the move into the
  // add that consumes it (a single add with a DPP source)
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int W> __device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<0xB1>(v);
  if constexpr (W >= 4) v += dpp_f<0x4E>(v);
  if constexpr (W >= 8) v += dpp_f<0x141>(v);
  if constexpr (W >= 16) v += dpp_f<0x140>(v);
  return v;
}

// 8 consecutive elements in the I/O type (the B and C rows are staged in LDS
// as given, so that binary32 inputs stay exact)
template <typename IO> struct Raw8;
template <> struct Raw8<_Float16> {
  h8 v;
  __device__ __forceinline__ void load(const _Float16* p) { v = *reinterpret_cast<const h8*>(p); }
  __device__ __forceinline__ void put(_Float16* p) const { *reinterpret_cast<h8*>(p) = v; }
  static __device__ __forceinline__ void get(const _Float16* p, float* f) {
    const h8 h = *reinterpret_cast<const h8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
  }
};
template <> struct Raw8<float> {
  f4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f4*>(p);
    b = *reinterpret_cast<const f4*>(p + 4);
  }
  __device__ __forceinline__ void put(float* p) const {
    *reinterpret_cast<f4*>(p) = a;
    *reinterpret_cast<f4*>(p + 4) = b;
  }
  static __device__ __forceinline__ void get(const float* p, float* f) {
    const f4 x = *reinterpret_cast<const f4*>(p), y = *reinterpret_cast<const f4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = x[i];
      f[4 + i] = y[i];
    }
  }
};

// RQ: the state is requantized to binary16 after every token (the pages'
// scoring mode); otherwise it stays binary32, the exact token-sequential form
// that serves binary32-I/O windows (the recurrence evaluated directly, with
// no binary16 operand anywhere).  x, B and C rows are xld and gld elements
// apart; xpk: their rows follow the caller's (packed) rows like dt and y,
// else the padded row b * L + t of a conv output staged in the workspace.
template <typename IO, int N, bool RQ>
__global__ __launch_bounds__(RqShape<N>::NTH) void requant_window_kernel(
    const IO* __restrict__ x, const IO* __restrict__ dt, const IO* __restrict__ Bm, const IO* __restrict__ Cm,
    const float* __restrict__ A, const float* __restrict__ D, const float* __restrict__ state_in,
    float* __restrict__ state_out, const int* __restrict__ seqlens, const int* __restrict__ cu_seqlens,
    IO* __restrict__ y, int L, int T, int H, int G, int dt_sp, const float* __restrict__ dt_bias, long long dtld,
    long long xld, long long gld, int xpk) {
  constexpr int P = 64;
  constexpr int ROWS = RqShape<N>::ROWS, RPT = RqShape<N>::RPT, NTH = RqShape<N>::NTH;
  constexpr int LPR = N / 8;                 // lanes per state row
  static_assert(ROWS == (NTH / LPR) * RPT, "rows per workgroup");
  constexpr int NBLK = P / ROWS;
  __shared__ alignas(16) IO sB[2][kRqTB][N];
  __shared__ alignas(16) IO sC[2][kRqTB][N];
  __shared__ alignas(16) float sX[2][kRqTB][ROWS];
  __shared__ alignas(16) float sA[2][kRqTB];
  __shared__ alignas(16) float sD[2][kRqTB];
  __shared__ float sY[kRqTB][ROWS];

  const int tid = threadIdx.x;
  const int blk = blockIdx.x % NBLK;
  const int bh = blockIdx.x / NBLK;
  const int b = bh / H, h = bh - b * H;
  const int g = h / (H / G);
  const int nc = (tid % LPR) * 8;            // first n of this thread
  const int r0 = tid / LPR;                  // first of its rows (stride NTH / LPR)
  constexpr int RSTRIDE = NTH / LPR;
  const int p0 = blk * ROWS;
  const SeqRows span = seq_rows(seqlens, cu_seqlens, b, L, T);
  const int len = span.len;
  const float Ah = A[h], Dh = D[h];
  const float dtb = dt_sp && dt_bias ? dt_bias[h] : 0.f;

  // state: binary16 in registers (the mixed-precision fmas read it directly),
  // or binary32 for the exact form
  using st_t = typename std::conditional<RQ, _Float16, float>::type;
  st_t S[RPT][8];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int p = p0 + r0 + k * RSTRIDE;
#pragma unroll
    for (int i = 0; i < 8; ++i) S[k][i] = (st_t)0.f;
    if (state_in) {
      float v[8];
      io<float>::load8(state_in + (((size_t)bh * P + p) * N + nc), v);
#pragma unroll
      for (int i = 0; i < 8; ++i) S[k][i] = (st_t)v[i];
    }
  }

  // ---- staging of one 32-token block --------------------------------------
  // B and C: NTH threads x 16 bytes cover kRqTB * N halfs per matrix when N
  // is 128; the loops below stride by NTH for the smaller N.
  constexpr int BC8 = kRqTB * N / 8;         // 8-element chunks per matrix
  constexpr int XC = kRqTB * ROWS;           // x elements per block
  struct Pre {
    Raw8<IO> b[(BC8 + NTH - 1) / NTH], c[(BC8 + NTH - 1) / NTH];
    float xv[(XC + NTH - 1) / NTH];
    float d;
  };
  const size_t seqtok = (size_t)span.base;   // the sequence's first row
  const size_t xtok = xpk ? seqtok : (size_t)b * L;   // its first row of x, B and C
  auto fetch = [&](Pre& r, int t0) {
#pragma unroll
    for (int k = 0; k < (BC8 + NTH - 1) / NTH; ++k) {
      const int id = tid + k * NTH;
      if (id < BC8) {
        const int t = id / (N / 8), c8 = id % (N / 8);
        const int tt = min(t0 + t, len - 1);
        const size_t off = (xtok + tt) * (size_t)gld + (size_t)g * N + c8 * 8;
        r.b[k].load(Bm + off);
        r.c[k].load(Cm + off);
      }
    }
#pragma unroll
    for (int k = 0; k < (XC + NTH - 1) / NTH; ++k) {
      const int id = tid + k * NTH;
      if (id < XC) {
        const int t = id / ROWS, rr = id % ROWS;
        const int tt = min(t0 + t, len - 1);
        r.xv[k] = io<IO>::load1(x + (xtok + tt) * (size_t)xld + (size_t)h * P + p0 + rr);
      }
    }
    r.d = 0.f;
    if (tid < kRqTB) {
      const int tt = min(t0 + tid, len - 1);
      r.d = io<IO>::load1(dt + (seqtok + tt) * dtld + h);
      if (dt_sp) r.d = dt_softplus(r.d, dtb);
    }
  };
  auto stage = [&](const Pre& r, int buf) {
#pragma unroll
    for (int k = 0; k < (BC8 + NTH - 1) / NTH; ++k) {
      const int id = tid + k * NTH;
      if (id < BC8) {
        const int t = id / (N / 8), c8 = id % (N / 8);
        r.b[k].put(&sB[buf][t][c8 * 8]);
        r.c[k].put(&sC[buf][t][c8 * 8]);
      }
    }
#pragma unroll
    for (int k = 0; k < (XC + NTH - 1) / NTH; ++k) {
      const int id = tid + k * NTH;
      if (id < XC) sX[buf][id / ROWS][id % ROWS] = r.xv[k];
    }
    if (tid < kRqTB) {
      sD[buf][tid] = r.d;
      sA[buf][tid] = (float)exp((double)r.d * (double)Ah);   // the decay, rounded once from double
    }
  };
  // y of a block: gathered in LDS, then 4 bytes (f16 pairs) or 8 per thread
  auto store_y = [&](int t0, int nt) {
    constexpr int PAIRS = kRqTB * ROWS / 2;
    for (int id = tid; id < PAIRS; id += NTH) {
      const int t = id / (ROWS / 2), c2 = (id % (ROWS / 2)) * 2;
      if (t < nt) {
        IO* dst = y + ((seqtok + t0 + t) * H + h) * P + p0 + c2;
        io<IO>::store1(dst, sY[t][c2]);
        io<IO>::store1(dst + 1, sY[t][c2 + 1]);
      }
    }
  };

  const int nblocks = (len + kRqTB - 1) / kRqTB;
  Pre pre;
  if (nblocks > 0) {
    fetch(pre, 0);
    stage(pre, 0);
  }
  __syncthreads();
  for (int kb = 0; kb < nblocks; ++kb) {
    const int buf = kb & 1;
    const int t0 = kb * kRqTB;
    const int nt = min(kRqTB, len - t0);
    if (kb + 1 < nblocks) fetch(pre, t0 + kRqTB);   // next block in flight
    // one token: the state update of this thread's rows and y of each row
    // (every lane of a row ends with the row's sum and writes the same value)
    // -0 as an opaque register value: fma(u, B, -0) is exactly u * B, and
    // kept as an fma it takes a binary16 B without a separate conversion
    float mzero = -0.f;
    asm volatile("" : "+v"(mzero));
    auto token = [&](int t, float d, float a, const float (&bv)[8], const float (&cv)[8], const float (&xr)[RPT]) {
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        float acc = 0.f;
        {
#pragma clang fp contract(off)
          const float u = d * xr[k];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float v = __builtin_fmaf(u, bv[i], mzero);   // exactly u * B
            float sn = __builtin_fmaf(a, (float)S[k][i], v);
            acc = __builtin_fmaf(sn, cv[i], acc);
            if constexpr (RQ) {
              // binary32 first, then binary16 (the empty asm keeps the two
              // roundings apart: a fused fma-to-binary16 would round once)
              asm volatile("" : "+v"(sn));
            }
            S[k][i] = (st_t)sn;
          }
        }
        acc = row_sum<LPR>(acc);
        sY[t][r0 + k * RSTRIDE] = acc + Dh * xr[k];
      }
    };
    auto operands = [&](int t, float (&bv)[8], float (&cv)[8], float (&xr)[RPT]) {
      Raw8<IO>::get(&sB[buf][t][nc], bv);
      Raw8<IO>::get(&sC[buf][t][nc], cv);
#pragma unroll
      for (int k = 0; k < RPT; ++k) xr[k] = sX[buf][t][r0 + k * RSTRIDE];
    };
    // four tokens at a time: all their LDS operands are read before the
    // first update, so the reads' latency is paid once per four tokens
    int t = 0;
    for (; t + 4 <= nt; t += 4) {
      const f4 dq = *reinterpret_cast<const f4*>(&sD[buf][t]);
      const f4 aq = *reinterpret_cast<const f4*>(&sA[buf][t]);
      float bv[4][8], cv[4][8], xr[4][RPT];
#pragma unroll
      for (int u = 0; u < 4; ++u) operands(t + u, bv[u], cv[u], xr[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) token(t + u, dq[u], aq[u], bv[u], cv[u], xr[u]);
    }
    for (; t < nt; ++t) {
      float bv[8], cv[8], xr[RPT];
      operands(t, bv, cv, xr);
      token(t, sD[buf][t], sA[buf][t], bv, cv, xr);
    }
    __syncthreads();                           // sY complete; buffer buf free
    store_y(t0, nt);
    if (kb + 1 < nblocks) stage(pre, buf ^ 1);
    __syncthreads();
  }

  if (state_out) {
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int p = p0 + r0 + k * RSTRIDE;
      float* dst = state_out + (((size_t)bh * P + p) * N + nc);
      *reinterpret_cast<f4*>(dst) = f4{(float)S[k][0], (float)S[k][1], (float)S[k][2], (float)S[k][3]};
      *reinterpret_cast<f4*>(dst + 4) = f4{(float)S[k][4], (float)S[k][5], (float)S[k][6], (float)S[k][7]};
    }
  }
}

template <typename IO, int N, bool RQ>
static hipError_t launch_rq(const mamba2_dims& d, const mamba2_window_io& io_, const IO* x, const IO* Bm,
                            const IO* Cm, long long xld, long long gld, int xpk, hipStream_t st) {
  constexpr int ROWS = RqShape<N>::ROWS, NTH = RqShape<N>::NTH;
  const unsigned grid = (unsigned)(d.batch * d.nheads * (64 / ROWS));
  requant_window_kernel<IO, N, RQ><<<grid, NTH, 0, st>>>(
      x, (const IO*)io_.dt, Bm, Cm, io_.A, io_.D, io_.state_in, io_.state_out, io_.seqlens, io_.cu_seqlens,
      (IO*)io_.y, d.seqlen, d.packed_tokens, d.nheads, d.ngroups, d.dt_softplus,
      d.dt_softplus ? io_.dt_bias : nullptr, io_.dt_ld > 0 ? (long long)io_.dt_ld : (long long)d.nheads, xld, gld,
      xpk);
  return hipGetLastError();
}

template <typename IO, bool RQ>
static hipError_t launch_rq_N(const mamba2_dims& d, const mamba2_window_io& io_, const IO* x, const IO* Bm,
                              const IO* Cm, long long xld, long long gld, int xpk, hipStream_t st) {
  switch (d.dstate) {
    case 16: return launch_rq<IO, 16, RQ>(d, io_, x, Bm, Cm, xld, gld, xpk, st);
    case 64: return launch_rq<IO, 64, RQ>(d, io_, x, Bm, Cm, xld, gld, xpk, st);
    default: return launch_rq<IO, 128, RQ>(d, io_, x, Bm, Cm, xld, gld, xpk, st);
  }
}

hipError_t launch_requant_window(const mamba2_dims& d, const mamba2_window_io& io_, hipStream_t st) {
  const long long xld = (long long)d.nheads * 64, gld = (long long)d.ngroups * d.dstate;
  if (d.io_dtype == MAMBA2_F16)
    return launch_rq_N<_Float16, true>(d, io_, (const _Float16*)io_.x, (const _Float16*)io_.B,
                                       (const _Float16*)io_.C, xld, gld, 1, st);
  return launch_rq_N<float, true>(d, io_, (const float*)io_.x, (const float*)io_.B, (const float*)io_.C, xld, gld, 1,
                                  st);
}

// The exact binary32 window scan (binary32 I/O): x, B, C are the caller's
// rows (xpk = 1) or the conv output staged in the workspace (xpk = 0, rows of
// xld = gld = conv_dim elements).
hipError_t launch_exact_window_f32(const mamba2_dims& d, const mamba2_window_io& io_, const float* x, const float* Bm,
                                   const float* Cm, long long xld, long long gld, int xpk, hipStream_t st) {
  return launch_rq_N<float, false>(d, io_, x, Bm, Cm, xld, gld, xpk, st);
}

}  // namespace m2

// Gradients of the selective state-space scan (the backward pass of the
// window scan), for training through the frozen mixer core (page
// "Mamb2_8B_FP4_Recall_SQ3.25" trains an adapter through the frozen stack).
//
// Per (sequence b, head h), with S_t the running log decay (S_t = A sum_{s<=t}
// dt_s), u_t = dt_t x_t (outer) B_t, h_t = exp(dt_t A) h_{t-1} + u_t,
// y_t = h_t . C_t + D x_t, and the loss's output gradients dy_t and dhT:
//   gh_t  = C_t (outer) dy_t + exp(dt_{t+1} A) gh_{t+1},  gh_len = C (x) dy + dhT
//           (the gradient with respect to h_t),
//   v_t   = gh_t . B_t  (a P-vector),  q_t = x_t . v_t,
//   dx_t  = D dy_t + dt_t v_t,   dB_t += dt_t gh_t^T x_t,   dC_t += h_t^T dy_t,
//   e_t   = dy_t . (h_t . C_t),  eT = <dhT, h_len>,
//   dL/dS_t = e_t + [t = last] eT - dt_t q_t,   R_t = sum_{t' >= t} dL/dS_t',
//   ddt_t = q_t + A R_t,   dA += dt_t R_t,   dD += dy_t . x_t,   dh0 = gradient
//   with respect to h_0.
// This form needs h_t only together with dy_t (a forward sweep: dC and e)
// and gh_t only together with x_t, B_t (a reverse sweep), never h_{t-1}
// beside gh_t, so neither sweep keeps or recomputes past states.  R is summed
// in double: it is a running sum over the whole window of terms that largely
// cancel.
//
// Work split: each sweep is one 256-thread workgroup per (sequence, head);
// a thread owns 8 consecutive n of KR rows p (the decode kernel's layout), so
// sums over n stay inside a wave and sums over p go through LDS once per
// block of kGTB tokens.  The per-head dB and dC, and the per-sequence dA, dD
// and dt-bias gradients, go to the workspace; a last kernel sums the heads of
// each group and the sequences of the batch in a fixed order.
#include "common.h"
#include "../../include/mamba2ssd.h"

namespace m2 {

constexpr int kGP = 64;        // head dim

template <typename IO> struct GradArgs {
  const IO* x;
  const IO* dt;
  const IO* Bm;
  const IO* Cm;
  const IO* dy;
  const float* A;
  const float* D;
  const float* dt_bias;
  const float* h0;         // (B,H,P,N) or null
  const float* dhT;        // (B,H,P,N) or null
  const int* seqlens;
  int dt_sp;
  int B, L, H, G;
  float* dx;               // (B,L,H,P)
  float* ddt;              // (B,L,H)
  float* dB;               // (B,L,G,N)
  float* dC;               // (B,L,G,N)
  float* dA;               // (H)
  float* dD;               // (H)
  float* dh0;              // (B,H,P,N) or null
  float* dbias;            // (H) or null
  // workspace
  float* dBh;              // (B,L,H,N) per-head dB
  float* dCh;              // (B,L,H,N) per-head dC
  float* e;                // (B,L,H) dy_t . (h_t . C_t)
  float* q;                // (B,L,H) x_t . (gh_t . B_t)
  float* eT;               // (B,H) <dhT, h_len>
  float* dAp;              // (B,H) per-sequence dA
  float* dDp;              // (B,H) per-sequence dD
  float* dbp;              // (B,H) per-sequence dt-bias gradient
};

template <typename IO> __device__ __forceinline__ float ldf(const IO* p) { return (float)*p; }

// Thread layout of a sweep: a thread owns 8 consecutive n (LPR lanes per row)
// of KR rows p = r0 + k * RPP.  N = 128 takes 512 threads with two rows each;
// the smaller N one row per thread.
template <int N> struct GradShape {
  static constexpr int LPR = N / 8;
  static constexpr int NTH = N == 128 ? 512 : 64 * LPR;
  static constexpr int RPP = NTH / LPR;
  static constexpr int KR = kGP / RPP;
  static constexpr int NW = NTH / 64;
  static constexpr int TB = N == 16 ? 16 : 4;    // tokens staged per block
  static_assert(KR * RPP == kGP, "rows");
};

template <int N> struct alignas(16) GradSmem {
  static constexpr int TB = GradShape<N>::TB, NW = GradShape<N>::NW;
  float x[2][TB][kGP];       // two staging buffers: the next block lands while this one is used
  float dy[2][TB][kGP];
  float b[2][TB][N];
  float c[2][TB][N];
  float dt[2][TB];
  float col[TB][GradShape<N>::RPP][N];   // per-thread partial sums over its rows (dC or dB)
  float rv[TB][kGP];        // per-row sums over n: (h_t . C_t)[p] or v_t[p]
  float red[2][16];
};

// One block of up to TB tokens: loaded into registers (zeros past nt) while
// the previous block is computed, then written to a staging buffer.
template <typename IO, int N> struct GradPre {
  static constexpr int TB = GradShape<N>::TB, NTH = GradShape<N>::NTH;
  static constexpr int PX = (TB * kGP + NTH - 1) / NTH, PB = (TB * N + NTH - 1) / NTH;
  IO x[PX], dy[PX], b[PB], c[PB];
  IO d;

  __device__ __forceinline__ void fetch(const GradArgs<IO>& a, int b_, int h, int g, int t0, int nt, int tid) {
#pragma unroll
    for (int k = 0; k < PX; ++k) {
      const int id = tid + k * NTH, j = id / kGP, p = id % kGP;
      const bool ok = id < TB * kGP && j < nt;
      const size_t row = ((size_t)b_ * a.L + t0 + j) * a.H + h;
      x[k] = ok ? a.x[row * kGP + p] : (IO)0;
      dy[k] = ok ? a.dy[row * kGP + p] : (IO)0;
    }
#pragma unroll
    for (int k = 0; k < PB; ++k) {
      const int id = tid + k * NTH, j = id / N, n = id % N;
      const bool ok = id < TB * N && j < nt;
      const size_t row = ((size_t)b_ * a.L + t0 + j) * a.G + g;
      b[k] = ok ? a.Bm[row * N + n] : (IO)0;
      c[k] = ok ? a.Cm[row * N + n] : (IO)0;
    }
    d = tid < nt ? a.dt[((size_t)b_ * a.L + t0 + tid) * a.H + h] : (IO)0;
  }
  __device__ __forceinline__ void put(GradSmem<N>& st, int buf, const GradArgs<IO>& a, int h, int nt, int tid) const {
#pragma unroll
    for (int k = 0; k < PX; ++k) {
      const int id = tid + k * NTH;
      if (id < TB * kGP) {
        st.x[buf][id / kGP][id % kGP] = (float)x[k];
        st.dy[buf][id / kGP][id % kGP] = (float)dy[k];
      }
    }
#pragma unroll
    for (int k = 0; k < PB; ++k) {
      const int id = tid + k * NTH;
      if (id < TB * N) {
        st.b[buf][id / N][id % N] = (float)b[k];
        st.c[buf][id / N][id % N] = (float)c[k];
      }
    }
    if (tid < TB) {
      float v = (float)d;
      if (a.dt_sp && tid < nt) v = dt_softplus(v, a.dt_bias ? a.dt_bias[h] : 0.f);
      st.dt[buf][tid] = v;
    }
  }
};

// Sum over the W lanes of a row (W <= 16, rows aligned to W): every lane of the
// row ends with the row's sum (DPP quad permutes, then half-row and row
// mirrors).
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  // old value 0 with bound control on: lets the compiler fold the move into
  // the add that consumes it (a single add with a DPP source)
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int W> __device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<0xB1>(v);
  if constexpr (W >= 4) v += dpp_f<0x4E>(v);
  if constexpr (W >= 8) v += dpp_f<0x141>(v);
  if constexpr (W >= 16) v += dpp_f<0x140>(v);
  return v;
}
// DPP rotation inside each 16-lane row: lane i receives lane (i + R) mod 16.
template <int R> __device__ __forceinline__ float row_ror(float v) { return dpp_f<0x120 + R>(v); }
// Sum over the row groups of a wave (lanes with the same lane % W), valid in
// lanes 0 .. 15: rotations by W, 2W, .. 8 inside each row, then the rows are
// paired with the lane-swap instructions (rows 1 and 3 onto rows 0 and 2, then
// lanes 32-63 onto lanes 0-31), all in the vector ALU.
template <int W> __device__ __forceinline__ float col_sum(float v) {
  if constexpr (W <= 8) v += row_ror<8>(v);
  if constexpr (W <= 4) v += row_ror<4>(v);
  if constexpr (W <= 2) v += row_ror<2>(v);
  // v_permlane16_swap a, b: odd rows of a <-> even rows of b; afterwards b's
  // even rows hold v's odd rows.  v_permlane32_swap a, b: lanes 32-63 of a <->
  // lanes 0-31 of b.  (Written out so that both operands are distinct
  // registers; the wait states cover the VALU writes before and after.)
  float a0 = v, b0 = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a0), "+v"(b0));
  v += b0;
  float a1 = v, b1 = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a1), "+v"(b1));
  v += b1;
  return v;
}
// Sum over the 64 lanes of a wave, valid in lanes 0 .. 15 (DPP inside rows,
// then the lane-swap steps across rows).
__device__ __forceinline__ float wave_sum(float v) { return col_sum<16>(row_sum<16>(v)); }

// ---- the two sweeps, one launch: workgroups [0, B*H) run the forward sweep
// (h_t, dC per head, e_t, eT), workgroups [B*H, 2*B*H) the reverse sweep (gh_t,
// dx, dB per head, q_t, dD, dh0).  They share nothing, so they run side by side.
template <typename IO, int N, bool rev>
__device__ __forceinline__ void grad_sweep(const GradArgs<IO>& a, GradSmem<N>& st, int bh) {
  using S = GradShape<N>;
  constexpr int LPR = S::LPR, RPP = S::RPP, KR = S::KR, NW = S::NW, TB = S::TB;
  const int b = bh / a.H, h = bh - b * a.H, g = h / (a.H / a.G);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nc = (tid % LPR) * 8, r0 = tid / LPR;
  int len = a.seqlens ? a.seqlens[b] : a.L;
  len = len < 0 ? 0 : (len > a.L ? a.L : len);
  const float Ah = a.A[h], Dh = a.D[h];

  // h (forward) or gh (reverse), in registers
  float sv[KR][8];
  const float* init = rev ? a.dhT : a.h0;
#pragma unroll
  for (int k = 0; k < KR; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[k][i] = init ? init[((size_t)bh * kGP + r0 + k * RPP) * N + nc + i] : 0.f;
  float dDacc = 0.f;

  const int nblk = (len + TB - 1) / TB;
  auto block_of = [&](int kk) { return rev ? nblk - 1 - kk : kk; };
  GradPre<IO, N> pre;
  if (nblk > 0) {
    const int t00 = block_of(0) * TB;
    pre.fetch(a, b, h, g, t00, min(TB, len - t00), tid);
    pre.put(st, 0, a, h, min(TB, len - t00), tid);
  }
  __syncthreads();
  for (int kk = 0; kk < nblk; ++kk) {
    const int cur = kk & 1;
    const int t0 = block_of(kk) * TB;
    const int nt = min(TB, len - t0);
    int tn = 0, ntn = 0;
    if (kk + 1 < nblk) {           // the next block's loads, in flight during this block
      tn = block_of(kk + 1) * TB;
      ntn = min(TB, len - tn);
      pre.fetch(a, b, h, g, tn, ntn, tid);
    }
    for (int jj = 0; jj < nt; ++jj) {
      const int j = rev ? nt - 1 - jj : jj;
      const float d = st.dt[cur][j];
      const float dec = __expf(d * Ah);
      float bv[8], cv[8], cs[8];
      {
        const f4 b0 = *reinterpret_cast<const f4*>(&st.b[cur][j][nc]), b1 = *reinterpret_cast<const f4*>(&st.b[cur][j][nc + 4]);
        const f4 c0 = *reinterpret_cast<const f4*>(&st.c[cur][j][nc]), c1 = *reinterpret_cast<const f4*>(&st.c[cur][j][nc + 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bv[i] = b0[i];
          bv[4 + i] = b1[i];
          cv[i] = c0[i];
          cv[4 + i] = c1[i];
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) cs[i] = 0.f;
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        const int p = r0 + k * RPP;
        const float xp = st.x[cur][j][p];
        const float dyp = st.dy[cur][j][p];
        float r = 0.f;
        if constexpr (!rev) {
          const float u = d * xp;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            sv[k][i] = __builtin_fmaf(dec, sv[k][i], u * bv[i]);   // h_t
            r = __builtin_fmaf(sv[k][i], cv[i], r);                // (h_t . C_t)[p]
            cs[i] = __builtin_fmaf(dyp, sv[k][i], cs[i]);          // dC partial
          }
          r = row_sum<LPR>(r);
          if ((tid % LPR) == 0) st.rv[j][p] = r;
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            sv[k][i] = __builtin_fmaf(cv[i], dyp, sv[k][i]);       // gradient with respect to h_t
            r = __builtin_fmaf(sv[k][i], bv[i], r);                // v_t[p]
            cs[i] = __builtin_fmaf(xp, sv[k][i], cs[i]);           // dB partial (before dt)
          }
          r = row_sum<LPR>(r);
          if ((tid % LPR) == 0) st.rv[j][p] = r;
#pragma unroll
          for (int i = 0; i < 8; ++i) sv[k][i] *= dec;             // ... and with respect to h_{t-1}
        }
      }
      // this thread's partial over its rows; the sum over the row groups is
      // taken once per block
      *reinterpret_cast<f4*>(&st.col[j][r0][nc]) = f4{cs[0], cs[1], cs[2], cs[3]};
      *reinterpret_cast<f4*>(&st.col[j][r0][nc + 4]) = f4{cs[4], cs[5], cs[6], cs[7]};
    }
    __syncthreads();
    if (kk + 1 < nblk) pre.put(st, cur ^ 1, a, h, ntn, tid);
    // the block's outputs: sums over the row groups in a fixed order
    float* colout = rev ? a.dBh : a.dCh;
    for (int id = tid; id < nt * N; id += S::NTH) {
      const int j = id / N, n = id % N;
      float v = 0.f;
#pragma unroll 8
      for (int r = 0; r < RPP; ++r) v += st.col[j][r][n];
      colout[(((size_t)b * a.L + t0 + j) * a.H + h) * N + n] = rev ? st.dt[cur][j] * v : v;
    }
    // per token (one wave each, lane = row p): e_t = dy . (h . C), or
    // dx = D dy + dt v, q_t = x . v and the token's share of dD
    for (int j = wv; j < nt; j += NW) {
      const float r = st.rv[j][lane], dyp = st.dy[cur][j][lane], xp = st.x[cur][j][lane];
      const size_t ti = ((size_t)b * a.L + t0 + j) * a.H + h;
      if constexpr (!rev) {
        const float ev = wave_sum(dyp * r);
        if (lane == 0) a.e[ti] = ev;
      } else {
        a.dx[ti * kGP + lane] = __builtin_fmaf(st.dt[cur][j], r, Dh * dyp);
        const float qv = wave_sum(xp * r);
        if (lane == 0) a.q[ti] = qv;
        dDacc = __builtin_fmaf(dyp, xp, dDacc);
      }
    }
    __syncthreads();
  }

  if constexpr (!rev) {
    // eT = <dhT, h_len>
    float et = 0.f;
    if (a.dhT) {
#pragma unroll
      for (int k = 0; k < KR; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          et = __builtin_fmaf(a.dhT[((size_t)bh * kGP + r0 + k * RPP) * N + nc + i], sv[k][i], et);
    }
    et = wave_sum(et);
    if (lane == 0) st.red[0][wv] = et;
    __syncthreads();
    if (tid == 0) {
      float v = 0.f;
      for (int w = 0; w < NW; ++w) v += st.red[0][w];
      a.eT[bh] = v;
    }
    return;
  } else {
  // reverse: rows past the length get zero gradients; dh0; dD
  for (int id = tid; id < (a.L - len) * kGP; id += S::NTH) {
    const int t = len + id / kGP, p = id % kGP;
    a.dx[(((size_t)b * a.L + t) * a.H + h) * kGP + p] = 0.f;
  }
  if (a.dh0) {
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      float* dst = a.dh0 + ((size_t)bh * kGP + r0 + k * RPP) * N + nc;
      *reinterpret_cast<f4*>(dst) = f4{sv[k][0], sv[k][1], sv[k][2], sv[k][3]};
      *reinterpret_cast<f4*>(dst + 4) = f4{sv[k][4], sv[k][5], sv[k][6], sv[k][7]};
    }
  }
  dDacc = wave_sum(dDacc);
  if (lane == 0) st.red[1][wv] = dDacc;
  __syncthreads();
  if (tid == 0) {
    float v = 0.f;
    for (int w = 0; w < NW; ++w) v += st.red[1][w];
    a.dDp[bh] = v;
  }
  }
}

template <typename IO, int N>
__global__ __launch_bounds__(GradShape<N>::NTH) void grad_sweep_kernel(const GradArgs<IO> a) {
  __shared__ GradSmem<N> st;
  const int BH = a.B * a.H;
  if ((int)blockIdx.x >= BH) grad_sweep<IO, N, true>(a, st, (int)blockIdx.x - BH);
  else grad_sweep<IO, N, false>(a, st, (int)blockIdx.x);
}

// ---- the dt chain: R_t = sum_{t' >= t} dL/dS_t' with dL/dS_t = e_t + [t = last]
// eT - dt_t q_t, then ddt_t = q_t + A R_t (times sp'(raw + bias) for a raw dt),
// dA += dt_t R_t.  One 256-thread block per (sequence, head): each thread takes
// a run of consecutive tokens, the runs' totals are suffix-summed across the
// block, all in double.
constexpr int kChainT = 256;
template <typename IO>
__global__ __launch_bounds__(kChainT) void grad_chain_kernel(const GradArgs<IO> a) {
  __shared__ double tot[kChainT];
  __shared__ double red[2][kChainT];
  const int bh = blockIdx.x, b = bh / a.H, h = bh - b * a.H;
  const int tid = threadIdx.x;
  int len = a.seqlens ? a.seqlens[b] : a.L;
  len = len < 0 ? 0 : (len > a.L ? a.L : len);
  const int per = (len + kChainT - 1) / kChainT;
  const int ta = min(tid * per, len), tb = min(ta + per, len);
  const double Ah = (double)a.A[h];
  const double eT = (double)a.eT[bh];
  const float bias = a.dt_sp && a.dt_bias ? a.dt_bias[h] : 0.f;
  auto dt_eff = [&](size_t ti) {
    const float d = ldf(a.dt + ti);
    return (double)(a.dt_sp ? dt_softplus(d, bias) : d);
  };
  auto dS = [&](int t) {
    const size_t ti = ((size_t)b * a.L + t) * a.H + h;
    return (double)a.e[ti] + (t == len - 1 ? eT : 0.0) - dt_eff(ti) * (double)a.q[ti];
  };
  double run = 0.0;
  for (int t = tb - 1; t >= ta; --t) run += dS(t);
  tot[tid] = run;
  __syncthreads();
  // suffix sums of the run totals (Hillis-Steele over the block)
  for (int off = 1; off < kChainT; off <<= 1) {
    const double v = tid + off < kChainT ? tot[tid + off] : 0.0;
    __syncthreads();
    tot[tid] += v;
    __syncthreads();
  }
  double R = tid + 1 < kChainT ? tot[tid + 1] : 0.0;   // everything after this run
  double dA_acc = 0.0, db_acc = 0.0;
  for (int t = tb - 1; t >= ta; --t) {
    const size_t ti = ((size_t)b * a.L + t) * a.H + h;
    R += dS(t);
    const double dte = dt_eff(ti);
    const double gdt = (double)a.q[ti] + Ah * R;
    dA_acc += dte * R;
    double graw = gdt;
    if (a.dt_sp) {
      const double v = (double)ldf(a.dt + ti) + (double)bias;
      graw = gdt * (v > 20.0 ? 1.0 : 1.0 / (1.0 + exp(-v)));
      db_acc += graw;
    }
    a.ddt[ti] = (float)graw;
  }
  for (int t = len + tid; t < a.L; t += kChainT) a.ddt[((size_t)b * a.L + t) * a.H + h] = 0.f;
  red[0][tid] = dA_acc;
  red[1][tid] = db_acc;
  __syncthreads();
  for (int off = kChainT / 2; off > 0; off >>= 1) {
    if (tid < off) {
      red[0][tid] += red[0][tid + off];
      red[1][tid] += red[1][tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.dAp[bh] = (float)red[0][0];
    a.dbp[bh] = (float)red[1][0];
  }
}

// ---- sums over the heads of each group and over the batch --------------------
// dB, dC: one thread per (b, t, g, n), heads of the group in index order (rows
// past a sequence's length are zero); dA, dD, dt-bias: one thread per head,
// sequences in index order.
template <int N>
__global__ __launch_bounds__(256) void grad_reduce_kernel(const GradArgs<float> a) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)a.B * a.L * a.G * N;
  const int hpg = a.H / a.G;
  if (idx < total) {
    const int n = (int)(idx % N);
    const long long r = idx / N;
    const int g = (int)(r % a.G);
    const long long bt = r / a.G;
    const int b = (int)(bt / a.L), t = (int)(bt % a.L);
    int len = a.seqlens ? a.seqlens[b] : a.L;
    len = len < 0 ? 0 : (len > a.L ? a.L : len);
    float sb = 0.f, sc = 0.f;
    if (t < len) {
      for (int k = 0; k < hpg; ++k) {
        const size_t src = (((size_t)bt * a.H) + g * hpg + k) * N + n;
        sb += a.dBh[src];
        sc += a.dCh[src];
      }
    }
    a.dB[idx] = sb;
    a.dC[idx] = sc;
  }
  if (blockIdx.x == 0) {
    for (int h = threadIdx.x; h < a.H; h += 256) {
      float sa = 0.f, sd = 0.f, sbias = 0.f;
      for (int b = 0; b < a.B; ++b) {
        sa += a.dAp[(size_t)b * a.H + h];
        sd += a.dDp[(size_t)b * a.H + h];
        sbias += a.dbp[(size_t)b * a.H + h];
      }
      a.dA[h] = sa;
      a.dD[h] = sd;
      if (a.dbias) a.dbias[h] = sbias;
    }
  }
}

// ---------------------------------------------------------------------------
struct GradWs {
  size_t dBh, dCh, e, q, eT, dAp, dDp, dbp, total;
};
static GradWs grad_ws(const mamba2_dims& d) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t B = d.batch, L = d.seqlen, H = d.nheads, N = d.dstate;
  GradWs w;
  w.dBh = 0;
  w.dCh = up(w.dBh + B * L * H * N * 4);
  w.e = up(w.dCh + B * L * H * N * 4);
  w.q = up(w.e + B * L * H * 4);
  w.eT = up(w.q + B * L * H * 4);
  w.dAp = up(w.eT + B * H * 4);
  w.dDp = up(w.dAp + B * H * 4);
  w.dbp = up(w.dDp + B * H * 4);
  w.total = up(w.dbp + B * H * 4);
  return w;
}

size_t scan_grad_workspace_bytes(const mamba2_dims& d) { return grad_ws(d).total; }

template <typename IO, int N>
static hipError_t launch_grad_N(const mamba2_dims& d, const GradArgs<IO>& a, hipStream_t st) {
  const unsigned bh = (unsigned)(d.batch * d.nheads);
  grad_sweep_kernel<IO, N><<<2 * bh, GradShape<N>::NTH, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  grad_chain_kernel<IO><<<bh, kChainT, 0, st>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the reduction reads only workspace and lengths: an argument block with
  // the I/O pointers left out
  GradArgs<float> r{};
  r.seqlens = a.seqlens;
  r.B = a.B; r.L = a.L; r.H = a.H; r.G = a.G;
  r.dB = a.dB; r.dC = a.dC; r.dA = a.dA; r.dD = a.dD; r.dbias = a.dbias;
  r.dBh = a.dBh; r.dCh = a.dCh; r.dAp = a.dAp; r.dDp = a.dDp; r.dbp = a.dbp;
  const long long total = (long long)d.batch * d.seqlen * d.ngroups * N;
  grad_reduce_kernel<N><<<(unsigned)((total + 255) / 256), 256, 0, st>>>(r);
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_grad_IO(const mamba2_dims& d, const mamba2_scan_grad_io& io_, void* ws, hipStream_t st) {
  const GradWs wl = grad_ws(d);
  char* base = (char*)ws;
  GradArgs<IO> a{};
  a.x = (const IO*)io_.x;
  a.dt = (const IO*)io_.dt;
  a.Bm = (const IO*)io_.B;
  a.Cm = (const IO*)io_.C;
  a.dy = (const IO*)io_.dy;
  a.A = io_.A;
  a.D = io_.D;
  a.dt_bias = d.dt_softplus ? io_.dt_bias : nullptr;
  a.h0 = io_.state_in;
  a.dhT = io_.dstate_out;
  a.seqlens = io_.seqlens;
  a.dt_sp = d.dt_softplus;
  a.B = d.batch; a.L = d.seqlen; a.H = d.nheads; a.G = d.ngroups;
  a.dx = io_.dx; a.ddt = io_.ddt; a.dB = io_.dB; a.dC = io_.dC; a.dA = io_.dA; a.dD = io_.dD;
  a.dh0 = io_.dstate_in;
  a.dbias = d.dt_softplus ? io_.ddt_bias : nullptr;
  a.dBh = (float*)(base + wl.dBh);
  a.dCh = (float*)(base + wl.dCh);
  a.e = (float*)(base + wl.e);
  a.q = (float*)(base + wl.q);
  a.eT = (float*)(base + wl.eT);
  a.dAp = (float*)(base + wl.dAp);
  a.dDp = (float*)(base + wl.dDp);
  a.dbp = (float*)(base + wl.dbp);
  switch (d.dstate) {
    case 16: return launch_grad_N<IO, 16>(d, a, st);
    case 64: return launch_grad_N<IO, 64>(d, a, st);
    default: return launch_grad_N<IO, 128>(d, a, st);
  }
}

hipError_t launch_scan_grad(const mamba2_dims& d, const mamba2_scan_grad_io& io_, void* ws, hipStream_t st) {
  if (d.io_dtype == MAMBA2_F16) return launch_grad_IO<_Float16>(d, io_, ws, st);
  return launch_grad_IO<float>(d, io_, ws, st);
}

}  // namespace m2

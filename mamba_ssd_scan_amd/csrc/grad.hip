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

constexpr int kGTB = 16;       // tokens staged per block
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
  float* e;                // (B,L,H)
  float* eT;               // (B,H)
  float* dAp;              // (B,H) per-sequence dA
  float* dDp;              // (B,H) per-sequence dD
  float* dbp;              // (B,H) per-sequence dt-bias gradient
};

template <typename IO> __device__ __forceinline__ float ldf(const IO* p) { return (float)*p; }

// Staging of one block of up to kGTB tokens into LDS (zeros past nt).
template <typename IO, int N> struct GradStage {
  float x[kGTB][kGP];
  float dy[kGTB][kGP];
  float b[kGTB][N];
  float c[kGTB][N];
  float dt[kGTB];
};

template <typename IO, int N>
__device__ __forceinline__ void grad_stage(GradStage<IO, N>& st, const GradArgs<IO>& a, int b, int h, int g, int t0,
                                           int nt, int tid) {
  for (int id = tid; id < kGTB * kGP; id += 256) {
    const int j = id / kGP, p = id % kGP;
    const bool ok = j < nt;
    const size_t row = ((size_t)b * a.L + t0 + j) * a.H + h;
    st.x[j][p] = ok ? ldf(a.x + row * kGP + p) : 0.f;
    st.dy[j][p] = ok ? ldf(a.dy + row * kGP + p) : 0.f;
  }
  for (int id = tid; id < kGTB * N; id += 256) {
    const int j = id / N, n = id % N;
    const bool ok = j < nt;
    const size_t row = ((size_t)b * a.L + t0 + j) * a.G + g;
    st.b[j][n] = ok ? ldf(a.Bm + row * N + n) : 0.f;
    st.c[j][n] = ok ? ldf(a.Cm + row * N + n) : 0.f;
  }
  if (tid < kGTB) {
    float d = 0.f;
    if (tid < nt) {
      d = ldf(a.dt + ((size_t)b * a.L + t0 + tid) * a.H + h);
      if (a.dt_sp) d = dt_softplus(d, a.dt_bias ? a.dt_bias[h] : 0.f);
    }
    st.dt[tid] = d;
  }
}

// Sum of v over the lanes of each row (LPR consecutive lanes): every lane of
// the row ends with the row's sum.
template <int LPR> __device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
// Sum over the row groups of a wave (lanes with the same lane % LPR).
template <int LPR> __device__ __forceinline__ float col_sum(float v) {
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---- forward sweep: h_t, dC (per head), e_t, eT --------------------------------
template <typename IO, int N>
__global__ __launch_bounds__(256) void grad_forward_kernel(const GradArgs<IO> a) {
  constexpr int LPR = N / 8, RPP = 256 / LPR;
  constexpr int KR = RPP >= kGP ? 1 : kGP / RPP;
  constexpr bool ROW_GUARD = RPP > kGP;
  __shared__ GradStage<IO, N> st;
  __shared__ float sdc[kGTB][4][N];       // per-wave dC partials
  __shared__ float se[kGTB][4];
  __shared__ float sred[4];
  const int bh = blockIdx.x, b = bh / a.H, h = bh - b * a.H, g = h / (a.H / a.G);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nc = (tid % LPR) * 8, r0 = tid / LPR;
  const bool has_row = !ROW_GUARD || r0 < kGP;
  int len = a.seqlens ? a.seqlens[b] : a.L;
  len = len < 0 ? 0 : (len > a.L ? a.L : len);
  const float Ah = a.A[h];

  float hs[KR][8];
#pragma unroll
  for (int k = 0; k < KR; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      hs[k][i] = (a.h0 && has_row) ? a.h0[((size_t)bh * kGP + r0 + k * RPP) * N + nc + i] : 0.f;

  for (int t0 = 0; t0 < len; t0 += kGTB) {
    const int nt = min(kGTB, len - t0);
    grad_stage<IO, N>(st, a, b, h, g, t0, nt, tid);
    __syncthreads();
    for (int j = 0; j < nt; ++j) {
      const float d = st.dt[j];
      const float dec = __expf(d * Ah);
      float bv[8], cv[8], dc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bv[i] = st.b[j][nc + i];
        cv[i] = st.c[j][nc + i];
        dc[i] = 0.f;
      }
      float ep = 0.f;
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        const int p = r0 + k * RPP;
        const float xp = has_row ? st.x[j][p] : 0.f;
        const float dyp = has_row ? st.dy[j][p] : 0.f;
        const float u = d * xp;
        float yc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          hs[k][i] = __builtin_fmaf(dec, hs[k][i], u * bv[i]);
          yc = __builtin_fmaf(hs[k][i], cv[i], yc);
          dc[i] = __builtin_fmaf(dyp, hs[k][i], dc[i]);
        }
        yc = row_sum<LPR>(yc);
        if ((tid % LPR) == 0) ep = __builtin_fmaf(dyp, yc, ep);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) dc[i] = col_sum<LPR>(dc[i]);
      if (lane < LPR) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sdc[j][wv][nc + i] = dc[i];
      }
      ep = wave_sum(ep);
      if (lane == 0) se[j][wv] = ep;
    }
    __syncthreads();
    for (int id = tid; id < nt * N; id += 256) {
      const int j = id / N, n = id % N;
      const float v = (sdc[j][0][n] + sdc[j][1][n]) + (sdc[j][2][n] + sdc[j][3][n]);
      a.dCh[(((size_t)b * a.L + t0 + j) * a.H + h) * N + n] = v;
    }
    if (tid < nt) a.e[((size_t)b * a.L + t0 + tid) * a.H + h] = (se[tid][0] + se[tid][1]) + (se[tid][2] + se[tid][3]);
    __syncthreads();
  }
  // eT = <dhT, h_len>
  float et = 0.f;
  if (a.dhT && has_row) {
#pragma unroll
    for (int k = 0; k < KR; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        et = __builtin_fmaf(a.dhT[((size_t)bh * kGP + r0 + k * RPP) * N + nc + i], hs[k][i], et);
  }
  et = wave_sum(et);
  if (lane == 0) sred[wv] = et;
  __syncthreads();
  if (tid == 0) a.eT[bh] = (sred[0] + sred[1]) + (sred[2] + sred[3]);
}

// ---- reverse sweep: gh_t, dx, dB (per head), ddt, dA, dD, dh0 ------------------
template <typename IO, int N>
__global__ __launch_bounds__(256) void grad_reverse_kernel(const GradArgs<IO> a) {
  constexpr int LPR = N / 8, RPP = 256 / LPR;
  constexpr int KR = RPP >= kGP ? 1 : kGP / RPP;
  constexpr bool ROW_GUARD = RPP > kGP;
  __shared__ GradStage<IO, N> st;
  __shared__ float sdb[kGTB][4][N];       // per-wave dB partials (before the dt factor)
  __shared__ float sq[kGTB][4];
  __shared__ float sdx[kGTB][kGP];
  __shared__ float sred[2][4];
  const int bh = blockIdx.x, b = bh / a.H, h = bh - b * a.H, g = h / (a.H / a.G);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nc = (tid % LPR) * 8, r0 = tid / LPR;
  const bool has_row = !ROW_GUARD || r0 < kGP;
  int len = a.seqlens ? a.seqlens[b] : a.L;
  len = len < 0 ? 0 : (len > a.L ? a.L : len);
  const float Ah = a.A[h], Dh = a.D[h];
  const float dtb = a.dt_sp && a.dt_bias ? a.dt_bias[h] : 0.f;

  float gh[KR][8];
#pragma unroll
  for (int k = 0; k < KR; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      gh[k][i] = (a.dhT && has_row) ? a.dhT[((size_t)bh * kGP + r0 + k * RPP) * N + nc + i] : 0.f;
  float dDacc = 0.f;
  // thread 0 runs the scalar chain over the tokens (in double)
  double R = 0.0, dA_acc = 0.0, dbias_acc = 0.0;
  const float eT = a.eT[bh];

  const int nblk = (len + kGTB - 1) / kGTB;
  for (int kb = nblk - 1; kb >= 0; --kb) {
    const int t0 = kb * kGTB;
    const int nt = min(kGTB, len - t0);
    grad_stage<IO, N>(st, a, b, h, g, t0, nt, tid);
    __syncthreads();
    for (int j = nt - 1; j >= 0; --j) {
      const float d = st.dt[j];
      const float dec = __expf(d * Ah);
      float bv[8], cv[8], db[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bv[i] = st.b[j][nc + i];
        cv[i] = st.c[j][nc + i];
        db[i] = 0.f;
      }
      float qp = 0.f;
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        const int p = r0 + k * RPP;
        const float xp = has_row ? st.x[j][p] : 0.f;
        const float dyp = has_row ? st.dy[j][p] : 0.f;
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          gh[k][i] = __builtin_fmaf(cv[i], dyp, gh[k][i]);   // gradient with respect to h_t
          v = __builtin_fmaf(gh[k][i], bv[i], v);
          db[i] = __builtin_fmaf(xp, gh[k][i], db[i]);
        }
        v = row_sum<LPR>(v);
        if (has_row && (tid % LPR) == 0) {
          sdx[j][p] = __builtin_fmaf(d, v, Dh * dyp);
          qp = __builtin_fmaf(xp, v, qp);
          dDacc = __builtin_fmaf(dyp, xp, dDacc);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) gh[k][i] *= dec;                // ... and with respect to h_{t-1}
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) db[i] = col_sum<LPR>(db[i]);
      if (lane < LPR) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sdb[j][wv][nc + i] = db[i];
      }
      qp = wave_sum(qp);
      if (lane == 0) sq[j][wv] = qp;
    }
    __syncthreads();
    for (int id = tid; id < nt * N; id += 256) {
      const int j = id / N, n = id % N;
      const float v = (sdb[j][0][n] + sdb[j][1][n]) + (sdb[j][2][n] + sdb[j][3][n]);
      a.dBh[(((size_t)b * a.L + t0 + j) * a.H + h) * N + n] = st.dt[j] * v;
    }
    for (int id = tid; id < nt * kGP; id += 256) {
      const int j = id / kGP, p = id % kGP;
      a.dx[(((size_t)b * a.L + t0 + j) * a.H + h) * kGP + p] = sdx[j][p];
    }
    if (tid == 0) {
      for (int j = nt - 1; j >= 0; --j) {
        const int t = t0 + j;
        const size_t ti = ((size_t)b * a.L + t) * a.H + h;
        const double q = (double)((sq[j][0] + sq[j][1]) + (sq[j][2] + sq[j][3]));
        const double d = (double)st.dt[j];
        R += (double)a.e[ti] + (t == len - 1 ? (double)eT : 0.0) - d * q;
        const double gdt = q + (double)Ah * R;
        dA_acc += d * R;
        double graw = gdt;
        if (a.dt_sp) {
          const double v = (double)ldf(a.dt + ti) + (double)dtb;
          graw = gdt * (v > 20.0 ? 1.0 : 1.0 / (1.0 + exp(-v)));
          dbias_acc += graw;
        }
        a.ddt[ti] = (float)graw;
      }
    }
    __syncthreads();
  }
  // rows past the length: zero gradients
  for (int id = tid; id < (a.L - len) * kGP; id += 256) {
    const int t = len + id / kGP, p = id % kGP;
    a.dx[(((size_t)b * a.L + t) * a.H + h) * kGP + p] = 0.f;
  }
  for (int t = len + tid; t < a.L; t += 256) a.ddt[((size_t)b * a.L + t) * a.H + h] = 0.f;
  if (a.dh0 && has_row) {
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      float* dst = a.dh0 + ((size_t)bh * kGP + r0 + k * RPP) * N + nc;
      *reinterpret_cast<f4*>(dst) = f4{gh[k][0], gh[k][1], gh[k][2], gh[k][3]};
      *reinterpret_cast<f4*>(dst + 4) = f4{gh[k][4], gh[k][5], gh[k][6], gh[k][7]};
    }
  }
  dDacc = wave_sum(dDacc);
  if (lane == 0) sred[0][wv] = dDacc;
  __syncthreads();
  if (tid == 0) {
    a.dDp[bh] = (sred[0][0] + sred[0][1]) + (sred[0][2] + sred[0][3]);
    a.dAp[bh] = (float)dA_acc;
    a.dbp[bh] = (float)dbias_acc;
  }
}

// ---- sums over the heads of each group and over the batch --------------------
// dB, dC: one thread per (b, t, g, n), heads of the group in index order (rows
// past a sequence's length are zero); dA, dD, dt-bias: one thread per head,
// sequences in index order.
template <int N>
__global__ __launch_bounds__(256) void grad_reduce_kernel(const GradArgs<float> a, int io_unused) {
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
  size_t dBh, dCh, e, eT, dAp, dDp, dbp, total;
};
static GradWs grad_ws(const mamba2_dims& d) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t B = d.batch, L = d.seqlen, H = d.nheads, N = d.dstate;
  GradWs w;
  w.dBh = 0;
  w.dCh = up(w.dBh + B * L * H * N * 4);
  w.e = up(w.dCh + B * L * H * N * 4);
  w.eT = up(w.e + B * L * H * 4);
  w.dAp = up(w.eT + B * H * 4);
  w.dDp = up(w.dAp + B * H * 4);
  w.dbp = up(w.dDp + B * H * 4);
  w.total = up(w.dbp + B * H * 4);
  return w;
}

size_t scan_grad_workspace_bytes(const mamba2_dims& d) { return grad_ws(d).total; }

template <typename IO, int N>
static hipError_t launch_grad_N(const mamba2_dims& d, const GradArgs<IO>& a, hipStream_t st) {
  const unsigned grid = (unsigned)(d.batch * d.nheads);
  grad_forward_kernel<IO, N><<<grid, 256, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  grad_reverse_kernel<IO, N><<<grid, 256, 0, st>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the reduction reads only workspace and lengths: reuse the argument block
  // with the I/O pointers left out
  GradArgs<float> r{};
  r.seqlens = a.seqlens;
  r.B = a.B; r.L = a.L; r.H = a.H; r.G = a.G;
  r.dB = a.dB; r.dC = a.dC; r.dA = a.dA; r.dD = a.dD; r.dbias = a.dbias;
  r.dBh = a.dBh; r.dCh = a.dCh; r.dAp = a.dAp; r.dDp = a.dDp; r.dbp = a.dbp;
  const long long total = (long long)d.batch * d.seqlen * d.ngroups * N;
  const unsigned rg = (unsigned)((total + 255) / 256);
  grad_reduce_kernel<N><<<rg > 0 ? rg : 1, 256, 0, st>>>(r, 0);
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

// Whole-window Mamba-2 scan for few sequences: one workgroup per (sequence,
// head, half of the head dim) runs the whole sequence, with the state split
// over n between its waves.
//
// The method is Mamba-2 / structured state-space duality (Dao and Gu 2024,
// listed under "References" on page "Mamb2_8B_FP4_Recall_SQ3.25").  Per head,
// with log2-decays S_t running from the start of a chunk, each 32-token step
// takes the state H entering it to
//   y_t = 2^{S_t - S_start} C_t . H                                 (readout)
//       + sum_{s <= t in the step} (C_t . B_s) dt_s 2^{S_t - S_s} x_s (diagonal)
//       + D x_t
//   H  <- 2^{S_end - S_start} H + sum_s dt_s 2^{S_end - S_s} x_s B_s^T.
// Both the readout C_t . H and the diagonal's C_t . B_s are sums over the
// state index n, and the state update is separable over n.  So the state of
// a (head, 32 columns of p) pair is split into four quarters of n, each held
// by two waves (16 columns of p each) as 16x16 fp32 MFMA tiles: a wave owns
// H[n in its quarter][p in its 16 columns] and computes its quarter's share
// of the step's outputs (readout and diagonal over its 32 values of n).  The
// four shares of each output are summed through LDS in the next step.  The
// recurrence never leaves the wave, so a sequence needs no split into
// segments and no hand-off between workgroups: x is read from HBM once, y is
// written once.  When the batch is small this gives 2 x heads x sequences
// workgroups (256 for one 8B-shape sequence), where splitting by heads alone
// would leave most compute units idle.  A wave's share of the state is a
// quarter of the segmented scan's, so per output its steps cost more (their
// barrier, LDS round trips and share sums are not amortized): the library
// routes only short windows here.
//
// Per wave and step: readout 2 MFMAs, its quarter's C.B^T blocks 3, the
// masked diagonal product 2, the state update 2 (16x16x32 f16, fp32
// accumulate).  The x, B and C rows of a step are loaded straight into LDS
// (buffer loads that write LDS) two steps ahead, one workgroup barrier per
// step; the barrier that publishes step k + 1's rows also publishes step k's
// output shares.
#include <stddef.h>

#include "common.h"
#include "gfx950_ops.h"
#include "ssd_scan.h"

namespace m2 {

namespace cs {
constexpr int TS = 32;     // tokens per step
constexpr int N = 128;     // state size
constexpr int P = 64;      // head dim
constexpr int PH = 32;     // head-dim columns per workgroup
constexpr int NWV = 8;     // waves: (quarter of n) x (16 columns of p)
constexpr int NTH = 64 * NWV;
constexpr int QMAX = 256;  // largest chunk
constexpr int DEPTH = 2;   // steps the loads run ahead of the step computed
constexpr int NSL = DEPTH + 1;

struct alignas(16) Slot {
  _Float16 x[TS * PH];   // 32 tokens x 64 bytes
  _Float16 b[TS * N];    // 32 tokens x 256 bytes
  _Float16 c[TS * N];
};

// Output shares: per (p block pq, n quarter nq) and t-tile T, the writer's
// lane (lr, q) puts its four values (t = 16 T + lr, p = 4 q .. 4 q + 3) at
// float 72 q + 4 lr: each 16-lane group writes 256 contiguous bytes, and the
// 8 bytes each reader lane takes (t = 4w + lane/16, p = 2 (lane%16), +1) of
// four q blocks 288 bytes apart fall on distinct banks; the two p blocks lie
// 128 bytes apart modulo the 256-byte bank width for the same reason.
constexpr int SH_Q = 72;              // floats per q block (64 + 8 pad)
constexpr int SH_T = 4 * SH_Q;        // per t-tile
constexpr int SH_NQ = 2 * SH_T;       // per (pq, nq) block
constexpr int SH_PQ = 4 * SH_NQ + 32;
constexpr int SH_BUF = 2 * SH_PQ;

// x row t (64 bytes, 4 units of 16 bytes): unit k at physical unit k ^ xsw(t).
// The transposed reads (rows 4q + i, 8-byte chunks of p) and the 8-byte row
// reads of a 16-row block fall on distinct banks.
__device__ __forceinline__ int xsw(int t) { return (2 * ((t >> 2) & 1)) ^ ((t >> 3) & 1); }
__device__ __forceinline__ int xo(int t, int k) { return t * PH + 8 * (k ^ xsw(t)); }
// B/C row s (256 bytes, 16 units): unit k at physical unit k ^ bsw(s), bsw a
// bijection of the row's low four bits (GF(2)-linear, row bits 0..3 to
// units 3, 4, 8, 9).  Row reads of 16 rows at one unit: 16 distinct units.
// Transposed reads (8 rows x 4 chunks of n): 16 distinct units x 2 halves.
__device__ __forceinline__ int bsw(int s) {
  return (3 * (s & 1)) ^ (4 * ((s >> 1) & 1)) ^ (8 * ((s >> 2) & 1)) ^ (9 * ((s >> 3) & 1));
}
__device__ __forceinline__ int bo(int s, int k) { return s * N + 8 * (k ^ bsw(s)); }
}  // namespace cs

__global__ __launch_bounds__(cs::NTH) void ssd_colscan_kernel(ScanArgs a) {
  using namespace cs;
  __shared__ Slot slots[NSL];
  __shared__ float shares[2 * SH_BUF];
  // per wave, the current chunk: log2-decay from the chunk start (inclusive),
  // dt, state-update weight, readout scale
  __shared__ float Sx[NWV][QMAX], Dx[NWV][QMAX], Wx[NWV][QMAX], Cx[NWV][QMAX];
  __shared__ unsigned dtr[2][QMAX];   // a chunk's dt, the dword that holds each token's element

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, q = lane >> 4;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pq = wid & 1, nq = wid >> 1;
  const int hpg = a.H / a.G;
  const int per = 2 * hpg;             // workgroups per (sequence, group)
  const int BG = a.B * a.G;
  // workgroups are dealt to the XCDs round-robin: with B*G a multiple of 8,
  // every workgroup of a (sequence, group) sits on one XCD and its L2 holds
  // the group's B and C rows once for all 2 x (heads per group) readers
  const int bid = (int)blockIdx.x;
  int bg, r;
  if (BG % 8 == 0) {
    const int s = bid >> 3;
    bg = (bid & 7) + 8 * (s / per);
    r = s % per;
  } else {
    bg = bid / per;
    r = bid % per;
  }
  const int b = bg / a.G, g = bg - b * a.G;
  const int h = g * hpg + (r >> 1), half = r & 1;
  const int hb = b * a.H + h;

  const SeqRows span = seq_rows(a.seqlens, a.cu, b, a.L, a.T);
  const int len = __builtin_amdgcn_readfirstlane(span.len);
  const int ubase = __builtin_amdgcn_readfirstlane((int)span.base);
  const size_t xbase = a.xpk ? (size_t)ubase : (size_t)b * a.L;
  const float Ah = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a.A[h] * kLog2e)));
  const float Dh = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a.D[h])));
  const float dtbl = a.dt_sp && a.dt_bias
                         ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a.dt_bias[h])))
                         : 0.f;

  // buffer views of this sequence (each range ends at its last token)
  constexpr unsigned ES = 2;
  const unsigned xrow = (unsigned)a.xstride * ES;
  const unsigned grow = (unsigned)a.gstride * ES;
  const unsigned yrow = (unsigned)(a.H * P) * ES;
  const unsigned xspan = len > 0 ? (unsigned)(len - 1) * xrow + PH * ES : 0u;
  const unsigned yspan = len > 0 ? (unsigned)(len - 1) * yrow + PH * ES : 0u;
  const unsigned gspan = len > 0 ? (unsigned)(len - 1) * grow + N * ES : 0u;
  const u4 rx = rsrc_words(a.x + xbase * a.xstride + (size_t)h * P + PH * half, xspan);
  const u4 rb = rsrc_words(a.Bm + xbase * a.gstride + (size_t)g * N, gspan);
  const u4 rc = rsrc_words(a.Cm + xbase * a.gstride + (size_t)g * N, gspan);
  const rsrc_t ry = mkr(a.y + ((size_t)ubase * a.H + h) * P + PH * half, yspan);
  // dt of this head: token t's element sits sh0 + t dtld elements past a
  // 4-byte aligned base (dt needs only element alignment, any row stride)
  const _Float16* const dt0 = a.dt + (size_t)ubase * a.dtld + h;
  const unsigned sh0 = (unsigned)(((size_t)dt0 >> 1) & 1);
  const unsigned dtld = (unsigned)a.dtld;
  const u4 rdt = rsrc_words(dt0 - sh0, len > 0 ? (((sh0 + (unsigned)(len - 1) * dtld) + 1u) * ES + 3u) & ~3u : 0u);

  float* const Sw = Sx[wid];
  float* const Dw = Dx[wid];
  float* const Ww = Wx[wid];
  float* const Cw = Cx[wid];

  // zero the slots once: rows a step loads past the sequence's end are
  // never written, and their (unused) values must be finite
  {
    constexpr int SLOT16 = (int)(sizeof(Slot) / 16);
    u4* z = reinterpret_cast<u4*>(&slots[0]);
    for (int i = tid; i < NSL * SLOT16; i += NTH) z[i] = u4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  const int Q = a.Q, J = Q / TS;
  const int nsteps = (len + TS - 1) / TS;
  const int nch = (len + Q - 1) / Q;

  // ---- loads (this wave's share) -------------------------------------------------
  // per step: waves 0 and 1 load 16 x rows each; every wave loads 4 rows of
  // B and 4 of C.  Per chunk: waves 0 .. Q/64 - 1 load 64 tokens' dt each.
  const int DL = wid < 2 ? 3 : 2;                 // loads per step of this wave
  const int DT = wid < Q / 64 ? 1 : 0;            // dt loads per chunk of this wave
  // (slot addresses as LDS byte offsets: the slot index is a runtime value)
  const unsigned lds_slots = lds_addr(&slots[0]);
  constexpr unsigned kSlotBytes = (unsigned)sizeof(Slot);
  constexpr unsigned kOffB = (unsigned)offsetof(Slot, b), kOffC = (unsigned)offsetof(Slot, c);
  auto issue = [&](int si, int tok0) __attribute__((always_inline)) {
    const unsigned t0 = (unsigned)tok0;
    const unsigned base = lds_slots + (unsigned)si * kSlotBytes;
    if (wid < 2) {
      const int row = 16 * wid + (lane >> 2), pk = lane & 3;
      dma16(rx, base + 1024u * (unsigned)wid, (t0 + (unsigned)row) * xrow + 16u * (unsigned)(pk ^ xsw(row)));
    }
    const int row = 4 * wid + (lane >> 4), pk = lane & 15;
    const unsigned go = (t0 + (unsigned)row) * grow + 16u * (unsigned)(pk ^ bsw(row));
    dma16(rb, base + kOffB + 1024u * (unsigned)wid, go);
    dma16(rc, base + kOffC + 1024u * (unsigned)wid, go);
  };
  auto issue_dt = [&](int c) __attribute__((always_inline)) {
    if (DT) {
      const unsigned e = sh0 + (unsigned)(c * Q + 64 * wid + lane) * dtld;
      dma4(rdt, lds_addr(&dtr[c & 1][64 * wid]), (e & ~1u) * ES);
    }
  };

  // ---- per chunk: dt and the running log2-decay (4 tokens per lane) -------------
  // Per token i: S_i, dt_i, the update weight w_i = dt_i 2^{S_end - S_i}
  // (S_end: the end of i's step) and the readout scale 2^{S_i - S_start}
  // (S_start: before i's step).  Only differences S_a - S_b with a later
  // than b are exponentiated, so both are at most dt_i and 1.  Tokens past
  // the sequence keep dt = 0: the state passes through them unchanged.
  auto scan_dt = [&](int c) __attribute__((always_inline)) {
    const u4 wd = *reinterpret_cast<const u4*>(&dtr[c & 1][4 * lane]);
    float d[4], v[4], run = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * lane + e;
      const unsigned par = (sh0 + (unsigned)(c * Q + i) * dtld) & 1u;
      float u = (float)__builtin_bit_cast(_Float16, (unsigned short)(par ? wd[e] >> 16 : wd[e] & 0xffffu));
      if (a.dt_sp) u = dt_softplus_fast(u, dtbl);
      if (i >= Q || c * Q + i >= len) u = 0.f;
      d[e] = u;
      run += u * Ah;
      v[e] = run;
    }
    float pre = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float u = __shfl_up(pre, off, 64);
      if (lane >= off) pre += u;
    }
    pre -= run;
    f4 sv, dv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = v[e] + pre;
      dv[e] = d[e];
    }
    // (each lane's four tokens lie in one step; a wave's LDS accesses
    // complete in order, so the reads below see the stores above)
    const bool in = 4 * lane < Q;
    if (in) {
      *reinterpret_cast<f4*>(&Sw[4 * lane]) = sv;
      *reinterpret_cast<f4*>(&Dw[4 * lane]) = dv;
    }
    const int step0 = (4 * lane) & ~(TS - 1);
    const float s_end = Sw[min(step0 + TS - 1, Q - 1)];
    const float s_start = step0 ? Sw[step0 - 1] : 0.f;
    f4 wv, cv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wv[e] = d[e] * ex2(s_end - sv[e]);
      cv[e] = ex2(sv[e] - s_start);
    }
    if (in) {
      *reinterpret_cast<f4*>(&Ww[4 * lane]) = wv;
      *reinterpret_cast<f4*>(&Cw[4 * lane]) = cv;
    }
  };

  // ---- the state: H[n][p], n = 32 nq + 16 j + 4 q + e, p = 16 pq + lr -------------
  f4 H[2];
  if (a.state_in) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      H[j] = *reinterpret_cast<const f4*>(a.state_in + ((size_t)hb * P + PH * half + 16 * pq + lr) * N + 32 * nq +
                                          16 * j + 4 * q);
  } else {
    H[0] = f4{0.f, 0.f, 0.f, 0.f};
    H[1] = H[0];
  }

  // ---- output shares of a step: summed over the four quarters of n, stored ------
  // wave w: tokens 4w .. 4w+3, lane: token 4w + lane/16, columns 2 (lane%16) and +1
  const int fin_t = 4 * wid + (lane >> 4), fin_p = lane & 15;
  const int fin_o = SH_PQ * (fin_p >> 3) + SH_T * (fin_t >> 4) + SH_Q * ((fin_p & 7) >> 1) + 4 * (fin_t & 15) +
                    2 * (fin_p & 1);
  auto finish = [&](int buf, int tok0) __attribute__((always_inline)) {
    const float* sb = shares + buf * SH_BUF + fin_o;
    const f2 s0 = *reinterpret_cast<const f2*>(sb);
    const f2 s1 = *reinterpret_cast<const f2*>(sb + SH_NQ);
    const f2 s2 = *reinterpret_cast<const f2*>(sb + 2 * SH_NQ);
    const f2 s3 = *reinterpret_cast<const f2*>(sb + 3 * SH_NQ);
    const f2 s = (s0 + s1) + (s2 + s3);
    const h2 hv = h2{(_Float16)s[0], (_Float16)s[1]};
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, hv), ry,
                                          (unsigned)(tok0 + fin_t) * yrow + (unsigned)(4 * fin_p), 0, 0);
  };

  // ---- the step in two halves -------------------------------------------------------
  // The front half (after the barrier that publishes the step's rows): its
  // LDS reads, the readout of the state entering it and its quarter's C.B^T
  // blocks (MFMA), the mask factors of its diagonal product, and the state
  // update.  The back half: the masked C.B^T as binary16, the diagonal
  // product (MFMA) on top of the scaled readout, and this wave's shares of
  // y written to LDS (t = 16 T + lr, p = 16 pq + 4 q + e), summed by finish
  // in the next step.  (Running the back half under the next step's reads
  // and products measured about 5 % slower: the values carried across the
  // barrier cost register moves every step.)
  // Passed from the front half to the back half:
  h8 c_xa;            // x^T of the step (the diagonal's A operand)
  f4 c_gb[3];         // C.B^T blocks (s-tile, t-tile) = (0,0), (0,1), (1,1)
  f4 c_yr[2];         // readout C.H of t-tiles 0, 1
  float c_fac[3][4];  // mask factors dt_s 2^{S_t - S_s} (0 where s > t)
  float c_sc[2];      // readout scales of the lane's two columns t
  h4 c_xr[2];         // x[t][p] for D x (first quarter of n)
  // k slots: the lane's causal positions in the diagonal blocks (4q + e <= lr)
  bool cz[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) cz[e] = 4 * q + e <= lr;
  const float Dq = nq == 0 ? Dh : 0.f;   // D x enters once, with the first quarter's shares

  auto front = [&](const Slot& sl, int i0) __attribute__((always_inline)) {
    const float Sj_start = i0 ? Sw[i0 - 1] : 0.f;
    const float Sj_end = Sw[i0 + TS - 1];
    // x^T rows p = 16 pq + lr over tokens s = 4q..4q+3, 16+4q..+3 (transposed
    // reads): the diagonal's A operand and, weighted, the update's B operand
    h8 xa;
    {
      const int k = 2 * pq + ((lr & 3) >> 1), o = 4 * (lr & 1);
      xa = cat(tr4(&sl.x[xo(4 * q + (lr >> 2), k) + o]), tr4(&sl.x[xo(16 + 4 * q + (lr >> 2), k) + o]));
    }
    // B^T rows n = 32 nq + 16 j + lr over the same tokens (transposed reads)
    h8 bt[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k = 4 * nq + 2 * j + ((lr & 3) >> 1), o = 4 * (lr & 1);
      bt[j] = cat(tr4(&sl.b[bo(4 * q + (lr >> 2), k) + o]), tr4(&sl.b[bo(16 + 4 * q + (lr >> 2), k) + o]));
    }
    // C rows t = 16 T + lr and B rows s = 16 S + lr at n = 32 nq + 4q..+3,
    // 32 nq + 16 + 4q..+3 (the k slots of the state's readout operand)
    h8 cf[2], bs[2];
    {
      const int k0 = 4 * nq + (q >> 1), k1 = k0 + 2, o = 4 * (q & 1);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        const int t = 16 * T + lr;
        cf[T] = cat(*reinterpret_cast<const h4*>(&sl.c[bo(t, k0) + o]), *reinterpret_cast<const h4*>(&sl.c[bo(t, k1) + o]));
        bs[T] = cat(*reinterpret_cast<const h4*>(&sl.b[bo(t, k0) + o]), *reinterpret_cast<const h4*>(&sl.b[bo(t, k1) + o]));
      }
    }
    const f4 w0 = *reinterpret_cast<const f4*>(&Ww[i0 + 4 * q]);
    const f4 w1 = *reinterpret_cast<const f4*>(&Ww[i0 + 16 + 4 * q]);
    float St[2], sc[2];
    h4 xr[2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const int t = 16 * T + lr;
      St[T] = Sw[i0 + t];
      sc[T] = Cw[i0 + t];
      xr[T] = *reinterpret_cast<const h4*>(&sl.x[xo(t, 2 * pq + (q >> 1)) + 4 * (q & 1)]);
    }
    return [=, &c_xa, &c_gb, &c_yr, &c_fac, &c_sc, &c_xr](f4 (&Hs)[2]) __attribute__((always_inline)) {
      // readout of the state entering the step: H as binary16 (k slots as cf)
      const h8 ra = h8{(_Float16)Hs[0][0], (_Float16)Hs[0][1], (_Float16)Hs[0][2], (_Float16)Hs[0][3],
                       (_Float16)Hs[1][0], (_Float16)Hs[1][1], (_Float16)Hs[1][2], (_Float16)Hs[1][3]};
#pragma unroll
      for (int T = 0; T < 2; ++T) c_yr[T] = mfma16(ra, cf[T], f4{0.f, 0.f, 0.f, 0.f});
      // this quarter's C.B^T blocks: rows s = 16 S + 4 q + e, column t = 16 T + lr
      c_gb[0] = mfma16(bs[0], cf[0], f4{0.f, 0.f, 0.f, 0.f});
      c_gb[1] = mfma16(bs[0], cf[1], f4{0.f, 0.f, 0.f, 0.f});
      c_gb[2] = mfma16(bs[1], cf[1], f4{0.f, 0.f, 0.f, 0.f});
      // update: H <- dec H + B^T (w x)
      const float dec = ex2(Sj_end - Sj_start);
      const float w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      h8 xw;
#pragma unroll
      for (int e = 0; e < 8; ++e) xw[e] = (_Float16)__builtin_fmaf((float)xa[e], w[e], 0.f);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        Hs[j] *= dec;
        Hs[j] = mfma16(bt[j], xw, Hs[j]);
      }
      // The mask factor of (s, t), s <= t, is dt_s 2^{S_t - S_s}.  It factors
      // as w_s 2^{S_t - S_end} with w_s = dt_s 2^{S_end - S_s} <= dt_s and
      // 2^{S_t - S_end} >= 1, both finite while the step decays by no more
      // than 2^-100; past that (rare) each factor is formed on its own, the
      // exponent clamped so that the masked entries (s > t) stay finite.
      if (__builtin_amdgcn_readfirstlane(Sj_start - Sj_end <= 100.f ? 1 : 0)) {
        const float u0 = ex2(St[0] - Sj_end), u1 = ex2(St[1] - Sj_end);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c_fac[0][e] = cz[e] ? w[e] * u0 : 0.f;
          c_fac[1][e] = w[e] * u1;
          c_fac[2][e] = cz[e] ? w[4 + e] * u1 : 0.f;
        }
      } else {
#pragma unroll
        for (int bk = 0; bk < 3; ++bk) {
          const int S = bk == 2 ? 1 : 0, T = bk == 0 ? 0 : 1;
          const f4 sv = *reinterpret_cast<const f4*>(&Sw[i0 + 16 * S + 4 * q]);
          const f4 dv = *reinterpret_cast<const f4*>(&Dw[i0 + 16 * S + 4 * q]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float f = dv[e] * ex2(fminf(St[T] - sv[e], 0.f));
            c_fac[bk][e] = (bk == 1 || cz[e]) ? f : 0.f;
          }
        }
      }
      c_xa = xa;
      c_sc[0] = sc[0];
      c_sc[1] = sc[1];
      c_xr[0] = xr[0];
      c_xr[1] = xr[1];
    };
  };
  auto back = [&](int buf) __attribute__((always_inline)) {
    h8 mf[2];
    {
      float v[3][4];
#pragma unroll
      for (int bk = 0; bk < 3; ++bk)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[bk][e] = c_gb[bk][e] * c_fac[bk][e];
      mf[0] = h8{(_Float16)v[0][0], (_Float16)v[0][1], (_Float16)v[0][2], (_Float16)v[0][3],
                 (_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
      mf[1] = h8{(_Float16)v[1][0], (_Float16)v[1][1], (_Float16)v[1][2], (_Float16)v[1][3],
                 (_Float16)v[2][0], (_Float16)v[2][1], (_Float16)v[2][2], (_Float16)v[2][3]};
    }
    float* const sb = shares + buf * SH_BUF + SH_PQ * pq + SH_NQ * nq;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      f4 init;
#pragma unroll
      for (int e = 0; e < 4; ++e) init[e] = __builtin_fmaf(Dq, (float)c_xr[T][e], c_yr[T][e] * c_sc[T]);
      const f4 ys = mfma16(c_xa, mf[T], init);
      *reinterpret_cast<f4*>(&sb[SH_T * T + SH_Q * q + 4 * lr]) = ys;
    }
  };

  // ---- streaming over the steps, DEPTH + 1 slots in rotation ---------------------
  // Per step k: the loads of step k + DEPTH (and at a chunk's first step the
  // next chunk's dt), step k - 1's outputs summed and stored, step k, then
  // the barrier that publishes step k + 1's rows and step k's shares.
  // Explicit waits: vector memory operations complete in issue order, so
  // before that barrier a wave waits until no more are outstanding than it
  // issued after step k + 1's loads (per step: its dt loads, its loads, its
  // store).
  static_assert(DEPTH == 2, "the wait count below is written for loads two steps ahead");
  if (nch > 0) issue_dt(0);
  if (nsteps > 0) issue(0, 0);
  if (nsteps > 1) issue(1, TS);
  if (nsteps > 0) {
    vm_wait(nsteps > 1 ? DL : 0);   // the first chunk's dt and step 0's loads
    slot_barrier();
    scan_dt(0);
  }
  int si = 0, kc = 0, c = 0;   // slot of step k, its step in the chunk, its chunk
  for (int k = 0; k < nsteps; ++k) {
    const bool ndt = kc == 0 && c + 1 < nch;
    if (ndt) issue_dt(c + 1);
    const bool more = k + 2 < nsteps;
    if (more) issue(si == 0 ? 2 : si - 1, (k + 2) * TS);
    if (k >= 1) finish((k - 1) & 1, (k - 1) * TS);
    auto rest = front(slots[si], kc * TS);
    rest(H);
    back(k & 1);
    // issued after step k + 1's loads (in step k - 1): that step's store,
    // then this step's dt loads, loads and store
    if (k + 1 < nsteps) vm_wait((k >= 2 ? 1 : 0) + (ndt ? DT : 0) + (more ? DL : 0) + (k >= 1 ? 1 : 0));
    slot_barrier();
    si = si == 2 ? 0 : si + 1;
    if (++kc == J) {
      kc = 0;
      ++c;
      if (k + 1 < nsteps) scan_dt(c);
    }
  }
  // the last step's outputs
  if (nsteps > 0) finish((nsteps - 1) & 1, (nsteps - 1) * TS);

  if (a.state_out) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      *reinterpret_cast<f4*>(a.state_out + ((size_t)hb * P + PH * half + 16 * pq + lr) * N + 32 * nq + 16 * j +
                             4 * q) = H[j];
  }
}

// Launch: one workgroup per (sequence, head, half of the head dim).  The
// caller checks binary16 I/O, N = 128, P = 64 and a chunk of 64, 128 or 256.
hipError_t launch_ssd_colscan(const ScanArgs& a, hipStream_t st) {
  const long long wgs = 2LL * a.B * a.H;
  if (wgs <= 0) return hipSuccess;
  ssd_colscan_kernel<<<(unsigned)wgs, cs::NTH, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace m2

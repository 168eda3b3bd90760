// Whole-window Mamba-2 scan in its chunked state-space-dual form, with the
// binary16 inputs streamed from HBM into LDS by buffer loads that write LDS
// directly, two 32-token steps ahead of the step being computed.
//
// The method is Mamba-2 / structured state-space duality (Dao and Gu 2024,
// listed under "References" on page "Mamb2_8B_FP4_Recall_SQ3.25").  For one
// head, with log-decays la_t = dt_t * A_h and their running sum S_t from the
// start of a chunk, the recurrence S <- e^{la_t} S + dt_t x_t B_t^T,
// y_t = S C_t + D x_t is evaluated step by step (32 tokens), with the state
// H entering the step:
//   y_t   = sum_{s<=t in step} (C_t.B_s) e^{S_t-S_s} dt_s x_s          (diagonal)
//         + e^{S_t - S_step} C_t . H                                  (readout)
//         + D x_t
//   H    <- e^{S_end - S_step} H + sum_s e^{S_end-S_s} dt_s x_s B_s^T  (state update)
// Only differences S_t - S_s with s <= t are exponentiated, so every factor
// is <= 1.
//
// Work split: one workgroup of eight waves per (segment, sequence, group,
// block of four heads of the group); wave = (head, half of the head dim).
// The recurrence is separable over p, so each half of a head is an
// independent scan whose 32 x N share of the state stays in registers as
// 16x16 fp32 MFMA tiles of S^T[n, p].  The four heads share the group's B
// and C rows in LDS.  A segment is a run of consecutive chunks: inside it the
// state passes from step to step in registers; segments hand their
// aggregates over through an indexed tree in the workspace (local-state pass,
// hand-off, output pass, as in the other window kernel).
//
// Streaming.  Every 32-token step occupies one of three LDS slots: the
// wave's own x rows (32 x 64 bytes) and the group's B and C rows (32 x 256
// bytes each).  Each wave issues its x rows and an eighth of B and C as
// 16-byte-per-lane buffer loads that write LDS directly (no registers, no
// staging arithmetic), two steps ahead; one workgroup barrier per step makes
// a slot visible once every wave's loads into it have landed.  The three
// slots are distinct LDS objects addressed only with compile-time slot
// choices, so the compiler's wait for an LDS-writing load covers exactly
// that slot's loads and leaves the next slot's loads in flight.  The x tile
// is weighted for the state update after its transposed read, in registers.
//
// LDS layouts (16-byte units swizzled by row): x row t, unit k at
// t*64 + 16*(k ^ xsw(t)); B/C row s, unit k at s*256 + 16*(k ^ bsw(s)).  The
// buffer loads put lane l's 16 bytes at slot + 16*l, so each lane loads the
// global unit that the swizzle maps there.  The B/C swizzle is the linear map
// over GF(2) that sends row bits 0..3 to units 3, 4, 8, 9: measured with the
// LDS bank-conflict counter on gfx950, it keeps the 16-byte row reads of B
// and C (lanes 16 rows x 4 units) free of conflicts, and gives the transposed
// 8-byte reads of B (rows 4q + lane/4) their minimum, two lanes per bank
// (32 lanes of 8 bytes against 16 distinct units).  The transposed reads of
// the x tile are free of conflicts.
#include <stddef.h>
#include <type_traits>

#include "common.h"
#include "gfx950_ops.h"
#include "ssd_scan.h"
#include "../../include/mamba2ssd.h"

namespace m2 {

namespace ps {
constexpr int TS = 32;       // tokens per step
constexpr int N = 128;       // state size
constexpr int P = 64;        // head dim
constexpr int KH = 4;        // heads per workgroup
constexpr int NT = N / 16;   // state tiles along n
constexpr int KM = N / 32;   // 32-wide k-steps over n
constexpr int MAXJ = 8;      // steps per chunk at most (chunk 256)
constexpr unsigned kSpinLimit = 1u << 22;

// control block of the workspace: eight claim counters and the done counter /
// generation / error word, each on its own 128-byte line
constexpr int kCtrlStride = 32;
constexpr int kCtrlDone = 8 * kCtrlStride;
constexpr int kCtrlGen = 9 * kCtrlStride;
constexpr int kCtrlErr = 10 * kCtrlStride;

// PH head-dim columns per wave: 32 (eight waves, two per SIMD, 256
// registers each) or 64 (four waves, one per SIMD, 512 registers each).
template <int PH> struct W {
  static constexpr int WPH = P / PH;             // waves per head
  static constexpr int NWV = KH * WPH;           // waves per workgroup
  static constexpr int NTH = 64 * NWV;
  static constexpr int PT = PH / 16;             // state tiles along p
  static constexpr int XU = PH / 8;              // 16-byte units per x row
  static constexpr int XI = TS * PH * 2 / 1024;  // x loads (1 KB each) per wave and step
  static constexpr int BI = 8 / NWV;             // B (and C) loads per wave and step
  // x row t, 16-byte unit k -> physical unit (rows of 64 or 128 bytes)
  static __device__ __forceinline__ int xsw(int t) {
    if constexpr (PH == 32) return (2 * ((t >> 2) & 1)) ^ ((t >> 3) & 1);
    else return (2 * ((t >> 1) & 3)) ^ ((t >> 3) & 1);
  }
  // half offset of unit k of row r
  static __device__ __forceinline__ int xo(int r, int k) { return r * PH + 8 * (k ^ xsw(r)); }
  // (with the binary16 remainder of B from the fused conv: its rows too)
  template <bool BLO> struct alignas(16) Slot {
    _Float16 x[NWV][TS * PH];   // per wave: 32 tokens x PH columns
    _Float16 b[TS * N];         // 32 tokens x 256 bytes
    _Float16 c[TS * N];
    _Float16 bl[BLO ? TS * N : 8];
  };
};

__device__ __forceinline__ int bsw(int s) {
  return (3 * (s & 1)) ^ (4 * ((s >> 1) & 1)) ^ (8 * ((s >> 2) & 1)) ^ (9 * ((s >> 3) & 1));
}
__device__ __forceinline__ int bo(int r, int k) { return r * N + 8 * (k ^ bsw(r)); }

// first state column of the 4-row group j of state tile nt: lane group j of
// k-step m reads n = 8 j + 32 m .. + 7, tiles 2m and 2m+1 hold its two halves
__device__ __forceinline__ int ncol(int nt, int j) { return 8 * j + 32 * (nt >> 1) + 4 * (nt & 1); }

}  // namespace ps

template <int PH, bool BLO, bool A16>
__global__ __launch_bounds__(ps::W<PH>::NTH) void ssd_scan_kernel(ScanArgs a) {
  using namespace ps;
  using Wd = W<PH>;
  using Slot = typename Wd::template Slot<BLO>;
  constexpr int NWV = Wd::NWV, NTH = Wd::NTH, PT = Wd::PT, WPH = Wd::WPH;
  __shared__ Slot rs[3];
  // per head of the block (the two waves of a head write the same values):
  __shared__ float Sx[KH][256];     // running log2-decay from the chunk start (inclusive)
  __shared__ float Dx[KH][256];     // the chunk's dt
  __shared__ float Wx[KH][256];     // state-update weight of each token (see scan_dt)
  // readout scale of each token (output pass); with the B remainder, whose
  // rows take that room, the scales are computed per step
  __shared__ float Cx[BLO ? 1 : KH][256];
  // the output steps' C.B^T blocks, each computed once per workgroup one step
  // ahead (two buffers; lane l's four values of block b at [b][l])
  __shared__ f4 cbs[2][3][64];
  __shared__ _Float16 dtr[2][256 * 8];    // a chunk's dt rows as read (8 elements per token from the aligned base), two chunks
  __shared__ unsigned sh_ticket, sh_gen;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, q = lane >> 4;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hpg = a.H / a.G;
  const int nhb = (hpg + KH - 1) / KH;
  const int BG = a.B * a.G;
  const int HV = WPH * a.H;   // hand-off items per sequence and segment: (head, wave of the head)
  const int BHV = a.B * HV;

  // ---- claim a workgroup item: the XCD's own (sequence, group) partition first, segment-major
  if (tid == 0) {
    sh_gen = __hip_atomic_load(&a.ctrl[kCtrlGen], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned x0 = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 7u;   // HW_REG_XCC_ID
    for (int k = 0; k < 8; ++k) {
      const unsigned px = (x0 + k) & 7u;
      const int npairs = BG > (int)px ? (BG - (int)px + 7) / 8 : 0;
      const unsigned n = (unsigned)(npairs * nhb * a.nseg);
      if (n == 0) continue;
      unsigned* cnt = &a.ctrl[px * kCtrlStride];
      // (the XCD's own partition is claimed from at once; others are read first)
      if (k > 0 && __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) continue;
      const unsigned t = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t < n) {
        const int per_c = npairs * nhb;
        const int cc = (int)t / per_c, rem = (int)t - cc * per_c;
        const int gid = (int)px + 8 * (rem / nhb);
        sh_ticket = (unsigned)((cc * BG + gid) * nhb + rem % nhb);
        break;
      }
    }
  }
  // zero the slots: rows past a sequence's end are never loaded, and their
  // (unused) values must be finite
  {
    constexpr int SLOT16 = (int)(sizeof(Slot) / 16);
    u4* z = reinterpret_cast<u4*>(&rs[0]);
    for (int i = tid; i < 3 * SLOT16; i += NTH) z[i] = u4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  const unsigned ticket = __builtin_amdgcn_readfirstlane(sh_ticket);
  const unsigned gen = __builtin_amdgcn_readfirstlane(sh_gen);
  const unsigned tag = (gen & 0x3fffffffu) << 2;
  const int hblk = (int)(ticket % (unsigned)nhb);
  const int sg = (int)(ticket / (unsigned)nhb) / BG;   // segment (= chunk when nseg > 1)
  const int gid = (int)(ticket / (unsigned)nhb) - sg * BG;
  const int b = gid / a.G, g = gid - b * a.G;
  const int hin = hblk * KH + wid / WPH;
  const bool live = hin < hpg;                  // waves past the group's last head only load B and C
  const int h = g * hpg + (live ? hin : 0);
  const int half = wid % WPH;
  const int hb = b * a.H + h;
  const int bhv = b * HV + WPH * h + half;
  const unsigned item = (unsigned)(sg * BHV + bhv);
  const SeqRows span = seq_rows(a.seqlens, a.cu, b, a.L, a.T);
  const int len = __builtin_amdgcn_readfirstlane(span.len);
  const int ubase = __builtin_amdgcn_readfirstlane((int)span.base);
  const size_t xbase = a.xpk ? (size_t)ubase : (size_t)b * a.L;
  int c0 = sg * a.cps;                                          // first chunk of the segment
  int c1 = min(c0 + a.cps, a.nchunks);                          // one past its last chunk
  const bool last = sg + 1 == a.nseg;
  const bool pair = a.pair != 0;
  // wave-uniform scalars (a value still pending from a load before the step
  // loops would make the compiler wait for all memory operations inside them)
  const float Ah = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a.A[h] * kLog2e)));
  const float Dh = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a.D[h])));

  // buffer views of this sequence (the range ends at its last token)
  constexpr unsigned ES = 2;
  const unsigned xrow = (unsigned)a.xstride * ES;
  const unsigned grow = (unsigned)a.gstride * ES;
  const unsigned yrow = (unsigned)(a.H * P) * ES;
  const unsigned xspan = len > 0 && live ? (unsigned)(len - 1) * xrow + PH * ES : 0u;
  const unsigned yspan = len > 0 && live ? (unsigned)(len - 1) * yrow + PH * ES : 0u;
  const unsigned gspan = len > 0 ? (unsigned)(len - 1) * grow + N * ES : 0u;
  const u4 rx = rsrc_words(a.x + xbase * a.xstride + (size_t)h * P + PH * half, xspan);
  const u4 rb = rsrc_words(a.Bm + xbase * a.gstride + (size_t)g * N, gspan);
  const u4 rc4 = rsrc_words(a.Cm + xbase * a.gstride + (size_t)g * N, gspan);
  const unsigned lrow = (unsigned)a.gn * ES;   // remainder rows of B (fused conv)
  const u4 rbl = BLO ? rsrc_words(a.Blo + xbase * a.gn + (size_t)g * N, len > 0 ? (unsigned)(len - 1) * lrow + N * ES : 0u)
                     : u4{0u, 0u, 0u, 0u};
  const rsrc_t ry = mkr(a.y + ((size_t)ubase * a.H + h) * P + PH * half, yspan);
  // dt of the block's heads: token t's row starts sh0 + t dtld elements past
  // a 4-byte aligned base (dt needs only element alignment, any row stride)
  const int h0 = g * hpg + hblk * KH;
  const _Float16* const dt0 = a.dt + (size_t)ubase * a.dtld + h0;
  const int sh0 = (int)(((size_t)dt0 >> 1) & 1);
  const u4 rdt = rsrc_words(dt0 - sh0, len > 0 ? ((unsigned)(sh0 + (len - 1) * a.dtld + (a.H - h0)) * ES + 3u) & ~3u : 0u);
  float* const Sw = Sx[wid / WPH];
  float* const Dw = Dx[wid / WPH];
  float* const Ww = Wx[wid / WPH];
  float* const Cw = Cx[BLO ? 0 : wid / WPH];

  // steps of chunk c that hold tokens of this sequence
  auto steps_of = [&](int c) { return (min(max(len - c * a.Q, 0), a.Q) + TS - 1) / TS; };
  // every step of the segment, in order
  int ncv = min(max((len - c0 * a.Q + a.Q - 1) / a.Q, 0), c1 - c0);   // chunks with tokens

  // ---- loads of one step into a slot (this wave's share) ----------------------
  // (DX + DBC per operand loads per wave and step; the explicit waits count them)
  constexpr int DX = Wd::XI, DBC = Wd::BI;
  auto loads_per_step = [&](bool with_c) { return DX + DBC * ((with_c ? 2 : 1) + (BLO ? 1 : 0)); };
  // (a slot's LDS byte address from the slots' base: the slot index of a
  // step is a runtime value)
  const unsigned lds_rs = lds_addr(&rs[0]);
  const unsigned lds_dtr = lds_addr(&dtr[0][0]);
  constexpr unsigned kSlotB = (unsigned)sizeof(Slot);
  constexpr unsigned kOx = (unsigned)offsetof(Slot, x), kOb = (unsigned)offsetof(Slot, b),
                     kOc = (unsigned)offsetof(Slot, c), kObl = (unsigned)offsetof(Slot, bl);
  auto issue = [&](int si, int tok0, bool with_c) {
    const unsigned t0 = (unsigned)tok0;
    const unsigned base = lds_rs + (unsigned)si * kSlotB;
    constexpr int XU = Wd::XU;
#pragma unroll
    for (int i = 0; i < DX; ++i) {
      const int row = (64 / XU) * i + lane / XU, pk = lane % XU;
      dma16(rx, base + kOx + (unsigned)(2 * (TS * PH * wid + 512 * i)), (t0 + row) * xrow + 16u * (unsigned)(pk ^ Wd::xsw(row)));
    }
#pragma unroll
    for (int i = 0; i < DBC; ++i) {
      const int blk = wid * DBC + i;
      const int row = 4 * blk + (lane >> 4), pk = lane & 15;
      const unsigned go = (t0 + row) * grow + 16u * (unsigned)(pk ^ bsw(row));
      dma16(rb, base + kOb + 1024u * (unsigned)blk, go);
      if (with_c) dma16(rc4, base + kOc + 1024u * (unsigned)blk, go);
      if constexpr (BLO) dma16(rbl, base + kObl + 1024u * (unsigned)blk, (t0 + row) * lrow + 16u * (unsigned)(pk ^ bsw(row)));
    }
  };

  // ---- per chunk: dt and the running log2-decay (4 tokens per lane) ----------
  // A chunk's dt of the block's four heads goes into LDS with the step loads,
  // one chunk ahead (two buffers): per token the 16 aligned bytes from the
  // dword that holds head h0, four lanes per token (the four heads lie at
  // elements sh .. sh + 3 of them, sh the row's misalignment); each wave
  // then scans its own head.
  constexpr int DTI = 256 / 16 / NWV;    // dt loads per wave for a chunk of up to 256 tokens
  auto dt_sh = [&](int tok) { return (unsigned)(sh0 + tok * a.dtld); };   // element offset of a token's row
  const float dtbl = a.dt_sp && a.dt_bias
                         ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a.dt_bias[h])))
                         : 0.f;
  auto issue_dt = [&](int cc) {
#pragma unroll
    for (int i = 0; i < DTI; ++i) {
      const int li = wid * DTI + i;
      const int t = 16 * li + (lane >> 2);   // tokens past the chunk load rows of the next one (unused)
      dma4(rdt, lds_dtr + (unsigned)(cc & 1) * (unsigned)sizeof(dtr[0]) + 256u * (unsigned)li,
           (dt_sh(cc * a.Q + t) & ~1u) * ES + 4u * (unsigned)(lane & 3));
    }
  };
  // dt and the running log2-decay of chunk cc (its dt in LDS); a raw dt goes
  // through the softplus, and tokens past the sequence keep dt = 0 (the state
  // passes through them unchanged).  Per token i it also stores the weight
  // of x_i in the state update, w_i = dt_i 2^{S_ref - S_i}, with S_ref the
  // log2-decay at the end of i's 32-token step (output pass) or at the end of
  // the chunk (local-state pass), and, for the output pass, the readout scale
  // 2^{S_i - S_start} with S_start the log2-decay before i's step.  Both are
  // at most 1: only differences S_a - S_b with a later than b are
  // exponentiated.
  auto scan_dt = [&](int cc, bool out_pass) {
    const _Float16* dc = dtr[cc & 1];
    const int hw = wid / WPH;              // this wave's head in the block
    float d[4], v[4], run = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * lane + e;
      float u = (float)dc[8 * i + (int)(dt_sh(cc * a.Q + i) & 1u) + hw];
      if (a.dt_sp) u = dt_softplus_fast(u, dtbl);
      if (i >= a.Q || cc * a.Q + i >= len) u = 0.f;
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
    pre -= run;   // exclusive prefix of the lane totals
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * lane + e;
      if (i < a.Q) {
        Sw[i] = v[e] + pre;
        Dw[i] = d[e];
      }
    }
    // (the wave's LDS accesses complete in order: the reads below see the
    // stores above)
    const int step0 = (4 * lane) & ~(TS - 1);
    const float s_end = Sw[out_pass ? step0 + TS - 1 : min(a.Q, len - cc * a.Q) - 1];
    const float s_start = step0 ? Sw[step0 - 1] : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * lane + e;
      if (i < a.Q) {
        const float si = v[e] + pre;
        Ww[i] = d[e] * ex2(s_end - si);
        if (out_pass && !BLO) Cw[i] = ex2(si - s_start);
      }
    }
  };

  // ---- one 32-token step of the output pass ---------------------------------------
  // R: the state entering the step (S^T tiles), advanced to its end when
  // `advance`; y of the step is stored
  f4 R[NT][PT];   // (set to zero before the hand-off: unused by the local-state pass)

  // x rows s = 4q..4q+3 and 16+4q..+3, column p = 16 pt + lr (transposed reads)
  auto x_frag = [&](const _Float16* xs, int pt) -> h8 {
    const int k = 2 * pt + ((lr & 3) >> 1), o = 4 * (lr & 1);
    const int ra0 = 4 * q + (lr >> 2), ra1 = 16 + 4 * q + (lr >> 2);
    return cat(tr4(&xs[Wd::xo(ra0, k) + o]), tr4(&xs[Wd::xo(ra1, k) + o]));
  };
  // acc[nt][pt] += sum_s B[s, n] w_s x[s, p] over a slot's 32 tokens, with the
  // per-token weights w of the lane's tokens (4q..4q+3, 16+4q..16+4q+3)
  auto weigh_x = [&](const h8 (&xa)[PT], const float (&w)[8], h8 (&xw)[PT]) __attribute__((always_inline)) {
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
      for (int e = 0; e < 8; ++e) xw[pt][e] = (_Float16)__builtin_fmaf((float)xa[pt][e], w[e], 0.f);
  };
  // B^T fragments: rows n (tile nt), tokens s = 4q..4q+3 and 16+4q..+3 (transposed reads)
  auto bt_frag = [&](const _Float16* bs, int nt) -> h8 {
    const int k = (lr & 3) + 4 * (nt >> 1), o = 4 * (nt & 1);
    const int rb0 = 4 * q + (lr >> 2), rb1 = 16 + 4 * q + (lr >> 2);
    return cat(tr4(&bs[bo(rb0, k) + o]), tr4(&bs[bo(rb1, k) + o]));
  };
  // acc += B^T xw, with B as its binary16 high part plus remainder when the
  // remainder is staged
  auto update = [&](const Slot& sl, const h8 (&xw)[PT], f4 (&acc)[NT][PT]) __attribute__((always_inline)) {
    h8 bt[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bt[nt] = bt_frag(sl.b, nt);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) acc[nt][pt] = mfma16(bt[nt], xw[pt], acc[nt][pt]);
    if constexpr (BLO) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bt[nt] = bt_frag(sl.bl, nt);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[nt][pt] = mfma16(bt[nt], xw[pt], acc[nt][pt]);
    }
  };

  // state-update weights of the lane's tokens of the step at i0
  auto weights = [&](int i0, float (&w)[8]) {
    const f4 w0 = *reinterpret_cast<const f4*>(&Ww[i0 + 4 * q]);
    const f4 w1 = *reinterpret_cast<const f4*>(&Ww[i0 + 16 + 4 * q]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[i] = w0[i];
      w[4 + i] = w1[i];
    }
  };

  // C.B^T block b of a step, (s-tile, t-tile) = (0, 0), (0, 1), (1, 1): rows
  // s = 16 S + 4 q .. + 3 of column t = 16 T + lr per lane, into buffer buf
  auto cb_block = [&](const Slot& sl, int b, int buf) __attribute__((always_inline)) {
    const int S = b == 2 ? 1 : 0, T = b == 0 ? 0 : 1;
    h8 bb[KM], cc[KM];
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      bb[m] = *reinterpret_cast<const h8*>(&sl.b[bo(16 * S + lr, q + 4 * m)]);
      cc[m] = *reinterpret_cast<const h8*>(&sl.c[bo(16 * T + lr, q + 4 * m)]);
    }
    f4 acc1 = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < KM; ++m) acc1 = mfma16(bb[m], cc[m], acc1);
    cbs[buf][b][lane] = acc1;
  };

  // The step in four stages, ordered so that the LDS, the vector ALU and the
  // matrix cores overlap:
  // (1) reads of the C rows while the state is converted to the readout
  //     operand;
  // (2) the readout C.R, with the state decayed over the step and the
  //     update's operands (x, B^T, weights) read under its products;
  // (3) the state update R += sum_s w_s B_s x_s, with the reads of the C.B^T
  //     blocks (computed during the previous step) and of the outputs'
  //     per-token values, and the decay mask formed under it;
  // (4) the masked product and the outputs.
  // (The readout operand dies with the readout, before the update's
  // operands are read: fewer registers are live at once than with the
  // update first.)
  // The state always advances: after a pass's last step it is used only
  // when it is the sequence's final state.  Scheduling barriers keep the
  // stages in order.
  auto step = [&](const Slot& sl, int i0, int tok0, int cbuf) __attribute__((always_inline)) {
    const _Float16* xs = sl.x[wid];
    const float Sj_start = i0 ? Sw[i0 - 1] : 0.f;
    const float Sj_end = Sw[i0 + TS - 1];
    // (1) C rows t = 16 T + lr, n = 8 q + 32 m .. + 7; the readout operand:
    // the state rows p as binary16
    h8 cf[2][KM];
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int m = 0; m < KM; ++m) cf[T][m] = *reinterpret_cast<const h8*>(&sl.c[bo(16 * T + lr, q + 4 * m)]);
    h8 ra[PT][KM];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const f4 s0 = R[2 * m][pt], s1 = R[2 * m + 1][pt];
        ra[pt][m] = h8{(_Float16)s0[0], (_Float16)s0[1], (_Float16)s0[2], (_Float16)s0[3],
                       (_Float16)s1[0], (_Float16)s1[1], (_Float16)s1[2], (_Float16)s1[3]};
      }
    __builtin_amdgcn_sched_barrier(0);
    // (2) the readout C.R while the state decays over the step; the update's
    // operands (x, B^T, weights) read
    f4 yr[PT][2];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        yr[pt][T] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < KM; ++m) yr[pt][T] = mfma16(ra[pt][m], cf[T][m], yr[pt][T]);
      }
    const float dec = ex2(Sj_end - Sj_start);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) R[nt][pt] *= dec;
    h8 xa[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) xa[pt] = x_frag(xs, pt);
    float w[8];
    weights(i0, w);
    h8 bt[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bt[nt] = bt_frag(sl.b, nt);
    __builtin_amdgcn_sched_barrier(0);
    // (3) the state update R += sum_s w_s B_s x_s; the C.B^T blocks and per
    // output column t = 16 T + lr its log2-decay, readout scale and x rows
    // (p = 16 pt + 4 q .. + 3); the decay mask formed under the products
    h8 xw[PT];
    weigh_x(xa, w, xw);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) R[nt][pt] = mfma16(bt[nt], xw[pt], R[nt][pt]);
    if constexpr (BLO) {
      // the remainder of B's binary16 rounding
      h8 bl[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bl[nt] = bt_frag(sl.bl, nt);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) R[nt][pt] = mfma16(bl[nt], xw[pt], R[nt][pt]);
    }
    f4 cb[3];
#pragma unroll
    for (int b = 0; b < 3; ++b) cb[b] = cbs[cbuf][b][lane];
    float St[2], sc[2];
    h4 xr[2][PT];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const int tl = 16 * T + lr;
      St[T] = Sw[i0 + tl];
      if constexpr (!BLO) sc[T] = Cw[i0 + tl];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
        xr[T][pt] = *reinterpret_cast<const h4*>(&xs[Wd::xo(tl, 2 * pt + (q >> 1)) + 4 * (q & 1)]);
    }
    // The mask entry of (s, t), s <= t, is dt_s 2^{S_t - S_s} C_t.B_s.  It
    // factors as w_s 2^{S_t - S_end} with the update weight w_s = dt_s
    // 2^{S_end - S_s} <= dt_s and 2^{S_t - S_end} >= 1, both finite while the
    // step's decay stays within 2^-100; past that (rare) the entries are
    // formed one by one, each exponent clamped so that the masked ones (s > t)
    // stay finite.
    float v[3][4];
    if (__builtin_amdgcn_readfirstlane(Sj_start - Sj_end <= 100.f ? 1 : 0)) {
      float u[2];
#pragma unroll
      for (int T = 0; T < 2; ++T) u[T] = ex2(St[T] - Sj_end);
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        const int S = b == 2 ? 1 : 0, T = b == 0 ? 0 : 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[b][e] = cb[b][e] * (w[4 * S + e] * u[T]);
      }
    } else {
      float Ss[2][4], ds[2][4];
#pragma unroll
      for (int S = 0; S < 2; ++S) {
        const f4 sv = *reinterpret_cast<const f4*>(&Sw[i0 + 16 * S + 4 * q]);
        const f4 dv = *reinterpret_cast<const f4*>(&Dw[i0 + 16 * S + 4 * q]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Ss[S][e] = sv[e];
          ds[S][e] = dv[e];
        }
      }
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        const int S = b == 2 ? 1 : 0, T = b == 0 ? 0 : 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[b][e] = cb[b][e] * ds[S][e] * ex2(fminf(St[T] - Ss[S][e], 0.f));
      }
    }
    // causal: the off-diagonal block (s-tile 0, t-tile 1) holds only s < t
#pragma unroll
    for (int b = 0; b < 3; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (b != 1 && 4 * q + e > lr) v[b][e] = 0.f;
    h8 mf[2];
    mf[0] = h8{(_Float16)v[0][0], (_Float16)v[0][1], (_Float16)v[0][2], (_Float16)v[0][3],
               (_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
    mf[1] = h8{(_Float16)v[1][0], (_Float16)v[1][1], (_Float16)v[1][2], (_Float16)v[1][3],
               (_Float16)v[2][0], (_Float16)v[2][1], (_Float16)v[2][2], (_Float16)v[2][3]};
    if constexpr (BLO) {
#pragma unroll
      for (int T = 0; T < 2; ++T) sc[T] = ex2(St[T] - Sj_start);
    }
    __builtin_amdgcn_sched_barrier(0);
    // (4) masked product and the outputs y = sc C.R + (masked C.B^T) x + D x
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const int tl = 16 * T + lr;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const f4 yd = mfma16(xa[pt], mf[T], f4{0.f, 0.f, 0.f, 0.f});
        const int p0 = 16 * pt + 4 * q;
        h4 hv;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hv[e] = (_Float16)(__builtin_fmaf(sc[T], yr[pt][T][e], yd[e]) + Dh * (float)xr[T][pt][e]);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, hv), ry,
                                              (unsigned)(tok0 + tl) * yrow + (unsigned)p0 * ES, 0, 0);
      }
    }
  };


  // ---- streaming over a segment's steps, three slots in rotation -----------------
  // Steps are numbered over the segment (chunk c0 + k / J, step k % J).
  const int J = a.Q / TS;                       // steps per full chunk
  const int lgJ = __builtin_ctz((unsigned)J);   // J = 2, 4 or 8
  auto tok_of = [&](int k) { return (c0 + (k >> lgJ)) * a.Q + (k & (J - 1)) * TS; };
  int nsteps = 0;                               // steps with tokens
  if (ncv > 0) nsteps = (ncv - 1) * J + steps_of(c0 + ncv - 1);
  // The pass over the segment: the loads of its first chunk's dt and of its
  // first two steps are already in flight (with_c: x, B and C, else x and B);
  // per step k the loads of step k + 2 (and, at a chunk's first step, of the
  // next chunk's dt), then body(k, slot of k, slot of k + 1), then the
  // barrier that publishes step k + 1.  At a chunk boundary each wave scans
  // the next chunk's dt after that barrier (the scan overwrites only its
  // head's arrays, which no wave reads any more).
  // Explicit waits: vector memory operations complete in issue order, so a
  // wave waits until no more are outstanding than it issued after the ones
  // that must have landed.  Before the barrier that publishes step k + 1:
  // - local-state pass: the loads of step k + 1; issued after them were the
  //   stores of steps k - 1 and k (stores_per_step each, when this wave
  //   stores) and the loads of step k + 2;
  // - output pass: the loads of step k + 2 as well, whose C.B^T blocks are
  //   computed during step k + 1; issued after them were the stores of
  //   step k.
  // Operations the count leaves out (dt loads, hand-off traffic) only make it
  // wait longer.  The output pass starts with the blocks of step 0, computed
  // by waves 0-2 between two barriers; during step k, waves (k + 1 + w) mod 8
  // = 0, 1, 2 compute block 0, 1, 2 of step k + 1.
  // The start of a pass, which needs only its prologue's loads: the first
  // chunk's dt scan and (output pass) the C.B^T blocks of step 0.
  auto pass_head = [&](bool with_c) __attribute__((always_inline)) {
    const int D = loads_per_step(with_c);
    if (nsteps > 0) vm_wait(nsteps > 1 && !with_c ? D : 0);   // the dt and step 0's loads (output pass: step 1's too)
    slot_barrier();
    if (ncv > 0) scan_dt(c0, with_c);
    if (with_c && nsteps > 0) {
      if (wid < 3) cb_block(rs[0], wid, 0);
      slot_barrier();
    }
  };
  auto pass_steps = [&](bool with_c, int stores_per_step, auto&& body) __attribute__((always_inline)) {
    const int D = loads_per_step(with_c);
    auto one = [&](int k, int si) __attribute__((always_inline)) {
      const int kc = k & (J - 1), cc = c0 + (k >> lgJ);
      const int nn = si == 2 ? 0 : si + 1, nx = si == 0 ? 2 : si - 1;   // slots of steps k + 1, k + 2
      if (kc == 0 && cc + 1 < c0 + ncv) issue_dt(cc + 1);
      const bool more = k + 2 < nsteps;
      if (more) issue(nx, tok_of(k + 2), with_c);
      body(k, rs[si], rs[nn]);
      if (k + 1 < nsteps)
        vm_wait(with_c ? stores_per_step : (k > 0 ? stores_per_step : 0) + (more ? D : 0) + stores_per_step);
      slot_barrier();
      if (k + 1 < nsteps && kc == J - 1) scan_dt(cc + 1, with_c);
    };
    for (int k = 0, si = 0; k < nsteps; ++k, si = si == 2 ? 0 : si + 1) one(k, si);
  };
  auto pass = [&](bool with_c, int stores_per_step, auto&& body) __attribute__((always_inline)) {
    pass_head(with_c);
    pass_steps(with_c, stores_per_step, body);
  };
  // the first loads of a pass
  auto prologue = [&](bool with_c) {
    if (ncv > 0) issue_dt(c0);
    if (nsteps > 0) issue(0, tok_of(0), with_c);
    if (nsteps > 1) issue(1, tok_of(1), with_c);
  };

  // ---- phase 1: the segment's local state (every segment but the last) ----------
  // acc is kept relative to the end of the current chunk: it is decayed over
  // each new chunk before that chunk's tokens are added.  With two segments
  // (pair) the first skips this pass and the second runs it over the first
  // segment's chunks instead: its result, with the initial state, is the
  // second segment's carry-in, and no hand-off is needed.  (A local-state
  // step costs a third to a quarter of an output step, so the first segment
  // gets the larger share of the chunks: see the launch.)
  float segdec = 1.f;                           // decay over the segment
  f4 acc[NT][PT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) acc[nt][pt] = f4{0.f, 0.f, 0.f, 0.f};
  const int own_c0 = c0, own_c1 = c1, own_ncv = ncv, own_nsteps = nsteps;
  if (pair && last) {
    c0 = 0;
    c1 = a.cps;
    ncv = min(max((len + a.Q - 1) / a.Q, 0), c1);
    nsteps = ncv > 0 ? (ncv - 1) * J + steps_of(ncv - 1) : 0;
  }
  if (pair ? last : !last) {
    prologue(false);
    pass(false, 0, [&](int k, const Slot& sl, const Slot&) __attribute__((always_inline)) {
      const int kc = k & (J - 1), i0 = kc * TS;
      const int cc = c0 + (k >> lgJ);
      const float Send = Sw[min(a.Q, len - cc * a.Q) - 1];   // dt = 0 past the end: S constant there
      if (kc == 0) {
        const float dec = ex2(Send);
        segdec *= dec;
        if (k > 0) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[nt][pt] *= dec;
        }
      }
      if (live) {
        // every operand read before the products
        h8 xa[PT], xw[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) xa[pt] = x_frag(sl.x[wid], pt);
        float w[8];
        weights(i0, w);
        weigh_x(xa, w, xw);
        update(sl, xw, acc);
      }
    });
  }
  c0 = own_c0;
  c1 = own_c1;
  ncv = own_ncv;
  nsteps = own_nsteps;
  // ---- phase 2: carry-in over an indexed tree of segments (radix r = 2^lg) --------
  // With i = sg + 1 and block(i) = r^(number of trailing zero base-r digits of
  // i), segment sg publishes the aggregate of segments (i - block(i), i]
  // (1-based), and its carry-in is the initial state advanced through the
  // aggregates that tile [1, i-1], taken newest first, n_1 = i-1,
  // n_{k+1} = n_k - block(n_k):
  //   carry = F(n_1) + D(n_1) F(n_2) + D(n_1) D(n_2) F(n_3) + ... + (prod D) h0
  // (F: aggregate state, D: its decay).  The first (r-1) log_r(block(i)) of
  // them cover (i - block(i), i-1]: once they are folded in, the running sum
  // combined with the local state is this segment's own aggregate.  A segment
  // waits only on earlier ones (claimed before it), and the order of the sums
  // is fixed, so results do not depend on timing.
  //
  // A segment whose block is itself (i not a multiple of r) publishes its
  // local aggregate at once, before the output pass's first loads are issued,
  // and waits only for its own stores before it raises the flag; the others
  // publish after their first folds.  Aggregates are read two at a time (the
  // next one's loads in flight while the current one is added).
  // A16 (no final state asked for): an aggregate is stored as binary16,
  // scaled by a power of two chosen from the wave's largest magnitude so
  // that it lies in [2^14, 2^15), with the inverse scale after its 16 tiles
  // (8 KB per item instead of 16 KB: half the publish stores and fold
  // loads).  Only the readouts then see the aggregates, and a readout takes
  // the state as binary16 anyway; a final state would carry their rounding
  // (up to 2^-11 of its largest entry per aggregate), so calls that ask for
  // one keep the binary32 aggregates.
  constexpr unsigned ESZ = A16 ? 2u : 4u;
  constexpr unsigned kStBytes = (unsigned)(N * PH) * ESZ + (A16 ? 4u : 0u);
  constexpr unsigned kScaleOff = (unsigned)(N * PH) * 2u;
  auto st_off = [&](int nt, int pt) -> unsigned { return (unsigned)((nt * PT + pt) * 256 + lane * 4) * ESZ; };
  auto node_item = [&](int j) -> unsigned { return (unsigned)((j - 1) * BHV + bhv); };   // j: 1-based segment
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) R[nt][pt] = f4{0.f, 0.f, 0.f, 0.f};
  const int si = sg + 1;
  const int lg = a.tree_lg;
  const int t_in = ((1 << lg) - 1) * (__builtin_ctz((unsigned)si) / lg);   // aggregates inside this segment's block
  int nodes = 0, my_node = 0;
  if (!pair)
    for (int n = si - 1; n > 0; n -= 1 << (lg * (__builtin_ctz((unsigned)n) / lg)), ++nodes)
      if (lane == nodes) my_node = n;
  const int tb = t_in < nodes ? t_in : nodes;
  const bool early = !pair && !last && tb == 0;
  float scale = 1.f;                            // product of the decays folded in
  if (pair && last) {
    // the first segment's local state is the whole carry-in but for h0
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) R[nt][pt] = acc[nt][pt];
    scale = segdec;
  }
  // own aggregate (segdec R + local, its decay segdec scale) into the workspace
  auto publish_stores = [&]() __attribute__((always_inline)) {
    const rsrc_t r = mkr(a.agg + (size_t)item * (N * PH), kStBytes);
    if constexpr (A16) {
      f4 v[NT][PT];
      float m = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          v[nt][pt] = acc[nt][pt];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[nt][pt][k] = __builtin_fmaf(segdec, R[nt][pt][k], v[nt][pt][k]);
            m = fmaxf(m, fabsf(v[nt][pt][k]));
          }
        }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
      // biased exponent eb of the largest magnitude, clamped so that the
      // scale 2^(141 - eb) and its inverse are normal binary32 numbers
      const unsigned eb = min(max((__float_as_uint(m) >> 23) & 0xffu, 15u), 254u);
      const float sc = __uint_as_float((268u - eb) << 23), inv = __uint_as_float((eb - 14u) << 23);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          const h4 hv = h4{(_Float16)(v[nt][pt][0] * sc), (_Float16)(v[nt][pt][1] * sc),
                           (_Float16)(v[nt][pt][2] * sc), (_Float16)(v[nt][pt][3] * sc)};
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, hv), r, st_off(nt, pt), 0, kSc1);
        }
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(inv), r, kScaleOff, 0, kSc1);
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          f4 v = acc[nt][pt];
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = __builtin_fmaf(segdec, R[nt][pt][k], v[k]);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, st_off(nt, pt), 0, kSc1);
        }
    }
  };
  auto publish_flag = [&]() __attribute__((always_inline)) {
    // compiler-only fence: no data store moves past the flag store
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const unsigned long long f =
        ((unsigned long long)__float_as_uint(segdec * scale) << 32) | (unsigned long long)(tag | 1u);
    if (lane == 0) __hip_atomic_store(&a.flags[item], f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if (early && live) publish_stores();

  // the output pass's first loads, in flight during the hand-off
  prologue(true);
  if (early && live) {
    // the stores were issued before the prologue's loads and complete in
    // order with them: wait until only those loads may be outstanding
    const int DP = loads_per_step(true);
    vm_wait((ncv > 0 ? DTI : 0) + (nsteps > 0 ? DP : 0) + (nsteps > 1 ? DP : 0));
    publish_flag();
  }
  // The output pass's start (its first chunk's dt scan and step 0's C.B^T
  // blocks) needs no carry-in: unless this segment publishes after its first
  // folds, it runs now, while the aggregates it waits for are published.
  const bool late_publish = !pair && !last && !early;
  if (!late_publish) pass_head(true);

  if (live) {
    // wait until aggregates k0 .. k1-1 are published (one flag per lane, all
    // polled together); the flag word also holds the aggregate's decay
    float my_dec = 1.f;
    auto wait_group = [&](int k0, int k1) {
      const bool mine = lane >= k0 && lane < k1;
      const unsigned it = mine ? node_item(my_node) : 0u;
      unsigned spins = 0;
      while (true) {
        bool ready = true;
        if (mine) {
          const unsigned long long f = __hip_atomic_load(&a.flags[it], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ready = (unsigned)f == (tag | 1u);
          my_dec = __uint_as_float((unsigned)(f >> 32));
        }
        if (__ballot(!ready) == 0) break;
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
          if (lane == 0) __hip_atomic_fetch_or(&a.ctrl[kCtrlErr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
      // compiler-only fence: the aggregate loads stay after the poll
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    // an aggregate's tiles (and with A16 its inverse scale: one load group)
    using Tile = typename std::conditional<A16, h4, f4>::type;
    struct Node {
      Tile t[NT][PT];
      float inv;
    };
    auto load_node = [&](int k, Node& buf) __attribute__((always_inline)) {
      const int n = __builtin_amdgcn_readlane(my_node, k);
      const rsrc_t r = mkr(a.agg + (size_t)node_item(n) * (N * PH), kStBytes);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          if constexpr (A16)
            buf.t[nt][pt] = __builtin_bit_cast(h4, __builtin_amdgcn_raw_buffer_load_b64(r, st_off(nt, pt), 0, kSc1));
          else
            buf.t[nt][pt] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, st_off(nt, pt), 0, kSc1));
        }
      if constexpr (A16) buf.inv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, kScaleOff, 0, kSc1));
    };
    auto add_node = [&](int k, const Node& buf) __attribute__((always_inline)) {
      float f = scale;
      if constexpr (A16) f *= __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, buf.inv)));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
          for (int e = 0; e < 4; ++e) R[nt][pt][e] = __builtin_fmaf(f, (float)buf.t[nt][pt][e], R[nt][pt][e]);
      scale *= __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_dec), k));
    };
    if (tb > 0) {
      // (the local state is still live here: one aggregate at a time)
      wait_group(0, tb);
      for (int k = 0; k < tb; ++k) {
        Node b0;
        load_node(k, b0);
        add_node(k, b0);
      }
    }
    if (!pair && !last && !early) {
      publish_stores();
      __builtin_amdgcn_s_waitcnt(0);
      publish_flag();
    }
    if (nodes > tb) {
      wait_group(tb, nodes);
      // Eight at most in straight-line code, two buffers: the next
      // aggregate's loads are issued before the current one is added.  Loads
      // are issued unconditionally (an index past the last repeats it,
      // unused) and the code leaves as soon as the last one is added, so
      // that every wait counts exactly the loads issued after the ones being
      // added.  Deeper trees add the rest one at a time.
      // (scheduling barriers keep each load group ahead of the additions
      // that follow it)
      const int kl = nodes - 1;
      Node b0, b1;
      load_node(tb, b0);
      load_node(min(tb + 1, kl), b1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        add_node(tb + j, b0);
        if (tb + j + 1 > kl) break;
        load_node(min(tb + j + 2, kl), b0);
        __builtin_amdgcn_sched_barrier(0);
        add_node(tb + j + 1, b1);
        if (tb + j + 2 > kl) break;
        load_node(min(tb + j + 3, kl), b1);
        __builtin_amdgcn_sched_barrier(0);
      }
      for (int k = tb + 8; k < nodes; ++k) {
        Node bk;
        load_node(k, bk);
        add_node(k, bk);
      }
    }
    if (a.state_in) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          const int p = PH * half + 16 * pt + lr, n = ncol(nt, q);
          const f4 h0v = *reinterpret_cast<const f4*>(a.state_in + ((size_t)hb * P + p) * N + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) R[nt][pt][e] = __builtin_fmaf(scale, h0v[e], R[nt][pt][e]);
        }
    }
  }

  // ---- phase 3: outputs; R runs from the carry-in through the segment ---------------
  const bool want_state = last && a.state_out != nullptr;
  if (late_publish) pass_head(true);
  pass_steps(true, live ? 2 * PT : 0, [&](int k, const Slot& sl, const Slot& nsl) __attribute__((always_inline)) {
    if (live) step(sl, (k & (J - 1)) * TS, tok_of(k), k & 1);
    const int blk = (wid + k + 1) & 7;
    if (k + 1 < nsteps && blk < 3) cb_block(nsl, blk, (k + 1) & 1);
  });
  if (want_state && live) {
    // Staged through the slots (every wave has passed the pass's last
    // barrier, so none reads them any more) so that each store writes two
    // whole 512-byte state rows: per wave and p tile, 16 rows of N floats,
    // rows SR floats apart so that the tile writes of 16 rows fall on
    // distinct banks.  A wave reads back only what it wrote itself (its LDS
    // accesses complete in order).
    constexpr int SR = N + 4;
    static_assert(NWV * 16 * SR * sizeof(float) <= 3 * sizeof(Slot), "staging fits the slots");
    float* const stg = reinterpret_cast<float*>(&rs[0]) + wid * (16 * SR);
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<f4*>(&stg[lr * SR + ncol(nt, q)]) = R[nt][pt];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 2 * i + (lane >> 5), c = 4 * (lane & 31);
        const f4 v = *reinterpret_cast<const f4*>(&stg[row * SR + c]);
        *reinterpret_cast<f4*>(a.state_out + ((size_t)hb * P + PH * half + 16 * pt + row) * N + c) = v;
      }
    }
  }

  // ---- retire -------------------------------------------------------------------
  if (tid == 0) {
    const unsigned total = (unsigned)(a.nseg * BG * nhb);
    const unsigned done = __hip_atomic_fetch_add(&a.ctrl[kCtrlDone], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == total - 1) {
      for (int k = 0; k < 8; ++k) __hip_atomic_store(&a.ctrl[k * kCtrlStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctrl[kCtrlDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctrl[kCtrlGen], gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Launch of the streamed scan (binary16 I/O, N = 128, P = 64 are the
// caller's to check).  Segments: as many runs of consecutive chunks per
// sequence as keep every CU busy with one workgroup; inside a segment the
// state passes from step to step in registers, segment boundaries go
// through the hand-off tree.
hipError_t launch_ssd_scan(const ScanArgs& in, int cus, hipStream_t st) {
  using namespace ps;
  ScanArgs a = in;
  const int hpg = a.H / a.G;
  const long long slots = (long long)a.B * a.G * ((hpg + KH - 1) / KH);   // workgroups per segment index
  int nseg = a.nseg > 0 ? a.nseg : (int)(cus / slots);
  nseg = nseg < 1 ? 1 : (nseg > a.nchunks ? a.nchunks : nseg);
  a.cps = (a.nchunks + nseg - 1) / nseg;
  a.nseg = (a.nchunks + a.cps - 1) / a.cps;
  // Two segments: the second runs the first's local-state pass itself, so
  // the first takes the larger share of the chunks (and leaves at least
  // one): about 60 %, or 75 % with the B remainder, whose output steps cost
  // more against its local-state steps (measured at 8 chunks: 5 and 6).
  a.pair = a.nseg == 2;
  if (a.pair) a.cps = min(a.Blo ? (3 * a.nchunks + 3) / 4 : (3 * a.nchunks + 4) / 5, a.nchunks - 1);
  const long long wgs = (long long)a.nseg * slots;
  // every workgroup resident at once: the chain of dependent publishes is the
  // critical path (radix 8); otherwise aggregate traffic matters more (radix 4)
  a.tree_lg = wgs <= cus ? 3 : 2;
  // binary16 aggregates when no final state is asked for (see the kernel)
  const bool a16 = a.state_out == nullptr;
  if (a.Blo) {
    if (a16) ssd_scan_kernel<32, true, true><<<(unsigned)wgs, W<32>::NTH, 0, st>>>(a);
    else ssd_scan_kernel<32, true, false><<<(unsigned)wgs, W<32>::NTH, 0, st>>>(a);
  } else {
    if (a16) ssd_scan_kernel<32, false, true><<<(unsigned)wgs, W<32>::NTH, 0, st>>>(a);
    else ssd_scan_kernel<32, false, false><<<(unsigned)wgs, W<32>::NTH, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace m2

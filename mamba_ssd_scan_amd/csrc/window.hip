// Whole-window Mamba-2 scan in its chunked state-space-dual form, with an
// optional causal conv1d(4)+SiLU before it and a gated RMSNorm after it.
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
// Kernels:
//  * conv_silu_kernel (mixer input only): conv1d(4) + SiLU over the raw xBC
//    channels, streamed in prefetched batches of token rows per thread,
//    written to a workspace copy in the xBC layout; it also writes the conv
//    state out;
//  * ssd_window_group_kernel: the chunked scan (see the comment above it);
//  * gate_norm_kernel: the gated RMSNorm of the window's outputs, one
//    streaming pass over y and z;
//  * gated_norm_kernel: the norm finish from per-head partial sums, for the
//    one-token mixer step.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "gfx950_ops.h"
#include "ssd_scan.h"
#include "../../include/mamba2ssd.h"

namespace m2 {

constexpr int kP = 64;                     // head dim
// longest window the column scan takes (see the launch of the binary16 scan)
constexpr int kColscanMaxL = 768;
constexpr unsigned kSpinLimit = 1u << 22;  // bounded waits: an error flag instead of a hang
constexpr int kNormParts = 2;              // partial sums of g^2 per (token, head) handed to the norm finish

template <typename IO> struct WinArgs {
  int B, L, H, G, Q, nchunks;
  const IO* x;        // x rows: token stride xstride elements
  const IO* Bm;       // B rows: token stride gstride elements
  const IO* Cm;       // C rows: token stride gstride elements
  const _Float16* Blo; // binary16 B from the conv: what its rounding dropped, rows of gn (else null)
  int gn;
  int xstride, gstride;
  const IO* dt;
  long long dtld;     // dt rows: token stride in elements
  const float* A;
  const float* D;
  const float* state_in;
  float* state_out;
  const int* seqlens;
  IO* y;
  unsigned* ctrl;     // per-partition claim counters, done counter, generation, error
  unsigned long long* flags;   // per item: decay bits << 32 | generation tag | 1 once its aggregate is published
  float* agg;         // per item segment aggregate state (private layout)
  int tree_lg;        // log2 of the radix of the segment tree
  int cps;            // chunks per segment: one workgroup runs a segment's chunks in order
  int nseg;           // segments per sequence
  int dt_sp;          // dt is raw: dt_eff = softplus(dt + dt_bias[h])
  const float* dt_bias;
  const int* cu;      // packed layout: row offsets (B+1) of the sequences, else null
  int T;              // packed layout: rows of the caller's per-token tensors
  int xpk;            // x, B, C are the caller's packed rows (not the conv output)
};

// control block: eight claim counters and the done counter / generation /
// error word, each on its own 128-byte line
constexpr int kCtrlStride = 32;
constexpr int kCtrlDone = 8 * kCtrlStride;
constexpr int kCtrlGen = 9 * kCtrlStride;
constexpr int kCtrlErr = 10 * kCtrlStride;
constexpr int kCtrlBytes = 11 * kCtrlStride * 4;


// Workgroup barrier that orders LDS only.  __syncthreads() would also wait for
// every outstanding global load, which would drain the loads prefetched for
// the next step at each barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}


// ---------------------------------------------------------------------------
// Causal depthwise conv1d (width 4) + SiLU over raw xBC (the mixer's input
// projection output), as the mixer core applies it before the scan: for
// channel c and token t, u = b_c + sum_k w[c,k] xin[t-3+k, c] (tap 3 is the
// current token; tokens before the window come from the conv state, zeros
// when none is given), then u * sigmoid(u).  Each thread owns 8 consecutive
// channels over TT consecutive tokens and keeps the 3-token history in
// registers, so every raw row is read once (plus a 3-row halo per tile).
// Rows at or past a sequence's length read as zero; the thread that sees a
// sequence's last token writes the last 3 raw tokens as the conv state out.
constexpr int kConvTT = 32;  // tokens per thread
constexpr int kConvRB = 8;   // raw rows per batch; batch k+1 is loaded while batch k is computed

// 8 raw channels of one token in the input's own type (packed: 4 registers for f16).
template <typename IO> struct Raw8;
template <> struct Raw8<_Float16> {
  h8 v;
  __device__ __forceinline__ void bload(rsrc_t r, unsigned off) {
    v = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
  __device__ __forceinline__ void bstore(rsrc_t r, unsigned off) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, 0);
  }
  __device__ __forceinline__ void zero() { v = h8{}; }
  __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
  __device__ __forceinline__ void set(int e, float x) { v[e] = (_Float16)x; }
};
template <> struct Raw8<float> {
  f4 a, b;
  __device__ __forceinline__ void bload(rsrc_t r, unsigned off) {
    a = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    b = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
  }
  __device__ __forceinline__ void bstore(rsrc_t r, unsigned off) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, a), r, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, b), r, off + 16, 0, 0);
  }
  __device__ __forceinline__ void zero() { a = f4{}; b = f4{}; }
  __device__ __forceinline__ float operator[](int e) const { return e < 4 ? a[e] : b[e - 4]; }
  __device__ __forceinline__ void set(int e, float x) { if (e < 4) a[e] = x; else b[e - 4] = x; }
};

template <typename IO>
__global__ __launch_bounds__(256) void conv_silu_kernel(const IO* __restrict__ xBC, const float* __restrict__ w,
                                                        const float* __restrict__ bias, const IO* __restrict__ cs_in,
                                                        IO* __restrict__ cs_out, const int* __restrict__ seqlens,
                                                        const int* __restrict__ cu, IO* __restrict__ out, int B,
                                                        int L, int T, int Cd, long long ld,
                                                        _Float16* __restrict__ blo, int bbeg, int gn) {
  // a workgroup per (sequence, 32-token tile) and 256 groups of 8 channels:
  // the tile's rows are wave-uniform
  const int ntt = (L + kConvTT - 1) / kConvTT;
  const int tt = (int)(blockIdx.x % (unsigned)ntt), b = (int)(blockIdx.x / (unsigned)ntt);
  const int cc = (int)blockIdx.y * 256 + (int)threadIdx.x;
  if (cc >= Cd / 8) return;
  const int c0 = cc * 8, t0 = tt * kConvTT;
  const SeqRows span = seq_rows(seqlens, cu, b, L, T);
  const int len = span.len;
  constexpr unsigned ES = sizeof(IO);
  const unsigned voff = (unsigned)c0 * ES;      // this lane's channels within a row
  const unsigned rowb = (unsigned)Cd * ES;
  const IO* const seq0 = xBC + (size_t)span.base * (size_t)ld;
  // Row t >= 0 of these channels, through a buffer view of that row alone
  // (address and range in scalar registers): the view is empty at or past
  // the length, so those loads return zero without touching memory, and the
  // loads carry no branch, select or per-lane address arithmetic.  A whole
  // batch of rows is in flight at once.
  auto row = [&](int t, Raw8<IO>& v) { v.bload(mkr(seq0 + (size_t)t * (size_t)ld, t < len ? rowb : 0u), voff); };
  Raw8<IO> h[3], cur[kConvRB], nxt[kConvRB];              // h: the 3 raw rows before the batch
  if (tt > 0) {
#pragma unroll
    for (int k = 0; k < 3; ++k) row(t0 - 3 + k, h[k]);
  } else {                                                // tokens before the window: the conv state
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      if (cs_in) {
#pragma unroll
        for (int e = 0; e < 8; ++e) h[k].set(e, io<IO>::load1(cs_in + ((size_t)b * Cd + c0 + e) * 3 + k));
      } else {
        h[k].zero();
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kConvRB; ++k) row(t0 + k, cur[k]);
  float wk[4][8], bs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const f4 v = *reinterpret_cast<const f4*>(w + (size_t)(c0 + e) * 4);
    wk[0][e] = v[0]; wk[1][e] = v[1]; wk[2][e] = v[2]; wk[3][e] = v[3];
    bs[e] = bias ? bias[c0 + e] : 0.f;
  }
  auto put_state = [&](const Raw8<IO>& r0, const Raw8<IO>& r1, const Raw8<IO>& r2) {  // oldest first
    if (!cs_out) return;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      IO* d = cs_out + ((size_t)b * Cd + c0 + e) * 3;
      io<IO>::store1(d + 0, r0[e]);
      io<IO>::store1(d + 1, r1[e]);
      io<IO>::store1(d + 2, r2[e]);
    }
  };
  if (len == 0 && tt == 0) put_state(h[0], h[1], h[2]);
  IO* const dst = out + (size_t)b * L * Cd;
  const bool lo_here = blo != nullptr && c0 >= bbeg && c0 < bbeg + gn;
#pragma unroll
  for (int kb = 0; kb < kConvTT / kConvRB; ++kb) {
    const int tb = t0 + kb * kConvRB;
    if (tb >= L) break;
    if (kb + 1 < kConvTT / kConvRB) {
#pragma unroll
      for (int k = 0; k < kConvRB; ++k) row(tb + kConvRB + k, nxt[k]);
    }
#pragma unroll
    for (int k = 0; k < kConvRB; ++k) {
      const int t = tb + k;
      if (t >= L) break;
      const Raw8<IO>& r0 = k >= 3 ? cur[k - 3] : h[k];
      const Raw8<IO>& r1 = k >= 2 ? cur[k - 2] : h[k + 1];
      const Raw8<IO>& r2 = k >= 1 ? cur[k - 1] : h[2];
      Raw8<IO> o;
      float uo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float u = bs[e];
        u = __builtin_fmaf(wk[0][e], r0[e], u);
        u = __builtin_fmaf(wk[1][e], r1[e], u);
        u = __builtin_fmaf(wk[2][e], r2[e], u);
        u = __builtin_fmaf(wk[3][e], cur[k][e], u);
        uo[e] = u * __builtin_amdgcn_rcpf(1.f + __expf(-u));
        o.set(e, uo[e]);
      }
      o.bstore(mkr(dst + (size_t)t * Cd, rowb), voff);
      if constexpr (sizeof(IO) == 2) {
        // B's channels also leave what their binary16 copy drops, for the
        // scan's state contraction
        if (lo_here) {
          h8 lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) lo[e] = (_Float16)(uo[e] - (float)o.v[e]);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, lo), mkr(blo + ((size_t)b * L + t) * gn, (unsigned)gn * 2u),
                                                 (unsigned)(c0 - bbeg) * 2u, 0, 0);
        }
      }
      if (t == len - 1) put_state(r1, r2, cur[k]);
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) h[k] = cur[kConvRB - 3 + k];
#pragma unroll
    for (int k = 0; k < kConvRB; ++k) cur[k] = nxt[k];
  }
}

// ===========================================================================
// Chunked scan: one workgroup per (segment, sequence, group, block of KH heads
// of the group), one wave per (head, half of the head dim).  A segment is a
// run of consecutive chunks: inside it the state passes from chunk to chunk
// in registers, and only segment boundaries go through the hand-off tree.
// x, B and C are token rows with a given token stride: the caller's tensors,
// or the conv kernel's output in the xBC layout.
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
// over n, and so that a C fragment is one contiguous 16-byte read that hits
// distinct LDS banks across the wave:
//   tile nt, row 4j + e  <->  n = 8 j + 32 (nt / 2) + 4 (nt % 2) + e      (N >= 32)
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
static_assert(TS == 32 && PH == 32, "the x tiles are moved as 16 tokens x 4 chunks of 16 bytes per wave access");
// (four neighbouring lanes load one token's 64 contiguous bytes: global
//  coalescing outweighs the LDS bank conflicts of the matching tile writes)


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
// 16 bytes per lane from a buffer straight into LDS: lane i's data lands at
// dst + 16 i (device-coherent read)
__device__ __forceinline__ void ld16_to_lds(rsrc_t r, void* dst, unsigned off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, kSc1);
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
  // pitch (halfs) of the [s][n] B and C tiles, chosen so that the row reads
  // of 8 consecutive n per lane hit distinct LDS banks
  static constexpr int NP = N == 128 ? N + 16 : N + 8;
  struct Tiles {
    alignas(16) _Float16 b[TS * NP];     // [s][n] B as read
    alignas(16) _Float16 c[TS * NP];     // [t][n] C as read
    alignas(16) _Float16 x[NWV][TS * XP];   // per wave: [s][p] x as read
    alignas(16) _Float16 xw[NWV][TS * XP];  // per wave: x times the state weight of token s
    alignas(16) _Float16 blo[TS * NP];   // binary32 B: what its binary16 copy leaves out
  };
  // the step tiles are idle during the hand-off, where each wave lands one
  // aggregate state in LDS while another one is in flight to its registers
  union {
    Tiles t;
    alignas(16) float land[NWV][N * PH];
  } u;
  alignas(16) float S[NWV][256];       // per wave: running log2-decay from the chunk start (inclusive)
  alignas(16) _Float16 dts[NWV][256];
  alignas(16) float dtl[KH][256];      // a chunk's dt of the block's heads, as loaded by the whole workgroup
  unsigned ticket, gen;
};

// first state column of the 4-row group j of state tile nt: lane group j of
// k-step m reads n = 8 j + 32 m .. + 7, tiles 2m and 2m+1 hold its two halves
template <int N> __device__ __forceinline__ int ncol(int nt, int j) {
  if constexpr (N >= 32) return 8 * j + 32 * (nt >> 1) + 4 * (nt & 1);
  else return 4 * j;
}
}  // namespace wv


template <typename IO, int N, bool BLO>
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
      const unsigned n = (unsigned)(npairs * nhb * a.nseg);
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
  const int sg = (int)(ticket / (unsigned)nhb) / BG;   // segment
  const int gid = (int)(ticket / (unsigned)nhb) - sg * BG;
  const int b = gid / a.G, g = gid - b * a.G;
  const int hin = hblk * KH + (wid >> 1);       // head within the group
  const bool live = hin < hpg;                  // waves past the group's last head only help load B, C
  const int h = g * hpg + (live ? hin : 0);
  const int half = wid & 1;
  const int hb = b * a.H + h;                   // (sequence, head) index
  const int bhv = b * HV + 2 * h + half;
  const unsigned item = (unsigned)(sg * BHV + bhv);
  // rows of the caller's tensors: sequence b starts at row ubase; x, B and C
  // staged by the conv kernel keep the padded row b * L
  const SeqRows span = seq_rows(a.seqlens, a.cu, b, a.L, a.T);
  const int len = __builtin_amdgcn_readfirstlane(span.len);
  const int ubase = __builtin_amdgcn_readfirstlane((int)span.base);
  const size_t xbase = a.xpk ? (size_t)ubase : (size_t)b * a.L;
  const int cb = sg * a.cps;                    // the segment's first chunk
  // chunks of the segment that hold tokens of this sequence, and the steps of each
  const int ncv = min(max((len - cb * a.Q + a.Q - 1) / a.Q, 0), min(a.cps, a.nchunks - cb));
  auto steps_of = [&](int ci) { return (min(max(len - (cb + ci) * a.Q, 0), a.Q) + TS - 1) / TS; };
  const float Ah = a.A[h] * kLog2e;
  const float Dh = a.D[h];

  // buffer views of this sequence (range ends at its last token)
  const unsigned xrow = (unsigned)a.xstride * ES;      // bytes between tokens in x
  const unsigned grow = (unsigned)a.gstride * ES;      // in B, C
  const unsigned yrow = (unsigned)(a.H * kP) * ES;     // in y, z
  const unsigned xspan = len > 0 && live ? (unsigned)(len - 1) * xrow + PH * ES : 0u;
  const unsigned yspan = len > 0 && live ? (unsigned)(len - 1) * yrow + PH * ES : 0u;
  const unsigned gspan = len > 0 ? (unsigned)(len - 1) * grow + N * ES : 0u;
  const size_t seq_x = xbase * a.xstride + (size_t)h * kP + PH * half;
  const size_t seq_y = ((size_t)ubase * a.H + h) * kP + PH * half;
  const size_t seq_g = xbase * a.gstride + (size_t)g * N;
  const rsrc_t rx = mkr(a.x + seq_x, xspan);
  const rsrc_t rb = mkr(a.Bm + seq_g, gspan);
  const rsrc_t rc = mkr(a.Cm + seq_g, gspan);
  const rsrc_t ry = mkr(a.y + seq_y, yspan);
  // dt of the block's KH heads (the row's last heads bound the range)
  const int h0 = g * hpg + hblk * KH;
  const rsrc_t rdt = mkr(a.dt + (size_t)ubase * a.dtld + h0,
                         len > 0 ? (unsigned)((len - 1) * a.dtld + (a.H - h0)) * ES : 0u);
  float* const Sw = sm.S[wid];
  _Float16* const dtw = sm.dts[wid];
  _Float16* const xs = sm.u.t.x[wid];
  _Float16* const xws = sm.u.t.xw[wid];
  _Float16* const smb = sm.u.t.b;
  _Float16* const smblo = sm.u.t.blo;
  _Float16* const smc = sm.u.t.c;

  // ---- per-step operands ---------------------------------------------------
  // With binary32 I/O, x and B stay binary32 until staging: x is rounded to
  // binary16 once, after its weighting, and B goes to the state contraction
  // as a binary16 pair (high part and remainder), so that the final state
  // carries one binary16 rounding per term, as with binary16 inputs.
  // Binary16 B from the conv kernel comes with the remainder its rounding
  // dropped (BLO), for the same two-part contraction.
  constexpr bool F32IO = sizeof(IO) == 4;
  constexpr bool BSPLIT = F32IO || BLO;
  struct F8 { f4 a, b; };
  using xv_t = typename std::conditional<F32IO, F8, h8>::type;
  struct XB { xv_t x[XPL]; xv_t b[BK]; h8 c[BK]; h8 bl[BLO ? BK : 1]; };
  rsrc_t rbl = rb;
  if constexpr (BLO) rbl = mkr(a.Blo + xbase * (size_t)a.gn + (size_t)g * N, len > 0 ? (unsigned)((len - 1) * a.gn + N) * 2u : 0u);
  auto ldx = [&](xv_t& v, rsrc_t r, unsigned off) {
    if constexpr (F32IO) {
      v.a = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
      v.b = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
    } else {
      v = ldh<IO, 8>(r, off);
    }
  };
  auto fetch = [&](XB& r, int tok0, bool with_c) {   // the step starting at token tok0
    const unsigned tok = (unsigned)tok0;
#pragma unroll
    for (int k = 0; k < XPL; ++k) {
      const int s = (lane >> 2) + 16 * k, pc = lane & 3;   // token, 16-byte column chunk
      ldx(r.x[k], rx, (tok + s) * xrow + (unsigned)(pc * 8) * ES);
    }
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      const int id = tid + NTH * k, s = id / NCH, nc = id % NCH;
      if (id < TS * NCH) {
        const unsigned off = (tok + s) * grow + (unsigned)(nc * 8) * ES;
        ldx(r.b[k], rb, off);
        if constexpr (BLO) r.bl[k] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rbl, ((tok + s) * (unsigned)a.gn + (unsigned)(nc * 8)) * 2u, 0, 0));
        if (with_c) r.c[k] = ldh<IO, 8>(rc, off);
      }
    }
  };
  // The last segment publishes nothing, so it skips the local-state pass: its
  // final state is the running state of the output pass.
  const bool last = sg + 1 == a.nseg;
  // the first step's loads go out before the dt scan, so both latencies overlap
  XB xb;
  if (ncv > 0) fetch(xb, cb * a.Q, last);

  // ---- phase 0 (per chunk): dt and the running log2-decay over the chunk --
  // (4 tokens per lane); the dt of the next chunk is loaded while a chunk runs
  // The workgroup loads a chunk's dt together: thread tid takes head tid % 4
  // of the block for tokens tid / 4 + 128 e, so the four lanes of a token
  // read one cache line (a wave-by-wave load of one head each would touch
  // 64 lines per instruction, eight times over).  scan_dt shares them out.
  const int dh = tid & 3, dtok = tid >> 2;
  const float dtbl = a.dt_sp && a.dt_bias ? a.dt_bias[min(h0 + dh, a.H - 1)] : 0.f;
  auto load_dt = [&](int cc, float (&d)[2]) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = dtok + 128 * e;
      d[e] = i < a.Q ? ld1<IO>(rdt, (unsigned)((cc * a.Q + i) * a.dtld + dh) * ES) : 0.f;
      // a raw dt goes through the softplus; tokens past the sequence keep
      // dt = 0 (the state passes through them unchanged)
      if (a.dt_sp) d[e] = i < a.Q && cc * a.Q + i < len ? dt_softplus_fast(d[e], dtbl) : 0.f;
    }
  };
  auto scan_dt = [&](const float (&dl)[2]) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = dtok + 128 * e;
      if (i < a.Q) sm.dtl[dh][i] = dl[e];
    }
    __syncthreads();
    float d[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * lane + e;
      d[e] = i < a.Q ? sm.dtl[wid >> 1][i] : 0.f;
    }
    float v[4];
    float run = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
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
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  float dtv[2];
  if (ncv > 0) load_dt(cb, dtv);

  // stage step j: B (and C) as read, x as read (phase 3 only) and x weighted
  // by dt_s e^{Sref - S_s} for the state contraction
  auto stage = [&](const XB& r, int j, float Sref, bool with_c) {
    const int i0 = j * TS;
#pragma unroll
    for (int k = 0; k < XPL; ++k) {
      const int s = (lane >> 2) + 16 * k, pc = lane & 3;   // token, 16-byte column chunk
      const float w = (float)dtw[i0 + s] * ex2(Sref - Sw[i0 + s]);
      h8 xw, xh;
      if constexpr (F32IO) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xw[e] = (_Float16)(r.x[k].a[e] * w);
          xw[4 + e] = (_Float16)(r.x[k].b[e] * w);
          xh[e] = (_Float16)r.x[k].a[e];
          xh[4 + e] = (_Float16)r.x[k].b[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xw[e] = (_Float16)__builtin_fmaf((float)r.x[k][e], w, 0.f);   // one mixed-precision op
        xh = r.x[k];
      }
      *reinterpret_cast<h8*>(&xws[s * XP + pc * 8]) = xw;
      if (with_c) *reinterpret_cast<h8*>(&xs[s * XP + pc * 8]) = xh;
    }
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      const int id = tid + NTH * k, s = id / NCH, nc = id % NCH;
      if (id < TS * NCH) {
        if constexpr (F32IO) {
          h8 hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hi[e] = (_Float16)r.b[k].a[e];
            hi[4 + e] = (_Float16)r.b[k].b[e];
            lo[e] = (_Float16)(r.b[k].a[e] - (float)hi[e]);
            lo[4 + e] = (_Float16)(r.b[k].b[e] - (float)hi[4 + e]);
          }
          *reinterpret_cast<h8*>(&smb[s * NP + nc * 8]) = hi;
          *reinterpret_cast<h8*>(&smblo[s * NP + nc * 8]) = lo;
        } else {
          *reinterpret_cast<h8*>(&smb[s * NP + nc * 8]) = r.b[k];
          if constexpr (BLO) *reinterpret_cast<h8*>(&smblo[s * NP + nc * 8]) = r.bl[k];
        }
        if (with_c) *reinterpret_cast<h8*>(&smc[s * NP + nc * 8]) = r.c[k];
      }
    }
  };
  // acc[nt][pt] += sum_s B[s, n] (w_s x[s, p]) over the staged step (K = 32
  // tokens; lane group q takes tokens 4q..4q+3 and 16+4q..16+4q+3)
  auto state_mfma = [&](f4 (&acc)[NT][PT]) {
    h8 xf[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      const int col = 16 * pt + 4 * (lr & 3);
      xf[pt] = cat(tr4(&xws[(4 * q + (lr >> 2)) * XP + col]), tr4(&xws[(16 + 4 * q + (lr >> 2)) * XP + col]));
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = ncol<N>(nt, lr & 3);
      const h8 af = cat(tr4(&smb[(4 * q + (lr >> 2)) * NP + col]), tr4(&smb[(16 + 4 * q + (lr >> 2)) * NP + col]));
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) acc[nt][pt] = mfma16(af, xf[pt], acc[nt][pt]);
      if constexpr (BSPLIT) {
        const h8 al = cat(tr4(&smblo[(4 * q + (lr >> 2)) * NP + col]), tr4(&smblo[(16 + 4 * q + (lr >> 2)) * NP + col]));
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[nt][pt] = mfma16(al, xf[pt], acc[nt][pt]);
      }
    }
  };
  // 8 (or 4) n of row r of an LDS [s][n] tile at the n-slots of k-step m
  auto row8 = [&](const _Float16* tile, int r, int m) -> h8 {
    const _Float16* row = tile + r * NP;
    if constexpr (NV == 8) return *reinterpret_cast<const h8*>(row + 8 * q + 32 * m);
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
  float segdec = 1.f;                             // decay over the segment

  // ---- phase 1: local segment state ----------------------------------------
  // acc is kept relative to the end of the current chunk: it is decayed over
  // each new chunk before that chunk's tokens are added.
  if (!last) {
    for (int ci = 0; ci < ncv; ++ci) {
      const int cc = cb + ci;
      scan_dt(dtv);
      load_dt(ci + 1 < ncv ? cc + 1 : cb, dtv);   // the output pass starts over at the first chunk
      const float Send = Sw[a.Q - 1];
      const float dec = ex2(Send);
      segdec *= dec;
      if (ci > 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) acc[nt][pt] *= dec;
      }
      const int Jc = steps_of(ci);
      for (int j = 0; j < Jc; ++j) {
        stage(xb, j, Send, false);
        lds_barrier();
        // next: this chunk's next step, the next chunk's first, or the output pass's first
        if (j + 1 < Jc) fetch(xb, cc * a.Q + (j + 1) * TS, false);
        else if (ci + 1 < ncv) fetch(xb, (cc + 1) * a.Q, false);
        else fetch(xb, cb * a.Q, true);
        if (live) state_mfma(acc);
        lds_barrier();
      }
    }
  }

  // ---- phase 2: carry-in state over an indexed tree of segments (radix r = 2^lg)
  // With i = sg + 1 and block(i) = r^(number of trailing zero base-r digits of i),
  // segment sg publishes the aggregate of segments (i - block(i), i] (1-based), and
  // its carry-in is the initial state advanced through the aggregates that
  // tile [1, i-1].  Those aggregates are taken newest first,
  // n_1 = i-1, n_{k+1} = n_k - block(n_k):
  //   carry = F(n_1) + D(n_1) F(n_2) + D(n_1) D(n_2) F(n_3) + ... + (prod D) h0
  // (F: aggregate state, D: its decay), so the aggregates that are ready first
  // are folded in first.  The first (r-1) log_r(block(i)) of them cover
  // (i - block(i), i-1]: once they are folded in, the running sum combined
  // with the local state is this segment's own aggregate, published for later
  // segments.  A segment waits only on earlier ones (claimed before it), and the
  // order of the sums is fixed, so results do not depend on timing.  A larger
  // radix means fewer dependent publishes (shorter latency chain) and more
  // aggregate loads (more traffic).
  // hand-off states: per item N*PH floats, tile-major, 16 contiguous bytes per lane
  constexpr unsigned kStBytes = (unsigned)(N * PH) * 4u;
  auto st_off = [&](int nt, int pt) -> unsigned { return (unsigned)((nt * PT + pt) * 256 + lane * 4) * 4u; };
  auto node_item = [&](int j) -> unsigned { return (unsigned)((j - 1) * BHV + bhv); };   // j: 1-based segment

  f4 R[NT][PT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) R[nt][pt] = f4{0.f, 0.f, 0.f, 0.f};
  if (live) {
    const int i = sg + 1;
    const int lg = a.tree_lg;                             // tree radix 2^lg
    const int t = ((1 << lg) - 1) * (__builtin_ctz((unsigned)i) / lg);   // aggregates inside this segment's block
    float scale = 1.f;                                     // product of the decays folded in so far
    auto publish = [&]() {                                 // own aggregate: (segdec R + local, segdec scale)
      const rsrc_t r = mkr(a.agg + (size_t)item * (N * PH), kStBytes);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          f4 v = acc[nt][pt];
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = __builtin_fmaf(segdec, R[nt][pt][k], v[k]);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, st_off(nt, pt), 0, kSc1);
        }
      __builtin_amdgcn_s_waitcnt(0);
      // compiler-only fence: no data store may be moved past the flag store
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      // one 64-bit word carries the aggregate's decay and the ready tag
      const unsigned long long f =
          ((unsigned long long)__float_as_uint(segdec * scale) << 32) | (unsigned long long)(tag | 1u);
      if (lane == 0) __hip_atomic_store(&a.flags[item], f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // the aggregates to fold, newest first: lane k holds the k-th (1-based chunk)
    int nodes = 0, my_node = 0;
    for (int n = i - 1; n > 0; n -= 1 << (lg * (__builtin_ctz((unsigned)n) / lg)), ++nodes)
      if (lane == nodes) my_node = n;
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
    // Aggregates k0 .. k1-1 are folded with two in flight: even positions land
    // in registers, odd ones in this wave's LDS area (direct loads, 1 KB per
    // instruction in the same lane order as the state tiles).
    float* const land = sm.u.land[wid];
    auto node_rsrc = [&](int k) {
      const int n = __builtin_amdgcn_readlane(my_node, k);
      return mkr(a.agg + (size_t)node_item(n) * (N * PH), kStBytes);
    };
    auto to_regs = [&](f4 (&F)[NT][PT], int k) {
      const rsrc_t r = node_rsrc(k);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
          F[nt][pt] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, st_off(nt, pt), 0, kSc1));
    };
    auto to_lds = [&](int k) {
      const rsrc_t r = node_rsrc(k);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
          ld16_to_lds(r, land + (nt * PT + pt) * 256, st_off(nt, pt));
    };
    auto dec_of = [&](int k) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_dec), k));
    };
    auto add_regs = [&](const f4 (&F)[NT][PT], int k) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
          for (int e = 0; e < 4; ++e) R[nt][pt][e] = __builtin_fmaf(scale, F[nt][pt][e], R[nt][pt][e]);
      scale *= dec_of(k);
    };
    auto add_lds = [&](int k) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          const f4 v = *reinterpret_cast<const f4*>(land + (nt * PT + pt) * 256 + lane * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) R[nt][pt][e] = __builtin_fmaf(scale, v[e], R[nt][pt][e]);
        }
        __builtin_amdgcn_sched_barrier(0);   // a few LDS reads at a time: no register peak
      }
      scale *= dec_of(k);
    };
    // the first t aggregates are this segment's block (the local state is still
    // live there: one at a time), then the own aggregate is published and the
    // rest are folded two in flight
    const int tb = t < nodes ? t : nodes;
    if (tb > 0) {
      wait_group(0, tb);
      for (int k = 0; k < tb; ++k) {
        f4 F[NT][PT];
        to_regs(F, k);
        add_regs(F, k);
      }
    }
    if (!last) publish();
    if (nodes > tb) {
      wait_group(tb, nodes);
      f4 F[NT][PT];
      to_regs(F, tb);
      if (tb + 1 < nodes) to_lds(tb + 1);
      for (int k = tb; k < nodes; k += 2) {
        add_regs(F, k);
        if (k + 2 < nodes) to_regs(F, k + 2);
        if (k + 1 < nodes) {
          add_lds(k + 1);
          if (k + 3 < nodes) to_lds(k + 3);
        }
      }
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
  }

  // the hand-off's landing areas overlay the step tiles
  lds_barrier();

  // ---- phase 3: outputs ------------------------------------------------------
  // R runs from the carry-in through every chunk of the segment
  for (int ci = 0; ci < ncv; ++ci) {
  const int t0 = (cb + ci) * a.Q;
  scan_dt(dtv);
  if (ci + 1 < ncv) load_dt(cb + ci + 1, dtv);
  const int Jv = steps_of(ci);
  const bool more = ci + 1 < ncv;                 // the state carries into the next chunk
  for (int j = 0; j < Jv; ++j) {
    const int i0 = j * TS;
    const float Sj_start = j ? Sw[i0 - 1] : 0.f;
    const float Sj_end = Sw[i0 + TS - 1];
    stage(xb, j, Sj_end, true);
    lds_barrier();
    if (j + 1 < Jv) fetch(xb, t0 + (j + 1) * TS, true);
    else if (more) fetch(xb, t0 + a.Q, true);
    if (live) {
      // C fragments: rows t = 16T + lr, n-slots of k-step m
      h8 cf[2][KM];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int m = 0; m < KM; ++m) cf[T][m] = row8(smc, 16 * T + lr, m);
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
            for (int m = 0; m < KM; ++m) mb[S] = mfma16(row8(smb, 16 * S + lr, m), cf[T][m], mb[S]);
            const f4 Ss = *reinterpret_cast<const f4*>(&Sw[i0 + 16 * S + 4 * q]);
            const h4 ds = *reinterpret_cast<const h4*>(&dtw[i0 + 16 * S + 4 * q]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // the exponent is clamped so that the masked entries (s > t) stay finite;
              // off-diagonal tiles (S < T) hold only s < t and need no mask
              const float v = mb[S][i] * (float)ds[i] * ex2(fminf(St - Ss[i], 0.f));
              mb[S][i] = (S < T || 4 * q + i <= lr) ? v : 0.f;
            }
          }
        }
        mf[T] = h8{(_Float16)mb[0][0], (_Float16)mb[0][1], (_Float16)mb[0][2], (_Float16)mb[0][3],
                   (_Float16)mb[1][0], (_Float16)mb[1][1], (_Float16)mb[1][2], (_Float16)mb[1][3]};
      }
      float sc[2];
#pragma unroll
      for (int T = 0; T < 2; ++T) sc[T] = ex2(Sw[i0 + 16 * T + lr] - Sj_start);
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
          const unsigned off = (unsigned)(t0 + i0 + tl) * yrow + (unsigned)p0 * ES;
          f4 out;
#pragma unroll
          for (int i = 0; i < 4; ++i) out[i] = __builtin_fmaf(sc[T], yr[i], yd[i]) + Dh * (float)xr[i];
          st4<IO>(ry, off, out);
        }
      }
      // running state for the next step: R <- e^{S_end_j - S_start_j} R + sum_s w_s B_s x_s
      // (after the last step of the last segment it is the window's final state)
      if (j + 1 < Jv || more || (last && a.state_out)) {
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
  }
  if (last && a.state_out && live) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const int p = PH * half + 16 * pt + lr, n = ncol<N>(nt, q);
        *reinterpret_cast<f4*>(a.state_out + ((size_t)hb * kP + p) * N + n) = R[nt][pt];
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

// Gated RMSNorm finish from partial sums: out = g * rsqrt(mean_group(g^2) +
// eps) * w, where y already holds g and the kNormParts partial sums of g^2 per
// (token, head) come from the kernel that produced g (the one-token mixer
// step).  One block per token.  The partials of a norm group are summed in a
// fixed order, so the result does not depend on timing: when a group spans
// whole waves of 64 partials, each wave sums its 64 with a butterfly and
// leaves one value per wave; otherwise each group's partials are added in
// index order by one thread.  Then every channel is rescaled in place.
template <typename IO>
__global__ __launch_bounds__(256) void gated_norm_kernel(IO* __restrict__ y, const float* __restrict__ normsum,
                                                         const float* __restrict__ nw, const int* __restrict__ seqlens,
                                                         const int* __restrict__ cu, int L, int T, int H, int group,
                                                         float eps) {
  constexpr int kMaxParts = 1024;                 // H * kNormParts <= 1024 is checked by the caller
  __shared__ float gs[256];
  __shared__ float part[kMaxParts];
  const int tok = blockIdx.x, b = tok / L, t = tok - b * L;   // (sequence, token) of the padded index
  const SeqRows span = seq_rows(seqlens, cu, b, L, T);
  if (t >= span.len) return;
  const int C = H * kP, ngr = C / group;
  const int np = H * kNormParts, seg = (group / kP) * kNormParts;   // partials per token, per group
  const float* ps = normsum + (size_t)tok * np;
  const bool wave_sums = seg % 64 == 0;
  for (int k0 = 0; k0 < np; k0 += 256) {
    const int k = k0 + (int)threadIdx.x;
    float v = k < np ? ps[k] : 0.f;
    if (wave_sums) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
      if ((threadIdx.x & 63) == 0 && k < np) part[k / 64] = v;
    } else if (k < np) {
      part[k] = v;
    }
  }
  __syncthreads();
  const int per = wave_sums ? seg / 64 : seg;     // values per group in `part`
  for (int gi = threadIdx.x; gi < ngr; gi += 256) {
    float acc = 0.f;
    for (int j = 0; j < per; ++j) acc += part[gi * per + j];
    gs[gi] = rsqrtf(acc / (float)group + eps);
  }
  __syncthreads();
  IO* row = y + (size_t)(span.base + t) * C;
  for (int c0 = threadIdx.x * 8; c0 < C; c0 += 256 * 8) {
    float v[8];
    io<IO>::load8(row + c0, v);
    const float r = gs[c0 / group];
    f4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) { lo[e] = v[e] * r * nw[c0 + e]; hi[e] = v[4 + e] * r * nw[c0 + 4 + e]; }
    io<IO>::store4(row + c0, lo);
    io<IO>::store4(row + c0 + 4, hi);
  }
}

// Gated RMSNorm of the window's outputs, one block per (padded) token: g =
// y * SiLU(z) over the token's C = H*P channels, out = g * rsqrt(mean of g^2
// over its norm group + eps) * w, written over y.  A thread takes 8 channels
// at a time, 2048 channels apart; the first kGateRegs of its runs keep g in
// registers between the sums and the rescale, later runs (C above 8192)
// recompute g from y and z, which the block has not yet overwritten.  The
// sums of g^2 are taken in a fixed order, so the result does not depend on
// timing: each wave sums a run of 512 channels (a group spans whole runs) or
// 8 lanes sum 64 channels (every group is whole heads of 64 channels), into
// one LDS slot per run; then each group's slots are added in channel order.
// Rows past a sequence's length are left untouched.
constexpr int kGateRegs = 4;
template <typename IO>
__device__ __forceinline__ void gate8(const IO* y, const IO* z, float (&g)[8]) {
  float v[8], u[8];
  io<IO>::load8(y, v);
  io<IO>::load8(z, u);
#pragma unroll
  for (int e = 0; e < 8; ++e) g[e] = v[e] * (u[e] * __builtin_amdgcn_rcpf(1.f + __expf(-u[e])));
}
template <typename IO>
__global__ __launch_bounds__(256) void gate_norm_kernel(IO* __restrict__ y, const IO* __restrict__ z,
                                                        const float* __restrict__ nw, const int* __restrict__ seqlens,
                                                        const int* __restrict__ cu, int L, int T, int C, int group,
                                                        float eps, long long zld) {
  constexpr int kMaxRuns = 1024;                  // C / 64 <= 1024 is checked by the caller
  __shared__ float gs[256];
  __shared__ float runs[kMaxRuns];
  const int tok = blockIdx.x, b = tok / L, t = tok - b * L;   // (sequence, token) of the padded index
  const SeqRows span = seq_rows(seqlens, cu, b, L, T);
  if (t >= span.len) return;
  const int ngr = C / group, lane = threadIdx.x & 63;
  IO* const yr = y + (size_t)(span.base + t) * C;
  const IO* const zr = z + (size_t)(span.base + t) * (size_t)zld;
  const bool wave_runs = group % 512 == 0;
  const int run = wave_runs ? 512 : 64;           // channels per slot
  auto add = [&](int c0, const float (&g)[8]) {   // every lane of the wave calls this together
    float sq = 0.f;
    if (c0 < C) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sq = __builtin_fmaf(g[e], g[e], sq);
    }
    sq += __shfl_xor(sq, 1, 64);
    sq += __shfl_xor(sq, 2, 64);
    sq += __shfl_xor(sq, 4, 64);
    if (wave_runs) {
      sq += __shfl_xor(sq, 8, 64);
      sq += __shfl_xor(sq, 16, 64);
      sq += __shfl_xor(sq, 32, 64);
      if (lane == 0 && c0 < C) runs[c0 / 512] = sq;
    } else if ((lane & 7) == 0 && c0 < C) {
      runs[c0 / 64] = sq;
    }
  };
  float g[kGateRegs][8];
#pragma unroll
  for (int k = 0; k < kGateRegs; ++k) {
    const int c0 = (int)threadIdx.x * 8 + 2048 * k;
    if (c0 < C) gate8<IO>(yr + c0, zr + c0, g[k]);
    add(c0, g[k]);
  }
  for (int k = kGateRegs; 2048 * k < C; ++k) {
    const int c0 = (int)threadIdx.x * 8 + 2048 * k;
    float gk[8];
    if (c0 < C) gate8<IO>(yr + c0, zr + c0, gk);
    add(c0, gk);
  }
  __syncthreads();
  const int per = group / run;                    // slots per group
  for (int gi = threadIdx.x; gi < ngr; gi += 256) {
    float acc = 0.f;
    for (int j = 0; j < per; ++j) acc += runs[gi * per + j];
    gs[gi] = rsqrtf(acc / (float)group + eps);
  }
  __syncthreads();
  auto put = [&](int c0, const float (&gk)[8]) {
    const float r = gs[c0 / group];
    const f4 w0 = *reinterpret_cast<const f4*>(nw + c0), w1 = *reinterpret_cast<const f4*>(nw + c0 + 4);
    f4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) { lo[e] = gk[e] * r * w0[e]; hi[e] = gk[4 + e] * r * w1[e]; }
    io<IO>::store4(yr + c0, lo);
    io<IO>::store4(yr + c0 + 4, hi);
  };
#pragma unroll
  for (int k = 0; k < kGateRegs; ++k) {
    const int c0 = (int)threadIdx.x * 8 + 2048 * k;
    if (c0 < C) put(c0, g[k]);
  }
  for (int c0 = (int)threadIdx.x * 8 + 2048 * kGateRegs; c0 < C; c0 += 2048) {
    float gk[8];
    gate8<IO>(yr + c0, zr + c0, gk);
    put(c0, gk);
  }
}

// The norm finish over ntok independent tokens of H*P channels, with the
// partial sums laid out as (token, head, kNormParts); the one-token mixer
// step uses it with one token per sequence.
hipError_t launch_gated_norm_tokens(int io_f16, void* y, const float* normsum, const float* nw, int ntok, int H,
                                    int group, float eps, hipStream_t st) {
  if (ntok <= 0) return hipSuccess;
  if (io_f16)
    gated_norm_kernel<_Float16><<<(unsigned)ntok, 256, 0, st>>>((_Float16*)y, normsum, nw, nullptr, nullptr, 1, ntok,
                                                                  H, group, eps);
  else
    gated_norm_kernel<float><<<(unsigned)ntok, 256, 0, st>>>((float*)y, normsum, nw, nullptr, nullptr, 1, ntok, H,
                                                               group, eps);
  return hipGetLastError();
}
int norm_parts_per_head() { return kNormParts; }

hipError_t launch_exact_window_f32(const mamba2_dims& d, const mamba2_window_io& io_, const float* x, const float* Bm,
                                   const float* Cm, long long xld, long long gld, int xpk, hipStream_t st);


// ---------------------------------------------------------------------------
struct WsLayout {
  size_t ctrl, flags, agg, convx, blo, total;
};
static WsLayout ws_layout(const mamba2_dims& d) {
  const size_t nchunks = ((size_t)d.seqlen + d.chunk - 1) / d.chunk;
  const size_t items = 2 * nchunks * d.batch * d.nheads;      // (chunk, sequence, head, half)
  const size_t es = d.io_dtype == MAMBA2_F16 ? 2 : 4;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  WsLayout w;
  w.ctrl = 0;
  w.flags = up(kCtrlBytes);
  w.agg = up(w.flags + items * 8);
  w.convx = up(w.agg + items * (size_t)d.dstate * (kP / 2) * 4);
  const size_t cd = (size_t)d.nheads * kP + 2 * (size_t)d.ngroups * d.dstate;
  w.blo = up(w.convx + (d.conv_width == 4 ? (size_t)d.batch * d.seqlen * cd * es : 0));
  // binary16 conv output: the remainder of its B channels
  const bool blo = d.conv_width == 4 && d.io_dtype == MAMBA2_F16;
  w.total = up(w.blo + (blo ? (size_t)d.batch * d.seqlen * d.ngroups * d.dstate * 2 : 0));
  return w;
}

size_t window_workspace_bytes(const mamba2_dims& d) { return ws_layout(d).total; }

// current device (0 when it cannot be read), for the per-device caches below
static int current_device() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess && dev >= 0 ? dev : 0;
}
constexpr int kMaxDevices = 64;

// compute units of the current device (cached per device; threads that race
// on a first query store the same value)
static int device_cus() {
  static std::atomic<int> cache[kMaxDevices];
  const int dev = current_device();
  if (dev >= kMaxDevices) return 256;
  const int c = cache[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <typename IO, int N, bool BLO>
static hipError_t launch_scan(const WinArgs<IO>& a, hipStream_t st) {
  const int hpg = a.H / a.G;
  const long long slots = (long long)a.B * a.G * ((hpg + wv::KH - 1) / wv::KH);   // workgroups per segment index
  // Resident workgroups per CU (the state lives in registers, so usually
  // one), cached per device as device_cus() is.
  static std::atomic<int> per_cu_cache[kMaxDevices];
  const int dev = current_device();
  int per_cu = dev < kMaxDevices ? per_cu_cache[dev].load(std::memory_order_relaxed) : 0;
  if (per_cu <= 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, ssd_window_group_kernel<IO, N, BLO>, 64 * wv::NWV, 0) !=
            hipSuccess || n <= 0)
      n = 1;
    per_cu = n;
    if (dev < kMaxDevices) per_cu_cache[dev].store(n, std::memory_order_relaxed);
  }
  const long long resident = (long long)device_cus() * per_cu;
  // Segments: as many consecutive-chunk runs per sequence as keep every
  // resident slot busy.  Chunks inside a segment pass the state in registers;
  // only segment boundaries go through the hand-off.
  WinArgs<IO> b = a;
  int nseg = a.nseg > 0 ? a.nseg : (int)(resident / slots);
  nseg = nseg < 1 ? 1 : (nseg > a.nchunks ? a.nchunks : nseg);
  b.cps = (a.nchunks + nseg - 1) / nseg;
  b.nseg = (a.nchunks + b.cps - 1) / b.cps;
  const unsigned wgs = (unsigned)(b.nseg * slots);
  // When every workgroup is resident at once, all segments reach the hand-off
  // together and the chain of dependent publishes is the critical path: a
  // radix-8 tree.  Otherwise segment levels are staggered in time and
  // aggregate traffic matters more: radix 4.
  b.tree_lg = wgs <= resident ? 3 : 2;
  ssd_window_group_kernel<IO, N, BLO><<<wgs, 64 * wv::NWV, 0, st>>>(b);
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_IO(const mamba2_dims& d, const mamba2_window_io& io_, void* ws, hipStream_t st) {
  const WsLayout wl = ws_layout(d);
  char* base = (char*)ws;
  WinArgs<IO> a;
  a.B = d.batch; a.L = d.seqlen; a.H = d.nheads; a.G = d.ngroups; a.Q = d.chunk;
  a.nchunks = (d.seqlen + d.chunk - 1) / d.chunk;
  a.nseg = d.segments;                           // 0: chosen at launch
  a.dt_sp = d.dt_softplus;
  a.dt_bias = d.dt_softplus ? io_.dt_bias : nullptr;
  a.dt = (const IO*)io_.dt; a.A = io_.A; a.D = io_.D;
  a.dtld = io_.dt_ld > 0 ? (long long)io_.dt_ld : (long long)d.nheads;
  a.state_in = io_.state_in; a.state_out = io_.state_out; a.seqlens = io_.seqlens;
  a.cu = io_.cu_seqlens;
  a.T = d.packed_tokens;
  a.xpk = io_.cu_seqlens != nullptr && d.conv_width == 0;
  a.y = (IO*)io_.y;
  a.ctrl = (unsigned*)(base + wl.ctrl);
  a.flags = (unsigned long long*)(base + wl.flags);
  a.agg = (float*)(base + wl.agg);
  if (d.conv_width == 4) {
    const int cd = d.nheads * kP + 2 * d.ngroups * d.dstate;
    IO* xc = (IO*)(base + wl.convx);
    // B's binary16 remainder keeps a final state within its tolerance (the
    // conv output is rounded to binary16 before the scan); without a final
    // state only y sees the state, through binary16 readouts, and the
    // remainder is neither written nor read
    _Float16* blo = sizeof(IO) == 2 && io_.state_out != nullptr ? (_Float16*)(base + wl.blo) : nullptr;
    const dim3 cgrid((unsigned)(d.batch * ((d.seqlen + kConvTT - 1) / kConvTT)), (unsigned)((cd / 8 + 255) / 256));
    conv_silu_kernel<IO><<<cgrid, 256, 0, st>>>(
        (const IO*)io_.xBC, io_.conv_w, io_.conv_b, (const IO*)io_.conv_state_in, (IO*)io_.conv_state_out,
        io_.seqlens, io_.cu_seqlens, xc, d.batch, d.seqlen, d.packed_tokens, cd,
        io_.xBC_ld > 0 ? io_.xBC_ld : (long long)cd, blo, d.nheads * kP, d.ngroups * d.dstate);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.x = xc;
    a.Bm = xc + d.nheads * kP;
    a.Cm = xc + d.nheads * kP + d.ngroups * d.dstate;
    a.xstride = a.gstride = cd;
    a.Blo = blo;
    a.gn = d.ngroups * d.dstate;
  } else {
    a.Blo = nullptr;
    a.gn = 0;
    a.x = (const IO*)io_.x; a.Bm = (const IO*)io_.B; a.Cm = (const IO*)io_.C;
    a.xstride = d.nheads * kP;
    a.gstride = d.ngroups * d.dstate;
  }
  hipError_t e;
  if constexpr (sizeof(IO) == 4) {
    // binary32 I/O: the exact token-sequential form in binary32 (the chunked
    // form's MFMA operands are binary16 and would round binary32 inputs)
    e = launch_exact_window_f32(d, io_, a.x, a.Bm, a.Cm, a.xstride, a.gstride, d.conv_width == 4 ? 0 : 1, st);
  } else if (d.dstate == 128) {
    // binary16 x, B, C at N = 128 (from the fused conv: B with its remainder): the streamed scan
    ScanArgs sa;
    sa.B = a.B; sa.L = a.L; sa.H = a.H; sa.G = a.G; sa.Q = a.Q; sa.nchunks = a.nchunks;
    sa.x = a.x; sa.Bm = a.Bm; sa.Cm = a.Cm; sa.xstride = a.xstride; sa.gstride = a.gstride;
    sa.dt = a.dt; sa.dtld = a.dtld; sa.A = a.A; sa.D = a.D;
    sa.state_in = a.state_in; sa.state_out = a.state_out; sa.seqlens = a.seqlens; sa.cu = a.cu; sa.T = a.T;
    sa.xpk = a.xpk; sa.y = a.y; sa.ctrl = a.ctrl; sa.flags = a.flags; sa.agg = a.agg;
    sa.nseg = a.nseg; sa.cps = 0; sa.tree_lg = 3; sa.dt_sp = a.dt_sp; sa.dt_bias = a.dt_bias;
    sa.Blo = a.Blo; sa.gn = a.gn;
    // One round of column-scan workgroups (2 x heads x sequences at most
    // one per compute unit) over short windows: the segmented scan would run
    // too few workgroups there (one chunk), or a hand-off between short
    // segments.  Measured on the 8B layer shape at batch 1 (column against
    // segmented): 16 against 27 us at L = 256, 26 against 35 us at 512, 36
    // against 40 us at 768, 41 against 40 us at 896, where the segmented
    // scan's larger steps begin to win.  Callers that ask for a segment
    // count get the segmented scan.
    const int cus = device_cus();
    if (a.Blo == nullptr && d.segments == 0 && 2LL * a.B * a.H <= cus && a.L <= kColscanMaxL) e = launch_ssd_colscan(sa, st);
    else e = launch_ssd_scan(sa, cus, st);
  } else {
    const bool blo = a.Blo != nullptr;   // only binary16 conv output carries a remainder
    switch (d.dstate) {
      case 16: e = blo ? launch_scan<IO, 16, true>(a, st) : launch_scan<IO, 16, false>(a, st); break;
      case 64: e = blo ? launch_scan<IO, 64, true>(a, st) : launch_scan<IO, 64, false>(a, st); break;
      default: e = blo ? launch_scan<IO, 128, true>(a, st) : launch_scan<IO, 128, false>(a, st); break;
    }
  }
  if (e != hipSuccess || d.norm_group == 0) return e;
  gate_norm_kernel<IO><<<(unsigned)(d.batch * d.seqlen), 256, 0, st>>>(
      (IO*)io_.y, (const IO*)io_.z, io_.norm_w, io_.seqlens, io_.cu_seqlens, d.seqlen, d.packed_tokens,
      d.nheads * kP, d.norm_group, d.norm_eps, io_.z_ld > 0 ? (long long)io_.z_ld : (long long)d.nheads * kP);
  return hipGetLastError();
}

// The workspace's error word, read after the stream's queued work and
// cleared when set.  Bit 0: some segment's bounded wait for an aggregate gave
// up (the outputs of that call are not valid).
__global__ void clear_word_kernel(unsigned* w) { *w = 0u; }

size_t window_control_bytes() { return (size_t)kCtrlBytes; }

hipError_t window_take_error(void* ws, unsigned* flags, hipStream_t st) {
  unsigned* w = (unsigned*)ws + kCtrlErr;
  unsigned v = 0;
  hipError_t e = hipMemcpyAsync(&v, w, sizeof(unsigned), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  if (v != 0u) {
    clear_word_kernel<<<1, 1, 0, st>>>(w);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return e;
  }
  *flags = v;
  return hipSuccess;
}

hipError_t launch_window(const mamba2_dims& d, const mamba2_window_io& io_, void* ws, hipStream_t st) {
  if (d.io_dtype == MAMBA2_F16) return launch_IO<_Float16>(d, io_, ws, st);
  return launch_IO<float>(d, io_, ws, st);
}

}  // namespace m2

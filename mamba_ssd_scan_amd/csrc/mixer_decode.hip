// Full one-token mixer step: the generation-time path of one Mamba-2 layer's
// mixer core for a batch of sequences, in one kernel.
//
//   1. causal depthwise conv1d (width 4) + SiLU over this token's raw x|B|C
//      channels, with the 3-token raw history (the convolution cache counted
//      in section "Storage and runtime memory" of page
//      "Mamb2_8B_FP4_Recall_SQ3.25") rolled by one token in place;
//   2. the selective state-space step of the decode kernel
//      (S <- exp(dt A) S + dt x (outer) B, y = S.C + D x), with the same
//      binary32 contract and binary16 store for a binary16 resident state
//      (section "Representation", paragraph "State");
//   3. the gated RMSNorm out = g / sqrt(mean(g^2) + eps) * w, g = y silu(z),
//      over groups of norm_group consecutive channels (section "Compatible
//      reference environment" pins an RMSNorm configuration), or y as is.
//
// Work split: one 256-thread workgroup per (sequence, head), as in the decode
// kernel.  Each workgroup convolves its head's P x channels and its group's
// 2N B and C channels (the heads of a group recompute the same B and C, a
// few hundred fmas, instead of waiting for one another), keeps the results
// in LDS in the I/O type's precision (as the window path stages its conv
// output) and streams the head's P x N state once.
//
// The B and C history of a group is read by all of its heads, so it is rolled
// by the head that arrives last at a (sequence, group) counter in the
// workspace, after every head has read it; the counter wraps back to zero for
// the next call.
//
// The norm spans norm_group / P heads, that is several workgroups.  Each head
// writes g = y silu(z) into y (I/O type) and the sums of g^2 over its two
// halves; the norm-finish kernel of the window source then finishes every
// sequence's token on the same stream.  (Finishing inside this
// kernel, by the last head of each norm group, needs every head to wait for
// its stores and an atomic before it retires; measured at 64 sequences that
// costs more than the second launch.)
#include <mutex>

#include "state_io.h"
#include "../../include/mamba2ssd.h"

namespace m2 {

// SiLU of the conv output u (taken in double precision: each tap product of a
// binary32 weight and an I/O value is exact in double, and the sum runs in
// the conv's tap order), rounded once to the I/O type (a few hundred channels
// per workgroup, so the cost is negligible).  The staged values are then the
// correctly rounded SiLU of the conv, not one that a binary32 evaluation may
// put on the other side of a rounding boundary.  Binary16 goes through
// binary32 with round-to-odd, which keeps the final round-to-nearest-even
// exact (binary32 carries 13 more fraction bits).
template <typename IO> __device__ __forceinline__ float silu_io(double u);
template <> __device__ __forceinline__ float silu_io<float>(double u) {
  const double v = u / (1.0 + exp(-u));
  return (float)v;
}
template <> __device__ __forceinline__ float silu_io<_Float16>(double u) {
  const double v = u / (1.0 + exp(-u));
  float f = (float)v;                                   // nearest binary32
  if ((double)f != v && (__float_as_uint(f) & 1u) == 0u) {  // inexact with an even last bit: the odd neighbour
    if (f == 0.f) f = __uint_as_float(v > 0.0 ? 1u : 0x80000001u);
    else f = __uint_as_float(__float_as_uint(f) + (fabs(v) > fabs((double)f) ? 1u : 0xffffffffu));
  }
  return (float)(_Float16)f;
}

template <typename IO> struct MixDecArgs {
  const IO* xBC;          // (B, Cd) this token's raw x | B | C
  const float* conv_w;    // (Cd, 4), tap 3 on the current token
  const float* conv_b;    // (Cd) or null
  IO* conv_state;         // (B, Cd, 3) raw history, oldest first, rolled in place
  const IO* dt;           // (B, H)
  const float* dt_bias;   // (H) or null
  int dt_sp;
  const float* A;
  const float* D;
  void* state;            // (B, H, P, N) resident type, in place
  const IO* z;            // (B, H*P), norm only
  const float* norm_w;    // (H*P), norm only
  IO* y;                  // (B, H*P)
  unsigned* cnt_grp;      // (B, G) arrivals
  float* normsum;         // (B, H, 2) sums of g^2 over each half of a head
  int H, G;
};

// Arrival at a counter of n: returns 0 .. n-1 in arrival order, and the n-th
// arrival (the one that gets n-1) leaves 0 behind for the next call (wrapping
// increment; unlike an add, the compiler keeps it a single atomic whose
// answer is awaited only where it is used).
__device__ __forceinline__ unsigned arrive(unsigned* cnt, unsigned n) {
  return __builtin_amdgcn_atomic_inc32(cnt, n - 1u, __ATOMIC_RELAXED, "agent");
}

// Workgroup barrier that orders LDS only (__syncthreads() would also wait for
// the global loads and the arrival atomic still in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename IO, typename ST, int N, bool NORM>
__global__ __launch_bounds__(256) void mixer_decode_kernel(const MixDecArgs<IO> a) {
  constexpr int P = 64;
  constexpr int LPR = N / 8;            // lanes per state row
  constexpr int RPP = 256 / LPR;        // rows covered by the workgroup per row slot
  constexpr int KR = RPP >= P ? 1 : P / RPP;   // row slots per thread: 4, 2, 1 for N = 128, 64, 16
  constexpr bool ROW_GUARD = RPP > P;   // N = 16: only the first P / 2 row groups have a row
  constexpr int NCONV = P + 2 * N;      // channels this workgroup convolves
  constexpr int NPT = (NCONV + 255) / 256;
  __shared__ float sx[P], sB[N], sC[N], sy[P];
  __shared__ unsigned sflag;
  const int H = a.H, G = a.G, hpg = H / G;
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh - b * H, g = h / hpg;
  const int HP = H * P, GN = G * N, Cd = HP + 2 * GN;
  const int tid = threadIdx.x;
  const int nc = (tid % LPR) * 8;
  const int r0 = tid / LPR;

  // ---- 0. this thread's state rows, in flight while the conv runs ----------------
  typename ST::T* S = (typename ST::T*)a.state + (size_t)bh * P * N;
  const bool has_row = !ROW_GUARD || r0 < P;
  typename ST::Raw raw[KR];
  if (has_row) {
#pragma unroll
    for (int k = 0; k < KR; ++k) raw[k] = ST::load_raw(S + (size_t)(r0 + k * RPP) * N + nc);
  }
  float d = io<IO>::load1(a.dt + bh);
  const float Ah = a.A[h], Dh = a.D[h];
  const float dtb = a.dt_sp && a.dt_bias ? a.dt_bias[h] : 0.f;

  // ---- 1. conv1d(4) + SiLU, raw history rolled --------------------------------------
  // new raw history of this thread's channels, stored after the state step
  // (x channels) or by the group's last head (B, C channels)
  float keep[NPT][3];
  int kc[NPT];
  IO rh[NPT][3], rx[NPT];                    // raw I/O values, widened after every load is out
  f4 w[NPT];
  float cb[NPT];
#pragma unroll
  for (int k = 0; k < NPT; ++k) {           // every load first, then the arithmetic
    // (no branch: a thread past the last channel reloads the head's first x
    // channel and discards it, so that no load waits for another)
    const int i = tid + 256 * k;
    const int c = i < P ? h * P + i
                        : (i < P + N ? HP + g * N + (i - P) : (i < NCONV ? HP + GN + g * N + (i - P - N) : h * P));
    const IO* cs = a.conv_state + ((size_t)b * Cd + c) * 3;
    rh[k][0] = cs[0];
    rh[k][1] = cs[1];
    rh[k][2] = cs[2];
    rx[k] = a.xBC[(size_t)b * Cd + c];
    w[k] = *reinterpret_cast<const f4*>(a.conv_w + (size_t)c * 4);
    cb[k] = a.conv_b ? a.conv_b[c] : 0.f;
    kc[k] = i < NCONV ? c : -1;
  }
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int i = tid + 256 * k;
    if (i < NCONV) {
      keep[k][0] = (float)rh[k][0];
      keep[k][1] = (float)rh[k][1];
      keep[k][2] = (float)rh[k][2];
      const float xk = (float)rx[k];
      double u = (double)cb[k];
      u = __builtin_fma((double)w[k][0], (double)keep[k][0], u);
      u = __builtin_fma((double)w[k][1], (double)keep[k][1], u);
      u = __builtin_fma((double)w[k][2], (double)keep[k][2], u);
      u = __builtin_fma((double)w[k][3], (double)xk, u);
      const float v = silu_io<IO>(u);
      if (i < P) sx[i] = v;
      else if (i < P + N) sB[i - P] = v;
      else sC[i - P - N] = v;
      // the rolled history: the two newest old taps and this token
      keep[k][0] = keep[k][1];
      keep[k][1] = keep[k][2];
      keep[k][2] = xk;
    }
  }
  // the step size and decay (the conv loads, issued after dt, have arrived)
  if (a.dt_sp) d = dt_softplus(d, dtb);
  // decay rounded once from a double-precision exponential (binary32 contract)
  const float dec = (float)exp((double)d * (double)Ah);
  lds_barrier();
  // Every thread has read its share of the group's B / C history (the values
  // are in LDS): count this head in.  The answer is only needed at the end.
  unsigned grp_old = 0;
  if (tid == 0) grp_old = arrive(a.cnt_grp + (size_t)b * G + g, (unsigned)hpg);

  // ---- 2. state-space step ------------------------------------------------------
  float bv[8], cv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bv[i] = sB[nc + i];
    cv[i] = sC[nc + i];
  }
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    const int p = r0 + k * RPP;
    const float xp = has_row ? sx[p] : 0.f;
    float sk[8];
    ST::widen(raw[k], sk);
    float acc = 0.f;
    {
#pragma clang fp contract(off)
      const float u = d * xp;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = u * bv[i];
        const float sn = __builtin_fmaf(dec, sk[i], v);
        sk[i] = sn;
        acc = __builtin_fmaf(sn, cv[i], acc);
      }
    }
    if (has_row) ST::store(S + (size_t)p * N + nc, sk);
    // every lane takes part in the row sum (lanes without a row add zeros)
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (has_row && (tid % LPR) == 0) sy[p] = acc + Dh * xp;
  }
  // this head's own x channels: nobody else reads their history
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    if (tid + 256 * k >= P) continue;
    IO* cs = a.conv_state + ((size_t)b * Cd + kc[k]) * 3;
    io<IO>::store1(cs, keep[k][0]);
    io<IO>::store1(cs + 1, keep[k][1]);
    io<IO>::store1(cs + 2, keep[k][2]);
  }
  lds_barrier();

  // ---- 3. output: y, or g = y silu(z) and its sums of g^2 for the norm ------------
  if (tid < P) {                        // wave 0: one channel per lane
    float out = sy[tid];
    if constexpr (NORM) {
      const float zz = io<IO>::load1(a.z + (size_t)bh * P + tid);
      out *= zz * __builtin_amdgcn_rcpf(1.f + __expf(-zz));
      float sq = out * out;
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) sq += __shfl_xor(sq, off, 64);
      if ((tid & 31) == 0) a.normsum[(size_t)bh * 2 + (tid >> 5)] = sq;
    }
    io<IO>::store1(a.y + (size_t)bh * P + tid, out);
  }
  // last head of the (sequence, group): roll the group's B / C history
  if (tid == 0) sflag = grp_old == (unsigned)(hpg - 1) ? 1u : 0u;
  lds_barrier();
  if (sflag) {
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      if (kc[k] < 0 || tid + 256 * k < P) continue;
      IO* cs = a.conv_state + ((size_t)b * Cd + kc[k]) * 3;
      io<IO>::store1(cs, keep[k][0]);
      io<IO>::store1(cs + 1, keep[k][1]);
      io<IO>::store1(cs + 2, keep[k][2]);
    }
  }
}

// ---------------------------------------------------------------------------
// Workspace: the (sequence, group) arrival counters (self-resetting) in a
// region of fixed size at its start, then the norm's partial sums.  The fixed
// region keeps every counter clear of the partial sums of any call, whatever
// its batch, so a workspace can serve calls of different sizes in turn.
hipError_t launch_gated_norm_tokens(int io_f16, void* y, const float* normsum, const float* nw, int ntok, int H,
                                    int group, float eps, hipStream_t st);
int norm_parts_per_head();

struct MixDecWs {
  size_t cnt_grp, normsum, total;
};
constexpr size_t kMixDecCounters = 16384;   // (sequence, group) counters at most
size_t mixer_decode_max_counters() { return kMixDecCounters; }
static MixDecWs mixdec_ws(const mamba2_dims& d) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  MixDecWs w;
  w.cnt_grp = 0;
  w.normsum = kMixDecCounters * 4;
  w.total = up(w.normsum + (d.norm_group > 0 ? (size_t)d.batch * d.nheads * 2 * 4 : 0));
  return w;
}

size_t mixer_decode_workspace_bytes(const mamba2_dims& d) { return mixdec_ws(d).total; }

template <typename IO, typename ST, int N>
static hipError_t launch_md(const mamba2_dims& d, const MixDecArgs<IO>& a, hipStream_t st) {
  const unsigned grid = (unsigned)(d.batch * d.nheads);
  if (d.norm_group > 0) mixer_decode_kernel<IO, ST, N, true><<<grid, 256, 0, st>>>(a);
  else mixer_decode_kernel<IO, ST, N, false><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <typename IO, typename ST>
static hipError_t launch_md_N(const mamba2_dims& d, const MixDecArgs<IO>& a, hipStream_t st) {
  switch (d.dstate) {
    case 16: return launch_md<IO, ST, 16>(d, a, st);
    case 64: return launch_md<IO, ST, 64>(d, a, st);
    default: return launch_md<IO, ST, 128>(d, a, st);
  }
}

template <typename IO>
static hipError_t launch_md_IO(const mamba2_dims& d, const mamba2_mixer_decode_io& io_, void* ws, hipStream_t st) {
  const MixDecWs wl = mixdec_ws(d);
  char* base = (char*)ws;
  MixDecArgs<IO> a;
  a.xBC = (const IO*)io_.xBC;
  a.conv_w = io_.conv_w;
  a.conv_b = io_.conv_b;
  a.conv_state = (IO*)io_.conv_state;
  a.dt = (const IO*)io_.dt;
  a.dt_sp = d.dt_softplus;
  a.dt_bias = d.dt_softplus ? io_.dt_bias : nullptr;
  a.A = io_.A;
  a.D = io_.D;
  a.state = io_.state;
  a.z = (const IO*)io_.z;
  a.norm_w = io_.norm_w;
  a.y = (IO*)io_.y;
  a.cnt_grp = (unsigned*)(base + wl.cnt_grp);
  a.normsum = (float*)(base + wl.normsum);
  a.H = d.nheads;
  a.G = d.ngroups;
  const hipError_t e = d.state_dtype == MAMBA2_F16 ? launch_md_N<IO, StateF16<8>>(d, a, st)
                                                   : launch_md_N<IO, StateF32<8>>(d, a, st);
  if (e != hipSuccess || d.norm_group == 0) return e;
  // the partials are laid out as the norm kernel reads them: two per head
  if (norm_parts_per_head() != 2) return hipErrorInvalidValue;
  return launch_gated_norm_tokens(sizeof(IO) == 2, io_.y, a.normsum, io_.norm_w, d.batch, d.nheads, d.norm_group,
                                  d.norm_eps, st);
}

hipError_t launch_mixer_decode(const mamba2_dims& d, const mamba2_mixer_decode_io& io_, void* ws, hipStream_t st) {
  if (d.io_dtype == MAMBA2_F16) return launch_md_IO<_Float16>(d, io_, ws, st);
  return launch_md_IO<float>(d, io_, ws, st);
}

// ---------------------------------------------------------------------------
// The step without a caller workspace, for callers that cannot allocate
// (graph capture, serving loops): the same kernels take their workspace from
// a fixed device array of this source file.  Each GPU holds its own copy of
// the array for the life of the process; host code reaches it only through
// the device address that hipGetSymbolAddress returns for the current device
// (the array's name is a host-side stand-in, not a device address).
//
// The array starts zeroed when the code object is loaded.  The arrival
// counters in it return to zero at the end of every call and the norm's
// partial sums are written before they are read, so every call finds it
// ready; calls that overlap on one GPU share it and race.
constexpr size_t kStaticScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t mixer_decode_static_scratch_bytes() { return kStaticScratchBytes; }

// Device address of the current device's scratch array, looked up once per
// device with that device current.
static hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_mixer_decode_static(const mamba2_dims& d, const mamba2_mixer_decode_io& io_, hipStream_t st) {
  void* ws = nullptr;
  const hipError_t e = static_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_mixer_decode(d, io_, ws, st);
}

}  // namespace m2

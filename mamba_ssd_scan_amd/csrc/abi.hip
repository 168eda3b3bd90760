// C ABI of the Mamba-2 mixer core: host-side validation and dispatch.
// Every request is checked here before anything is enqueued; a request the
// kernels do not cover returns MAMBA2_EUNSUPPORTED (there is no fallback).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/mamba2ssd.h"

namespace m2 {
hipError_t launch_decode(int io_f16, int state_f16, int N, const void* x, const void* dt, const void* Bm,
                         const void* Cm, const float* A, const float* D, void* state, void* y, int Bsz,
                         int H, int P, int G, int dt_sp, const float* dt_bias, hipStream_t st);
hipError_t launch_state_convert(int to_resident, int state_f16, const void* src, void* dst, size_t n,
                                hipStream_t st);
size_t window_workspace_bytes(const mamba2_dims& d);
size_t window_control_bytes();
hipError_t window_take_error(void* ws, unsigned* flags, hipStream_t st);
hipError_t launch_window(const mamba2_dims& d, const mamba2_window_io& io, void* ws, hipStream_t st);
hipError_t launch_requant_window(const mamba2_dims& d, const mamba2_window_io& io, hipStream_t st);
size_t mixer_decode_workspace_bytes(const mamba2_dims& d);
size_t mixer_decode_max_counters();
size_t scan_grad_workspace_bytes(const mamba2_dims& d);
hipError_t launch_scan_grad(const mamba2_dims& d, const mamba2_scan_grad_io& io, void* ws, hipStream_t st);
hipError_t launch_mixer_decode(const mamba2_dims& d, const mamba2_mixer_decode_io& io, void* ws, hipStream_t st);
hipError_t launch_mixer_decode_static(const mamba2_dims& d, const mamba2_mixer_decode_io& io, hipStream_t st);
size_t mixer_decode_static_scratch_bytes();
}  // namespace m2

namespace {

thread_local int32_t g_last_hip_error = 0;

int32_t hip_status(hipError_t e) {
  if (e == hipSuccess) return MAMBA2_OK;
  g_last_hip_error = (int32_t)e;
  return MAMBA2_EHIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
  const char* lo;
  const char* hi;
};
Range rng(const void* p, size_t bytes) { return Range{(const char*)p, (const char*)p + bytes}; }
bool overlap(Range a, Range b) {
  if (!a.lo || !b.lo || a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

size_t esize(int32_t dtype) { return dtype == MAMBA2_F16 ? 2 : 4; }

// Shape checks shared by every entry point.
int32_t check_common(const mamba2_dims* d) {
  if (!d) return MAMBA2_EINVAL;
  if (d->batch < 1 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 || d->ngroups < 1)
    return MAMBA2_EINVAL;
  if (d->nheads % d->ngroups != 0) return MAMBA2_EINVAL;
  if (d->io_dtype != MAMBA2_F16 && d->io_dtype != MAMBA2_F32) return MAMBA2_EINVAL;
  if (d->state_dtype != MAMBA2_F16 && d->state_dtype != MAMBA2_F32) return MAMBA2_EINVAL;
  if (d->dt_softplus != 0 && d->dt_softplus != 1) return MAMBA2_EINVAL;
  if (d->packed_tokens < 0) return MAMBA2_EINVAL;
  if (d->dstate != 16 && d->dstate != 64 && d->dstate != 128) return MAMBA2_EUNSUPPORTED;
  // Every tensor stays well inside 2^31 elements per sequence-head slice and
  // 2^62 bytes overall.
  if ((int64_t)d->headdim * d->dstate > (1 << 24)) return MAMBA2_EUNSUPPORTED;
  return MAMBA2_OK;
}

}  // namespace

extern "C" {

int32_t mamba2_abi_version(void) { return MAMBA2_ABI_VERSION; }

const char* mamba2_status_str(int32_t s) {
  switch (s) {
    case MAMBA2_OK: return "ok";
    case MAMBA2_EINVAL: return "invalid argument";
    case MAMBA2_EUNSUPPORTED: return "unsupported configuration";
    case MAMBA2_EALIGN: return "pointer not 16-byte aligned";
    case MAMBA2_EWORKSPACE: return "workspace missing or too small";
    case MAMBA2_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t mamba2_last_hip_error(void) { return g_last_hip_error; }

int32_t mamba2_decode_step(const mamba2_dims* d, const mamba2_decode_io* io, void* stream) {
  int32_t s = check_common(d);
  if (s != MAMBA2_OK) return s;
  if (!io) return MAMBA2_EINVAL;
  if (!io->x || !io->dt || !io->B || !io->C || !io->A || !io->D || !io->state || !io->y) return MAMBA2_EINVAL;
  if (d->headdim % 8 != 0) return MAMBA2_EUNSUPPORTED;
  if (!aligned16(io->x) || !aligned16(io->B) || !aligned16(io->C) || !aligned16(io->state) ||
      !aligned16(io->y))
    return MAMBA2_EALIGN;
  if (((uintptr_t)io->dt % esize(d->io_dtype)) || ((uintptr_t)io->A & 3) || ((uintptr_t)io->D & 3) ||
      ((uintptr_t)io->dt_bias & 3))
    return MAMBA2_EALIGN;
  const size_t es = esize(d->io_dtype);
  const size_t BH = (size_t)d->batch * d->nheads;
  const size_t BG = (size_t)d->batch * d->ngroups;
  Range ry = rng(io->y, BH * d->headdim * es);
  Range rs = rng(io->state, BH * d->headdim * d->dstate * esize(d->state_dtype));
  Range ins[] = {rng(io->x, BH * d->headdim * es), rng(io->dt, BH * es), rng(io->B, BG * d->dstate * es),
                 rng(io->C, BG * d->dstate * es), rng(io->A, d->nheads * 4), rng(io->D, d->nheads * 4),
                 rng(io->dt_bias, d->dt_softplus ? d->nheads * 4 : 0)};
  if (overlap(ry, rs)) return MAMBA2_EINVAL;
  for (const Range& r : ins)
    if (overlap(r, ry) || overlap(r, rs)) return MAMBA2_EINVAL;
  return hip_status(m2::launch_decode(d->io_dtype == MAMBA2_F16, d->state_dtype == MAMBA2_F16, d->dstate,
                                      io->x, io->dt, io->B, io->C, io->A, io->D, io->state, io->y, d->batch,
                                      d->nheads, d->headdim, d->ngroups, d->dt_softplus,
                                      d->dt_softplus ? io->dt_bias : nullptr, (hipStream_t)stream));
}

static int32_t state_convert(const mamba2_dims* d, const void* src, void* dst, int to_resident, void* stream) {
  int32_t s = check_common(d);
  if (s != MAMBA2_OK) return s;
  if (!src || !dst) return MAMBA2_EINVAL;
  if (!aligned16(src) || !aligned16(dst)) return MAMBA2_EALIGN;
  const size_t n = (size_t)d->batch * d->nheads * d->headdim * d->dstate;
  const size_t rb = n * esize(d->state_dtype);
  Range a = rng(src, to_resident ? n * 4 : rb), b = rng(dst, to_resident ? rb : n * 4);
  if (overlap(a, b)) return MAMBA2_EINVAL;
  return hip_status(m2::launch_state_convert(to_resident, d->state_dtype == MAMBA2_F16, src, dst, n,
                                             (hipStream_t)stream));
}

int32_t mamba2_state_load(const mamba2_dims* d, const float* src, void* dst, void* stream) {
  return state_convert(d, src, dst, 1, stream);
}

int32_t mamba2_state_store(const mamba2_dims* d, const void* src, float* dst, void* stream) {
  return state_convert(d, src, dst, 0, stream);
}

// Validation for the window scan.  Returns OK when the request is covered.
static int32_t check_window(const mamba2_dims* d) {
  int32_t s = check_common(d);
  if (s != MAMBA2_OK) return s;
  if (d->seqlen < 1) return MAMBA2_EINVAL;
  if (d->conv_width != 0 && d->conv_width != 4) return MAMBA2_EUNSUPPORTED;
  if (d->norm_group < 0) return MAMBA2_EINVAL;
  if (d->norm_group > 0 && (d->nheads * d->headdim) % d->norm_group != 0) return MAMBA2_EINVAL;
  // the norm kernels sum whole heads: a group must be a multiple of P
  if (d->norm_group > 0 && d->norm_group % d->headdim != 0) return MAMBA2_EUNSUPPORTED;
  if (d->norm_group > 0 && !(d->norm_eps >= 0.f)) return MAMBA2_EINVAL;
  // the norm finish keeps one scale per group of a token in LDS (256 slots)
  if (d->norm_group > 0 && (d->nheads * d->headdim) / d->norm_group > 256) return MAMBA2_EUNSUPPORTED;
  // the norm sums g^2 over runs of 64 channels in LDS (1024 slots)
  if (d->norm_group > 0 && (int64_t)d->nheads * d->headdim > 1024 * 64) return MAMBA2_EUNSUPPORTED;
  if (d->headdim != 64) return MAMBA2_EUNSUPPORTED;
  if (d->chunk != 64 && d->chunk != 128 && d->chunk != 256) return MAMBA2_EUNSUPPORTED;
  if (d->segments < 0) return MAMBA2_EINVAL;
  const int64_t nchunks = ((int64_t)d->seqlen + d->chunk - 1) / d->chunk;
  const int64_t items = nchunks * d->batch * d->nheads;
  if (items > (int64_t)1 << 29) return MAMBA2_EUNSUPPORTED;
  // one sequence's rows of x, B, C, y, z (or of xBC) are addressed with 32-bit
  // byte offsets
  const int64_t es = d->io_dtype == MAMBA2_F16 ? 2 : 4;
  const int64_t row = d->conv_width == 4 ? (int64_t)d->nheads * d->headdim + 2 * (int64_t)d->ngroups * d->dstate
                                         : (int64_t)d->nheads * d->headdim;
  if ((int64_t)d->seqlen * row * es >= ((int64_t)1 << 31)) return MAMBA2_EUNSUPPORTED;
  return MAMBA2_OK;
}

int32_t mamba2_window_workspace_bytes(const mamba2_dims* d, size_t* bytes) {
  if (!bytes) return MAMBA2_EINVAL;
  int32_t s = check_window(d);
  if (s != MAMBA2_OK) return s;
  *bytes = m2::window_workspace_bytes(*d);
  return MAMBA2_OK;
}

int32_t mamba2_conv_scan_window(const mamba2_dims* d, const mamba2_window_io* io, void* ws, size_t ws_bytes,
                                void* stream) {
  int32_t s = check_window(d);
  if (s != MAMBA2_OK) return s;
  if (!io) return MAMBA2_EINVAL;
  const size_t es = esize(d->io_dtype);
  const size_t Bsz = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate, G = d->ngroups;
  const size_t conv_dim = H * P + 2 * G * N;
  // required pointers
  if (!io->dt || !io->A || !io->D || !io->y) return MAMBA2_EINVAL;
  if (d->conv_width == 0 && (!io->x || !io->B || !io->C)) return MAMBA2_EINVAL;
  if (d->conv_width == 4 && (!io->xBC || !io->conv_w)) return MAMBA2_EINVAL;
  if (d->norm_group > 0 && (!io->z || !io->norm_w)) return MAMBA2_EINVAL;
  // packed layout: row offsets instead of lengths
  if ((d->packed_tokens > 0) != (io->cu_seqlens != nullptr) || (io->cu_seqlens && io->seqlens))
    return MAMBA2_EINVAL;
  // xBC rows: dense, or a stride of at least conv_dim that keeps rows 16-byte aligned
  const size_t xld = d->conv_width == 4 && io->xBC_ld > 0 ? (size_t)io->xBC_ld : conv_dim;
  if (d->conv_width == 4 && io->xBC_ld < 0) return MAMBA2_EINVAL;
  if (d->conv_width == 4 && io->xBC_ld > 0) {
    if ((size_t)io->xBC_ld < conv_dim || io->xBC_ld > ((int64_t)1 << 40)) return MAMBA2_EINVAL;
    if ((xld * es) % 16) return MAMBA2_EALIGN;
  }
  // z and dt rows: dense, or strides of at least a row (z rows 16-byte aligned)
  const size_t zld = d->norm_group > 0 && io->z_ld > 0 ? (size_t)io->z_ld : H * P;
  if (d->norm_group > 0 && io->z_ld != 0) {
    if (io->z_ld < 0 || (size_t)io->z_ld < H * P || io->z_ld > ((int64_t)1 << 40)) return MAMBA2_EINVAL;
    if ((zld * es) % 16) return MAMBA2_EALIGN;
  }
  if (io->dt_ld < 0 || (io->dt_ld > 0 && ((size_t)io->dt_ld < H || io->dt_ld > ((int64_t)1 << 40))))
    return MAMBA2_EINVAL;
  const size_t dtld = io->dt_ld > 0 ? (size_t)io->dt_ld : H;
  if ((L - 1) * dtld * es + H * es >= ((size_t)1 << 31)) return MAMBA2_EUNSUPPORTED;   // one sequence's dt rows
  // alignment
  const void* vec[] = {io->x, io->B, io->C, io->xBC, io->z, io->y, io->state_in, io->state_out, io->conv_w,
                       io->norm_w};
  for (const void* p : vec)
    if (p && !aligned16(p)) return MAMBA2_EALIGN;
  if (((uintptr_t)io->dt % es) || ((uintptr_t)io->A & 3) || ((uintptr_t)io->D & 3) ||
      ((uintptr_t)io->seqlens & 3) || ((uintptr_t)io->conv_b & 3) || ((uintptr_t)io->conv_state_in % es) ||
      ((uintptr_t)io->conv_state_out % es) || ((uintptr_t)io->dt_bias & 3) || ((uintptr_t)io->cu_seqlens & 3))
    return MAMBA2_EALIGN;
  // workspace
  const size_t need = m2::window_workspace_bytes(*d);
  if (!ws || ws_bytes < need) return MAMBA2_EWORKSPACE;
  if ((uintptr_t)ws & 255) return MAMBA2_EALIGN;
  // aliasing: outputs against inputs and against each other
  const size_t tok = d->packed_tokens > 0 ? (size_t)d->packed_tokens : Bsz * L;
  Range outs[] = {rng(io->y, tok * H * P * es), rng(io->state_out, Bsz * H * P * N * 4),
                  rng(io->conv_state_out, d->conv_width ? Bsz * conv_dim * 3 * es : 0), rng(ws, need)};
  Range ins[] = {rng(io->x, d->conv_width ? 0 : tok * H * P * es),
                 rng(io->B, d->conv_width ? 0 : tok * G * N * es),
                 rng(io->C, d->conv_width ? 0 : tok * G * N * es),
                 rng(io->xBC, d->conv_width ? ((tok - 1) * xld + conv_dim) * es : 0),
                 rng(io->conv_w, d->conv_width ? conv_dim * 4 * 4 : 0),
                 rng(io->conv_b, d->conv_width ? conv_dim * 4 : 0),
                 rng(io->conv_state_in, d->conv_width ? Bsz * conv_dim * 3 * es : 0),
                 rng(io->dt, ((tok - 1) * dtld + H) * es), rng(io->A, H * 4), rng(io->D, H * 4),
                 rng(io->state_in, Bsz * H * P * N * 4), rng(io->seqlens, Bsz * 4),
                 rng(io->z, d->norm_group ? ((tok - 1) * zld + H * P) * es : 0),
                 rng(io->norm_w, d->norm_group ? H * P * 4 : 0),
                 rng(io->dt_bias, d->dt_softplus ? H * 4 : 0), rng(io->cu_seqlens, (Bsz + 1) * 4)};
  const size_t nout = sizeof(outs) / sizeof(outs[0]);
  for (size_t i = 0; i < nout; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return MAMBA2_EINVAL;
    for (size_t j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return MAMBA2_EINVAL;
  }
  return hip_status(m2::launch_window(*d, *io, ws, (hipStream_t)stream));
}

int32_t mamba2_window_take_error(void* ws, size_t ws_bytes, uint32_t* flags, void* stream) {
  if (!ws || !flags) return MAMBA2_EINVAL;
  if (ws_bytes < m2::window_control_bytes()) return MAMBA2_EWORKSPACE;
  if ((uintptr_t)ws & 255) return MAMBA2_EALIGN;
  unsigned v = 0;
  const int32_t s = hip_status(m2::window_take_error(ws, &v, (hipStream_t)stream));
  if (s != MAMBA2_OK) return s;
  *flags = v;
  return MAMBA2_OK;
}

int32_t mamba2_requant_window(const mamba2_dims* d, const mamba2_window_io* io, void* stream) {
  int32_t s = check_common(d);
  if (s != MAMBA2_OK) return s;
  if (d->seqlen < 1) return MAMBA2_EINVAL;
  if (!io) return MAMBA2_EINVAL;
  // plain x, B, C only: no fused conv, no norm
  if (d->conv_width != 0 || d->norm_group != 0) return MAMBA2_EUNSUPPORTED;
  if (d->headdim != 64) return MAMBA2_EUNSUPPORTED;
  const size_t es = esize(d->io_dtype);
  const size_t Bsz = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate, G = d->ngroups;
  if (!io->x || !io->B || !io->C || !io->dt || !io->A || !io->D || !io->y) return MAMBA2_EINVAL;
  if ((d->packed_tokens > 0) != (io->cu_seqlens != nullptr) || (io->cu_seqlens && io->seqlens))
    return MAMBA2_EINVAL;
  const void* vec[] = {io->B, io->C, io->state_in, io->state_out};
  for (const void* p : vec)
    if (p && !aligned16(p)) return MAMBA2_EALIGN;
  if (((uintptr_t)io->x % es) || ((uintptr_t)io->y % es) || ((uintptr_t)io->dt % es) || ((uintptr_t)io->A & 3) ||
      ((uintptr_t)io->D & 3) || ((uintptr_t)io->seqlens & 3) || ((uintptr_t)io->dt_bias & 3) ||
      ((uintptr_t)io->cu_seqlens & 3))
    return MAMBA2_EALIGN;
  if (io->dt_ld < 0 || (io->dt_ld > 0 && ((size_t)io->dt_ld < H || io->dt_ld > ((int64_t)1 << 40))))
    return MAMBA2_EINVAL;
  const size_t dtld = io->dt_ld > 0 ? (size_t)io->dt_ld : H;
  const size_t tok = d->packed_tokens > 0 ? (size_t)d->packed_tokens : Bsz * L;
  Range outs[] = {rng(io->y, tok * H * P * es), rng(io->state_out, Bsz * H * P * N * 4)};
  Range ins[] = {rng(io->x, tok * H * P * es), rng(io->B, tok * G * N * es), rng(io->C, tok * G * N * es),
                 rng(io->dt, ((tok - 1) * dtld + H) * es), rng(io->A, H * 4), rng(io->D, H * 4),
                 rng(io->state_in, Bsz * H * P * N * 4), rng(io->seqlens, Bsz * 4),
                 rng(io->dt_bias, d->dt_softplus ? H * 4 : 0), rng(io->cu_seqlens, (Bsz + 1) * 4)};
  for (const Range& o : outs)
    for (const Range& r : ins)
      if (overlap(o, r)) return MAMBA2_EINVAL;
  if (overlap(outs[0], outs[1])) return MAMBA2_EINVAL;
  return hip_status(m2::launch_requant_window(*d, *io, (hipStream_t)stream));
}

// Validation for the fused one-token mixer step.
static int32_t check_mixer_decode(const mamba2_dims* d) {
  int32_t s = check_common(d);
  if (s != MAMBA2_OK) return s;
  if (d->conv_width != 4) return MAMBA2_EUNSUPPORTED;
  if (d->headdim != 64) return MAMBA2_EUNSUPPORTED;
  const int64_t hp = (int64_t)d->nheads * d->headdim;
  if (d->norm_group < 0 || d->norm_group > hp) return MAMBA2_EINVAL;
  if (d->norm_group > 0 && (hp % d->norm_group != 0 || !(d->norm_eps >= 0.f))) return MAMBA2_EINVAL;
  if (d->norm_group > 0 && d->norm_group % d->headdim != 0) return MAMBA2_EUNSUPPORTED;
  // the norm finish keeps one scale per norm group of a token in LDS (256 slots)
  if (d->norm_group > 0 && hp / d->norm_group > 256) return MAMBA2_EUNSUPPORTED;
  // the norm finish stages two partial sums per head in LDS (1024 slots)
  if (d->norm_group > 0 && d->nheads > 512) return MAMBA2_EUNSUPPORTED;
  if ((int64_t)d->batch * d->nheads > ((int64_t)1 << 31) - 1) return MAMBA2_EUNSUPPORTED;
  // one arrival counter per (sequence, group) in the workspace's fixed region
  if ((int64_t)d->batch * d->ngroups > (int64_t)m2::mixer_decode_max_counters()) return MAMBA2_EUNSUPPORTED;
  return MAMBA2_OK;
}

int32_t mamba2_mixer_decode_workspace_bytes(const mamba2_dims* d, size_t* bytes) {
  if (!bytes) return MAMBA2_EINVAL;
  int32_t s = check_mixer_decode(d);
  if (s != MAMBA2_OK) return s;
  *bytes = m2::mixer_decode_workspace_bytes(*d);
  return MAMBA2_OK;
}

// Arguments of a fused one-token mixer step.  ws is the workspace the
// kernels will use (caller-owned, or null for the library's static one, in
// which case need is only checked against its size by the caller).
static int32_t check_mixer_decode_args(const mamba2_dims* d, const mamba2_mixer_decode_io* io, const void* ws,
                                       size_t need) {
  if (!io) return MAMBA2_EINVAL;
  const size_t es = esize(d->io_dtype);
  const size_t Bsz = d->batch, H = d->nheads, P = d->headdim, N = d->dstate, G = d->ngroups;
  const size_t cd = H * P + 2 * G * N;
  if (!io->xBC || !io->conv_w || !io->conv_state || !io->dt || !io->A || !io->D || !io->state || !io->y)
    return MAMBA2_EINVAL;
  if (d->norm_group > 0 && (!io->z || !io->norm_w)) return MAMBA2_EINVAL;
  if (!aligned16(io->conv_w) || !aligned16(io->state)) return MAMBA2_EALIGN;
  if (((uintptr_t)io->xBC % es) || ((uintptr_t)io->conv_state % es) || ((uintptr_t)io->dt % es) ||
      ((uintptr_t)io->z % es) || ((uintptr_t)io->y % es) || ((uintptr_t)io->conv_b & 3) ||
      ((uintptr_t)io->dt_bias & 3) || ((uintptr_t)io->A & 3) || ((uintptr_t)io->D & 3) ||
      ((uintptr_t)io->norm_w & 3))
    return MAMBA2_EALIGN;
  // outputs (y; state and conv_state in place; workspace) against inputs and
  // against each other
  Range outs[] = {rng(io->y, Bsz * H * P * es), rng(io->state, Bsz * H * P * N * esize(d->state_dtype)),
                  rng(io->conv_state, Bsz * cd * 3 * es), rng(ws, ws ? need : 0)};
  Range ins[] = {rng(io->xBC, Bsz * cd * es), rng(io->conv_w, cd * 16), rng(io->conv_b, io->conv_b ? cd * 4 : 0),
                 rng(io->dt, Bsz * H * es), rng(io->dt_bias, d->dt_softplus ? H * 4 : 0), rng(io->A, H * 4),
                 rng(io->D, H * 4), rng(io->z, d->norm_group ? Bsz * H * P * es : 0),
                 rng(io->norm_w, d->norm_group ? H * P * 4 : 0)};
  const size_t nout = sizeof(outs) / sizeof(outs[0]);
  for (size_t i = 0; i < nout; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return MAMBA2_EINVAL;
    for (size_t j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return MAMBA2_EINVAL;
  }
  return MAMBA2_OK;
}

int32_t mamba2_mixer_decode_step(const mamba2_dims* d, const mamba2_mixer_decode_io* io, void* ws, size_t ws_bytes,
                                 void* stream) {
  int32_t s = check_mixer_decode(d);
  if (s != MAMBA2_OK) return s;
  if (!io) return MAMBA2_EINVAL;
  const size_t need = m2::mixer_decode_workspace_bytes(*d);
  s = check_mixer_decode_args(d, io, nullptr, 0);
  if (s != MAMBA2_OK) return s;
  if (!ws || ws_bytes < need) return MAMBA2_EWORKSPACE;
  if ((uintptr_t)ws & 255) return MAMBA2_EALIGN;
  s = check_mixer_decode_args(d, io, ws, need);
  if (s != MAMBA2_OK) return s;
  return hip_status(m2::launch_mixer_decode(*d, *io, ws, (hipStream_t)stream));
}

size_t mamba2_mixer_decode_noalloc_max_bytes(void) { return m2::mixer_decode_static_scratch_bytes(); }

int32_t mamba2_mixer_decode_step_noalloc(const mamba2_dims* d, const mamba2_mixer_decode_io* io, void* stream) {
  int32_t s = check_mixer_decode(d);
  if (s != MAMBA2_OK) return s;
  s = check_mixer_decode_args(d, io, nullptr, 0);
  if (s != MAMBA2_OK) return s;
  if (m2::mixer_decode_workspace_bytes(*d) > m2::mixer_decode_static_scratch_bytes()) return MAMBA2_EWORKSPACE;
  return hip_status(m2::launch_mixer_decode_static(*d, *io, (hipStream_t)stream));
}

// Validation for the scan's backward pass.
static int32_t check_scan_grad(const mamba2_dims* d) {
  int32_t s = check_common(d);
  if (s != MAMBA2_OK) return s;
  if (d->seqlen < 1) return MAMBA2_EINVAL;
  if (d->conv_width != 0 || d->norm_group != 0 || d->packed_tokens != 0) return MAMBA2_EUNSUPPORTED;
  if (d->headdim != 64) return MAMBA2_EUNSUPPORTED;
  if ((int64_t)d->batch * d->seqlen * d->nheads * d->dstate > ((int64_t)1 << 40)) return MAMBA2_EUNSUPPORTED;
  return MAMBA2_OK;
}

int32_t mamba2_scan_grad_workspace_bytes(const mamba2_dims* d, size_t* bytes) {
  if (!bytes) return MAMBA2_EINVAL;
  int32_t s = check_scan_grad(d);
  if (s != MAMBA2_OK) return s;
  *bytes = m2::scan_grad_workspace_bytes(*d);
  return MAMBA2_OK;
}

int32_t mamba2_scan_grad(const mamba2_dims* d, const mamba2_scan_grad_io* io, void* ws, size_t ws_bytes,
                         void* stream) {
  int32_t s = check_scan_grad(d);
  if (s != MAMBA2_OK) return s;
  if (!io) return MAMBA2_EINVAL;
  const size_t es = esize(d->io_dtype);
  const size_t Bsz = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate, G = d->ngroups;
  if (!io->x || !io->dt || !io->A || !io->B || !io->C || !io->D || !io->dy || !io->dx || !io->ddt || !io->dB ||
      !io->dC || !io->dA || !io->dD)
    return MAMBA2_EINVAL;
  if (d->dt_softplus && !io->ddt_bias) return MAMBA2_EINVAL;
  if (((uintptr_t)io->x % es) || ((uintptr_t)io->dt % es) || ((uintptr_t)io->B % es) || ((uintptr_t)io->C % es) ||
      ((uintptr_t)io->dy % es) || ((uintptr_t)io->dt_bias & 3) || ((uintptr_t)io->A & 3) || ((uintptr_t)io->D & 3) ||
      ((uintptr_t)io->state_in & 3) || ((uintptr_t)io->seqlens & 3) || ((uintptr_t)io->dstate_out & 3) ||
      ((uintptr_t)io->dx & 3) || ((uintptr_t)io->ddt & 3) || ((uintptr_t)io->dB & 3) || ((uintptr_t)io->dC & 3) ||
      ((uintptr_t)io->dA & 3) || ((uintptr_t)io->dD & 3) || ((uintptr_t)io->ddt_bias & 3) ||
      (io->dstate_in && !aligned16(io->dstate_in)))
    return MAMBA2_EALIGN;
  const size_t need = m2::scan_grad_workspace_bytes(*d);
  if (!ws || ws_bytes < need) return MAMBA2_EWORKSPACE;
  if ((uintptr_t)ws & 255) return MAMBA2_EALIGN;
  const size_t tok = Bsz * L;
  Range outs[] = {rng(io->dx, tok * H * P * 4), rng(io->ddt, tok * H * 4), rng(io->dB, tok * G * N * 4),
                  rng(io->dC, tok * G * N * 4), rng(io->dA, H * 4), rng(io->dD, H * 4),
                  rng(io->dstate_in, Bsz * H * P * N * 4), rng(io->ddt_bias, d->dt_softplus ? H * 4 : 0),
                  rng(ws, need)};
  Range ins[] = {rng(io->x, tok * H * P * es), rng(io->dt, tok * H * es), rng(io->dt_bias, d->dt_softplus ? H * 4 : 0),
                 rng(io->A, H * 4), rng(io->B, tok * G * N * es), rng(io->C, tok * G * N * es), rng(io->D, H * 4),
                 rng(io->state_in, Bsz * H * P * N * 4), rng(io->seqlens, Bsz * 4), rng(io->dy, tok * H * P * es),
                 rng(io->dstate_out, Bsz * H * P * N * 4)};
  const size_t nout = sizeof(outs) / sizeof(outs[0]);
  for (size_t i = 0; i < nout; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return MAMBA2_EINVAL;
    for (size_t j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return MAMBA2_EINVAL;
  }
  return hip_status(m2::launch_scan_grad(*d, *io, ws, (hipStream_t)stream));
}

}  // extern "C"

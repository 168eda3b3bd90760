/*
 * mamba2ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 mixer core.
 *
 * The operation (Mamba-2 / structured state-space duality, the method listed
 * under "References" on page "Mamb2_8B_FP4_Recall_SQ3.25"; that page scores a
 * pure Mamba-2 8B model on 2048-token windows with the state reset per window,
 * section "Measured quality"):
 *
 *   per sequence b, head h (group g = h / (H/G)), P x N state S:
 *     S   <- exp(dt_t * A_h) * S + dt_t * x_t (outer) B_t
 *     y_t  = S . C_t + D_h * x_t                 (y_t sees token t's update)
 *
 * optionally preceded by a causal depthwise conv1d of width 4 + SiLU over the
 * xBC channels (the "convolution caches" of section "Storage and runtime
 * memory") and followed by a gated RMSNorm  out = g / sqrt(mean(g^2)+eps) * w,
 * g = y * silu(z)  (the "pinned RMSNorm configuration" of section "Compatible
 * reference environment").  The one-token decode step stores the state to
 * binary16 after every token when the resident state is f16 ("A recurrent row
 * is requantized each token", section "Representation", paragraph "State").
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers to caller-owned memory, dense and
 *    row-major in the layouts given below, 16-byte aligned.  The library
 *    allocates nothing and keeps no per-call state outside the workspace.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *    asynchronous on that stream; results are ready when the stream is.
 *  - Return value: MAMBA2_OK (0) or a negative MAMBA2_E* code.  Arguments are
 *    validated on the host before anything is enqueued; on error nothing is
 *    enqueued and no output is touched.  There is no fallback path: a shape
 *    the kernels do not cover returns MAMBA2_EUNSUPPORTED.
 *  - NaN/Inf in the inputs propagate to the outputs; they are not errors.
 *  - Inputs and outputs must not overlap, except where stated (in place).
 *  - Thread safety: calls on different streams may run concurrently if they
 *    use different workspaces.
 */
#ifndef MAMBA2SSD_H
#define MAMBA2SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MAMBA2_ABI_VERSION 8

enum {
    MAMBA2_OK = 0,
    MAMBA2_EINVAL = -1,        /* bad pointer, dimension, length or aliasing   */
    MAMBA2_EUNSUPPORTED = -2,  /* valid request with no kernel for it          */
    MAMBA2_EALIGN = -3,        /* a pointer is not 16-byte aligned             */
    MAMBA2_EWORKSPACE = -4,    /* workspace missing or too small               */
    MAMBA2_EHIP = -5           /* the HIP runtime refused a launch             */
};

enum { MAMBA2_F32 = 0, MAMBA2_F16 = 1 };

typedef struct mamba2_dims {
    int32_t batch;       /* B  sequences                                        */
    int32_t seqlen;      /* L  tokens per sequence (window); ignored by decode  */
    int32_t nheads;      /* H                                                    */
    int32_t headdim;     /* P  (kernels: 64)                                     */
    int32_t dstate;      /* N  (kernels: 16, 64 or 128)                          */
    int32_t ngroups;     /* G  (H % G == 0; head h uses group h / (H/G))         */
    int32_t chunk;       /* Q  chunk length of the window scan: 64, 128 or 256   */
    int32_t conv_width;  /* 0: x, B, C given; 4: fused conv1d(4)+SiLU over xBC  */
    int32_t norm_group;  /* 0: output y; >0: gated RMSNorm over groups of this
                            many consecutive channels (must divide H*P)         */
    int32_t io_dtype;    /* MAMBA2_F16 or MAMBA2_F32 for x/dt/B/C/xBC/z/y       */
    int32_t state_dtype; /* resident decode state: MAMBA2_F32 or MAMBA2_F16     */
    float norm_eps;      /* epsilon inside the RMSNorm square root              */
    int32_t segments;    /* window scan work split: 0 lets the library choose;
                            k > 0 splits each sequence into up to min(k,
                            chunks) runs of consecutive chunks.  Chunks
                            inside a run pass the state on in registers;
                            runs hand it over through the workspace, except
                            that with two runs (binary16 I/O, dstate 128) the
                            second computes the first's state itself and the
                            first takes the larger share of the chunks.
                            With 0, binary16 windows at dstate 128 of at
                            most 768 tokens whose 2 x heads x batch fits one
                            workgroup per compute unit run unsplit, each
                            workgroup a whole sequence for half a head with
                            the state split over dstate between its waves.
                            Results agree up to rounding for every k.       */
    int32_t dt_softplus; /* 0: dt is given positive and used as is;
                            1: dt is the raw pre-activation, dt_eff =
                            sp(dt + dt_bias[h]), sp(v) = v for v > 20 and
                            log1p(exp(v)) otherwise (no clamp).  Decode, the
                            one-token mixer, the requantized window, binary32
                            windows and the backward evaluate it as
                            (float) sp((double) dt + (double) dt_bias[h]);
                            binary16 window scans evaluate it in binary32
                            with the hardware exponential and logarithm
                            (relative error below about 6e-5, within the
                            window tolerance)                               */
    int32_t packed_tokens; /* window calls: 0 for the (B, L, ...) layout; T > 0
                            for packed variable-length windows: every
                            per-token tensor (x, B, C, xBC, dt, z, y) holds T
                            rows and sequence b is rows cu_seqlens[b] ..
                            cu_seqlens[b+1]-1 of it (io.cu_seqlens required,
                            io.seqlens NULL); dims.seqlen is then the
                            longest length.  A sequence longer than
                            dims.seqlen is cut at dims.seqlen tokens and rows
                            at or past T are never read or written.  Decode
                            and state calls ignore it.                       */
} mamba2_dims;

/* ------------------------------------------------------------------------ */
/* Whole-window chunked scan (the state-space-dual form).
 *
 * Layouts (io = io_dtype):
 *   conv_width == 0:  x (B,L,H,P) io;  B, C (B,L,G,N) io
 *   conv_width == 4:  xBC (B,L,H*P+2*G*N) io, raw pre-conv activations with
 *                     channel order x | B | C (x channel h*P+p, B/C channel
 *                     g*N+n).  xBC_ld: elements between consecutive tokens'
 *                     rows of xBC, 0 for dense rows (H*P+2*G*N); a larger
 *                     stride reads xBC as a slice of wider rows (such as the
 *                     input projection's output) without a copy.  A
 *                     negative stride or one below H*P+2*G*N is
 *                     MAMBA2_EINVAL, rows not 16-byte aligned MAMBA2_EALIGN;
 *                     the field is ignored without the fused conv;
 *                     conv_w (H*P+2*G*N, 4) f32 with tap 3 applied to
 *                     the current token and tap 3-k to the token k back;
 *                     conv_b (H*P+2*G*N) f32 or NULL (zero);
 *                     conv_state_in (B, H*P+2*G*N, 3) io or NULL (zero history,
 *                     a window reset), the 3 raw tokens preceding the window,
 *                     oldest first; conv_state_out same shape or NULL: the last
 *                     3 raw tokens before seqlens[b].
 *   dt (B,L,H) io: positive, or raw when dims.dt_softplus == 1 (then
 *             dt_bias (H) f32 or NULL (zero) is added before the softplus)
 *   A, D (H) f32
 *   state_in  (B,H,P,N) f32 or NULL (zero initial state)
 *   state_out (B,H,P,N) f32 or NULL: state after token seqlens[b]-1.
 *             With NULL (binary16 I/O, dstate 128), segments of a sequence
 *             hand their aggregate states over as binary16 scaled by a
 *             power of two, and with the fused conv B enters the scan as
 *             its binary16 value alone (no remainder): only the readouts of
 *             y see the state then (y within the same tolerance).  With a
 *             state_out the aggregates stay binary32 and B keeps its
 *             binary16 remainder, so the final state meets its own.
 *   seqlens   device int32 (B) or NULL (all L); each value is clamped to
 *             [0, L].  Rows t >= seqlens[b] of y are not written.
 *   cu_seqlens device int32 (B+1), packed layout only (dims.packed_tokens
 *             > 0): non-decreasing row offsets of the sequences in the
 *             packed tensors, which then have T = dims.packed_tokens rows in
 *             place of (B, L): x (T,H,P), B/C (T,G,N), xBC (T,conv_dim),
 *             dt (T,H), z and y (T,H*P).  Per-sequence tensors (state_*,
 *             conv_state_*) keep their (B, ...) shapes.  NULL otherwise.
 *   norm_group == 0: y (B,L,H*P) io receives y.
 *   norm_group  > 0: z (B,L,H*P) io and norm_w (H*P) f32 are required and
 *             y receives the gated RMSNorm output.  z_ld: elements between
 *             consecutive tokens' rows of z, 0 for dense rows (H*P); a larger
 *             stride reads z in place from wider rows (16-byte aligned rows;
 *             below H*P or negative is MAMBA2_EINVAL, misaligned
 *             MAMBA2_EALIGN).  Ignored without the norm.
 *   dt_ld:    elements between consecutive tokens' rows of dt, 0 for dense
 *             rows (H); a larger stride reads dt in place from wider rows,
 *             e.g. the last H columns of the input projection's output
 *             [z | xBC | dt].  Below H or negative is MAMBA2_EINVAL.
 *   ws, ws_bytes: workspace of at least mamba2_window_workspace_bytes()
 *             bytes, 256-byte aligned, ZERO-FILLED BEFORE ITS FIRST USE.  The
 *             library leaves it ready for the next call on the same stream; it
 *             must not be shared by calls that may overlap.
 */
typedef struct mamba2_window_io {
    const void* x;
    const void* B;
    const void* C;
    const void* xBC;
    const float* conv_w;
    const float* conv_b;
    const void* conv_state_in;
    void* conv_state_out;
    const void* dt;
    const float* A;
    const float* D;
    const float* state_in;
    float* state_out;
    const int32_t* seqlens;
    const void* z;
    const float* norm_w;
    void* y;
    const float* dt_bias;
    const int32_t* cu_seqlens;
    int64_t xBC_ld;
    int64_t z_ld;
    int64_t dt_ld;
} mamba2_window_io;

/* Workspace size for a window call with these dims (host only, no GPU call).
 * Errors: MAMBA2_EINVAL (NULL argument or invalid dims), MAMBA2_EUNSUPPORTED. */
int32_t mamba2_window_workspace_bytes(const mamba2_dims* dims, size_t* bytes);

/* Runs the window scan.  Errors: EINVAL, EUNSUPPORTED, EALIGN, EWORKSPACE,
 * EHIP. */
int32_t mamba2_conv_scan_window(const mamba2_dims* dims, const mamba2_window_io* io,
                                void* ws, size_t ws_bytes, void* stream);

/* Reads and clears the error word of a window workspace.  Waits for all
 * work queued on `stream` so far (synchronous), then stores the word in
 * *flags and, when it is set, clears it (also synchronously, with a kernel on
 * the same stream).  *flags == 0: every window call on this workspace since
 * the last query completed its hand-offs.  Bit 0 set: in some call a
 * segment's bounded wait for an earlier segment's aggregate gave up (it
 * never returns early otherwise), so that call's y and final states are not
 * valid; the window entry point itself cannot report this, since it returns
 * before the kernels run.  ws and ws_bytes as given to the window calls
 * (at least the control block: MAMBA2_EWORKSPACE otherwise).
 * Errors: EINVAL (NULL ws or flags), EWORKSPACE, EALIGN, EHIP. */
int32_t mamba2_window_take_error(void* ws, size_t ws_bytes, uint32_t* flags, void* stream);

/* ------------------------------------------------------------------------ */
/* Whole window with the recurrent state requantized to binary16 after every
 * token, the way page "Mamb2_8B_FP4_Recall_SQ3.25" scores its windows (carry
 * requantized each token, section "Representation", paragraph "State"; state
 * reset per window, section "Measured quality").  Each token is the
 * one-token step of mamba2_decode_step with a binary16 state (same binary32
 * contract), run over the window's tokens with the state kept on chip, so
 * the final state equals that many decode steps bit for bit.
 *   dims: conv_width 0 and norm_group 0 (EUNSUPPORTED otherwise); headdim 64;
 *         dstate 16, 64 or 128; chunk, segments and state_dtype are ignored.
 *   io:   x, B, C, dt, A, D, y as for mamba2_conv_scan_window (x and y need
 *         only element alignment, B and C 16 bytes); xBC, conv_*, z, norm_w
 *         are ignored.
 *         state_in  (B,H,P,N) f32 or NULL (zeros): rounded once to binary16
 *                   (nearest even) before the first token;
 *         state_out (B,H,P,N) f32 or NULL: the binary16 state after the
 *                   sequence's last token, widened exactly;
 *         seqlens   device int32 (B) or NULL: tokens at or past a sequence's
 *                   length are not processed and their y rows not written;
 *         cu_seqlens with dims.packed_tokens as for mamba2_conv_scan_window.
 * No workspace.  Outputs must not overlap inputs or each other.
 * Errors: EINVAL, EUNSUPPORTED, EALIGN, EHIP. */
int32_t mamba2_requant_window(const mamba2_dims* dims, const mamba2_window_io* io, void* stream);

/* ------------------------------------------------------------------------ */
/* Gradients of the window scan (the backward pass), for training through the
 * frozen mixer core (page "Mamb2_8B_FP4_Recall_SQ3.25" trains an adapter
 * through the frozen stack).  For the scan of mamba2_conv_scan_window with
 * conv_width 0 and norm_group 0 (y and the final state as outputs), and a
 * loss whose gradients with respect to them are dy and dstate_out, returns
 * the gradients with respect to every input.
 *   dims: conv_width 0, norm_group 0, packed_tokens 0 (EUNSUPPORTED
 *         otherwise); headdim 64; dstate 16, 64 or 128; dt_softplus as in
 *         the forward call; chunk and segments are ignored.
 *   inputs (as for mamba2_conv_scan_window, element alignment suffices for
 *         the io tensors): x, dt, dt_bias (with dt_softplus), A, B, C, D,
 *         state_in (B,H,P,N) f32 or NULL, seqlens or NULL;
 *         dy (B,L,H,P) io: the gradient with respect to y;
 *         dstate_out (B,H,P,N) f32 or NULL (zero).
 *   outputs, all f32 and written in full (rows at or past a sequence's
 *         length are zero):
 *         dx (B,L,H,P); ddt (B,L,H), with respect to the dt given (the raw
 *         one with dt_softplus); dB, dC (B,L,G,N), summed over each group's
 *         heads; dA, dD (H), summed over the batch; dstate_in (B,H,P,N) or
 *         NULL (not computed; 16-byte aligned); ddt_bias (H) with
 *         dt_softplus (summed over batch and tokens), else ignored.
 *   ws, ws_bytes: workspace of at least mamba2_scan_grad_workspace_bytes()
 *         bytes, 256-byte aligned; its contents on entry do not matter.
 * Outputs must not overlap inputs or each other.
 * Errors: EINVAL, EUNSUPPORTED, EALIGN, EWORKSPACE, EHIP. */
typedef struct mamba2_scan_grad_io {
    const void* x;
    const void* dt;
    const float* dt_bias;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const float* state_in;
    const int32_t* seqlens;
    const void* dy;
    const float* dstate_out;
    float* dx;
    float* ddt;
    float* dB;
    float* dC;
    float* dA;
    float* dD;
    float* dstate_in;
    float* ddt_bias;
} mamba2_scan_grad_io;

int32_t mamba2_scan_grad_workspace_bytes(const mamba2_dims* dims, size_t* bytes);
int32_t mamba2_scan_grad(const mamba2_dims* dims, const mamba2_scan_grad_io* io, void* ws, size_t ws_bytes,
                         void* stream);

/* ------------------------------------------------------------------------ */
/* One-token recurrent step for B sequences (dims.seqlen is ignored).
 *   x (B,H,P) io; dt (B,H) io (positive, or raw with dims.dt_softplus);
 *   B, C (B,G,N) io; A, D (H) f32
 *   state (B,H,P,N) in state_dtype, read and updated IN PLACE
 *   y (B,H,P) io
 * With an f16 resident state the step is evaluated in binary32 as
 *   a = (float)exp((double)dt * (double)A);  u = dt*x;  v = u*B[n];
 *   s = fmaf(a, S_old, v);  y accumulates s*C[n];  S_new = f16_rne(s)
 * (y uses the pre-store value s).  With an f32 state S_new = s.
 * Errors: EINVAL, EUNSUPPORTED, EALIGN, EHIP. */
typedef struct mamba2_decode_io {
    const void* x;
    const void* dt;
    const void* B;
    const void* C;
    const float* A;
    const float* D;
    void* state;
    void* y;
    const float* dt_bias;   /* (H) f32 or NULL, used when dims.dt_softplus == 1 */
} mamba2_decode_io;

int32_t mamba2_decode_step(const mamba2_dims* dims, const mamba2_decode_io* io, void* stream);

/* ------------------------------------------------------------------------ */
/* Full one-token mixer step for B sequences: the generation path of one
 * layer's mixer core (page "Mamb2_8B_FP4_Recall_SQ3.25": the convolution
 * caches of section "Storage and runtime memory", the per-token requantized
 * recurrent row of section "Representation", the gated RMSNorm of section
 * "Compatible reference environment").  For every sequence:
 *   u   = silu(conv_b + sum_k conv_w[:, k] * [history, xBC][k])  (width 4,
 *         tap 3 on this token), rounded once (correctly) to the I/O type, split x | B | C;
 *   history <- (history[1], history[2], xBC)                     (in place);
 *   the decode step of mamba2_decode_step on (x, dt, B, C);
 *   y = the step's output, or with norm_group > 0 the gated RMSNorm
 *       g / sqrt(mean_group(g^2) + eps) * norm_w,  g = y * silu(z).
 * T consecutive calls from the window's conv_state_out and state_out give
 * that window's outputs for its next T tokens (the conv state layout is the
 * one mamba2_conv_scan_window reads and writes).
 *   dims: conv_width 4; headdim 64; dstate 16, 64 or 128; state_dtype the
 *         resident type; norm_group 0 or a multiple of 64 dividing H*P (at
 *         most H*P); norm_eps; dt_softplus.  seqlen, chunk, segments and
 *         packed_tokens are ignored.
 *   io:   xBC (B, conv_dim) io raw in_proj output for this token;
 *         conv_w (conv_dim, 4) f32; conv_b (conv_dim) f32 or NULL;
 *         conv_state (B, conv_dim, 3) io, the 3 raw tokens before this one
 *         (oldest first), read and rolled IN PLACE;
 *         dt (B, H) io, dt_bias (H) f32 or NULL (with dt_softplus); A, D (H);
 *         state (B,H,P,N) resident type, read and updated IN PLACE;
 *         z (B, H*P) io and norm_w (H*P) f32 when norm_group > 0;
 *         y (B, H*P) io.
 *   dims.batch * dims.ngroups at most 16384 (MAMBA2_EUNSUPPORTED beyond).
 *   ws, ws_bytes: workspace of at least mamba2_mixer_decode_workspace_bytes()
 *         bytes, 256-byte aligned, ZERO-FILLED BEFORE ITS FIRST USE; every
 *         call leaves it ready for the next one on the same stream, whatever
 *         the next call's batch (calls that may overlap must not share it).
 * Errors: EINVAL, EUNSUPPORTED, EALIGN, EWORKSPACE, EHIP. */
typedef struct mamba2_mixer_decode_io {
    const void* xBC;
    const float* conv_w;
    const float* conv_b;
    void* conv_state;
    const void* dt;
    const float* dt_bias;
    const float* A;
    const float* D;
    void* state;
    const void* z;
    const float* norm_w;
    void* y;
} mamba2_mixer_decode_io;

int32_t mamba2_mixer_decode_workspace_bytes(const mamba2_dims* dims, size_t* bytes);
int32_t mamba2_mixer_decode_step(const mamba2_dims* dims, const mamba2_mixer_decode_io* io, void* ws,
                                 size_t ws_bytes, void* stream);

/* The same one-token mixer step for callers that cannot allocate device
 * memory or pass a workspace: code recorded under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Arguments, layouts,
 * results and errors are those of mamba2_mixer_decode_step (the same kernels
 * run), except that the workspace is a fixed array inside the library:
 * mamba2_mixer_decode_noalloc_max_bytes() bytes per GPU, held by each GPU the
 * library runs on until the process ends.  A request whose
 * mamba2_mixer_decode_workspace_bytes() exceeds that size returns
 * MAMBA2_EWORKSPACE before anything is enqueued (4 MiB: 4,032 sequences at
 * H = 128 with the norm).  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); its first call on a
 * device looks up that device's copy of the array (HIP runtime error ->
 * MAMBA2_EHIP).  Every call on one GPU shares that GPU's array, which needs
 * no clearing between calls (its arrival counters return to zero at the end
 * of each call); calls that may overlap on one GPU (different streams) race
 * and must be serialized by the caller.
 * Errors: EINVAL, EUNSUPPORTED, EALIGN, EWORKSPACE, EHIP. */
size_t mamba2_mixer_decode_noalloc_max_bytes(void);
int32_t mamba2_mixer_decode_step_noalloc(const mamba2_dims* dims, const mamba2_mixer_decode_io* io, void* stream);

/* State load/store between f32 (B,H,P,N) and the resident state_dtype
 * (f16: round to nearest even, subnormals kept; f32: copy).  src and dst must
 * not overlap.  Errors: EINVAL, EUNSUPPORTED, EALIGN, EHIP. */
int32_t mamba2_state_load(const mamba2_dims* dims, const float* src_f32, void* dst_resident, void* stream);
int32_t mamba2_state_store(const mamba2_dims* dims, const void* src_resident, float* dst_f32, void* stream);

/* ------------------------------------------------------------------------ */
int32_t mamba2_abi_version(void);
/* Static string for a status code (never NULL). */
const char* mamba2_status_str(int32_t status);
/* The hipError_t of the last MAMBA2_EHIP returned on this thread (0 if none). */
int32_t mamba2_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MAMBA2SSD_H */

"""MI355X (gfx950) Mamba-2 mixer core: Python binding of libmamba2ssd.so.

Argument marshalling only: every step of the scan, convolution, norm and
decode runs in the HIP kernels behind the C ABI declared in
``include/mamba2ssd.h``.  PyTorch provides device memory and the stream.
There is no CPU or PyTorch fallback: if the library is missing, every entry
point raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "F16", "F32", "Dims", "Mamba2Error", "library_path", "load_library",
    "window_workspace_bytes", "alloc_workspace", "conv_scan_window", "window_take_error", "decode_step", "requant_window",
    "mixer_decode_workspace_bytes", "alloc_mixer_decode_workspace", "mixer_decode_step",
    "mixer_decode_noalloc_max_bytes", "mixer_decode_step_noalloc",
    "scan_grad_workspace_bytes", "alloc_scan_grad_workspace", "scan_grad",
    "state_load", "state_store", "abi_version",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmamba2ssd.so")

F32, F16 = 0, 1
_STATUS = {0: "ok", -1: "EINVAL", -2: "EUNSUPPORTED", -3: "EALIGN", -4: "EWORKSPACE", -5: "EHIP"}


class Mamba2Error(RuntimeError):
    def __init__(self, fn, status, lib):
        self.status = status
        msg = lib.mamba2_status_str(status).decode()
        if status == -5:
            msg += f" (hipError {lib.mamba2_last_hip_error()})"
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "chunk",
        "conv_width", "norm_group", "io_dtype", "state_dtype")] + [("norm_eps", ctypes.c_float),
                                                                   ("segments", ctypes.c_int32),
                                                                   ("dt_softplus", ctypes.c_int32),
                                                                   ("packed_tokens", ctypes.c_int32)]


class _WindowIO(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "B", "C", "xBC", "conv_w", "conv_b", "conv_state_in", "conv_state_out", "dt", "A", "D",
        "state_in", "state_out", "seqlens", "z", "norm_w", "y", "dt_bias", "cu_seqlens")] + [
        ("xBC_ld", ctypes.c_int64), ("z_ld", ctypes.c_int64), ("dt_ld", ctypes.c_int64)]


class _MixerDecodeIO(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "xBC", "conv_w", "conv_b", "conv_state", "dt", "dt_bias", "A", "D", "state", "z", "norm_w", "y")]


class _ScanGradIO(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "dt", "dt_bias", "A", "B", "C", "D", "state_in", "seqlens", "dy", "dstate_out",
        "dx", "ddt", "dB", "dC", "dA", "dD", "dstate_in", "ddt_bias")]


class _DecodeIO(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("x", "dt", "B", "C", "A", "D", "state", "y", "dt_bias")]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmamba2ssd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950); there is no fallback path")
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(Dims)
        vp = ctypes.c_void_p
        lib.mamba2_abi_version.restype = ctypes.c_int32
        lib.mamba2_status_str.restype = ctypes.c_char_p
        lib.mamba2_status_str.argtypes = [ctypes.c_int32]
        lib.mamba2_last_hip_error.restype = ctypes.c_int32
        lib.mamba2_window_workspace_bytes.restype = ctypes.c_int32
        lib.mamba2_window_workspace_bytes.argtypes = [dp, ctypes.POINTER(ctypes.c_size_t)]
        lib.mamba2_conv_scan_window.restype = ctypes.c_int32
        lib.mamba2_conv_scan_window.argtypes = [dp, ctypes.POINTER(_WindowIO), vp, ctypes.c_size_t, vp]
        lib.mamba2_window_take_error.restype = ctypes.c_int32
        lib.mamba2_window_take_error.argtypes = [vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_uint32), vp]
        lib.mamba2_requant_window.restype = ctypes.c_int32
        lib.mamba2_requant_window.argtypes = [dp, ctypes.POINTER(_WindowIO), vp]
        lib.mamba2_mixer_decode_workspace_bytes.restype = ctypes.c_int32
        lib.mamba2_mixer_decode_workspace_bytes.argtypes = [dp, ctypes.POINTER(ctypes.c_size_t)]
        lib.mamba2_mixer_decode_step.restype = ctypes.c_int32
        lib.mamba2_mixer_decode_step.argtypes = [dp, ctypes.POINTER(_MixerDecodeIO), vp, ctypes.c_size_t, vp]
        lib.mamba2_mixer_decode_noalloc_max_bytes.restype = ctypes.c_size_t
        lib.mamba2_mixer_decode_noalloc_max_bytes.argtypes = []
        lib.mamba2_mixer_decode_step_noalloc.restype = ctypes.c_int32
        lib.mamba2_mixer_decode_step_noalloc.argtypes = [dp, ctypes.POINTER(_MixerDecodeIO), vp]
        lib.mamba2_scan_grad_workspace_bytes.restype = ctypes.c_int32
        lib.mamba2_scan_grad_workspace_bytes.argtypes = [dp, ctypes.POINTER(ctypes.c_size_t)]
        lib.mamba2_scan_grad.restype = ctypes.c_int32
        lib.mamba2_scan_grad.argtypes = [dp, ctypes.POINTER(_ScanGradIO), vp, ctypes.c_size_t, vp]
        lib.mamba2_decode_step.restype = ctypes.c_int32
        lib.mamba2_decode_step.argtypes = [dp, ctypes.POINTER(_DecodeIO), vp]
        lib.mamba2_state_load.restype = ctypes.c_int32
        lib.mamba2_state_load.argtypes = [dp, vp, vp, vp]
        lib.mamba2_state_store.restype = ctypes.c_int32
        lib.mamba2_state_store.argtypes = [dp, vp, vp, vp]
        _lib = lib
    return _lib


def abi_version() -> int:
    return load_library().mamba2_abi_version()


def _check(fn, status):
    if status != 0:
        raise Mamba2Error(fn, status, load_library())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _rows(t, name="xBC"):
    """(pointer, row stride) of a tensor whose rows may be a slice of wider
    rows: the last dimension contiguous and the leading dimensions dense in
    units of the row stride."""
    if t is None:
        return None, 0
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if t.is_contiguous():
        return t.data_ptr(), 0
    ld = t.stride(-2)
    if t.stride(-1) != 1 or ld < t.shape[-1] or (t.dim() == 3 and t.stride(0) != t.shape[1] * ld):
        raise ValueError(f"{name} must have contiguous channels and evenly strided token rows")
    return t.data_ptr(), ld


def _stream(t, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _io_dtype(t):
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported I/O dtype {t.dtype}")


def make_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk=256, conv_width=0, norm_group=0,
              io_dtype=F16, state_dtype=F32, norm_eps=1e-5, segments=0, dt_softplus=0, packed_tokens=0) -> Dims:
    return Dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, conv_width, norm_group, io_dtype,
                state_dtype, norm_eps, segments, dt_softplus, packed_tokens)


def _window_shape(dt, cu_seqlens, max_seqlen):
    """(batch, seqlen, nheads, packed_tokens) of a window call: dt (B,L,H), or
    dt (T,H) with cu_seqlens (B+1) and the longest length max_seqlen."""
    if cu_seqlens is None:
        Bsz, L, H = dt.shape
        return Bsz, L, H, 0
    if max_seqlen is None:
        raise ValueError("packed windows need max_seqlen (an upper bound on every length)")
    T, H = dt.shape
    return cu_seqlens.numel() - 1, int(max_seqlen), H, T


def window_workspace_bytes(dims: Dims) -> int:
    n = ctypes.c_size_t(0)
    _check("mamba2_window_workspace_bytes", load_library().mamba2_window_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def alloc_workspace(dims: Dims, device) -> torch.Tensor:
    """A zero-filled workspace for window calls with these dims (reusable
    across calls on one stream)."""
    return torch.zeros(window_workspace_bytes(dims), dtype=torch.uint8, device=device)


def conv_scan_window(dt, A, D, y, workspace, *, x=None, B=None, C=None, xBC=None, conv_w=None, conv_b=None,
                     conv_state_in=None, conv_state_out=None, state_in=None, state_out=None, seqlens=None,
                     z=None, norm_w=None, chunk=256, norm_group=0, norm_eps=1e-5, ngroups=None, dstate=None,
                     headdim=None, segments=0, dt_softplus=False, dt_bias=None, cu_seqlens=None, max_seqlen=None,
                     stream=None):
    """Whole-window scan.  Shapes: x (B,L,H,P), B/C (B,L,G,N) -- or xBC
    (B,L,H*P+2*G*N) with conv_w (H*P+2*G*N, 4) for the fused conv --, dt
    (B,L,H), A/D (H) f32, y (B,L,H*P) (or (B,L,H,P)).  Packed windows: every
    per-token tensor has T rows in place of (B,L), with cu_seqlens (B+1)
    int32 row offsets and max_seqlen the longest length.  xBC, z and dt may
    be column slices of wider rows, e.g. of the input projection's output
    ``zxbcdt = [z | xBC | dt]``: contiguous channels, rows a fixed stride
    apart (16-byte aligned for xBC and z).  See include/mamba2ssd.h."""
    Bsz, L, H, T = _window_shape(dt, cu_seqlens, max_seqlen)
    conv = xBC is not None
    if conv:
        if ngroups is None or dstate is None:
            raise ValueError("the fused conv needs ngroups and dstate")
        P = 64 if headdim is None else headdim
        G, N = ngroups, dstate
    else:
        P = x.shape[-1]
        G, N = B.shape[-2], B.shape[-1]
    dims = make_dims(Bsz, L, H, P, N, G, chunk, 4 if conv else 0, norm_group, _io_dtype(dt), F32, norm_eps,
                     segments, int(bool(dt_softplus)), T)
    xp, xld = _rows(xBC)
    zp, zld = _rows(z, "z")
    dp, dld = _rows(dt, "dt")
    io = _WindowIO(_ptr(x), _ptr(B), _ptr(C), xp, _ptr(conv_w), _ptr(conv_b), _ptr(conv_state_in),
                   _ptr(conv_state_out), dp, _ptr(A), _ptr(D), _ptr(state_in), _ptr(state_out),
                   _ptr(seqlens), zp, _ptr(norm_w), _ptr(y), _ptr(dt_bias), _ptr(cu_seqlens), xld, zld, dld)
    _check("mamba2_conv_scan_window",
           load_library().mamba2_conv_scan_window(ctypes.byref(dims), ctypes.byref(io), _ptr(workspace),
                                                  workspace.numel(), _stream(dt, stream)))


def window_take_error(workspace, stream=None) -> int:
    """Error word of a window workspace after the work queued on the stream
    (0: every hand-off completed; bit 0: a bounded wait gave up and that
    call's outputs are invalid); the word is cleared.  Synchronizes the
    stream."""
    v = ctypes.c_uint32(0)
    _check("mamba2_window_take_error",
           load_library().mamba2_window_take_error(_ptr(workspace), workspace.numel(), ctypes.byref(v),
                                                   _stream(workspace, stream)))
    return v.value


def requant_window(dt, A, D, y, *, x, B, C, state_in=None, state_out=None, seqlens=None, dt_softplus=False,
                   dt_bias=None, cu_seqlens=None, max_seqlen=None, stream=None):
    """Whole window with the state requantized to binary16 after every token.
    Shapes: x (B,L,H,P), B/C (B,L,G,N), dt (B,L,H), A/D (H) f32, y (B,L,H*P)
    (or (B,L,H,P)); state_in/state_out (B,H,P,N) f32; packed windows as for
    conv_scan_window.  See include/mamba2ssd.h."""
    Bsz, L, H, T = _window_shape(dt, cu_seqlens, max_seqlen)
    P = x.shape[-1]
    G, N = B.shape[-2], B.shape[-1]
    dims = make_dims(Bsz, L, H, P, N, G, 256, 0, 0, _io_dtype(dt), F16, dt_softplus=int(bool(dt_softplus)),
                     packed_tokens=T)
    dp, dld = _rows(dt, "dt")
    io = _WindowIO(_ptr(x), _ptr(B), _ptr(C), None, None, None, None, None, dp, _ptr(A), _ptr(D),
                   _ptr(state_in), _ptr(state_out), _ptr(seqlens), None, None, _ptr(y), _ptr(dt_bias),
                   _ptr(cu_seqlens), 0, 0, dld)
    _check("mamba2_requant_window", load_library().mamba2_requant_window(ctypes.byref(dims), ctypes.byref(io),
                                                                         _stream(dt, stream)))


def decode_step(x, dt, B, C, A, D, state, y, dt_softplus=False, dt_bias=None, stream=None):
    """One token for each of B sequences: x (B,H,P), dt (B,H), B/C (B,G,N),
    A/D (H) f32, state (B,H,P,N) f16 or f32 updated in place, y (B,H,P)."""
    Bsz, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    sd = F16 if state.dtype == torch.float16 else F32
    dims = make_dims(Bsz, 1, H, P, N, G, 256, 0, 0, _io_dtype(x), sd, dt_softplus=int(bool(dt_softplus)))
    io = _DecodeIO(_ptr(x), _ptr(dt), _ptr(B), _ptr(C), _ptr(A), _ptr(D), _ptr(state), _ptr(y), _ptr(dt_bias))
    _check("mamba2_decode_step", load_library().mamba2_decode_step(ctypes.byref(dims), ctypes.byref(io),
                                                                   _stream(x, stream)))


def mixer_decode_dims(batch, nheads, headdim, dstate, ngroups, norm_group=0, io_dtype=F16, state_dtype=F16,
                      norm_eps=1e-5, dt_softplus=False) -> Dims:
    return make_dims(batch, 1, nheads, headdim, dstate, ngroups, 256, 4, norm_group, io_dtype, state_dtype, norm_eps,
                     dt_softplus=int(bool(dt_softplus)))


def mixer_decode_workspace_bytes(dims: Dims) -> int:
    n = ctypes.c_size_t(0)
    _check("mamba2_mixer_decode_workspace_bytes",
           load_library().mamba2_mixer_decode_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def alloc_mixer_decode_workspace(dims: Dims, device) -> torch.Tensor:
    """A zero-filled workspace for fused decode steps with these dims (reusable
    across calls on one stream)."""
    return torch.zeros(max(mixer_decode_workspace_bytes(dims), 1), dtype=torch.uint8, device=device)


def mixer_decode_step(xBC, conv_w, conv_state, dt, A, D, state, y, workspace, *, conv_b=None, z=None, norm_w=None,
                      ngroups, dstate, headdim=64, norm_group=0, norm_eps=1e-5, dt_softplus=False, dt_bias=None,
                      stream=None):
    """One token of the full mixer for B sequences: xBC (B, H*P+2*G*N) raw,
    conv_w (conv_dim, 4) f32, conv_state (B, conv_dim, 3) rolled in place,
    dt (B, H), A/D (H) f32, state (B,H,P,N) f16 or f32 updated in place,
    y (B, H*P); z (B, H*P) and norm_w (H*P) with norm_group > 0.  See
    include/mamba2ssd.h."""
    Bsz, H = dt.shape
    sd = F16 if state.dtype == torch.float16 else F32
    dims = mixer_decode_dims(Bsz, H, headdim, dstate, ngroups, norm_group, _io_dtype(xBC), sd, norm_eps, dt_softplus)
    io = _MixerDecodeIO(_ptr(xBC), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(dt), _ptr(dt_bias), _ptr(A),
                        _ptr(D), _ptr(state), _ptr(z), _ptr(norm_w), _ptr(y))
    _check("mamba2_mixer_decode_step",
           load_library().mamba2_mixer_decode_step(ctypes.byref(dims), ctypes.byref(io), _ptr(workspace),
                                                   workspace.numel(), _stream(xBC, stream)))


def mixer_decode_noalloc_max_bytes() -> int:
    """Size of the library's fixed workspace for mixer_decode_step_noalloc."""
    return load_library().mamba2_mixer_decode_noalloc_max_bytes()


def mixer_decode_step_noalloc(xBC, conv_w, conv_state, dt, A, D, state, y, *, conv_b=None, z=None, norm_w=None,
                              ngroups, dstate, headdim=64, norm_group=0, norm_eps=1e-5, dt_softplus=False,
                              dt_bias=None, stream=None):
    """mixer_decode_step without a workspace argument: the library's fixed
    per-GPU array serves as the workspace and nothing is allocated.  Calls
    that may overlap on one GPU race.  See include/mamba2ssd.h."""
    Bsz, H = dt.shape
    sd = F16 if state.dtype == torch.float16 else F32
    dims = mixer_decode_dims(Bsz, H, headdim, dstate, ngroups, norm_group, _io_dtype(xBC), sd, norm_eps, dt_softplus)
    io = _MixerDecodeIO(_ptr(xBC), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(dt), _ptr(dt_bias), _ptr(A),
                        _ptr(D), _ptr(state), _ptr(z), _ptr(norm_w), _ptr(y))
    _check("mamba2_mixer_decode_step_noalloc",
           load_library().mamba2_mixer_decode_step_noalloc(ctypes.byref(dims), ctypes.byref(io), _stream(xBC, stream)))


def scan_grad_workspace_bytes(dims: Dims) -> int:
    n = ctypes.c_size_t(0)
    _check("mamba2_scan_grad_workspace_bytes",
           load_library().mamba2_scan_grad_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def alloc_scan_grad_workspace(dims: Dims, device) -> torch.Tensor:
    """Workspace for scan_grad calls with these dims (no clearing needed)."""
    return torch.empty(scan_grad_workspace_bytes(dims), dtype=torch.uint8, device=device)


def scan_grad(dt, A, D, dy, workspace, *, x, B, C, dx, ddt, dB, dC, dA, dD, state_in=None, seqlens=None,
              dstate_out=None, dstate_in=None, dt_softplus=False, dt_bias=None, ddt_bias=None, stream=None):
    """Gradients of the window scan.  Inputs as conv_scan_window (x (B,L,H,P),
    B/C (B,L,G,N), dt (B,L,H)), dy (B,L,H,P) and dstate_out (B,H,P,N) f32 or
    None; f32 outputs dx, ddt, dB, dC, dA, dD, dstate_in (or None) and, with
    dt_softplus, ddt_bias.  See include/mamba2ssd.h."""
    Bsz, L, H = dt.shape
    P = x.shape[-1]
    G, N = B.shape[-2], B.shape[-1]
    dims = make_dims(Bsz, L, H, P, N, G, 256, 0, 0, _io_dtype(dt), F32, dt_softplus=int(bool(dt_softplus)))
    io = _ScanGradIO(_ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(state_in),
                     _ptr(seqlens), _ptr(dy), _ptr(dstate_out), _ptr(dx), _ptr(ddt), _ptr(dB), _ptr(dC), _ptr(dA),
                     _ptr(dD), _ptr(dstate_in), _ptr(ddt_bias))
    _check("mamba2_scan_grad", load_library().mamba2_scan_grad(ctypes.byref(dims), ctypes.byref(io), _ptr(workspace),
                                                               workspace.numel(), _stream(dt, stream)))


def _state_dims(t, resident_dtype):
    Bsz, H, P, N = t.shape
    sd = F16 if resident_dtype == torch.float16 else F32
    return make_dims(Bsz, 1, H, P, N, 1, 256, 0, 0, F16, sd)


def state_load(src_f32, dst_resident, stream=None):
    """f32 (B,H,P,N) -> resident state (f16: round to nearest even)."""
    dims = _state_dims(src_f32, dst_resident.dtype)
    _check("mamba2_state_load", load_library().mamba2_state_load(ctypes.byref(dims), _ptr(src_f32),
                                                                 _ptr(dst_resident), _stream(src_f32, stream)))


def state_store(src_resident, dst_f32, stream=None):
    """Resident state -> f32 (B,H,P,N)."""
    dims = _state_dims(dst_f32, src_resident.dtype)
    _check("mamba2_state_store", load_library().mamba2_state_store(ctypes.byref(dims), _ptr(src_resident),
                                                                   _ptr(dst_f32), _stream(dst_f32, stream)))

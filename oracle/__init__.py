"""Plain, slow, obviously-correct CPU oracle for the Mamba-2 mixer core.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``mamba_ssd_scan_amd``) never imports it, and it never imports the
product path.

The arithmetic lives in ``ssd_oracle.c`` (fp64, sequential, built with gcc
without fast-math); this module only marshals numpy arrays.  What each routine
computes, and which passage of the pages it follows, is stated in the C file.
Pins that tie the oracle to something other than itself are in
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ssd_oracle.c into liboracle.so with gcc (fp64, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        fp = ctypes.POINTER(ctypes.c_float)
        ip = ctypes.POINTER(ctypes.c_int32)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i, i64 = ctypes.c_int, ctypes.c_int64
        lib.oracle_f16_round.restype = ctypes.c_double
        lib.oracle_f16_round.argtypes = [ctypes.c_double]
        lib.oracle_f16_round_array.argtypes = [dp, dp, i64]
        lib.oracle_f16_bits_to_double_array.argtypes = [u16p, dp, i64]
        lib.oracle_double_to_f16_bits_array.argtypes = [dp, u16p, i64]
        lib.oracle_decode_f16state_fp64.argtypes = [i, i, i, i, i, i, fp, fp, fp, fp, fp, fp, u16p, dp, i, i, i]
        lib.oracle_conv_silu.argtypes = [i, i, i, i, dp, dp, dp, dp, ip, dp, dp]
        lib.oracle_ssd_scan.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, ip, dp, dp, dp, i]
        lib.oracle_gated_rmsnorm.argtypes = [i64, i, i, dp, dp, dp, ctypes.c_double, dp]
        lib.oracle_decode_f16state.argtypes = [i, i, i, i, i, i, fp, fp, fp, fp, fp, fp, u16p, dp, i, i, i]
        lib.oracle_dt_softplus.argtypes = [i64, i, dp, dp, dp]
        lib.oracle_ssd_scan_grad.argtypes = [i, i, i, i, i, i] + [dp] * 7 + [ip] + [dp] * 10 + [i]
        lib.oracle_dt_softplus_grad.argtypes = [i64, i, dp, dp, dp, dp]
        lib.oracle_dt_softplus_f32.argtypes = [i64, i, fp, fp, fp]
        lib.oracle_threads_used.restype = ctypes.c_int
        lib.oracle_threads_used.argtypes = [i]
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def threads_used(nthreads: int = 0) -> int:
    """Number of OpenMP threads the oracle runs with for this request (0 = default)."""
    return _load().oracle_threads_used(int(nthreads))


def f16_round(v):
    """Round fp64 values to the nearest IEEE binary16 value (ties to even)."""
    v = _f64(v)
    out = np.empty_like(v)
    _load().oracle_f16_round_array(_ptr(v, ctypes.c_double), _ptr(out, ctypes.c_double), v.size)
    return out


def f16_bits_to_double(bits):
    """binary16 bit patterns (uint16) -> their exact values as fp64."""
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    out = np.empty(bits.shape, np.float64)
    _load().oracle_f16_bits_to_double_array(_ptr(bits, ctypes.c_uint16), _ptr(out, ctypes.c_double), bits.size)
    return out


def double_to_f16_bits(v):
    """fp64 values that are binary16 values -> their bit patterns (uint16)."""
    v = _f64(v)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_double_to_f16_bits_array(_ptr(v, ctypes.c_double), _ptr(out, ctypes.c_uint16), v.size)
    return out


def conv_silu(xin, w, bias=None, state_in=None, seqlens=None):
    """Causal depthwise conv1d + SiLU.  xin (B, L, C); w (C, W); bias (C);
    state_in (B, C, W-1) history (None = zeros).  Returns (out (B, L, C),
    state_out (B, C, W-1)); rows t >= seqlens[b] of out are NaN."""
    xin, w = _f64(xin), _f64(w)
    B, L, C = xin.shape
    W = w.shape[1]
    bias = _f64(bias) if bias is not None else None
    state_in = _f64(state_in) if state_in is not None else None
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32)) if seqlens is not None else None
    out = np.full((B, L, C), np.nan)
    st = np.zeros((B, C, W - 1))
    _load().oracle_conv_silu(B, L, C, W, _ptr(xin, ctypes.c_double), _ptr(w, ctypes.c_double),
                             _ptr(bias, ctypes.c_double), _ptr(state_in, ctypes.c_double),
                             _ptr(sl, ctypes.c_int32), _ptr(out, ctypes.c_double), _ptr(st, ctypes.c_double))
    return out, st


def dt_softplus(raw, bias=None):
    """fp64 step sizes from raw dt: sp(raw + bias[h]) over the last axis (H)."""
    raw = _f64(raw)
    H = raw.shape[-1]
    bias = _f64(bias) if bias is not None else None
    assert bias is None or bias.shape == (H,)
    out = np.empty_like(raw)
    _load().oracle_dt_softplus(raw.size, H, _ptr(raw, ctypes.c_double), _ptr(bias, ctypes.c_double),
                               _ptr(out, ctypes.c_double))
    return out


def dt_softplus_f32(raw, bias=None):
    """Binary32 step sizes from binary32 raw dt: (float) sp((double) raw +
    (double) bias[h]), the decode step's contract."""
    raw = _f32(raw)
    H = raw.shape[-1]
    bias = _f32(bias) if bias is not None else None
    assert bias is None or bias.shape == (H,)
    out = np.empty_like(raw)
    _load().oracle_dt_softplus_f32(raw.size, H, _ptr(raw, ctypes.c_float), _ptr(bias, ctypes.c_float),
                                   _ptr(out, ctypes.c_float))
    return out


def ssd_scan(x, dt, A, Bm, Cm, D, h0=None, seqlens=None, nthreads: int = 0, dt_bias=None,
             dt_softplus_raw: bool = False):
    """Sequential fp64 selective-scan.  x (B, L, H, P); dt (B, L, H); A, D (H);
    Bm, Cm (B, L, G, N); h0 (B, H, P, N) or None.  With dt_softplus_raw, dt is
    the raw pre-activation and the step size is sp(dt + dt_bias[h]) in fp64.
    Returns (y (B, L, H, P), final state (B, H, P, N)); y rows t >= seqlens[b]
    are NaN."""
    if dt_softplus_raw:
        dt = dt_softplus(dt, dt_bias)
    x, dt, A, Bm, Cm, D = (_f64(a) for a in (x, dt, A, Bm, Cm, D))
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    assert dt.shape == (B, L, H) and Bm.shape == (B, L, G, N) and Cm.shape == Bm.shape
    assert A.shape == (H,) and D.shape == (H,) and H % G == 0
    h0 = _f64(h0) if h0 is not None else None
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32)) if seqlens is not None else None
    y = np.full((B, L, H, P), np.nan)
    hT = np.empty((B, H, P, N))
    work = np.empty((B * H, P, N))
    _load().oracle_ssd_scan(B, L, H, P, N, G, *(_ptr(a, ctypes.c_double) for a in (x, dt, A, Bm, Cm, D, h0)),
                            _ptr(sl, ctypes.c_int32), _ptr(y, ctypes.c_double), _ptr(hT, ctypes.c_double),
                            _ptr(work, ctypes.c_double), int(nthreads))
    return y, hT


def ssd_scan_grad(x, dt, A, Bm, Cm, D, dy, h0=None, dhT=None, seqlens=None, nthreads: int = 0, dt_bias=None,
                  dt_softplus_raw: bool = False):
    """Gradients of ssd_scan (fp64 reverse mode) for the loss whose gradients
    with respect to y and the final state are dy (B, L, H, P) and dhT (B, H,
    P, N) or None.  Returns a dict with dx, ddt, dB, dC, dA, dD, dh0 (and
    ddt_bias with a raw dt, when ddt is with respect to the raw dt)."""
    raw = dt
    if dt_softplus_raw:
        dt = dt_softplus(dt, dt_bias)
    x, dt, A, Bm, Cm, D, dy = (_f64(a) for a in (x, dt, A, Bm, Cm, D, dy))
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    assert dt.shape == (B, L, H) and Bm.shape == (B, L, G, N) and Cm.shape == Bm.shape and dy.shape == x.shape
    h0 = _f64(h0) if h0 is not None else None
    dhT = _f64(dhT) if dhT is not None else None
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32)) if seqlens is not None else None
    nt = threads_used(nthreads)
    out = dict(dx=np.empty((B, L, H, P)), ddt=np.empty((B, L, H)), dB=np.empty((B, L, G, N)),
               dC=np.empty((B, L, G, N)), dA=np.empty(H), dD=np.empty(H), dh0=np.empty((B, H, P, N)))
    work = np.empty(2 * B * L * H * N + 2 * B * H + nt * (L + 1) * P * N)
    _load().oracle_ssd_scan_grad(B, L, H, P, N, G, *(_ptr(a, ctypes.c_double) for a in (x, dt, A, Bm, Cm, D, h0)),
                                 _ptr(sl, ctypes.c_int32), _ptr(dy, ctypes.c_double), _ptr(dhT, ctypes.c_double),
                                 *(_ptr(out[k], ctypes.c_double) for k in ("dx", "ddt", "dB", "dC", "dA", "dD", "dh0")),
                                 _ptr(work, ctypes.c_double), int(nt))
    if dt_softplus_raw:
        raw = _f64(raw)
        bias = _f64(dt_bias) if dt_bias is not None else None
        g = np.empty_like(raw)
        _load().oracle_dt_softplus_grad(raw.size, H, _ptr(raw, ctypes.c_double), _ptr(bias, ctypes.c_double),
                                        _ptr(out["ddt"], ctypes.c_double), _ptr(g, ctypes.c_double))
        out["ddt"] = g
        out["ddt_bias"] = g.reshape(-1, H).sum(0)
    return out


def gated_rmsnorm(y, z, w, group, eps=1e-5):
    """g = y * silu(z); out = g / sqrt(mean over each group of `group`
    consecutive channels of g^2 + eps) * w.  y, z (..., C); w (C)."""
    y, z, w = _f64(y), _f64(z), _f64(w)
    C = y.shape[-1]
    assert C % group == 0
    T = y.size // C
    out = np.empty_like(y)
    _load().oracle_gated_rmsnorm(T, C, int(group), _ptr(y, ctypes.c_double), _ptr(z, ctypes.c_double),
                                 _ptr(w, ctypes.c_double), float(eps), _ptr(out, ctypes.c_double))
    return out


def mixer_core(xin, conv_w, conv_b, dt, A, D, z, norm_w, H, P, G, N, norm_group, eps=1e-5,
               conv_state=None, h0=None, seqlens=None, nthreads: int = 0, dt_bias=None,
               dt_softplus_raw: bool = False):
    """Full mixer core minus projections: conv1d+SiLU over xBC, split into
    x | B | C, sequential scan, gated RMSNorm.  xin (B, L, H*P + 2*G*N).
    Returns (out (B, L, H*P), final state, conv state out)."""
    Bsz, L, Cn = xin.shape
    assert Cn == H * P + 2 * G * N
    u, cst = conv_silu(xin, conv_w, conv_b, conv_state, seqlens)
    u = np.nan_to_num(u, nan=0.0)
    x = u[..., : H * P].reshape(Bsz, L, H, P)
    Bm = u[..., H * P: H * P + G * N].reshape(Bsz, L, G, N)
    Cm = u[..., H * P + G * N:].reshape(Bsz, L, G, N)
    y, hT = ssd_scan(x, dt, A, Bm, Cm, D, h0, seqlens, nthreads, dt_bias, dt_softplus_raw)
    yf = np.nan_to_num(y.reshape(Bsz, L, H * P), nan=0.0)
    out = gated_rmsnorm(yf, z, norm_w, norm_group, eps)
    if seqlens is not None:
        for b, n in enumerate(seqlens):
            out[b, n:] = np.nan
    return out, hT, cst


def decode_f16state(x, dt, A, Bm, Cm, D, state_bits, b_range=None, nthreads: int = 0, dt_bias=None,
                    dt_softplus_raw: bool = False):
    """Consecutive single-token steps with the state stored to binary16 after
    each step.  x (T, B, H, P); dt (T, B, H); Bm, Cm (T, B, G, N); A, D (H);
    state_bits (B, H, P, N) uint16 binary16 patterns, updated in place for the
    sequences in b_range = (lo, hi).  With dt_softplus_raw, dt is raw and the
    binary32 step size is dt_softplus_f32(dt, dt_bias).  Returns y (T, B, H, P)
    in fp64 (NaN outside b_range)."""
    if dt_softplus_raw:
        dt = dt_softplus_f32(dt, dt_bias)
    x, dt, A, Bm, Cm, D = (_f32(a) for a in (x, dt, A, Bm, Cm, D))
    T, B, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    assert state_bits.dtype == np.uint16 and state_bits.shape == (B, H, P, N) and state_bits.flags.c_contiguous
    lo, hi = b_range if b_range is not None else (0, B)
    y = np.full((T, B, H, P), np.nan)
    _load().oracle_decode_f16state(T, B, H, P, N, G, *(_ptr(a, ctypes.c_float) for a in (x, dt, A, Bm, Cm, D)),
                                   _ptr(state_bits, ctypes.c_uint16), _ptr(y, ctypes.c_double), int(lo), int(hi),
                                   int(nthreads))
    return y


def decode_f16state_fp64(x, dt, A, Bm, Cm, D, state_bits, b_range=None, nthreads: int = 0):
    """decode_f16state with every step taken in fp64 and rounded straight to
    binary16 (no binary32 stage).  Same arguments and layouts (dt positive);
    the state is updated in place for the sequences in b_range; returns y."""
    x, dt, A, Bm, Cm, D = (_f32(a) for a in (x, dt, A, Bm, Cm, D))
    T, B, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    assert state_bits.dtype == np.uint16 and state_bits.shape == (B, H, P, N) and state_bits.flags.c_contiguous
    lo, hi = b_range if b_range is not None else (0, B)
    y = np.full((T, B, H, P), np.nan)
    _load().oracle_decode_f16state_fp64(T, B, H, P, N, G, *(_ptr(a, ctypes.c_float) for a in (x, dt, A, Bm, Cm, D)),
                                        _ptr(state_bits, ctypes.c_uint16), _ptr(y, ctypes.c_double), int(lo),
                                        int(hi), int(nthreads))
    return y

"""Seeded synthetic inputs for the Mamba-2 mixer core.

This module is shared by the tests, the benchmark and the smoke check; it feeds
both the HIP path and the CPU oracle.  It holds input generation only: no step
of the scan, the convolution or the norm is computed here.

The pages score on WikiText-2 through trained weights (page
"Mamb2_8B_FP4_Recall_SQ3.25", section "Measured quality"), none of which is
available; the mixer core only ever sees activations, so seeded draws with the
shapes of one Mamba2-8B layer stand in for them:

  H=128 heads, P=64 head dim, N=128 state, G=8 groups, conv_dim 10240
  (these shapes make the page's "Recurrent state, convolution caches, and
  permutation table" byte count in section "Storage and runtime memory"
  decompose exactly), 2048-token reset windows and a final partial window
  of 1,955 tokens (section "Measured quality").

Draws are fp64 from numpy's PCG64 and rounded once to the I/O dtype.  Each
sequence of a batch has its own generator stream, so a sequence drawn alone
equals the same sequence drawn inside a batch.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F16 = np.float16
F32 = np.float32


def _rng(seed: int, *keys: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), *[int(k) for k in keys]])


def _softplus(v):
    return np.logaddexp(0.0, v)


@dataclass
class WindowShape:
    batch: int
    seqlen: int
    nheads: int = 128
    headdim: int = 64
    dstate: int = 128
    ngroups: int = 8
    chunk: int = 256
    io_dtype: type = F16
    dt_mode: str = "wide"          # "narrow": softplus(N(0,1) - 4); "wide": per-head dt0
    lengths: list = field(default_factory=list)   # per-sequence lengths ([] = all seqlen)

    @property
    def seqlens(self):
        return list(self.lengths) if self.lengths else [self.seqlen] * self.batch


# The five workloads (sizes from the problem statement of this path).
def tiny_scan() -> WindowShape:
    """Batch 1, L=256, H=4, P=64, N=16, G=1, chunk 64, fp32 I/O."""
    return WindowShape(1, 256, 4, 64, 16, 1, 64, F32, "narrow")


def layer_window() -> WindowShape:
    """One Mamba2-8B-shape layer over one 2048-token window, fp16 I/O."""
    return WindowShape(1, 2048, 128, 64, 128, 8, 256, F16, "wide")


def batched_windows() -> WindowShape:
    """Eight windows of the layer shape: seven of 2048 tokens, one of 1955."""
    return WindowShape(8, 2048, 128, 64, 128, 8, 256, F16, "wide", [2048] * 7 + [1955])


def mixer_window() -> WindowShape:
    """Batch 4, L=2048, the layer shape, behind conv1d+SiLU and gated RMSNorm."""
    return WindowShape(4, 2048, 128, 64, 128, 8, 256, F16, "wide")


DECODE = dict(batch=64, nheads=128, headdim=64, dstate=128, ngroups=8, steps=1024)


def head_params(nheads: int, seed: int, dt_mode: str):
    """A (f32, negative), D (f32) and, for the wide dt mode, dt0 per head."""
    r = _rng(seed, 0)
    A = -np.exp(r.uniform(0.0, math.log(16.0), nheads))
    D = r.standard_normal(nheads)
    dt0 = np.exp(r.uniform(math.log(1e-3), math.log(1e-1), nheads))
    return A.astype(F32), D.astype(F32), dt0


def _dt_from_noise(noise, dt_mode, dt0):
    if dt_mode == "narrow":
        return _softplus(noise - 4.0)
    return _softplus(noise + np.log(np.expm1(dt0)))


def _raw_dt_from_noise(noise, dt_mode):
    """The pre-activation that _dt_from_noise passes through softplus, less the
    per-head bias (see dt_bias)."""
    return noise - 4.0 if dt_mode == "narrow" else noise


def dt_bias(dt_mode, dt0):
    """Per-head f32 bias that, added to the raw draw, gives the softplus
    argument of _dt_from_noise: log(expm1(dt0)) (narrow mode: zero)."""
    if dt_mode == "narrow":
        return np.zeros(len(dt0), F32)
    return np.log(np.expm1(dt0)).astype(F32)


def window_inputs(s: WindowShape, seed: int, raw_dt: bool = False):
    """x (B,L,H,P), dt (B,L,H), Bm, Cm (B,L,G,N) in the I/O dtype; A, D (H) f32.
    raw_dt: dt holds the raw draw and dt_bias (H) f32 is added (same noise)."""
    B, L, H, P, N, G = s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups
    A, D, dt0 = head_params(H, seed, s.dt_mode)
    x = np.empty((B, L, H, P), s.io_dtype)
    dt = np.empty((B, L, H), s.io_dtype)
    Bm = np.empty((B, L, G, N), s.io_dtype)
    Cm = np.empty((B, L, G, N), s.io_dtype)
    for b in range(B):
        r = _rng(seed, 1, b)
        x[b] = r.standard_normal((L, H, P))
        noise = r.standard_normal((L, H))
        dt[b] = _raw_dt_from_noise(noise, s.dt_mode) if raw_dt else _dt_from_noise(noise, s.dt_mode, dt0)
        Bm[b] = r.standard_normal((L, G, N)) / math.sqrt(N)
        Cm[b] = r.standard_normal((L, G, N)) / math.sqrt(N)
    out = dict(x=x, dt=dt, B=Bm, C=Cm, A=A, D=D)
    if raw_dt:
        out["dt_bias"] = dt_bias(s.dt_mode, dt0)
    return out


def mixer_inputs(s: WindowShape, seed: int, raw_dt: bool = False):
    """Raw xBC (B,L,H*P+2*G*N) ~ N(0,1), conv weights (conv_dim, 4) ~ N(0, 0.5)
    as f32 with zero bias, dt (B,L,H) as for the layer window, z ~ N(0,1),
    norm weight 1."""
    B, L, H, P, N, G = s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups
    Cn = H * P + 2 * G * N
    A, D, dt0 = head_params(H, seed, s.dt_mode)
    r = _rng(seed, 3)
    conv_w = (r.standard_normal((Cn, 4)) * 0.5).astype(F32)
    conv_b = np.zeros(Cn, F32)
    xBC = np.empty((B, L, Cn), s.io_dtype)
    dt = np.empty((B, L, H), s.io_dtype)
    z = np.empty((B, L, H * P), s.io_dtype)
    for b in range(B):
        r = _rng(seed, 4, b)
        xBC[b] = r.standard_normal((L, Cn))
        noise = r.standard_normal((L, H))
        dt[b] = _raw_dt_from_noise(noise, s.dt_mode) if raw_dt else _dt_from_noise(noise, s.dt_mode, dt0)
        z[b] = r.standard_normal((L, H * P))
    out = dict(xBC=xBC, conv_w=conv_w, conv_b=conv_b, dt=dt, z=z,
               norm_w=np.ones(H * P, F32), A=A, D=D)
    if raw_dt:
        out["dt_bias"] = dt_bias(s.dt_mode, dt0)
    return out


def decode_params(seed: int, batch=64, nheads=128, headdim=64, dstate=128):
    """A, D, dt0 per head and the fp32 seed state (B,H,P,N) ~ N(0, 0.1)."""
    A, D, dt0 = head_params(nheads, seed, "wide")
    state = (_rng(seed, 2).standard_normal((batch, nheads, headdim, dstate)) * 0.1).astype(F32)
    return dict(A=A, D=D, dt0=dt0, state=state)


def decode_step_inputs(seed: int, step: int, dt0, batch=64, nheads=128, headdim=64, dstate=128,
                       ngroups=8, io_dtype=F16, raw_dt=False):
    """Per-step x (B,H,P), dt (B,H), Bm, Cm (B,G,N), drawn like the layer window
    (raw_dt: dt is the raw draw; the bias is dt_bias("wide", dt0))."""
    r = _rng(seed, 5, step)
    x = r.standard_normal((batch, nheads, headdim)).astype(io_dtype)
    noise = r.standard_normal((batch, nheads))
    dt = (noise if raw_dt else _dt_from_noise(noise, "wide", dt0)).astype(io_dtype)
    Bm = (r.standard_normal((batch, ngroups, dstate)) / math.sqrt(dstate)).astype(io_dtype)
    Cm = (r.standard_normal((batch, ngroups, dstate)) / math.sqrt(dstate)).astype(io_dtype)
    return dict(x=x, dt=dt, B=Bm, C=Cm)

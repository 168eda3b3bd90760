"""Helpers shared by the GPU tests and the benchmark: run the HIP path from
numpy inputs and measure errors against the oracle.  No arithmetic of the
method lives here."""
from __future__ import annotations

import numpy as np
import torch

import mamba_ssd_scan_amd as m2

DEV = torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def window_checked(dt, A, D, y, workspace, **kw):
    """mamba2_conv_scan_window, then the workspace's error word, which must
    be clear (every segment hand-off completed)."""
    m2.conv_scan_window(dt, A, D, y, workspace, **kw)
    flags = m2.window_take_error(workspace)
    assert flags == 0, f"window hand-off error word {flags:#x}"


def slice_err(got, ref, nlead):
    """max over slices of max|got-ref| / max|ref|; a slice is one index of the
    first `nlead` axes (e.g. (b, h)).  NaN/Inf anywhere in got -> inf."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.all(np.isfinite(got)):
        return float("inf")
    lead = int(np.prod(got.shape[:nlead]))
    g = got.reshape(lead, -1)
    r = ref.reshape(lead, -1)
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((np.abs(g - r).max(axis=1) / den).max())


def raw_dt_args(inp):
    """Keyword arguments that hand a raw dt and its bias to the kernels (empty
    for a positive dt)."""
    if "dt_bias" not in inp:
        return {}
    return dict(dt_softplus=True, dt_bias=to_dev(inp["dt_bias"]))


def run_window(inp, chunk, seqlens=None, state_in=None, want_state=True, ws=None, y_fill=None, segments=0):
    """Run the window scan on the GPU from numpy inputs x, dt, B, C, A, D."""
    x, dt, Bm, Cm = (to_dev(inp[k]) for k in ("x", "dt", "B", "C"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    Bsz, L, H, P = inp["x"].shape
    G, N = inp["B"].shape[2], inp["B"].shape[3]
    y = torch.empty((Bsz, L, H * P), dtype=x.dtype, device=DEV)
    if y_fill is not None:
        y.fill_(y_fill)
    hT = torch.empty((Bsz, H, P, N), dtype=torch.float32, device=DEV) if want_state else None
    sl = torch.tensor(seqlens, dtype=torch.int32, device=DEV) if seqlens is not None else None
    h0 = to_dev(np.asarray(state_in, np.float32)) if state_in is not None else None
    if ws is None:
        dims = m2.make_dims(Bsz, L, H, P, N, G, chunk, io_dtype=m2.F16 if x.dtype == torch.float16 else m2.F32)
        ws = m2.alloc_workspace(dims, DEV)
    window_checked(dt, A, D, y, ws, x=x, B=Bm, C=Cm, state_in=h0, state_out=hT, seqlens=sl, chunk=chunk,
                        segments=segments, **raw_dt_args(inp))
    torch.cuda.synchronize()
    return y.cpu().numpy().reshape(Bsz, L, H, P), (hT.cpu().numpy() if want_state else None)


def run_requant(inp, seqlens=None, state_in=None, y_fill=None):
    """Run the per-token-requantized window on the GPU from numpy inputs."""
    x, dt, Bm, Cm = (to_dev(inp[k]) for k in ("x", "dt", "B", "C"))
    A, D = to_dev(inp["A"]), to_dev(inp["D"])
    Bsz, L, H, P = inp["x"].shape
    N = inp["B"].shape[3]
    y = torch.empty((Bsz, L, H * P), dtype=x.dtype, device=DEV)
    if y_fill is not None:
        y.fill_(y_fill)
    hT = torch.empty((Bsz, H, P, N), dtype=torch.float32, device=DEV)
    sl = torch.tensor(seqlens, dtype=torch.int32, device=DEV) if seqlens is not None else None
    h0 = to_dev(np.asarray(state_in, np.float32)) if state_in is not None else None
    m2.requant_window(dt, A, D, y, x=x, B=Bm, C=Cm, state_in=h0, state_out=hT, seqlens=sl, **raw_dt_args(inp))
    torch.cuda.synchronize()
    return y.cpu().numpy().reshape(Bsz, L, H, P), hT.cpu().numpy()


def projection_rows(xbc, lead, tail):
    """xBC as the column slice [lead, lead + Cn) of wider rows, the columns
    around it NaN, so that a read outside the slice shows in the output."""
    Cn = xbc.shape[-1]
    wide = torch.full(xbc.shape[:-1] + (lead + Cn + tail,), float("nan"), dtype=xbc.dtype, device=xbc.device)
    wide[..., lead:lead + Cn] = xbc
    return wide[..., lead:lead + Cn]


def run_mixer(inp, H, P, G, N, chunk, norm_group, seqlens=None, conv_state_in=None, state_in=None,
              want_conv_state=True, segments=0, xbc_in_rows=None, want_state=True):
    xBC = to_dev(inp["xBC"])
    if xbc_in_rows is not None:
        xBC = projection_rows(xBC, *xbc_in_rows)
    Bsz, L, Cn = inp["xBC"].shape
    y = torch.empty((Bsz, L, H * P), dtype=xBC.dtype, device=DEV)
    hT = torch.empty((Bsz, H, P, N), dtype=torch.float32, device=DEV) if want_state else None
    cso = torch.empty((Bsz, Cn, 3), dtype=xBC.dtype, device=DEV) if want_conv_state else None
    csi = to_dev(conv_state_in) if conv_state_in is not None else None
    h0 = to_dev(np.asarray(state_in, np.float32)) if state_in is not None else None
    sl = torch.tensor(seqlens, dtype=torch.int32, device=DEV) if seqlens is not None else None
    dims = m2.make_dims(Bsz, L, H, P, N, G, chunk, conv_width=4, norm_group=norm_group,
                        io_dtype=m2.F16 if xBC.dtype == torch.float16 else m2.F32)
    ws = m2.alloc_workspace(dims, DEV)
    window_checked(to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]), y, ws, xBC=xBC,
                        conv_w=to_dev(inp["conv_w"]), conv_b=to_dev(inp["conv_b"]), conv_state_in=csi,
                        conv_state_out=cso, state_in=h0, state_out=hT, seqlens=sl,
                        z=to_dev(inp["z"]) if norm_group else None,
                        norm_w=to_dev(inp["norm_w"]) if norm_group else None,
                        chunk=chunk, norm_group=norm_group, ngroups=G, dstate=N, headdim=P, segments=segments,
                        **raw_dt_args(inp))
    torch.cuda.synchronize()
    return (y.cpu().numpy(), hT.cpu().numpy() if want_state else None,
            cso.cpu().numpy() if want_conv_state else None)


def pack_rows(a, lens):
    """Rows 0 .. lens[b]-1 of each sequence of a padded (B, L, ...) array,
    concatenated into a packed (T, ...) array."""
    return np.ascontiguousarray(np.concatenate([a[b, :n] for b, n in enumerate(lens)], 0))


def cu_of(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def unpack_rows(a, lens, L, fill=np.nan):
    """Inverse of pack_rows: (T, ...) -> (B, L, ...), rows past a length = fill."""
    out = np.full((len(lens), L) + a.shape[1:], fill, dtype=np.float64)
    for b, (s, n) in enumerate(zip(cu_of(lens)[:-1], lens)):
        out[b, :n] = a[s:s + n]
    return out


def run_window_packed(inp, lens, chunk, state_in=None, spare_rows=16, fill=12345.0, segments=0):
    """The window scan on packed rows built from padded numpy inputs.  y gets
    spare_rows extra rows filled with `fill`; returns (y packed incl. spare
    rows, final state)."""
    Bsz, L, H, P = inp["x"].shape
    G, N = inp["B"].shape[2], inp["B"].shape[3]
    x, dt, Bm, Cm = (to_dev(pack_rows(inp[k], lens)) for k in ("x", "dt", "B", "C"))
    T = dt.shape[0]
    y = torch.full((T + spare_rows, H * P), fill, dtype=x.dtype, device=DEV)
    hT = torch.empty((Bsz, H, P, N), dtype=torch.float32, device=DEV)
    cu = to_dev(cu_of(lens))
    h0 = to_dev(np.asarray(state_in, np.float32)) if state_in is not None else None
    dims = m2.make_dims(Bsz, L, H, P, N, G, chunk, io_dtype=m2.F16 if x.dtype == torch.float16 else m2.F32,
                        packed_tokens=T)
    ws = m2.alloc_workspace(dims, DEV)
    window_checked(dt, to_dev(inp["A"]), to_dev(inp["D"]), y, ws, x=x, B=Bm, C=Cm, state_in=h0,
                        state_out=hT, chunk=chunk, segments=segments, cu_seqlens=cu, max_seqlen=L,
                        **raw_dt_args(inp))
    torch.cuda.synchronize()
    return y.cpu().numpy(), hT.cpu().numpy()

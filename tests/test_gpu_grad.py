"""GPU parity of the scan's backward pass (mamba2_scan_grad) through the C
ABI, against the oracle's fp64 reverse mode (``oracle.ssd_scan_grad``, pinned
by central differences in test_oracle_pins.py).

The kernels use a different but equivalent form of the gradient (the
log-decay sums, with no past state kept), in binary32 with the step size's
decay from the fast exponential; the bar is a per-slice error of 1e-3 of the
slice's largest value -- slices: (sequence, head) for dx, ddt and dstate_in,
(sequence, group) for dB and dC, the whole vector for dA and dD.
"""
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import mamba_ssd_scan_amd as m2  # noqa: E402
from tests.gpu_helpers import DEV, slice_err, to_dev  # noqa: E402

G_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def grad_case(seed, Bsz, L, H, N, G, dtype=np.float16, dt_mode="wide", raw_dt=False, with_h0=True, with_dhT=True):
    s = synth.WindowShape(Bsz, L, H, 64, N, G, 256, dtype, dt_mode)
    inp = synth.window_inputs(s, seed, raw_dt=raw_dt)
    r = np.random.default_rng(seed + 7)
    inp["dy"] = r.standard_normal((Bsz, L, H, 64)).astype(dtype)
    inp["h0"] = (r.standard_normal((Bsz, H, 64, N)) * 0.3).astype(np.float32) if with_h0 else None
    inp["dhT"] = (r.standard_normal((Bsz, H, 64, N)) * 0.3).astype(np.float32) if with_dhT else None
    return inp


def run_grad(inp, seqlens=None):
    Bsz, L, H, P = inp["x"].shape
    G, N = inp["B"].shape[2], inp["B"].shape[3]
    raw = "dt_bias" in inp
    dims = m2.make_dims(Bsz, L, H, P, N, G, 256, io_dtype=m2.F16 if inp["x"].dtype == np.float16 else m2.F32,
                        dt_softplus=int(raw))
    ws = m2.alloc_scan_grad_workspace(dims, DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    out = dict(dx=torch.full((Bsz, L, H, P), 7.0, **f32), ddt=torch.full((Bsz, L, H), 7.0, **f32),
               dB=torch.full((Bsz, L, G, N), 7.0, **f32), dC=torch.full((Bsz, L, G, N), 7.0, **f32),
               dA=torch.empty(H, **f32), dD=torch.empty(H, **f32), dh0=torch.empty((Bsz, H, P, N), **f32))
    if raw:
        out["ddt_bias"] = torch.empty(H, **f32)
    sl = torch.tensor(seqlens, dtype=torch.int32, device=DEV) if seqlens is not None else None
    m2.scan_grad(to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]), to_dev(inp["dy"]), ws, x=to_dev(inp["x"]),
                 B=to_dev(inp["B"]), C=to_dev(inp["C"]), dx=out["dx"], ddt=out["ddt"], dB=out["dB"], dC=out["dC"],
                 dA=out["dA"], dD=out["dD"], dstate_in=out["dh0"],
                 state_in=to_dev(inp["h0"]) if inp["h0"] is not None else None, seqlens=sl,
                 dstate_out=to_dev(inp["dhT"]) if inp["dhT"] is not None else None, dt_softplus=raw,
                 dt_bias=to_dev(inp["dt_bias"]) if raw else None, ddt_bias=out.get("ddt_bias"))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def oracle_grad(inp, seqlens=None):
    raw = "dt_bias" in inp
    return oracle.ssd_scan_grad(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["dy"],
                                h0=inp["h0"], dhT=inp["dhT"], seqlens=seqlens, dt_bias=inp.get("dt_bias"),
                                dt_softplus_raw=raw)


def compare(name, got, ref):
    errs = {
        "dx": slice_err(np.transpose(got["dx"], (0, 2, 1, 3)), np.transpose(ref["dx"], (0, 2, 1, 3)), 2),
        "ddt": slice_err(np.transpose(got["ddt"], (0, 2, 1)), np.transpose(ref["ddt"], (0, 2, 1)), 2),
        "dB": slice_err(np.transpose(got["dB"], (0, 2, 1, 3)), np.transpose(ref["dB"], (0, 2, 1, 3)), 2),
        "dC": slice_err(np.transpose(got["dC"], (0, 2, 1, 3)), np.transpose(ref["dC"], (0, 2, 1, 3)), 2),
        "dA": slice_err(got["dA"][None], ref["dA"][None], 1),
        "dD": slice_err(got["dD"][None], ref["dD"][None], 1),
        "dh0": slice_err(got["dh0"], ref["dh0"], 2),
    }
    if "ddt_bias" in ref:
        errs["ddt_bias"] = slice_err(got["ddt_bias"][None], ref["ddt_bias"][None], 1)
    say(f"[grad] {name}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= G_TOL, (k, v)


@pytest.mark.parametrize("N", [16, 64, 128])
def test_scan_grad_small_ragged(N):
    inp = grad_case(500 + N, 2, 300, 8, N, 2)
    lens = [300, 177]
    say(f"[grad] N={N} lengths {lens}")
    got = run_grad(inp, lens)
    ref = oracle_grad(inp, lens)
    compare(f"N={N}", got, ref)
    # rows past the length are zero
    for k in ("dx", "ddt", "dB", "dC"):
        assert np.all(got[k][1, 177:] == 0), k


def test_scan_grad_fp32_narrow_no_state():
    inp = grad_case(510, 1, 256, 4, 16, 1, dtype=np.float32, dt_mode="narrow", with_h0=False, with_dhT=False)
    say("[grad] fp32 tiny, no initial state, no final-state gradient")
    compare("fp32 tiny", run_grad(inp), oracle_grad(inp))


def test_scan_grad_raw_dt():
    inp = grad_case(520, 2, 200, 8, 128, 2, raw_dt=True)
    lens = [200, 63]
    say(f"[grad] raw dt lengths {lens}")
    compare("raw dt", run_grad(inp, lens), oracle_grad(inp, lens))


def test_scan_grad_zero_length_sequence():
    inp = grad_case(530, 2, 64, 4, 64, 2)
    got = run_grad(inp, [64, 0])
    ref = oracle_grad(inp, [64, 0])
    compare("zero length", got, ref)
    assert np.array_equal(got["dh0"][1], inp["dhT"][1])
    for k in ("dx", "ddt", "dB", "dC"):
        assert np.all(got[k][1] == 0), k


def test_scan_grad_layer_window_sampled():
    # the layer window's shape; the oracle runs on the 16 heads of group 5
    s = synth.layer_window()
    inp = grad_case(540, 1, s.seqlen, s.nheads, s.dstate, s.ngroups)
    say("[grad] layer window L=2048 H=128 N=128")
    got = run_grad(inp)
    hs = slice(80, 96)
    sub = dict(x=inp["x"][:, :, hs], dt=inp["dt"][:, :, hs], A=inp["A"][hs], D=inp["D"][hs],
               B=inp["B"][:, :, 5:6], C=inp["C"][:, :, 5:6], dy=inp["dy"][:, :, hs], h0=inp["h0"][:, hs],
               dhT=inp["dhT"][:, hs])
    ref = oracle_grad(sub)
    gsub = dict(dx=got["dx"][:, :, hs], ddt=got["ddt"][:, :, hs], dB=got["dB"][:, :, 5:6], dC=got["dC"][:, :, 5:6],
                dA=got["dA"][hs], dD=got["dD"][hs], dh0=got["dh0"][:, hs])
    compare("layer window, heads 80..95", gsub, ref)

"""GPU check of the one-token mixer step that allocates nothing
(mamba2_mixer_decode_step_noalloc): through the C ABI it must give exactly
what mamba2_mixer_decode_step gives with a caller workspace (the same
kernels run on the same inputs), on two calls in a row, the second with a
smaller batch, so that the fixed per-GPU array is reused with a different
layout of its counters and partial sums."""
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import mamba_ssd_scan_amd as m2  # noqa: E402
from tests.gpu_helpers import DEV, to_dev  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def inputs(seed, Bsz, H, G, N, P=64):
    s = synth.WindowShape(Bsz, 1, H, P, N, G, 256, np.float16, "wide")
    inp = synth.mixer_inputs(s, seed, raw_dt=True)
    Cn = H * P + 2 * G * N
    r = np.random.default_rng(seed + 1)
    conv_b = (r.standard_normal(Cn) * 0.1).astype(np.float32)
    norm_w = r.uniform(0.5, 1.5, H * P).astype(np.float32)
    cs0 = r.standard_normal((Bsz, Cn, 3)).astype(np.float16)
    h0 = (r.standard_normal((Bsz, H, P, N)) * 0.1).astype(np.float16)
    return dict(xBC=inp["xBC"][:, 0], conv_w=inp["conv_w"], conv_b=conv_b, dt=inp["dt"][:, 0],
                dt_bias=inp["dt_bias"], A=inp["A"], D=inp["D"], z=inp["z"][:, 0], norm_w=norm_w, cs0=cs0, h0=h0)


def one_step(inp, H, G, N, noalloc, norm_group):
    Bsz = inp["xBC"].shape[0]
    cs = to_dev(inp["cs0"]).clone()
    st = to_dev(inp["h0"]).clone()
    y = torch.full((Bsz, H * 64), float("nan"), dtype=torch.float16, device=DEV)
    args = (to_dev(inp["xBC"]), to_dev(inp["conv_w"]), cs, to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]),
            st, y)
    kw = dict(conv_b=to_dev(inp["conv_b"]), ngroups=G, dstate=N, norm_group=norm_group, dt_softplus=True,
              dt_bias=to_dev(inp["dt_bias"]))
    if norm_group:
        kw.update(z=to_dev(inp["z"]), norm_w=to_dev(inp["norm_w"]))
    if noalloc:
        m2.mixer_decode_step_noalloc(*args, **kw)
    else:
        dims = m2.mixer_decode_dims(Bsz, H, 64, N, G, norm_group, m2.F16, m2.F16, dt_softplus=True)
        ws = m2.alloc_mixer_decode_workspace(dims, DEV)
        m2.mixer_decode_step(*args, ws, **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy(), st.cpu().numpy(), cs.cpu().numpy()


@pytest.mark.parametrize("norm_group", [8192, 1024])
def test_noalloc_step_equals_workspace_step(norm_group):
    H, G, N = 128, 8, 128
    for call, Bsz in enumerate((64, 24)):     # the second call is smaller
        say(f"noalloc mixer step: call {call}, batch {Bsz}, norm_group {norm_group}")
        inp = inputs(4100 + call, Bsz, H, G, N)
        ref = one_step(inp, H, G, N, False, norm_group)
        got = one_step(inp, H, G, N, True, norm_group)
        for name, a, b in zip(("y", "state", "conv_state"), got, ref):
            assert np.all(np.isfinite(a.astype(np.float64))), name
            same = np.mean(a.view(np.uint16) == b.view(np.uint16))
            say(f"  {name}: identical fraction {same:.6f}")
            assert same == 1.0, name

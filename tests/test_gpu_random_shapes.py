"""GPU parity of the window scan through the C ABI over randomly drawn small
configurations, against the fp64 oracle: batch, window length (from 1
token), heads and groups, state size, chunk, segment count, ragged lengths
(zero included), raw or positive dt, an initial state or none, binary16 or
binary32 I/O.  Each case prints its draw before it runs.  Bars as in the
other parity tests: 2e-3 on y per (sequence, head), 1e-3 on the final
state per (sequence, head); rows past a length keep their canary."""
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
from tests.gpu_helpers import DEV, slice_err, to_dev, window_checked  # noqa: E402

Y_TOL, S_TOL = 2e-3, 1e-3


EDGES = {
    # a one-token window beside an empty sequence, raw dt and an initial state
    16: dict(B=2, L=1, H=8, G=2, N=128, chunk=64, segments=2, lens=[1, 0], raw=True, h0=True, dtype=np.float16),
    # a long window with an empty middle sequence, three segments of 64-token chunks
    17: dict(B=3, L=700, H=4, G=1, N=16, chunk=64, segments=3, lens=[700, 0, 699], raw=False, h0=True,
             dtype=np.float32),
}


def draw(seed):
    if seed in EDGES:
        return dict(EDGES[seed])
    r = np.random.default_rng(7000 + seed)
    B = int(r.integers(1, 5))
    L = int(r.choice([1, 31, 32, 33, 100, 255, 256, 257, 511, 700]))
    H = int(r.choice([4, 8, 12, 16]))
    G = int(r.choice([g for g in (1, 2, 4) if H % g == 0]))
    N = int(r.choice([16, 64, 128]))
    chunk = int(r.choice([64, 128, 256]))
    segments = int(r.choice([0, 1, 2, 3]))
    lens = [int(v) for v in r.integers(0, L + 1, size=B)]
    lens[int(r.integers(0, B))] = L               # one full-length sequence
    raw = bool(r.integers(0, 2))
    h0 = bool(r.integers(0, 2))
    dtype = np.float16 if r.integers(0, 3) else np.float32
    return dict(B=B, L=L, H=H, G=G, N=N, chunk=chunk, segments=segments, lens=lens, raw=raw, h0=h0, dtype=dtype)


@pytest.mark.parametrize("seed", range(18))
def test_window_random_configuration(seed):
    c = draw(seed)
    print(f"[random] seed {seed}: {c}", flush=True)
    sys.stdout.flush()
    s = synth.WindowShape(c["B"], c["L"], c["H"], 64, c["N"], c["G"], c["chunk"], c["dtype"], "wide")
    inp = synth.window_inputs(s, 7100 + seed, raw_dt=c["raw"])
    B, L, H, N = c["B"], c["L"], c["H"], c["N"]
    h0 = (np.random.default_rng(7200 + seed).standard_normal((B, H, 64, N)) * 0.5).astype(np.float32) if c["h0"] else None
    tdt = torch.float16 if c["dtype"] == np.float16 else torch.float32
    y = torch.full((B, L, H * 64), 1234.0, dtype=tdt, device=DEV)
    hT = torch.empty((B, H, 64, N), dtype=torch.float32, device=DEV)
    dims = m2.make_dims(B, L, H, 64, N, c["G"], c["chunk"], io_dtype=m2.F16 if tdt == torch.float16 else m2.F32,
                        segments=c["segments"], dt_softplus=int(c["raw"]))
    ws = m2.alloc_workspace(dims, DEV)
    kw = dict(dt_softplus=True, dt_bias=to_dev(inp["dt_bias"])) if c["raw"] else {}
    dt = to_dev(inp["dt"])
    if "dt_cols" in c:
        # dt as columns [off, off + H) of wider rows (width H + extra)
        off, extra = c["dt_cols"]
        wide = torch.zeros((B, L, H + extra), dtype=dt.dtype, device=DEV)
        wide[:, :, off:off + H] = dt
        dt = wide[:, :, off:off + H]
    window_checked(dt, to_dev(inp["A"]), to_dev(inp["D"]), y, ws, x=to_dev(inp["x"]),
                        B=to_dev(inp["B"]), C=to_dev(inp["C"]), state_in=to_dev(h0) if h0 is not None else None,
                        state_out=hT, seqlens=torch.tensor(c["lens"], dtype=torch.int32, device=DEV),
                        chunk=c["chunk"], segments=c["segments"], **kw)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64).reshape(B, L, H, 64)
    yr, hr = oracle.ssd_scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], h0=h0, seqlens=c["lens"],
                             dt_bias=inp.get("dt_bias"), dt_softplus_raw=c["raw"])
    ey = 0.0
    for b, n in enumerate(c["lens"]):
        assert np.all(got[b, n:] == 1234.0), b
        if n > 0:
            ey = max(ey, slice_err(np.transpose(got[b:b + 1, :n], (0, 2, 1, 3)), np.transpose(yr[b:b + 1, :n], (0, 2, 1, 3)), 2))
    es = slice_err(hT.cpu().numpy(), hr, 2)
    print(f"[random] seed {seed}: y {ey:.3e} state {es:.3e}", flush=True)
    assert ey <= Y_TOL and es <= S_TOL


def test_window_one_token_cancelling_factor_f32():
    # draw 304 of a wider sweep: three one-token binary32 windows with a raw
    # dt; sequence 1, head 5 has dt C.B = +0.0027 against D = -0.0037, so
    # every output of that slice is x times a factor of -0.00099 (binary32
    # windows take the exact binary32 recurrence, with no binary16 operand)
    test_window_random_configuration(304)


@pytest.mark.parametrize("seed", [400, 401, 402, 403])
def test_window_random_configuration_more(seed):
    test_window_random_configuration(seed)


@pytest.mark.parametrize("H,G,off,extra", [(12, 4, 1, 3), (4, 4, 1, 2), (8, 8, 3, 6), (16, 2, 1, 1)])
def test_window_dt_column_slice(H, G, off, extra):
    # dt read in place from wider rows at an odd element offset, with odd and
    # even row strides and groups of 1, 2 or 3 heads (blocks of heads that
    # start at odd head indices)
    c = dict(B=2, L=300, H=H, G=G, N=128, chunk=64, segments=2, lens=[300, 177], raw=True, h0=True,
             dtype=np.float16, dt_cols=(off, extra))
    seed = 500 + H + G + off + extra
    EDGES[seed] = c
    try:
        test_window_random_configuration(seed)
    finally:
        del EDGES[seed]

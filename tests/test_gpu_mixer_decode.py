"""GPU parity of the fused one-token mixer step (conv1d + SiLU with the conv
history rolled in place, the state-space step, the gated RMSNorm) through the
C ABI, against the CPU oracle.

T consecutive one-token steps equal the whole-window mixer over those T
tokens (pinned for the oracle in test_oracle_pins.py), so the oracle for a
run of steps is ``oracle.mixer_core`` over the same tokens with the same
initial conv history and state.  With a binary16 resident state the oracle is
the same composition with the binary32 decode contract: conv + SiLU in fp64,
rounded to the I/O type as the kernel stages it, then ``decode_f16state``,
then the norm.

Bar: per-slice error <= 2e-3 on the output and <= 1e-3 on the final state
(slices: (sequence, norm group) over the steps; (sequence, head) for y and
the state); the conv history is raw data and must match exactly.
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
from tests.gpu_helpers import DEV, slice_err, to_dev, window_checked  # noqa: E402

Y_TOL, S_TOL = 2e-3, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def case(seed, Bsz, T, H, G, N, raw_dt=False, P=64):
    """T tokens of mixer inputs, an initial conv history and an initial state."""
    s = synth.WindowShape(Bsz, T, H, P, N, G, 256, np.float16, "wide")
    inp = synth.mixer_inputs(s, seed, raw_dt=raw_dt)
    Cn = H * P + 2 * G * N
    r = np.random.default_rng(seed + 1)
    inp["conv_b"] = (r.standard_normal(Cn) * 0.1).astype(np.float32)
    inp["norm_w"] = r.uniform(0.5, 1.5, H * P).astype(np.float32)
    cs0 = r.standard_normal((Bsz, Cn, 3)).astype(np.float16)
    h0 = (r.standard_normal((Bsz, H, P, N)) * 0.1).astype(np.float32)
    return inp, cs0, h0


def run_steps(inp, cs0, h0, H, G, N, norm_group, state_dtype, P=64):
    """T fused steps on the GPU; returns (y (B,T,H*P), final state as f32,
    final conv history)."""
    Bsz, T, Cn = inp["xBC"].shape
    cs = to_dev(cs0).clone()
    st = to_dev(h0).to(torch.float16 if state_dtype == m2.F16 else torch.float32)
    if state_dtype == m2.F16:   # f32 seed rounded once to the resident type
        st16 = torch.empty((Bsz, H, P, N), dtype=torch.float16, device=DEV)
        m2.state_load(to_dev(h0), st16)
        st = st16
    dims = m2.mixer_decode_dims(Bsz, H, P, N, G, norm_group, m2.F16, state_dtype)
    ws = m2.alloc_mixer_decode_workspace(dims, DEV)
    A, D, w, b = (to_dev(inp[k]) for k in ("A", "D", "conv_w", "conv_b"))
    nw = to_dev(inp["norm_w"])
    raw = "dt_bias" in inp
    bias = to_dev(inp["dt_bias"]) if raw else None
    ys = []
    for t in range(T):
        y = torch.empty((Bsz, H * P), dtype=torch.float16, device=DEV)
        m2.mixer_decode_step(to_dev(np.ascontiguousarray(inp["xBC"][:, t])), w, cs,
                             to_dev(np.ascontiguousarray(inp["dt"][:, t])), A, D, st, y, ws, conv_b=b,
                             z=to_dev(np.ascontiguousarray(inp["z"][:, t])) if norm_group else None,
                             norm_w=nw if norm_group else None, ngroups=G, dstate=N, norm_group=norm_group,
                             dt_softplus=raw, dt_bias=bias)
        ys.append(y)
    torch.cuda.synchronize()
    y = torch.stack(ys, 1).cpu().numpy()
    return y, st.float().cpu().numpy(), cs.cpu().numpy()


def oracle_f32(inp, cs0, h0, H, G, N, norm_group, P=64):
    """Whole-window oracle over the same tokens: (y or normed out, state, conv history)."""
    raw = "dt_bias" in inp
    kw = dict(dt_bias=inp.get("dt_bias"), dt_softplus_raw=raw)
    if norm_group:
        return oracle.mixer_core(inp["xBC"], inp["conv_w"], inp["conv_b"], inp["dt"], inp["A"], inp["D"], inp["z"],
                                 inp["norm_w"], H, P, G, N, norm_group, conv_state=cs0, h0=h0, **kw)
    Bsz, T, _ = inp["xBC"].shape
    u, cs = oracle.conv_silu(inp["xBC"], inp["conv_w"], inp["conv_b"], cs0)
    y, hT = oracle.ssd_scan(u[..., :H * P].reshape(Bsz, T, H, P), inp["dt"], inp["A"],
                            u[..., H * P:H * P + G * N].reshape(Bsz, T, G, N),
                            u[..., H * P + G * N:].reshape(Bsz, T, G, N), inp["D"], h0=h0, **kw)
    return y.reshape(Bsz, T, H * P), hT, cs


def oracle_f16(inp, cs0, h0, H, G, N, norm_group, seqs, P=64):
    """The binary16-state composition for the sequences in `seqs`."""
    xin = inp["xBC"][seqs]
    Bsz, T, _ = xin.shape
    u, cs = oracle.conv_silu(xin, inp["conv_w"], inp["conv_b"], cs0[seqs])
    u = u.astype(np.float16).astype(np.float32)          # staged in the I/O type
    tr = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1))
    x = tr(u[..., :H * P].reshape(Bsz, T, H, P))
    Bm = tr(u[..., H * P:H * P + G * N].reshape(Bsz, T, G, N))
    Cm = tr(u[..., H * P + G * N:].reshape(Bsz, T, G, N))
    bits = np.ascontiguousarray(h0[seqs].astype(np.float16)).view(np.uint16)
    raw = "dt_bias" in inp
    y = oracle.decode_f16state(x, tr(inp["dt"][seqs]), inp["A"], Bm, Cm, inp["D"], bits, dt_bias=inp.get("dt_bias"),
                               dt_softplus_raw=raw)
    y = np.swapaxes(y, 0, 1).reshape(Bsz, T, H * P)
    if norm_group:
        y = oracle.gated_rmsnorm(y, inp["z"][seqs], inp["norm_w"], norm_group)
    return y, bits.view(np.float16).astype(np.float64), cs


def out_err(got, ref, norm_group, H, P=64):
    Bsz, T, C = got.shape
    if norm_group:   # slice: (sequence, norm group) over all steps
        k = C // norm_group
        g = got.reshape(Bsz, T, k, norm_group).transpose(0, 2, 1, 3)
        r = ref.reshape(Bsz, T, k, norm_group).transpose(0, 2, 1, 3)
        return slice_err(g, r, 2)
    g = got.reshape(Bsz, T, H, P).transpose(0, 2, 1, 3)   # slice: (sequence, head)
    r = ref.reshape(Bsz, T, H, P).transpose(0, 2, 1, 3)
    return slice_err(g, r, 2)


@pytest.mark.parametrize("N,norm_group,raw_dt", [(16, 0, False), (64, 512, False), (128, 1024, False),
                                                 (128, 0, True), (128, 64, True)])
def test_mixer_decode_f32_state(N, norm_group, raw_dt):
    Bsz, T, H, G = 3, 5, 16, 2
    inp, cs0, h0 = case(100 + N + norm_group, Bsz, T, H, G, N, raw_dt)
    say(f"[mixer decode] f32 state N={N} norm_group={norm_group} raw_dt={raw_dt}")
    y, st, cs = run_steps(inp, cs0, h0, H, G, N, norm_group, m2.F32)
    yr, hr, csr = oracle_f32(inp, cs0, h0, H, G, N, norm_group)
    ey, es = out_err(y, yr, norm_group, H), slice_err(st, hr, 2)
    say(f"[mixer decode] out err {ey:.3e} state err {es:.3e}")
    assert ey <= Y_TOL and es <= S_TOL
    assert np.array_equal(cs.astype(np.float64), csr)


@pytest.mark.parametrize("N,norm_group", [(64, 1024), (128, 512)])
def test_mixer_decode_f16_state(N, norm_group):
    Bsz, T, H, G = 3, 6, 16, 2
    inp, cs0, h0 = case(200 + N, Bsz, T, H, G, N)
    say(f"[mixer decode] f16 state N={N} norm_group={norm_group}")
    y, st, cs = run_steps(inp, cs0, h0, H, G, N, norm_group, m2.F16)
    yr, sr, csr = oracle_f16(inp, cs0, h0, H, G, N, norm_group, slice(0, Bsz))
    same = float(np.mean(st == sr))
    ey, es = out_err(y, yr, norm_group, H), slice_err(st, sr, 2)
    say(f"[mixer decode] state identical {same:.6f} out err {ey:.3e} state err {es:.3e}")
    # the conv output is the correctly rounded binary16 SiLU on both sides
    # (the header's contract), so the binary32 step contract holds bit for bit
    assert same == 1.0 and ey <= Y_TOL and es <= S_TOL
    assert np.array_equal(cs.astype(np.float64), csr)


def test_mixer_decode_fp32_io():
    Bsz, T, H, G, N = 2, 4, 8, 2, 64
    s = synth.WindowShape(Bsz, T, H, 64, N, G, 256, np.float32, "narrow")
    inp = synth.mixer_inputs(s, 250)
    r = np.random.default_rng(251)
    Cn = H * 64 + 2 * G * N
    cs0 = r.standard_normal((Bsz, Cn, 3)).astype(np.float32)
    h0 = (r.standard_normal((Bsz, H, 64, N)) * 0.1).astype(np.float32)
    cs = to_dev(cs0).clone()
    st = to_dev(h0).clone()
    dims = m2.mixer_decode_dims(Bsz, H, 64, N, G, 512, m2.F32, m2.F32)
    ws = m2.alloc_mixer_decode_workspace(dims, DEV)
    say("[mixer decode] f32 I/O")
    ys = []
    for t in range(T):
        y = torch.empty((Bsz, H * 64), dtype=torch.float32, device=DEV)
        m2.mixer_decode_step(to_dev(np.ascontiguousarray(inp["xBC"][:, t])), to_dev(inp["conv_w"]), cs,
                             to_dev(np.ascontiguousarray(inp["dt"][:, t])), to_dev(inp["A"]), to_dev(inp["D"]), st, y,
                             ws, conv_b=to_dev(inp["conv_b"]), z=to_dev(np.ascontiguousarray(inp["z"][:, t])),
                             norm_w=to_dev(inp["norm_w"]), ngroups=G, dstate=N, norm_group=512)
        ys.append(y)
    torch.cuda.synchronize()
    y = torch.stack(ys, 1).cpu().numpy()
    out_r, h_r, cs_r = oracle.mixer_core(inp["xBC"], inp["conv_w"], inp["conv_b"], inp["dt"], inp["A"], inp["D"],
                                         inp["z"], inp["norm_w"], H, 64, G, N, 512, conv_state=cs0, h0=h0)
    ey, es = out_err(y, out_r, 512, H), slice_err(st.cpu().numpy(), h_r, 2)
    say(f"[mixer decode] f32 I/O: out err {ey:.3e} state err {es:.3e}")
    assert ey <= Y_TOL and es <= S_TOL
    assert np.array_equal(cs.cpu().numpy().astype(np.float64), cs_r)


def test_window_then_mixer_decode_continues_the_window():
    # a window of 300 tokens through the window entry, then 4 fused steps from
    # its conv history and state: the outputs are those of a 304-token window
    H, G, N, P, L, T = 16, 2, 128, 64, 300, 4
    s = synth.WindowShape(2, L + T, H, P, N, G, 256, np.float16, "wide")
    inp = synth.mixer_inputs(s, 300)
    Cn = H * P + 2 * G * N
    xBC = to_dev(np.ascontiguousarray(inp["xBC"][:, :L]))
    yw = torch.empty((2, L, H * P), dtype=torch.float16, device=DEV)
    hT = torch.empty((2, H, P, N), dtype=torch.float32, device=DEV)
    cso = torch.empty((2, Cn, 3), dtype=torch.float16, device=DEV)
    dims = m2.make_dims(2, L, H, P, N, G, 256, conv_width=4, norm_group=1024)
    ws = m2.alloc_workspace(dims, DEV)
    say("[mixer decode] window 300 + 4 steps")
    window_checked(to_dev(np.ascontiguousarray(inp["dt"][:, :L])), to_dev(inp["A"]), to_dev(inp["D"]), yw, ws,
                        xBC=xBC, conv_w=to_dev(inp["conv_w"]), conv_b=to_dev(inp["conv_b"]), conv_state_out=cso,
                        state_out=hT, z=to_dev(np.ascontiguousarray(inp["z"][:, :L])), norm_w=to_dev(inp["norm_w"]),
                        chunk=256, norm_group=1024, ngroups=G, dstate=N, headdim=P)
    torch.cuda.synchronize()
    tail = {k: (np.ascontiguousarray(v[:, L:]) if k in ("xBC", "dt", "z") else v) for k, v in inp.items()}
    y, st, cs = run_steps(tail, cso.cpu().numpy(), hT.cpu().numpy(), H, G, N, 1024, m2.F32)
    out_r, h_r, cs_r = oracle.mixer_core(inp["xBC"], inp["conv_w"], inp["conv_b"], inp["dt"], inp["A"], inp["D"],
                                         inp["z"], inp["norm_w"], H, P, G, N, 1024)
    ey = out_err(y, out_r[:, L:], 1024, H)
    es = slice_err(st, h_r, 2)
    say(f"[mixer decode] continued window: out err {ey:.3e} state err {es:.3e}")
    assert ey <= Y_TOL and es <= S_TOL
    assert np.array_equal(cs.astype(np.float64), cs_r)


def test_mixer_decode_full_size_sampled():
    # 64 sequences of the layer shape, f16 resident state, one RMS over all
    # 8192 channels (128 heads per norm group), 3 steps
    d = synth.DECODE
    Bsz, H, P, N, G = d["batch"], d["nheads"], d["headdim"], d["dstate"], d["ngroups"]
    T, norm_group = 3, H * P
    inp, cs0, h0 = case(400, Bsz, T, H, G, N)
    say(f"[mixer decode] full size B={Bsz} H={H} N={N} norm over {norm_group}")
    y, st, cs = run_steps(inp, cs0, h0, H, G, N, norm_group, m2.F16)
    seqs = [0, 37, 63]
    yr, sr, csr = oracle_f16(inp, cs0, h0, H, G, N, norm_group, seqs)
    same = float(np.mean(st[seqs] == sr))
    ey, es = out_err(y[seqs], yr, norm_group, H), slice_err(st[seqs], sr, 2)
    say(f"[mixer decode] full: state identical {same:.6f} out err {ey:.3e} state err {es:.3e}")
    assert same == 1.0 and ey <= Y_TOL and es <= S_TOL
    assert np.array_equal(cs[seqs].astype(np.float64), csr)

"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar (fp16 I/O, fp32 accumulate): per-slice max error / slice max magnitude
<= 2e-3 on y (and on the normed output) and <= 1e-3 on final states; a slice
is one (sequence, head) -- for the normed output one (sequence, token).
"""
import math
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
from tests.gpu_helpers import (DEV, cu_of, pack_rows, projection_rows, run_mixer, run_requant, run_window,  # noqa: E402
                               run_window_packed, slice_err, to_dev, unpack_rows, window_checked)

Y_TOL, S_TOL = 2e-3, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rand_window(seed, B, L, H, N, G, dtype=np.float16, dt_mode="wide", P=64):
    s = synth.WindowShape(B, L, H, P, N, G, 256, dtype, dt_mode)
    return synth.window_inputs(s, seed)


def oracle_window(inp, seqlens=None, state_in=None, nthreads=0):
    return oracle.ssd_scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], h0=state_in,
                           seqlens=seqlens, nthreads=nthreads, dt_bias=inp.get("dt_bias"),
                           dt_softplus_raw="dt_bias" in inp)


def check_window(name, inp, chunk, seqlens=None, state_in=None, segments=0):
    say(f"[window] {name}: shape x{inp['x'].shape} chunk {chunk} seqlens {seqlens} segments {segments}")
    y, hT = run_window(inp, chunk, seqlens=seqlens, state_in=state_in, y_fill=12345.0, segments=segments)
    yr, hr = oracle_window(inp, seqlens, state_in)
    Bsz = y.shape[0]
    ey = 0.0
    for b in range(Bsz):
        n = seqlens[b] if seqlens is not None else y.shape[1]
        if n > 0:
            ey = max(ey, slice_err(np.transpose(y[b:b + 1, :n], (0, 2, 1, 3)),
                                   np.transpose(yr[b:b + 1, :n], (0, 2, 1, 3)), 2))
        # rows past the sequence end are untouched
        assert np.all(y[b, n:] == np.float16(12345.0) if y.dtype == np.float16 else y[b, n:] == 12345.0)
    es = slice_err(hT, hr, 2)
    say(f"[window] {name}: y err {ey:.3e}  state err {es:.3e}")
    assert ey <= Y_TOL and es <= S_TOL
    return y, hT


# ---------------------------------------------------------------------------
def test_tiny_fp32_scan():
    s = synth.tiny_scan()
    check_window("tiny fp32", synth.window_inputs(s, 1000), s.chunk)


@pytest.mark.parametrize("chunk", [64, 128, 256])
@pytest.mark.parametrize("N", [16, 64, 128])
def test_chunk_sizes_and_state_sizes(chunk, N):
    inp = rand_window(11 + N + chunk, 1, 300, 8, N, 2)
    check_window(f"N={N}", inp, chunk)


@pytest.mark.parametrize("B", [1, 8])
def test_many_chunks_carry_tree(B):
    # 64 chunks per sequence: a deep carry tree.  One sequence fits the chip in
    # one pass of workgroups (radix-8 tree); eight do not (radix-4 tree).
    inp = rand_window(31 + B, B, 4096, 4, 16, 1)
    lens = [4096] * B if B == 1 else [4096, 4000, 3, 64, 65, 2048, 4095, 1000]
    h0 = np.random.default_rng(32).standard_normal((B, 4, 64, 16)).astype(np.float32) * 0.3
    check_window(f"64 chunks B={B}", inp, 64, seqlens=lens, state_in=h0)


@pytest.mark.parametrize("segments", [1, 2, 3, 9])
def test_segments_of_consecutive_chunks(segments):
    # 9 chunks of 128 tokens run as 1, 2, 3 or 9 segments (runs of 9, 6 + 3,
    # 3 or 1 chunks passing the state in registers; with two segments the
    # second computes the first one's local state itself, no hand-off); the
    # lengths end inside the first chunk, inside an earlier segment and at
    # the window end
    inp = rand_window(51 + segments, 3, 1100, 16, 128, 2)
    h0 = np.random.default_rng(52).standard_normal((3, 16, 64, 128)).astype(np.float32) * 0.5
    check_window(f"segments={segments}", inp, 128, seqlens=[1100, 700, 100], state_in=h0, segments=segments)


def test_streamed_scan_more_workgroups_than_compute_units():
    # The binary16 N = 128 scan with 8 sequences of 5 chunks as 5 segments
    # each: 320 workgroups, more than the compute units, so the hand-off takes
    # the radix-4 tree and a segment may wait on one that is not resident at
    # the same time (it waits only on segments claimed before it).  Lengths
    # end inside every segment, at one token and at zero.
    inp = rand_window(71, 8, 640, 32, 128, 8)
    lens = [640, 600, 1, 129, 384, 640, 257, 0]
    h0 = np.random.default_rng(72).standard_normal((8, 32, 64, 128)).astype(np.float32) * 0.3
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert 8 * 8 * 5 > cus
    check_window("more workgroups than compute units", inp, 128, seqlens=lens, state_in=h0, segments=5)


# Calls that ask for no final state hand segment aggregates over as scaled
# binary16 (only the readouts see them); y against the oracle.
def check_window_y_only(name, inp, chunk, seqlens=None, state_in=None, segments=0):
    say(f"[window, no final state] {name}: shape x{inp['x'].shape} chunk {chunk} segments {segments}")
    y, _ = run_window(inp, chunk, seqlens=seqlens, state_in=state_in, want_state=False, y_fill=12345.0,
                      segments=segments)
    yr, _ = oracle_window(inp, seqlens, state_in)
    ey = 0.0
    for b in range(y.shape[0]):
        n = seqlens[b] if seqlens is not None else y.shape[1]
        if n > 0:
            ey = max(ey, slice_err(np.transpose(y[b:b + 1, :n], (0, 2, 1, 3)),
                                   np.transpose(yr[b:b + 1, :n], (0, 2, 1, 3)), 2))
        assert np.all(y[b, n:] == np.float16(12345.0))
    say(f"[window, no final state] {name}: y err {ey:.3e}")
    assert ey <= Y_TOL


def test_windows_without_final_state():
    s = synth.layer_window()
    check_window_y_only("layer L=2048", synth.window_inputs(s, 1001), s.chunk)
    # a two-level tree (nine segments) and a three-level one (more workgroups
    # than compute units: radix 4, late publishers re-rounding combined
    # aggregates), with initial states and ragged lengths
    inp = rand_window(54, 3, 1100, 16, 128, 2)
    h0 = np.random.default_rng(55).standard_normal((3, 16, 64, 128)).astype(np.float32) * 0.5
    check_window_y_only("segments=9", inp, 128, seqlens=[1100, 700, 100], state_in=h0, segments=9)
    inp = rand_window(71, 8, 640, 32, 128, 8)
    lens = [640, 600, 1, 129, 384, 640, 257, 0]
    h0 = np.random.default_rng(72).standard_normal((8, 32, 64, 128)).astype(np.float32) * 0.3
    check_window_y_only("more workgroups than compute units", inp, 128, seqlens=lens, state_in=h0, segments=5)
    s2 = synth.WindowShape(2, 600, 8, 64, 128, 2, 256, np.float16, "wide")
    inp = synth.window_inputs(s2, 81, raw_dt=True)
    check_window_y_only("raw dt", inp, 256, seqlens=[600, 411], segments=3)
    # packed rows, three segments, no final state
    lens = [600, 411, 0, 257, 1]
    inp = rand_window(86, len(lens), 600, 8, 128, 2)
    h0 = np.random.default_rng(87).standard_normal((len(lens), 8, 64, 128)).astype(np.float32) * 0.3
    x, dt, Bm, Cm = (to_dev(pack_rows(inp[k], lens)) for k in ("x", "dt", "B", "C"))
    T = dt.shape[0]
    y = torch.full((T + 16, 8 * 64), 12345.0, dtype=x.dtype, device=DEV)
    dims = m2.make_dims(len(lens), 600, 8, 64, 128, 2, 256, packed_tokens=T)
    ws = m2.alloc_workspace(dims, DEV)
    window_checked(dt, to_dev(inp["A"]), to_dev(inp["D"]), y, ws, x=x, B=Bm, C=Cm, state_in=to_dev(h0),
                   chunk=256, segments=3, cu_seqlens=to_dev(cu_of(lens)), max_seqlen=600)
    torch.cuda.synchronize()
    yp = y.cpu().numpy()
    assert np.all(yp[T:] == np.float16(12345.0))
    yu = unpack_rows(yp[:T], lens, 600).reshape(len(lens), 600, 8, 64)
    yr, _ = oracle_window(inp, lens, h0)
    ey = max(slice_err(np.transpose(yu[b:b + 1, :n], (0, 2, 1, 3)), np.transpose(yr[b:b + 1, :n], (0, 2, 1, 3)), 2)
             for b, n in enumerate(lens) if n > 0)
    say(f"[window, no final state] packed: y err {ey:.3e}")
    assert ey <= Y_TOL


def test_ragged_batch_with_initial_state():
    inp = rand_window(21, 3, 700, 16, 128, 2)
    h0 = np.random.default_rng(22).standard_normal((3, 16, 64, 128)).astype(np.float32) * 0.5
    check_window("ragged+h0", inp, 256, seqlens=[700, 513, 1], state_in=h0)


def test_zero_length_sequence_passes_state_through():
    inp = rand_window(23, 2, 130, 8, 64, 1)
    h0 = np.random.default_rng(24).standard_normal((2, 8, 64, 64)).astype(np.float32)
    y, hT = run_window(inp, 64, seqlens=[0, 130], state_in=h0, y_fill=7.0)
    assert np.all(y[0] == np.float16(7.0))
    assert np.array_equal(hT[0], h0[0])


def test_dt_zero_gives_skip_and_keeps_state():
    inp = rand_window(25, 1, 512, 8, 128, 2)
    inp["dt"][:] = 0
    h0 = np.random.default_rng(26).standard_normal((1, 8, 64, 128)).astype(np.float32)
    y, hT = run_window(inp, 256, state_in=None)
    ref = (inp["D"][None, None, :, None].astype(np.float32) * inp["x"].astype(np.float32))
    assert np.max(np.abs(y.astype(np.float64) - ref.astype(np.float16).astype(np.float64))
                  / np.maximum(np.abs(ref.astype(np.float16).astype(np.float64)), 6e-5)) <= 2 ** -10
    assert np.all(hT == 0)
    _, hT2 = run_window(inp, 256, state_in=h0)
    assert np.array_equal(hT2, h0)


@pytest.mark.parametrize("segments", [0, 3])
def test_window_steps_with_strong_decay(segments):
    """Heads whose 32-token steps decay by more than 2^-100 (the scan then
    forms the intra-step decay mask entry by entry), heads that straddle
    that bound from step to step, and ordinary heads, in one window."""
    inp = rand_window(61, 1, 900, 8, 128, 2)
    rng = np.random.default_rng(62)
    A = inp["A"].copy()
    A[:4] = -16.0
    inp["A"] = A
    dt = inp["dt"].astype(np.float32)
    # per-token log2 decay 16 dt log2(e): about 11.5 (heads 0, 1), and
    # around 100 / 32 per token (heads 2, 3)
    dt[..., 0:2] = 0.5 + 0.05 * rng.standard_normal(dt[..., 0:2].shape)
    dt[..., 2:4] = 0.135 * np.exp(0.3 * rng.standard_normal(dt[..., 2:4].shape))
    inp["dt"] = dt.astype(inp["dt"].dtype)
    lg = -16.0 * math.log2(math.e) * inp["dt"].astype(np.float64)[0, :, 2:4]
    steps = np.add.reduceat(lg, np.arange(0, 900, 32), axis=0)
    assert (steps < -100).any() and (steps > -100).any()
    h0 = np.random.default_rng(63).standard_normal((1, 8, 64, 128)).astype(np.float32)
    check_window(f"strong decay, segments {segments}", inp, 256, seqlens=[900], state_in=h0, segments=segments)


def test_split_window_carry_matches_unsplit():
    inp = rand_window(27, 1, 1024, 16, 128, 2)
    y, hT = run_window(inp, 256)
    for m in (256, 300):
        a = {k: (v[:, :m] if v.ndim > 1 else v) for k, v in inp.items()}
        b = {k: (v[:, m:] if v.ndim > 1 else v) for k, v in inp.items()}
        y1, h1 = run_window(a, 256)
        y2, h2 = run_window(b, 256, state_in=h1)
        ey = slice_err(np.transpose(np.concatenate([y1, y2], 1), (0, 2, 1, 3)), np.transpose(y, (0, 2, 1, 3)), 2)
        es = slice_err(h2, hT, 2)
        say(f"[split] m={m}: y {ey:.3e} state {es:.3e}")
        assert ey <= Y_TOL and es <= S_TOL


# ---------------------------------------------------------------------------
# Short windows of one round of (sequence, head, half) workgroups run the
# column scan (the state split over n between a workgroup's waves, one
# workgroup per sequence and half head); these cases take that path.
@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_short_window_full_heads_column_scan(chunk):
    # one 8B-shape window of 512 tokens, every head, with an initial state;
    # and a ragged length with canaries past it
    inp = rand_window(91 + chunk, 1, 512, 128, 128, 8)
    h0 = np.random.default_rng(92).standard_normal((1, 128, 64, 128)).astype(np.float32) * 0.3
    check_window(f"column scan L=512 chunk {chunk}", inp, chunk, state_in=h0)
    check_window(f"column scan L=437 of 512 chunk {chunk}", inp, chunk, seqlens=[437], state_in=h0)


def test_column_scan_routing_boundary():
    # 768 tokens run the column scan, 769 the segmented scan (four runs of
    # 256-token chunks); both against the oracle at the full head count
    inp = rand_window(100, 1, 769, 128, 128, 8)
    h0 = np.random.default_rng(101).standard_normal((1, 128, 64, 128)).astype(np.float32) * 0.3
    short = {k: (v[:, :768] if v.ndim > 1 else v) for k, v in inp.items()}
    check_window("L=768 (column scan)", short, 256, state_in=h0)
    check_window("L=769 (segmented scan)", inp, 256, state_in=h0)


def test_short_windows_column_scan_ragged_zero_and_one_token():
    inp = rand_window(93, 3, 300, 16, 128, 2)
    h0 = np.random.default_rng(94).standard_normal((3, 16, 64, 128)).astype(np.float32) * 0.5
    check_window("column scan ragged", inp, 64, seqlens=[300, 1, 0], state_in=h0)
    y, hT = run_window(inp, 64, seqlens=[300, 1, 0], state_in=h0, y_fill=3.0)
    assert np.array_equal(hT[2], h0[2]) and np.all(y[2] == np.float16(3.0))


def test_short_window_column_scan_raw_dt_and_packed():
    s = synth.WindowShape(2, 500, 16, 64, 128, 2, 256, np.float16, "wide")
    inp = synth.window_inputs(s, 95, raw_dt=True)
    h0 = np.random.default_rng(96).standard_normal((2, 16, 64, 128)).astype(np.float32) * 0.3
    check_window("column scan raw dt", inp, 128, seqlens=[500, 263], state_in=h0)
    lens = [500, 263]
    yp, hT = run_window_packed(inp, lens, 128, state_in=h0)
    T = sum(lens)
    assert np.all(yp[T:] == np.float16(12345.0))       # nothing past the packed rows
    y = unpack_rows(yp[:T], lens, 500).reshape(len(lens), 500, 16, 64)
    yr, hr = oracle_window(inp, lens, h0)
    ey = max(slice_err(np.transpose(y[b:b + 1, :n], (0, 2, 1, 3)), np.transpose(yr[b:b + 1, :n], (0, 2, 1, 3)), 2)
             for b, n in enumerate(lens))
    es = slice_err(hT, hr, 2)
    say(f"[column scan packed] y {ey:.3e} state {es:.3e}")
    assert ey <= Y_TOL and es <= S_TOL


def test_short_window_column_scan_strong_decay():
    # steps decaying by more than 2^-100 take the entry-by-entry mask factors
    inp = rand_window(97, 1, 480, 8, 128, 2)
    A = inp["A"].copy()
    A[:4] = -16.0
    inp["A"] = A
    dt = inp["dt"].astype(np.float32)
    rng = np.random.default_rng(98)
    dt[..., 0:2] = 0.5 + 0.05 * rng.standard_normal(dt[..., 0:2].shape)
    dt[..., 2:4] = 0.135 * np.exp(0.3 * rng.standard_normal(dt[..., 2:4].shape))
    inp["dt"] = dt.astype(inp["dt"].dtype)
    lg = -16.0 * math.log2(math.e) * inp["dt"].astype(np.float64)[0, :, 2:4]
    steps = np.add.reduceat(lg, np.arange(0, 480, 32), axis=0)
    assert (steps < -100).any() and (steps > -100).any()
    h0 = np.random.default_rng(99).standard_normal((1, 8, 64, 128)).astype(np.float32)
    check_window("column scan strong decay", inp, 256, seqlens=[480], state_in=h0)


def test_layer_window_full_size():
    s = synth.layer_window()
    check_window("layer L=2048", synth.window_inputs(s, 1001), s.chunk)


def test_batched_windows_full_size():
    # all eight sequences (seven of 2048 tokens and the 1955-token partial
    # window) and all eight final states against the oracle
    s = synth.batched_windows()
    inp = synth.window_inputs(s, 1002)
    say(f"[window] batched: x{inp['x'].shape} lengths {s.seqlens}")
    y, hT = run_window(inp, s.chunk, seqlens=s.seqlens, y_fill=12345.0)
    yr, hr = oracle_window(inp, list(s.seqlens))
    for b in range(s.batch):
        n = s.seqlens[b]
        ey = slice_err(np.transpose(y[b:b + 1, :n], (0, 2, 1, 3)), np.transpose(yr[b:b + 1, :n], (0, 2, 1, 3)), 2)
        es = slice_err(hT[b:b + 1], hr[b:b + 1], 2)
        say(f"[window] batched seq {b} (len {n}): y {ey:.3e} state {es:.3e}")
        assert ey <= Y_TOL and es <= S_TOL
        assert np.all(y[b, n:] == np.float16(12345.0))


# ---- packed variable-length windows (row offsets instead of padding) ------------
@pytest.mark.parametrize("segments", [0, 2])
def test_packed_windows_match_oracle(segments):
    lens = [600, 411, 0, 257, 1]
    inp = rand_window(86, len(lens), 600, 8, 128, 2)
    h0 = np.random.default_rng(87).standard_normal((len(lens), 8, 64, 128)).astype(np.float32) * 0.3
    say(f"[packed] lengths {lens} segments {segments}")
    yp, hT = run_window_packed(inp, lens, 256, state_in=h0, segments=segments)
    T = sum(lens)
    assert np.all(yp[T:] == np.float16(12345.0))       # nothing past the packed rows
    y = unpack_rows(yp[:T], lens, 600).reshape(len(lens), 600, 8, 64)
    yr, hr = oracle_window(inp, lens, h0)
    ey = max(slice_err(np.transpose(y[b:b + 1, :n], (0, 2, 1, 3)), np.transpose(yr[b:b + 1, :n], (0, 2, 1, 3)), 2)
             for b, n in enumerate(lens) if n > 0)
    es = slice_err(hT, hr, 2)
    say(f"[packed] y err {ey:.3e} state err {es:.3e}")
    assert ey <= Y_TOL and es <= S_TOL
    # a zero-length sequence hands its initial state through
    assert np.array_equal(hT[2], h0[2])


def test_packed_sequence_longer_than_seqlen_is_cut():
    # dims.seqlen bounds every length: a longer packed sequence is processed
    # for its first seqlen tokens and its later rows are left untouched
    lens = [300, 500]
    inp = rand_window(91, 2, 500, 4, 64, 1)
    x, dt, Bm, Cm = (to_dev(pack_rows(inp[k], lens)) for k in ("x", "dt", "B", "C"))
    T = sum(lens)
    y = torch.full((T, 4 * 64), 12345.0, dtype=torch.float16, device=DEV)
    hT = torch.empty((2, 4, 64, 64), dtype=torch.float32, device=DEV)
    dims = m2.make_dims(2, 400, 4, 64, 64, 1, 256, packed_tokens=T)
    ws = m2.alloc_workspace(dims, DEV)
    say("[packed] second sequence cut at seqlen 400")
    window_checked(dt, to_dev(inp["A"]), to_dev(inp["D"]), y, ws, x=x, B=Bm, C=Cm, state_out=hT,
                        cu_seqlens=to_dev(cu_of(lens)), max_seqlen=400)
    torch.cuda.synchronize()
    yp, hT = y.cpu().numpy(), hT.cpu().numpy()
    assert np.all(yp[300 + 400:] == np.float16(12345.0))
    sub = {k: (v[1:2, :400] if v.ndim > 1 else v) for k, v in inp.items()}
    yr, hr = oracle_window(sub)
    ey = slice_err(np.transpose(yp[300:700].reshape(1, 400, 4, 64), (0, 2, 1, 3)), np.transpose(yr, (0, 2, 1, 3)), 2)
    es = slice_err(hT[1:2], hr, 2)
    say(f"[packed] cut sequence: y {ey:.3e} state {es:.3e}")
    assert ey <= Y_TOL and es <= S_TOL


def test_packed_batched_windows_equal_padded_bit_for_bit():
    # eight windows of the layer shape packed back to back (7 x 2048 + 1955
    # rows): only the row addressing differs from the padded call
    s = synth.batched_windows()
    inp = synth.window_inputs(s, 1002)
    lens = s.seqlens
    say(f"[packed] batched: {sum(lens)} rows")
    yp, hp = run_window_packed(inp, lens, s.chunk)
    y, hT = run_window(inp, s.chunk, seqlens=lens)
    T = sum(lens)
    assert np.all(yp[T:] == np.float16(12345.0))
    assert np.array_equal(yp[:T], pack_rows(y.reshape(8, 2048, -1), lens))
    assert np.array_equal(hp, hT)
    b, n = 7, lens[7]
    sub = {k: (v[b:b + 1] if v.ndim > 1 else v) for k, v in inp.items()}
    yr, hr = oracle_window(sub, [n])
    ey = slice_err(np.transpose(y[b:b + 1, :n], (0, 2, 1, 3)), np.transpose(yr[:, :n], (0, 2, 1, 3)), 2)
    say(f"[packed] batched: identical to padded; seq 7 y {ey:.3e} state {slice_err(hp[7:], hr, 2):.3e}")
    assert ey <= Y_TOL and slice_err(hp[7:], hr, 2) <= S_TOL


def test_packed_requant_window_bit_exact_state():
    lens = [300, 0, 177, 33]
    inp = rand_window(88, len(lens), 300, 8, 64, 2)
    x, dt, Bm, Cm = (to_dev(pack_rows(inp[k], lens)) for k in ("x", "dt", "B", "C"))
    T = sum(lens)
    y = torch.full((T + 8, 8 * 64), 12345.0, dtype=torch.float16, device=DEV)
    hT = torch.empty((len(lens), 8, 64, 64), dtype=torch.float32, device=DEV)
    say(f"[packed] requant lengths {lens}")
    m2.requant_window(dt, to_dev(inp["A"]), to_dev(inp["D"]), y, x=x, B=Bm, C=Cm, state_out=hT,
                      cu_seqlens=to_dev(cu_of(lens)), max_seqlen=300)
    torch.cuda.synchronize()
    yp, hT = y.cpu().numpy(), hT.cpu().numpy()
    assert np.all(yp[T:] == np.float16(12345.0))
    yr, bits = oracle_requant(inp, lens)
    got = np.ascontiguousarray(hT.astype(np.float16)).view(np.uint16)
    yu = unpack_rows(yp[:T], lens, 300).reshape(len(lens), 300, 8, 64)
    ey = max(slice_err(np.transpose(yu[b:b + 1, :n], (0, 2, 1, 3)), np.transpose(yr[b:b + 1, :n], (0, 2, 1, 3)), 2)
             for b, n in enumerate(lens) if n > 0)
    say(f"[packed] requant: state identical {np.mean(got == bits):.6f} y err {ey:.3e}")
    assert np.array_equal(got, bits) and ey <= Y_TOL


def test_packed_mixer_core_with_conv_state_and_norm():
    H, P, G, N, L = 16, 64, 2, 128, 300
    lens = [300, 157, 0, 64]
    s = synth.WindowShape(len(lens), L, H, P, N, G, 256, np.float16, "wide")
    inp = synth.mixer_inputs(s, 89, raw_dt=True)
    Cn = H * P + 2 * G * N
    csi = np.random.default_rng(90).standard_normal((len(lens), Cn, 3)).astype(np.float16)
    T = sum(lens)
    xBC, dt, z = (to_dev(pack_rows(inp[k], lens)) for k in ("xBC", "dt", "z"))
    y = torch.full((T + 8, H * P), 12345.0, dtype=torch.float16, device=DEV)
    hT = torch.empty((len(lens), H, P, N), dtype=torch.float32, device=DEV)
    cso = torch.empty((len(lens), Cn, 3), dtype=torch.float16, device=DEV)
    dims = m2.make_dims(len(lens), L, H, P, N, G, 256, conv_width=4, norm_group=512, packed_tokens=T)
    ws = m2.alloc_workspace(dims, DEV)
    say(f"[packed] mixer lengths {lens}")
    window_checked(dt, to_dev(inp["A"]), to_dev(inp["D"]), y, ws, xBC=xBC, conv_w=to_dev(inp["conv_w"]),
                        conv_b=to_dev(inp["conv_b"]), conv_state_in=to_dev(csi), conv_state_out=cso, state_out=hT,
                        z=z, norm_w=to_dev(inp["norm_w"]), chunk=256, norm_group=512, ngroups=G, dstate=N,
                        headdim=P, dt_softplus=True, dt_bias=to_dev(inp["dt_bias"]), cu_seqlens=to_dev(cu_of(lens)),
                        max_seqlen=L)
    torch.cuda.synchronize()
    yp = y.cpu().numpy()
    assert np.all(yp[T:] == np.float16(12345.0))
    out_r, h_r, cs_r = oracle.mixer_core(inp["xBC"], inp["conv_w"], inp["conv_b"], inp["dt"], inp["A"], inp["D"],
                                         inp["z"], inp["norm_w"], H, P, G, N, 512, conv_state=csi, seqlens=lens,
                                         dt_bias=inp["dt_bias"], dt_softplus_raw=True)
    yu = unpack_rows(yp[:T], lens, L)
    for b, n in enumerate(lens):
        if n == 0:
            continue
        got = yu[b, :n].reshape(n, -1, 512).transpose(1, 0, 2)
        ref = out_r[b, :n].reshape(n, -1, 512).transpose(1, 0, 2)
        e = slice_err(got, ref, 1)
        say(f"[packed] mixer out seq {b}: {e:.3e}")
        assert e <= Y_TOL
    assert slice_err(hT.cpu().numpy(), h_r, 2) <= S_TOL
    assert np.array_equal(cso.cpu().numpy().astype(np.float64), cs_r)


def test_sequence_alone_equals_sequence_in_batch():
    inp = rand_window(31, 4, 600, 16, 128, 2)
    y, hT = run_window(inp, 256, seqlens=[600, 600, 431, 600])
    sub = {k: (v[2:3] if v.ndim > 1 else v) for k, v in inp.items()}
    y1, h1 = run_window(sub, 256, seqlens=[431])
    assert np.array_equal(y1[0, :431], y[2, :431]) and np.array_equal(h1[0], hT[2])


def test_deterministic_and_workspace_reuse():
    inp = rand_window(33, 2, 777, 16, 128, 2)
    dims = m2.make_dims(2, 777, 16, 64, 128, 2, 256)
    ws = m2.alloc_workspace(dims, DEV)
    outs = [run_window(inp, 256, ws=ws) for _ in range(3)]
    for y, h in outs[1:]:
        assert np.array_equal(y, outs[0][0]) and np.array_equal(h, outs[0][1])
    # a smaller problem through the same workspace, then the first again
    small = {k: (v[:1, :100] if v.ndim > 1 else v) for k, v in inp.items()}
    ys, hs = run_window(small, 256, ws=ws)
    yr, hr = oracle_window(small)
    assert slice_err(hs, hr, 2) <= S_TOL
    y3, h3 = run_window(inp, 256, ws=ws)
    assert np.array_equal(y3, outs[0][0]) and np.array_equal(h3, outs[0][1])


# ---- window with the state requantized every token ------------------------------
def oracle_requant(inp, seqlens=None, state_in=None, heads=None):
    """The oracle's decode steps run over each sequence's tokens (binary16
    state after every token).  heads: optional slice of heads sharing one
    group, checked on their own."""
    x, dt, Bm, Cm, A, D = (inp[k] for k in ("x", "dt", "B", "C", "A", "D"))
    bias = inp.get("dt_bias")
    Bsz, L, H, P = x.shape
    N = Bm.shape[3]
    if heads is not None:
        g = heads.start // (H // Bm.shape[2])
        x, dt, A, D = x[:, :, heads], dt[:, :, heads], A[heads], D[heads]
        bias = bias[heads] if bias is not None else None
        Bm, Cm = Bm[:, :, g:g + 1], Cm[:, :, g:g + 1]
        H = x.shape[2]
        if state_in is not None:
            state_in = state_in[:, heads]
    h0 = np.zeros((Bsz, H, P, N), np.float32) if state_in is None else np.asarray(state_in, np.float32)
    bits = np.ascontiguousarray(h0.astype(np.float16)).view(np.uint16)
    y = np.full((Bsz, L, H, P), np.nan)
    for b in range(Bsz):
        n = L if seqlens is None else seqlens[b]
        if n == 0:
            continue
        sb = np.ascontiguousarray(bits[b:b + 1])
        yt = oracle.decode_f16state(np.ascontiguousarray(x[b:b + 1, :n].transpose(1, 0, 2, 3)),
                                    np.ascontiguousarray(dt[b:b + 1, :n].transpose(1, 0, 2)), A,
                                    np.ascontiguousarray(Bm[b:b + 1, :n].transpose(1, 0, 2, 3)),
                                    np.ascontiguousarray(Cm[b:b + 1, :n].transpose(1, 0, 2, 3)), D, sb,
                                    dt_bias=bias, dt_softplus_raw=bias is not None)
        bits[b] = sb[0]
        y[b, :n] = yt[:, 0]
    return y, bits


def check_requant(name, inp, seqlens=None, state_in=None):
    say(f"[requant] {name}: shape x{inp['x'].shape} seqlens {seqlens}")
    y, hT = run_requant(inp, seqlens=seqlens, state_in=state_in, y_fill=12345.0)
    yr, bits = oracle_requant(inp, seqlens, state_in)
    got_bits = np.ascontiguousarray(hT.astype(np.float16)).view(np.uint16)
    # the state holds binary16 values: widening back is exact
    assert np.array_equal(got_bits.view(np.float16).astype(np.float32), hT)
    same = float(np.mean(got_bits == bits))
    ey = 0.0
    for b in range(y.shape[0]):
        n = seqlens[b] if seqlens is not None else y.shape[1]
        if n > 0:
            ey = max(ey, slice_err(np.transpose(y[b:b + 1, :n], (0, 2, 1, 3)),
                                   np.transpose(yr[b:b + 1, :n], (0, 2, 1, 3)), 2))
        assert np.all(y[b, n:] == np.float16(12345.0) if y.dtype == np.float16 else y[b, n:] == 12345.0)
    say(f"[requant] {name}: state identical {same:.6f}  y err {ey:.3e}")
    assert same == 1.0 and ey <= Y_TOL


@pytest.mark.parametrize("N", [16, 64, 128])
def test_requant_window_small(N):
    inp = rand_window(61 + N, 2, 300, 8, N, 2)
    h0 = np.random.default_rng(62).standard_normal((2, 8, 64, N)).astype(np.float32) * 0.3
    check_requant(f"N={N}", inp, seqlens=[300, 177], state_in=h0)


def test_requant_window_fp32_io_and_zero_length():
    inp = synth.window_inputs(synth.WindowShape(2, 256, 4, 64, 16, 1, 64, np.float32, "narrow"), 1010)
    check_requant("fp32 tiny", inp, seqlens=[256, 0])


def test_requant_window_layer_shape_sampled():
    # the layer window's shape, checked on the 16 heads of group 3
    s = synth.layer_window()
    inp = synth.window_inputs(s, 1011)
    y, hT = run_requant(inp)
    heads = slice(48, 64)
    yr, bits = oracle_requant(inp, heads=heads)
    got = np.ascontiguousarray(hT[:, heads].astype(np.float16)).view(np.uint16)
    same = float(np.mean(got == bits))
    ey = slice_err(np.transpose(y[:, :, heads], (0, 2, 1, 3)), np.transpose(yr, (0, 2, 1, 3)), 2)
    say(f"[requant] layer shape, heads 48..63: state identical {same:.6f}  y err {ey:.3e}")
    assert same == 1.0 and ey <= Y_TOL


# ---- raw dt: bias + softplus inside the kernels ------------------------------------
@pytest.mark.parametrize("segments", [0, 2])
def test_raw_dt_window_ragged(segments):
    # tokens past a sequence's length must keep dt = 0 although sp(0 + bias) > 0
    s = synth.WindowShape(2, 600, 8, 64, 128, 2, 256, np.float16, "wide")
    inp = synth.window_inputs(s, 81, raw_dt=True)
    h0 = np.random.default_rng(82).standard_normal((2, 8, 64, 128)).astype(np.float32) * 0.3
    check_window("raw dt", inp, 256, seqlens=[600, 411], state_in=h0, segments=segments)


def test_raw_dt_window_fp32_narrow():
    inp = synth.window_inputs(synth.WindowShape(1, 256, 4, 64, 16, 1, 64, np.float32, "narrow"), 83,
                              raw_dt=True)
    check_window("raw dt fp32", inp, 64)


def test_raw_dt_layer_window_full_size():
    s = synth.layer_window()
    check_window("raw dt layer L=2048", synth.window_inputs(s, 1001, raw_dt=True), s.chunk)


def test_raw_dt_requant_window():
    inp = synth.window_inputs(synth.WindowShape(2, 300, 8, 64, 128, 2, 256, np.float16, "wide"), 84,
                              raw_dt=True)
    check_requant("raw dt", inp, seqlens=[300, 131])


def test_raw_dt_mixer_core():
    H, P, G, N, L, Bsz = 16, 64, 2, 128, 300, 2
    s = synth.WindowShape(Bsz, L, H, P, N, G, 256, np.float16, "wide")
    inp = synth.mixer_inputs(s, 85, raw_dt=True)
    lens = [300, 157]
    say("[mixer] raw dt, norm_group 1024")
    y, hT, _ = run_mixer(inp, H, P, G, N, 256, 1024, seqlens=lens, want_conv_state=False)
    out_r, h_r, _ = oracle.mixer_core(inp["xBC"], inp["conv_w"], inp["conv_b"], inp["dt"], inp["A"], inp["D"],
                                      inp["z"], inp["norm_w"], H, P, G, N, 1024, seqlens=lens,
                                      dt_bias=inp["dt_bias"], dt_softplus_raw=True)
    for b, n in enumerate(lens):
        got = y[b, :n].reshape(n, -1, 1024).transpose(1, 0, 2)
        ref = out_r[b, :n].reshape(n, -1, 1024).transpose(1, 0, 2)
        e = slice_err(got, ref, 1)
        say(f"[mixer] raw dt out seq {b}: {e:.3e}")
        assert e <= Y_TOL
    assert slice_err(hT, h_r, 2) <= S_TOL


# ---- fused conv + gated norm ----------------------------------------------------
def small_mixer(seed, B, L, H, G, N):
    s = synth.WindowShape(B, L, H, 64, N, G, 256, np.float16, "wide")
    return synth.mixer_inputs(s, seed)


@pytest.mark.parametrize("norm_group,segments", [(0, 0), (1024, 0), (512, 0), (1024, 1), (512, 2)])
def test_mixer_core_small(norm_group, segments):
    H, P, G, N, L, Bsz = 16, 64, 2, 128, 300, 2
    inp = small_mixer(41, Bsz, L, H, G, N)
    Cn = H * P + 2 * G * N
    csi = (np.random.default_rng(42).standard_normal((Bsz, Cn, 3))).astype(np.float16)
    lens = [300, 157]
    say(f"[mixer] small norm_group={norm_group} segments={segments}")
    y, hT, cso = run_mixer(inp, H, P, G, N, 256, norm_group, seqlens=lens, conv_state_in=csi, segments=segments)
    out_r, h_r, cs_r = oracle.mixer_core(inp["xBC"], inp["conv_w"], inp["conv_b"], inp["dt"], inp["A"], inp["D"],
                                         inp["z"], inp["norm_w"], H, P, G, N, norm_group or H * P,
                                         conv_state=csi, seqlens=lens)
    if norm_group == 0:
        u, _ = oracle.conv_silu(inp["xBC"], inp["conv_w"], inp["conv_b"], csi, lens)
        u = np.nan_to_num(u)
        yr, _ = oracle.ssd_scan(u[..., :H * P].reshape(Bsz, L, H, P), inp["dt"], inp["A"],
                                u[..., H * P:H * P + G * N].reshape(Bsz, L, G, N),
                                u[..., H * P + G * N:].reshape(Bsz, L, G, N), inp["D"], seqlens=lens)
        for b, n in enumerate(lens):
            e = slice_err(np.transpose(y[b:b + 1, :n].reshape(1, n, H, P), (0, 2, 1, 3)),
                          np.transpose(yr[b:b + 1, :n], (0, 2, 1, 3)), 2)
            say(f"[mixer] y seq {b}: {e:.3e}")
            assert e <= Y_TOL
    else:
        for b, n in enumerate(lens):
            # slice = (sequence, norm group) over all tokens of the sequence
            got = y[b, :n].reshape(n, -1, norm_group).transpose(1, 0, 2)
            ref = out_r[b, :n].reshape(n, -1, norm_group).transpose(1, 0, 2)
            e = slice_err(got, ref, 1)
            say(f"[mixer] out seq {b}: {e:.3e} (per token and group: {slice_err(got.transpose(1, 0, 2), ref.transpose(1, 0, 2), 2):.3e})")
            assert e <= Y_TOL
    es = slice_err(hT, h_r, 2)
    assert es <= S_TOL, es
    assert np.array_equal(cso.astype(np.float64), cs_r)


@pytest.mark.parametrize("H,G,group,dtype", [
    (12, 2, 192, np.float16),     # groups of 3 heads: sums per 8 lanes
    (12, 2, 64, np.float32),      # one head per group, binary32 I/O
    (160, 2, 2048, np.float16),   # 10240-channel rows: g recomputed past 8192, sums per wave
    (160, 2, 640, np.float16),    # 10240-channel rows, sums per 8 lanes
])
def test_window_gated_norm_group_shapes(H, G, group, dtype):
    # the scan with the gated norm on post-conv inputs, against the oracle's
    # scan followed by its gated RMSNorm; rows past a length keep their canary
    L, N, P = 100, 16, 64
    lens = [100, 37]
    inp = rand_window(60 + H + group, 2, L, H, N, G, dtype=dtype)
    r = np.random.default_rng(61)
    z = r.standard_normal((2, L, H * P)).astype(dtype)
    w = (1.0 + 0.1 * r.standard_normal(H * P)).astype(np.float32)
    tdt = torch.float16 if dtype == np.float16 else torch.float32
    y = torch.full((2, L, H * P), 1234.0, dtype=tdt, device=DEV)   # exact in binary16
    dims = m2.make_dims(2, L, H, P, N, G, 64, norm_group=group, io_dtype=m2.F16 if dtype == np.float16 else m2.F32)
    ws = m2.alloc_workspace(dims, DEV)
    say(f"[norm] H={H} G={G} group={group} {np.dtype(dtype).name}")
    window_checked(to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["D"]), y, ws, x=to_dev(inp["x"]),
                        B=to_dev(inp["B"]), C=to_dev(inp["C"]), seqlens=torch.tensor(lens, dtype=torch.int32,
                                                                                     device=DEV),
                        z=to_dev(z), norm_w=to_dev(w), chunk=64, norm_group=group)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    yr, _ = oracle.ssd_scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], seqlens=lens)
    for b, n in enumerate(lens):
        ref = oracle.gated_rmsnorm(yr[b, :n].reshape(n, H * P), z[b, :n], w, group)
        e = slice_err(got[b, :n].reshape(n, -1, group).transpose(1, 0, 2), ref.reshape(n, -1, group).transpose(1, 0, 2), 1)
        say(f"[norm] seq {b}: {e:.3e}")
        assert e <= Y_TOL
        assert np.all(got[b, n:] == 1234.0)


def test_mixer_core_xbc_slice_of_projection_rows():
    # xBC read in place from the input projection's rows [z | xBC | dt]: the
    # same bits as from a dense copy, and nothing read outside the slice
    H, P, G, N, L, Bsz = 16, 64, 2, 128, 300, 2
    inp = small_mixer(45, Bsz, L, H, G, N)
    Cn = H * P + 2 * G * N
    csi = (np.random.default_rng(46).standard_normal((Bsz, Cn, 3))).astype(np.float16)
    lens = [300, 157]
    say(f"[mixer] xBC as columns [{H * P}, {H * P + Cn}) of {2 * H * P + 2 * G * N + H + 8}-wide rows")
    dense = run_mixer(inp, H, P, G, N, 256, 512, seqlens=lens, conv_state_in=csi)
    strided = run_mixer(inp, H, P, G, N, 256, 512, seqlens=lens, conv_state_in=csi, xbc_in_rows=(H * P, H + 8))
    # y rows past a sequence's length are not written
    for b, n in enumerate(lens):
        assert np.array_equal(dense[0][b, :n], strided[0][b, :n])
        assert not np.isnan(strided[0][b, :n]).any()
    assert np.array_equal(dense[1], strided[1]) and np.array_equal(dense[2], strided[2])


def _projection(parts, pad):
    """The parts side by side in one tensor of wider rows ([z | xBC | dt] of
    an input projection, then `pad` NaN columns), and a view of each part."""
    lead = parts[0].shape[:-1]
    widths = [p.shape[-1] for p in parts]
    full = torch.full(lead + (sum(widths) + pad,), float("nan"), dtype=parts[0].dtype, device=DEV)
    views, c = [], 0
    for p, w in zip(parts, widths):
        full[..., c:c + w] = p
        views.append(full[..., c:c + w])
        c += w
    return views


@pytest.mark.parametrize("packed", [False, True])
def test_mixer_core_reads_z_xbc_dt_in_projection_rows(packed):
    # the whole mixer core on one projection output [z | xBC | dt]: raw dt
    # with its bias, conv state in and out, the gated norm; bit for bit the
    # result of dense copies, with NaN columns around the parts
    H, P, G, N, L = 16, 64, 2, 128, 300
    lens = [300, 157, 0, 64] if packed else [300, 157]
    s = synth.WindowShape(len(lens), L, H, P, N, G, 256, np.float16, "wide")
    inp = synth.mixer_inputs(s, 91, raw_dt=True)
    Cn = H * P + 2 * G * N
    csi = to_dev(np.random.default_rng(92).standard_normal((len(lens), Cn, 3)).astype(np.float16))
    if packed:
        z, xBC, dt = (to_dev(pack_rows(inp[k], lens)) for k in ("z", "xBC", "dt"))
        T = sum(lens)
        extra = dict(cu_seqlens=to_dev(cu_of(lens)), max_seqlen=L)
        dims = m2.make_dims(len(lens), L, H, P, N, G, 256, conv_width=4, norm_group=1024, packed_tokens=T)
        yshape = (T, H * P)
    else:
        z, xBC, dt = (to_dev(inp[k]) for k in ("z", "xBC", "dt"))
        extra = dict(seqlens=torch.tensor(lens, dtype=torch.int32, device=DEV))
        dims = m2.make_dims(len(lens), L, H, P, N, G, 256, conv_width=4, norm_group=1024)
        yshape = (len(lens), L, H * P)
    outs = []
    for zz, xx, dd in ((z, xBC, dt), tuple(_projection([z, xBC, dt], 24))):
        y = torch.full(yshape, 1234.0, dtype=torch.float16, device=DEV)
        hT = torch.empty((len(lens), H, P, N), dtype=torch.float32, device=DEV)
        cso = torch.empty((len(lens), Cn, 3), dtype=torch.float16, device=DEV)
        ws = m2.alloc_workspace(dims, DEV)
        window_checked(dd, to_dev(inp["A"]), to_dev(inp["D"]), y, ws, xBC=xx, conv_w=to_dev(inp["conv_w"]),
                            conv_b=to_dev(inp["conv_b"]), conv_state_in=csi, conv_state_out=cso, state_out=hT, z=zz,
                            norm_w=to_dev(inp["norm_w"]), chunk=256, norm_group=1024, ngroups=G, dstate=N,
                            headdim=P, dt_softplus=True, dt_bias=to_dev(inp["dt_bias"]), **extra)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (y, hT, cso)])
    say(f"[mixer] z, xBC and dt in projection rows, packed={packed}, lengths {lens}")
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    assert not np.isnan(outs[1][0]).any()
    # and the dense run against the oracle
    out_r, h_r, _ = oracle.mixer_core(inp["xBC"], inp["conv_w"], inp["conv_b"], inp["dt"], inp["A"], inp["D"],
                                      inp["z"], inp["norm_w"], H, P, G, N, 1024, conv_state=csi.cpu().numpy(),
                                      seqlens=lens, dt_bias=inp["dt_bias"], dt_softplus_raw=True)
    yd = unpack_rows(outs[0][0], lens, L) if packed else outs[0][0]
    for b, n in enumerate(lens):
        if n == 0:
            continue
        e = slice_err(yd[b, :n].reshape(n, -1, 1024).transpose(1, 0, 2), out_r[b, :n].reshape(n, -1, 1024).transpose(1, 0, 2), 1)
        assert e <= Y_TOL, (b, e)
    assert slice_err(outs[0][1], h_r, 2) <= S_TOL


def test_requant_window_reads_dt_in_wider_rows():
    inp = rand_window(93, 2, 300, 8, 128, 2)
    dense = run_requant(inp, seqlens=[300, 190])
    x, Bm, Cm = (to_dev(inp[k]) for k in ("x", "B", "C"))
    dt = _projection([to_dev(inp["dt"])], 40)[0]
    y = torch.empty((2, 300, 8 * 64), dtype=torch.float16, device=DEV)
    hT = torch.empty((2, 8, 64, 128), dtype=torch.float32, device=DEV)
    m2.requant_window(dt, to_dev(inp["A"]), to_dev(inp["D"]), y, x=x, B=Bm, C=Cm, state_out=hT,
                      seqlens=torch.tensor([300, 190], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    say("[requant] dt read from 48-column rows")
    got = y.cpu().numpy().reshape(2, 300, 8, 64)
    assert np.array_equal(got[0], dense[0][0]) and np.array_equal(got[1, :190], dense[0][1, :190])
    assert np.array_equal(hT.cpu().numpy(), dense[1])


def test_packed_mixer_core_xbc_slice_of_projection_rows():
    H, P, G, N, L = 16, 64, 2, 128, 300
    lens = [300, 0, 157, 64]
    s = synth.WindowShape(len(lens), L, H, P, N, G, 256, np.float16, "wide")
    inp = synth.mixer_inputs(s, 47)
    Cn = H * P + 2 * G * N
    T = sum(lens)
    xBC, dt, z = (to_dev(pack_rows(inp[k], lens)) for k in ("xBC", "dt", "z"))
    outs = []
    for x in (xBC, projection_rows(xBC, H * P, H + 24)):
        y = torch.full((T, H * P), 12345.0, dtype=torch.float16, device=DEV)
        hT = torch.empty((len(lens), H, P, N), dtype=torch.float32, device=DEV)
        cso = torch.empty((len(lens), Cn, 3), dtype=torch.float16, device=DEV)
        dims = m2.make_dims(len(lens), L, H, P, N, G, 256, conv_width=4, norm_group=1024, packed_tokens=T)
        ws = m2.alloc_workspace(dims, DEV)
        window_checked(dt, to_dev(inp["A"]), to_dev(inp["D"]), y, ws, xBC=x, conv_w=to_dev(inp["conv_w"]),
                            conv_b=to_dev(inp["conv_b"]), conv_state_out=cso, state_out=hT, z=z,
                            norm_w=to_dev(inp["norm_w"]), chunk=256, norm_group=1024, ngroups=G, dstate=N,
                            headdim=P, cu_seqlens=to_dev(cu_of(lens)), max_seqlen=L)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (y, hT, cso)])
    say(f"[packed] mixer with xBC in projection rows, lengths {lens}")
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    assert not np.isnan(outs[1][0]).any()


def test_mixer_core_full_size_sampled():
    s = synth.mixer_window()
    inp = synth.mixer_inputs(s, 1004)
    H, P, G, N = s.nheads, s.headdim, s.ngroups, s.dstate
    say("[mixer] full size B=4 L=2048")
    y, hT, _ = run_mixer(inp, H, P, G, N, s.chunk, H * P, want_conv_state=False)
    # without a final state (the conv writes no binary16 remainder of B, the
    # scan takes B as binary16 alone)
    y_ns, _, _ = run_mixer(inp, H, P, G, N, s.chunk, H * P, want_conv_state=False, want_state=False)
    for b in range(s.batch):
        sub = {k: (v[b:b + 1] if (v.ndim > 1 and k in ("xBC", "dt", "z")) else v) for k, v in inp.items()}
        out_r, h_r, _ = oracle.mixer_core(sub["xBC"], inp["conv_w"], inp["conv_b"], sub["dt"], inp["A"], inp["D"],
                                          sub["z"], inp["norm_w"], H, P, G, N, H * P)
        e = slice_err(y[b][None], out_r[0][None], 1)
        es = slice_err(hT[b:b + 1], h_r, 2)
        e_ns = slice_err(y_ns[b][None], out_r[0][None], 1)
        say(f"[mixer] seq {b}: out {e:.3e} state {es:.3e}; without a final state: out {e_ns:.3e}")
        assert e <= Y_TOL and es <= S_TOL and e_ns <= Y_TOL


# ---- decode --------------------------------------------------------------------
def decode_inputs(seed, T, Bsz, H, N, G, P=64):
    prm = synth.decode_params(seed, Bsz, H, P, N)
    steps = [synth.decode_step_inputs(seed, t, prm["dt0"], Bsz, H, P, N, G) for t in range(T)]
    stack = {k: np.stack([s[k] for s in steps]) for k in ("x", "dt", "B", "C")}
    return prm, stack


@pytest.mark.parametrize("N", [16, 64, 128])
def test_decode_f16_state_small(N):
    T, Bsz, H, G = 8, 3, 16, 2
    prm, st = decode_inputs(51 + N, T, Bsz, H, N, G)
    s16 = torch.empty((Bsz, H, 64, N), dtype=torch.float16, device=DEV)
    m2.state_load(to_dev(prm["state"]), s16)
    bits = prm["state"].astype(np.float16).view(np.uint16).copy()
    torch.cuda.synchronize()
    assert np.array_equal(s16.cpu().numpy().view(np.uint16), bits)
    yg = []
    for t in range(T):
        y = torch.empty((Bsz, H, 64), dtype=torch.float16, device=DEV)
        m2.decode_step(to_dev(st["x"][t]), to_dev(st["dt"][t]), to_dev(st["B"][t]), to_dev(st["C"][t]),
                       to_dev(prm["A"]), to_dev(prm["D"]), s16, y)
        yg.append(y.cpu().numpy())
    yr = oracle.decode_f16state(st["x"], st["dt"], prm["A"], st["B"], st["C"], prm["D"], bits)
    sg = s16.cpu().numpy()
    same = np.mean(sg.view(np.uint16) == bits)
    ey = slice_err(np.stack(yg).transpose(1, 2, 0, 3), yr.transpose(1, 2, 0, 3), 2)
    es = slice_err(sg.astype(np.float64), bits.view(np.float16).astype(np.float64), 2)
    say(f"[decode] N={N}: state identical {same:.6f} state err {es:.2e} y err {ey:.2e}")
    assert same == 1.0 and es <= S_TOL and ey <= Y_TOL


def test_decode_raw_dt_f16_state_bit_exact():
    T, Bsz, H, N, G = 6, 3, 16, 128, 2
    prm = synth.decode_params(91, Bsz, H, 64, N)
    steps = [synth.decode_step_inputs(91, t, prm["dt0"], Bsz, H, 64, N, G, raw_dt=True) for t in range(T)]
    st = {k: np.stack([s[k] for s in steps]) for k in ("x", "dt", "B", "C")}
    bias = synth.dt_bias("wide", prm["dt0"])
    s16 = torch.empty((Bsz, H, 64, N), dtype=torch.float16, device=DEV)
    m2.state_load(to_dev(prm["state"]), s16)
    bits = prm["state"].astype(np.float16).view(np.uint16).copy()
    yg = []
    for t in range(T):
        y = torch.empty((Bsz, H, 64), dtype=torch.float16, device=DEV)
        m2.decode_step(to_dev(st["x"][t]), to_dev(st["dt"][t]), to_dev(st["B"][t]), to_dev(st["C"][t]),
                       to_dev(prm["A"]), to_dev(prm["D"]), s16, y, dt_softplus=True, dt_bias=to_dev(bias))
        yg.append(y.cpu().numpy())
    yr = oracle.decode_f16state(st["x"], st["dt"], prm["A"], st["B"], st["C"], prm["D"], bits, dt_bias=bias,
                                dt_softplus_raw=True)
    same = np.mean(s16.cpu().numpy().view(np.uint16) == bits)
    ey = slice_err(np.stack(yg).transpose(1, 2, 0, 3), yr.transpose(1, 2, 0, 3), 2)
    say(f"[decode] raw dt: state identical {same:.6f} y err {ey:.2e}")
    assert same == 1.0 and ey <= Y_TOL


def test_decode_f32_state_matches_fp64_recurrence():
    T, Bsz, H, N, G = 12, 2, 8, 128, 2
    prm, st = decode_inputs(61, T, Bsz, H, N, G)
    s32 = to_dev(prm["state"]).clone()
    yg = []
    for t in range(T):
        y = torch.empty((Bsz, H, 64), dtype=torch.float16, device=DEV)
        m2.decode_step(to_dev(st["x"][t]), to_dev(st["dt"][t]), to_dev(st["B"][t]), to_dev(st["C"][t]),
                       to_dev(prm["A"]), to_dev(prm["D"]), s32, y)
        yg.append(y.cpu().numpy())
    tr = lambda a: np.transpose(a, (1, 0) + tuple(range(2, a.ndim)))
    yr, hr = oracle.ssd_scan(tr(st["x"]), tr(st["dt"]), prm["A"], tr(st["B"]), tr(st["C"]), prm["D"],
                             h0=prm["state"].astype(np.float64))
    ey = slice_err(np.stack(yg).transpose(1, 2, 0, 3), np.transpose(yr, (0, 2, 1, 3)), 2)
    es = slice_err(s32.cpu().numpy(), hr, 2)
    say(f"[decode f32] y {ey:.2e} state {es:.2e}")
    assert ey <= Y_TOL and es <= S_TOL


def test_state_store_roundtrip():
    r = np.random.default_rng(71)
    v = (r.standard_normal((2, 4, 64, 128)) * np.exp2(r.integers(-26, 17, (2, 4, 64, 128)))).astype(np.float32)
    s16 = torch.empty(v.shape, dtype=torch.float16, device=DEV)
    m2.state_load(to_dev(v), s16)
    back = torch.empty(v.shape, dtype=torch.float32, device=DEV)
    m2.state_store(s16, back)
    torch.cuda.synchronize()
    assert np.array_equal(s16.cpu().numpy().view(np.uint16), v.astype(np.float16).view(np.uint16))
    assert np.array_equal(back.cpu().numpy(), v.astype(np.float16).astype(np.float32))


def test_decode_full_size_1024_steps_sampled():
    d = synth.DECODE
    Bsz, H, P, N, G, T = d["batch"], d["nheads"], d["headdim"], d["dstate"], d["ngroups"], d["steps"]
    seed = 1003
    prm = synth.decode_params(seed, Bsz, H, P, N)
    s16 = torch.empty((Bsz, H, P, N), dtype=torch.float16, device=DEV)
    m2.state_load(to_dev(prm["state"]), s16)
    sample = (0, 9, 18, 27, 37, 45, 54, 63)     # eight sequences spread over the 64, the last included
    keep = {k: [] for k in ("x", "dt", "B", "C", "y")}
    A, D = to_dev(prm["A"]), to_dev(prm["D"])
    y = torch.empty((Bsz, H, P), dtype=torch.float16, device=DEV)
    say(f"[decode] full: {T} steps, B={Bsz}")
    for t in range(T):
        st = synth.decode_step_inputs(seed, t, prm["dt0"], Bsz, H, P, N, G)
        m2.decode_step(to_dev(st["x"]), to_dev(st["dt"]), to_dev(st["B"]), to_dev(st["C"]), A, D, s16, y)
        for k in ("x", "dt", "B", "C"):
            keep[k].append(st[k][list(sample)])
        keep["y"].append(y[list(sample)].cpu().numpy())
    torch.cuda.synchronize()
    bits = prm["state"][list(sample)].astype(np.float16).view(np.uint16).copy()
    yr = oracle.decode_f16state(*(np.stack(keep[k]) for k in ("x", "dt")), prm["A"],
                                np.stack(keep["B"]), np.stack(keep["C"]), prm["D"], bits)
    sg = s16.cpu().numpy()[list(sample)]
    same = np.mean(sg.view(np.uint16) == bits)
    es = slice_err(sg.astype(np.float64), bits.view(np.float16).astype(np.float64), 2)
    ey = slice_err(np.stack(keep["y"]).transpose(1, 2, 0, 3), yr.transpose(1, 2, 0, 3), 2)
    say(f"[decode] full sampled: identical {same:.6f} state err {es:.2e} y err {ey:.2e}")
    assert same == 1.0 and es <= S_TOL and ey <= Y_TOL

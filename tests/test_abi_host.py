"""Host-side checks of the C ABI: the library loads without a GPU, exports
every entry point the header declares, and validates arguments before
enqueuing anything (the pointers below are never dereferenced: each case
is refused on the host)."""
import ctypes
import os
import re

import pytest

import mamba_ssd_scan_amd as m2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    text = open(os.path.join(ROOT, "include", "mamba2ssd.h")).read()
    return sorted(set(re.findall(r"\b(mamba2_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = m2.load_library()
    syms = header_symbols()
    assert len(syms) >= 8
    for s in syms:
        assert hasattr(lib, s), s


def test_version_and_status_strings():
    lib = m2.load_library()
    assert m2.abi_version() == 8
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.mamba2_status_str(code)
    assert lib.mamba2_status_str(77) == b"unknown status"


def layer_dims(**kw):
    base = dict(batch=1, seqlen=2048, nheads=128, headdim=64, dstate=128, ngroups=8, chunk=256)
    base.update(kw)
    return m2.make_dims(**base)


def ws_formula(chunk_items, N, conv_bytes=0, blo_bytes=0):
    # control block; per (chunk, sequence, head, half) item a 64-bit flag word
    # and an fp32 aggregate of N x 32; the conv output and, for binary16, the
    # remainder of its B channels (the gated norm needs no workspace)
    up = lambda v: (v + 255) // 256 * 256
    items = 2 * chunk_items
    off = up(11 * 32 * 4)
    off = up(off + items * 8)
    off = up(off + items * N * 32 * 4)
    off = up(off + conv_bytes)
    return up(off + blo_bytes)


def test_workspace_size_formula():
    assert m2.window_workspace_bytes(layer_dims()) == ws_formula(8 * 128, 128)
    n2 = m2.window_workspace_bytes(layer_dims(batch=4, norm_group=8192, conv_width=4))
    assert n2 == ws_formula(8 * 4 * 128, 128, 4 * 2048 * 10240 * 2, 4 * 2048 * 8 * 128 * 2)
    assert m2.window_workspace_bytes(layer_dims(dstate=16, ngroups=1, nheads=4, seqlen=256, chunk=64)) == \
        ws_formula(4 * 4, 16)


def test_segment_count_does_not_change_the_workspace():
    # the hand-off area is sized for one segment per chunk, the most there can be
    for k in (0, 1, 3, 8, 100):
        assert m2.window_workspace_bytes(layer_dims(segments=k)) == ws_formula(8 * 128, 128)


def test_long_sequences_beyond_32_bit_rows_are_refused():
    # 2^31 bytes of one sequence's x rows: 131072 tokens x 8192 channels x 2 bytes
    n = ctypes.c_size_t(0)
    lib = m2.load_library()
    assert lib.mamba2_window_workspace_bytes(ctypes.byref(layer_dims(seqlen=131072)), ctypes.byref(n)) == -2
    assert lib.mamba2_window_workspace_bytes(ctypes.byref(layer_dims(seqlen=131071)), ctypes.byref(n)) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(headdim=32), -2), (dict(dstate=96), -2), (dict(chunk=100), -2), (dict(conv_width=3), -2),
    (dict(nheads=100, ngroups=8), -1), (dict(batch=0), -1), (dict(seqlen=0), -1),
    (dict(norm_group=1000), -1), (dict(norm_group=32), -2), (dict(norm_group=-1), -1),
    (dict(io_dtype=7), -1), (dict(segments=-1), -1), (dict(dt_softplus=2), -1),
    (dict(packed_tokens=-1), -1),
])
def test_workspace_query_rejects(kw, code):
    lib = m2.load_library()
    n = ctypes.c_size_t(0)
    assert lib.mamba2_window_workspace_bytes(ctypes.byref(layer_dims(**kw)), ctypes.byref(n)) == code


FAKE = 0x7F0000000000  # never dereferenced: every call below is refused on the host


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0   # counts devices without initialising them
    except Exception:
        return False


# The refusals below pass placeholder pointers: they run where no GPU is
# visible, so that a refusal that failed could never launch on them.
fake_pointers = pytest.mark.skipif(_gpu_visible(), reason="placeholder-pointer calls run only where no GPU is visible")


def window_io(**over):
    L, H, P, N, G = 2048, 128, 64, 128, 8
    MB = 1 << 26
    base = dict(x=FAKE, B=FAKE + MB, C=FAKE + 2 * MB, dt=FAKE + 3 * MB, A=FAKE + 4 * MB, D=FAKE + 4 * MB + 4096,
                y=FAKE + 8 * MB)
    base.update(over)
    return m2._WindowIO(**base)


def call_window(io, dims=None, ws=FAKE + (1 << 30), ws_bytes=None):
    lib = m2.load_library()
    dims = dims or layer_dims()
    if ws_bytes is None:
        ws_bytes = m2.window_workspace_bytes(dims)
    return lib.mamba2_conv_scan_window(ctypes.byref(dims), ctypes.byref(io), ctypes.c_void_p(ws), ws_bytes, None)


@fake_pointers
def test_window_validation_codes():
    assert call_window(window_io(x=None)) == -1
    assert call_window(window_io(y=None)) == -1
    assert call_window(window_io(x=FAKE + 2)) == -3
    assert call_window(window_io(), ws=None) == -4
    assert call_window(window_io(), ws_bytes=1024) == -4
    assert call_window(window_io(), ws=FAKE + (1 << 30) + 16) == -3
    # output overlapping an input
    assert call_window(window_io(y=FAKE + 1024)) == -1
    # workspace overlapping the output
    assert call_window(window_io(), ws=FAKE + 8 * (1 << 26)) == -1
    # fused conv needs xBC and conv weights; the norm needs z and its weight
    assert call_window(window_io(), dims=layer_dims(conv_width=4)) == -1
    assert call_window(window_io(), dims=layer_dims(norm_group=8192)) == -1


@fake_pointers
def test_packed_layout_validation_codes():
    MB = 1 << 26
    packed = layer_dims(batch=4, packed_tokens=5000)
    cu = FAKE + 5 * MB
    # packed rows need their offsets, and offsets need the packed layout
    assert call_window(window_io(), dims=packed) == -1
    assert call_window(window_io(cu_seqlens=cu)) == -1
    # lengths and offsets are exclusive
    assert call_window(window_io(cu_seqlens=cu, seqlens=cu + 4096), dims=packed) == -1
    assert call_window(window_io(cu_seqlens=cu + 2), dims=packed) == -3
    # offsets overlapping an output
    assert call_window(window_io(cu_seqlens=FAKE + 8 * MB + 64), dims=packed) == -1
    # the same rules for the requantized window
    assert call_requant(window_io(), dims=packed) == -1
    assert call_requant(window_io(cu_seqlens=cu)) == -1
    assert call_requant(window_io(cu_seqlens=cu + 2), dims=packed) == -3
    # the workspace is sized by batch x seqlen whatever the packed row count
    assert m2.window_workspace_bytes(packed) == m2.window_workspace_bytes(layer_dims(batch=4))


@fake_pointers
def test_xbc_row_stride_validation_codes():
    # xBC as a slice of wider rows: at least conv_dim (10240) elements apart,
    # 16-byte aligned rows; the stride sets the range checked for overlaps
    MB = 1 << 26
    conv = layer_dims(conv_width=4)
    io = lambda **kw: window_io(x=None, B=None, C=None, xBC=FAKE + 6 * MB, conv_w=FAKE + 5 * MB, **kw)
    assert call_window(io(xBC_ld=10239), dims=conv) == -1
    assert call_window(io(xBC_ld=-1), dims=conv) == -1
    assert call_window(io(xBC_ld=1 << 41), dims=conv) == -1
    assert call_window(io(xBC_ld=10244), dims=conv) == -3       # 20488-byte rows
    # 2048 rows of 4 x 10240 elements from 6 x 64 MiB reach y at 8 x 64 MiB
    assert call_window(io(xBC_ld=40960), dims=conv) == -1


@fake_pointers
def test_z_and_dt_row_stride_validation_codes():
    # z rows: at least H*P (8192) elements apart, 16-byte aligned; dt rows at
    # least H (128) apart; a negative stride is invalid
    MB = 1 << 26
    norm = layer_dims(norm_group=8192)
    io = lambda **kw: window_io(z=FAKE + 5 * MB, norm_w=FAKE + 4 * MB + 8192, **kw)
    assert call_window(io(z_ld=8191), dims=norm) == -1
    assert call_window(io(z_ld=-8), dims=norm) == -1
    assert call_window(io(z_ld=8196), dims=norm) == -3        # 16392-byte rows
    assert call_window(window_io(dt_ld=127)) == -1
    assert call_window(window_io(dt_ld=-1)) == -1
    # one sequence's dt rows must stay within 2^31 bytes: 2048 rows of 2^20 elements
    assert call_window(window_io(dt_ld=1 << 20)) == -2
    # the stride sets the range checked for overlaps: 2048 rows 120000
    # elements apart from 3 x 64 MiB run past y at 8 x 64 MiB
    assert call_window(window_io(dt_ld=120000)) == -1
    assert call_requant(window_io(dt_ld=127)) == -1
    assert call_requant(window_io(dt_ld=120000)) == -1


def call_requant(io, dims=None):
    lib = m2.load_library()
    dims = dims or layer_dims()
    return lib.mamba2_requant_window(ctypes.byref(dims), ctypes.byref(io), None)


@fake_pointers
def test_requant_window_validation_codes():
    # plain x, B, C only; every refusal happens on the host
    assert call_requant(window_io(), dims=layer_dims(conv_width=4)) == -2
    assert call_requant(window_io(), dims=layer_dims(norm_group=8192)) == -2
    assert call_requant(window_io(), dims=layer_dims(headdim=32)) == -2
    assert call_requant(window_io(), dims=layer_dims(seqlen=0)) == -1
    assert call_requant(window_io(x=None)) == -1
    assert call_requant(window_io(y=None)) == -1
    assert call_requant(window_io(B=FAKE + (1 << 26) + 8)) == -3
    # y overlapping x
    assert call_requant(window_io(y=FAKE + 1024)) == -1


@fake_pointers
def test_decode_and_state_validation_codes():
    lib = m2.load_library()
    d = m2.make_dims(64, 1, 128, 64, 128, 8, 256, state_dtype=m2.F16)
    MB = 1 << 26
    io = m2._DecodeIO(FAKE, FAKE + MB, FAKE + 2 * MB, FAKE + 3 * MB, FAKE + 4 * MB, FAKE + 5 * MB,
                      FAKE + 6 * MB, FAKE + 20 * MB)
    bad = m2._DecodeIO(FAKE, FAKE + MB, FAKE + 2 * MB, FAKE + 3 * MB, FAKE + 4 * MB, FAKE + 5 * MB,
                       FAKE + 6 * MB, FAKE + 6 * MB + 64)
    assert lib.mamba2_decode_step(ctypes.byref(d), ctypes.byref(bad), None) == -1   # y inside the state
    null = m2._DecodeIO(FAKE, FAKE + MB, None, FAKE + 3 * MB, FAKE + 4 * MB, FAKE + 5 * MB, FAKE + 6 * MB,
                        FAKE + 20 * MB)
    assert lib.mamba2_decode_step(ctypes.byref(d), ctypes.byref(null), None) == -1
    mis = m2._DecodeIO(FAKE + 8, FAKE + MB, FAKE + 2 * MB, FAKE + 3 * MB, FAKE + 4 * MB, FAKE + 5 * MB,
                       FAKE + 6 * MB, FAKE + 20 * MB)
    assert lib.mamba2_decode_step(ctypes.byref(d), ctypes.byref(mis), None) == -3
    d2 = m2.make_dims(64, 1, 128, 64, 100, 8, 256)
    assert lib.mamba2_decode_step(ctypes.byref(d2), ctypes.byref(io), None) == -2
    assert lib.mamba2_state_load(ctypes.byref(d), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 64), None) == -1
    assert lib.mamba2_state_load(ctypes.byref(d), None, ctypes.c_void_p(FAKE), None) == -1
    assert lib.mamba2_state_store(ctypes.byref(d), ctypes.c_void_p(FAKE + 2), ctypes.c_void_p(FAKE + MB * 40),
                                  None) == -3


@fake_pointers
def test_mixer_decode_validation_codes():
    lib = m2.load_library()
    MB = 1 << 26
    H, P, N, G = 128, 64, 128, 8

    def dims(**kw):
        base = dict(batch=64, nheads=H, headdim=P, dstate=N, ngroups=G, norm_group=8192)
        base.update(kw)
        return m2.mixer_decode_dims(**base)

    def io(**over):
        base = dict(xBC=FAKE, conv_w=FAKE + MB, conv_state=FAKE + 2 * MB, dt=FAKE + 3 * MB, A=FAKE + 4 * MB,
                    D=FAKE + 4 * MB + 4096, state=FAKE + 8 * MB, z=FAKE + 5 * MB, norm_w=FAKE + 6 * MB,
                    y=FAKE + 7 * MB)
        base.update(over)
        return m2._MixerDecodeIO(**base)

    def call(i, d=None, ws=FAKE + (1 << 30), ws_bytes=None):
        d = d or dims()
        if ws_bytes is None:
            ws_bytes = m2.mixer_decode_workspace_bytes(d)
        return lib.mamba2_mixer_decode_step(ctypes.byref(d), ctypes.byref(i), ctypes.c_void_p(ws), ws_bytes, None)

    n = ctypes.c_size_t(0)
    for kw, code in ((dict(norm_group=100), -1), (dict(norm_group=16384), -1), (dict(norm_group=32), -2),
                     (dict(norm_group=-1), -1), (dict(headdim=32), -2), (dict(dstate=96), -2)):
        assert lib.mamba2_mixer_decode_workspace_bytes(ctypes.byref(dims(**kw)), ctypes.byref(n)) == code, kw
    d3 = m2.make_dims(64, 1, H, P, N, G, 256, conv_width=0)
    assert lib.mamba2_mixer_decode_workspace_bytes(ctypes.byref(d3), ctypes.byref(n)) == -2   # needs the conv
    # a fixed region of 16384 arrival counters (one per (sequence, group)),
    # then, with the norm, the sums of g^2 over each half of every head
    up = lambda v: (v + 255) // 256 * 256
    assert m2.mixer_decode_workspace_bytes(dims()) == up(16384 * 4 + 64 * H * 2 * 4)
    assert m2.mixer_decode_workspace_bytes(dims(norm_group=0)) == 16384 * 4
    assert lib.mamba2_mixer_decode_workspace_bytes(ctypes.byref(dims(batch=2048)), ctypes.byref(n)) == 0
    assert lib.mamba2_mixer_decode_workspace_bytes(ctypes.byref(dims(batch=2049)), ctypes.byref(n)) == -2
    # more than 256 norm groups per token
    assert lib.mamba2_mixer_decode_workspace_bytes(ctypes.byref(m2.mixer_decode_dims(4, 512, 64, 128, 8, 64)),
                                                   ctypes.byref(n)) == -2
    assert call(io(xBC=None)) == -1
    assert call(io(z=None)) == -1
    assert call(io(conv_w=FAKE + MB + 4)) == -3
    assert call(io(state=FAKE + 8 * MB + 8)) == -3
    assert call(io(y=FAKE + 7 * MB + 1)) == -3
    assert call(io(), ws=None) == -4
    assert call(io(), ws_bytes=1024) == -4
    assert call(io(), ws=FAKE + (1 << 30) + 64) == -3
    # y inside the state; the conv history overlapping the raw input; the
    # workspace overlapping the conv history
    assert call(io(y=FAKE + 8 * MB + 4096)) == -1
    assert call(io(conv_state=FAKE + 1024)) == -1
    assert call(io(), ws=FAKE + 2 * MB) == -1


@fake_pointers
def test_window_take_error_validation_codes():
    lib = m2.load_library()
    v = ctypes.c_uint32(7)
    ws = ctypes.c_void_p(FAKE)
    assert lib.mamba2_window_take_error(None, 1 << 20, ctypes.byref(v), None) == -1
    assert lib.mamba2_window_take_error(ws, 1 << 20, None, None) == -1
    assert lib.mamba2_window_take_error(ws, 64, ctypes.byref(v), None) == -4      # smaller than the control block
    assert lib.mamba2_window_take_error(ctypes.c_void_p(FAKE + 128), 1 << 20, ctypes.byref(v), None) == -3
    assert v.value == 7                                                            # untouched on error


@fake_pointers
def test_mixer_decode_noalloc_validation_codes():
    """The no-allocation step refuses on the host what the workspace form
    refuses, plus requests whose workspace would exceed the fixed array."""
    lib = m2.load_library()
    MB = 1 << 36            # far enough apart that no batch below makes the ranges overlap
    H, P, N, G = 128, 64, 128, 8
    cap = m2.mixer_decode_noalloc_max_bytes()
    assert cap == 4 << 20

    def io(**over):
        base = dict(xBC=FAKE, conv_w=FAKE + MB, conv_state=FAKE + 2 * MB, dt=FAKE + 3 * MB, A=FAKE + 4 * MB,
                    D=FAKE + 4 * MB + 4096, state=FAKE + 8 * MB, z=FAKE + 5 * MB, norm_w=FAKE + 6 * MB,
                    y=FAKE + 7 * MB)
        base.update(over)
        return m2._MixerDecodeIO(**base)

    def call(i, batch=64, **kw):
        d = m2.mixer_decode_dims(batch, H, P, N, G, **kw)
        return lib.mamba2_mixer_decode_step_noalloc(ctypes.byref(d), ctypes.byref(i), None)

    assert call(io(xBC=None), norm_group=8192) == -1
    assert call(io(z=None), norm_group=8192) == -1
    assert call(io(conv_w=FAKE + MB + 4), norm_group=8192) == -3
    assert call(io(y=FAKE + 8 * MB + 4096), norm_group=8192) == -1
    assert call(io(), norm_group=100) == -1
    assert lib.mamba2_mixer_decode_step_noalloc(None, ctypes.byref(io()), None) == -1
    d = m2.mixer_decode_dims(64, H, P, N, G, 8192)
    assert lib.mamba2_mixer_decode_step_noalloc(ctypes.byref(d), None, None) == -1
    # the largest batch whose workspace fits, and the first that does not
    # (one group, so that the counter limit of 16384 (sequence, group) pairs
    # is not what refuses the request)
    per_seq = lambda b: m2.mixer_decode_workspace_bytes(m2.mixer_decode_dims(b, H, P, N, 1, 8192))
    big = 1
    while per_seq(big * 2) <= cap:
        big *= 2
    while per_seq(big + 1) <= cap:
        big += 1
    assert per_seq(big) <= cap < per_seq(big + 1) and big == 4032
    d1 = m2.mixer_decode_dims(big + 1, H, P, N, 1, 8192)
    assert lib.mamba2_mixer_decode_step_noalloc(ctypes.byref(d1), ctypes.byref(io()), None) == -4


@fake_pointers
def test_scan_grad_validation_codes():
    lib = m2.load_library()
    MB = 1 << 26
    n = ctypes.c_size_t(0)
    for kw, code in ((dict(conv_width=4), -2), (dict(norm_group=8192), -2), (dict(packed_tokens=100), -2),
                     (dict(headdim=32), -2), (dict(dstate=96), -2), (dict(seqlen=0), -1)):
        assert lib.mamba2_scan_grad_workspace_bytes(ctypes.byref(layer_dims(**kw)), ctypes.byref(n)) == code, kw
    # per-head dB and dC, then e and q per (token, head) and four per-(sequence, head) scalars
    up = lambda v: (v + 255) // 256 * 256
    L, H, N = 2048, 128, 128
    w = up(L * H * N * 4)
    w = up(w + L * H * N * 4)
    for _ in range(2):
        w = up(w + L * H * 4)
    for _ in range(4):
        w = up(w + H * 4)
    assert m2.scan_grad_workspace_bytes(layer_dims()) == w

    def io(**over):
        base = dict(x=FAKE, dt=FAKE + MB, A=FAKE + 2 * MB, B=FAKE + 3 * MB, C=FAKE + 4 * MB, D=FAKE + 2 * MB + 4096,
                    dy=FAKE + 5 * MB, dx=FAKE + 8 * MB, ddt=FAKE + 10 * MB, dB=FAKE + 11 * MB, dC=FAKE + 12 * MB,
                    dA=FAKE + 13 * MB, dD=FAKE + 13 * MB + 4096)
        base.update(over)
        return m2._ScanGradIO(**base)

    def call(i, d=None, ws=FAKE + (1 << 32), ws_bytes=None):
        d = d or layer_dims()
        if ws_bytes is None:
            ws_bytes = m2.scan_grad_workspace_bytes(d)
        return lib.mamba2_scan_grad(ctypes.byref(d), ctypes.byref(i), ctypes.c_void_p(ws), ws_bytes, None)

    assert call(io(dy=None)) == -1
    assert call(io(dC=None)) == -1
    assert call(io(), d=layer_dims(dt_softplus=1)) == -1          # needs ddt_bias
    assert call(io(dx=FAKE + 8 * MB + 2)) == -3
    assert call(io(dstate_in=FAKE + 14 * MB + 4)) == -3
    assert call(io(), ws=None) == -4
    assert call(io(), ws_bytes=1024) == -4
    assert call(io(), ws=FAKE + (1 << 32) + 128) == -3
    assert call(io(dx=FAKE + 1024)) == -1                            # dx over x
    assert call(io(dB=FAKE + 10 * MB + 4096)) == -1                  # dB over ddt
    assert call(io(), ws=FAKE + 8 * MB) == -1                        # workspace over dx


def test_binding_raises_without_gpu_tensors():
    import torch
    with pytest.raises(ValueError):
        m2._ptr(torch.zeros(4))

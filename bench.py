"""Benchmark of the Mamba-2 mixer core on one MI355X.

Headline: the chunked (state-space-dual) window scan at the Mamba2-8B layer
shape -- batch 1, L=2048, H=128, P=64, N=128, G=8, chunk 256, fp16 I/O, fp32
state -- in tokens/s.  A "step" is one call of mamba2_conv_scan_window over
one window.  Inputs are resident in HBM before timing starts; several buffer
sets are rotated so that the working set exceeds the 256 MB Infinity Cache.
The one-token decode step (64 sequences, binary16 resident state) is timed in
the same run and reported in microseconds per step.  Parity against the CPU
oracle is re-checked on the timed buffers before any number is printed.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints one JSON line.

  --copy-probe MIB   copy MIB of device memory a few times and exit; the HBM
                     counters of this plain copy calibrate the counters of the
                     scan kernel (profiles/window_layer_traffic.txt)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MFMA_F16_PEAK = 2500.0     # TFLOP/s dense f16
# fp32 VALU lane-operations: 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz (a 64-wide
# fp32 multiply issues in two clocks, which is also the published 157.3 TFLOP/s
# fp32 vector rate counting an fma as two flops); no packed math
VALU_PEAK_TOPS = 256 * 4 * 32 * 2.4e9 / 1e12
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "window_layer_traffic.txt")
# the window kernel's sources: the kernel, its argument block and the helpers it includes
KERNEL_SOURCES = [os.path.join(ROOT, "mamba_ssd_scan_amd", "csrc", n)
                  for n in ("ssd_scan.hip", "ssd_scan.h", "gfx950_ops.h", "common.h")]


def kernel_source_hash():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the scan kernel from the committed counter
    summary, or None when the summary is missing or was taken on a different
    kernel source."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if "=" in line and not line.lstrip().startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256_16") != kernel_source_hash():
            return None
        return int(float(kv["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def copy_probe(mib):
    """Plain device copies of known size (counter calibration)."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch_read": n, "copy_bytes_per_launch_write": n, "launches": 5}), flush=True)


def run_metadata(torch, m2):
    """Where the numbers come from: the tree the library was built from, its
    ABI version, the GPU architecture, the ROCm and torch builds, the host
    CPU."""
    meta = {"abi_version": m2.abi_version()}
    info = os.path.join(ROOT, "mamba_ssd_scan_amd", "build_info.json")
    try:
        with open(info) as f:
            meta.update(json.load(f))
    except (OSError, ValueError):
        meta["git_sha"] = None
    props = torch.cuda.get_device_properties(0)
    meta["gpu"] = props.name
    meta["gfx_arch"] = getattr(props, "gcnArchName", None)
    meta["cus"] = props.multi_processor_count
    meta["torch"] = torch.__version__
    meta["hip"] = getattr(torch.version, "hip", None)
    try:
        with open("/opt/rocm/.info/version") as f:
            meta["rocm"] = f.read().strip()
    except OSError:
        meta["rocm"] = None
    meta["cpu_model"] = cpu_model()
    meta["cpu_threads_available"] = len(os.sched_getaffinity(0))
    return meta


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_bandwidth(torch, dev, stream, mib=1024, reps=10):
    """Read + write bytes per second of a plain device-to-device copy of
    `mib` MiB, timed with events on the benchmark's stream (the practical
    ceiling of a streaming kernel on this part)."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        for _ in range(3):
            dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n / sec / 1e9


def window_bytes(B, L, H, P, N, G, lens=None):
    """Algorithmic HBM bytes of one window call: every input element read once,
    every output written once, fp16 I/O, fp32 final state."""
    toks = sum(lens) if lens else B * L
    per_tok = 2 * H * P + 2 * H + 2 * 2 * G * N + 2 * H * P   # x, dt, B, C in; y out
    return toks * per_tok + B * H * P * N * 4 + 2 * H * 4       # final state, A, D


def mixer_bytes(B, L, H, P, N, G):
    """Algorithmic bytes of one mixer-core call (f16 I/O, no conv state in):
    raw xBC, dt and z read, the normed output written, the final states and
    the conv states written, the conv weights and bias read."""
    Cd = H * P + 2 * G * N
    return B * L * (2 * Cd + 2 * H + 2 * H * P + 2 * H * P) + B * H * P * N * 4 + B * Cd * 3 * 2 + Cd * 5 * 4


def decode_bytes(B, H, P, N, G):
    """Algorithmic bytes of one decode step with a binary16 resident state."""
    return B * H * P * N * 2 * 2 + B * H * P * 2 * 2 + B * G * N * 2 * 2 + B * H * 2 + 2 * H * 4


def mixer_decode_bytes(B, H, P, N, G):
    """Algorithmic bytes of one fused mixer step (f16 I/O, binary16 resident
    state): the state read and written, this token's raw xBC, dt and z read,
    the conv history read and written, the output written, the conv weights,
    conv bias, norm weight, A and D read."""
    Cd = H * P + 2 * G * N
    return (B * H * P * N * 2 * 2 + B * Cd * 2 + B * Cd * 3 * 2 * 2 + B * H * 2 + B * H * P * 2 * 2
            + Cd * 4 * 4 + Cd * 4 + H * P * 4 + 2 * H * 4)


def window_mfma_flops(L, H, P, N, Q=256, segments=8, step=32, half=32, heads_per_block=4):
    """f16 MFMA flops the window kernel issues for one sequence with a final
    state (16x16x32 instructions, 16384 flops each), for the chunks split into
    `segments` runs of consecutive chunks (the split the library picks for
    one layer window).  Per (half of a head) and 32-token step: the local-state
    pass, run on every segment but the last, takes N/16 x half/16
    instructions; the output pass takes the masked product (2 x half/16), the
    carry readout (2 x half/16 x N/32) and the running-state update
    (N/16 x half/16) on every step, and a share of the causal C.B^T blocks
    (3 blocks x N/32 per step), which one workgroup of heads_per_block heads
    (two waves per head) computes once."""
    J = Q // step
    C = L // Q
    cps = -(-C // segments)
    nt, pt, km = N // 16, half // 16, max(N // 32, 1)
    waves = heads_per_block * (P // half)
    local = nt * pt * J * (C - cps)                      # all chunks outside the last segment
    out = (2 * pt + 2 * pt * km) * J * C
    upd = nt * pt * J * C
    cb = 3 * km * J * C / waves
    return H * (P // half) * (local + out + upd + cb) * 16384


def _timed(fn, min_s=2.0, max_reps=20):
    """Seconds per call of fn, repeated until min_s has passed."""
    t0 = time.perf_counter()
    reps = 0
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_s or reps >= max_reps:
            return el / reps, reps


def cpu_baselines(inp, s, args):
    """The oracle as it stands (fp64 sequential C, OpenMP over (sequence,
    head)), timed on this host on bounded samples of each workload and scaled
    to the whole workload: all available cores and one thread.  Reported
    beside the GPU figures, never a target."""
    import oracle
    import synth
    nth = len(os.sched_getaffinity(0))
    used = oracle.threads_used(nth)
    B, L, H, P, N, G = s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups
    hpg = H // G

    def window_rate(x, dt, A, Bm, Cm, D, heads, threads, seqlens=None, min_s=3.0):
        g = max(heads // hpg, 1)
        sec, reps = _timed(lambda: oracle.ssd_scan(x[:, :, :heads], dt[:, :, :heads], A[:heads], Bm[:, :, :g],
                                                    Cm[:, :, :g], D[:heads], seqlens=seqlens, nthreads=threads),
                           min_s)
        return sec * (H / heads), reps

    # layer window: all cores on 32 heads, one thread on 2 heads
    per_win, reps = window_rate(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], 32, nth)
    per_win1, reps1 = window_rate(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], 2, 1, min_s=2.0)
    out = {"value": round(B * L / per_win, 1), "unit": "tokens/s", "cores": used, "kind": "oracle",
           "sample": f"32 of {H} heads of one L={L} layer window (fp64 sequential recurrence, OpenMP over heads), "
                     f"{reps} runs, scaled to all {H} heads",
           "cpu_model": cpu_model(),
           "single_thread": {"value": round(B * L / per_win1, 1), "unit": "tokens/s", "cores": 1,
                             "sample": f"2 of {H} heads, {reps1} runs, scaled to all {H} heads"}}
    # batched windows: the 1955-token partial window and one full window, 16 heads each
    sb = synth.batched_windows()
    sub = synth.window_inputs(synth.WindowShape(2, L, 16, P, N, 1, s.chunk), 1102)
    lens2 = [L, sb.seqlens[-1]]
    sec, reps = _timed(lambda: oracle.ssd_scan(sub["x"], sub["dt"], sub["A"], sub["B"], sub["C"], sub["D"],
                                               seqlens=lens2, nthreads=nth), 3.0)
    tok_s = sum(lens2) * 16 / H / sec
    out["batched"] = {"value": round(tok_s, 1), "unit": "tokens/s", "cores": used,
                      "sample": f"2 of 8 windows (2048 and 1955 tokens), 16 of {H} heads, {reps} runs, scaled"}
    # decode: 4 steps of 4 of 64 sequences on all cores; a 16-step prefix of one sequence on one thread
    d = synth.DECODE
    prm = synth.decode_params(1003, d["batch"], d["nheads"], d["headdim"], d["dstate"])
    steps = [synth.decode_step_inputs(1003, t, prm["dt0"], d["batch"], d["nheads"], d["headdim"], d["dstate"],
                                      d["ngroups"]) for t in range(16)]
    stk = {k: np.stack([st[k] for st in steps]) for k in ("x", "dt", "B", "C")}

    def dec(T, b_hi, threads):
        bits = prm["state"].astype(np.float16).view(np.uint16).copy()
        oracle.decode_f16state(stk["x"][:T], stk["dt"][:T], prm["A"], stk["B"][:T], stk["C"][:T], prm["D"], bits,
                               b_range=(0, b_hi), nthreads=threads)

    sec, reps = _timed(lambda: dec(4, 4, nth), 2.0)
    sec1, reps1 = _timed(lambda: dec(16, 1, 1), 2.0, max_reps=3)
    out["decode"] = {"us_per_step": round(sec / 4 * (d["batch"] / 4) * 1e6, 1), "cores": used,
                     "sample": f"4 steps of 4 of {d['batch']} sequences, {reps} runs, scaled to {d['batch']}",
                     "single_thread_us_per_step": round(sec1 / 16 * d["batch"] * 1e6, 1),
                     "single_thread_sample": f"16-step prefix of 1 of {d['batch']} sequences, {reps1} runs, scaled"}
    # mixer core: 512 tokens of one sequence, every head (conv, scan, norm)
    sm = synth.mixer_window()
    msub = synth.mixer_inputs(synth.WindowShape(1, 512, sm.nheads, P, sm.dstate, sm.ngroups, s.chunk), 1104)
    sec, reps = _timed(lambda: oracle.mixer_core(msub["xBC"], msub["conv_w"], msub["conv_b"], msub["dt"], msub["A"],
                                                 msub["D"], msub["z"], msub["norm_w"], sm.nheads, P, sm.ngroups,
                                                 sm.dstate, sm.nheads * P, nthreads=nth), 3.0)
    out["mixer"] = {"value": round(512 / sec, 1), "unit": "tokens/s", "cores": used,
                    "sample": f"512 tokens of one sequence, all {sm.nheads} heads, {reps} runs"}
    return out


def time_mixer(torch, m2, synth, dev, stream, P, Q, calls=20):
    """Microseconds per call of the mixer core (batch 4, L=2048: conv1d+SiLU,
    scan, gated RMSNorm), inputs drawn on the device."""
    # timing only (parity of this path is covered by the GPU tests); inputs are
    # drawn on the device with the mixer workload's distributions
    ms_ = synth.mixer_window()
    MB_, ML_, MH_, MN_, MG_ = ms_.batch, ms_.seqlen, ms_.nheads, ms_.dstate, ms_.ngroups
    Cd_ = MH_ * P + 2 * MG_ * MN_
    gen = torch.Generator(device=dev).manual_seed(1004)
    mx = {
        "xBC": torch.randn(MB_, ML_, Cd_, device=dev, generator=gen).half(),
        "conv_w": torch.randn(Cd_, 4, device=dev, generator=gen) * 0.5,
        "conv_b": torch.zeros(Cd_, device=dev),
        # dt as the layer window draws it: softplus(N(0,1) + log(expm1(dt0))),
        # dt0 log-uniform on [1e-3, 1e-1], one per head
        "dt": torch.nn.functional.softplus(
            torch.randn(MB_, ML_, MH_, device=dev, generator=gen)
            + torch.log(torch.expm1(torch.exp(torch.rand(MH_, device=dev, generator=gen) * float(np.log(100.0))
                                              + float(np.log(1e-3)))))).half(),
        "z": torch.randn(MB_, ML_, MH_ * P, device=dev, generator=gen).half(),
        "norm_w": torch.ones(MH_ * P, device=dev),
    }
    mA = -torch.exp(torch.rand(MH_, device=dev, generator=gen) * float(np.log(16.0)))
    mD = torch.randn(MH_, device=dev, generator=gen)
    my = torch.empty(MB_, ML_, MH_ * P, dtype=torch.float16, device=dev)
    mh = torch.empty(MB_, MH_, P, MN_, dtype=torch.float32, device=dev)
    mcs = torch.empty(MB_, Cd_, 3, dtype=torch.float16, device=dev)
    mdims = m2.make_dims(MB_, ML_, MH_, P, MN_, MG_, Q, conv_width=4, norm_group=MH_ * P)
    mws = m2.alloc_workspace(mdims, dev)

    def mstep():
        m2.conv_scan_window(mx["dt"], mA, mD, my, mws, xBC=mx["xBC"], conv_w=mx["conv_w"], conv_b=mx["conv_b"],
                            conv_state_out=mcs, state_out=mh, z=mx["z"], norm_w=mx["norm_w"], chunk=Q,
                            norm_group=MH_ * P, ngroups=MG_, dstate=MN_, headdim=P, stream=stream)

    for _ in range(3):
        mstep()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(calls):
        mstep()
    ev1.record(stream)
    torch.cuda.synchronize()
    mix_us = ev0.elapsed_time(ev1) * 1e3 / calls

    # the same calls without final states (scoring windows discard the scan
    # and conv states; the conv then writes no binary16 remainder of B)
    def mstep_ns():
        m2.conv_scan_window(mx["dt"], mA, mD, my, mws, xBC=mx["xBC"], conv_w=mx["conv_w"], conv_b=mx["conv_b"],
                            z=mx["z"], norm_w=mx["norm_w"], chunk=Q, norm_group=MH_ * P, ngroups=MG_, dstate=MN_,
                            headdim=P, stream=stream)

    for _ in range(3):
        mstep_ns()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(calls):
        mstep_ns()
    ev1.record(stream)
    torch.cuda.synchronize()
    mix_ns_us = ev0.elapsed_time(ev1) * 1e3 / calls
    if m2.window_take_error(mws, stream=stream) != 0:
        print("a segment hand-off gave up in the mixer calls: results invalid", file=sys.stderr)
        sys.exit(1)
    del mx, my, mh, mcs, mws
    torch.cuda.empty_cache()
    return mix_us, MB_, ML_, MH_, MN_, MG_, mix_ns_us


def time_batched(torch, m2, dev, stream, L, H, P, N, G, Q, calls=20):
    """Microseconds per call of the batched windows (8 sequences, seven of
    2048 tokens and one of 1955), inputs drawn on the device with the layer
    window's distributions; returns (us, lengths)."""
    # timing only (parity of this workload is covered by the GPU tests); inputs
    # are drawn on the device with the layer window's distributions
    BB, blens = 8, [L] * 7 + [1955]
    gen = torch.Generator(device=dev).manual_seed(1005)
    bsets = []
    for k in range(2):
        dt0 = torch.exp(torch.rand(H, device=dev, generator=gen) * float(np.log(100.0)) + float(np.log(1e-3)))
        bsets.append({
            "x": torch.randn(BB, L, H, P, device=dev, generator=gen).half(),
            "dt": torch.nn.functional.softplus(torch.randn(BB, L, H, device=dev, generator=gen)
                                               + torch.log(torch.expm1(dt0))).half(),
            "B": (torch.randn(BB, L, G, N, device=dev, generator=gen) / N ** 0.5).half(),
            "C": (torch.randn(BB, L, G, N, device=dev, generator=gen) / N ** 0.5).half(),
            "y": torch.empty(BB, L, H * P, dtype=torch.float16, device=dev),
            "hT": torch.empty(BB, H, P, N, dtype=torch.float32, device=dev),
        })
    bA = -torch.exp(torch.rand(H, device=dev, generator=gen) * float(np.log(16.0)))
    bD = torch.randn(H, device=dev, generator=gen)
    bsl = torch.tensor(blens, dtype=torch.int32, device=dev)
    bdims = m2.make_dims(BB, L, H, P, N, G, Q)
    bws = m2.alloc_workspace(bdims, dev)

    def bstep(k):
        t = bsets[k % len(bsets)]
        m2.conv_scan_window(t["dt"], bA, bD, t["y"], bws, x=t["x"], B=t["B"], C=t["C"], state_out=t["hT"],
                            seqlens=bsl, chunk=Q, stream=stream)

    for k in range(3):
        bstep(k)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for k in range(calls):
        bstep(k)
    ev1.record(stream)
    torch.cuda.synchronize()
    bat_us = ev0.elapsed_time(ev1) * 1e3 / calls
    if m2.window_take_error(bws, stream=stream) != 0:
        print("a segment hand-off gave up in the batched calls: results invalid", file=sys.stderr)
        sys.exit(1)
    del bsets, bws
    torch.cuda.empty_cache()
    return bat_us, blens


def time_short(torch, m2, dev, stream, H, P, N, G, Q, L=512, calls=50):
    """Microseconds per call of one short window at the layer shape (batch 1,
    L = 512, final state), inputs drawn on the device with the layer window's
    distributions and rotated over four sets (the short-window path)."""
    # timing only (parity of this shape is covered by the GPU tests)
    gen = torch.Generator(device=dev).manual_seed(1007)
    ssets = []
    for k in range(4):
        dt0 = torch.exp(torch.rand(H, device=dev, generator=gen) * float(np.log(100.0)) + float(np.log(1e-3)))
        ssets.append({
            "x": torch.randn(1, L, H, P, device=dev, generator=gen).half(),
            "dt": torch.nn.functional.softplus(torch.randn(1, L, H, device=dev, generator=gen)
                                               + torch.log(torch.expm1(dt0))).half(),
            "B": (torch.randn(1, L, G, N, device=dev, generator=gen) / N ** 0.5).half(),
            "C": (torch.randn(1, L, G, N, device=dev, generator=gen) / N ** 0.5).half(),
            "y": torch.empty(1, L, H * P, dtype=torch.float16, device=dev),
            "hT": torch.empty(1, H, P, N, dtype=torch.float32, device=dev),
        })
    sA = -torch.exp(torch.rand(H, device=dev, generator=gen) * float(np.log(16.0)))
    sD = torch.randn(H, device=dev, generator=gen)
    sws = m2.alloc_workspace(m2.make_dims(1, L, H, P, N, G, Q), dev)

    def sstep(k):
        t = ssets[k % len(ssets)]
        m2.conv_scan_window(t["dt"], sA, sD, t["y"], sws, x=t["x"], B=t["B"], C=t["C"], state_out=t["hT"],
                            chunk=Q, stream=stream)

    for k in range(5):
        sstep(k)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for k in range(calls):
        sstep(k)
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / calls
    del ssets, sws
    torch.cuda.empty_cache()
    return us, L


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sets", type=int, default=5, help="rotated input/output buffer sets")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the layer window and print its fields (for kernel traces of that workload)")
    ap.add_argument("--only", choices=["layer", "batched", "mixer", "short"], default=None,
                    help="time one workload alone (--steps calls after the warmup) and print its fields, for "
                         "kernel traces and counters of that workload; layer is the same as --headline-only")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the scan shards by sequence and by head group with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch

    import mamba_ssd_scan_amd as m2
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    s = synth.layer_window()
    B, L, H, P, N, G, Q = s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk
    if args.only == "layer":
        args.headline_only = True
    elif args.only == "batched":
        bus, blens = time_batched(torch, m2, dev, stream, L, H, P, N, G, Q, calls=args.steps)
        bb = window_bytes(8, L, H, P, N, G, lens=blens)
        print(json.dumps({"workload": "batched windows", "us": round(bus, 2), "calls": args.steps,
                          "algorithmic_bytes": bb, "achieved_GBs": round(bb / (bus * 1e-6) / 1e9, 1)}), flush=True)
        return
    elif args.only == "short":
        sus, SL_ = time_short(torch, m2, dev, stream, H, P, N, G, Q, calls=args.steps)
        sb = window_bytes(1, SL_, H, P, N, G)
        print(json.dumps({"workload": "short window", "us": round(sus, 2), "calls": args.steps,
                          "algorithmic_bytes": sb, "achieved_GBs": round(sb / (sus * 1e-6) / 1e9, 1)}), flush=True)
        return
    elif args.only == "mixer":
        mus, MB_, ML_, MH_, MN_, MG_, mus_ns = time_mixer(torch, m2, synth, dev, stream, P, Q, calls=args.steps)
        mb = mixer_bytes(MB_, ML_, MH_, P, MN_, MG_)
        print(json.dumps({"workload": "mixer core", "us": round(mus, 2), "us_no_final_state": round(mus_ns, 2),
                          "calls": args.steps,
                          "algorithmic_bytes": mb, "achieved_GBs": round(mb / (mus * 1e-6) / 1e9, 1)}), flush=True)
        return

    # ---- inputs resident in HBM, rotated sets ---------------------------------
    sets = []
    for k in range(args.sets):
        inp = synth.window_inputs(s, 1001 + 100 * k)
        t = {kk: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for kk, v in inp.items()}
        t["y"] = torch.empty((B, L, H * P), dtype=torch.float16, device=dev)
        t["hT"] = torch.empty((B, H, P, N), dtype=torch.float32, device=dev)
        t["np"] = inp if k == 0 else None
        sets.append(t)
    dims = m2.make_dims(B, L, H, P, N, G, Q)
    ws = m2.alloc_workspace(dims, dev)

    def step(k):
        t = sets[k % len(sets)]
        m2.conv_scan_window(t["dt"], t["A"], t["D"], t["y"], ws, x=t["x"], B=t["B"], C=t["C"], state_out=t["hT"],
                            chunk=Q, stream=stream)

    # one call on the first buffer set for the parity check, which runs on the
    # host; the warmup follows it, so that the timed calls do not start on a
    # GPU that idled through the check
    step(0)
    torch.cuda.synchronize()

    # ---- parity on the timed buffers (sampled heads, one per group) -----------
    import oracle
    t0 = sets[0]
    inp = t0["np"]
    y = t0["y"].cpu().numpy().reshape(B, L, H, P).astype(np.float64)
    hT = t0["hT"].cpu().numpy()
    heads = [g * (H // G) + (g * 5) % (H // G) for g in range(G)]
    worst_y = worst_s = 0.0
    for h in heads:
        g = h // (H // G)
        yr, hr = oracle.ssd_scan(inp["x"][:, :, h:h + 1], inp["dt"][:, :, h:h + 1], inp["A"][h:h + 1],
                                 inp["B"][:, :, g:g + 1], inp["C"][:, :, g:g + 1], inp["D"][h:h + 1])
        worst_y = max(worst_y, np.abs(y[:, :, h] - yr[:, :, 0]).max() / np.abs(yr).max())
        worst_s = max(worst_s, np.abs(hT[:, h] - hr[:, 0]).max() / np.abs(hr).max())
    if not (worst_y <= 2e-3 and worst_s <= 1e-3):
        print(f"parity check failed before timing: y {worst_y:.3e} state {worst_s:.3e}", file=sys.stderr)
        sys.exit(1)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # ---- timed region: K window calls ------------------------------------------
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for k in range(args.steps):
        step(k)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    tok_s = B * L / (ms * 1e-3)
    wbytes = window_bytes(B, L, H, P, N, G)
    achieved = wbytes / (ms * 1e-3) / 1e9

    # three more repeats of 50 back-to-back calls each, for the spread
    rep_us = []
    for r in range(3):
        torch.cuda.synchronize()
        ev0.record(stream)
        for k in range(50):
            step(k)
        ev1.record(stream)
        torch.cuda.synchronize()
        rep_us.append(ev0.elapsed_time(ev1) / 50 * 1e3)

    # the same calls without a final state (scoring windows discard it; the
    # segment hand-off then carries binary16 aggregates)
    def step_ns(k):
        t = sets[k % len(sets)]
        m2.conv_scan_window(t["dt"], t["A"], t["D"], t["y"], ws, x=t["x"], B=t["B"], C=t["C"], chunk=Q, stream=stream)

    for k in range(10):
        step_ns(k)
    ns_us = []
    for r in range(3):
        torch.cuda.synchronize()
        ev0.record(stream)
        for k in range(50):
            step_ns(k)
        ev1.record(stream)
        torch.cuda.synchronize()
        ns_us.append(ev0.elapsed_time(ev1) / 50 * 1e3)

    # single-call latency (one launch, synchronized)
    lat = []
    for k in range(20):
        torch.cuda.synchronize()
        ev0.record(stream)
        step(k)
        ev1.record(stream)
        torch.cuda.synchronize()
        lat.append(ev0.elapsed_time(ev1) * 1e3)
    lat_us = float(np.median(lat))
    if m2.window_take_error(ws, stream=stream) != 0:
        print("a segment hand-off gave up during the timed calls: results invalid", file=sys.stderr)
        sys.exit(1)
    copy_gbs = copy_bandwidth(torch, dev, stream)
    if args.headline_only:
        print(json.dumps({"metric": "SSD window-scan tokens/s at 8B layer shape L=2048", "value": round(tok_s, 1),
                          "unit": "tokens/s", "ms_per_step": round(ms, 6), "steps": args.steps,
                          "warmup": args.warmup, "window_us": round(ms * 1e3, 2),
                          "achieved_GBs": round(achieved, 1)}), flush=True)
        return

    # ---- the same window with the state requantized to binary16 every token ----
    # (the pages' scoring semantics; VALU-bound: per state element and token a
    # product, an fma, a binary16 rounding and an fma into y)
    def rqstep(k):
        t = sets[k % len(sets)]
        m2.requant_window(t["dt"], t["A"], t["D"], t["y"], x=t["x"], B=t["B"], C=t["C"], state_out=t["hT"],
                          stream=stream)

    for k in range(2):
        rqstep(k)
    torch.cuda.synchronize()
    ev0.record(stream)
    for k in range(10):
        rqstep(k)
    ev1.record(stream)
    torch.cuda.synchronize()
    rq_us = ev0.elapsed_time(ev1) * 1e3 / 10
    rq_updates = B * L * H * P * N

    # ---- backward pass of the layer window scan ------------------------------------
    gdims = m2.make_dims(B, L, H, P, N, G, Q)
    gws = m2.alloc_scan_grad_workspace(gdims, dev)
    ggen = torch.Generator(device=dev).manual_seed(1007)
    gdy = torch.randn(B, L, H, P, device=dev, generator=ggen).half()
    gdhT = torch.randn(B, H, P, N, device=dev, generator=ggen) * 0.3
    f32 = dict(dtype=torch.float32, device=dev)
    gout = dict(dx=torch.empty(B, L, H, P, **f32), ddt=torch.empty(B, L, H, **f32),
                dB=torch.empty(B, L, G, N, **f32), dC=torch.empty(B, L, G, N, **f32), dA=torch.empty(H, **f32),
                dD=torch.empty(H, **f32), dstate_in=torch.empty(B, H, P, N, **f32))

    def gstep(k):
        t = sets[k % len(sets)]
        m2.scan_grad(t["dt"], t["A"], t["D"], gdy, gws, x=t["x"], B=t["B"], C=t["C"], dstate_out=gdhT,
                     stream=stream, **gout)

    for k in range(2):
        gstep(k)
    torch.cuda.synchronize()
    ev0.record(stream)
    for k in range(5):
        gstep(k)
    ev1.record(stream)
    torch.cuda.synchronize()
    grad_us = ev0.elapsed_time(ev1) * 1e3 / 5
    # two sweeps, four lane-operations per state element and token in each
    grad_ops = 8 * B * L * H * P * N
    del gws, gdy, gdhT, gout
    del sets
    torch.cuda.empty_cache()

    mix_us, MB_, ML_, MH_, MN_, MG_, mix_ns_us = time_mixer(torch, m2, synth, dev, stream, P, Q)
    mbytes = mixer_bytes(MB_, ML_, MH_, P, MN_, MG_)

    # ---- decode: 64 sequences, binary16 resident state ------------------------
    d = synth.DECODE
    DB, DH, DP, DN, DG, T = d["batch"], d["nheads"], d["headdim"], d["dstate"], d["ngroups"], args.decode_steps
    prm = synth.decode_params(1003, DB, DH, DP, DN)
    nin = 8
    steps_in = []
    for k in range(nin):
        si = synth.decode_step_inputs(1003, k, prm["dt0"], DB, DH, DP, DN, DG)
        steps_in.append({kk: torch.from_numpy(v).to(dev) for kk, v in si.items()})
    A, Dd = torch.from_numpy(prm["A"]).to(dev), torch.from_numpy(prm["D"]).to(dev)
    nstate = 3
    states = [torch.empty((DB, DH, DP, DN), dtype=torch.float16, device=dev) for _ in range(nstate)]
    seed32 = torch.from_numpy(prm["state"]).to(dev)
    for st_ in states:
        m2.state_load(seed32, st_, stream=stream)
    ydec = torch.empty((DB, DH, DP), dtype=torch.float16, device=dev)

    def dstep(k, st_):
        si = steps_in[k % nin]
        m2.decode_step(si["x"], si["dt"], si["B"], si["C"], A, Dd, st_, ydec, stream=stream)

    for k in range(10):
        dstep(k, states[0])
    torch.cuda.synchronize()
    # as written: one resident state, T consecutive steps
    ev0.record(stream)
    for k in range(T):
        dstep(k, states[0])
    ev1.record(stream)
    torch.cuda.synchronize()
    dec_us = ev0.elapsed_time(ev1) * 1e3 / T
    # rotated: three resident states (384 MiB > Infinity Cache)
    ev0.record(stream)
    for k in range(T):
        dstep(k, states[k % nstate])
    ev1.record(stream)
    torch.cuda.synchronize()
    dec_rot_us = ev0.elapsed_time(ev1) * 1e3 / T
    dbytes = decode_bytes(DB, DH, DP, DN, DG)

    # ---- fused mixer step: conv history + SiLU + step + gated RMSNorm ---------
    DCd = DH * DP + 2 * DG * DN
    mgen = torch.Generator(device=dev).manual_seed(1006)
    md_in = [{"xBC": torch.randn(DB, DCd, device=dev, generator=mgen).half(),
              "z": torch.randn(DB, DH * DP, device=dev, generator=mgen).half()} for _ in range(nin)]
    md_w = (torch.randn(DCd, 4, device=dev, generator=mgen) * 0.5).contiguous()
    md_b = torch.zeros(DCd, device=dev)
    md_cs = torch.randn(DB, DCd, 3, device=dev, generator=mgen).half()
    md_nw = torch.ones(DH * DP, device=dev)
    md_dims = m2.mixer_decode_dims(DB, DH, DP, DN, DG, DH * DP, m2.F16, m2.F16)
    md_ws = m2.alloc_mixer_decode_workspace(md_dims, dev)
    md_y = torch.empty(DB, DH * DP, dtype=torch.float16, device=dev)

    def mdstep(k, st_):
        si, mi = steps_in[k % nin], md_in[k % nin]
        m2.mixer_decode_step(mi["xBC"], md_w, md_cs, si["dt"], A, Dd, st_, md_y, md_ws, conv_b=md_b, z=mi["z"],
                             norm_w=md_nw, ngroups=DG, dstate=DN, norm_group=DH * DP, stream=stream)

    for k in range(10):
        mdstep(k, states[0])
    torch.cuda.synchronize()
    ev0.record(stream)
    for k in range(T):
        mdstep(k, states[k % nstate])
    ev1.record(stream)
    torch.cuda.synchronize()
    md_us = ev0.elapsed_time(ev1) * 1e3 / T
    mdbytes = mixer_decode_bytes(DB, DH, DP, DN, DG)

    bat_us, blens = time_batched(torch, m2, dev, stream, L, H, P, N, G, Q)
    bbytes = window_bytes(8, L, H, P, N, G, lens=blens)
    sh_us, SL_ = time_short(torch, m2, dev, stream, H, P, N, G, Q)
    shbytes = window_bytes(1, SL_, H, P, N, G)

    # ---- CPU baseline: the oracle on bounded samples of each workload ----------
    cpu = cpu_baselines(inp, s, args) if not args.no_cpu_baseline else None

    mflops = window_mfma_flops(L, H, P, N, Q)
    out = {
        "metric": "SSD window-scan tokens/s at 8B layer shape L=2048 + decode us/step; % HBM roofline",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "mamba2-8b layer window scan", "batch": B, "seq_len": L, "nheads": H,
                   "headdim": P, "dstate": N, "ngroups": G, "chunk": Q, "io": "f16", "state": "f32",
                   "buffer_sets": args.sets},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic()},
        "cpu_baseline": cpu,
        "copy_GBs": round(copy_gbs, 1),
        "frac_of_copy": round(achieved / copy_gbs, 4),
        "meta": run_metadata(torch, m2),
        "window_us": round(ms * 1e3, 2),
        "window_latency_us": round(lat_us, 2),
        "window_repeats_us": {"median": round(float(np.median(rep_us)), 2), "min": round(float(np.min(rep_us)), 2),
                              "sd": round(float(np.std(rep_us)), 2), "repeats": len(rep_us), "calls_each": 50},
        "window_no_final_state_us": {"median": round(float(np.median(ns_us)), 2), "min": round(float(np.min(ns_us)), 2),
                                     "calls_each": 50, "algorithmic_bytes": wbytes - B * H * P * N * 4},
        "window_algorithmic_bytes": wbytes,
        "window_mfma_tflops": round(mflops / (ms * 1e-3) / 1e12, 1),
        "window_mfma_frac": round(mflops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK, 4),
        "parity": {"y": float(f"{worst_y:.3e}"), "state": float(f"{worst_s:.3e}")},
        "mixer": {"workload": "conv1d(4)+SiLU, scan, gated RMSNorm over 8192 channels", "batch": MB_,
                  "seq_len": ML_, "us": round(mix_us, 2), "tokens_per_s": round(MB_ * ML_ / (mix_us * 1e-6), 1),
                  "algorithmic_bytes": mbytes, "achieved_GBs": round(mbytes / (mix_us * 1e-6) / 1e9, 1),
                  "frac": round(mbytes / (mix_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  "us_no_final_state": round(mix_ns_us, 2)},
        "batched": {"workload": "8 layer windows, 7 x 2048 + 1955 tokens, final states", "us": round(bat_us, 2),
                    "tokens_per_s": round(sum(blens) / (bat_us * 1e-6), 1), "algorithmic_bytes": bbytes,
                    "achieved_GBs": round(bbytes / (bat_us * 1e-6) / 1e9, 1),
                    "frac": round(bbytes / (bat_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "short_window": {"workload": "one window of 512 tokens at the layer shape, final state (column scan)",
                         "us": round(sh_us, 2), "tokens_per_s": round(SL_ / (sh_us * 1e-6), 1),
                         "algorithmic_bytes": shbytes, "achieved_GBs": round(shbytes / (sh_us * 1e-6) / 1e9, 1),
                         "frac": round(shbytes / (sh_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "requant_window": {"workload": "layer window, state requantized to binary16 after every token",
                           "us": round(rq_us, 2), "tokens_per_s": round(B * L / (rq_us * 1e-6), 1),
                           "state_updates_per_s": round(rq_updates / (rq_us * 1e-6), 1),
                           "roofline": {"bound": "alu", "ops_per_update": 4,
                                        "achieved": round(4 * rq_updates / (rq_us * 1e-6) / 1e12, 2),
                                        "peak": VALU_PEAK_TOPS, "unit": "T lane-ops/s",
                                        "frac": round(4 * rq_updates / (rq_us * 1e-6) / 1e12 / VALU_PEAK_TOPS, 4)}},
        "scan_grad": {"workload": "backward of the layer window scan: dx, ddt, dB, dC, dA, dD, dstate_in",
                      "us": round(grad_us, 2), "tokens_per_s": round(B * L / (grad_us * 1e-6), 1),
                      "roofline": {"bound": "alu", "ops_per_update": 8,
                                   "achieved": round(grad_ops / (grad_us * 1e-6) / 1e12, 2),
                                   "peak": VALU_PEAK_TOPS, "unit": "T lane-ops/s",
                                   "frac": round(grad_ops / (grad_us * 1e-6) / 1e12 / VALU_PEAK_TOPS, 4)}},
        "decode": {"us_per_step": round(dec_us, 2), "us_per_step_rotated_states": round(dec_rot_us, 2),
                   "algorithmic_bytes": dbytes, "achieved_GBs": round(dbytes / (dec_rot_us * 1e-6) / 1e9, 1),
                   "frac": round(dbytes / (dec_rot_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "batch": DB, "steps": T, "state": "f16"},
        "mixer_decode": {"workload": "one token of the full mixer: conv history + SiLU, step, gated RMSNorm "
                                     "over 8192 channels", "us_per_step_rotated_states": round(md_us, 2),
                         "algorithmic_bytes": mdbytes, "achieved_GBs": round(mdbytes / (md_us * 1e-6) / 1e9, 1),
                         "frac": round(mdbytes / (md_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "batch": DB, "steps": T, "state": "f16"},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

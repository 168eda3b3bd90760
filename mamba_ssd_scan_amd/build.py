"""Builds the gfx950 HIP library libmamba2ssd.so in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmamba2ssd.so")
SOURCES = ["abi.hip", "colscan.hip", "decode.hip", "grad.hip", "mixer_decode.hip", "requant.hip", "ssd_scan.hip", "window.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc, *FLAGS, "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to build libmamba2ssd.so")
    os.replace(tmp, LIB)
    write_build_info()
    return LIB


def write_build_info() -> None:
    """Record, beside the library, which tree it was built from (the git
    commit when there is one, whether tracked files differed from it, and a
    hash of the sources), for the benchmark's metadata."""
    import hashlib
    import json
    root = os.path.dirname(HERE)
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(root, "include", "mamba2ssd.h"), "rb") as f:
        h.update(f.read())
    info = {"source_sha256_16": h.hexdigest()[:16], "git_sha": None, "git_dirty": None}
    try:
        sha = subprocess.run(["git", "rev-parse", "HEAD"], cwd=root, capture_output=True, text=True)
        if sha.returncode == 0:
            info["git_sha"] = sha.stdout.strip()
            st = subprocess.run(["git", "status", "--porcelain", "--untracked-files=no"], cwd=root,
                                capture_output=True, text=True)
            info["git_dirty"] = bool(st.stdout.strip()) if st.returncode == 0 else None
    except OSError:
        pass
    with open(os.path.join(HERE, "build_info.json"), "w") as f:
        json.dump(info, f)


if __name__ == "__main__":
    print(build(verbose=True))

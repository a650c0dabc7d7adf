"""Build libfa355.so in-tree with hipcc for gfx950.

    python -m exact_io_aware_65_amd.build

Each source compiles to its own object (in parallel) under _build/, then the
objects link into exact_io_aware_65_amd/libfa355.so.  The streaming-read probe
that bench.py reports decode against (probe/read_bw.hip) and the LDS bank probe
(probe/lds_banks.hip, bench.py --lds-probe) build into their own library,
exact_io_aware_65_amd/libfa355_probe.so.

    python -m exact_io_aware_65_amd.build --poison-lds

builds the debug variant libfa355_poison_lds.so instead: every kernel fills
its LDS with NaN words before first use, so reads of LDS never written show up
as NaN outputs.  Select it for a test run with FA355_LIBRARY=<path>.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libfa355.so")
BUILD_INFO = os.path.join(PKG, "build_info.json")
PROBE_SOURCES = [os.path.join(PKG, "probe", "read_bw.hip"), os.path.join(PKG, "probe", "lds_banks.hip")]
PROBE_LIBRARY = os.path.join(PKG, "libfa355_probe.so")
POISON_LIBRARY = os.path.join(PKG, "libfa355_poison_lds.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["fa_fwd.hip", "fa_decode.hip", "fa_bwd.hip", "fa_fp8.hip", "fa_abi.cpp"]

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # keep hipcc from forming packed fp32 arithmetic on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _compile(src: str, verbose: bool, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build_poison_lds(verbose: bool = False) -> str:
    """The debug variant of the library with LDS poisoned before use."""
    out_dir = os.path.join(BUILD, "poison_lds")
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, out_dir, ("-DFA355_POISON_LDS",)), SOURCES))
    tmp = POISON_LIBRARY + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, POISON_LIBRARY)
    return POISON_LIBRARY


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES) + len(PROBE_SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + PROBE_SOURCES))
    n = len(SOURCES)
    for lib, parts in ((LIBRARY, objs[:n]), (PROBE_LIBRARY, objs[n:])):
        tmp = lib + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *parts, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    _write_build_info()
    return LIBRARY


def _write_build_info() -> None:
    """Record which sources the libraries were built from (git commit, and whether
    the tree had uncommitted changes) beside them, for the benchmark's record."""
    def git(*args):
        try:
            r = subprocess.run(["git", "-C", ROOT, *args], capture_output=True, text=True, timeout=20)
            return r.stdout.strip() if r.returncode == 0 else None
        except (OSError, subprocess.SubprocessError):
            return None
    status = git("status", "--porcelain", "--untracked-files=no")
    info = {"git_commit": git("rev-parse", "HEAD"), "git_dirty": None if status is None else bool(status),
            "built_utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime()), "arch": ARCH}
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f)


if __name__ == "__main__":
    if "--poison-lds" in sys.argv:
        print(build_poison_lds(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))

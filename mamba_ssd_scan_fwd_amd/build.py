"""Build libssd.so (C ABI + HIP kernels for gfx950) in-tree with hipcc.

Usage: python -m mamba_ssd_scan_fwd_amd.build [-j JOBS] [--verbose]

Every source under csrc/ is compiled to an object in ``_build/`` (in
parallel), then linked into ``mamba_ssd_scan_fwd_amd/libssd.so``. The build
always recompiles; it never needs a GPU (hipcc cross-compiles for gfx950).

``--host-sanitize`` builds a second copy, ``_build/libssd_host_san.so``, whose
host code (argument validation, planning, launch set-up) is instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer; the device code is built as
usual. It serves the host-side ABI tests, which reach no kernel:

    python -m mamba_ssd_scan_fwd_amd.build --host-sanitize
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
      LD_PRELOAD=$(hipcc --print-file-name=libclang_rt.asan-x86_64.so) \
      SSD_LIB=mamba_ssd_scan_fwd_amd/_build/libssd_host_san.so \
      python -m pytest tests/test_abi_host.py -q
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libssd.so")
ARCH = "gfx950"

COMMON = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: a ROCm installation is required to build libssd.so")


def sources():
    out = []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hip") or f.endswith(".cpp"):
            out.append(os.path.join(CSRC, f))
    return out


# host-only instrumentation (each flag applies to the host compilation only)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_BUILD = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(BUILD, "libssd_host_san.so")


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_BUILD if sanitize else BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *(HOST_SAN if sanitize else []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = False, host_sanitize: bool = False) -> str:
    os.makedirs(SAN_BUILD if host_sanitize else BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(os.cpu_count() or 1, 16)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, host_sanitize), srcs))
    out = SAN_LIB if host_sanitize else LIB
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *(HOST_SAN if host_sanitize else []), "-o", tmp,
           *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", "--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--host-sanitize", action="store_true",
                    help="build _build/libssd_host_san.so with ASan/UBSan host instrumentation instead")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose, a.host_sanitize))


if __name__ == "__main__":
    main()

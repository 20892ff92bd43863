"""Build libmoe_layer.so in-tree with hipcc for gfx950.

Usage: python -m moe_ffn_amd.build [--jobs N]

Every source under csrc/ is compiled to an object in _build/ (in parallel),
then linked into moe_ffn_amd/libmoe_layer.so.  The library is always rebuilt.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe_layer.so")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build the library")
    return p


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *CFLAGS, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


# The host code with AddressSanitizer (every -fsanitize behind -Xarch_host:
# the device code is built as usual, without it): the library's sources and a
# C++ driver of the ABI's validation and error paths
# (tests/asan/abi_host_check.cpp) linked into one executable.
ASAN_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
              "-Wno-unused-command-line-argument",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build_host_asan(out_dir: str | None = None, jobs: int | None = None) -> str:
    out_dir = out_dir or os.path.join(BUILD, "host_asan")
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources() + [os.path.join(ROOT, "tests", "asan", "abi_host_check.cpp")]

    def one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        r = subprocess.run([_hipcc(), *ASAN_FLAGS, "-x", "hip", "-c", src, "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"host ASan compile failed: {src}\n{r.stdout}{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs or min(len(srcs), os.cpu_count() or 4, 16)) as ex:
        objs = list(ex.map(one, srcs))
    exe = os.path.join(out_dir, "abi_host_check")
    r = subprocess.run([_hipcc(), "--offload-arch=" + ARCH, "-Xarch_host", "-fsanitize=address",
                        "-o", exe, *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("host ASan link failed:\n" + r.stdout + r.stderr)
    return exe


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    build(ap.parse_args().jobs)

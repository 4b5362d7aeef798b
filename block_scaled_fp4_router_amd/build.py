"""Builds libftmoe.so (all HIP sources under csrc/) for gfx950 with hipcc.

    python -m block_scaled_fp4_router_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libftmoe.so")
ARCH = "gfx950"

# Packed-fp32 instructions are disabled for every HIP translation unit: the
# compiler forms them from ordinary float code, and this code base does not
# rely on them.
HIPFLAGS = [
    "-O3", "-std=c++20", f"--offload-arch={ARCH}", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-I", os.path.join(ROOT, "include"),
]


# Device-side code generation flags every HIP translation unit needs.
HIPFLAGS_DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics"]

# Host-only C++ (the host half of CPU-GPU co-execution): built by the host
# compiler; functions that need AVX2/FMA carry their own target attribute.
CXXFLAGS = ["-O3", "-std=c++20", "-fPIC", "-Wall", "-pthread", "-I", os.path.join(ROOT, "include")]


def cxx() -> str:
    for c in (os.environ.get("CXX"), shutil.which("g++"), "/opt/rocm/llvm/bin/clang++"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("no host C++ compiler found")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ftmoe library needs ROCm's hipcc to build")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):
        cmd = [cxx(), *CXXFLAGS, "-c", src, "-o", obj]
    else:
        cmd = [hipcc(), *HIPFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiler failed on {src}:\n{r.stderr}")
    return obj


def _check_resolved(lib: str) -> None:
    """A kernel whose host stub the compiler dropped shows up as an undefined
    ftmoe symbol: refuse such a library instead of failing at load time."""
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    r = subprocess.run([nm, "-u", "-C", lib], capture_output=True, text=True)
    bad = [ln.strip() for ln in r.stdout.splitlines() if "ftmoe::" in ln]
    if bad:
        raise RuntimeError("libftmoe.so has unresolved ftmoe symbols:\n" + "\n".join(bad[:20]))


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    _check_resolved(tmp)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


# Sanitizer builds of the host code (not the GPU kernels): every HIP source
# compiled for the host only, the host C++ and the check program in
# tests/host_check.cpp, each instrumented, linked into one executable that
# runs without a GPU.  "address" is AddressSanitizer with
# UndefinedBehaviorSanitizer, "thread" ThreadSanitizer.
SANITIZERS = {"address": ["address", "undefined"], "thread": ["thread"]}


def host_clang() -> str:
    for c in (os.environ.get("FTMOE_HOST_CLANG"), "/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("no clang++ found for the sanitizer build")


def build_host_check(kind: str, jobs: int | None = None) -> str:
    """Builds _build/san-<kind>/host_check; returns its path."""
    out = os.path.join(BUILD, f"san-{kind}")
    os.makedirs(out, exist_ok=True)
    san = [f"-fsanitize={x}" for x in SANITIZERS[kind]]
    common = ["-O1", "-g", "-std=c++20", "-fPIC", "-fno-omit-frame-pointer", "-pthread", "-I", os.path.join(ROOT, "include")]
    host_san = [f for x in san for f in ("-Xarch_host", x)]   # each sanitizer flag for the host compilation only
    check = os.path.join(ROOT, "tests", "host_check.cpp")

    def one(src: str) -> str:
        obj = os.path.join(out, os.path.basename(src) + ".o")
        if src.endswith(".hip"):
            cmd = [hipcc(), *common, f"--offload-arch={ARCH}", *HIPFLAGS_DEVICE, *host_san, "-c", src, "-o", obj]
        else:
            cmd = [host_clang(), *common, *san, "-I", CSRC, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compiler failed on {src}:\n{r.stderr}")
        return obj

    srcs = sources() + [check]
    with ThreadPoolExecutor(jobs or min(len(srcs), 8)) as ex:
        objs = list(ex.map(one, srcs))
    exe = os.path.join(out, "host_check")
    cmd = [hipcc(), f"--offload-arch={ARCH}", *host_san, "-pthread", *objs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return exe


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--sanitize", choices=sorted(SANITIZERS), default=None,
                    help="build the host-code check program under a sanitizer instead of the library")
    a = ap.parse_args()
    if a.sanitize:
        print(build_host_check(a.sanitize, a.jobs))
    else:
        build(a.jobs, verbose=True)

"""Build libmoe_hip.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m routed_expert_ffn_05_amd.build [--jobs N]

Every HIP source is compiled to an object of its own (in parallel) and linked into
``routed_expert_ffn_05_amd/libmoe_hip.so``.  hipcc cross-compiles: no GPU is needed.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_hip.so")
ARCH = "gfx950"

SOURCES = ["moe_abi.cpp", "router.hip", "permute.hip", "gemv_dispatch.cpp", "gemv_f32.hip", "gemv_bf16.hip",
           "gemv_fp8.hip", "gemv_mxfp4.hip", "gemm.hip", "combine.hip", "actq.hip", "plan.hip"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 (v_pk_*_f32) code generation in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, src + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc(), *lang, *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = False, extra=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every source and link ``out``; ``extra`` adds compiler flags (e.g. -D tuning
    constants for an experimental build written elsewhere)."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


# The host-side argument checking and workspace carving of the C ABI (moe_abi.cpp) built with the
# address and undefined-behaviour sanitizers on its host code only, linked with the ordinary
# objects of every other source into a second library for the CPU tests.  Loading it needs the
# sanitizer runtime preloaded (sanitizer_runtime()).
SAN_LIB = os.path.join(PKG, "libmoe_hip_san.so")
SAN_FLAGS = ["-g", "-O1", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """The clang address-sanitizer runtime (it carries the undefined-behaviour runtime too)."""
    import glob
    cands = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/lib/llvm")
    return cands[-1]


def build_sanitized_abi(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    san_dir = os.path.join(BUILD, "san")
    os.makedirs(san_dir, exist_ok=True)
    others = [src for src in SOURCES if src != "moe_abi.cpp"]
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(lambda s_: _compile(s_, BUILD), others))
    objs.append(_compile("moe_abi.cpp", san_dir, SAN_FLAGS))
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--sanitized-abi", action="store_true", help="also build libmoe_hip_san.so")
    a = ap.parse_args(argv)
    build(a.jobs, verbose=True)
    if a.sanitized_abi:
        build_sanitized_abi(a.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

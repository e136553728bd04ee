"""Build libmoe.so: the gfx950 kernels and the C ABI of include/moe.h.

    python -m mixture_experts_layer_logit_amd.build

Compiles every source under csrc/ with hipcc for gfx950 (in parallel) and
links them into csrc/../libmoe.so inside the package directory.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["route.hip", "permute.hip", "grouped_gemm.hip", "combine.hip", "quant.hip", "backward.hip", "api.cpp"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip())
    if warn:
        print(f"[{src}]\n{warn}", file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_host_sanitized(out: str) -> str:
    """A copy of libmoe.so whose host code (api.cpp: argument checks,
    workspace layouts, launch set-up) carries AddressSanitizer and
    UndefinedBehaviorSanitizer checks; device code is not instrumented.  The
    kernels' objects come from the last build().  Load it with clang's ASan
    runtime preloaded (LD_PRELOAD) and MOE_LIB=<out>."""
    objs = [os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o") for src in SOURCES if src != "api.cpp"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise FileNotFoundError(f"run build() first: {missing}")
    # each sanitizer flag applies to the host compilation only
    san = []
    for check in ("address", "undefined"):
        san += ["-Xarch_host", "-fsanitize=" + check]
    san += ["-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_obj = out + ".api.o"
    flags = [f for f in COMMON if f != "-O3"] + ["-O1", "-g"]
    cmd = [HIPCC, "-x", "hip", "-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj] + flags + san
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on api.cpp (sanitized):\n{r.stdout}\n{r.stderr}")
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-shared-libsan"] + san + ["-o", out] + objs + [api_obj]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.remove(api_obj)
    return out


def asan_runtime() -> str:
    """Path of the ASan runtime that build_host_sanitized() links against."""
    r = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang++"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


if __name__ == "__main__":
    build()

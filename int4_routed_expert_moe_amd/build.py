"""Build libmoe_int4.so (hand-written HIP for gfx950) in-tree with hipcc.

Usage: python -m int4_routed_expert_moe_amd.build   (or call build()).
Every HIP source is compiled with contraction off (the router and the exact
mode are specified operation by operation) and without packed-fp32 code
generation.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoe_int4.so")
# the benchmark's HBM read and matrix-core rate probes: their own library, outside the layer's C ABI
PROBE_SOURCES = ["hbm_probe.hip", "mfma_probe.hip"]
PROBE_OUT = os.path.join(HERE, "libmoe_probe.so")
OBJDIR = os.path.join(ROOT, "_build")

SOURCES = ["status.cpp", "route.hip", "permute.hip", "grouped_gemm.hip", "combine.hip", "dense.hip",
           "group_sums.hip", "exact_linear.hip"]

ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


# host-side sanitizers for the argument checks (the device code is built as usual)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, objdir: str = OBJDIR, extra=()) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out, extra=()):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    """Compile every source for gfx950 and link libmoe_int4.so and the benchmark's
    probe library libmoe_probe.so (always rebuilds)."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], PROBE_OUT)
    if verbose:
        print(f"built {OUT} and {PROBE_OUT}")
    return OUT


def build_sanitized(verbose: bool = True) -> str:
    """libmoe_int4_san.so: the same sources with the host code under AddressSanitizer and
    UndefinedBehaviorSanitizer, for the CPU-side argument checks (load it with clang's
    ASan runtime preloaded; no GPU is needed for the checks)."""
    objdir = os.path.join(OBJDIR, "san")
    os.makedirs(objdir, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, objdir, SAN_FLAGS), SOURCES))
    out = os.path.join(HERE, "libmoe_int4_san.so")
    _link(objs, out, ["-fsanitize=address,undefined"])
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build_sanitized() if "--sanitize" in sys.argv else build()
    sys.exit(0)

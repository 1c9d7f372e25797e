"""Build libfgb.so (the HIP library behind include/fgb.h) in-tree for gfx950.

Usage: ``python -m fine_grained_block_amd.build`` or ``build_library()``.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfgb.so")
SOURCES = ["abi.hip", "quant.hip", "gemm.hip", "swiglu.hip"]
# the benchmark's clock probe: a library of its own, not linked into libfgb.so
PROBE_LIB = os.path.join(PKG, "libfgb_probe.so")
PROBE_SOURCES = ["probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 anywhere.  Denormals are kept
# (IEEE fp32), no FMA contraction except where the code asks for fmaf.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Sources whose kernels must not use scratch memory: a spilled register in the
# GEMM main loop is reloaded with a vector-memory load whose wait also drains
# the in-flight direct-to-LDS prefetch, so a spill is a build error there.
NO_SCRATCH = {"gemm.hip"}


def _scratch_users(remarks: str) -> list:
    """Kernels with a non-zero ScratchSize in hipcc's resource-usage remarks."""
    users, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            users.append((name, int(m.group(1))))
    return users


def _compile(src: str, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    extra = ["-Rpass-analysis=kernel-resource-usage"] if src in NO_SCRATCH else []
    cmd = [HIPCC, *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if src in NO_SCRATCH:
        bad = _scratch_users(r.stderr)
        if bad:
            os.remove(obj)
            raise RuntimeError(f"{src}: kernels use scratch memory (register spills): {bad}")
    return obj


def _link(objs, out: str):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build_library(verbose: bool = False) -> str:
    """Build libfgb.so and the benchmark's libfgb_probe.so; returns libfgb.so's path."""
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, build_dir), srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)

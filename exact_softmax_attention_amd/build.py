"""Build libattn.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m exact_softmax_attention_amd.build

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")

SOURCES = ["api.cpp", "fwd_bf16.hip", "fwd_f32.hip", "decode_paged.hip", "bwd_bf16.hip", "merge.hip"]
# The decode kernel multiplies its matrix-core accumulators by the softmax
# rescale factor on the vector ALUs every block; keeping them in ordinary
# VGPRs (rather than AGPRs) avoids copying them back and forth.
EXTRA_FLAGS = {"decode_paged.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
        "-Wno-unused-command-line-argument",
    ]


_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]):\s+(\S+)")


def _resources(stderr: str):
    """Per-kernel resource usage from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for key, val in _REMARK.findall(stderr):
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" ")[0]] = int(val)
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + EXTRA_FLAGS.get(src, []) + ["-Rpass-analysis=kernel-resource-usage",
                                        "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        errs = "\n".join(ln for ln in res.stderr.splitlines() if "remark:" not in ln)
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}{errs}")
    usage = _resources(res.stderr)
    # A kernel that spills or keeps arrays in scratch memory is a build error:
    # it is always a performance bug in these kernels.
    bad = {k: v for k, v in usage.items() if v.get("ScratchSize", 0) > 0}
    if bad:
        raise RuntimeError(f"{src}: kernels use scratch memory: {bad}")
    return obj, usage


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        for _, usage in results:
            for name, u in sorted(usage.items()):
                f.write(f"{name}: {u}\n")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_read_ceiling()
    return LIB


# The decode's read-bandwidth ceiling probe: a program of its own (not part of
# the library), run by `bench.py --mode ceiling`.
CEILING_SRC = os.path.join(CSRC, "read_ceiling.hip")
CEILING_BIN = os.path.join(PKG, "read_ceiling")


def build_read_ceiling() -> str:
    tmp = CEILING_BIN + ".tmp"
    cmd = [hipcc()] + common_flags() + ["-o", tmp, CEILING_SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling read_ceiling failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, CEILING_BIN)
    return CEILING_BIN


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

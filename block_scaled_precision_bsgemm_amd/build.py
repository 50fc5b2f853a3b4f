"""Build the HIP library ``libbsgemm.so`` in-tree with hipcc for gfx950.

Usage: ``python -m block_scaled_precision_bsgemm_amd.build`` (or ``build()``).
Every source is compiled for gfx950 only, with packed-FP32 instruction
generation disabled; the quantizers are also compiled without FP contraction
(``-ffp-contract=off``) so that their FP32 steps round exactly as written.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbsgemm.so")

SOURCES = ["api.cpp", "quantize.hip", "gemm_mx.hip", "gemm_mx8_exact.hip", "gemm_nvfp4.hip", "grouped.hip",
           "w4a16.hip", "w4a16_tile.hip"]
COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I" + INCLUDE, "-I" + CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
EXTRA_FLAGS = {"quantize.hip": ["-ffp-contract=off"]}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src):
    out = os.path.join(OBJDIR, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [_hipcc()] + COMMON_FLAGS + EXTRA_FLAGS.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    return out, msgs


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libbsgemm.so``; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for (_, msgs), src in zip(results, SOURCES):
        if msgs.strip() and verbose:
            print(f"[{src}]\n{msgs}")
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

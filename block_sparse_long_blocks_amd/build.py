"""Build libfp2.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python block_sparse_long_blocks_amd/build.py [--debug]   (from the repository root; running it as a
module would import the package, which needs the library first)
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp2.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["fp2_api.cpp", "fp2_validate.cpp", "block_stats.hip", "plan_mask.hip", "prefill_attn.hip",
           "attn_d128.hip"]

COMMON = ["-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{ROOT}/include", f"-I{CSRC}"]
# gfx950 device code; packed-fp32 instructions are disabled on purpose.
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The bf16 attention kernel never produces a NaN (padding is staged as zeros,
# masks are -inf), so its max reductions need no NaN quieting.
EXTRA = {"attn_d128.hip": ["-fno-honor-nans"]}


def _compile(src, opt):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, *EXTRA.get(src, []), opt, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]


def build(debug: bool = False, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    opt = "-O1" if debug else "-O3"
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, opt), SOURCES))
    for _, warn in results:
        if verbose and warn:
            print("\n".join(warn), file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(debug="--debug" in sys.argv))

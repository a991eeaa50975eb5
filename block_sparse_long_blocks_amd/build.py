"""Build libfp2.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python block_sparse_long_blocks_amd/build.py [--debug] [--debug-bounds]   (from the repository root;
running it as a module would import the package, which needs the library first)

--debug-bounds builds libfp2_bounds.so beside libfp2.so: the same sources with FP2_DEBUG_BOUNDS, whose calls
check page ids and the CSR on the device (fp2_debug_bounds_word in include/fp2.h).  The package always loads
libfp2.so; tests load the bounds build by path.

build_sanitized() links a second library for host-side checking only: the C-ABI host code (argument checks,
launch set-up) built with AddressSanitizer and UndefinedBehaviorSanitizer by the host compiler, beside the
usual gfx950 kernel objects.  It is loaded by tests with the sanitizer runtime preloaded, never by the package.
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
LIB_BOUNDS = os.path.join(PKG, "libfp2_bounds.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["fp2_api.cpp", "fp2_validate.cpp", "block_stats.hip", "plan_mask.hip", "prefill_attn.hip",
           "attn_d128.hip", "debug_bounds.hip"]
HOST_SOURCES = ["fp2_api.cpp", "fp2_validate.cpp"]  # plain host C++ (HIP runtime API only)
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
ASAN_RUNTIME = "libclang_rt.asan-x86_64.so"

COMMON = ["-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{ROOT}/include", f"-I{CSRC}"]
# gfx950 device code; packed-fp32 instructions are disabled on purpose.
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The bf16 attention kernel never produces a NaN (padding is staged as zeros,
# masks are -inf), so its max reductions need no NaN quieting.
EXTRA = {"attn_d128.hip": ["-fno-honor-nans"]}


def _compile(src, opt, out_dir=BUILD, defines=()):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, *EXTRA.get(src, []), *defines, opt, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]


def build(debug: bool = False, verbose: bool = True, bounds: bool = False) -> str:
    """libfp2.so, or with bounds=True libfp2_bounds.so (FP2_DEBUG_BOUNDS); returns its path."""
    out_dir = os.path.join(BUILD, "bounds") if bounds else BUILD
    lib = LIB_BOUNDS if bounds else LIB
    defines = ("-DFP2_DEBUG_BOUNDS",) if bounds else ()
    os.makedirs(out_dir, exist_ok=True)
    opt = "-O1" if debug else "-O3"
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, opt, out_dir, defines), SOURCES))
    for _, warn in results:
        if verbose and warn:
            print("\n".join(warn), file=sys.stderr)
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def asan_runtime() -> str:
    """Path of the host compiler's AddressSanitizer runtime (to preload when loading the sanitized library)."""
    r = subprocess.run([CLANGXX, f"-print-file-name={ASAN_RUNTIME}"], capture_output=True, text=True, check=True)
    return r.stdout.strip()


def build_sanitized(verbose: bool = False) -> str:
    """_build/san/libfp2_san.so: HOST_SOURCES with ASan + UBSan (host compiler, no device code), linked with
    the gfx950 kernel objects of the other sources (rebuilt when older than their source)."""
    san = os.path.join(BUILD, "san")
    os.makedirs(san, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(san, src + ".o")
        cmd = [CLANGXX, "-x", "c++", "-std=c++17", "-fPIC", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
               *SAN_FLAGS, f"-I{ROOT}/include", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    os.makedirs(BUILD, exist_ok=True)
    for src in SOURCES:
        if src in HOST_SOURCES:
            continue
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(os.path.join(CSRC, src)):
            _compile(src, "-O3")
        objs.append(obj)
    out = os.path.join(san, "libfp2_san.so")
    cmd = [CLANGXX, "-shared", "-shared-libasan", *SAN_FLAGS, "-o", out, *objs, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(out)
    return out


if __name__ == "__main__":
    print(build(debug="--debug" in sys.argv, bounds="--debug-bounds" in sys.argv))

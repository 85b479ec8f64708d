"""Build libdilated_attn.so (the C-ABI library) in-tree for gfx950.

Each HIP source compiles to an object in parallel, then one shared library is
linked. Packed fp32 instructions are disabled for all device code.
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdilated_attn.so")
# Host code under AddressSanitizer and UndefinedBehaviorSanitizer (device code
# unchanged): for CPU-only test runs with clang's ASan runtime preloaded.
LIB_ASAN = os.path.join(PKG, "libdilated_attn_asan.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SOURCES = ["api.hip", "attn_kernel.hip", "merge_kernel.hip", "bwd_kernel.hip",
           "qknorm_kernel.hip"]
HEADERS = ["da_common.hpp", "kernels.hpp"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: no accvgpr copies around the
    # softmax and fewer registers (three waves per SIMD instead of two)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source extra flags. The attention kernel's scores and maxima are never
# NaN (masked scores are -inf and every processed row has a finite maximum),
# so max operations need no NaN canonicalisation. (The bf16 row-sum MFMA can
# see 0 * inf on a tile whose probabilities overflow; that tile's overflow
# test compares bit patterns, which this flag cannot fold away.)
EXTRA = {"attn_kernel.hip": ["-fno-honor-nans"]}


def _compile(src, verbose, sanitize=False):
    sub = os.path.join(BUILD_DIR, "asan") if sanitize else BUILD_DIR
    obj = os.path.join(sub, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + (SAN_FLAGS if sanitize else []) + [
        "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library
    (with sanitize: the host-sanitized copy, LIB_ASAN)."""
    os.makedirs(os.path.join(BUILD_DIR, "asan") if sanitize else BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), SOURCES))
    lib = LIB_ASAN if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + (
        SAN_FLAGS if sanitize else []) + objs
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))

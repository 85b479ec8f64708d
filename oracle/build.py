"""Build the CPU oracle's shared library (test infrastructure only).

Plain gcc, -O2, OpenMP, IEEE arithmetic (no fast-math): the oracle must be
the straightforward definition, not a tuned kernel.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
# under AddressSanitizer and UndefinedBehaviorSanitizer, for test runs with
# gcc's ASan runtime preloaded
LIB_ASAN = os.path.join(HERE, "liboracle_asan.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]
SRCS = [os.path.join(HERE, "dilated_oracle.c")]
DEPS = SRCS + [os.path.join(HERE, "oracle_core.inc")]


def build(force: bool = True, verbose: bool = False, sanitize: bool = False) -> str:
    """Compile oracle/liboracle.so (with sanitize: liboracle_asan.so). Returns its path."""
    lib = LIB_ASAN if sanitize else LIB
    if not force and os.path.exists(lib):
        newest = max(os.path.getmtime(p) for p in DEPS)
        if os.path.getmtime(lib) >= newest:
            return lib
    tmp = lib + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-Wno-unused-parameter"] + (SAN_FLAGS if sanitize else []) + ["-o", tmp] + SRCS + [
               "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))

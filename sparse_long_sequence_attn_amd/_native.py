"""ctypes binding of libdilated_attn.so (the C ABI in include/dilated_attn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI. torch provides device memory and the current
stream. There is no CPU fallback: if the library is missing or the tensors
are not on a GPU, calls raise.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# DILATED_ATTN_LIB names another build of the same library (the
# host-sanitized one, for CPU-only test runs); default: the in-tree build
LIB_PATH = os.environ.get("DILATED_ATTN_LIB") or os.path.join(PKG, "libdilated_attn.so")

DA_F32, DA_BF16 = 0, 1
DA_HEAD_DIM = 64
DA_MAX_PATTERNS = 8
DA_NOALLOC_MAX_WORKSPACE_BYTES = 64 << 20

ERROR_NAMES = {
    0: "DA_OK", -1: "DA_ERR_NULL", -2: "DA_ERR_SHAPE", -3: "DA_ERR_PATTERN", -4: "DA_ERR_DTYPE",
    -5: "DA_ERR_HEADDIM", -6: "DA_ERR_WORKSPACE", -7: "DA_ERR_ALIGN", -8: "DA_ERR_ALIAS",
    -9: "DA_ERR_ARG", -10: "DA_ERR_LAUNCH",
}

# Every function the header declares, with its ctypes signature.
_P = ctypes.c_void_p
_I64, _I32, _SZ = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


class DaPattern(ctypes.Structure):
    _fields_ = [("w", ctypes.c_int32), ("r", ctypes.c_int32)]


_FWD_ARGS = [_P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _I32, _I32, _I32, ctypes.c_float,
             _P, _SZ, _P]
_BWD_ARGS = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _I32, _I32, _I32,
             ctypes.c_float, _P, _SZ, _P]
DA_BWD_PREP, DA_BWD_KV, DA_BWD_Q, DA_BWD_MERGE, DA_BWD_ALL = 1, 2, 4, 8, 15
SIGNATURES = {
    "dilated_attn_workspace_bytes": ([_I64, _I64, _I32, _I32, _P, _I32, _I32,
                                      ctypes.POINTER(_SZ)], ctypes.c_int),
    "dilated_attn_fwd": (_FWD_ARGS, ctypes.c_int),
    "dilated_attn_fwd_attention": (_FWD_ARGS, ctypes.c_int),
    "dilated_attn_fwd_merge": (_FWD_ARGS, ctypes.c_int),
    "dilated_attn_bwd_workspace_bytes": ([_I64, _I64, _I32, _I32, _P, _I32, _I32,
                                          ctypes.POINTER(_SZ)], ctypes.c_int),
    "dilated_attn_bwd": (_BWD_ARGS, ctypes.c_int),
    "dilated_attn_bwd_stages": ([_I32] + _BWD_ARGS, ctypes.c_int),
    "dilated_attn_qk_norm_fwd": ([_P] * 8 + [_I64, _I32, _I32, ctypes.c_float, _P], ctypes.c_int),
    "dilated_attn_qk_norm_workspace_bytes": ([_I64, ctypes.POINTER(_SZ)], ctypes.c_int),
    "dilated_attn_qk_norm_bwd": ([_P] * 9 + [_I64, _I32, _I32, ctypes.c_float, _P, _SZ, _P],
                                 ctypes.c_int),
    "dilated_attn_fwd_onepass": (_FWD_ARGS[:-3] + [_P], ctypes.c_int),
    "dilated_attn_fwd_noalloc": (_FWD_ARGS[:-3] + [_P], ctypes.c_int),
    "dilated_attn_fwd_qknorm": ([_P] * 7 + [ctypes.c_float, _P, _P, _I64, _I64, _I32, _I32, _I64,
                                           _P, _I32, _I32, _I32, ctypes.c_float, _P], ctypes.c_int),
    "dilated_attn_bwd_qknorm_workspace_bytes": ([_I64, _I64, _I32, _I32, _P, _I32, _I32,
                                                  ctypes.POINTER(_SZ)], ctypes.c_int),
    "dilated_attn_bwd_qknorm": ([_P] * 7 + [ctypes.c_float] + [_P] * 7 +
                                [_I64, _I64, _I32, _I32, _I64, _P, _I32, _I32, _I32,
                                 ctypes.c_float, _P, _SZ, _P], ctypes.c_int),
    "dilated_attn_gather_map": ([_I64, _I32, DaPattern, _I32, _P, _I64, ctypes.POINTER(_I64), _P],
                                ctypes.c_int),
    "dilated_attn_coverage_map": ([_I64, _I32, DaPattern, _I32, _P, _I64, _P], ctypes.c_int),
    "dilated_attn_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "dilated_attn_version": ([], ctypes.c_int),
}

_lib = None


class DilatedAttnError(RuntimeError):
    def __init__(self, code, fn):
        self.code = code
        super().__init__(f"{fn}: {ERROR_NAMES.get(code, code)} ({strerror(code)})")


def load_library(path=None):
    """Load the C-ABI library (built in-tree by build.py)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"{p} is missing: build it with `python -m sparse_long_sequence_attn_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(p)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def strerror(code):
    return load_library().dilated_attn_strerror(int(code)).decode()


def version():
    return load_library().dilated_attn_version()


def pattern_array(patterns):
    arr = (DaPattern * max(len(patterns), 1))()
    for i, (w, r) in enumerate(patterns):
        arr[i].w, arr[i].r = int(w), int(r)
    return arr


def check(code, fn):
    if code != 0:
        raise DilatedAttnError(code, fn)


def workspace_bytes(B, N, H, Dh, patterns, dtype):
    out = _SZ(0)
    code = load_library().dilated_attn_workspace_bytes(B, N, H, Dh, pattern_array(patterns),
                                                       len(patterns), dtype, ctypes.byref(out))
    check(code, "dilated_attn_workspace_bytes")
    return out.value


def bwd_workspace_bytes(B, N, H, Dh, patterns, dtype):
    out = _SZ(0)
    code = load_library().dilated_attn_bwd_workspace_bytes(B, N, H, Dh, pattern_array(patterns),
                                                           len(patterns), dtype,
                                                           ctypes.byref(out))
    check(code, "dilated_attn_bwd_workspace_bytes")
    return out.value


def bwd_qknorm_workspace_bytes(B, N, H, Dh, patterns, dtype):
    out = _SZ(0)
    code = load_library().dilated_attn_bwd_qknorm_workspace_bytes(
        B, N, H, Dh, pattern_array(patterns), len(patterns), dtype, ctypes.byref(out))
    check(code, "dilated_attn_bwd_qknorm_workspace_bytes")
    return out.value


def qk_norm_workspace_bytes(rows):
    out = _SZ(0)
    check(load_library().dilated_attn_qk_norm_workspace_bytes(rows, ctypes.byref(out)),
          "dilated_attn_qk_norm_workspace_bytes")
    return out.value

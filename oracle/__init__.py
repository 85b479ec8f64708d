"""CPU oracle for the dilated-attention forward pass.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this package. The product library never imports it and
shares no code with it. The arithmetic lives in ``dilated_oracle.c`` (plain
C, fp64, with an fp32 copy); this module only marshals NumPy arrays.

Inputs are NumPy arrays of shape [B, N, H, Dh]: float64, float32, or uint16
holding bf16 bit patterns (widened exactly by the C code).
"""
import ctypes
import os

import numpy as np

from . import build as _build


class _Pattern(ctypes.Structure):
    _fields_ = [("w", ctypes.c_int32), ("r", ctypes.c_int32)]


_IN_F64, _IN_F32, _IN_BF16 = 0, 1, 2


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.orc_geometry.argtypes = [i64, i32, i32, i32] + [ctypes.POINTER(i64)] * 4
    lib.orc_geometry.restype = ctypes.c_int
    lib.orc_gather_map.argtypes = [i64, i32, i32, i32, P, i64]
    lib.orc_gather_map.restype = i64
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = ctypes.c_int
    for sfx in ("f64", "f32"):
        f = getattr(lib, "orc_fwd_" + sfx)
        f.argtypes = [P, P, P, ctypes.c_int, i64, i64, i32, i32, P, i32, i32,
                      ctypes.c_double, ctypes.c_int, P, P, P, P]
        f.restype = ctypes.c_int
        g = getattr(lib, "orc_rows_" + sfx)
        g.argtypes = [P, P, P, ctypes.c_int, i64, i64, i32, i32, P, i32, i32,
                      ctypes.c_double, ctypes.c_int, P, i64, P, P, P]
        g.restype = ctypes.c_int
        bw = getattr(lib, "orc_bwd_" + sfx)
        bw.argtypes = [P, P, P, P, ctypes.c_int, i64, i64, i32, i32, P, i32, i32,
                       ctypes.c_double, ctypes.c_int, P, P, P]
        bw.restype = ctypes.c_int
        br = getattr(lib, "orc_bwd_rows_" + sfx)
        br.argtypes = [P, P, P, P, ctypes.c_int, i64, i64, i32, i32, P, i32, i32,
                       ctypes.c_double, ctypes.c_int, P, i64, P, P, P]
        br.restype = ctypes.c_int
    return lib


def _in_dtype(a):
    if a.dtype == np.float64:
        return _IN_F64
    if a.dtype == np.float32:
        return _IN_F32
    if a.dtype == np.uint16:
        return _IN_BF16
    raise TypeError(f"oracle inputs must be float64, float32 or uint16 (bf16 bits), got {a.dtype}")


def _patterns(patterns):
    arr = (_Pattern * len(patterns))()
    for i, (w, r) in enumerate(patterns):
        arr[i].w, arr[i].r = int(w), int(r)
    return arr


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _check_inputs(q, k, v):
    for a in (q, k, v):
        if a.ndim != 4 or not a.flags.c_contiguous:
            raise ValueError("q, k, v must be C-contiguous [B, N, H, Dh]")
    if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")


class Oracle:
    """The oracle functions bound to one build of the C library."""

    def __init__(self, path=None):
        if path is None:
            # ORACLE_LIB names another build (the sanitized one)
            path = os.environ.get("ORACLE_LIB") or _build.LIB
            if not os.path.exists(path):
                _build.build(force=True)
        self.path = path
        self._lib = _bind(path)

    def max_threads(self):
        return self._lib.orc_max_threads()

    def geometry(self, N, w, r, h):
        """(wp, nseg, off, L) of pattern (w, r) for head h; raises on bad shapes."""
        lib = self._lib
        out = [ctypes.c_int64() for _ in range(4)]
        rc = lib.orc_geometry(N, w, r, h, *[ctypes.byref(o) for o in out])
        if rc:
            raise ValueError(f"orc_geometry({N}, {w}, {r}, {h}) -> {rc}")
        return tuple(o.value for o in out)

    def gather_map(self, N, w, r, h):
        """Gathered positions of pattern (w, r), head h, segment-major: int64 [nseg, L]."""
        wp, nseg, off, L = self.geometry(N, w, r, h)
        out = np.empty(max(nseg * L, 1), dtype=np.int64)
        n = self._lib.orc_gather_map(N, w, r, h, _ptr(out), out.size)
        if n < 0:
            raise ValueError(f"orc_gather_map -> {n}")
        return out[:n].reshape(nseg, L)

    def fwd(self, q, k, v, patterns, causal=True, scale=None, precision="f64", threads=0,
            return_patterns=False):
        """Dilated attention, segment formulation.

        Returns (out [B,N,H,Dh], lse [B,H,N]) in the chosen precision, and with
        return_patterns also (pat_out [np,B,N,H,Dh], pat_lse [np,B,H,N]).
        """
        _check_inputs(q, k, v)
        lib = self._lib
        B, N, H, Dh = q.shape
        real = np.float64 if precision == "f64" else np.float32
        fn = lib.orc_fwd_f64 if precision == "f64" else lib.orc_fwd_f32
        out = np.empty((B, N, H, Dh), dtype=real)
        lse = np.empty((B, H, N), dtype=real)
        npat = len(patterns)
        pat_out = np.empty((npat, B, N, H, Dh), dtype=real) if return_patterns else None
        pat_lse = np.empty((npat, B, H, N), dtype=real) if return_patterns else None
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _in_dtype(q), B, N, H, Dh, _patterns(patterns), npat,
                1 if causal else 0, float(scale or 0.0), int(threads), _ptr(out), _ptr(lse),
                _ptr(pat_out), _ptr(pat_lse))
        if rc:
            raise RuntimeError(f"orc_fwd_{precision} -> {rc}")
        if return_patterns:
            return out, lse, pat_out, pat_lse
        return out, lse

    def rows(self, q, k, v, patterns, row_idx, causal=True, scale=None, precision="f64", threads=0,
             return_pattern_lse=False):
        """Dilated attention for selected rows, row formulation.

        row_idx: int64 [n, 3] of (b, t, h). Returns (out [n, Dh], lse [n]) and with
        return_pattern_lse also pat_lse [n, np].
        """
        _check_inputs(q, k, v)
        lib = self._lib
        B, N, H, Dh = q.shape
        row_idx = np.ascontiguousarray(row_idx, dtype=np.int64).reshape(-1, 3)
        n = row_idx.shape[0]
        real = np.float64 if precision == "f64" else np.float32
        fn = lib.orc_rows_f64 if precision == "f64" else lib.orc_rows_f32
        out = np.empty((n, Dh), dtype=real)
        lse = np.empty((n,), dtype=real)
        pl = np.empty((n, len(patterns)), dtype=real) if return_pattern_lse else None
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _in_dtype(q), B, N, H, Dh, _patterns(patterns),
                len(patterns), 1 if causal else 0, float(scale or 0.0), int(threads), _ptr(row_idx),
                n, _ptr(out), _ptr(lse), _ptr(pl))
        if rc:
            raise RuntimeError(f"orc_rows_{precision} -> {rc}")
        if return_pattern_lse:
            return out, lse, pl
        return out, lse

    def bwd(self, q, k, v, dout, patterns, causal=True, scale=None, precision="f64", threads=0):
        """Gradients (dq, dk, dv) of sum(dout * out), each [B, N, H, Dh]."""
        _check_inputs(q, k, v)
        _check_inputs(q, dout, dout)
        lib = self._lib
        B, N, H, Dh = q.shape
        real = np.float64 if precision == "f64" else np.float32
        fn = lib.orc_bwd_f64 if precision == "f64" else lib.orc_bwd_f32
        dq, dk, dv = (np.empty((B, N, H, Dh), dtype=real) for _ in range(3))
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _in_dtype(q), B, N, H, Dh,
                _patterns(patterns), len(patterns), 1 if causal else 0, float(scale or 0.0),
                int(threads), _ptr(dq), _ptr(dk), _ptr(dv))
        if rc:
            raise RuntimeError(f"orc_bwd_{precision} -> {rc}")
        return dq, dk, dv

    def bwd_rows(self, q, k, v, dout, patterns, row_idx, causal=True, scale=None,
                 want_dq=True, want_dkv=True, precision="f64", threads=0):
        """Backward pass at selected rows (row formulation). row_idx: int64
        [n, 3] of (b, t, h). Returns (dq, dk, dv), each [n, Dh] or None."""
        _check_inputs(q, k, v)
        _check_inputs(q, dout, dout)
        lib = self._lib
        B, N, H, Dh = q.shape
        row_idx = np.ascontiguousarray(row_idx, dtype=np.int64).reshape(-1, 3)
        n = row_idx.shape[0]
        real = np.float64 if precision == "f64" else np.float32
        fn = lib.orc_bwd_rows_f64 if precision == "f64" else lib.orc_bwd_rows_f32
        dq = np.empty((n, Dh), dtype=real) if want_dq else None
        dk = np.empty((n, Dh), dtype=real) if want_dkv else None
        dv = np.empty((n, Dh), dtype=real) if want_dkv else None
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _in_dtype(q), B, N, H, Dh,
                _patterns(patterns), len(patterns), 1 if causal else 0, float(scale or 0.0),
                int(threads), _ptr(row_idx), n, _ptr(dq), _ptr(dk), _ptr(dv))
        if rc:
            raise RuntimeError(f"orc_bwd_rows_{precision} -> {rc}")
        return dq, dk, dv


_default = None


def default():
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def max_threads():
    return default().max_threads()


def geometry(N, w, r, h):
    return default().geometry(N, w, r, h)


def gather_map(N, w, r, h):
    return default().gather_map(N, w, r, h)


def fwd(*args, **kwargs):
    return default().fwd(*args, **kwargs)


def rows(*args, **kwargs):
    return default().rows(*args, **kwargs)


def bwd(*args, **kwargs):
    return default().bwd(*args, **kwargs)


def bwd_rows(*args, **kwargs):
    return default().bwd_rows(*args, **kwargs)

"""The C-ABI library without a GPU: it loads, exports every symbol the
header declares, and rejects every invalid call before touching HIP.

Pointers here are fake device addresses: validation never dereferences them,
and every case below fails validation, so no HIP call is made.
"""
import ctypes
import math
import os
import re

import pytest

from sparse_long_sequence_attn_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dilated_attn.h")

A = 1 << 20          # distinct, 256-byte aligned fake device addresses
Q, K, V, OUT, LSE, WS = (A * i for i in range(1, 7))


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dilated_attn_\w+)\s*\(", text)))


def header_constants():
    text = open(HEADER).read()
    return {m[0]: int(m[1]) for m in re.findall(r"\b(DA_\w+)\s*=\s*(-?\d+)", text)}


@pytest.fixture(scope="module")
def lib():
    return _native.load_library()


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) == 19
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_native.SIGNATURES)


def test_binding_constants_match_header():
    c = header_constants()
    assert c["DA_F32"] == _native.DA_F32 and c["DA_BF16"] == _native.DA_BF16
    for name in ("DA_BWD_PREP", "DA_BWD_KV", "DA_BWD_Q", "DA_BWD_MERGE", "DA_BWD_ALL"):
        assert c[name] == getattr(_native, name)
    assert c["DA_BWD_ALL"] == c["DA_BWD_PREP"] | c["DA_BWD_KV"] | c["DA_BWD_Q"] | c["DA_BWD_MERGE"]
    for code, name in _native.ERROR_NAMES.items():
        assert c[name] == code
    text = open(HEADER).read()
    assert int(re.search(r"#define DA_MAX_PATTERNS (\d+)", text)[1]) == _native.DA_MAX_PATTERNS
    assert int(re.search(r"#define DA_HEAD_DIM (\d+)", text)[1]) == _native.DA_HEAD_DIM
    m = re.search(r"#define DA_NOALLOC_MAX_WORKSPACE_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert (int(m[1]) << int(m[2])) == _native.DA_NOALLOC_MAX_WORKSPACE_BYTES
    assert int(re.search(r"#define DA_VERSION (\d+)", text)[1]) == _native.version()


def test_strerror_covers_every_code(lib):
    seen = set()
    for code in _native.ERROR_NAMES:
        s = _native.strerror(code)
        assert s and s != "unknown error code"
        seen.add(s)
    assert len(seen) == len(_native.ERROR_NAMES)
    assert _native.strerror(12345) == "unknown error code"


def fwd(lib, fn="dilated_attn_fwd", q=Q, k=K, v=V, out=OUT, lse=LSE, B=1, N=64, H=4, Dh=64,
        pats=((16, 2), (32, 4)), npat=None, causal=1, dtype=_native.DA_BF16, scale=0.0, ws=WS,
        wsb=1 << 30):
    arr = _native.pattern_array(pats) if pats is not None else None
    return getattr(lib, fn)(q, k, v, out, lse, B, N, H, Dh, arr,
                            len(pats) if npat is None else npat, causal, dtype, scale, ws, wsb, None)


@pytest.mark.parametrize("fn", ["dilated_attn_fwd", "dilated_attn_fwd_attention",
                                "dilated_attn_fwd_merge"])
@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(out=None), -1),
    (dict(lse=None), -1), (dict(pats=None, npat=1), -1),
    (dict(B=-1), -2), (dict(N=-4), -2), (dict(H=-1), -2), (dict(N=60), -2),
    (dict(B=70000), -2), (dict(N=1 << 31), -2),
    (dict(pats=()), -3), (dict(pats=((16, 2),) * 9), -3), (dict(pats=((0, 1),)), -3),
    (dict(pats=((16, 0),)), -3), (dict(pats=((8, 9),)), -3), (dict(pats=((128, 65),)), -3),
    (dict(dtype=2), -4), (dict(dtype=-1), -4),
    (dict(Dh=128), -5), (dict(Dh=32), -5),
    (dict(ws=None), -6), (dict(wsb=100), -6),
    (dict(q=Q + 8), -7), (dict(out=OUT + 4), -7), (dict(lse=LSE + 2), -7), (dict(ws=WS + 64), -7),
    (dict(out=Q), -8), (dict(lse=K + 64), -8), (dict(ws=V), -8), (dict(out=LSE), -8),
    (dict(causal=2), -9), (dict(scale=math.inf), -9), (dict(scale=math.nan), -9),
])
def test_invalid_calls_rejected(lib, fn, kwargs, code):
    assert fwd(lib, fn, **kwargs) == code


def test_empty_problems_are_accepted_without_launch(lib):
    # nothing to do: no pointer is needed and nothing is launched
    for B, N, H in [(0, 64, 4), (1, 0, 4), (1, 64, 0)]:
        assert fwd(lib, B=B, N=N, H=H, q=None, k=None, v=None, out=None, lse=None, ws=None,
                   wsb=0) == 0


def ws_expected(B, N, H, pats):
    """Workspace size from the layout the header describes: per pattern, a
    float partial row (64 values) and a float lse per gathered row slot
    (segments x ceil(w'/r)), each region rounded up to 256 bytes."""
    if len(pats) == 1:
        return 0
    tot = 0
    for (w, r) in pats:
        wp = min(w, N)
        rows = B * H * (N // wp) * (-(-wp // r))
        tot += -(-rows * 64 * 4 // 256) * 256 + -(-rows * 4 // 256) * 256
    return tot


@pytest.mark.parametrize("B,N,H,pats", [
    (1, 512, 8, [(64, 2)]),
    (4, 8192, 12, [(2048, 1), (4096, 2), (8192, 4)]),
    (1, 32768, 16, [(2048, 1), (4096, 2), (8192, 4), (16384, 6), (32768, 12)]),
    (2, 96, 3, [(1000, 7), (8, 1), (96, 96)]),
])
def test_workspace_bytes(B, N, H, pats):
    assert _native.workspace_bytes(B, N, H, 64, pats, _native.DA_BF16) == ws_expected(B, N, H, pats)


def test_workspace_bytes_errors(lib):
    out = ctypes.c_size_t(0)
    arr = _native.pattern_array([(16, 2)])
    assert lib.dilated_attn_workspace_bytes(1, 64, 4, 64, arr, 1, 1, None) == -1
    assert lib.dilated_attn_workspace_bytes(1, 60, 4, 64, arr, 1, 1, ctypes.byref(out)) == -2
    assert lib.dilated_attn_workspace_bytes(1, 64, 4, 32, arr, 1, 1, ctypes.byref(out)) == -5


@pytest.mark.parametrize("fn", ["dilated_attn_gather_map", "dilated_attn_coverage_map"])
def test_map_hooks_validate(lib, fn):
    g = getattr(lib, fn)
    if fn == "dilated_attn_gather_map":
        def f(N, H, p, h, out, cap, stream):
            return g(N, H, p, h, out, cap, None, stream)
    else:
        f = g
    p = _native.DaPattern(16, 2)
    assert f(64, 4, p, 0, None, 1 << 20, None) == -1
    assert f(60, 4, p, 0, A, 1 << 20, None) == -2
    assert f(64, 4, _native.DaPattern(16, 0), 0, A, 1 << 20, None) == -3
    assert f(64, 4, p, 4, A, 1 << 20, None) == -9
    assert f(64, 4, p, -1, A, 1 << 20, None) == -9
    assert f(64, 4, p, 0, A, 3, None) == -9
    assert f(64, 4, p, 0, A + 4, 1 << 20, None) == -7


# ---------------------------------------------------------------- backward

DOUT, DQ, DK, DV = (A * i for i in range(7, 11))


def bwd(lib, stages=None, q=Q, k=K, v=V, out=OUT, lse=LSE, dout=DOUT, dq=DQ, dk=DK, dv=DV, B=1,
        N=64, H=4, Dh=64, pats=((16, 2), (32, 4)), npat=None, causal=1, dtype=_native.DA_BF16,
        scale=0.0, ws=WS, wsb=1 << 30):
    arr = _native.pattern_array(pats) if pats is not None else None
    args = (q, k, v, out, lse, dout, dq, dk, dv, B, N, H, Dh, arr,
            len(pats) if npat is None else npat, causal, dtype, scale, ws, wsb, None)
    if stages is None:
        return lib.dilated_attn_bwd(*args)
    return lib.dilated_attn_bwd_stages(stages, *args)


@pytest.mark.parametrize("stages", [None, 15, 1, 8])
@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(lse=None), -1), (dict(dout=None), -1),
    (dict(dq=None), -1), (dict(dk=None), -1), (dict(dv=None), -1), (dict(pats=None, npat=1), -1),
    (dict(B=-1), -2), (dict(N=60), -2), (dict(N=1 << 31), -2),
    (dict(pats=()), -3), (dict(pats=((8, 9),)), -3),
    (dict(dtype=2), -4), (dict(Dh=128), -5),
    (dict(ws=None), -6), (dict(wsb=100), -6), (dict(pats=((16, 2),), wsb=4), -6),
    (dict(dout=DOUT + 8), -7), (dict(dq=DQ + 8), -7), (dict(dv=DV + 2), -7),
    (dict(lse=LSE + 2), -7), (dict(ws=WS + 64), -7),
    (dict(dq=Q), -8), (dict(dk=OUT), -8), (dict(dv=DOUT + 64), -8), (dict(ws=LSE), -8),
    (dict(dq=DK), -8), (dict(dv=DK + 256), -8), (dict(ws=DQ), -8),
    (dict(causal=2), -9), (dict(scale=math.nan), -9),
])
def test_bwd_invalid_calls_rejected(lib, stages, kwargs, code):
    assert bwd(lib, stages, **kwargs) == code


@pytest.mark.parametrize("stages", [0, 16, -1, 31])
def test_bwd_stage_flags_validated(lib, stages):
    assert bwd(lib, stages) == -9


def test_bwd_inputs_may_alias_each_other(lib):
    # q, k, v, out, dout read-only: sharing is allowed, so validation passes
    # until the (absent) workspace check
    assert bwd(lib, k=Q, v=Q, dout=Q, ws=None) == -6


def test_bwd_empty_problems_are_accepted_without_launch(lib):
    for B, N, H in [(0, 64, 4), (1, 0, 4), (1, 64, 0)]:
        assert bwd(lib, B=B, N=N, H=H, q=None, k=None, v=None, out=None, lse=None, dout=None,
                   dq=None, dk=None, dv=None, ws=None, wsb=0) == 0


def bwd_ws_expected(B, N, H, pats, es):
    """Backward workspace from the documented layout: a float D per row
    (rounded up to 256 bytes), then for two or more patterns three partial
    rows (dq, dk, dv) per gathered row slot in the gradients' dtype (es bytes
    an element), per pattern rounded up to 256 bytes."""
    tot = -(-B * H * N * 4 // 256) * 256
    if len(pats) > 1:
        for (w, r) in pats:
            wp = min(w, N)
            rows = B * H * (N // wp) * (-(-wp // r))
            tot += -(-3 * rows * 64 * es // 256) * 256
    return tot


@pytest.mark.parametrize("B,N,H,pats", [
    (1, 512, 8, [(64, 2)]),
    (4, 8192, 12, [(2048, 1), (4096, 2), (8192, 4)]),
    (1, 32768, 16, [(2048, 1), (4096, 2), (8192, 4), (16384, 6), (32768, 12)]),
    (2, 96, 3, [(1000, 7), (8, 1), (96, 96)]),
])
@pytest.mark.parametrize("dtype,es", [(_native.DA_BF16, 2), (_native.DA_F32, 4)])
def test_bwd_workspace_bytes(B, N, H, pats, dtype, es):
    got = _native.bwd_workspace_bytes(B, N, H, 64, pats, dtype)
    assert got == bwd_ws_expected(B, N, H, pats, es)


def test_bwd_workspace_bytes_errors(lib):
    out = ctypes.c_size_t(0)
    arr = _native.pattern_array([(16, 2)])
    assert lib.dilated_attn_bwd_workspace_bytes(1, 64, 4, 64, arr, 1, 1, None) == -1
    assert lib.dilated_attn_bwd_workspace_bytes(1, 60, 4, 64, arr, 1, 1, ctypes.byref(out)) == -2
    assert lib.dilated_attn_bwd_workspace_bytes(0, 64, 4, 64, arr, 1, 1, ctypes.byref(out)) == 0
    assert out.value == 0


# ---------------------------------------------------------------- qk_norm

XQ, XK, GQ, BQ, GK, BK, YQ, YK = (A * i for i in range(11, 19))
DPAR, QWS = A * 19, A * 20


def qkn_fwd(lib, xq=XQ, xk=XK, gq=GQ, bq=BQ, gk=GK, bk=BK, yq=YQ, yk=YK, rows=256, Dh=64,
            dtype=_native.DA_BF16, eps=1e-5):
    return lib.dilated_attn_qk_norm_fwd(xq, xk, gq, bq, gk, bk, yq, yk, rows, Dh, dtype, eps, None)


def qkn_bwd(lib, xq=XQ, xk=XK, dyq=YQ, dyk=YK, gq=GQ, gk=GK, dxq=DQ, dxk=DK, dpar=DPAR, rows=256,
            Dh=64, dtype=_native.DA_BF16, eps=1e-5, ws=QWS, wsb=1 << 20):
    return lib.dilated_attn_qk_norm_bwd(xq, xk, dyq, dyk, gq, gk, dxq, dxk, dpar, rows, Dh, dtype,
                                        eps, ws, wsb, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(xq=None), -1), (dict(bk=None), -1), (dict(yk=None), -1),
    (dict(rows=-1), -2), (dict(dtype=3), -4), (dict(Dh=32), -5),
    (dict(xq=XQ + 8), -7), (dict(gk=GK + 4), -7), (dict(yq=YQ + 2), -7),
    (dict(yq=XQ), -8), (dict(yk=XK + 64), -8), (dict(yk=YQ), -8), (dict(yq=GQ), -8),
    (dict(eps=0.0), -9), (dict(eps=-1.0), -9), (dict(eps=math.nan), -9),
])
def test_qk_norm_fwd_invalid_calls_rejected(lib, kwargs, code):
    assert qkn_fwd(lib, **kwargs) == code


@pytest.mark.parametrize("kwargs,code", [
    (dict(dyq=None), -1), (dict(dpar=None), -1), (dict(dxk=None), -1),
    (dict(rows=-5), -2), (dict(dtype=2), -4), (dict(Dh=128), -5),
    (dict(ws=None), -6), (dict(wsb=16), -6),
    (dict(dxq=DQ + 8), -7), (dict(dpar=DPAR + 2), -7), (dict(ws=QWS + 16), -7),
    (dict(dxq=XQ), -8), (dict(dxk=YK), -8), (dict(dpar=GK), -8), (dict(ws=DQ), -8),
    (dict(dxk=DQ), -8),
    (dict(eps=math.inf), -9),
])
def test_qk_norm_bwd_invalid_calls_rejected(lib, kwargs, code):
    assert qkn_bwd(lib, **kwargs) == code


def test_qk_norm_zero_rows_is_a_no_op(lib):
    assert qkn_fwd(lib, rows=0, xq=None, xk=None, yq=None, yk=None) == 0
    assert qkn_bwd(lib, rows=0, xq=None, dxq=None, ws=None, wsb=0) == 0


def test_qk_norm_workspace_bytes(lib):
    assert _native.qk_norm_workspace_bytes(0) == 0
    assert _native.qk_norm_workspace_bytes(1) == 2 * 1 * 128 * 4
    assert _native.qk_norm_workspace_bytes(32 * 1024 * 100) == 2 * 1024 * 128 * 4
    out = ctypes.c_size_t(0)
    assert lib.dilated_attn_qk_norm_workspace_bytes(-1, ctypes.byref(out)) == -2
    assert lib.dilated_attn_qk_norm_workspace_bytes(5, None) == -1


# ---------------------------------------------------------------- qk_norm fused into the attention

QKN_PATS = ((32, 2),)


def fqkn_fwd(lib, xq=Q, xk=K, v=V, gq=GQ, bq=BQ, gk=GK, bk=BK, eps=1e-5, out=OUT, lse=LSE, B=1,
             N=64, H=4, Dh=64, rs=0, pats=QKN_PATS, causal=1, dtype=_native.DA_BF16, scale=0.0):
    arr = _native.pattern_array(pats)
    return lib.dilated_attn_fwd_qknorm(xq, xk, v, gq, bq, gk, bk, eps, out, lse, B, N, H, Dh, rs,
                                       arr, len(pats), causal, dtype, scale, None)


def fqkn_bwd(lib, xq=Q, xk=K, v=V, gq=GQ, bq=BQ, gk=GK, bk=BK, eps=1e-5, out=OUT, lse=LSE,
             dout=DOUT, dxq=DQ, dxk=DK, dv=DV, dpar=DPAR, B=1, N=64, H=4, Dh=64, rs=0,
             pats=QKN_PATS, causal=1, dtype=_native.DA_BF16, scale=0.0, ws=WS, wsb=1 << 20):
    arr = _native.pattern_array(pats)
    return lib.dilated_attn_bwd_qknorm(xq, xk, v, gq, bq, gk, bk, eps, out, lse, dout, dxq, dxk,
                                       dv, dpar, B, N, H, Dh, rs, arr, len(pats), causal, dtype,
                                       scale, ws, wsb, None)


COMMON_FUSED_ERRORS = [
    (dict(xq=None), -1), (dict(gq=None), -1), (dict(bk=None), -1),
    (dict(N=60), -2), (dict(B=-1), -2),
    (dict(pats=((16, 2), (32, 4))), -3),  # two patterns
    (dict(pats=((64, 1),)), -3),          # 64 rows per segment
    (dict(dtype=2), -4), (dict(Dh=128), -5),
    (dict(gq=GQ + 8), -7), (dict(bk=BK + 4), -7),  # gains and biases: 16-byte aligned
    (dict(eps=0.0), -9), (dict(eps=math.nan), -9), (dict(causal=3), -9),
    (dict(rs=-1), -9), (dict(rs=128), -9),   # below H * Dh = 256
    (dict(rs=260), -7),                      # rows of 520 bytes: not 16-byte aligned
]


@pytest.mark.parametrize("kwargs,code", COMMON_FUSED_ERRORS + [
    (dict(out=GQ), -8), (dict(lse=BK), -8), (dict(out=None), -1),
])
def test_fused_qknorm_fwd_invalid_calls_rejected(lib, kwargs, code):
    assert fqkn_fwd(lib, **kwargs) == code


@pytest.mark.parametrize("kwargs,code", COMMON_FUSED_ERRORS + [
    (dict(dpar=None), -1), (dict(dout=None), -1),
    (dict(ws=None), -6), (dict(wsb=1024), -6),
    (dict(dpar=DPAR + 2), -7),
    (dict(dpar=Q), -8), (dict(dpar=DQ + 64), -8), (dict(dpar=WS + 256), -8),
    (dict(dxq=GK), -8), (dict(ws=GQ - 256), -8),
    # q, k, v and their gradients as parts of one [B, N, 3, H, Dh] buffer
    # (rows of 512 bytes every 1536): gradient rows on top of each other,
    # or on the inputs, are aliases
    (dict(rs=768, xk=Q + 512, v=Q + 1024, dxk=DQ + 64, dv=DQ + 1024), -8),
    (dict(rs=768, xk=Q + 512, v=Q + 1024, dxq=Q + 1024, dxk=DQ + 512, dv=DQ + 1024), -8),
    (dict(rs=768, xk=Q + 512, v=Q + 1024, dxk=DQ + 512, dv=DQ + 1024, ws=DQ + 4096), -8),
])
def test_fused_qknorm_bwd_invalid_calls_rejected(lib, kwargs, code):
    assert fqkn_bwd(lib, **kwargs) == code


def test_fused_qknorm_empty_problem_is_a_no_op(lib):
    assert fqkn_fwd(lib, B=0, xq=None, xk=None, v=None, out=None, lse=None) == 0
    assert fqkn_bwd(lib, N=0, xq=None, dxq=None, ws=None, wsb=0, dpar=None) == 0


@pytest.mark.parametrize("B,N,H,w,r", [(32, 8192, 8, 64, 2), (1, 64, 4, 32, 2), (3, 240, 3, 40, 3),
                                       (1, 32, 5, 64, 2)])
def test_fused_qknorm_workspace_bytes(B, N, H, w, r):
    """The plain backward's workspace, then float [2][units][128] partials,
    then float [2][min(units, 1024)][128] folded sums, each region starting
    on a 256-byte boundary; units = B * H * segments."""
    up = lambda x: -(-x // 256) * 256
    units = B * H * (N // min(w, N))
    plain = _native.bwd_workspace_bytes(B, N, H, 64, [(w, r)], _native.DA_BF16)
    exp = up(up(plain) + 2 * units * 128 * 4) + 2 * min(units, 1024) * 128 * 4
    assert _native.bwd_qknorm_workspace_bytes(B, N, H, 64, [(w, r)], _native.DA_BF16) == exp


def test_fused_qknorm_workspace_bytes_errors(lib):
    out = ctypes.c_size_t(7)
    arr = _native.pattern_array([(64, 1)])
    assert lib.dilated_attn_bwd_qknorm_workspace_bytes(1, 64, 4, 64, arr, 1, 1,
                                                       ctypes.byref(out)) == -3
    arr = _native.pattern_array([(32, 2)])
    assert lib.dilated_attn_bwd_qknorm_workspace_bytes(1, 64, 4, 64, arr, 1, 1, None) == -1
    assert lib.dilated_attn_bwd_qknorm_workspace_bytes(0, 64, 4, 64, arr, 1, 1,
                                                       ctypes.byref(out)) == 0
    assert out.value == 0


# ---------------------------------------------------------------- one-pass forward


def onepass(lib, q=Q, k=K, v=V, out=OUT, lse=LSE, B=1, N=64, H=4, Dh=64, pats=((16, 2), (32, 4)),
            causal=1, dtype=_native.DA_BF16, scale=0.0):
    arr = _native.pattern_array(pats)
    return lib.dilated_attn_fwd_onepass(q, k, v, out, lse, B, N, H, Dh, arr, len(pats), causal,
                                        dtype, scale, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), -1), (dict(lse=None), -1),
    (dict(N=60), -2), (dict(B=-1), -2),
    (dict(pats=((16, 0),)), -3), (dict(pats=((16, 2),) * 9), -3),
    (dict(pats=((8, 5), (8, 7))), -3),  # lcm(r) = 35 above gcd(w) = 8
    (dict(dtype=_native.DA_F32), -4), (dict(dtype=2), -4), (dict(Dh=32), -5),
    (dict(q=Q + 8), -7), (dict(lse=LSE + 2), -7),
    (dict(out=Q), -8), (dict(lse=K + 64), -8), (dict(out=LSE), -8),
    (dict(causal=2), -9), (dict(scale=math.nan), -9),
])
def test_onepass_invalid_calls_rejected(lib, kwargs, code):
    assert onepass(lib, **kwargs) == code


def test_onepass_empty_problem_is_a_no_op(lib):
    assert onepass(lib, B=0, q=None, k=None, v=None, out=None, lse=None) == 0


def noalloc(lib, q=Q, k=K, v=V, out=OUT, lse=LSE, B=1, N=64, H=4, Dh=64, pats=((16, 2), (32, 4)),
            causal=1, dtype=_native.DA_BF16, scale=0.0):
    arr = _native.pattern_array(pats)
    return lib.dilated_attn_fwd_noalloc(q, k, v, out, lse, B, N, H, Dh, arr, len(pats), causal,
                                        dtype, scale, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), -1), (dict(lse=None), -1),
    (dict(N=60), -2), (dict(B=-1), -2),
    (dict(pats=((16, 0),)), -3), (dict(pats=((16, 2),) * 9), -3),
    (dict(dtype=2), -4), (dict(Dh=32), -5),
    (dict(q=Q + 8), -7), (dict(lse=LSE + 2), -7),
    (dict(out=Q), -8), (dict(lse=K + 64), -8), (dict(out=LSE), -8),
    (dict(causal=2), -9), (dict(scale=math.nan), -9),
])
def test_noalloc_invalid_calls_rejected(lib, kwargs, code):
    assert noalloc(lib, **kwargs) == code


def test_noalloc_rejects_workspaces_beyond_its_array(lib):
    """A problem whose workspace exceeds the library's array is refused before
    anything touches HIP; one just inside it only fails on the fake pointers'
    overlap, also before any HIP call."""
    limit = _native.DA_NOALLOC_MAX_WORKSPACE_BYTES
    pats = ((64, 1), (128, 2))
    big = 1
    while _native.workspace_bytes(1, 1 << big, 16, 64, pats, _native.DA_BF16) <= limit:
        big += 1
    N = 1 << big
    assert _native.workspace_bytes(1, N, 16, 64, pats, _native.DA_BF16) > limit
    assert noalloc(lib, N=N, H=16, pats=pats) == -6
    assert noalloc(lib, N=N, H=16, pats=pats, out=Q) == -6  # the size is checked first


def test_noalloc_empty_problem_is_a_no_op(lib):
    assert noalloc(lib, B=0, q=None, k=None, v=None, out=None, lse=None) == 0


@pytest.mark.parametrize("N,w,r", [(64, 16, 2), (96, 1000, 7), (32768, 16384, 6), (120, 40, 6),
                                   (64, 64, 64)])
def test_gather_map_shape_from_the_library(lib, N, w, r):
    """The library reports the gather map's shape (segments, rows per
    segment) without launching anything when no output buffer is given."""
    shape = (ctypes.c_int64 * 2)()
    assert lib.dilated_attn_gather_map(N, 4, _native.DaPattern(w, r), 0, None, 0, shape,
                                       None) == 0
    wp = min(w, N)
    assert (shape[0], shape[1]) == (N // wp, -(-wp // r))
    assert lib.dilated_attn_gather_map(N, 4, _native.DaPattern(w, r), 0, None, 0, None,
                                       None) == -1

"""Dilated attention (LongNet) forward and backward passes for AMD MI355X
(gfx950).

Python face of the C-ABI library: ``dilated_attn`` takes projected q, k, v
of shape [B, N, H, 64] (bf16 or fp32, on the GPU) and a list of
(segment length w, dilation r) patterns, and returns (out [B, N, H, 64],
lse [B, H, N] float32); ``dilated_attn_bwd`` takes those plus dout and
returns (dq, dk, dv). All computation happens in the HIP kernels; torch
only allocates memory and supplies the current stream.
"""
from . import _native
from ._native import (DA_BF16, DA_BWD_ALL, DA_BWD_KV, DA_BWD_MERGE, DA_BWD_PREP, DA_BWD_Q, DA_F32,
                      DA_HEAD_DIM, DA_MAX_PATTERNS, DA_NOALLOC_MAX_WORKSPACE_BYTES,
                      DilatedAttnError, bwd_workspace_bytes, load_library, strerror, version,
                      workspace_bytes)

__all__ = [
    "dilated_attn", "dilated_attn_attention_stage", "dilated_attn_merge_stage", "gather_map",
    "coverage_map", "workspace_bytes", "strerror", "version", "load_library", "DilatedAttnError",
    "DA_F32", "DA_BF16", "DA_HEAD_DIM", "DA_MAX_PATTERNS", "Problem", "dilated_attn_bwd",
    "BwdProblem", "bwd_workspace_bytes", "DA_BWD_PREP", "DA_BWD_KV", "DA_BWD_Q", "DA_BWD_MERGE",
    "DA_BWD_ALL", "qk_norm_fwd", "qk_norm_bwd", "qknorm_fused_supported", "dilated_attn_qknorm",
    "dilated_attn_qknorm_bwd", "dilated_attn_onepass", "dilated_attn_noalloc",
    "DA_NOALLOC_MAX_WORKSPACE_BYTES",
]


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return DA_BF16
    if t.dtype == torch.float32:
        return DA_F32
    raise TypeError(f"q, k, v must be bfloat16 or float32, got {t.dtype}")


class Problem:
    """Validated tensors and buffers of one forward call (reusable across
    calls with the same shapes, e.g. in a timing loop)."""

    def __init__(self, q, k, v, patterns, causal=True, scale=None, out=None, lse=None,
                 workspace=None):
        import torch

        for name, t in (("q", q), ("k", k), ("v", v)):
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name} must be a torch.Tensor")
            if t.device.type != "cuda":
                raise ValueError(f"{name} must be on the GPU (got {t.device}); no CPU path exists")
            if t.dim() != 4 or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous [B, N, H, Dh] tensor")
        if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype):
            raise ValueError("q, k, v must share shape and dtype")
        if not (q.device == k.device == v.device):
            raise ValueError("q, k, v must be on one device")
        self.q, self.k, self.v = q, k, v
        self.B, self.N, self.H, self.Dh = (int(x) for x in q.shape)
        self.patterns = [(int(w), int(r)) for (w, r) in patterns]
        self.causal = bool(causal)
        self.scale = float(scale) if scale else 0.0
        self.dtype = _dtype_code(q)
        self._pats = _native.pattern_array(self.patterns)
        ws = workspace_bytes(self.B, self.N, self.H, self.Dh, self.patterns, self.dtype)
        self.out = out if out is not None else torch.empty_like(q)
        self.lse = lse if lse is not None else torch.empty(
            (self.B, self.H, self.N), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=q.device)
        _check_workspace(workspace, q.device)
        self.workspace = workspace
        self.ws_bytes = workspace.numel() * workspace.element_size()
        _check_out("out", self.out, q.shape, q.dtype, q.device)
        _check_out("lse", self.lse, (self.B, self.H, self.N), torch.float32, q.device)

    def _call(self, fn_name, stream=None):
        import torch

        lib = load_library()
        if stream is None:
            stream = torch.cuda.current_stream(self.q.device)
        code = getattr(lib, fn_name)(
            self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.out.data_ptr(),
            self.lse.data_ptr(), self.B, self.N, self.H, self.Dh, self._pats, len(self.patterns),
            1 if self.causal else 0, self.dtype, self.scale, self.workspace.data_ptr(),
            self.ws_bytes, stream.cuda_stream)
        _native.check(code, fn_name)

    def run(self, stream=None):
        self._call("dilated_attn_fwd", stream)
        return self.out, self.lse

    def attention_stage(self, stream=None):
        self._call("dilated_attn_fwd_attention", stream)

    def merge_stage(self, stream=None):
        self._call("dilated_attn_fwd_merge", stream)


class BwdProblem:
    """Validated tensors and buffers of one backward call: q, k, v, out, lse
    as in the forward call, dout like q; dq, dk, dv and the workspace are
    allocated unless given."""

    def __init__(self, q, k, v, out, lse, dout, patterns, causal=True, scale=None, dq=None,
                 dk=None, dv=None, workspace=None):
        import torch

        for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name} must be a torch.Tensor")
            if t.device.type != "cuda":
                raise ValueError(f"{name} must be on the GPU (got {t.device}); no CPU path exists")
            if t.dim() != 4 or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous [B, N, H, Dh] tensor")
            if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
                raise ValueError(f"{name} must match q in shape, dtype and device")
        self.q, self.k, self.v, self.out, self.dout = q, k, v, out, dout
        self.B, self.N, self.H, self.Dh = (int(x) for x in q.shape)
        if (not isinstance(lse, torch.Tensor) or lse.shape != (self.B, self.H, self.N)
                or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device):
            raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
        self.lse = lse
        self.patterns = [(int(w), int(r)) for (w, r) in patterns]
        self.causal = bool(causal)
        self.scale = float(scale) if scale else 0.0
        self.dtype = _dtype_code(q)
        self._pats = _native.pattern_array(self.patterns)
        self.dq = dq if dq is not None else torch.empty_like(q)
        self.dk = dk if dk is not None else torch.empty_like(q)
        self.dv = dv if dv is not None else torch.empty_like(q)
        for name, t in (("dq", self.dq), ("dk", self.dk), ("dv", self.dv)):
            _check_out(name, t, q.shape, q.dtype, q.device)
        ws = bwd_workspace_bytes(self.B, self.N, self.H, self.Dh, self.patterns, self.dtype)
        if workspace is None:
            workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=q.device)
        _check_workspace(workspace, q.device)
        self.workspace = workspace
        self.ws_bytes = workspace.numel() * workspace.element_size()

    def run(self, stages=DA_BWD_ALL, stream=None):
        import torch

        lib = load_library()
        if stream is None:
            stream = torch.cuda.current_stream(self.q.device)
        code = lib.dilated_attn_bwd_stages(
            int(stages), self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(),
            self.out.data_ptr(), self.lse.data_ptr(), self.dout.data_ptr(), self.dq.data_ptr(),
            self.dk.data_ptr(), self.dv.data_ptr(), self.B, self.N, self.H, self.Dh, self._pats,
            len(self.patterns), 1 if self.causal else 0, self.dtype, self.scale,
            self.workspace.data_ptr(), self.ws_bytes, stream.cuda_stream)
        _native.check(code, "dilated_attn_bwd_stages")
        return self.dq, self.dk, self.dv


def dilated_attn_bwd(q, k, v, out, lse, dout, patterns, causal=True, scale=None, dq=None, dk=None,
                     dv=None, workspace=None):
    """Dilated-attention backward. Returns (dq, dk, dv); see include/dilated_attn.h."""
    return BwdProblem(q, k, v, out, lse, dout, patterns, causal, scale, dq, dk, dv,
                      workspace).run()


def dilated_attn(q, k, v, patterns, causal=True, scale=None, out=None, lse=None, workspace=None):
    """Dilated-attention forward. Returns (out, lse); see include/dilated_attn.h."""
    return Problem(q, k, v, patterns, causal, scale, out, lse, workspace).run()


def dilated_attn_onepass(q, k, v, patterns, causal=True, scale=None, out=None, lse=None):
    """The forward in one launch (bf16): every row's covering patterns run
    through one online softmax, no workspace and no merge pass. Returns
    (out, lse); see include/dilated_attn.h."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor; no CPU path exists")
        if t.dim() != 4 or not t.is_contiguous() or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a contiguous [B, N, H, Dh] tensor like q")
    B, N, H, Dh = (int(x) for x in q.shape)
    pats = [(int(w), int(r)) for (w, r) in patterns]
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_out("out", out, q.shape, q.dtype, q.device)
    _check_out("lse", lse, (B, H, N), torch.float32, q.device)
    code = load_library().dilated_attn_fwd_onepass(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, N, H, Dh,
        _native.pattern_array(pats), len(pats), 1 if causal else 0, _dtype_code(q),
        float(scale) if scale else 0.0, torch.cuda.current_stream(q.device).cuda_stream)
    _native.check(code, "dilated_attn_fwd_onepass")
    return out, lse


def dilated_attn_noalloc(q, k, v, patterns, causal=True, scale=None, out=None, lse=None):
    """The forward pass with the workspace taken from the library's own
    per-GPU array (at most DA_NOALLOC_MAX_WORKSPACE_BYTES): the library
    allocates nothing. out and lse must be given to allocate nothing here
    either. Returns (out, lse); see include/dilated_attn.h."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor; no CPU path exists")
        if t.dim() != 4 or not t.is_contiguous() or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a contiguous [B, N, H, Dh] tensor like q")
    B, N, H, Dh = (int(x) for x in q.shape)
    pats = [(int(w), int(r)) for (w, r) in patterns]
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_out("out", out, q.shape, q.dtype, q.device)
    _check_out("lse", lse, (B, H, N), torch.float32, q.device)
    code = load_library().dilated_attn_fwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, N, H, Dh,
        _native.pattern_array(pats), len(pats), 1 if causal else 0, _dtype_code(q),
        float(scale) if scale else 0.0, torch.cuda.current_stream(q.device).cuda_stream)
    _native.check(code, "dilated_attn_fwd_noalloc")
    return out, lse


def dilated_attn_attention_stage(prob, stream=None):
    prob.attention_stage(stream)


def dilated_attn_merge_stage(prob, stream=None):
    prob.merge_stage(stream)


def gather_map(N, H, pattern, h, device="cuda"):
    """Device dump of the gather map: int64 [nseg, lmax], -1 past L(h); the
    library reports the shape."""
    import ctypes

    import torch

    lib = load_library()
    pat = _native.DaPattern(int(pattern[0]), int(pattern[1]))
    shape = (ctypes.c_int64 * 2)()
    code = lib.dilated_attn_gather_map(int(N), int(H), pat, int(h), None, 0, shape, None)
    _native.check(code, "dilated_attn_gather_map")
    nseg, lmax = int(shape[0]), int(shape[1])
    out = torch.empty(max(nseg * lmax, 1), dtype=torch.int64, device=device)
    code = lib.dilated_attn_gather_map(int(N), int(H), pat, int(h), out.data_ptr(), out.numel(),
                                       None, torch.cuda.current_stream(out.device).cuda_stream)
    _native.check(code, "dilated_attn_gather_map")
    return out[:nseg * lmax].view(nseg, lmax)


def coverage_map(N, H, pattern, h, device="cuda"):
    """Device dump of the inverse map: int64 [N], compact index or -1."""
    import torch

    out = torch.empty(max(int(N), 1), dtype=torch.int64, device=device)
    code = load_library().dilated_attn_coverage_map(
        int(N), int(H), _native.DaPattern(int(pattern[0]), int(pattern[1])), int(h),
        out.data_ptr(), out.numel(), torch.cuda.current_stream(out.device).cuda_stream)
    _native.check(code, "dilated_attn_coverage_map")
    return out[:int(N)]


def _check_rows(name, t, like):
    import torch

    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor; no CPU path exists")
    if not t.is_contiguous() or t.dtype != like.dtype or t.device != like.device:
        raise ValueError(f"{name} must be contiguous with q's dtype and device")


def qk_norm_fwd(xq, xk, gain_q, bias_q, gain_k, bias_k, eps=1e-5, yq=None, yk=None):
    """Layer norm of every 64-value row of xq and xk ([..., 64]); see
    include/dilated_attn.h. Returns (yq, yk)."""
    import torch

    for n, t in (("xk", xk), ("gain_q", gain_q), ("bias_q", bias_q), ("gain_k", gain_k),
                 ("bias_k", bias_k)):
        _check_rows(n, t, xq)
    _check_rows("xq", xq, xq)
    if xq.shape != xk.shape or xq.shape[-1] != DA_HEAD_DIM:
        raise ValueError("xq and xk must share a shape ending in 64")
    yq = torch.empty_like(xq) if yq is None else yq
    yk = torch.empty_like(xk) if yk is None else yk
    _check_out("yq", yq, xq.shape, xq.dtype, xq.device)
    _check_out("yk", yk, xk.shape, xk.dtype, xk.device)
    rows = xq.numel() // DA_HEAD_DIM
    code = load_library().dilated_attn_qk_norm_fwd(
        xq.data_ptr(), xk.data_ptr(), gain_q.data_ptr(), bias_q.data_ptr(), gain_k.data_ptr(),
        bias_k.data_ptr(), yq.data_ptr(), yk.data_ptr(), rows, DA_HEAD_DIM, _dtype_code(xq),
        float(eps), torch.cuda.current_stream(xq.device).cuda_stream)
    _native.check(code, "dilated_attn_qk_norm_fwd")
    return yq, yk


def qk_norm_bwd(xq, xk, dyq, dyk, gain_q, gain_k, eps=1e-5):
    """Backward of qk_norm_fwd. Returns (dxq, dxk, dparams) with dparams a
    float32 [2, 2, 64] tensor: [q|k][gain|bias]."""
    import torch

    for n, t in (("xk", xk), ("dyq", dyq), ("dyk", dyk), ("gain_q", gain_q), ("gain_k", gain_k)):
        _check_rows(n, t, xq)
    _check_rows("xq", xq, xq)
    rows = xq.numel() // DA_HEAD_DIM
    dxq, dxk = torch.empty_like(xq), torch.empty_like(xk)
    dparams = torch.empty((2, 2, DA_HEAD_DIM), dtype=torch.float32, device=xq.device)
    ws = torch.empty(max(_native.qk_norm_workspace_bytes(rows), 1), dtype=torch.uint8,
                     device=xq.device)
    code = load_library().dilated_attn_qk_norm_bwd(
        xq.data_ptr(), xk.data_ptr(), dyq.data_ptr(), dyk.data_ptr(), gain_q.data_ptr(),
        gain_k.data_ptr(), dxq.data_ptr(), dxk.data_ptr(), dparams.data_ptr(), rows, DA_HEAD_DIM,
        _dtype_code(xq), float(eps), ws.data_ptr(), ws.numel(),
        torch.cuda.current_stream(xq.device).cuda_stream)
    _native.check(code, "dilated_attn_qk_norm_bwd")
    return dxq, dxk, dparams


def qknorm_fused_supported(B, N, H, patterns, dtype_code):
    """True when dilated_attn_qknorm serves this shape and pattern list (one
    pattern whose segments gather at most 32 rows); asks the library."""
    try:
        _native.bwd_qknorm_workspace_bytes(int(B), int(N), int(H), DA_HEAD_DIM,
                                           [(int(w), int(r)) for (w, r) in patterns],
                                           int(dtype_code))
    except DilatedAttnError as e:
        if e.code == -3:  # DA_ERR_PATTERN
            return False
        raise
    return True


def _check_out(name, t, shape, dtype, device):
    import torch

    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype
            or t.device != device or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}")


def _check_workspace(t, device):
    """The library cannot tell host from device memory: a workspace must be
    a contiguous tensor on the inputs' GPU."""
    import torch

    if not isinstance(t, torch.Tensor) or t.device != device or not t.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")


def _row_stride(named):
    """Common stride (elements) between consecutive positions of [B, N, H,
    Dh] tensors whose [H, Dh] rows are dense, e.g. the three parts
    qkv[:, :, i] of one [B, N, 3, H, Dh] buffer; 0 when they are dense."""
    rs = None
    for name, t in named:
        B, N, H, Dh = t.shape
        ok = t.stride(3) == 1 and t.stride(2) == Dh and (B == 1 or t.stride(0) == N * t.stride(1))
        if not ok or (rs is not None and t.stride(1) != rs):
            raise ValueError(f"{name} must be [B, N, H, Dh] with dense [H, Dh] rows at one common "
                             "stride between positions (e.g. contiguous, or a part of a "
                             "[B, N, 3, H, Dh] buffer)")
        rs = t.stride(1)
    B, N, H, Dh = named[0][1].shape
    return 0 if rs == H * Dh else int(rs)


def _check_fused(xq, xk, v, params):
    import torch

    for name, t in (("xq", xq), ("xk", xk), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor; no CPU path exists")
        if t.dim() != 4:
            raise ValueError(f"{name} must be a [B, N, H, Dh] tensor")
        if t.shape != xq.shape or t.dtype != xq.dtype or t.device != xq.device:
            raise ValueError(f"{name} must match xq in shape, dtype and device")
    for name, t in zip(("gain_q", "bias_q", "gain_k", "bias_k"), params):
        _check_rows(name, t, xq)
        if t.numel() != DA_HEAD_DIM:
            raise ValueError(f"{name} must hold {DA_HEAD_DIM} values")
    return _row_stride((("xq", xq), ("xk", xk), ("v", v)))


def dilated_attn_qknorm(xq, xk, v, gain_q, bias_q, gain_k, bias_k, patterns, eps=1e-5,
                        causal=True, scale=None, out=None, lse=None):
    """Forward of attention over qk_norm(xq), qk_norm(xk), v with the layer
    norm applied inside the attention kernel. Returns (out, lse); one pattern
    with segments of at most 32 gathered rows (see qknorm_fused_supported).
    xq, xk, v may be the parts qkv[:, :, 0..2] of one [B, N, 3, H, Dh]
    buffer; out is a dense [B, N, H, Dh] tensor."""
    import torch

    params = (gain_q, bias_q, gain_k, bias_k)
    rs = _check_fused(xq, xk, v, params)
    B, N, H, Dh = (int(x) for x in xq.shape)
    pats = [(int(w), int(r)) for (w, r) in patterns]
    out = torch.empty((B, N, H, Dh), dtype=xq.dtype, device=xq.device) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=xq.device) if lse is None else lse
    _check_out("out", out, xq.shape, xq.dtype, xq.device)
    _check_out("lse", lse, (B, H, N), torch.float32, xq.device)
    code = load_library().dilated_attn_fwd_qknorm(
        xq.data_ptr(), xk.data_ptr(), v.data_ptr(), *(t.data_ptr() for t in params), float(eps),
        out.data_ptr(), lse.data_ptr(), B, N, H, Dh, rs, _native.pattern_array(pats), len(pats),
        1 if causal else 0, _dtype_code(xq), float(scale) if scale else 0.0,
        torch.cuda.current_stream(xq.device).cuda_stream)
    _native.check(code, "dilated_attn_fwd_qknorm")
    return out, lse


def dilated_attn_qknorm_bwd(xq, xk, v, gain_q, bias_q, gain_k, bias_k, out, lse, dout, patterns,
                            eps=1e-5, causal=True, scale=None, workspace=None, dxq=None,
                            dxk=None, dv=None, dparams=None):
    """Backward of dilated_attn_qknorm. Returns (dxq, dxk, dv, dparams), with
    dparams a float32 [2, 2, 64] tensor: [q|k][gain|bias]. dxq, dxk, dv take
    the layout of xq, xk, v (given ones must match it; allocated ones are
    parts of one [B, N, 3, H, Dh] buffer when xq, xk, v are)."""
    import torch

    params = (gain_q, bias_q, gain_k, bias_k)
    rs = _check_fused(xq, xk, v, params)
    for name, t in (("out", out), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or t.shape != xq.shape or t.dtype != xq.dtype \
                or t.device != xq.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor like xq")
    B, N, H, Dh = (int(x) for x in xq.shape)
    if (not isinstance(lse, torch.Tensor) or lse.shape != (B, H, N) or lse.dtype != torch.float32
            or not lse.is_contiguous() or lse.device != xq.device):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on xq's device")
    pats = [(int(w), int(r)) for (w, r) in patterns]
    dt = _dtype_code(xq)
    if workspace is None:
        ws = _native.bwd_qknorm_workspace_bytes(B, N, H, Dh, pats, dt)
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=xq.device)
    _check_workspace(workspace, xq.device)
    if dxq is None and dxk is None and dv is None:
        if rs == 0:
            dxq, dxk, dv = (torch.empty((B, N, H, Dh), dtype=xq.dtype, device=xq.device)
                            for _ in range(3))
        else:
            if rs >= 3 * H * Dh:  # one buffer, the three interleaved
                g = torch.empty((B, N, rs), dtype=xq.dtype, device=xq.device)
                dxq, dxk, dv = (g[:, :, i * H * Dh:(i + 1) * H * Dh].unflatten(2, (H, Dh))
                                for i in range(3))
            else:  # three buffers of that layout
                dxq, dxk, dv = (torch.empty((B, N, rs), dtype=xq.dtype, device=xq.device)
                                [:, :, :H * Dh].unflatten(2, (H, Dh)) for _ in range(3))
    if dxq is None or dxk is None or dv is None:
        raise ValueError("give all of dxq, dxk, dv or none")
    for name, t in (("dxq", dxq), ("dxk", dxk), ("dv", dv)):
        if (not isinstance(t, torch.Tensor) or t.shape != xq.shape or t.dtype != xq.dtype
                or t.device != xq.device):
            raise ValueError(f"{name} must be a tensor like xq")
    if _row_stride((("dxq", dxq), ("dxk", dxk), ("dv", dv))) != rs:
        raise ValueError("dxq, dxk, dv must have the layout of xq, xk, v")
    if dparams is None:
        dparams = torch.empty((2, 2, DA_HEAD_DIM), dtype=torch.float32, device=xq.device)
    _check_out("dparams", dparams, (2, 2, DA_HEAD_DIM), torch.float32, xq.device)
    code = load_library().dilated_attn_bwd_qknorm(
        xq.data_ptr(), xk.data_ptr(), v.data_ptr(), *(t.data_ptr() for t in params), float(eps),
        out.data_ptr(), lse.data_ptr(), dout.data_ptr(), dxq.data_ptr(), dxk.data_ptr(),
        dv.data_ptr(), dparams.data_ptr(), B, N, H, Dh, rs, _native.pattern_array(pats),
        len(pats), 1 if causal else 0, dt, float(scale) if scale else 0.0, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(),
        torch.cuda.current_stream(xq.device).cuda_stream)
    _native.check(code, "dilated_attn_bwd_qknorm")
    return dxq, dxk, dv, dparams

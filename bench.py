"""Benchmark of the dilated-attention forward (default) or backward pass on
one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]
                    [--pass fwd|bwd|module]

Forward: a step is one whole forward pass (the attention kernel over every
pattern, then the log-sum-exp merge). Backward (--pass bwd): a step is one
whole backward pass (D = dout . out, the dK/dV kernel, the dQ kernel, the
partial sums), given the forward pass's out and lse. Module (--pass module):
a step is one training step of the DilatedAttention module (projections,
qk_norm, attention, output projection; forward, then backward into x and
every parameter) at the README's usage shape. Inputs are resident in
GPU memory. W untimed steps run first; K steps are then timed between two
device synchronisations. Inside the timed region HIP events on the launch
stream bracket every kernel of every step, which gives each kernel's
average launch duration for the roofline figure.

Prints one JSON line. `value` is tokens/s (B * N / step time). `roofline`
reports the dominant kernel (the attention kernel; for the backward pass
the dK/dV kernel) against the bf16 MFMA peak using the algorithmic FLOP
count; `cpu_baseline` times the CPU oracle on a bounded sample of the same
workload on this host's cores.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dilated-attention fwd tokens/sec and % bf16 MFMA peak at N=32K, 1 GPU"
METRIC_BWD = "dilated-attention bwd tokens/sec and % bf16 MFMA peak at N=32K, 1 GPU"
TRAFFIC = {
    "fwd": (os.path.join(ROOT, "profiles", "traffic_attn_fwd_paper_mixture_n32768.json"),
            ["attn_kernel.hip", "da_common.hpp"]),
    "bwd": (os.path.join(ROOT, "profiles", "traffic_bwd_kv_paper_mixture_n32768.json"),
            ["bwd_kernel.hip", "da_common.hpp", "da_bwd.hpp", "da_device.hpp"]),
}


def kernel_source_hash(sources):
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "sparse_long_sequence_attn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(which, workload):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, or None when there is none or the kernel's
    sources changed since."""
    path, sources = TRAFFIC[which]
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("source_sha256") != kernel_source_hash(sources):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_model():
    """The host CPU's model name, as the kernel reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def gpu_max_sclk_mhz(device=0):
    """The device's peak engine clock as the HIP runtime reports it (MHz),
    or None. The published bf16 peak assumes 2400 MHz. Asked in-process (no
    child process, which a profiler would follow)."""
    import ctypes

    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return None
    khz = ctypes.c_int(0)
    # hipDeviceGetAttribute(&value, hipDeviceAttributeClockRate (= 5, kHz), device)
    if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, int(device)) != 0 or khz.value <= 0:
        return None
    return khz.value // 1000


def parity_figures(out_gpu, lse_gpu, out_o, lse_o):
    """Max-abs errors of the GPU result against the oracle's on the same
    elements, the output error in units of the bf16 spacing at the oracle's
    value (2^(floor(log2 |x|) - 7), with |x| floored at 1/16 so that values
    near zero are judged at a fixed absolute scale), and how many oracle
    values have |x| >= 4, where one bf16 spacing (2^-5) already exceeds
    2e-2."""
    import numpy as np

    d = np.abs(out_gpu - out_o)
    mag = np.maximum(np.abs(out_o), 1.0 / 16)
    spacing = np.exp2(np.floor(np.log2(mag)) - 7)
    fin = np.isfinite(lse_o)
    return {
        "max_abs_err_out": float(d.max()),
        "max_err_out_bf16_spacings_min_x_1_16": float((d / spacing).max()),
        "count_abs_oracle_ge_4": int((np.abs(out_o) >= 4).sum()),
        "max_abs_err_lse": float(np.abs(lse_gpu[fin] - lse_o[fin]).max()) if fin.any() else 0.0,
        "lse_inf_match": bool(np.array_equal(np.isfinite(lse_gpu), fin)),
        "elements_compared": int(d.size),
    }


def cpu_baseline(w, heads, out_gpu=None, lse_gpu=None):
    """The oracle (as it stands) on the first `heads` heads of the workload:
    heads are independent, so the full workload costs H / heads times as much.
    With the GPU's out and lse (torch tensors) its result is also compared
    with the oracle's on those heads."""
    import numpy as np

    import oracle
    from sparse_long_sequence_attn_amd.workloads import host_inputs

    q, k, v = host_inputs(w)
    q, k, v = (np.ascontiguousarray(x[:, :, :heads]) for x in (q, k, v))
    t0 = time.perf_counter()
    out_o, lse_o = oracle.fwd(q, k, v, w.patterns, causal=w.causal)
    dt = time.perf_counter() - t0
    full = dt * w.H / heads
    parity = None
    if out_gpu is not None:
        og = out_gpu.float().cpu().numpy().astype(np.float64)[:, :, :heads]
        lg = lse_gpu.cpu().numpy().astype(np.float64)[:, :heads]
        parity = parity_figures(og, lg, out_o, lse_o)
    return {
        "value": w.tokens / full,
        "unit": "tokens/s",
        "cores": oracle.max_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"heads 0-{heads - 1} of {w.H} of the same workload (all {w.B * w.N} tokens, "
                  f"all patterns), fp64 C oracle, {dt:.2f} s measured, scaled by {w.H}/{heads}",
        "oracle_seconds": round(dt, 3),
        "parity_vs_gpu": parity,
    }


def oracle_row_sample(w, per_head):
    """A deterministic row sample of a workload too large for the whole
    oracle: for every head, the first and last gathered position of every
    segment of every pattern, then evenly spaced positions up to `per_head`
    rows. Returns int64 [n, 3] of (b, t, h), batch 0."""
    import numpy as np

    rows = []
    for h in range(w.H):
        ts = set()
        for (pw, r) in w.patterns:
            wp = min(pw, w.N)
            off = h % r
            last = off + ((wp - 1 - off) // r) * r
            starts = np.arange(0, w.N, wp)
            ts.update((starts + off).tolist())
            ts.update((starts + last).tolist())
        fill = per_head - len(ts)
        if fill > 0:
            for t in np.linspace(0, w.N - 1, fill + len(ts)).astype(np.int64).tolist():
                if len(ts) >= per_head:
                    break
                ts.add(int(t))
        rows.extend((0, t, h) for t in sorted(ts))
    return np.array(rows, dtype=np.int64)


def cpu_baseline_sampled(w, q, k, v, per_head, out_gpu=None, lse_gpu=None):
    """The row-wise oracle (as it stands) on a deterministic row sample of a
    device-generated workload, with the time extrapolated linearly to all
    B * N * H rows. With the GPU's out and lse its rows are compared with
    the oracle's at the sampled rows."""
    import numpy as np

    import oracle
    from sparse_long_sequence_attn_amd.workloads import from_torch_bits

    qh, kh, vh = (from_torch_bits(x) for x in (q, k, v))
    rows = oracle_row_sample(w, per_head)
    t0 = time.perf_counter()
    out_o, lse_o = oracle.rows(qh, kh, vh, w.patterns, rows, causal=w.causal)
    dt = time.perf_counter() - t0
    parity = None
    if out_gpu is not None:
        import torch

        idx = torch.as_tensor(rows, device=out_gpu.device)
        og = out_gpu[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy().astype(np.float64)
        lg = lse_gpu[idx[:, 0], idx[:, 2], idx[:, 1]].cpu().numpy().astype(np.float64)
        parity = parity_figures(og, lg, out_o, lse_o)
    total = w.B * w.N * w.H
    full = dt * total / len(rows)
    return {
        "value": w.tokens / full,
        "unit": "tokens/s",
        "cores": oracle.max_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{len(rows)} rows (every head: each pattern's first and last gathered row "
                  f"of every segment, then evenly spaced positions; {per_head} rows per head) "
                  f"of the same workload, fp64 C row-wise oracle, {dt:.2f} s measured; value is "
                  f"a LINEAR EXTRAPOLATION by row count to all {total} rows "
                  f"({full:.0f} s estimated)",
        "oracle_seconds": round(dt, 3),
        "parity_vs_gpu": parity,
    }


def cpu_baseline_bwd(w, heads):
    """The oracle's backward pass (as it stands) on the first `heads` heads."""
    import numpy as np

    import oracle
    from sparse_long_sequence_attn_amd.workloads import host_inputs, workload_grad_output

    q, k, v = host_inputs(w)
    d = workload_grad_output(w)
    q, k, v, d = (np.ascontiguousarray(x[:, :, :heads]) for x in (q, k, v, d))
    t0 = time.perf_counter()
    oracle.bwd(q, k, v, d, w.patterns, causal=w.causal)
    dt = time.perf_counter() - t0
    full = dt * w.H / heads
    return {
        "value": w.tokens / full,
        "unit": "tokens/s",
        "cores": oracle.max_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"backward, heads 0-{heads - 1} of {w.H} of the same workload (all "
                  f"{w.B * w.N} tokens, all patterns), fp64 C oracle, {dt:.2f} s measured, "
                  f"scaled by {w.H}/{heads}",
    }


def run_bwd(args, w, dev, q, k, v):
    import torch

    from sparse_long_sequence_attn_amd import (DA_BWD_KV, DA_BWD_MERGE, DA_BWD_PREP, DA_BWD_Q,
                                               BwdProblem, Problem)
    from sparse_long_sequence_attn_amd.costs import PEAK_HBM_GBS, bwd_cost, peak_tflops
    from sparse_long_sequence_attn_amd.workloads import to_torch, workload_grad_output

    if w.device_generated:
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed + 100_000)
        dout = torch.randn(q.shape, generator=g, device=dev, dtype=torch.float32).to(q.dtype)
    else:
        dout = to_torch(workload_grad_output(w), dev)
    fwd = Problem(q, k, v, w.patterns, w.causal)
    fwd.run()
    bp = BwdProblem(q, k, v, fwd.out, fwd.lse, dout, w.patterns, w.causal)
    stream = torch.cuda.current_stream(dev)
    stages = (DA_BWD_PREP, DA_BWD_KV, DA_BWD_Q, DA_BWD_MERGE)
    for _ in range(args.warmup):
        for st in stages:
            bp.run(st, stream)
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        for j, st in enumerate(stages):
            bp.run(st, stream)
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
    names = ["prep", "kv", "q", "merge"]
    kms = {n: sum(e[j].elapsed_time(e[j + 1]) for e in ev) / K for j, n in enumerate(names)}

    c = bwd_cost(w.B, w.N, w.H, w.Dh, w.patterns, w.causal, 2 if w.dtype == "bf16" else 4)
    peak = peak_tflops(w.dtype)
    kv_tflops = c.flops_kv / (kms["kv"] / 1e3) / 1e12
    q_tflops = c.flops_q / (kms["q"] / 1e3) / 1e12
    step_tflops = c.flops_alg / (ms_step / 1e3) / 1e12
    # short segments (the usage shape: 32 rows) leave the products tiny and
    # the kernel bound by its row traffic
    mfma_bound = len(w.patterns) > 1 or max(
        -(-min(pw, w.N) // r) for pw, r in w.patterns) > 256
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(kv_tflops, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(kv_tflops / peak, 4)}
    else:
        gbs = c.kv_bytes / (kms["kv"] / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    roof.update({"traffic": measured_traffic("bwd", w.name),
                 "kernel": "bwd_short_kernel" if c.fused else "bwd_kv_kernel",
                 "kernel_ms": round(kms["kv"], 4)})
    result = {
        "metric": METRIC_BWD,
        "value": round(w.tokens / (ms_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal q, k, v, dout; see workloads.py)",
        "config": {"workload": w.name, "pass": "bwd", "B": w.B, "N": w.N, "H": w.H, "Dh": w.Dh,
                   "patterns": [list(p) for p in w.patterns], "causal": w.causal,
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "single GPU"},
        "roofline": roof,
        "detail": {
            "kernel_ms": {n: round(x, 4) for n, x in kms.items()},
            "tflops_kv_kernel": round(kv_tflops, 2),
            "tflops_q_kernel": None if c.fused else round(q_tflops, 2),
            "pct_bf16_peak_q_kernel": None if c.fused else round(100 * q_tflops / peak, 2),
            "tflops_algorithmic_step": round(step_tflops, 2),
            "pct_bf16_peak_algorithmic_step": round(100 * step_tflops / peak, 2),
            "flops_algorithmic": c.flops_alg,
            "flops_kv_kernel": c.flops_kv,
            "flops_q_kernel": c.flops_q,
            "gbs_prep": None if c.fused else round(c.prep_bytes / (kms["prep"] / 1e3) / 1e9, 1),
            "fused_short_segments": c.fused,
            "gbs_merge": round(c.merge_bytes / (kms["merge"] / 1e3) / 1e9, 1)
            if c.merge_bytes > 0 else None,
            "kv_algorithmic_bytes": c.kv_bytes,
            "gbs_kv_algorithmic": round(c.kv_bytes / (kms["kv"] / 1e3) / 1e9, 1),
            "q_algorithmic_bytes": c.q_bytes,
            "device": torch.cuda.get_device_name(dev),
        },
    }
    if not args.no_cpu_baseline and not w.device_generated:
        result["cpu_baseline"] = cpu_baseline_bwd(w, min(args.cpu_heads, w.H))
    print(json.dumps(result), flush=True)


MODULE_CONFIG = {"workload": "readme_module_b32_n8192_d512_h8_w64r2_qknorm_bf16", "B": 32,
                 "N": 8192, "dim": 512, "heads": 8, "segment_size": 64, "dilation_rate": 2,
                 "qk_norm": True, "causal": True, "seed": 400}
METRIC_MODULE = "DilatedAttention module fwd+bwd tokens/sec, README usage shape, 1 GPU"


def run_module(args, dev):
    """One training step of the DilatedAttention module (forward, then
    backward into x and every parameter) at the README's usage shape."""
    import torch

    from sparse_long_sequence_attn_amd._native import bwd_qknorm_workspace_bytes
    from sparse_long_sequence_attn_amd.costs import PEAK_HBM_GBS, bwd_cost, cost
    from sparse_long_sequence_attn_amd.module import DilatedAttention
    from sparse_long_sequence_attn_amd.workloads import module_params, module_x

    c = MODULE_CONFIG
    B, N, dim, heads = c["B"], c["N"], c["dim"], c["heads"]
    mod = DilatedAttention(dim, heads, c["dilation_rate"], c["segment_size"], qk_norm=c["qk_norm"],
                           causal=c["causal"], device=dev, dtype=torch.bfloat16)
    named = dict(mod.named_parameters())
    names = {"wq": "to_q.weight", "wk": "to_k.weight", "wv": "to_v.weight", "wo": "to_out.weight",
             "q_gain": "q_norm.weight", "q_bias": "q_norm.bias", "k_gain": "k_norm.weight",
             "k_bias": "k_norm.bias"}
    with torch.no_grad():
        for k, v in module_params(dim, heads, c["qk_norm"], False, c["seed"]).items():
            if v is not None:
                named[names[k]].copy_(torch.from_numpy(v))
    x = torch.from_numpy(module_x(B, N, dim, c["seed"] + 1)).to(dev, torch.bfloat16)
    x.requires_grad_()
    # the projections are library GEMMs; PyTorch's TunableOp times the
    # library's candidate kernels for each GEMM shape on first use (here in
    # the untimed warm-up steps) and keeps the fastest
    tuning = args.gemm_tuning == "on" and hasattr(torch.cuda, "tunable")
    if tuning:
        import tempfile

        torch.cuda.tunable.set_filename(os.path.join(tempfile.gettempdir(),
                                                     "dilated_attn_tunableop.csv"))
        torch.cuda.tunable.enable(True)
        torch.cuda.tunable.tuning_enable(True)
    dy = torch.from_numpy(module_x(B, N, dim, c["seed"] + 2)).to(dev, torch.bfloat16)
    stream = torch.cuda.current_stream(dev)

    def step():
        mod.zero_grad(set_to_none=True)
        x.grad = None
        mod(x).backward(dy)

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    if tuning:
        torch.cuda.tunable.tuning_enable(False)  # the choices are fixed from here on
    K = args.steps
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K

    # the library's kernels on the step's own shapes, timed alone: with
    # qk_norm fused (one pattern of at most 32 rows per segment) the two
    # fused calls, else the attention passes on normalised q and k
    from sparse_long_sequence_attn_amd import (BwdProblem, Problem, dilated_attn_qknorm,
                                               dilated_attn_qknorm_bwd, qk_norm_fwd)

    fused = mod._fused(x, B, N)
    pats = list(mod.patterns)
    with torch.no_grad():
        shape = (B, N, heads, 64)
        xq, xk = mod.to_q(x).view(shape), mod.to_k(x).view(shape)
        v = mod.to_v(x).view(shape).contiguous()
        gb = (mod.q_norm.weight, mod.q_norm.bias, mod.k_norm.weight, mod.k_norm.bias)
        dout = torch.randn_like(v)
        if fused:
            out, lse = dilated_attn_qknorm(xq, xk, v, *gb, pats, mod.q_norm.eps)
            ws = torch.empty(max(bwd_qknorm_workspace_bytes(B, N, heads, 64, pats, 1), 1),
                             dtype=torch.uint8, device=dev)
            grads = [torch.empty_like(v) for _ in range(3)]
            dpar = torch.empty((2, 2, 64), dtype=torch.float32, device=dev)

            def run_fwd():
                dilated_attn_qknorm(xq, xk, v, *gb, pats, mod.q_norm.eps, out=out, lse=lse)

            def run_bwd():
                dilated_attn_qknorm_bwd(xq, xk, v, *gb, out, lse, dout, pats, mod.q_norm.eps,
                                        workspace=ws, dxq=grads[0], dxk=grads[1], dv=grads[2],
                                        dparams=dpar)
        else:
            q, k = qk_norm_fwd(xq, xk, *gb, mod.q_norm.eps) if c["qk_norm"] else (xq, xk)
            fp = Problem(q, k, v, pats)
            fp.run()
            bp = BwdProblem(q, k, v, fp.out, fp.lse, dout, pats)

            def run_fwd():
                fp.attention_stage(stream)

            def run_bwd():
                bp.run(stream=stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for _ in range(3):
        run_fwd()
        run_bwd()
    reps = max(K, 10)
    ev[0].record(stream)
    for _ in range(reps):
        run_fwd()
    ev[1].record(stream)
    for _ in range(reps):
        run_bwd()
    ev[2].record(stream)
    torch.cuda.synchronize()
    attn_ms = ev[0].elapsed_time(ev[1]) / reps
    bwd_ms = ev[1].elapsed_time(ev[2]) / reps
    fc = cost(B, N, heads, 64, pats, c["causal"], 2)
    bc = bwd_cost(B, N, heads, 64, pats, c["causal"], 2)
    gbs = fc.attn_bytes / (attn_ms / 1e3) / 1e9
    proj_flops = 2.0 * B * N * dim * dim * 4 * 3  # four projections, forward + two backward GEMMs
    result = {
        "metric": METRIC_MODULE,
        "value": round(B * N / (ms_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal x, dy and weights; see workloads.py)",
        "config": dict(c, **{"pass": "module fwd+bwd", "global_batch": B, "seq_len": N,
                             "parallelism": "single GPU"}),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": ("attn_fwd_kernel with qk_norm fused (on the module's xq, xk, v)"
                                if fused else "attn_fwd_kernel (on the module's q, k, v)"),
                     "kernel_ms": round(attn_ms, 4)},
        "detail": {
            "attention_fwd_ms": round(attn_ms, 4),
            "attention_bwd_ms": round(bwd_ms, 4),
            "attention_share_of_step": round((attn_ms + bwd_ms) / ms_step, 4),
            "qk_norm": ("fused into the attention kernels" if fused else
                        "separate layer-norm kernels" if c["qk_norm"] else "off"),
            "attention_bwd_algorithmic_bytes": bc.kv_bytes + bc.q_bytes + bc.prep_bytes +
            bc.merge_bytes,
            "projection_gemm_flops": proj_flops,
            "gemm_selection": "torch TunableOp, tuned in the warm-up steps" if tuning
            else "library default",
            "device": torch.cuda.get_device_name(dev),
        },
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="paper_mixture_n32768_h16_bf16")
    ap.add_argument("--cpu-heads", type=int, default=16,
                    help="heads of the workload the CPU oracle is timed on")
    ap.add_argument("--cpu-rows-per-head", type=int, default=32768,
                    help="rows per head of the CPU oracle's sample on device-generated "
                         "workloads (the million-token one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd", "module"], default="fwd")
    ap.add_argument("--gemm-tuning", choices=["on", "off"], default="on",
                    help="module pass: let PyTorch's TunableOp pick the projection GEMM kernels")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="after the timed region, run one device copy of this many MiB "
                         "(a known-size kernel for scaling rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the method's sequence-parallel split across GPUs is not built).", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_long_sequence_attn_amd import Problem
    from sparse_long_sequence_attn_amd.costs import PEAK_HBM_GBS, cost, peak_tflops
    from sparse_long_sequence_attn_amd.workloads import WORKLOADS, device_inputs, host_inputs, to_torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.which == "module":
        run_module(args, dev)
        return
    w = WORKLOADS[args.workload]
    if w.device_generated:
        q, k, v = device_inputs(w)
    else:
        q, k, v = (to_torch(x, dev) for x in host_inputs(w))
    if args.which == "bwd":
        run_bwd(args, w, dev, q, k, v)
        return
    prob = Problem(q, k, v, w.patterns, w.causal)
    stream = torch.cuda.current_stream(dev)

    for _ in range(args.warmup):
        prob.attention_stage(stream)
        prob.merge_stage(stream)
    torch.cuda.synchronize()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        prob.attention_stage(stream)
        ev[i][1].record(stream)
        prob.merge_stage(stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_step = (t1 - t0) * 1e3 / K
    attn_times = sorted(e[0].elapsed_time(e[1]) for e in ev)
    merge_times = sorted(e[1].elapsed_time(e[2]) for e in ev)
    step_times = sorted(e[0].elapsed_time(e[2]) for e in ev)
    attn_ms = sum(attn_times) / K
    merge_ms = sum(merge_times) / K

    # the same call with the caches flushed first: a 1 GiB write before each
    # rep evicts the inputs from L2 and the 256 MB Infinity Cache (the
    # workload's q, k, v would otherwise stay resident between reps)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    reps = min(K, 20)
    fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for i in range(reps):
        flush.fill_(i & 0xFF)
        fev[i][0].record(stream)
        prob.attention_stage(stream)
        prob.merge_stage(stream)
        fev[i][1].record(stream)
    torch.cuda.synchronize()
    flushed = sorted(a.elapsed_time(b) for a, b in fev)
    del flush
    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    # practical MFMA ceiling of this GPU for context: a dense bf16 matmul
    a_m = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b_m = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a_m, b_m)
    mev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    mev[0].record(stream)
    for _ in range(10):
        torch.matmul(a_m, b_m)
    mev[1].record(stream)
    torch.cuda.synchronize()
    matmul_tflops = 2.0 * 8192 ** 3 / (mev[0].elapsed_time(mev[1]) / 10 / 1e3) / 1e12
    del a_m, b_m

    # the one-pass variant (one launch, every covering pattern in one online
    # softmax, no merge pass) on the same inputs, for comparison
    onepass_ms = None
    if w.dtype == "bf16" and len(w.patterns) > 1:
        from sparse_long_sequence_attn_amd import DilatedAttnError, dilated_attn_onepass

        o1, l1 = torch.empty_like(q), torch.empty_like(prob.lse)
        try:
            for _ in range(3):
                dilated_attn_onepass(q, k, v, w.patterns, w.causal, out=o1, lse=l1)
            oev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(10)]
            for e0, e1 in oev:
                e0.record(stream)
                dilated_attn_onepass(q, k, v, w.patterns, w.causal, out=o1, lse=l1)
                e1.record(stream)
            torch.cuda.synchronize()
            onepass_ms = sorted(a.elapsed_time(b) for a, b in oev)[5]
        except DilatedAttnError:  # the pattern list has no one-pass form
            onepass_ms = None
        del o1, l1

    c = cost(w.B, w.N, w.H, w.Dh, w.patterns, w.causal, 2 if w.dtype == "bf16" else 4)
    tokens_s = w.tokens / (ms_step / 1e3)
    peak = peak_tflops(w.dtype)
    attn_tflops = c.flops_alg / (attn_ms / 1e3) / 1e12
    step_tflops_alg = c.flops_alg / (ms_step / 1e3) / 1e12
    step_tflops_ns = c.flops_ns / (ms_step / 1e3) / 1e12
    mfma_bound = len(w.patterns) > 1 or max(
        -(-min(pw, w.N) // r) for pw, r in w.patterns) > 256
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4)}
    else:
        gbs = c.attn_bytes / (attn_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    roof["traffic"] = measured_traffic("fwd", w.name)
    roof["kernel"] = "attn_fwd_kernel"
    roof["kernel_ms"] = round(attn_ms, 4)
    # the published peak's clock, checked against the agent's own figure
    sclk = gpu_max_sclk_mhz(dev.index or 0)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    result = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal q, k, v; see workloads.py)",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "H": w.H, "Dh": w.Dh,
                   "patterns": [list(p) for p in w.patterns], "causal": w.causal,
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "single GPU"},
        "roofline": roof,
        "detail": {
            "tflops_algorithmic_step": round(step_tflops_alg, 2),
            "tflops_nominal_count_step": round(step_tflops_ns, 2),
            "pct_bf16_peak_algorithmic_step": round(100 * step_tflops_alg / peak, 2),
            "pct_bf16_peak_nominal_count_step": round(100 * step_tflops_ns / peak, 2),
            "flops_algorithmic": c.flops_alg,
            "flops_nominal_count": c.flops_ns,
            "bf16_matmul_8192_tflops": round(matmul_tflops, 1),
            "attn_frac_of_bf16_matmul": round(attn_tflops / matmul_tflops, 4),
            "step_ms_median": round(step_times[K // 2], 4),
            "flushed_step_ms_median": round(flushed[reps // 2], 4),
            "flushed_tokens_per_s": round(w.tokens / (flushed[reps // 2] / 1e3), 1),
            "attn_kernel_ms": round(attn_ms, 4),
            "attn_kernel_ms_median": round(attn_times[K // 2], 4),
            "merge_kernel_ms": round(merge_ms, 4),
            "merge_kernel_ms_median": round(merge_times[K // 2], 4),
            "attn_algorithmic_bytes": c.attn_bytes,
            "attn_gbs_algorithmic": round(c.attn_bytes / (attn_ms / 1e3) / 1e9, 1),
            "merge_algorithmic_bytes": c.merge_bytes,
            "merge_gbs_algorithmic": round(c.merge_bytes / (merge_ms / 1e3) / 1e9, 1)
            if merge_ms > 0 and c.merge_bytes > 0 else None,
            "onepass_step_ms_median": round(onepass_ms, 4) if onepass_ms else None,
            "onepass_tflops_algorithmic": round(c.flops_alg / (onepass_ms / 1e3) / 1e12, 2)
            if onepass_ms else None,
            "device": torch.cuda.get_device_name(dev),
            "max_sclk_mhz": sclk,
            "bf16_peak_at_max_sclk_tflops": round(cus * 4096 * sclk * 1e6 / 1e12, 1)
            if sclk else None,
        },
    }
    if not args.no_cpu_baseline:
        # the last timed forward's out and lse are compared with the oracle's
        if w.device_generated:
            result["cpu_baseline"] = cpu_baseline_sampled(w, q, k, v, args.cpu_rows_per_head,
                                                          prob.out, prob.lse)
        else:
            result["cpu_baseline"] = cpu_baseline(w, min(args.cpu_heads, w.H), prob.out, prob.lse)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

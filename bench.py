#!/usr/bin/env python3
"""Throughput of the group-sparse SwiGLU hot path on one MI355X.

One step is the whole path over one batch of seeded synthetic input already
resident in HBM: grouped top-k selection (with per-group counts), the forward
(CSR bucketing, fused grouped GEMMs, slot-order sum), the backward (dh+dx,
dW) and the load-balance bias update from the step's counts.

Prints ONE JSON line.  ``value`` is tokens per second of the whole step.  The
``roofline`` object describes the kernel that takes the most time in the step:
algorithmic FLOPs per launch divided by its average duration, measured with
HIP events on its launch stream over a second timed region of the same number
of eagerly launched steps (the headline steps replay one captured HIP graph).
``cpu_baseline`` is
the CPU oracle timed on this host's cores on a bounded slice of the same
workload.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload s1p3b_bf16]
    python bench.py --k-sweep          # tokens/s against the active fraction k*gs/d_ff
    python bench.py --skew             # 4 groups made hot by the bias
    python bench.py --peak             # measured bf16 MFMA and GEMM rates
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "sparse SwiGLU fwd+bwd tokens/s and active-FLOP MFMA % of bf16 peak"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # MI355X dense MFMA (fp32: vector/MFMA fp32 peak)
HBM_GBS = 8000.0

# per-kernel algorithmic work (FLOPs) per launch, in units of (tokens of the
# launch)*k*gs*d.  The dense backward recomputes gate/up (4 units per token in
# dense_rec) without credit: only its dA product (2 units) is the method's.
KERNEL_FLOP_UNITS = {"fwd_grouped": 6, "bwd_dh_dx": 6, "bwd_dw": 6,
                     "dense_fwd": 6, "dense_rec": 2, "dense_dx": 4, "dense_dw": 6}
DENSE_CHUNK_TOKENS = 8192   # token chunk of the dense backward (one launch each of rec/dx/dw)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="s1p3b_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-oracle time budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true", help="skip the per-kernel HIP events")
    ap.add_argument("--backward-streams", choices=["auto", "1", "2"], default="auto",
                    help="1: the weight gradients follow the dx sum on the step's stream; 2: they run on a second "
                         "stream beside it (esg_sparse_swiglu_bwd_overlap); auto: both step graphs are captured, "
                         "timed for a few replays each, and the faster one is timed (the line reports the choice)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of replaying the step as one HIP graph")
    ap.add_argument("--inference", action="store_true",
                    help="forward only (selection + forward, nothing saved): tokens/s of serving steps")
    ap.add_argument("--routing", default=None, metavar="WORKLOAD",
                    help="time sigmoid top-k routing on a routing workload (route_e256_k8, route_e43_k11) instead")
    ap.add_argument("--mlp", default=None, metavar="WORKLOAD",
                    help="time the LeakyReLU(0.5)^2 MLP fwd+bwd on an MLP workload (leaky_mlp_d512) instead")
    ap.add_argument("--mhffn", default=None, metavar="WORKLOAD",
                    help="time the FlashFFN multi-head sub-network core (mhffn1p3b) instead")
    ap.add_argument("--k-sweep", default=None, nargs="?", const="1,4,8,11,22,43", metavar="KS",
                    help="time the step of --workload's shape for each k in KS (comma list)")
    ap.add_argument("--skew", action="store_true",
                    help="the load-balance bias makes 4 groups hot (+10 on groups 0, G/4, G/2, 3G/4)")
    ap.add_argument("--peak", action="store_true", help="only measure the bf16 MFMA probe and a bf16 GEMM")
    ap.add_argument("--no-peak-probe", action="store_true", help="skip the MFMA probe in the main line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run one device-to-device copy of MIB MiB (reference for the HBM counters)")
    return ap.parse_args()


def dataclasses_replace(obj, **kw):
    import dataclasses
    return dataclasses.replace(obj, **kw)


def kernel_source_digest(kernel: str) -> str:
    """sha256 over the shared HIP headers and the sources that launch `kernel` (by its timing name):
    traffic counters apply only to the code they were taken on."""
    import hashlib
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "group_sparse_swiglu_amd", "csrc")
    h = hashlib.sha256()
    tag = ('"' + kernel + '"').encode()
    for name in sorted(os.listdir(root)):
        with open(os.path.join(root, name), "rb") as f:
            text = f.read()
        if name.endswith(".hpp") or (name.endswith(".hip") and tag in text):
            h.update(name.encode() + b"\0" + text)
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from profiles/hbm_traffic_<workload>.md (FETCH_SIZE + WRITE_SIZE
    per dispatch, scaled by the copy-kernel calibration), or None when absent or taken on other sources."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    digest = kernel_source_digest(kernel)
    for line in open(path):
        cells = [c.strip().strip("`") for c in line.strip().strip("|").split("|")]
        if len(cells) >= 5 and cells[0] == kernel and cells[1] == digest:
            try:
                return float(cells[4])
            except ValueError:
                return None
    return None


def copy_calibration(mib: int):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n}), flush=True)


def host_threads() -> int:
    """The host cores this process may use; numpy's BLAS and torch are pinned
    to that many threads for the CPU baseline."""
    n = len(os.sched_getaffinity(0))
    try:
        import torch
        torch.set_num_threads(n)
    except Exception:  # pragma: no cover
        pass
    return n


def cpu_baseline(w, inp, seconds):
    """The CPU oracle (as it stands) in float32, dense-masked, on consecutive
    token slices of the same inputs until `seconds` have passed: selection,
    forward, backward and the bias update per slice, with numpy's BLAS on all
    the host cores this process may use."""
    import numpy as np
    from oracle import esg_oracle as O
    cores = host_threads()
    try:
        from threadpoolctl import threadpool_limits
        limits = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        limits = None
    x, wg, wu, wd, dy, bias, sub = inp
    f32 = lambda t: t.float().numpy()
    W = (f32(wg), f32(wu), f32(wd))
    subn = None if sub is None else sub.numpy()
    biasn = None if bias is None else bias.numpy()
    G = w.groups
    slice_tokens = min(1024, w.tokens)
    ema = np.full(G, w.k / G, dtype=np.float32)
    b = np.zeros(G, dtype=np.float32) if biasn is None else biasn.astype(np.float32)
    done, t0 = 0, time.perf_counter()
    while True:
        s0 = done % w.tokens
        xs, dys = f32(x[s0:s0 + slice_tokens]), f32(dy[s0:s0 + slice_tokens])
        if w.dense:
            idx = np.tile(np.arange(G, dtype=np.int32), (xs.shape[0], 1))
        else:
            idx, _ = O.grouped_topk_select(xs, W[0], w.group_size, w.k, subn, w.spg, b, dtype=np.float32)
        O.sparse_swiglu_forward(xs, *W, idx, w.group_size, dtype=np.float32)
        O.sparse_swiglu_backward(dys, xs, *W, idx, w.group_size, dtype=np.float32)
        if w.bias_update:
            cur = O.frequency_from_counts(O.group_counts(idx, G), xs.shape[0], np.float32)
            b, ema = O.update_load_balance_bias(b, ema, cur, w.k / G, 1e-3, 0.5, 0.99, np.float32)
        done += xs.shape[0]
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    if limits is not None:
        limits.restore_original_limits()
    return {"value": done / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} tokens of {w.name} in slices of {slice_tokens} (fp32 dense-masked "
                      f"{'fwd+bwd' if w.dense else 'select+fwd+bwd'}"
                      f"{'+bias update' if w.bias_update else ''}, numpy BLAS on {cores} threads), {el:.1f} s"}


def mfma_probe_tflops(dev, reps: int = 5) -> float:
    """Measured bf16 matrix-core rate: the library's probe kernel (eight
    independent 16x16x32 MFMAs per wave and iteration, register operands, no
    memory traffic) over 2048 workgroups of 4 waves, best of `reps` runs."""
    import torch
    import group_sparse_swiglu_amd as E
    blocks, iters = 2048, 20000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    E.mfma_rate_probe(blocks, 100, out)   # warm-up
    torch.cuda.synchronize()
    flops = float(blocks) * 4 * iters * 8 * 16 * 16 * 32 * 2
    best = 0.0
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        E.mfma_rate_probe(blocks, iters, out)
        b.record()
        b.synchronize()
        best = max(best, flops / (a.elapsed_time(b) * 1e-3) / 1e12)
    return best


def gemm_tflops(dev, n: int = 8192, reps: int = 20) -> float:
    """bf16 GEMM rate of the platform library (torch.matmul -> hipBLASLt),
    [n, n] x [n, n], average over `reps` calls after a warm-up."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(0)
    A = torch.randn(n, n, generator=g).to(dev, torch.bfloat16)
    B = torch.randn(n, n, generator=g).to(dev, torch.bfloat16)
    for _ in range(3):
        torch.matmul(A, B)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        torch.matmul(A, B)
    b.record()
    b.synchronize()
    return 2.0 * n ** 3 * reps / (a.elapsed_time(b) * 1e-3) / 1e12


def peak_main(args):
    import torch
    import group_sparse_swiglu_amd as E
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    E.lib()
    probe = mfma_probe_tflops(dev)
    gemm = gemm_tflops(dev)
    print(json.dumps({"metric": "measured bf16 MFMA rate", "value": round(probe, 1), "unit": "TFLOP/s",
                      "spec_peak": PEAK_TFLOPS["bf16"], "probe_frac_of_spec": round(probe / PEAK_TFLOPS["bf16"], 4),
                      "hipblaslt_gemm_8192_tflops": round(gemm, 1),
                      "gemm_frac_of_spec": round(gemm / PEAK_TFLOPS["bf16"], 4),
                      "probe": "2048 workgroups x 4 waves x 20000 iterations x 8 v_mfma_f32_16x16x32_bf16, "
                               "register operands, best of 5", "n_gpus": 1}), flush=True)


def routing_cpu_baseline(logits, bias, k, scaling, seconds):
    """The routing oracle (as it stands: a Python loop over rows, one core)
    on consecutive rows of the same logits until `seconds` have passed."""
    from oracle import routing_oracle as R
    ln, bn = logits.numpy(), bias.numpy()
    rows, done, t0 = 256, 0, time.perf_counter()
    while True:
        s0 = done % ln.shape[0]
        R.sigmoid_topk_routing(ln[s0:s0 + rows], bn, k, scaling)
        done += min(rows, ln.shape[0] - s0)
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(done / el, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} rows of the same logits in slices of {rows}, {el:.1f} s"}


def routing_main(args):
    """Sigmoid top-k routing alone: one launch per step over [tokens, experts]
    fp32 logits resident in HBM."""
    import torch
    import esg_inputs as I
    import group_sparse_swiglu_amd as E

    w = I.ROUTING_WORKLOADS[args.routing]
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    E.lib()
    logits, bias = I.make_routing_inputs(w.tokens, w.experts, seed=0)
    L, B = logits.to(dev), bias.to(dev)
    P = torch.empty(w.tokens, w.k, dtype=torch.float32, device=dev)
    IX = torch.empty(w.tokens, w.k, dtype=torch.int64, device=dev)

    def step():
        E.sigmoid_topk_routing(L, B, w.k, w.scaling, out=(P, IX))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay() if graph is not None else step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = 1e3 * elapsed / args.steps

    roofline = None
    if not args.no_kernel_timing:
        E.timing_reset()
        E.timing_enable(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        ms, n = E.timing_read("sigmoid_topk")
        E.timing_enable(False)
        E.timing_reset()
        avg_us = 1e3 * ms / n
        # algorithmic bytes: read the logits and the bias, write fp32 weights and int64 indices
        nbytes = w.tokens * (w.experts * 4 + w.k * 12) + w.experts * 4
        achieved = nbytes / (avg_us * 1e-6) / 1e9
        roofline = {"kernel": "sigmoid_topk", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_GBS, 4),
                    "traffic": recorded_traffic(w.name, "sigmoid_topk"), "bytes_per_launch": nbytes,
                    "avg_launch_us": round(avg_us, 2)}
    line = {
        "metric": "sigmoid top-k routing tokens/s",
        "value": round(w.tokens / (elapsed / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "experts": w.experts, "k": w.k,
                   "scaling_factor": w.scaling, "step": "sigmoid top-k routing"},
        "launch": "hip_graph_replay" if graph is not None else "eager",
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = routing_cpu_baseline(logits, bias, w.k, w.scaling, min(args.cpu_seconds, 10.0))
    print(json.dumps(line), flush=True)


MLP_KERNELS = ("mlp_up_act", "mlp_down", "mlp_dpre", "mlp_dx", "mlp_dw_down", "mlp_dw_up", "mlp_dw_reduce")


def mlp_cpu_baseline(x, wu, wd, dy, seconds):
    """The MLP oracle (fp64 numpy, as it stands) on consecutive token slices
    of the same inputs until `seconds` have passed: forward and backward."""
    import numpy as np
    from oracle import mlp_oracle as M
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 0) for p in threadpool_info()] or [0]) or os.cpu_count()
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    f64 = lambda t: t.float().numpy().astype(np.float64)
    W = (f64(wu), f64(wd))
    rows, done, t0 = 512, 0, time.perf_counter()
    while True:
        s0 = done % x.shape[0]
        xs, dys = f64(x[s0:s0 + rows]), f64(dy[s0:s0 + rows])
        _, post, ag = M.mlp_forward(xs, *W)
        M.mlp_backward(dys, xs, *W, post, ag)
        done += xs.shape[0]
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(done / el, 1), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} tokens in slices of {rows} (fp64 fwd+bwd), {el:.1f} s"}


def mlp_main(args):
    """LeakyReLU(0.5)^2 MLP: forward (fused up projection + activation, down
    projection) and backward (fused dpre, dx, both weight gradients) per step."""
    import torch
    import esg_inputs as I
    import group_sparse_swiglu_amd as E

    w = I.MLP_WORKLOADS[args.mlp]
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    E.lib()
    x, wu, wd, dy = I.make_mlp_inputs(w.tokens, w.d_model, w.d_ff, seed=0)
    X, WU, WD, DY = (t.to(dev) for t in (x, wu, wd, dy))
    sv, _ = E.leaky_mlp_workspace_size(w.tokens, w.d_model, w.d_ff)
    SAVED = torch.empty(sv, dtype=torch.uint8, device=dev)
    Y = torch.empty_like(X)
    GR = (torch.empty_like(X), torch.empty_like(WU), torch.empty_like(WD))
    ws = {}

    def step():
        E.leaky_mlp_fwd(X, WU, WD, out=Y, saved=SAVED)
        E.leaky_mlp_bwd(DY, X, WU, WD, SAVED, workspace=ws, outs=GR)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay() if graph is not None else step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = 1e3 * elapsed / args.steps
    gemm_flops = 2.0 * w.tokens * w.d_model * w.d_ff
    active = 6 * gemm_flops
    peak = PEAK_TFLOPS["bf16"]
    per_kernel, roofline = {}, None
    if not args.no_kernel_timing:
        E.timing_reset()
        E.timing_enable(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        for k in MLP_KERNELS:
            ms, n = E.timing_read(k)
            if n:
                per_kernel[k] = {"avg_us": 1e3 * ms / n, "us_per_step": 1e3 * ms / args.steps}
        E.timing_enable(False)
        E.timing_reset()
        gemms = [k for k in per_kernel if k != "mlp_dw_reduce"]
        dom = max(gemms, key=lambda k: per_kernel[k]["us_per_step"])
        achieved = gemm_flops / (per_kernel[dom]["avg_us"] * 1e-6) / 1e12
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": recorded_traffic(w.name, dom),
                    "flops_per_launch": gemm_flops, "avg_launch_us": round(per_kernel[dom]["avg_us"], 2)}
    line = {
        "metric": "LeakyReLU(0.5)^2 MLP fwd+bwd tokens/s",
        "value": round(w.tokens / (elapsed / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "d_model": w.d_model, "d_ff": w.d_ff,
                   "step": "up+act, down, dpre, dx, dW_down, dW_up"},
        "launch": "hip_graph_replay" if graph is not None else "eager",
        "active_tflops": round(active / (elapsed / args.steps) / 1e12, 2),
        "active_mfma_frac": round(active / (elapsed / args.steps) / 1e12 / peak, 4),
        "roofline": roofline,
    }
    if per_kernel:
        line["kernels_us_per_step"] = {k: round(v["us_per_step"], 2) for k, v in per_kernel.items()}
        line["kernels_algorithmic_tflops"] = {k: round(gemm_flops / (v["avg_us"] * 1e-6) / 1e12, 1)
                                              for k, v in per_kernel.items() if k != "mlp_dw_reduce"}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = mlp_cpu_baseline(x, wu, wd, dy, min(args.cpu_seconds, 10.0))
    print(json.dumps(line), flush=True)


def mhffn_cpu_baseline(q, r, k, u, v, do, seconds):
    """The multi-head core oracle (fp64 numpy, as it stands) on consecutive
    token slices until `seconds` have passed: forward and backward."""
    import numpy as np
    from oracle import mhffn_oracle as M
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 0) for p in threadpool_info()] or [0]) or os.cpu_count()
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    f64 = lambda t: t.float().numpy().astype(np.float64)
    W = (f64(k), f64(u), f64(v))
    rows, done, t0 = 64, 0, time.perf_counter()
    while True:
        s0 = done % q.shape[0]
        qs, rs, ds = f64(q[s0:s0 + rows]), f64(r[s0:s0 + rows]), f64(do[s0:s0 + rows])
        M.mhffn_forward(qs, rs, *W)
        M.mhffn_backward(ds, qs, rs, *W)
        done += qs.shape[0]
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(done / el, 1), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} tokens in slices of {rows} (fp64 forward + backward), {el:.1f} s"}


MHFFN_KERNEL_UNITS = {"mhffn_fwd": 6, "mhffn_bwd_dq": 6, "mhffn_bwd_dw": 6}   # x tokens*heads*E*d_sub*d_head


def mhffn_main(args):
    """FlashFFN multi-head sub-network core: fused forward, then the backward
    (dQ/dR kernel and weight-gradient kernel, both recomputing) per step."""
    import torch
    import esg_inputs as I
    import group_sparse_swiglu_amd as E

    w = I.MHFFN_WORKLOADS[args.mhffn]
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    E.lib()
    host = I.make_mhffn_inputs(w.tokens, w.heads, w.d_head, w.subnets, w.d_sub, seed=0)
    Q, R, K, U, V, DO = (t.to(dev) for t in host)
    O = torch.empty_like(Q)
    GR = (torch.empty_like(Q), torch.empty_like(R), torch.empty_like(K), torch.empty_like(U), torch.empty_like(V))

    def step():
        E.mhffn_fwd(Q, R, K, U, V, out=O)
        E.mhffn_bwd(DO, Q, R, K, U, V, outs=GR)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay() if graph is not None else step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    unit = float(w.tokens) * w.heads * w.subnets * w.d_sub * w.d_head
    active = 18.0 * unit      # forward 6 units, backward 12 (recompute not credited)
    peak = PEAK_TFLOPS["bf16"]
    roofline, per_kernel = None, {}
    if not args.no_kernel_timing:
        E.timing_reset()
        E.timing_enable(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        for k_ in MHFFN_KERNEL_UNITS:
            ms, n = E.timing_read(k_)
            if n:
                per_kernel[k_] = 1e3 * ms / n
        E.timing_enable(False)
        E.timing_reset()
        dom = max(per_kernel, key=per_kernel.get)
        flops = MHFFN_KERNEL_UNITS[dom] * unit
        ach = flops / (per_kernel[dom] * 1e-6) / 1e12
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(ach / peak, 4), "traffic": recorded_traffic(w.name, dom), "flops_per_launch": flops,
                    "avg_launch_us": round(per_kernel[dom], 2)}
    sec = elapsed / args.steps
    line = {
        "metric": "FlashFFN multi-head sub-network FFN fwd+bwd tokens/s",
        "value": round(w.tokens / sec, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(1e3 * sec, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "heads": w.heads, "d_head": w.d_head,
                   "subnets": w.subnets, "d_sub": w.d_sub, "step": "fused forward, dQ/dR, dK/dU/dV"},
        "launch": "hip_graph_replay" if graph is not None else "eager",
        "active_tflops": round(active / sec / 1e12, 2), "active_mfma_frac": round(active / sec / 1e12 / peak, 4),
        "roofline": roofline,
    }
    if per_kernel:
        line["kernels_us_per_step"] = {k_: round(v_, 2) for k_, v_ in per_kernel.items()}
        line["kernels_algorithmic_tflops"] = {k_: round(MHFFN_KERNEL_UNITS[k_] * unit / (v_ * 1e-6) / 1e12, 1)
                                              for k_, v_ in per_kernel.items()}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = mhffn_cpu_baseline(*host, min(args.cpu_seconds, 10.0))
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no multi-GPU leg.",
              file=sys.stderr)
        sys.exit(2)
    if args.routing:
        routing_main(args)
        return
    if args.mlp:
        mlp_main(args)
        return
    if args.mhffn:
        mhffn_main(args)
        return
    if args.peak:
        peak_main(args)
        return
    if args.k_sweep:
        sweep_main(args)
        return

    import torch
    import esg_inputs as I
    import group_sparse_swiglu_amd as E

    w = I.WORKLOADS[args.workload]
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    E.lib()
    line = measure(args, w, dev)
    print(json.dumps(line), flush=True)


def skew_groups(G: int):
    """The 4 groups the skewed load makes hot (spread over the group range)."""
    return sorted({0, G // 4, G // 2, (3 * G) // 4})


def sweep_main(args):
    """Tokens/s of the step of --workload's shape for each k in --k-sweep: the
    scaling with the active-group fraction k*gs/d_ff (eugen_sparse README,
    "Parameters and how to choose them").  One JSON line with the table."""
    import dataclasses
    import torch
    import esg_inputs as I
    import group_sparse_swiglu_amd as E
    base = I.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    E.lib()
    rows = []
    for k in [int(v) for v in args.k_sweep.split(",")]:
        w = dataclasses.replace(base, k=k, name=f"{base.name}_k{k}")
        print(f"[sweep] k={k}", file=sys.stderr, flush=True)
        line = measure(args, w, dev, cpu=False)
        rows.append({"k": k, "active_fraction": round(k * w.group_size / w.d_ff, 4),
                     "tokens_per_s": line["value"], "ms_per_step": line["ms_per_step"],
                     "active_tflops": line["active_tflops"], "active_mfma_frac": line["active_mfma_frac"],
                     "kernels_us_per_step": line.get("kernels_us_per_step")})
    print(json.dumps({"metric": "sparse SwiGLU fwd+bwd tokens/s against the active-group fraction",
                      "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "dtype": base.dtype, "data": "synthetic",
                      "config": {"workload": base.name, "tokens": base.tokens, "d_model": base.d_model,
                                 "d_ff": base.d_ff, "group_size": base.group_size,
                                 "samples_per_group": base.spg, "bias": base.bias},
                      "sweep": rows}), flush=True)


def measure(args, w, dev, cpu=True):
    """One bench line for workload `w` (see the module docstring)."""
    import torch
    import esg_inputs as I
    import group_sparse_swiglu_amd as E

    x, wg, wu, wd, dy, bias = I.make_workload_inputs(w, seed=0)
    hot = None
    if args.skew and not w.dense:
        bias = (bias if bias is not None else torch.zeros(w.groups)).clone()
        hot = skew_groups(w.groups)
        bias[hot] += 10.0   # far above the energy spread: every token takes the hot groups
        w = dataclasses_replace(w, bias=True, name=w.name + "_skew")
    sub = E.make_subsample_index(w.d_ff, w.group_size, w.spg, 0)[0] if w.spg else None
    host_inputs = (x, wg, wu, wd, dy, bias, sub)
    X, WG, WU, WD, DY = (t.to(dev) for t in (x, wg, wu, wd, dy))
    SUB = None if sub is None else sub.to(dev)
    G = w.groups
    BIAS = (bias if bias is not None else torch.zeros(G)).to(dev)
    EMA = torch.full((G,), w.k / G, dtype=torch.float32, device=dev)
    IDX = torch.empty(w.tokens, w.k, dtype=torch.int32, device=dev)
    Y = torch.empty_like(X)
    GRADS = (torch.empty_like(X), torch.empty_like(WG), torch.empty_like(WU), torch.empty_like(WD))
    # the selection's energy table (used by batches too small to fill the CUs)
    SELWS = torch.empty(max(16, E.select_workspace_size(w.tokens, w.d_ff, w.group_size)), dtype=torch.uint8,
                        device=dev)
    ws = {}
    saved = [None]
    # optionally a second stream for the weight gradients beside the dx sum
    # (the library creates none of its own)
    AUX2 = torch.cuda.Stream(device=dev)
    uses_aux = not (args.inference or w.dense)
    stream_modes = [1, 2] if (args.backward_streams == "auto" and uses_aux) else \
        [int(args.backward_streams) if args.backward_streams != "auto" and uses_aux else 1]
    aux_of = {1: None, 2: AUX2}
    cur = {"aux": aux_of[stream_modes[0]]}

    def step():
        if args.inference:
            if w.dense:
                E.sparse_swiglu_fwd(X, WG, WU, WD, None, w.group_size, workspace=ws, out=Y, for_backward=False)
                return
            E.grouped_topk_select(X, WG, w.group_size, w.k, SUB, w.spg, BIAS if w.bias else None, out=IDX,
                                  workspace=SELWS)
            E.sparse_swiglu_fwd(X, WG, WU, WD, IDX, w.group_size, workspace=ws, out=Y, for_backward=False)
            return
        if w.dense:   # every group active: no selection, fused dense forward, recompute backward
            _, ctx = E.sparse_swiglu_fwd(X, WG, WU, WD, None, w.group_size, workspace=ws, out=Y, saved=saved[0])
            saved[0] = ctx.saved
            E.sparse_swiglu_bwd(DY, X, WG, WU, WD, ctx, workspace=ws, outs=GRADS)
            return
        # the bias update takes its per-group counts from the routing the forward
        # saved, so the selection runs without counts
        E.grouped_topk_select(X, WG, w.group_size, w.k, SUB, w.spg, BIAS if w.bias else None, out=IDX,
                              workspace=SELWS)
        _, ctx = E.sparse_swiglu_fwd(X, WG, WU, WD, IDX, w.group_size, workspace=ws, out=Y, saved=saved[0])
        saved[0] = ctx.saved
        E.sparse_swiglu_bwd(DY, X, WG, WU, WD, ctx, workspace=ws, outs=GRADS, aux_stream=cur["aux"])
        if w.bias_update:
            E.update_load_balance_bias_from_routing(BIAS, EMA, ctx, w.k / G, 1e-3, 0.5, 0.99)

    for mode in stream_modes:
        cur["aux"] = aux_of[mode]
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()

    # Headline: the step's launches captured once as a HIP graph and replayed (the library enqueues
    # kernels only: no host synchronisation, allocation or memset inside a step).  With two backward
    # arrangements to choose from, each is captured and timed for a few replays, and the faster is timed.
    graphs = {}
    for mode in stream_modes:
        cur["aux"] = aux_of[mode]
        if args.no_graph:
            graphs[mode] = None
            continue
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        graphs[mode] = g
    trial_ms = {}
    if len(stream_modes) > 1:
        n_trial = max(3, min(10, args.steps // 4))
        for _rep in range(3):   # alternate the two, keep each one's best of three
            for mode in stream_modes:
                cur["aux"] = aux_of[mode]
                run = graphs[mode].replay if graphs[mode] is not None else step
                run()
                torch.cuda.synchronize()
                tt = time.perf_counter()
                for _ in range(n_trial):
                    run()
                torch.cuda.synchronize()
                ms = 1e3 * (time.perf_counter() - tt) / n_trial
                trial_ms[mode] = min(ms, trial_ms.get(mode, ms))
    # the second stream only when it is clearly faster (by more than 0.5 %)
    chosen = 2 if trial_ms and trial_ms[2] < 0.995 * trial_ms[1] else stream_modes[0]
    cur["aux"] = aux_of[chosen]
    graph = graphs[chosen]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Per-kernel durations: the same steps launched eagerly, each kernel bracketed by HIP events on its stream.
    kernels = ["select", "select_rank", "fill", "bucket_single", "bucket_count", "bucket_place", "bucket_scan",
               "bucket_scatter", "fwd_grouped", "rowsum", "bwd_dh_dx", "bwd_dw", "bias_update", "dense_fwd",
               "dense_route", "dense_rec", "dense_dx", "dense_dw"]
    timing = not args.no_kernel_timing
    eager_ms = None
    if timing:
        # on the step's one stream, so that each kernel's duration is its own
        # (beside a second stream two kernels would share the GPU)
        cur["aux"] = None
        E.timing_reset()
        E.timing_enable(True)
        torch.cuda.synchronize()
        te = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        eager_ms = 1e3 * (time.perf_counter() - te) / args.steps
    per_kernel = {}
    if timing:
        for k in kernels:
            ms, n = E.timing_read(k)
            if n:
                per_kernel[k] = {"avg_us": 1e3 * ms / n, "launches_per_step": n / args.steps,
                                 "us_per_step": 1e3 * ms / args.steps}
        E.timing_enable(False)
        E.timing_reset()

    ms_step = 1e3 * elapsed / args.steps
    tokens_per_s = w.tokens / (elapsed / args.steps)
    unit_flops = float(w.tokens) * w.k * w.group_size * w.d_model
    active = (6.0 if args.inference else 18.0) * unit_flops
    peak = PEAK_TFLOPS[w.dtype]
    roofline = None
    fwd_bwd_us = None
    if per_kernel:
        dom = max((k for k in per_kernel if k in KERNEL_FLOP_UNITS), key=lambda k: per_kernel[k]["us_per_step"])
        # tokens one launch processes (the dense backward runs once per token chunk)
        launch_tokens = w.tokens / per_kernel[dom]["launches_per_step"]
        flops = KERNEL_FLOP_UNITS[dom] * launch_tokens * w.k * w.group_size * w.d_model
        achieved = flops / (per_kernel[dom]["avg_us"] * 1e-6) / 1e12
        traffic = recorded_traffic(w.name, dom)
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                    "flops_per_launch": flops, "avg_launch_us": round(per_kernel[dom]["avg_us"], 2)}
        if traffic:
            roofline["traffic_gbs"] = round(traffic / (per_kernel[dom]["avg_us"] * 1e-6) / 1e9, 1)
        # forward + backward kernels only (the counts fill belongs to the selection call)
        fwd_bwd_us = sum(v["us_per_step"] for k, v in per_kernel.items()
                         if k not in ("select", "fill", "bias_update"))
        line_kernel_flops = {k: KERNEL_FLOP_UNITS[k] * (w.tokens / v["launches_per_step"]) * w.k * w.group_size
                             * w.d_model / (v["avg_us"] * 1e-6) / 1e12
                             for k, v in per_kernel.items() if k in KERNEL_FLOP_UNITS}

    line = {
        "metric": METRIC if not args.inference else "sparse SwiGLU forward-only (inference) tokens/s",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "d_model": w.d_model, "d_ff": w.d_ff,
                   "group_size": w.group_size, "groups": G, "k": w.k, "samples_per_group": w.spg,
                   "bias": w.bias, "bias_update": w.bias_update,
                   "step": (("dense fwd" if w.dense else "select+bucket+fwd") + " (inference)" if args.inference
                            else "dense fwd+bwd (recompute)" if w.dense else
                            "select+bucket+fwd+bwd" + ("+bias_update" if w.bias_update else ""))},
        "launch": "hip_graph_replay" if graph is not None else "eager",
        "backward_streams": chosen if uses_aux else None,
        "backward_streams_trial_ms": {str(m): round(v, 4) for m, v in trial_ms.items()} or None,
        "active_tflops": round(active / (elapsed / args.steps) / 1e12, 2),
        "active_mfma_frac": round(active / (elapsed / args.steps) / 1e12 / peak, 4),
        "roofline": roofline,
    }
    if eager_ms is not None:
        line["eager_ms_per_step_with_kernel_events"] = round(eager_ms, 4)
    if fwd_bwd_us:
        line["fwd_bwd_kernel_us"] = round(fwd_bwd_us, 2)
        line["fwd_bwd_tokens_per_s"] = round(w.tokens / (fwd_bwd_us * 1e-6), 1)
        line["fwd_bwd_active_mfma_frac"] = round(active / (fwd_bwd_us * 1e-6) / 1e12 / peak, 4)
    if per_kernel:
        line["kernels_us_per_step"] = {k: round(v["us_per_step"], 2) for k, v in per_kernel.items()}
        line["kernels_algorithmic_tflops"] = {k: round(v, 1) for k, v in line_kernel_flops.items()}
    if hot is not None:
        counts = torch.bincount(IDX.flatten().long(), minlength=G).cpu()
        line["config"]["skew"] = {"hot_groups": hot, "hot_bias": 10.0,
                                  "hot_load_share": round(float(counts[hot].sum()) / float(counts.sum()), 4),
                                  "max_group_tokens": int(counts.max()), "min_group_tokens": int(counts.min())}
    if not getattr(args, "no_peak_probe", False) and cpu:
        peak_meas = mfma_probe_tflops(dev)
        line["mfma_peak_measured_tflops"] = round(peak_meas, 1)
        line["active_frac_of_measured_peak"] = round(line["active_tflops"] / peak_meas, 4)
        if line.get("roofline"):
            line["roofline"]["frac_of_measured_peak"] = round(line["roofline"]["achieved"] / peak_meas, 4)
    if cpu and not args.no_cpu_baseline and not args.inference:
        line["cpu_baseline"] = cpu_baseline(w, host_inputs, args.cpu_seconds)
    return line


if __name__ == "__main__":
    main()

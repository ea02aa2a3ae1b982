#!/usr/bin/env python3
"""Benchmark: seconds to prune one LLaMA-7B-shaped MLP down_proj layer with 2:4
block-wise (Thanos-style) pruning on one MI355X, plus the Hessian TFLOP/s.

A step is one call of th_prune_layer on inputs resident in HBM: W (4096 x 11008
bf16, restored from a pristine copy at the start of the step) and calibration
activations X (262144 tokens x 11008 bf16, ReLU-like with 110 channels x30). The
step runs the whole path: H = 2XX^T + lambda*I (bf16 MFMA), factor + inverse,
per-block 2:4 selection, joint solves and updates (block size 128), and the
cast back to bf16.

Prints one JSON line. `roofline` is for the dominant kernel (the bf16 syrk),
timed with HIP events on the stream it runs on; `cpu_baseline` is the fp64
oracle on a bounded sample of the same workload, scaled to seconds per layer.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--pattern 2:4|4:8|unstructured]
                       [--sparsity 0.5] [--layer down_proj-4096x11008|down_proj-8192x28672]
                       [--no-cpu-baseline]
(the headline line is the default: 2:4 on the 4096 x 11008 down_proj; the other
patterns and the LLaMA-2-70B-shaped 8192 x 28672 down_proj on 65536 tokens with
1% of its channels x100 are extra measurements)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "seconds per layer (4096×11008 down_proj, 2:4) + XXᵀ TFLOP/s vs MFMA peak"
# --layer choices: (synthetic workload id, layer name)
LAYERS = {"down_proj-4096x11008": (3, "down_proj"), "down_proj-8192x28672": (5, "down_proj")}
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E (datasheet)
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (datasheet)
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 MFMA (datasheet)


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _ev_time(fn, reps, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        start.record(stream)
        fn()
        end.record(stream)
        end.synchronize()
        times.append(start.elapsed_time(end))
    return times


def syrk_traffic():
    """HBM-side bytes per syrk launch from the committed counter summary, or None
    if the kernel source changed since the counters were taken."""
    import hashlib
    import re
    prof = os.path.join(ROOT, "profiles", "syrk_rect_down_proj_11008x262144_traffic.md")
    try:
        txt = open(prof).read()
        d = json.loads(re.search(r"```json\n(.*?)\n```", txt, re.S).group(1))
        src = open(os.path.join(ROOT, d["source"]), "rb").read()
        if hashlib.sha256(src).hexdigest() != d["source_sha256"]:
            return None
        return float(d["traffic_bytes_per_launch"])
    except Exception:
        return None


def _host_facts():
    """Cores this process may run on, the CPU model and the BLAS numpy uses."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = "unknown", cores
    try:
        import numpy  # noqa: F401  (loads the BLAS that threadpoolctl then reports)
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = (f"{info[0].get('internal_api')} {info[0].get('version')} "
                    f"({info[0].get('architecture')} kernels)")
            threads = max(i.get("num_threads", 1) for i in info)
    except Exception:
        pass
    return cores, model, blas, threads


def cpu_baseline(X, W, c, b, n, pattern, block, lam_rel, sparsity=0.5):
    """fp64 oracle on a bounded sample of the same workload, scaled to seconds per layer.

    Measured: G from the first n/8 tokens (12.5% of the stream; scaled by 8), the
    Cholesky check and LU inverse of the damped b x b H at full size, and the
    first 3 column blocks of the block loop with all rows. Scaled: the G time by
    the token ratio, the block time by the modelled flops of all blocks (Schur
    downdate 2|F'|^2 B + 2|F'| B^2, update 2 c B |F|, per-row solves c s^3/3)."""
    import numpy as np
    import oracle as O
    cores, model, blas, threads = _host_facts()
    n_s = max(1024, n // 8)
    t0 = time.perf_counter()
    G = np.zeros((b, b))
    for a in range(0, n_s, 8192):  # copied to the host and summed chunk by chunk
        G += O.gram(X[a:min(n_s, a + 8192)].cpu())
    t_g_meas = time.perf_counter() - t0
    t_g = t_g_meas * (n / n_s)
    Wn = W.float().cpu().numpy()
    k_s = 3
    t0 = time.perf_counter()
    O.prune_layer(Wn, G, sparsity=sparsity, pattern=pattern, block=block, lam=lam_rel,
                  max_blocks=k_s)
    t_rest = time.perf_counter() - t0
    # split t_rest into the (unscaled) inverse and the sampled blocks
    H = O.hessian(G, O.damping(G, lam_rel))
    t0 = time.perf_counter()
    np.linalg.cholesky(H)
    np.linalg.inv(H)
    t_inv = time.perf_counter() - t0
    t_blocks_s = max(t_rest - t_inv, 0.0)
    s = (block * (pattern[1] - pattern[0]) // pattern[1]) if pattern else round(block * sparsity)

    def cost(j0):
        f = b - j0
        fp = max(f - block, 0)
        return 2 * fp * fp * block + 2 * fp * block * block + 2 * c * block * f + c * s ** 3 / 3

    total = sum(cost(j0) for j0 in range(0, b, block))
    sampled = sum(cost(j0) for j0 in range(0, min(b, k_s * block), block))
    t_blocks = t_blocks_s * total / sampled
    value = t_g + t_inv + t_blocks
    return {"value": value, "unit": "s", "cores": int(threads), "kind": "oracle",
            "sample": (f"G on {n_s} of {n} tokens ({100.0 * n_s / n:.1f}%, x{n / n_s:g}); Cholesky "
                       f"check + LU inverse at full b={b}; first {k_s} of {-(-b // block)} blocks "
                       f"with all {c} rows, scaled by modelled flops (x{total / sampled:.1f})"),
            "measured_s": {"G_sample": round(t_g_meas, 2), "inverse": round(t_inv, 2),
                           "blocks_sample": round(t_blocks_s, 2)},
            "scaled_s": {"G": round(t_g, 1), "inverse": round(t_inv, 1), "blocks": round(t_blocks, 1)},
            "host": {"cores_available": cores, "cpu": model, "blas": blas,
                     "blas_threads": threads}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--pattern", default="2:4", help="N:M such as 2:4 or 4:8, or unstructured")
    ap.add_argument("--sparsity", type=float, default=0.5, help="unstructured sparsity")
    ap.add_argument("--layer", default="down_proj-4096x11008", choices=sorted(LAYERS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from layer_wise_obs_amd import _lib as L
    from layer_wise_obs_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg_id, lname = LAYERS[args.layer]
    cfg = synth.config(cfg_id)
    layer = [l for l in cfg.layers if l.name == lname][0]
    st = cfg.streams[layer.hessian]
    c, b, n = layer.c, layer.b, st.n
    unstructured = args.pattern == "unstructured"
    pn, pm = (0, 1) if unstructured else (int(v) for v in args.pattern.split(":"))
    pattern = None if unstructured else (pn, pm)
    pat_name = f"{args.sparsity:g} unstructured" if unstructured else f"{pn}:{pm}"
    block, lam_rel = cfg.block, cfg.lambda_rel

    _log(f"generating X [{n} x {b}] bf16 and W [{c} x {b}] on the GPU")
    X = torch.empty((n, b), dtype=torch.bfloat16, device=dev)
    cfg.activations(layer.hessian, device=dev, out=X)
    W0 = cfg.weights(layer, device=dev)
    W = torch.empty_like(W0)
    torch.cuda.synchronize()

    params = L.make_params(sparsity=args.sparsity, pattern=pattern, block=block, lam=lam_rel,
                           relative=True)
    ws = L.workspace(L.prune_layer_workspace_size(c, b, n, True, params), dev)
    Wout = torch.empty((c, b), dtype=torch.float32, device=dev)
    mask = torch.empty((c, b), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        W.copy_(W0)
        return L.prune_layer(W, X=X, params=params, W_out=Wout, mask_out=mask, ws=ws)

    for i in range(args.warmup):
        _log(f"warmup step {i + 1}/{args.warmup}")
        info = step()
    torch.cuda.synchronize()
    _log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        info = step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1000.0 / max(args.steps, 1)
    _log(f"{ms_step:.2f} ms per layer")

    # dominant kernel: the bf16 syrk, same launch as inside the step (with a
    # workspace, as th_prune_layer gives it: 384 x 256 rectangles, the last round's
    # tiles cut into pieces summed by a fix-up kernel; the events cover both)
    H = torch.zeros((b, b), dtype=torch.float32, device=dev)
    hws = L.workspace(L.hessian_workspace_size(n, b), dev)
    syrk_ms = _ev_time(lambda: L.hessian_accumulate(H, X, hws), max(args.steps, 3), stream)
    syrk_avg = sum(syrk_ms) / len(syrk_ms)
    syrk_flops = float(n) * b * (b + 1)  # one triangle of X^T X: n*b(b+1)
    achieved = syrk_flops / (syrk_avg * 1e-3) / 1e12
    _log(f"syrk {syrk_avg:.2f} ms = {achieved:.0f} TFLOP/s")

    # the layer from a given Hessian (factor + block loop only)
    H.zero_()
    L.hessian_accumulate(H, X, hws)
    lam_h = L.hessian_finalize(H, lam_rel, True)

    def step_h():
        W.copy_(W0)
        return L.prune_layer(W, H=H, params=params, W_out=Wout, mask_out=mask, ws=ws)

    step_h()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(max(args.steps, 1)):
        step_h()
    torch.cuda.synchronize()
    ms_given_h = (time.perf_counter() - t1) * 1000.0 / max(args.steps, 1)

    # reconstruction error of the last result (reported, not part of the step)
    W32 = W0.float()
    t2 = time.perf_counter()
    E, E_rel = L.reconstruction_error(W32, Wout, G=H_undamped(H, lam_h))
    ms_err = (time.perf_counter() - t2) * 1000.0

    fact_flops = 2.0 * b ** 3 / 3.0
    nblk = -(-b // block)
    fsum = sum(b - j * block for j in range(nblk))
    upd_flops = 2.0 * block * block * fsum + 2.0 * c * block * fsum
    floor_ms = (syrk_flops / (PEAK_BF16_TFLOPS * 1e12)
                + (fact_flops + upd_flops) / (PEAK_FP32_TFLOPS * 1e12)) * 1e3
    floor_h_ms = (fact_flops + upd_flops) / (PEAK_FP32_TFLOPS * 1e12) * 1e3
    # unstructured: the global selection reads W[:, F] (fp32) at least once per block
    select_floor_ms = (4.0 * c * fsum / (HBM_PEAK_GBS * 1e9) * 1e3) if unstructured else 0.0
    m = mask.bool()
    if unstructured:  # the global budget is met exactly
        count_ok = int(m.sum().item()) == info["pruned"] == round(args.sparsity * c * b)
    else:  # exactly m - n pruned in every group of m
        count_ok = bool((m.view(c, -1, pm).sum(dim=2) == pm - pn).all().item())

    out = {
        "metric": METRIC.replace("4096×11008", f"{c}×{b}").replace("2:4", pat_name),
        "value": ms_step / 1000.0,
        "unit": "s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/fp32",
        "data": "synthetic",
        "config": {"workload": f"down_proj {c}x{b}, {pat_name}, block {block}, X {n} tokens bf16 "
                               f"({'ReLU-like, ' if st.relu else ''}{st.outlier_count} channels x{st.outlier_scale:g}), "
                               f"lambda {lam_rel} relative"},
        "roofline": {"bound": "mfma", "kernel": "syrk_rect_kernel (+ syrk_rect_fix_kernel)",
                     "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": syrk_traffic() if args.layer == "down_proj-4096x11008" else None,
                     "launch_ms": syrk_avg,
                     "algorithmic": f"n*b*(b+1) = {syrk_flops:.4g} flop per launch"},
        "extra": {
            "hessian_tflops": achieved,
            "ms_per_layer_given_H": ms_given_h,
            "pruned_weights_per_s": info["pruned"] / (ms_step / 1000.0),
            "pruned": info["pruned"],
            "counts_exact": count_ok,
            "at_peak_floor_ms": floor_ms + select_floor_ms,
            "at_peak_floor_given_H_ms": floor_h_ms + select_floor_ms,
            "select_hbm_floor_ms": select_floor_ms,
            "mfma_utilisation_e2e": floor_ms / ms_step,
            "recon_error_rel": E_rel,
            "recon_error_ms": ms_err,
        },
    }
    if not args.no_cpu_baseline and args.layer != "down_proj-4096x11008":
        _log("no CPU baseline for this layer: its fp64 inverse alone takes minutes")
    elif not args.no_cpu_baseline:
        _log("timing the fp64 oracle on a bounded sample (CPU)")
        out["cpu_baseline"] = cpu_baseline(X, W0, c, b, n, pattern, block, lam_rel, args.sparsity)
    print(json.dumps(out), flush=True)


def H_undamped(H, lam):
    """G = (H - lambda I) / 2 from the finalized Hessian (for the error report)."""
    import torch
    G = H.clone()
    G.diagonal().sub_(lam)
    G.mul_(0.5)
    return G


if __name__ == "__main__":
    main()

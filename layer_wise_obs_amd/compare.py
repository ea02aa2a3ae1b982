"""Reconstruction error of the joint-compensation method against its comparators
(SparseGPT's column-sequential schedule; Wanda and magnitude pruning, no
compensation) on the synthetic workloads.

Usage: python -m layer_wise_obs_amd.compare [--configs 1 2 3 4 5]

For every layer and pattern of a workload: H from the layer's synthetic input
stream (th_hessian_accumulate, th_hessian_finalize), then th_prune_layer (the
method), th_prune_layer_alpha (alpha = 0.1, N:M patterns only), th_prune_sparsegpt,
th_prune_baseline with G_qq from th_column_sq_norms (Wanda) and without
(magnitude), and th_reconstruction_error against G = (H - lambda I) / 2. Every
step runs in the HIP library; this file only moves tensors and prints one JSON
line per (workload, layer, pattern).
"""
from __future__ import annotations

import argparse
import json
import time

import torch

from . import _lib as L
from . import synth

DEV = "cuda:0"


def _ms(t0):
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def _pattern_args(pat):
    if pat[0] == "unstructured":
        return {"sparsity": pat[1], "pattern": None}, f"unstructured {pat[1]:g}"
    return {"sparsity": 0.5, "pattern": (pat[1], pat[2])}, f"{pat[1]}:{pat[2]}"


def run_config(cid: int):
    cfg = synth.config(cid)
    cache = {}
    for layer in cfg.layers:
        if layer.hessian not in cache:
            s = cfg.streams[layer.hessian]
            X = torch.empty((s.n, s.b), dtype=cfg.xdtype, device=DEV)
            cfg.activations(layer.hessian, device=DEV, out=X)
            H = torch.zeros((s.b, s.b), dtype=torch.float32, device=DEV)
            ws = L.workspace(L.hessian_workspace_size(s.n, s.b), DEV)
            L.hessian_accumulate(H, X, ws)
            lam = L.hessian_finalize(H, cfg.lambda_rel, True)
            g = L.column_sq_norms(X)
            G = H.clone()
            G.diagonal().sub_(lam)
            G.mul_(0.5)
            del X, ws
            cache = {layer.hessian: (H, lam, g, G)}  # one stream's tensors at a time
        H, lam, g, G = cache[layer.hessian]
        W0 = cfg.weights(layer, device=DEV)
        for pat in cfg.patterns:
            kw, name = _pattern_args(pat)
            params = L.make_params(block=cfg.block, lam=cfg.lambda_rel, **kw)
            out = {"config": cid, "layer": layer.name, "c": layer.c, "b": layer.b,
                   "pattern": name, "E_rel": {}, "ms": {}}
            for name, fn in (("thanos", L.prune_layer), ("sparsegpt", L.prune_sparsegpt)):
                W = W0.clone()
                Wout = torch.empty(W.shape, dtype=torch.float32, device=DEV)
                t0 = time.perf_counter()
                fn(W, H=H, params=params, W_out=Wout)
                out["ms"][name] = round(_ms(t0), 3)
                out["E_rel"][name] = L.reconstruction_error(W0.float(), Wout, G=G)[1]
                del W, Wout
            if pat[0] == "nm":  # the alpha = 0.1 variant the pages report for N:M
                W = W0.clone()
                Wout = torch.empty(W.shape, dtype=torch.float32, device=DEV)
                t0 = time.perf_counter()
                L.prune_layer_alpha(W, 0.1, H=H, params=params, W_out=Wout)
                out["ms"]["thanos_alpha0.1"] = round(_ms(t0), 3)
                out["E_rel"]["thanos_alpha0.1"] = L.reconstruction_error(W0.float(), Wout, G=G)[1]
                del W, Wout
            for method in ("wanda", "magnitude"):
                W = W0.clone()
                t0 = time.perf_counter()
                L.prune_baseline(W, method, gdiag=g if method == "wanda" else None, params=params)
                out["ms"][method] = round(_ms(t0), 3)
                out["E_rel"][method] = L.reconstruction_error(W0, W, G=G)[1]
                del W
            print(json.dumps(out), flush=True)
        del W0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--configs", type=int, nargs="+", default=[1, 2, 3, 4, 5])
    args = ap.parse_args()
    assert torch.cuda.is_available(), "needs a GPU"
    for cid in args.configs:
        run_config(cid)
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()

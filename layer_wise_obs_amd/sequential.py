"""One transformer block pruned in order, with shared factors and the feed-forward
input propagated from the pruned layers.

Usage: python -m layer_wise_obs_amd.sequential [--config 4] [--pattern 2:4]

"Pruning LLMs with Thanos", section "The layer-reconstruction lens": every linear
layer is reconstructed from its own calibration inputs; layers that read the same
input (q/k/v; gate/up) share one Hessian, so its factor U (H^-1 = U^T U) is
computed once (th_factor) and each of them is pruned from it
(th_prune_layer_factored). down_proj's input is not an independent stream: it is
produced by the pruned gate and up projections through the gated feed-forward
(th_gated_ffn_input, section "The compression target: linear layers"), and down
is pruned on the Hessian of that input. The attention output feeding o_proj
would need the attention itself; it stays the independent synthetic stream.

Every step runs in the HIP library; this module only orders the calls, owns the
tensors and prints one JSON line per layer plus a summary.
"""
from __future__ import annotations

import argparse
import json
import time

import torch

from . import _lib as L
from . import synth

DEV = "cuda:0"


def _sync_ms(t0):
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def _params(cfg, pattern):
    if pattern is None:
        p = cfg.patterns[0]
        if p[0] == "unstructured":
            return L.make_params(sparsity=p[1], block=cfg.block, lam=cfg.lambda_rel)
        return L.make_params(pattern=(p[1], p[2]), block=cfg.block, lam=cfg.lambda_rel)
    return L.make_params(pattern=pattern, block=cfg.block, lam=cfg.lambda_rel)


def prune_block(cfg, params, propagate=True, report=print):
    """Prune the block's layers in order. Returns {layer: (W_hat bf16, info)} and the
    timing of each phase in ms."""
    layers = {l.name: l for l in cfg.layers}
    out, times = {}, {}

    def stream_x(name):
        s = cfg.streams[name]
        X = torch.empty((s.n, s.b), dtype=cfg.xdtype, device=DEV)
        cfg.activations(name, device=DEV, out=X)
        torch.cuda.synchronize()  # generation is not part of any timed phase
        return X

    def prune_group(X, names, tag):
        t0 = time.perf_counter()
        U, lam = L.factor(X=X, lam=cfg.lambda_rel, relative=True)
        times[f"factor {tag}"] = round(_sync_ms(t0), 3)
        for nm in names:
            W = cfg.weights(layers[nm], device=DEV)
            W0 = W.clone()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            info = L.prune_layer_factored(W, U, params=params)
            times[nm] = round(_sync_ms(t0), 3)
            _, er = L.reconstruction_error(W0, W, X=X)
            out[nm] = (W, info)
            report(json.dumps({"layer": nm, "c": W.shape[0], "b": W.shape[1],
                               "input": tag, "E_rel": er, "pruned": info["pruned"],
                               "ms": times[nm]}))
        del U

    X = stream_x("attn_in")
    prune_group(X, [n for n in ("q_proj", "k_proj", "v_proj") if n in layers], "attn_in")
    del X
    X = stream_x("o_in")
    prune_group(X, ["o_proj"], "o_in")
    del X
    X = stream_x("mlp_in")
    prune_group(X, ["gate_proj", "up_proj"], "mlp_in")
    if propagate:
        t0 = time.perf_counter()
        Xd = L.gated_ffn_input(X, out["gate_proj"][0], out["up_proj"][0])
        times["gated ffn"] = round(_sync_ms(t0), 3)
        tag = "gated(mlp_in)"
    else:
        Xd, tag = stream_x("down_in"), "down_in"
    del X
    prune_group(Xd, ["down_proj"], tag)
    return out, times


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--pattern", default=None, help="n:m (default: the workload's own)")
    ap.add_argument("--independent", action="store_true",
                    help="down_proj on its independent synthetic stream instead")
    args = ap.parse_args()
    assert torch.cuda.is_available(), "needs a GPU"
    cfg = synth.config(args.config)
    pattern = tuple(int(v) for v in args.pattern.split(":")) if args.pattern else None
    _, times = prune_block(cfg, _params(cfg, pattern), propagate=not args.independent)
    print(json.dumps({"config": args.config, "times_ms": times,
                      "total_ms": round(sum(times.values()), 1)}))


if __name__ == "__main__":
    main()

"""Write the oracle's expected values for the full-size workloads (tests/golden/fullsize/).

Every value stored here comes from the fp64 oracle (``oracle/``) run on the CPU on
the seeded synthetic inputs (``layer_wise_obs_amd.synth``, which holds none of the
pruning arithmetic). Nothing is read from the GPU library.

Per case (workload, layer, pattern) it stores:

* ``rows``: the sampled output rows (sorted); ``mask_rows`` (bit-packed, 1 = pruned)
  and ``what_rows`` (fp32) of the oracle's result on those rows;
* ``gap_rows`` (fp32, N:M): per row and aligned group, the relative gap between
  the (m-n)-th and the next-lowest oracle score when the group's mask was chosen,
  (s_hi - s_lo) / s_hi; a GPU decision that differs there is an fp32 near-tie only
  if this gap is small;
* ``dist_rows`` (fp32, unstructured): per row and column, |S - T| / T at the
  column's own block, T being that block's threshold (the r-th smallest score of
  the active region);
* ``thresholds``, ``budgets`` and ``near_counts`` (unstructured): per block T, the
  remaining budget r and how many scores of the whole active region lie within
  relative windows 1e-6, 1e-5, 1e-4 and 1e-3 of T;
* ``counts`` (per block), ``row_counts`` (unstructured: every row), ``lam``,
  ``k_total``, ``diag_inv`` (diag of H^-1, the block-0 OBS denominators);
* the error: ``e_row`` / ``base_row`` per sampled row (D_k G D_k^T and
  W_k G W_k^T, D = W - W_hat) and, when the oracle prunes every row
  (unstructured), the layer's ``e_all`` / ``base_all``.

N:M rows are independent given H ("Pruning LLMs with Thanos", section "The
layer-reconstruction lens": the objective decomposes over rows; the N:M masks
have no budget shared across rows), so the oracle prunes only the sampled rows.
The global budget of unstructured sparsity couples all rows ("Contribution two"),
so there the oracle prunes the whole layer.

Usage: python tests/golden/make_fullsize.py [--cases NAME ...] [--cache DIR]
(about an hour on 8 cores for every case; --cache keeps the fp64 Gram matrices
as .npy files between runs.)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from layer_wise_obs_amd import synth  # noqa: E402

OUT = os.path.join(HERE, "fullsize")
WINDOWS = (1e-6, 1e-5, 1e-4, 1e-3)


def case_list():
    """(name, config id, layer, pattern, sampled rows). pattern: ("unstructured", p) or ("nm", n, m)."""
    out = []
    out.append(("cfg2_q_proj_2of4", 2, "q_proj", ("nm", 2, 4), 32))
    out.append(("cfg3_down_proj_2of4", 3, "down_proj", ("nm", 2, 4), 32))
    out.append(("cfg3_down_proj_4of8", 3, "down_proj", ("nm", 4, 8), 32))
    for name in ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj"):
        out.append((f"cfg4_{name}_unstructured50", 4, name, ("unstructured", 0.5), 16))
    for name in ("k_proj", "v_proj", "q_proj", "o_proj", "down_proj"):
        rows = 8 if name == "down_proj" else 16
        out.append((f"cfg5_{name}_unstructured60", 5, name, ("unstructured", 0.6), rows))
        out.append((f"cfg5_{name}_2of4", 5, name, ("nm", 2, 4), rows))
    return out


def gram_of_stream(cfg, stream, cache):
    """fp64 G = X X^T of a whole calibration stream, generated and summed chunk by chunk."""
    path = None
    if cache:
        path = os.path.join(cache, f"G_cfg{cfg.cid}_{stream}.npy")
        if os.path.exists(path):
            return np.load(path)
    s = cfg.streams[stream]
    G = np.zeros((s.b, s.b), dtype=np.float64)
    step = 8192
    t0 = time.perf_counter()
    for a in range(0, s.n, step):
        Xc = cfg.activations(stream, n=min(step, s.n - a), token_offset=a)
        G += O.gram(Xc)
        if (a // step) % 8 == 0:
            print(f"  gram {stream}: {a + step}/{s.n} tokens, {time.perf_counter() - t0:.0f} s",
                  flush=True)
    if path:
        np.save(path, G)
    return G


def nm_gaps(S_J, n, m):
    """(s_hi - s_lo) / s_hi between the (m-n)-th lowest and the next score of each group."""
    c, blk = S_J.shape
    g = np.sort(S_J.reshape(c, blk // m, m), axis=2)
    lo, hi = g[:, :, m - n - 1], g[:, :, m - n]
    with np.errstate(divide="ignore", invalid="ignore"):
        gap = np.where(hi > 0, (hi - lo) / hi, 0.0)
    return gap


_DIAG_INV = {}


def run_case(name, cid, lname, pat, nrows, cache):
    cfg = synth.config(cid)
    layer = [l for l in cfg.layers if l.name == lname][0]
    c, b = layer.c, layer.b
    rng = np.random.default_rng([cid, sum(map(ord, name))])
    rows = np.sort(rng.choice(c, size=min(nrows, c), replace=False))
    W = cfg.weights(layer)  # bf16 on the CPU
    G = gram_of_stream(cfg, layer.hessian, cache)
    block = cfg.block
    rec = {"rows": rows.astype(np.int32)}
    t0 = time.perf_counter()
    if pat[0] == "nm":
        n_, m_ = pat[1], pat[2]
        gaps = []

        def on_block(j0, S, r, sel, g=None):
            gaps.append(nm_gaps(S, n_, m_))

        Wr = W[rows]
        ora = O.prune_layer(Wr, G, pattern=(n_, m_), block=block, lam=cfg.lambda_rel,
                            on_block=on_block)
        rec["gap_rows"] = np.concatenate(gaps, axis=1).astype(np.float32)
        W_rows = O.thanos_oracle._f64(Wr)
        Wh_rows, mask_rows = ora["W_hat"], ora["mask"]
        rec["counts"] = np.asarray(ora["counts"], np.int64)  # of the sampled rows
        rec["k_total"] = np.int64(-1)
    else:
        p = pat[1]
        thr, bud, near, dist = [], [], [], []

        def on_block(j0, S, r, sel, g=None):
            blk = sel.shape[1]
            flat = S.ravel()
            if 0 < r < flat.size:
                T = float(np.partition(flat, r - 1)[r - 1])
            else:
                T = float("nan")
            thr.append(T)
            bud.append(r)
            if np.isfinite(T) and T > 0:
                rel = np.abs(flat - T) / T
                near.append([int(np.count_nonzero(rel <= w)) for w in WINDOWS])
                dist.append((np.abs(S[rows, :blk] - T) / T).astype(np.float32))
                del rel
            else:
                near.append([0] * len(WINDOWS))
                dist.append(np.full((len(rows), blk), np.inf, np.float32))

        ora = O.prune_layer(W, G, sparsity=p, block=block, lam=cfg.lambda_rel, on_block=on_block)
        rec["thresholds"] = np.asarray(thr, np.float64)
        rec["budgets"] = np.asarray(bud, np.int64)
        rec["near_counts"] = np.asarray(near, np.int64)
        rec["dist_rows"] = np.concatenate(dist, axis=1)
        rec["row_counts"] = ora["mask"].sum(axis=1).astype(np.int32)
        rec["counts"] = np.asarray(ora["counts"], np.int64)
        rec["k_total"] = np.int64(ora["k_total"])
        W0 = O.thanos_oracle._f64(W)
        e_all, er_all = O.reconstruction_error(W0, ora["W_hat"], G)
        rec["e_all"] = np.float64(e_all)
        rec["base_all"] = np.float64(e_all / er_all if er_all > 0 else 0.0)
        W_rows = W0[rows]
        Wh_rows, mask_rows = ora["W_hat"][rows], ora["mask"][rows]
    t_prune = time.perf_counter() - t0
    D = W_rows - Wh_rows
    rec["e_row"] = np.sum((D @ G) * D, axis=1)  # per sampled row: D_k G D_k^T
    rec["base_row"] = np.sum((W_rows @ G) * W_rows, axis=1)
    rec["lam"] = np.float64(ora["lam"])
    rec["mask_rows"] = np.packbits(mask_rows.astype(np.uint8), axis=1)
    rec["what_rows"] = Wh_rows.astype(np.float32)
    key = (cid, layer.hessian)
    if key not in _DIAG_INV:
        H = O.hessian(G, ora["lam"])
        _DIAG_INV[key] = np.diag(np.linalg.inv(H)).copy()
        del H
    rec["diag_inv"] = _DIAG_INV[key]
    rec["shape"] = np.array([c, b], np.int64)
    np.savez_compressed(os.path.join(OUT, f"{name}.npz"), **rec)
    return t_prune


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--cases", nargs="*", default=None)
    ap.add_argument("--cache", default=None, help="directory for fp64 Gram matrices (.npy)")
    args = ap.parse_args()
    os.makedirs(OUT, exist_ok=True)
    if args.cache:
        os.makedirs(args.cache, exist_ok=True)
    man_path = os.path.join(OUT, "manifest.json")
    manifest = json.load(open(man_path)) if os.path.exists(man_path) else {}
    for name, cid, lname, pat, nrows in case_list():
        if args.cases and name not in args.cases:
            continue
        print(f"[golden] {name}", flush=True)
        t = run_case(name, cid, lname, pat, nrows, args.cache)
        manifest[name] = {"config": cid, "layer": lname, "pattern": list(pat),
                          "oracle_prune_s": round(t, 1)}
        json.dump(manifest, open(man_path, "w"), indent=1, sort_keys=True)
        print(f"[golden] {name} done: oracle layer step {t:.1f} s", flush=True)


if __name__ == "__main__":
    main()

"""Helpers that compare the HIP path with the fp64 oracle (shared by the GPU tests,
the smoke check and the benchmark's spot checks)."""
from __future__ import annotations

import numpy as np

# Tolerances (the target the method's parity is held to):
H_RTOL = 1e-4       # ||H_gpu - H_ora||_F / ||H_ora||_F, fp32 accumulation
W_RTOL = 1e-3       # ||W_gpu - W_ora||_F / ||W_ora||_F on rows with identical masks
E_RTOL = 1e-3       # |E_gpu - E_ora| / E_ora
NEAR_TIE = 1e-3     # relative score gap under which an fp32 decision may differ


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def first_diff_block(mask_a, mask_b, k, block):
    d = np.flatnonzero(mask_a[k] != mask_b[k])
    return None if len(d) == 0 else int(d[0] // block) * block


def explain_nm_flip(trace, k, j0, m, n, gpu_mask, ora_mask, block):
    """At the first differing block of row k, every differing group must be a
    near-tie in the oracle's own scores (the (m-n)-th and next-lowest scores)."""
    S = next(t["S"] for t in trace if t["j0"] == j0)
    blk = S.shape[1]
    for g0 in range(0, blk, m):
        a = gpu_mask[k, j0 + g0:j0 + g0 + m]
        o = ora_mask[k, j0 + g0:j0 + g0 + m]
        if np.array_equal(a, o):
            continue
        s = np.sort(S[k, g0:g0 + m])
        lo, hi = s[m - n - 1], s[m - n]
        if not (hi - lo <= NEAR_TIE * max(abs(hi), 1e-30)):
            return False
    return True


def explain_unstructured_flip(trace, k, j0, gpu_mask, ora_mask):
    """At the first differing block, each differing entry's oracle score lies
    within NEAR_TIE of the oracle's threshold (the r-th smallest score)."""
    t = next(t for t in trace if t["j0"] == j0)
    S, r = t["S"], t["r"]
    flat = np.sort(S.ravel())
    T = flat[max(r, 1) - 1]
    blk_w = min(S.shape[1], gpu_mask.shape[1] - j0)
    d = np.flatnonzero(gpu_mask[k, j0:j0 + blk_w] != ora_mask[k, j0:j0 + blk_w])
    for q in d:
        if abs(S[k, q] - T) > NEAR_TIE * max(abs(T), 1e-30):
            return False
    return True


def compare_pruned(W_gpu, mask_gpu, ora, block, pattern=None, trace=None, max_flip_frac=0.01):
    """Masks must match row by row, except rows whose first difference is an
    explained near-tie (bounded fraction); on matching rows W_hat must agree
    within W_RTOL. Returns a report dict."""
    W_gpu = np.asarray(W_gpu, np.float64)
    mask_gpu = np.asarray(mask_gpu).astype(bool)
    W_o, mask_o = ora["W_hat"], ora["mask"]
    c = W_o.shape[0]
    same = np.all(mask_gpu == mask_o, axis=1)
    flips = np.flatnonzero(~same)
    unexplained = []
    for k in flips:
        j0 = first_diff_block(mask_gpu, mask_o, k, block)
        if trace is None:
            unexplained.append(int(k))
        elif pattern is None:
            if not explain_unstructured_flip(trace, k, j0, mask_gpu, mask_o):
                unexplained.append(int(k))
        else:
            n_, m_ = pattern
            if not explain_nm_flip(trace, k, j0, m_, n_, mask_gpu, mask_o, block):
                unexplained.append(int(k))
    err_same = rel_fro(W_gpu[same], W_o[same]) if same.any() else 0.0
    return {
        "rows": c,
        "flip_rows": int(len(flips)),
        "unexplained_rows": unexplained,
        "w_rel_err_same_rows": err_same,
        "w_rel_err_all": rel_fro(W_gpu, W_o),
        "ok": (len(unexplained) == 0 and len(flips) <= max(1, int(max_flip_frac * c))
               and err_same <= W_RTOL),
    }

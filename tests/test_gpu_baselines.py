"""Parity of the comparators (magnitude and Wanda pruning, no compensation) with the
fp64 oracle, through the C ABI.

The explainer's section "Wanda: Pruning by Weights and Activations" (score
|W_kq| ||X_q||_2, thresholds per output row, no update of the remaining weights),
section "The Failure of Magnitude Pruning in Large Transformers" (rank by |W_kq|)
and section "N:M Semi-Structured Sparsity (2:4 Pattern)". Both sides compute the
same fp32 keys from the same fp32 G_qq, so masks are compared bit for bit; kept
weights must be unchanged and pruned ones exactly zero. G_qq itself is compared
with the oracle's fp64 sums rounded to fp32 (at most one ulp apart).
"""
import numpy as np
import pytest
import torch

import oracle as O
from layer_wise_obs_amd import _lib as L
from layer_wise_obs_amd import synth
from tests import _parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("xdtype,n,b", [(torch.bfloat16, 3000, 1000), (torch.float32, 5000, 257),
                                        (torch.bfloat16, 1, 64)])
def test_column_sq_norms_match_oracle(xdtype, n, b):
    _say(f"column norms {xdtype} n={n} b={b}")
    X = synth.activations(n, b, 5, 1, 3, 30.0, True, xdtype)
    g = L.column_sq_norms(X.to(DEV)).cpu().numpy()
    ref = O.column_sq_norms(X)
    assert g.dtype == np.float32 and g.shape == (b,)
    # fp64 sums in a different order, each rounded once to fp32: equal or one ulp apart
    assert np.all(np.abs(g.astype(np.float64) - ref) <= np.spacing(ref).astype(np.float64))


CASES = [
    # method, W dtype, c, b, sparsity, pattern
    ("magnitude", torch.bfloat16, 96, 1000, 0.5, None),   # bf16: many equal magnitudes (ties)
    ("wanda", torch.bfloat16, 96, 1000, 0.5, None),
    ("wanda", torch.float32, 64, 1003, 0.3, None),        # ragged last 256-column tile
    ("magnitude", torch.float32, 33, 5000, 0.77, None),   # 20 tiles per row
    ("wanda", torch.bfloat16, 1, 300, 0.5, None),         # one row
    ("wanda", torch.bfloat16, 16, 512, 0.0, None),        # nothing pruned
    ("magnitude", torch.bfloat16, 16, 512, 1.0, None),    # everything pruned
    ("wanda", torch.bfloat16, 96, 1000, None, (2, 4)),
    ("magnitude", torch.bfloat16, 96, 1000, None, (2, 4)),
    ("wanda", torch.float32, 40, 1024, None, (4, 8)),
    ("wanda", torch.bfloat16, 40, 1002, None, (1, 6)),
    ("magnitude", torch.bfloat16, 8, 256, None, (0, 128)),  # widest group, all pruned
]


@pytest.mark.parametrize("method,wdtype,c,b,sparsity,pattern", CASES)
def test_baseline_matches_oracle_bit_exact(method, wdtype, c, b, sparsity, pattern):
    _say(f"baseline {method} {wdtype} c={c} b={b} p={sparsity} pattern={pattern}")
    W = synth.weights(c, b, 0.02, 11, 100, wdtype)
    X = synth.activations(2048, b, 11, 1, 3, 30.0, True, torch.bfloat16)
    g = L.column_sq_norms(X.to(DEV)) if method == "wanda" else None
    Wd = W.to(DEV).clone()
    mask = torch.empty((c, b), dtype=torch.uint8, device=DEV)
    params = L.make_params(sparsity=0.5 if sparsity is None else sparsity, pattern=pattern,
                           block=128)
    L.prune_baseline(Wd, method, gdiag=g, params=params, mask_out=mask)
    ora = O.prune_baseline(W, method, gdiag=None if g is None else g.cpu().numpy(),
                           sparsity=0.5 if sparsity is None else sparsity, pattern=pattern)
    mg = mask.cpu().numpy().astype(bool)
    assert np.array_equal(mg, ora["mask"])
    # kept entries bit-identical to W, pruned entries exactly zero
    Wh = Wd.float().cpu().numpy()
    assert np.array_equal(Wh, ora["W_hat"].astype(np.float32))
    if pattern is None:
        assert np.all(mg.sum(axis=1) == int(np.round(sparsity * b)))
    else:
        n, m = pattern
        assert np.all(mg.reshape(c, b // m, m).sum(axis=2) == m - n)


def test_baseline_error_matches_oracle_and_exceeds_thanos():
    """E of the comparators against the oracle's, and the method's own layer step
    (joint compensation) reaching a lower error on the same layer ("Pruning LLMs
    with Thanos", section "Contribution one": compensation of the kept weights)."""
    c, b, n = 64, 512, 4096
    _say(f"baseline error c={c} b={b} n={n}")
    W = synth.weights(c, b, 0.02, 13, 100, torch.bfloat16)
    X = synth.activations(n, b, 13, 1, 3, 30.0, True, torch.bfloat16)
    G = O.gram(X)
    Xd = X.to(DEV)
    g = L.column_sq_norms(Xd)
    errs = {}
    for method in ("magnitude", "wanda"):
        Wd = W.to(DEV).clone()
        L.prune_baseline(Wd, method, gdiag=g, params=L.make_params(pattern=(2, 4)))
        e, er = L.reconstruction_error(W.to(DEV), Wd, X=Xd)
        ora = O.prune_baseline(W, method, gdiag=g.cpu().numpy(), pattern=(2, 4))
        eo, ero = O.reconstruction_error(W, ora["W_hat"], G)
        assert abs(e - eo) <= P.E_RTOL * eo
        errs[method] = er
    Wt = W.to(DEV).clone()
    Wout = torch.empty((c, b), dtype=torch.float32, device=DEV)
    L.prune_layer(Wt, X=Xd, params=L.make_params(pattern=(2, 4), block=128), W_out=Wout)
    _, er_thanos = L.reconstruction_error(W.to(DEV).float(), Wout, X=Xd.float())
    assert er_thanos < errs["wanda"] < errs["magnitude"], (er_thanos, errs)

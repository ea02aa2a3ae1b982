"""The alpha variant (rows of largest output energy kept dense, the others pruned
as a layer of their own) through the C ABI.

"Pruning LLMs with Thanos", section "What the experiments show" (alpha = 0.1 keeps
10% of the rows as outliers, 50% becomes 45%). Every case is compared end to end
with the oracle's prune_layer_alpha on the oracle's own fp64 Gram matrix: the
dense rows must be the oracle's, except rows whose fp32 energies lie within an
fp32 near-tie of the cut (the GPU forms G_qq from X or from its fp32 H); the
pruned rows follow the oracle's layer step on those rows (and are bit-identical
to th_prune_layer on the gathered rows).
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


def _inputs(c, b, n, seed, relu=False):
    W = synth.weights(c, b, 0.02, seed, 100, torch.bfloat16)
    X = synth.activations(n, b, seed, 1, 3, 30.0, relu, torch.bfloat16)
    return W, X


def _check_dense(dense, W, gdiag, alpha, exact=False):
    """The GPU's dense rows against the oracle's choice from its own G_qq; a row
    may differ only if its oracle energy is within NEAR_TIE of the cut (the
    smallest dense energy), and not at all where exact is set."""
    ref = O.outlier_rows(W, gdiag, alpha)
    diff = np.flatnonzero(dense != ref)
    if len(diff):
        assert not exact, diff
        s = O.row_energies(W, gdiag).astype(np.float64)
        cut = s[ref].min()
        gaps = np.abs(s[diff] - cut) / cut
        print(f"dense rows differing at near-ties: {len(diff)}, largest gap {gaps.max():.2e}",
              flush=True)
        assert np.all(gaps <= P.NEAR_TIE), gaps
    return ref


def _oracle_rest(ora, trace, dense, W, G, pattern, block):
    """The oracle's result on the GPU's pruned rows: its own alpha step when the
    dense rows agree; otherwise (N:M only, after near-ties at the cut) its layer
    step on exactly those rows, which N:M allows since rows are independent."""
    rest = np.flatnonzero(~dense)
    if np.array_equal(dense, ora["dense"]):
        return {"W_hat": ora["W_hat"][rest], "mask": ora["mask"][rest]}, trace
    assert pattern is not None
    tr = []
    sub = O.prune_layer(W.float().numpy()[rest], G, pattern=pattern, block=block, trace=tr)
    return sub, tr


def _run(W, alpha, **kw):
    Wd = W.to(DEV).clone()
    c, b = W.shape
    Wout = torch.empty((c, b), dtype=torch.float32, device=DEV)
    mask = torch.empty((c, b), dtype=torch.uint8, device=DEV)
    dense = torch.empty((c,), dtype=torch.uint8, device=DEV)
    info = L.prune_layer_alpha(Wd, alpha, W_out=Wout, mask_out=mask, dense_out=dense, **kw)
    return (Wd.cpu(), Wout.cpu().numpy(), mask.cpu().numpy().astype(bool),
            dense.cpu().numpy().astype(bool), info)


@pytest.mark.parametrize("pattern,sparsity,alpha,c,b", [((2, 4), 0.5, 0.1, 200, 392),
                                                        (None, 0.6, 0.05, 150, 304),
                                                        ((4, 8), 0.5, 0.25, 64, 256)])
def test_alpha_matches_oracle(pattern, sparsity, alpha, c, b):
    _say(f"alpha {alpha} {pattern or sparsity} c={c} b={b}")
    W, X = _inputs(c, b, 3000, 71, relu=True)
    Xd = X.to(DEV)
    params = L.make_params(sparsity=sparsity, pattern=pattern, block=128)
    Wb, Wf, m, dense, info = _run(W, alpha, X=Xd, params=params)
    G = O.gram(X)
    trace = []
    ora = O.prune_layer_alpha(W, G, alpha, sparsity=sparsity, pattern=pattern, block=128,
                              trace=trace)
    # the oracle's G_qq: diag of its fp64 G rounded to fp32 (= column_sq_norms of X)
    _check_dense(dense, W, np.diag(G).astype(np.float32), alpha, exact=pattern is None)
    r = int(np.round(alpha * c))
    assert dense.sum() == r
    # dense rows untouched
    W32 = W.float().numpy()
    assert np.array_equal(Wf[dense], W32[dense]) and not m[dense].any()
    assert torch.equal(Wb[torch.tensor(dense)], W[torch.tensor(dense)])
    # the others: the oracle's layer step on the same rows
    rest = np.flatnonzero(~dense)
    sub, tr = _oracle_rest(ora, trace, dense, W, G, pattern, 128)
    rep = P.compare_pruned(Wf[rest], m[rest], sub, 128, pattern, tr)
    print(rep, flush=True)
    assert rep["ok"], rep
    assert info["pruned"] == int(m.sum())
    if pattern is None:
        assert info["pruned"] == O.k_total(sparsity, c - r, b)


@pytest.mark.parametrize("pattern,sparsity", [((2, 4), 0.5), (None, 0.5)])
def test_alpha_rest_equals_prune_layer_on_gathered_rows(pattern, sparsity):
    """From a given H: the pruned rows are bit-identical to th_prune_layer on the
    gathered rows; the dense rows and the pruned rows follow the oracle's
    prune_layer_alpha on its own fp64 G (the library forms G_qq = (H_qq - lambda)/2
    from the fp32 H, so the dense choice may differ only at near-ties)."""
    _say(f"alpha from H, gathered rows {pattern or sparsity}")
    c, b = 300, 512
    W, X = _inputs(c, b, 4096, 72)
    H = torch.zeros((b, b), dtype=torch.float32, device=DEV)
    L.hessian_accumulate(H, X.to(DEV))
    L.hessian_finalize(H, 0.01, True)
    params = L.make_params(sparsity=sparsity, pattern=pattern, block=128)
    Wb, Wf, m, dense, info = _run(W, 0.1, H=H, params=params)
    G = O.gram(X)
    trace = []
    ora = O.prune_layer_alpha(W, G, 0.1, sparsity=sparsity, pattern=pattern, block=128,
                              trace=trace)
    _check_dense(dense, W, np.diag(G).astype(np.float32), 0.1, exact=pattern is None)
    rr = np.flatnonzero(~dense)
    sub, tr = _oracle_rest(ora, trace, dense, W, G, pattern, 128)
    rep = P.compare_pruned(Wf[rr], m[rr], sub, 128, pattern, tr)
    print(rep, flush=True)
    assert rep["ok"], rep
    rest = torch.tensor(np.flatnonzero(~dense))
    Ws = W[rest].to(DEV).contiguous()
    Wsf = torch.empty(Ws.shape, dtype=torch.float32, device=DEV)
    ms = torch.empty(Ws.shape, dtype=torch.uint8, device=DEV)
    info2 = L.prune_layer(Ws, H=H, params=params, W_out=Wsf, mask_out=ms)
    assert np.array_equal(Wf[rest.numpy()], Wsf.cpu().numpy())
    assert np.array_equal(m[rest.numpy()], ms.cpu().numpy().astype(bool))
    assert torch.equal(Wb[rest], Ws.cpu())
    assert info["counts"] == info2["counts"]


def test_alpha_limits():
    _say("alpha 0 and 1")
    W, X = _inputs(96, 256, 2048, 73)
    Xd = X.to(DEV)
    params = L.make_params(pattern=(2, 4), block=64)
    Wb, Wf, m, dense, info = _run(W, 0.0, X=Xd, params=params)
    Wd = W.to(DEV).clone()
    Wf2 = torch.empty((96, 256), dtype=torch.float32, device=DEV)
    m2 = torch.empty((96, 256), dtype=torch.uint8, device=DEV)
    L.prune_layer(Wd, X=Xd, params=params, W_out=Wf2, mask_out=m2)
    assert not dense.any()
    assert np.array_equal(Wf, Wf2.cpu().numpy()) and np.array_equal(m, m2.cpu().numpy().astype(bool))
    Wb, Wf, m, dense, info = _run(W, 1.0, X=Xd, params=params)
    assert dense.all() and not m.any() and torch.equal(Wb, W) and info["pruned"] == 0


def test_alpha_reports_nonfinite_in_a_dense_row():
    _say("alpha non-finite weight")
    W, X = _inputs(64, 128, 1024, 74)
    W[5, 7] = float("inf")  # this row's energy is infinite, so it is kept dense
    with pytest.raises(L.ThanosError) as e:
        _run(W, 0.1, X=X.to(DEV), params=L.make_params(pattern=(2, 4), block=64))
    assert e.value.status == L.TH_ERR_NONFINITE


def test_alpha_full_size_q_proj():
    """4096 x 4096 q_proj, 262144 tokens, 2:4 with alpha = 0.1: 410 dense rows,
    45% zeros, exact group counts on the others, energy order of the dense rows."""
    _say("alpha full size q_proj 2:4")
    cfg = synth.config(2)
    layer = cfg.layers[0]
    s = cfg.streams["attn_in"]
    X = torch.empty((s.n, s.b), dtype=torch.bfloat16, device=DEV)
    cfg.activations("attn_in", device=DEV, out=X)
    W = cfg.weights(layer, device=DEV)
    W0 = W.clone()
    mask = torch.empty(W.shape, dtype=torch.uint8, device=DEV)
    dense = torch.empty((W.shape[0],), dtype=torch.uint8, device=DEV)
    info = L.prune_layer_alpha(W, 0.1, X=X, params=L.make_params(pattern=(2, 4)), mask_out=mask,
                               dense_out=dense)
    d = dense.bool()
    assert int(d.sum()) == 410
    assert info["pruned"] == (4096 - 410) * 4096 // 2
    assert abs(int(mask.sum()) / mask.numel() - 0.45) < 1e-3
    assert bool((mask[~d].view(4096 - 410, -1, 4).sum(dim=2) == 2).all())
    assert torch.equal(W[d], W0[d]) and int(mask[d].sum()) == 0
    g = O.column_sq_norms(X.cpu())  # fp64 sums over token chunks, rounded to fp32
    _check_dense(dense.cpu().numpy().astype(bool), W0.cpu(), g, 0.1)

"""Parity of the column-sequential comparator (SparseGPT's schedule) with the fp64
oracle, through the C ABI.

"Pruning LLMs with Thanos", section "The scaling problem, and what SparseGPT
changes", and the explainer's section "SparseGPT: Second-Order Reconstruction at
Scale". The oracle builds every column's row of the inverse over the active
columns by Schur downdates and applies the update column by column; the GPU uses
U (H^-1 = U^T U), a per-row error recurrence and one GEMM per block. Masks are
compared row by row (a row may differ only at an explained fp32 near-tie of the
oracle's own scores), W_hat within 1e-3 relative on rows whose masks agree, E
within 1e-3 of the oracle's.
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


def _inputs(c, b, n, seed, wdtype=torch.bfloat16, xdtype=torch.bfloat16, relu=False,
            outliers=3, scale=30.0):
    W = synth.weights(c, b, 0.02, seed, 100, wdtype)
    X = synth.activations(n, b, seed, 1, outliers, scale, relu, xdtype)
    return W, X


def _run_gpu(W, X=None, H=None, **kw):
    Wd = W.to(DEV).contiguous()
    Wout = torch.empty(W.shape, dtype=torch.float32, device=DEV)
    mask = torch.empty(W.shape, dtype=torch.uint8, device=DEV)
    info = L.prune_sparsegpt(Wd, X=None if X is None else X.to(DEV), H=H,
                             params=L.make_params(**kw), W_out=Wout, mask_out=mask)
    return Wd, Wout.cpu().numpy(), mask.cpu().numpy().astype(bool), info


def _check(W, X, sparsity=0.5, pattern=None, block=128, max_flip_frac=0.01):
    G = O.gram(X)
    trace = []
    ora = O.prune_sparsegpt(W, G, sparsity=sparsity, pattern=pattern, block=block, trace=trace)
    Wd, Wg, mg, info = _run_gpu(W, X, sparsity=sparsity, pattern=pattern, block=block)
    rep = P.compare_pruned(Wg, mg, ora, block, pattern, trace, max_flip_frac)
    print(rep, flush=True)
    assert rep["ok"], rep
    c, b = W.shape
    assert np.all(Wg[mg] == 0.0)
    # per-block counts on the GPU's own mask: the quota, or the group counts
    got = [int(mg[:, j0:j0 + block].sum()) for j0 in range(0, b, block)]
    assert info["counts"] == got
    if pattern is None:
        assert got == ora["counts"]  # round-half-even(p * c * |J|) for every block
    else:
        n_, m_ = pattern
        assert np.all(mg.reshape(c, -1, m_).sum(axis=2) == m_ - n_)
    assert info["pruned"] == int(mg.sum())
    assert abs(info["lambda"] - ora["lam"]) <= 1e-5 * ora["lam"]
    W32 = torch.tensor(O.thanos_oracle._f64(W), dtype=torch.float32, device=DEV)
    e_gpu, _ = L.reconstruction_error(W32, torch.tensor(Wg, device=DEV),
                                      G=torch.tensor(G, dtype=torch.float32, device=DEV))
    e_ora, _ = O.reconstruction_error(W, ora["W_hat"], G)
    assert abs(e_gpu - e_ora) <= P.E_RTOL * e_ora, (e_gpu, e_ora)
    if W.dtype == torch.bfloat16:
        assert torch.equal(Wd.cpu(), torch.tensor(Wg).to(torch.bfloat16))
    return ora, Wg, mg, info


def test_sparsegpt_config1_unstructured():
    _say("sparsegpt config 1 (128x256 fp32, 50% unstructured, B=32)")
    cfg = synth.config(1)
    _check(cfg.weights(cfg.layers[0]), cfg.activations("x"), sparsity=0.5, block=32)


@pytest.mark.parametrize("pattern", [(2, 4), (4, 8), (1, 4)])
def test_sparsegpt_nm_several_tiles(pattern):
    _say(f"sparsegpt N:M {pattern} c=300 b=512")
    W, X = _inputs(300, 512, 4096, 51, relu=True)
    _check(W, X, pattern=pattern, block=128)


@pytest.mark.parametrize("pattern,sparsity,block,c,b", [
    ((2, 4), None, 32, 200, 1096),   # five groups of eight blocks, ragged 8-column last block
    (None, 0.6, 32, 160, 600),       # unstructured, ragged 24-column last block
    (None, 0.5, 128, 96, 1160),      # 128-wide blocks, a second group, ragged last block
])
def test_sparsegpt_across_super_blocks(pattern, sparsity, block, c, b):
    """Compensation beyond each group of eight blocks is deferred to the group's
    end (both masks depend only on their block)."""
    _say(f"sparsegpt {pattern or sparsity} B={block} c={c} b={b} (several block groups)")
    W, X = _inputs(c, b, 4096, 52, relu=True)
    _check(W, X, sparsity=sparsity or 0.5, pattern=pattern, block=block)


def test_sparsegpt_unstructured_ragged_and_high_sparsity():
    _say("sparsegpt unstructured c=200 b=392 and 70% B=48")
    W, X = _inputs(200, 392, 3000, 53)
    _check(W, X, sparsity=0.5, block=128)
    W, X = _inputs(96, 240, 2000, 54, relu=True)
    _check(W, X, sparsity=0.7, block=48)


@pytest.mark.parametrize("c,b,n,block,pattern,sparsity,dtype", [
    (1, 64, 256, 16, None, 0.5, torch.bfloat16),      # one output row
    (7, 40, 300, 8, (2, 4), 0.5, torch.float32),      # fp32, tiny blocks
    (33, 136, 512, 1, None, 0.3, torch.float32),      # B = 1: one column per block
    (64, 8, 64, 8, (4, 8), 0.5, torch.bfloat16),      # b = 8
    (20, 200, 1000, 128, None, 0.9, torch.bfloat16),  # 90%, ragged 72-column last block
])
def test_sparsegpt_degenerate_shapes(c, b, n, block, pattern, sparsity, dtype):
    _say(f"sparsegpt degenerate c={c} b={b} n={n} B={block} {pattern or sparsity} {dtype}")
    W, X = _inputs(c, b, n, 55, wdtype=dtype, xdtype=dtype, outliers=2)
    _check(W, X, sparsity=sparsity, pattern=pattern, block=block, max_flip_frac=1.0)


def test_sparsegpt_limits():
    _say("sparsegpt limits p=0, p=1")
    W, X = _inputs(64, 128, 1024, 56)
    _, Wg, mg, _ = _run_gpu(W, X, sparsity=0.0, block=64)
    assert not mg.any() and np.array_equal(Wg, W.float().numpy())
    _, Wg, mg, _ = _run_gpu(W, X, sparsity=1.0, block=64)
    assert mg.all() and np.all(Wg == 0.0)


def test_sparsegpt_from_hessian_equals_from_activations_and_is_deterministic():
    _say("sparsegpt from H vs from X, determinism")
    W, X = _inputs(128, 256, 2048, 57)
    Hd = torch.zeros((256, 256), dtype=torch.float32, device=DEV)
    L.hessian_accumulate(Hd, X.to(DEV))
    L.hessian_finalize(Hd, 0.01, True)
    _, Wa, ma, _ = _run_gpu(W, X, pattern=(2, 4), block=128)
    _, Wb, mb, _ = _run_gpu(W, H=Hd, pattern=(2, 4), block=128)
    assert np.array_equal(ma, mb) and P.rel_fro(Wb, Wa) <= 1e-5
    _, Wc, mc, _ = _run_gpu(W, X, sparsity=0.5, block=128)
    _, Wd, md, _ = _run_gpu(W, X, sparsity=0.5, block=128)
    assert np.array_equal(mc, md) and np.array_equal(Wc, Wd)

"""Shared factor, pruning from a given factor, the gated feed-forward input and the
sequential block, through the C ABI.

"Pruning LLMs with Thanos", sections "The layer-reconstruction lens" (each layer
reconstructed from its own inputs) and "The compression target: linear layers"
(feed-forward projections joined by a nonlinearity). Pruning from a factor must
give bit-identical results to th_prune_layer on the same Hessian; the gated
feed-forward output must be the bf16 rounding of the fp64 value except where the
fp32 sums land on the other side of a rounding boundary (then one bf16 ulp); the
sequential block is compared with the oracle's composition.
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


def _inputs(c, b, n, seed, relu=False, outliers=3, scale=30.0):
    W = synth.weights(c, b, 0.02, seed, 100, torch.bfloat16)
    X = synth.activations(n, b, seed, 1, outliers, scale, relu, torch.bfloat16)
    return W, X


def _prune(fn, W, *args, **kw):
    Wd = W.to(DEV).clone()
    Wout = torch.empty(W.shape, dtype=torch.float32, device=DEV)
    mask = torch.empty(W.shape, dtype=torch.uint8, device=DEV)
    info = fn(Wd, *args, W_out=Wout, mask_out=mask, **kw)
    return Wd.cpu(), Wout.cpu().numpy(), mask.cpu().numpy().astype(bool), info


@pytest.mark.parametrize("pattern,sparsity,block", [((2, 4), 0.5, 128), (None, 0.6, 64),
                                                    ((4, 8), 0.5, 32)])
def test_factored_equals_prune_layer_bit_for_bit(pattern, sparsity, block):
    """Three layers on one input: th_factor once, th_prune_layer_factored for each,
    against th_prune_layer from X for each (bit-identical), and the first against
    the oracle."""
    _say(f"factored vs prune_layer {pattern or sparsity} B={block}")
    b, n = 392, 3000
    _, X = _inputs(8, b, n, 61, relu=True)
    Xd = X.to(DEV)
    U, lam = L.factor(X=Xd, lam=0.01, relative=True)
    params = L.make_params(sparsity=sparsity, pattern=pattern, block=block)
    for i, c in enumerate((200, 64, 333)):
        W, _ = _inputs(c, b, 8, 62 + i)
        Wa, fa, ma, ia = _prune(L.prune_layer_factored, W, U, params=params)
        Wb, fb, mb, ib = _prune(L.prune_layer, W, X=Xd, params=params)
        assert torch.equal(Wa, Wb) and np.array_equal(fa, fb) and np.array_equal(ma, mb)
        assert ia["counts"] == ib["counts"] and ia["pruned"] == ib["pruned"]
        assert abs(ib["lambda"] - lam) <= 1e-6 * lam
        if i == 0:
            trace = []
            ora = O.prune_layer(W, O.gram(X), sparsity=sparsity, pattern=pattern, block=block,
                                trace=trace)
            rep = P.compare_pruned(fa, ma, ora, block, pattern, trace)
            print(rep, flush=True)
            assert rep["ok"], rep


def test_factor_matches_debug_factor_and_inverse_cholesky():
    _say("th_factor from H")
    b = 520
    _, X = _inputs(8, b, 2000, 63)
    G = O.gram(X)
    lam = O.damping(G, 0.01, True)
    H = torch.tensor(O.hessian(G, lam), dtype=torch.float32, device=DEV)
    U, lam_out = L.factor(H=H, lam=0.01, relative=True)
    assert abs(lam_out - lam) <= 1e-5 * lam  # the damping a given H is taken to carry
    assert torch.equal(U, L.debug_factor(H))
    Hn = H.double().cpu().numpy()
    U_ref = np.linalg.cholesky(np.linalg.inv(Hn)).T
    assert P.rel_fro(U.cpu().numpy(), U_ref) <= 5e-4
    assert np.all(np.tril(U.cpu().numpy(), -1) == 0.0)


def test_factor_reports_not_spd():
    _say("th_factor not SPD")
    H = -torch.eye(64, dtype=torch.float32, device=DEV)
    with pytest.raises(L.ThanosError) as e:
        L.factor(H=H, lam=0.0, relative=False)
    assert e.value.status == L.TH_ERR_NOT_SPD


def _ffn_check(X, Wg, Wu, Y):
    ref = O.gated_ffn_input(X, Wg, Wu)
    ref_b = O.thanos_oracle._bf16_round(ref)
    got = Y.double().cpu().numpy()
    exact = np.mean(got == ref_b)
    # one bf16 ulp of the reference value (2^-7 relative to its power of two)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(got - ref) <= ulp + 1e-6 * np.max(np.abs(ref))), np.max(np.abs(got - ref))
    assert exact >= 0.99, exact
    return exact


@pytest.mark.parametrize("n,d,f", [(300, 264, 200), (1000, 512, 700), (1, 8, 1), (257, 40, 129),
                                   (512, 4096, 256)])
def test_gated_ffn_matches_oracle(n, d, f):
    """Ragged tiles in every dimension, a contraction tail (d % 32 != 0), the
    smallest shape, and a LLaMA-width contraction."""
    _say(f"gated ffn n={n} d={d} f={f}")
    X = synth.activations(n, d, 64, 1, 2, 20.0, False, torch.bfloat16)
    Wg = synth.weights(f, d, 0.05, 64, 101, torch.bfloat16)
    Wu = synth.weights(f, d, 0.05, 64, 102, torch.bfloat16)
    Y = L.gated_ffn_input(X.to(DEV), Wg.to(DEV), Wu.to(DEV))
    exact = _ffn_check(X, Wg, Wu, Y)
    print(f"exact fraction {exact:.5f}", flush=True)


def test_gated_ffn_full_size_sampled():
    """The block's feed-forward at its real shape (131072 tokens, 4096 -> 11008):
    sampled outputs against fp64 dot products of the sampled rows."""
    _say("gated ffn full size 131072 x 4096 -> 11008")
    cfg = synth.config(4)
    s = cfg.streams["mlp_in"]
    X = torch.empty((s.n, s.b), dtype=torch.bfloat16, device=DEV)
    cfg.activations("mlp_in", device=DEV, out=X)
    lay = {l.name: l for l in cfg.layers}
    Wg = cfg.weights(lay["gate_proj"], device=DEV)
    Wu = cfg.weights(lay["up_proj"], device=DEV)
    Y = L.gated_ffn_input(X, Wg, Wu)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(s.n, 96, replace=False))
    cols = np.sort(rng.choice(Wg.shape[0], 128, replace=False))
    Xs = X[rows].cpu()
    got = Y[rows][:, cols].cpu()
    exact = _ffn_check(Xs, Wg[cols].cpu(), Wu[cols].cpu(), got)
    print(f"exact fraction {exact:.5f}", flush=True)


def test_sequential_mlp_block_matches_oracle():
    """gate and up pruned from one factor, down on the input they produce, against
    the oracle's composition (down's masks may differ only at near-ties, because
    its input is built from slightly different gate and up weights)."""
    _say("sequential mlp block d=256 f=512 n=2048")
    d, f, n = 256, 512, 2048
    X = synth.activations(n, d, 65, 1, 2, 20.0, False, torch.bfloat16)
    Wg = synth.weights(f, d, 0.05, 65, 101, torch.bfloat16)
    Wu = synth.weights(f, d, 0.05, 65, 102, torch.bfloat16)
    Wdn = synth.weights(d, f, 0.05, 65, 103, torch.bfloat16)
    block = 64
    params = L.make_params(pattern=(2, 4), block=block)
    ora = O.prune_mlp_sequential(X, Wg, Wu, Wdn, pattern=(2, 4), block=block)
    Xd = X.to(DEV)
    U, _ = L.factor(X=Xd)
    res = {}
    for name, W in (("gate", Wg), ("up", Wu)):
        Wb, Wf, m, _ = _prune(L.prune_layer_factored, W, U, params=params)
        trace = []
        O.prune_layer(W, ora["G_mlp"], pattern=(2, 4), block=block, trace=trace)
        rep = P.compare_pruned(Wf, m, ora[name], block, (2, 4), trace)
        print(name, rep, flush=True)
        assert rep["ok"], rep
        res[name] = Wb.to(DEV)
    Xdown = L.gated_ffn_input(Xd, res["gate"], res["up"])
    xg = Xdown.double().cpu().numpy()
    assert P.rel_fro(xg, ora["X_down"]) <= 1e-3
    assert np.mean(xg == ora["X_down"]) >= 0.95
    Ud, _ = L.factor(X=Xdown)
    _, Wf, m, info = _prune(L.prune_layer_factored, Wdn, Ud, params=params)
    trace = []
    O.prune_layer(Wdn, ora["G_down"], pattern=(2, 4), block=block, trace=trace)
    # down's input differs from the oracle's by bf16 roundings of the propagated
    # activations (about 0.05% of the entries by one bf16 unit, 2^-8 relative), a
    # perturbation of G far above fp32 rounding: near-ties up to 1e-3 are allowed
    rep = P.compare_pruned(Wf, m, ora["down"], block, (2, 4), trace, max_flip_frac=0.05,
                           near_tie=1e-3)
    print("down", rep, flush=True)
    assert rep["ok"], rep
    assert np.all(m.reshape(d, -1, 4).sum(axis=2) == 2)


def test_factored_from_fp32_activations():
    """th_factor on fp32 X (the fp32 Hessian path) then the factored layer step:
    bit-identical to th_prune_layer on the same fp32 X."""
    _say("factored from fp32 X")
    c, b, n = 96, 200, 1500
    W = synth.weights(c, b, 0.02, 66, 100, torch.float32)
    X = synth.activations(n, b, 66, 1, 3, 30.0, False, torch.float32)
    Xd = X.to(DEV)
    U, lam = L.factor(X=Xd, lam=0.01, relative=True)
    params = L.make_params(sparsity=0.5, block=64)
    Wa, fa, ma, ia = _prune(L.prune_layer_factored, W, U, params=params)
    Wb, fb, mb, ib = _prune(L.prune_layer, W, X=Xd, params=params)
    assert np.array_equal(fa, fb) and np.array_equal(ma, mb) and torch.equal(Wa, Wb)
    assert abs(ib["lambda"] - lam) <= 1e-6 * lam

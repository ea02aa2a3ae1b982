"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

None of these re-types the oracle's own formulas. They use closed forms, least
squares on an augmented design matrix, brute-force enumeration, textbook special
cases (the SparseGPT column update, a diagonal Gram matrix) and invariants the
pages state ("Pruning LLMs with Thanos": exact zeros on the selected set, exact
group counts, the global budget met exactly, padding contributes nothing).
"""
import itertools

import numpy as np
import pytest

import oracle as O

RNG_SEED = 1234


def _problem(c, b, n, seed, outliers=1, scale=20.0, corr=True):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, b))
    if corr:  # correlated features so that compensation matters
        mix = np.eye(b) + 0.3 * rng.standard_normal((b, b)) / np.sqrt(b)
        X = X @ mix
    cols = rng.choice(b, outliers, replace=False)
    X[:, cols] *= scale
    if corr and b >= 4:
        # a near-duplicate feature: OBS sees that one of the pair is cheap to
        # delete, a diagonal (Wanda-style) score does not
        X[:, 1] = 3.0 * X[:, 0] + 0.05 * rng.standard_normal(n)
    W = 0.02 * rng.standard_normal((c, b))
    return W, X


def _chol_factor(H):
    """C with H = C C^T (so that d H d^T = ||d C||^2)."""
    return np.linalg.cholesky(H)


def _constrained_min(w, H, fixed_zero, delete):
    """argmin_{w'} (w'-w) H (w'-w)^T subject to w'[delete]=0 and w'[fixed_zero]=w[fixed_zero]
    (i.e. the change is 0 on frozen columns), by least squares on C^T."""
    b = len(w)
    C = _chol_factor(H)
    d = np.zeros(b)
    d[delete] = -w[delete]
    free = np.setdiff1d(np.arange(b), np.union1d(fixed_zero, delete))
    if len(free):
        y = -(d[delete] @ C[delete, :])
        x, *_ = np.linalg.lstsq(C[free, :].T, y, rcond=None)
        d[free] = x
    return w + d, float(d @ H @ d)


def _reference_prune(W, G, lam_abs, block, sparsity=None, pattern=None, score="obs"):
    """Independent block-wise procedure: direct sub-matrix inverses for the scores,
    lexsort selection, and least-squares compensation with frozen columns fixed."""
    c, b = W.shape
    H = 2 * G + lam_abs * np.eye(b)
    Wc = W.copy()
    mask = np.zeros((c, b), bool)
    ktot = int(np.round(sparsity * c * b)) if pattern is None else None
    pruned = 0
    for j0 in range(0, b, block):
        blk = min(block, b - j0)
        F = np.arange(j0, b)
        AF = np.linalg.inv(H[np.ix_(F, F)])
        g = 1.0 / np.diag(AF) if score == "obs" else np.diag(G)[F]
        S = Wc[:, F] ** 2 * g
        sel = np.zeros((c, blk), bool)
        if pattern is None:
            r = ktot - pruned
            rows, cols = np.meshgrid(np.arange(c), F, indexing="ij")
            flat = (rows * b + cols).ravel()
            order = np.lexsort((flat, S.ravel()))
            cand = np.zeros(c * len(F), bool)
            cand[order[:max(r, 0)]] = True
            sel = cand.reshape(c, len(F))[:, :blk]
        else:
            n_, m_ = pattern
            for k in range(c):
                for g0 in range(0, blk, m_):
                    grp = S[k, g0:g0 + m_]
                    order = sorted(range(m_), key=lambda i: (grp[i], i))
                    for i in order[: m_ - n_]:
                        sel[k, g0 + i] = True
        frozen = np.arange(0, j0)
        for k in range(c):
            Q = j0 + np.flatnonzero(sel[k])
            if len(Q):
                Wc[k], _ = _constrained_min(Wc[k], H, frozen, Q)
                Wc[k, Q] = 0.0
        mask[:, j0:j0 + blk] = sel
        pruned += int(sel.sum())
    return Wc, mask


# ---------------------------------------------------------------- P1

def test_p1_single_deletion_error_closed_form():
    """Deleting one weight with no compensation costs W_kq^2 (XX^T)_qq
    ("Why magnitude alone misses important weights")."""
    W, X = _problem(4, 10, 64, RNG_SEED)
    G = O.gram(X)
    k, q = 2, 7
    Wh = W.copy()
    Wh[k, q] = 0.0
    E, _ = O.reconstruction_error(W, Wh, G)
    direct = np.linalg.norm((W - Wh) @ X.T) ** 2
    closed = W[k, q] ** 2 * np.sum(X[:, q] ** 2)
    assert np.isclose(E, direct, rtol=1e-12)
    assert np.isclose(E, closed, rtol=1e-12)


def test_p1_error_equals_direct_frobenius_for_dense_change():
    W, X = _problem(5, 9, 40, RNG_SEED + 1)
    G = O.gram(X, chunk=7)
    Wh = W + 0.01 * np.random.default_rng(3).standard_normal(W.shape)
    E, Er = O.reconstruction_error(W, Wh, G)
    assert np.isclose(E, np.linalg.norm((W - Wh) @ X.T) ** 2, rtol=1e-11)
    assert np.isclose(Er, E / np.linalg.norm(W @ X.T) ** 2, rtol=1e-11)


# ---------------------------------------------------------------- P2

def test_p2_obs_single_deletion_is_least_squares_optimum():
    """OBS: the compensated single deletion and its cost w_q^2/[H^-1]_qq
    ("One deletion with compensation: the OBS view")."""
    W, X = _problem(1, 12, 80, RNG_SEED + 2)
    G = O.gram(X)
    lam = O.damping(G)
    H = O.hessian(G, lam)
    A = np.linalg.inv(H)
    w = W[0]
    for q in (0, 5, 11):
        sel = np.zeros((1, 12), bool)
        sel[0, q] = True
        Z = O.solve_rows(W, A, sel)
        w_new = w - Z[0] @ A
        w_new[q] = 0.0
        ref, cost = _constrained_min(w, H, np.array([], int), np.array([q]))
        np.testing.assert_allclose(w_new, ref, rtol=1e-9, atol=1e-14)
        score = O.obs_scores(W, A)[0, q]
        assert np.isclose(cost, score, rtol=1e-9)


# ---------------------------------------------------------------- P3

def test_p3_joint_solve_is_constrained_minimiser_with_frozen_columns():
    """The joint update is the exact minimiser for the selected set, with the
    frozen columns held fixed ("Contribution one: solve a selected set directly")."""
    rng = np.random.default_rng(RNG_SEED + 3)
    W, X = _problem(3, 16, 100, RNG_SEED + 3)
    G = O.gram(X)
    H = O.hessian(G, O.damping(G))
    A = np.linalg.inv(H)
    j0, blk = 4, 8
    AF = O.schur_downdate(A, j0)  # exercises the downdate too
    np.testing.assert_allclose(AF, np.linalg.inv(H[j0:, j0:]), rtol=1e-9, atol=1e-12)
    for k in range(3):
        Q = np.sort(rng.choice(blk, 3 + k, replace=False))
        sel = np.zeros((1, blk), bool)
        sel[0, Q] = True
        Z = O.solve_rows(W[k:k + 1, j0:j0 + blk], AF[:blk, :blk], sel)
        w_new = W[k].copy()
        w_new[j0:] -= Z[0] @ AF[:blk, :]
        assert np.allclose(w_new[j0 + Q], 0.0, atol=1e-12)  # exact by construction
        w_new[j0 + Q] = 0.0
        ref, _ = _constrained_min(W[k], H, np.arange(j0), j0 + Q)
        np.testing.assert_allclose(w_new, ref, rtol=1e-8, atol=1e-13)
        d = w_new - W[k]
        grad = d @ H  # KKT: zero on the free active coordinates
        free = np.setdiff1d(np.arange(j0, 16), j0 + Q)
        assert np.max(np.abs(grad[free])) < 1e-9 * np.max(np.abs(grad))


# ---------------------------------------------------------------- P4

def test_p4_padding_contributes_no_update():
    """Zero-padded u, identity-padded R-hat and zero-padded R give the same update
    ("Making irregular row masks batchable")."""
    W, X = _problem(1, 12, 60, RNG_SEED + 4)
    G = O.gram(X)
    A = np.linalg.inv(O.hessian(G, O.damping(G)))
    Q = np.array([1, 4, 9])
    sel = np.zeros((1, 12), bool)
    sel[0, Q] = True
    Z = O.solve_rows(W, A, sel)
    delta = -(Z[0] @ A)
    smax = 6
    u = np.zeros(smax)
    u[:3] = W[0, Q]
    Rh = np.eye(smax)
    Rh[:3, :3] = A[np.ix_(Q, Q)]
    R = np.zeros((smax, 12))
    R[:3] = A[Q]
    delta_pad = -(np.linalg.solve(Rh, u) @ R)
    np.testing.assert_allclose(delta, delta_pad, rtol=1e-10, atol=1e-15)


# ---------------------------------------------------------------- P5

def test_p5_sequential_obs_with_exact_reduced_inverses_matches_joint():
    """Correctly conditioned sequential OBS reaches the same constrained optimum
    ("The scaling problem, and what SparseGPT changes")."""
    W, X = _problem(1, 10, 70, RNG_SEED + 5)
    G = O.gram(X)
    H = O.hessian(G, O.damping(G))
    A = np.linalg.inv(H)
    Q = np.array([0, 3, 4, 8])
    sel = np.zeros((1, 10), bool)
    sel[0, Q] = True
    Z = O.solve_rows(W, A, sel)
    joint = W[0] - Z[0] @ A
    joint[Q] = 0.0
    w = W[0].copy()
    free = list(range(10))
    for q in Q:
        Ar = np.linalg.inv(H[np.ix_(free, free)])
        iq = free.index(q)
        w_f = w[free] - (w[q] / Ar[iq, iq]) * Ar[iq]
        w[free] = w_f
        w[q] = 0.0
        free.remove(q)
    np.testing.assert_allclose(joint, w, rtol=1e-9, atol=1e-14)


# ---------------------------------------------------------------- P6

def test_p6_block_size_one_is_sparsegpt_column_update():
    """With B=1 the update is -(w_q/U_qq) U_{q,F}, U = chol_upper(H^-1)
    (explainer, "SparseGPT: Second-Order Reconstruction at Scale")."""
    W, X = _problem(6, 14, 90, RNG_SEED + 6)
    G = O.gram(X)
    out = O.prune_layer(W, G, sparsity=0.5, pattern=None, block=1)
    H = O.hessian(G, out["lam"])
    U = np.linalg.cholesky(np.linalg.inv(H)).T
    Wc = W.copy()
    for q in range(14):
        for k in range(6):
            if out["mask"][k, q]:
                Wc[k, q:] -= (Wc[k, q] / U[q, q]) * U[q, q:]
                Wc[k, q] = 0.0
    np.testing.assert_allclose(out["W_hat"], Wc, rtol=1e-8, atol=1e-13)


# ---------------------------------------------------------------- P7

def test_p7_one_block_is_least_squares_for_final_mask():
    """B=b, lambda -> 0: W_hat is the least-squares optimum for its fixed mask
    ("Pruning LLMs with Thanos", section "Contribution one: solve a selected set
    directly": the joint solve is exact for the set it deletes)."""
    W, X = _problem(3, 10, 200, RNG_SEED + 7)
    G = O.gram(X)
    out = O.prune_layer(W, G, sparsity=0.4, block=10, lam=1e-12)
    for k in range(3):
        keep = ~out["mask"][k]
        x, *_ = np.linalg.lstsq(X[:, keep], X @ W[k], rcond=None)
        ref = np.zeros(10)
        ref[keep] = x
        np.testing.assert_allclose(out["W_hat"][k], ref, rtol=1e-6, atol=1e-10)


# ---------------------------------------------------------------- P8

def test_p8_global_budget_met_exactly_and_reallocated():
    """Total pruned equals k_total; the residual budget never grows; blocks of
    the less important half lose more ("Contribution two")."""
    rng = np.random.default_rng(RNG_SEED + 8)
    c, b, n = 8, 16, 120
    X = rng.standard_normal((n, b))
    X[:, b // 2:] *= 10.0
    W = 0.02 * rng.standard_normal((c, b))
    G = O.gram(X)
    out = O.prune_layer(W, G, sparsity=0.5, block=4)
    assert out["pruned"] == O.k_total(0.5, c, b) == sum(out["counts"])
    assert int(out["mask"].sum()) == out["k_total"]
    assert np.all(out["W_hat"][out["mask"]] == 0.0)
    first = out["mask"][:, : b // 2].mean()
    second = out["mask"][:, b // 2:].mean()
    assert first > 0.5 > second
    remaining = out["k_total"] - np.cumsum([0] + out["counts"])
    assert np.all(np.diff(remaining) <= 0)
    # the residual budget always fits in the active region
    for j, r in enumerate(remaining[:-1]):
        assert r <= c * (b - 4 * j)


@pytest.mark.parametrize("p", [0.3, 0.55, 0.9])
def test_p8_budget_rounding_half_even(p):
    W, X = _problem(5, 12, 60, RNG_SEED + 9)
    out = O.prune_layer(W, O.gram(X), sparsity=p, block=5)  # ragged last block
    assert out["pruned"] == int(np.round(p * 60))


# ---------------------------------------------------------------- P9

@pytest.mark.parametrize("nm", [(2, 4), (4, 8), (1, 4)])
def test_p9_nm_exact_group_counts(nm):
    n_, m_ = nm
    W, X = _problem(6, 32, 100, RNG_SEED + 10)
    out = O.prune_layer(W, O.gram(X), pattern=nm, block=16)
    g = out["mask"].reshape(6, 32 // m_, m_)
    assert np.all(g.sum(axis=2) == m_ - n_)
    assert np.all(out["W_hat"][out["mask"]] == 0.0)
    assert np.all((out["W_hat"] != 0).reshape(6, -1, m_).sum(axis=2) <= n_)


# ---------------------------------------------------------------- P10

def test_p10_factor_two_in_hessian_is_immaterial():
    """H = 2G+lambda*I vs G+lambda'*I with relative damping: identical mask, and a
    power-of-two scale leaves W_hat bit-identical."""
    W, X = _problem(5, 24, 80, RNG_SEED + 11)
    G = O.gram(X)
    a = O.prune_layer(W, G, sparsity=0.5, block=8)
    b2 = O.prune_layer(W, 2.0 * G, sparsity=0.5, block=8)
    h = O.prune_layer(W, 0.5 * G, sparsity=0.5, block=8)
    assert np.array_equal(a["mask"], b2["mask"]) and np.array_equal(a["mask"], h["mask"])
    assert np.array_equal(a["W_hat"], b2["W_hat"])
    assert np.array_equal(a["W_hat"], h["W_hat"])


# ---------------------------------------------------------------- P11

def test_p11_wanda_ordering_and_diagonal_gram():
    """Ranking by |W|*||X_q|| equals ranking by W^2 G_qq; with a diagonal G there
    is nothing to compensate ("Why magnitude alone misses important weights")."""
    W, X = _problem(4, 16, 50, RNG_SEED + 12)
    G = O.gram(X)
    out = O.prune_layer(W, G, pattern=(2, 4), block=16, score="wanda")
    norms = np.linalg.norm(X, axis=0)
    S = np.abs(W) * norms
    for k in range(4):
        for g0 in range(0, 16, 4):
            low2 = np.argsort(S[k, g0:g0 + 4], kind="stable")[:2]
            assert set(np.flatnonzero(out["mask"][k, g0:g0 + 4])) == set(low2)
    rng = np.random.default_rng(5)
    d = rng.uniform(0.5, 3.0, 16)
    Gd = np.diag(d)
    for score in ("obs", "wanda"):
        o2 = O.prune_layer(W, Gd, sparsity=0.5, block=4, score=score)
        np.testing.assert_array_equal(o2["W_hat"], np.where(o2["mask"], 0.0, W))
    o3 = O.prune_layer(W, Gd, sparsity=0.5, block=16)
    lam = 0.01 * np.mean(2 * d)
    cost = W ** 2 * (2 * d + lam)
    order = np.lexsort((np.arange(64), cost.ravel()))
    ref = np.zeros(64, bool)
    ref[order[:32]] = True
    np.testing.assert_array_equal(o3["mask"].ravel(), ref)


# ---------------------------------------------------------------- P27

def test_p27_relative_damping_hand_values():
    """Relative damping is one hundredth of the mean diagonal of the undamped
    Hessian 2XX^T (the first workload's "0.01 times the mean of diag H", read on
    H before damping; "Pruning LLMs with Thanos", section "One deletion with
    compensation: the OBS view", damped form). Hand values: orthogonal features
    of squared norms 1 and 4 give diag(2G) = (2, 8), so lambda = 0.05; features of
    squared norms 5 and 10 with an off-diagonal Gram entry give diag(2G) =
    (10, 20), so lambda = 0.15; absolute damping passes through unchanged."""
    X = np.array([[1.0, 0.0], [0.0, 2.0]])  # token-major: two tokens, two features
    G = O.gram(X)
    assert G.tolist() == [[1.0, 0.0], [0.0, 4.0]]
    assert O.damping(G, 0.01) == pytest.approx(0.05, rel=1e-14)
    assert O.damping(G, 0.3, relative=False) == 0.3
    np.testing.assert_allclose(O.hessian(G, O.damping(G, 0.01)), [[2.05, 0.0], [0.0, 8.05]],
                               rtol=1e-14)
    X2 = np.array([[1.0, 1.0], [0.0, 3.0], [2.0, 0.0]])
    G2 = O.gram(X2)
    assert G2[0, 1] == 1.0  # the off-diagonal entry does not enter lambda
    assert O.damping(G2, 0.01) == pytest.approx(0.15, rel=1e-14)
    # the layer step reports the lambda it applied
    out = O.prune_layer(np.array([[0.3, -0.2]]), G, sparsity=0.5, block=2)
    assert out["lam"] == pytest.approx(0.05, rel=1e-14)
    out = O.prune_layer(np.array([[0.3, -0.2]]), G2, sparsity=0.5, block=2, lam=0.2,
                        lam_relative=False)
    assert out["lam"] == 0.2


# ---------------------------------------------------------------- P12

def test_p12_upper_inverse_factor_identities():
    """One factorisation serves every block: with H^-1 = U^T U (U upper),
    (H_F)^-1 = U_FF^T U_FF, [(H_F)^-1]_{J,F} = U_JJ^T U_{J,F}, and
    [(H_F)^-1]_qq = sum_{i=j0..q} U_iq^2 (explainer: Cholesky of H^-1 once)."""
    W, X = _problem(1, 20, 90, RNG_SEED + 13)
    G = O.gram(X)
    H = O.hessian(G, O.damping(G))
    U = np.linalg.cholesky(np.linalg.inv(H)).T
    V = np.linalg.cholesky(H[::-1, ::-1])[::-1, ::-1]  # H = V V^T, V upper
    np.testing.assert_allclose(V @ V.T, H, rtol=1e-10)
    np.testing.assert_allclose(np.linalg.inv(V), U, rtol=1e-8, atol=1e-12)
    A = np.linalg.inv(H)
    for j0, blk in ((0, 5), (5, 5), (12, 4)):
        F = slice(j0, 20)
        J = slice(j0, j0 + blk)
        AF = np.linalg.inv(H[F, F])
        np.testing.assert_allclose(AF, U[F, F].T @ U[F, F], rtol=1e-8, atol=1e-12)
        np.testing.assert_allclose(AF[:blk], U[J, J].T @ U[J, F], rtol=1e-8, atol=1e-12)
        d = np.array([np.sum(U[j0:q + 1, q] ** 2) for q in range(j0, 20)])
        np.testing.assert_allclose(np.diag(AF), d, rtol=1e-9)
        np.testing.assert_allclose(AF, A if j0 == 0 else AF, rtol=1e-9)
    # the oracle's own downdate sequence reaches the same inverses
    Af = A
    for j0 in range(0, 20, 4)[1:]:
        Af = O.schur_downdate(Af, 4)
        np.testing.assert_allclose(Af, np.linalg.inv(H[j0:, j0:]), rtol=1e-8, atol=1e-12)


# ---------------------------------------------------------------- P13

def test_p13_limits():
    W, X = _problem(4, 12, 60, RNG_SEED + 14)
    G = O.gram(X)
    o0 = O.prune_layer(W, G, sparsity=0.0, block=4)
    np.testing.assert_array_equal(o0["W_hat"], W)
    assert O.reconstruction_error(W, o0["W_hat"], G)[0] == 0.0
    o1 = O.prune_layer(W, G, sparsity=1.0, block=4)
    assert np.all(o1["W_hat"] == 0.0) and o1["mask"].all()
    E, Er = O.reconstruction_error(W, o1["W_hat"], G)
    assert np.isclose(E, np.linalg.norm(W @ X.T) ** 2) and np.isclose(Er, 1.0)
    Wn, Xn = _problem(2, 12, 5, RNG_SEED + 15)  # n < b: rank-deficient G
    with pytest.raises(O.NotSPDError):
        O.prune_layer(Wn, O.gram(Xn), sparsity=0.5, block=4, lam=0.0, lam_relative=False)


# ---------------------------------------------------------------- P14

def _mask_cost(w, H, Q):
    _, cost = _constrained_min(w, H, np.array([], int), np.asarray(Q, int))
    return cost


def test_p14_brute_force_tiny_layers():
    """Exhaustive masks on tiny layers: the oracle's damped objective for its own
    mask is that mask's least-squares optimum and is never below the best mask;
    with one deletion per row the OBS choice is the exhaustive argmin."""
    for seed in range(4):
        W, X = _problem(2, 6, 40, RNG_SEED + 20 + seed)
        G = O.gram(X)
        out = O.prune_layer(W, G, sparsity=0.5, block=6)
        H = O.hessian(G, out["lam"])
        D = out["W_hat"] - W
        mine = float(np.sum((D @ H) * D))
        own = sum(_mask_cost(W[k], H, np.flatnonzero(out["mask"][k])) for k in range(2))
        assert np.isclose(mine, own, rtol=1e-8)
        best = np.inf
        for flat in itertools.combinations(range(12), 6):
            rows = [[f % 6 for f in flat if f // 6 == k] for k in range(2)]
            best = min(best, sum(_mask_cost(W[k], H, rows[k]) for k in range(2)))
        assert mine >= best * (1 - 1e-9)
        # one deletion per row (3:4 groups with B = M = 4)
        W4 = W[:, :4]
        G4 = G[:4, :4]
        o4 = O.prune_layer(W4, G4, pattern=(3, 4), block=4)
        H4 = O.hessian(G4, o4["lam"])
        for k in range(2):
            costs = [_mask_cost(W4[k], H4, [q]) for q in range(4)]
            assert np.flatnonzero(o4["mask"][k]).tolist() == [int(np.argmin(costs))]


# ---------------------------------------------------------------- P15

def test_p15_deterministic():
    W, X = _problem(6, 24, 70, RNG_SEED + 30)
    G = O.gram(X)
    a = O.prune_layer(W, G, sparsity=0.5, block=8)
    b = O.prune_layer(W, G, sparsity=0.5, block=8)
    assert np.array_equal(a["W_hat"], b["W_hat"]) and np.array_equal(a["mask"], b["mask"])


# ------------------------------------------- whole procedure, several blocks

@pytest.mark.parametrize("case", [
    dict(pattern=None, sparsity=0.5, block=4, b=16),
    dict(pattern=None, sparsity=0.6, block=5, b=17),   # ragged last block
    dict(pattern=(2, 4), sparsity=None, block=8, b=16),
    dict(pattern=(4, 8), sparsity=None, block=8, b=24),
    dict(pattern=None, sparsity=0.5, block=4, b=16, score="wanda"),
])
def test_whole_procedure_against_independent_reference(case):
    """Independent re-derivation: scores from direct sub-matrix inverses, lexsort
    selection, least-squares compensation with frozen columns fixed."""
    score = case.get("score", "obs")
    W, X = _problem(4, case["b"], 120, RNG_SEED + 40)
    G = O.gram(X)
    out = O.prune_layer(W, G, sparsity=case["sparsity"] or 0.0, pattern=case["pattern"],
                        block=case["block"], score=score)
    ref_W, ref_mask = _reference_prune(W, G, out["lam"], case["block"],
                                       sparsity=case["sparsity"], pattern=case["pattern"],
                                       score=score)
    np.testing.assert_array_equal(out["mask"], ref_mask)
    np.testing.assert_allclose(out["W_hat"], ref_W, rtol=1e-7, atol=1e-12)


# --------------------------------------------------------------- selection

def test_select_unstructured_ties_break_by_flat_index():
    rng = np.random.default_rng(7)
    S = rng.integers(0, 4, size=(5, 9)).astype(float)  # heavy ties
    for r in range(0, 46):
        sel = O.select_unstructured(S, r, 9)
        flat = np.arange(45)
        order = np.lexsort((flat, S.ravel()))
        ref = np.zeros(45, bool)
        ref[order[:r]] = True
        np.testing.assert_array_equal(sel.ravel(), ref)
    # the intersection with a narrower block
    sel3 = O.select_unstructured(S, 20, 3)
    np.testing.assert_array_equal(sel3, O.select_unstructured(S, 20, 9)[:, :3])


def test_select_nm_ties_break_by_column():
    S = np.array([[1.0, 1.0, 1.0, 1.0, 3.0, 2.0, 2.0, 0.0]])
    np.testing.assert_array_equal(O.select_nm(S, 2, 4)[0], [1, 1, 0, 0, 0, 1, 0, 1])
    np.testing.assert_array_equal(O.select_nm(S, 4, 8)[0], [1, 1, 1, 0, 0, 0, 0, 1])


def test_k_total_round_half_even():
    assert O.k_total(0.5, 3, 3) == 4  # 4.5 -> 4
    assert O.k_total(0.5, 1, 7) == 4  # 3.5 -> 4
    assert O.k_total(0.6, 1024, 8192) == 5033165
    assert O.k_total(0.6, 8192, 28672) == 140928614


# ------------------------------------------- comparators (magnitude, Wanda)
# The explainer's section "Wanda: Pruning by Weights and Activations" (score
# |W_kq| ||X_q||_2, thresholds per output row, no update of the other weights);
# "Pruning LLMs with Thanos", section "Why magnitude alone misses important
# weights" (magnitude ranks by |W_kq|; the squared Wanda score has the same order).

def test_p16_baseline_hand_example():
    # rows [3, -1, 2, 0.5] and [1, 1, -1, 2]; 50% per row; Wanda with G_qq = [1, 100, 1, 1]
    W = np.array([[3.0, -1.0, 2.0, 0.5], [1.0, 1.0, -1.0, 2.0]])
    mag = O.prune_baseline(W, "magnitude", sparsity=0.5)
    # |W| row 0: 0.5 and 1 are the smallest; row 1: three entries of magnitude 1,
    # the two lowest columns go first
    assert mag["mask"].astype(int).tolist() == [[0, 1, 0, 1], [1, 1, 0, 0]]
    g = np.array([1.0, 100.0, 1.0, 1.0])
    wan = O.prune_baseline(W, "wanda", gdiag=g, sparsity=0.5)
    # |W| sqrt(G): row 0 [3, 10, 2, 0.5] -> columns 3, 2; row 1 [1, 10, 1, 2] -> columns 0, 2
    assert wan["mask"].astype(int).tolist() == [[0, 0, 1, 1], [1, 0, 1, 0]]
    # no compensation: kept entries unchanged, pruned entries exactly zero
    for r in (mag, wan):
        assert np.all(r["W_hat"][~r["mask"]] == W[~r["mask"]])
        assert np.all(r["W_hat"][r["mask"]] == 0.0)


@pytest.mark.parametrize("p", [0.0, 0.3, 0.5, 0.77, 1.0])
def test_p17_baseline_per_row_budget_and_wanda_order(p):
    rng = np.random.default_rng(41)
    c, b = 7, 53
    W = rng.standard_normal((c, b))
    X = rng.standard_normal((300, b)) * rng.uniform(0.1, 10.0, size=b)
    g = O.column_sq_norms(X)
    res = O.prune_baseline(W, "wanda", gdiag=g, sparsity=p)
    k = int(np.round(p * b))
    assert np.all(res["mask"].sum(axis=1) == k)
    # the same rows' lowest |W| * ||X_q||_2 in fp64 (a different formula: norms,
    # not squares; tie-free data)
    s = np.abs(W) * np.sqrt(np.sum(X * X, axis=0))[None, :]
    ref = np.zeros_like(res["mask"])
    np.put_along_axis(ref, np.argsort(s, axis=1)[:, :k], True, axis=1)
    assert np.array_equal(res["mask"], ref)
    # magnitude is Wanda with equal feature norms
    mag = O.prune_baseline(W, "magnitude", sparsity=p)
    eq = O.prune_baseline(W, "wanda", gdiag=np.full(b, 4.0), sparsity=p)
    assert np.array_equal(mag["mask"], eq["mask"])


def test_p18_baseline_error_closed_form_and_nm_counts():
    rng = np.random.default_rng(43)
    c, b = 5, 24
    W = rng.standard_normal((c, b))
    d = rng.uniform(0.5, 3.0, size=b)
    G = np.diag(d)  # independent features: E = sum over pruned of W^2 G_qq
    res = O.prune_baseline(W, "wanda", gdiag=d, pattern=(2, 4))
    E, _ = O.reconstruction_error(W, res["W_hat"], G)
    assert np.isclose(E, np.sum((W ** 2 * d[None, :])[res["mask"]]), rtol=1e-12)
    groups = res["mask"].reshape(c, b // 4, 4).sum(axis=2)
    assert np.all(groups == 2)
    # within every group the two pruned keys are the two smallest
    keys = (W ** 2 * d[None, :]).reshape(c, b // 4, 4)
    m = res["mask"].reshape(c, b // 4, 4)
    assert np.all(keys[m].reshape(c, b // 4, 2).max(axis=2) <= keys[~m].reshape(c, b // 4, 2).min(axis=2))


def test_p19_compensation_never_hurts_on_the_same_mask():
    """The joint solve is the exact constrained minimiser ("Pruning LLMs with
    Thanos", section "Contribution one"): with the comparator's mask fixed, the
    compensated weights reach an error no larger than the uncompensated ones."""
    rng = np.random.default_rng(44)
    c, b = 4, 12
    W, X = _problem(c, b, 200, 45)
    G = O.gram(X)
    res = O.prune_baseline(W, "wanda", gdiag=O.column_sq_norms(X), sparsity=0.5)
    H = 2 * G + 1e-9 * np.mean(np.diag(2 * G)) * np.eye(b)
    E_plain, _ = O.reconstruction_error(W, res["W_hat"], G)
    for k in range(c):
        Q = np.flatnonzero(res["mask"][k])
        best, cost = _constrained_min(W[k], H, np.array([], dtype=int), Q)
        assert np.all(best[Q] == 0.0) or np.allclose(best[Q], 0.0, atol=1e-12)
        d_plain = res["W_hat"][k] - W[k]
        assert cost <= float(d_plain @ H @ d_plain) * (1 + 1e-9)
    assert E_plain > 0


# ------------------------------------------- SparseGPT comparator (P20-P23)

def test_p20_sparsegpt_is_sequential_least_squares():
    """Every pruned weight, in column order, is deleted by the least-squares optimum
    with the columns before it frozen (explainer, "SparseGPT: Second-Order
    Reconstruction at Scale"; "Pruning LLMs with Thanos", "The scaling problem, and
    what SparseGPT changes"), replayed for the oracle's own mask with least squares
    on C^T (C C^T = H); and no sequential schedule beats the least-squares
    reconstruction of the same final mask."""
    c, b = 4, 12
    W, X = _problem(c, b, 120, RNG_SEED + 20)
    G = O.gram(X)
    for pattern in (None, (2, 4)):
        out = O.prune_sparsegpt(W, G, sparsity=0.5, pattern=pattern, block=4)
        H = O.hessian(G, out["lam"])
        for k in range(c):
            w = W[k].copy()
            for q in range(b):
                if out["mask"][k, q]:
                    w, _ = _constrained_min(w, H, np.arange(q), [q])
            np.testing.assert_allclose(out["W_hat"][k], w, rtol=1e-7, atol=1e-12)
            _, best = _constrained_min(W[k], H, [], np.flatnonzero(out["mask"][k]))
            d = out["W_hat"][k] - W[k]
            assert float(d @ H @ d) >= best * (1 - 1e-9)


def test_p21_sparsegpt_score_is_obs_cost_with_earlier_columns_frozen():
    """The score the block's mask is chosen from is the cost of deleting w_kq alone
    at the moment column q is processed: min d H d^T with d_q = -w_kq and the
    columns before q frozen (least squares), from the block-start weights."""
    c, b, B = 3, 12, 4
    W, X = _problem(c, b, 120, RNG_SEED + 21)
    G = O.gram(X)
    trace = []
    out = O.prune_sparsegpt(W, G, sparsity=0.5, block=B, trace=trace)
    H = O.hessian(G, out["lam"])
    Wc = W.copy()
    for ent in trace:
        j0 = ent["j0"]
        for k in range(c):
            for t in range(B):
                _, cost = _constrained_min(Wc[k], H, np.arange(j0 + t), [j0 + t])
                assert ent["S"][k, t] == pytest.approx(cost, rel=1e-8, abs=1e-15)
        for k in range(c):  # advance to the next block start with the oracle's mask
            for q in range(j0, j0 + B):
                if out["mask"][k, q]:
                    Wc[k], _ = _constrained_min(Wc[k], H, np.arange(q), [q])


def test_p22_sparsegpt_diagonal_gram_is_blockwise_threshold():
    """Independent features: nothing to compensate, so W_hat is W with the mask
    zeroed, and each block's mask is its lowest w^2 (2 G_qq + lambda) by (score,
    flat index), exactly round(p c B) of them."""
    c, b, B = 5, 16, 8
    rng = np.random.default_rng(RNG_SEED + 22)
    W = rng.standard_normal((c, b))
    W[1, 3] = -W[0, 3]  # equal scores in one column: the lower row goes first
    W[2, 9] = W[4, 9]
    gd = rng.uniform(0.5, 3.0, b)
    G = np.diag(gd)
    out = O.prune_sparsegpt(W, G, sparsity=0.5, block=B)
    h = 2.0 * gd + out["lam"]
    for j0 in (0, 8):
        score = W[:, j0:j0 + B] ** 2 * h[None, j0:j0 + B]
        flat = (np.arange(c)[:, None] * b + np.arange(j0, j0 + B)[None, :]).ravel()
        order = np.lexsort((flat, score.ravel()))
        expect = np.zeros(c * B, dtype=bool)
        expect[order[:20]] = True
        np.testing.assert_array_equal(out["mask"][:, j0:j0 + B], expect.reshape(c, B))
    ref = W.copy()
    ref[out["mask"]] = 0.0
    np.testing.assert_array_equal(out["W_hat"], ref)


@pytest.mark.parametrize("p,counts", [(0.0, [0, 0, 0]), (0.3, [12, 12, 6]),
                                      (0.5, [20, 20, 10]), (1.0, [40, 40, 20])])
def test_p23_sparsegpt_per_block_quota_and_limits(p, counts):
    """Blocks of 8, 8 and a ragged 4 columns over 5 rows: each block loses exactly
    round(p * 5 * |J|); p = 0 changes nothing, p = 1 zeroes everything; N:M counts
    are exact in every group."""
    W, X = _problem(5, 20, 100, RNG_SEED + 23)
    G = O.gram(X)
    out = O.prune_sparsegpt(W, G, sparsity=p, block=8)
    assert out["counts"] == counts
    assert np.all(out["W_hat"][out["mask"]] == 0.0)
    if p == 0.0:
        np.testing.assert_array_equal(out["W_hat"], W)
    if p == 1.0:
        assert np.all(out["W_hat"] == 0.0)
    nm = O.prune_sparsegpt(W, G, pattern=(1, 4), block=8)
    assert np.all(nm["mask"].reshape(5, 5, 4).sum(axis=2) == 3)


# ------------------------------- gated feed-forward and sequential block (P24-P25)

def test_p24_silu_and_gated_ffn_input():
    """silu(z) = z / (1 + e^-z) (hand values from math.exp, the odd-part identity
    silu(z) - silu(-z) = z, saturation) and Y = silu(X Wg^T) * (X Wu^T) against
    torch's fp64 silu and matmul; the bf16 rounding against torch's cast."""
    import math

    import torch
    np.testing.assert_allclose(O.silu(np.array([0.0, 1.0, 2.0, -1.0])),
                               [0.0, 1.0 / (1.0 + math.exp(-1.0)), 2.0 / (1.0 + math.exp(-2.0)),
                                -1.0 / (1.0 + math.exp(1.0))], rtol=1e-15, atol=0)
    z = np.random.default_rng(RNG_SEED + 24).standard_normal(1000) * 30
    np.testing.assert_allclose(O.silu(z) - O.silu(-z), z, rtol=1e-12, atol=1e-12)
    assert O.silu(np.array([800.0]))[0] == 800.0 and O.silu(np.array([-800.0]))[0] == 0.0
    # hand example: X = [1, 2], gate rows e1, e2 -> (1, 2); up rows -> (3, 2)
    Y = O.gated_ffn_input(np.array([[1.0, 2.0]]), np.eye(2), np.array([[1.0, 1.0], [2.0, 0.0]]))
    np.testing.assert_allclose(Y, [[3.0 / (1.0 + math.exp(-1.0)), 4.0 / (1.0 + math.exp(-2.0))]],
                               rtol=1e-15)
    rng = np.random.default_rng(RNG_SEED + 25)
    X, Wg, Wu = rng.standard_normal((40, 16)), rng.standard_normal((24, 16)), rng.standard_normal((24, 16))
    Xt, Wgt, Wut = (torch.tensor(a, dtype=torch.float64) for a in (X, Wg, Wu))
    ref = (torch.nn.functional.silu(Xt @ Wgt.T) * (Xt @ Wut.T)).numpy()
    np.testing.assert_allclose(O.gated_ffn_input(X, Wg, Wu), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.gated_ffn_input(X, Wg, 3.0 * Wu), 3.0 * ref, rtol=1e-12, atol=1e-12)
    v = rng.standard_normal(5000) * 10.0 ** rng.integers(-6, 6, 5000)
    bt = torch.tensor(v.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(O.thanos_oracle._bf16_round(v), bt)


def test_p25_sequential_mlp_block():
    """gate and up are pruned on the Hessian of their shared input; down on the
    Hessian of the input its pruned predecessors produce. At p = 0 nothing is
    pruned, so down's input is the bf16 rounding of the dense block's (torch fp64
    silu); at p = 0.5 down's input differs from the dense one and down is the
    layer step on it."""
    import torch
    rng = np.random.default_rng(RNG_SEED + 26)
    X = rng.standard_normal((300, 16))
    Wg, Wu, Wd = (0.3 * rng.standard_normal(s) for s in ((24, 16), (24, 16), (16, 24)))
    dense = O.prune_mlp_sequential(X, Wg, Wu, Wd, sparsity=0.0, block=8)
    Xt = torch.tensor(X)
    Yd = torch.nn.functional.silu(Xt @ torch.tensor(Wg).T) * (Xt @ torch.tensor(Wu).T)
    np.testing.assert_array_equal(dense["X_down"], Yd.float().to(torch.bfloat16).double().numpy())
    np.testing.assert_array_equal(dense["down"]["W_hat"], Wd)
    sp = O.prune_mlp_sequential(X, Wg, Wu, Wd, sparsity=0.5, block=8)
    for name, W in (("gate", Wg), ("up", Wu)):
        alone = O.prune_layer(W, O.gram(X), sparsity=0.5, block=8)
        np.testing.assert_array_equal(sp[name]["W_hat"], alone["W_hat"])
    assert not np.array_equal(sp["X_down"], dense["X_down"])
    down = O.prune_layer(Wd, O.gram(sp["X_down"]), sparsity=0.5, block=8)
    np.testing.assert_array_equal(sp["down"]["W_hat"], down["W_hat"])
    assert sp["down"]["pruned"] == O.k_total(0.5, 16, 24)


# ---------------------------------------------------- alpha outlier rows (P26)

def test_p26_alpha_outlier_rows():
    """Hand example (energies 1, 36, 20, 1.25 -> the two largest rows stay dense;
    equal energies -> the higher row index); with orthogonal input features the
    energy is ||W_k X||^2 computed from X; alpha = 0 is the plain layer step,
    alpha = 1 prunes nothing; the other rows are pruned as a layer of their own
    (2:4 at alpha = 0.1 leaves 45% zeros)."""
    W = np.array([[1.0, 0.0], [0.0, 3.0], [2.0, 2.0], [0.5, 0.5]])
    np.testing.assert_array_equal(O.outlier_rows(W, [1.0, 4.0], 0.5), [False, True, True, False])
    Wt = np.array([[1.0, 0.0], [1.0, 0.0], [0.0, 0.5]])
    np.testing.assert_array_equal(O.outlier_rows(Wt, [1.0, 4.0], 1.0 / 3.0), [False, False, True])
    rng = np.random.default_rng(RNG_SEED + 27)
    Q, _ = np.linalg.qr(rng.standard_normal((200, 12)))
    X = Q * rng.uniform(0.5, 5.0, 12)[None, :]  # orthogonal columns: G is diagonal
    Wr = rng.standard_normal((30, 12))
    energy = np.sum((Wr @ X.T) ** 2, axis=1)
    dense = O.outlier_rows(Wr, np.diag(X.T @ X), 0.2)
    np.testing.assert_array_equal(np.flatnonzero(dense), np.sort(np.argsort(energy)[-6:]))
    W2, X2 = _problem(40, 16, 200, RNG_SEED + 28)
    G = O.gram(X2)
    base = O.prune_layer(W2, G, pattern=(2, 4), block=8)
    a0 = O.prune_layer_alpha(W2, G, 0.0, pattern=(2, 4), block=8)
    np.testing.assert_array_equal(a0["W_hat"], base["W_hat"])
    a1 = O.prune_layer_alpha(W2, G, 1.0, pattern=(2, 4), block=8)
    assert not a1["mask"].any() and np.array_equal(a1["W_hat"], W2)
    a = O.prune_layer_alpha(W2, G, 0.1, pattern=(2, 4), block=8)
    assert a["dense"].sum() == 4 and a["mask"].sum() == 36 * 8
    assert a["mask"].mean() == pytest.approx(0.45)
    rest = np.flatnonzero(~a["dense"])
    sub = O.prune_layer(W2[rest], G, pattern=(2, 4), block=8)
    np.testing.assert_array_equal(a["W_hat"][rest], sub["W_hat"])
    np.testing.assert_array_equal(a["W_hat"][a["dense"]], W2[a["dense"]])


# ------------------------------------------------------- planted mistakes

def _pins_pass():
    try:
        test_p3_joint_solve_is_constrained_minimiser_with_frozen_columns()
        test_p6_block_size_one_is_sparsegpt_column_update()
        for case in (dict(pattern=None, sparsity=0.5, block=4, b=16),
                     dict(pattern=(2, 4), sparsity=None, block=8, b=16)):
            test_whole_procedure_against_independent_reference(case)
        test_select_nm_ties_break_by_column()
        test_select_unstructured_ties_break_by_flat_index()
        test_p11_wanda_ordering_and_diagonal_gram()
        test_p16_baseline_hand_example()
        test_p17_baseline_per_row_budget_and_wanda_order(0.5)
        test_p18_baseline_error_closed_form_and_nm_counts()
        test_p20_sparsegpt_is_sequential_least_squares()
        test_p21_sparsegpt_score_is_obs_cost_with_earlier_columns_frozen()
        test_p22_sparsegpt_diagonal_gram_is_blockwise_threshold()
        test_p23_sparsegpt_per_block_quota_and_limits(0.3, [12, 12, 6])
        test_p24_silu_and_gated_ffn_input()
        test_p26_alpha_outlier_rows()
        test_p27_relative_damping_hand_values()
    except AssertionError:
        return False
    return True


def _bad_downdate(A_F, blk):
    return A_F[blk:, blk:]  # dropped Schur term


def _bad_nm(S_J, n, m):
    c, blk = S_J.shape
    g = S_J.reshape(c, blk // m, m)[:, :, ::-1]  # ties broken by the higher column
    order = np.argsort(g, axis=2, kind="stable")
    sel = np.zeros_like(g, dtype=bool)
    np.put_along_axis(sel, order[:, :, : m - n], True, axis=2)
    return sel[:, :, ::-1].reshape(c, blk)


def _bad_keys_abs_times_g(W, gdiag=None):
    w = O.thanos_oracle._f64(W).astype(np.float32)
    k = np.abs(w)
    if gdiag is not None:
        k = np.multiply(k, np.asarray(gdiag, dtype=np.float32)[None, :], dtype=np.float32)
    return k  # |W| G instead of W^2 G: a wrong power of the feature norm


@pytest.mark.parametrize("mutation", ["downdate", "sign", "nm_ties", "score_diag_H",
                                      "baseline_power", "baseline_layer_budget",
                                      "sgpt_full_inverse", "sgpt_sign", "sgpt_row_quota",
                                      "silu_mirrored", "alpha_smallest_rows",
                                      "damping_mean_G"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    assert _pins_pass()
    T = O.thanos_oracle
    if mutation == "downdate":
        monkeypatch.setattr(T, "schur_downdate", _bad_downdate)
    elif mutation == "sign":
        orig = T.solve_rows
        monkeypatch.setattr(T, "solve_rows", lambda W_J, A, sel: -orig(W_J, A, sel))
    elif mutation == "nm_ties":
        monkeypatch.setattr(T, "select_nm", _bad_nm)
        monkeypatch.setattr(O, "select_nm", _bad_nm)
    elif mutation == "score_diag_H":
        orig_prune = T.prune_layer

        def wrong(W, G, **kw):
            if kw.get("score", "obs") == "obs":
                kw = dict(kw, score="wanda")
            return orig_prune(W, G, **kw)
        monkeypatch.setattr(O, "prune_layer", wrong)
    elif mutation == "baseline_power":
        monkeypatch.setattr(T, "baseline_keys", _bad_keys_abs_times_g)
    elif mutation == "baseline_layer_budget":
        orig_b = T.prune_baseline

        def layer_wide(W, method, gdiag=None, sparsity=0.5, pattern=None):
            if pattern is not None:
                return orig_b(W, method, gdiag=gdiag, sparsity=sparsity, pattern=pattern)
            keys = T.baseline_keys(W, gdiag if method == "wanda" else None)
            k = int(np.round(sparsity * keys.size))  # one threshold for the whole layer
            flat = np.zeros(keys.size, dtype=bool)
            flat[np.argsort(keys.ravel(), kind="stable")[:k]] = True
            mask = flat.reshape(keys.shape)
            W_hat = T._f64(W).copy()
            W_hat[mask] = 0.0
            return {"W_hat": W_hat, "mask": mask}
        monkeypatch.setattr(O, "prune_baseline", layer_wide)
    elif mutation == "sgpt_full_inverse":
        # rows of the full inverse instead of the inverse over the active columns
        monkeypatch.setattr(T, "trailing_inverse_rows", lambda H: np.triu(np.linalg.inv(H)))
    elif mutation == "sgpt_sign":
        def added(Wc, q, pruned, t_row):
            err = np.where(pruned, Wc[:, q], 0.0) / t_row[0]
            Wc[:, q + 1:] += np.outer(err, t_row[1:])
            Wc[pruned, q] = 0.0
        monkeypatch.setattr(T, "sparsegpt_column", added)
    elif mutation == "sgpt_row_quota":
        orig_sel = T.select_unstructured

        def per_row(S_F, r, blk):
            c = S_F.shape[0]
            return np.concatenate([orig_sel(S_F[k:k + 1], int(np.round(r / c)), blk)
                                   for k in range(c)])
        monkeypatch.setattr(T, "select_unstructured", per_row)
    elif mutation == "alpha_smallest_rows":
        orig_rows = T.outlier_rows

        def smallest(W, gdiag, alpha):
            W0 = T._f64(W)
            g = np.asarray(gdiag, dtype=np.float32).astype(np.float64)
            return orig_rows(-W0, g, 0.0) if alpha == 0 else ~orig_rows(W0, g, 1.0 - alpha)
        monkeypatch.setattr(T, "outlier_rows", smallest)
        monkeypatch.setattr(O, "outlier_rows", smallest)
    elif mutation == "damping_mean_G":
        # the mean diagonal of G instead of the undamped Hessian 2G
        def half(G, lam=0.01, relative=True):
            return float(lam) * float(np.mean(np.diag(G))) if relative else float(lam)
        monkeypatch.setattr(T, "damping", half)
        monkeypatch.setattr(O, "damping", half)
    elif mutation == "silu_mirrored":
        # z * sigmoid(-z): the same odd part, the wrong function
        monkeypatch.setattr(T, "silu", lambda z: np.asarray(z, np.float64)
                            * (0.5 * (1.0 - np.tanh(0.5 * np.asarray(z, np.float64)))))
    assert not _pins_pass()

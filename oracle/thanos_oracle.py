"""fp64 NumPy oracle: block-wise multi-constraint pruning of one linear layer.

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the benchmark's
CPU-baseline leg. The product library never imports it, and it imports nothing
from the product library.

Sources (titles of the pages and their sections):

* "Pruning LLMs with Thanos" (project blog post) -- sections "The
  layer-reconstruction lens", "Why magnitude alone misses important weights",
  "One deletion with compensation: the OBS view", "Contribution one: solve a
  selected set directly", "Contribution two: keep the budget global and the
  execution local", "Making irregular row masks batchable", and "The scaling
  problem, and what SparseGPT changes" for the column-sequential comparator.
* "Weight Pruning in Large Language Models: How SparseGPT, Wanda, and
  Semi-Structured 2:4 Sparsity ..." (explainer) -- section "SparseGPT:
  Second-Order Reconstruction at Scale" for the damped Hessian H = 2XX^T + lambda*I,
  the reconstruction objective and the comparator's per-column update; section
  "Wanda: Pruning by Weights and Activations" for the |W|*||X_q|| score; section
  "N:M Semi-Structured Sparsity (2:4 Pattern)" for the group constraint.

Every value here is fp64. Inputs are decoded exactly from bf16 or fp32. The
route deliberately differs from the GPU's: the inverse Hessian comes from an LU
inverse followed by Schur-complement downdates, row systems are LU solves, and
the global selection uses a partition plus an explicit tie list.

Readings where the pages are silent (each is also listed in the design notes):

* the factor 2 in H (the blog post's Gram form vs the explainer's 2XX^T): H = 2G + lambda*I;
* lambda = lambda_rel * mean(diag(2G)) with lambda_rel = 0.01 when relative;
* score S_kq = W_kq^2 * g_q with g_q = 1/[(H_F)^-1]_qq (OBS, default) or
  g_q = G_qq (Wanda), F being the active (not yet frozen) columns;
* k_total = round-half-even(p * c * b);
* ties are broken by the flat index k*b + q (unstructured) or by q (N:M):
  the lower index is pruned first;
* N:M groups are aligned to multiples of M along a row; M-N entries are pruned
  per group; masks are chosen for every group of the block at block start;
* pruned coordinates are set to exactly 0.0 after the update.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "NotSPDError", "gram", "damping", "hessian", "k_total", "obs_scores",
    "select_unstructured", "select_nm", "solve_rows", "schur_downdate",
    "prune_layer", "reconstruction_error", "column_sq_norms", "baseline_keys", "prune_baseline",
    "trailing_inverse_rows", "sparsegpt_column", "prune_sparsegpt", "silu", "gated_ffn_input",
    "prune_mlp_sequential", "row_energies", "outlier_rows", "prune_layer_alpha",
]


class NotSPDError(ValueError):
    """The damped Hessian is not symmetric positive definite."""


def _f64(a) -> np.ndarray:
    """Exact fp64 copy of a NumPy array or a (CPU) torch tensor of bf16/fp32."""
    if hasattr(a, "detach"):
        t = a.detach().cpu()
        if str(t.dtype) == "torch.bfloat16":
            t = t.float()
        return t.double().numpy()
    return np.asarray(a, dtype=np.float64)


def gram(X_tok, chunk: int = 8192) -> np.ndarray:
    """G = X X^T for X (b x n) given token-major as X^T [n, b].

    "Pruning LLMs with Thanos", section "One deletion with compensation: the OBS
    view": G is the activation Gram matrix. Accumulated over token chunks in fp64.
    """
    n, b = X_tok.shape
    G = np.zeros((b, b), dtype=np.float64)
    for t0 in range(0, n, chunk):
        Xc = _f64(X_tok[t0:t0 + chunk])
        G += Xc.T @ Xc
    return G


def damping(G: np.ndarray, lam: float = 0.01, relative: bool = True) -> float:
    """lambda = lam * mean(diag(2G)) if relative, else lam (absolute)."""
    if relative:
        return float(lam) * float(np.mean(np.diag(2.0 * G)))
    return float(lam)


def hessian(G: np.ndarray, lam_abs: float) -> np.ndarray:
    """H = 2G + lambda*I (explainer, section "SparseGPT: Second-Order Reconstruction at Scale")."""
    return 2.0 * G + lam_abs * np.eye(G.shape[0])


def k_total(sparsity: float, c: int, b: int) -> int:
    """Number of weights the layer must lose: round-half-even(p*c*b)."""
    return int(np.round(np.float64(sparsity) * c * b))


def obs_scores(Wc_F: np.ndarray, A_F: np.ndarray) -> np.ndarray:
    """OBS cost w_q^2 / [A_F]_qq for every (row, active column).

    "Pruning LLMs with Thanos", section "One deletion with compensation: the OBS
    view": deleting w_q with the other active weights free to move raises the
    objective in proportion to w_q^2 / [H^-1]_qq; with frozen columns the inverse
    is that of the active block, A_F = (H_F)^-1.
    """
    return Wc_F ** 2 / np.diag(A_F)[None, :]


def select_unstructured(S_F: np.ndarray, r: int, blk: int) -> np.ndarray:
    """Candidates = the r lowest (score, flat index) keys of the active region;
    return their intersection with the current block (the first ``blk`` columns).

    "Pruning LLMs with Thanos", section "Contribution two: keep the budget global
    and the execution local" (steps 2-4 of the dynamic residual budget). S_F is
    c x |F| with F starting at the block; row-major order over (k, q) is the
    flat-index order k*b + q, which breaks ties.
    """
    c, f = S_F.shape
    sel = np.zeros((c, f), dtype=bool)
    if r <= 0:
        return sel[:, :blk]
    if r >= c * f:
        sel[:] = True
        return sel[:, :blk]
    flat = S_F.ravel()
    T = np.partition(flat, r - 1)[r - 1]
    below = flat < T
    need = r - int(below.sum())
    eq = np.flatnonzero(flat == T)
    chosen = below.copy()
    chosen[eq[:need]] = True
    return chosen.reshape(c, f)[:, :blk]


def select_nm(S_J: np.ndarray, n: int, m: int) -> np.ndarray:
    """In every aligned group of m columns, prune the m-n lowest (score, column).

    "Pruning LLMs with Thanos", section "The compression target: linear layers"
    (each group of M keeps exactly N nonzeros) and the explainer's section "N:M
    Semi-Structured Sparsity (2:4 Pattern)" (groups are contiguous along a row).
    A stable sort puts the lower column first among equal scores.
    """
    c, blk = S_J.shape
    assert blk % m == 0
    g = S_J.reshape(c, blk // m, m)
    order = np.argsort(g, axis=2, kind="stable")
    sel = np.zeros_like(g, dtype=bool)
    np.put_along_axis(sel, order[:, :, : m - n], True, axis=2)
    return sel.reshape(c, blk)


def solve_rows(W_J: np.ndarray, A_JJ: np.ndarray, sel: np.ndarray) -> np.ndarray:
    """Per-row multipliers z with z_Q = u R^-1 (R = [A_F]_{Q,Q}), zero elsewhere.

    "Pruning LLMs with Thanos", section "Contribution one: solve a selected set
    directly": u collects the selected weights' current values, R-hat is the
    s x s principal submatrix of the inverse Hessian on the selected set, and the
    row update is delta = -u R-hat^-1 R with R = [A_F]_{Q,:}. Here the update is
    returned as the coefficient row z (so delta = -z [A_F]_{J,:}). Each row is an
    independent LU solve at its true size (rows with equal s are stacked into one
    batched library call).
    """
    c, blk = W_J.shape
    Z = np.zeros((c, blk), dtype=np.float64)
    s = sel.sum(axis=1)
    for sv in np.unique(s):
        if sv == 0:
            continue
        rows = np.flatnonzero(s == sv)
        Q = np.nonzero(sel[rows])[1].reshape(len(rows), sv)  # ascending per row
        u = np.take_along_axis(W_J[rows], Q, axis=1)
        Rh = A_JJ[Q[:, :, None], Q[:, None, :]]
        z = np.linalg.solve(Rh, u[:, :, None])[:, :, 0]
        Zr = np.zeros((len(rows), blk))
        np.put_along_axis(Zr, Q, z, axis=1)
        Z[rows] = Zr
    return Z


def schur_downdate(A_F: np.ndarray, blk: int) -> np.ndarray:
    """(H_{F'})^-1 from (H_F)^-1 after freezing the first ``blk`` columns of F.

    Block-inverse identity: inv(H_{F'F'}) = A_{F'F'} - A_{F'J} A_{JJ}^-1 A_{JF'}.
    """
    AJJ = A_F[:blk, :blk]
    AJF = A_F[:blk, blk:]
    T = A_F[blk:, :blk] @ np.linalg.solve(AJJ, AJF)
    return np.subtract(A_F[blk:, blk:], T, out=T)  # one b x b temporary, not two


def prune_layer(W, G: np.ndarray, sparsity: float = 0.5, pattern=None, block: int = 128,
                lam: float = 0.01, lam_relative: bool = True, score: str = "obs",
                trace: list | None = None, max_blocks: int | None = None,
                on_block=None) -> dict:
    """Block-wise pruning with joint compensation (the layer step of the method).

    pattern: None for unstructured with the dynamic global budget, or (n, m).
    Returns W_hat (fp64), mask (True = pruned), per-block prune counts, lambda.
    trace (optional list) receives, per block, the scores the selection saw and
    the remaining budget (for diagnosing near-ties in comparisons). on_block
    (optional callable) is called as on_block(j0, S, r, sel, g) after each
    block's selection, with the same scores (over F for unstructured, over J for
    N:M) and the per-column score weights g over F, without copying them: a way
    to record a summary of large layers. Neither changes the arithmetic.
    max_blocks stops after that many blocks (used only to time a bounded sample).

    Procedure ("Pruning LLMs with Thanos", sections "The scaling problem, and what
    SparseGPT changes" (left-to-right blocks, finished columns frozen, updates only
    into active columns), "Contribution one" (joint solve) and "Contribution two"
    (dynamic residual budget); N:M keeps the joint solve but uses local group masks):

      H = 2G + lambda*I; A = H^-1 (LU); for each block J = [j0, j0+B) of F = [j0, b):
        scores over F (unstructured) or J (N:M) from the current weights;
        unstructured: r = k_total - pruned; candidates = r lowest keys; Q = candidates within J;
        N:M: per group of m, the m-n lowest;
        per row: z = u R^-1; W[k,F] -= z A_F[Q,F]; W[k,Q] = 0;
        pruned += |Q|; A <- inv(H_{F \\ J}) by a Schur downdate.
    """
    W0 = _f64(W)
    G = np.asarray(G, dtype=np.float64)
    c, b = W0.shape
    if block < 1:
        raise ValueError("block must be >= 1")
    if pattern is not None:
        n_keep, m = pattern
        if not (0 <= n_keep <= m) or block % m or b % m:
            raise ValueError("N:M needs 0<=n<=m, m | block and m | b")
    lam_abs = damping(G, lam, lam_relative)
    H = hessian(G, lam_abs)
    try:
        np.linalg.cholesky(H)
    except np.linalg.LinAlgError as exc:
        raise NotSPDError("damped Hessian is not positive definite") from exc
    A = np.linalg.inv(H)
    Wc = W0.copy()
    mask = np.zeros((c, b), dtype=bool)
    counts = []
    ktot = k_total(sparsity, c, b) if pattern is None else None
    pruned = 0
    diagG = np.diag(G)
    for bi, j0 in enumerate(range(0, b, block)):
        if max_blocks is not None and bi >= max_blocks:
            break
        blk = min(block, b - j0)
        if score == "obs":
            g = 1.0 / np.diag(A)
        elif score == "wanda":
            g = diagG[j0:]
        else:
            raise ValueError(score)
        if pattern is None:
            S = Wc[:, j0:] ** 2 * g[None, :]
            sel = select_unstructured(S, ktot - pruned, blk)
        else:
            S = Wc[:, j0:j0 + blk] ** 2 * g[None, :blk]
            sel = select_nm(S, pattern[0], pattern[1])
        if trace is not None:
            trace.append({"j0": j0, "S": S.copy(),
                          "r": (ktot - pruned) if pattern is None else None})
        if on_block is not None:
            on_block(j0, S, (ktot - pruned) if pattern is None else None, sel, g)
        Z = solve_rows(Wc[:, j0:j0 + blk], A[:blk, :blk], sel)
        Wc[:, j0:] -= Z @ A[:blk, :]
        blockW = Wc[:, j0:j0 + blk]
        blockW[sel] = 0.0
        mask[:, j0:j0 + blk] = sel
        cnt = int(sel.sum())
        counts.append(cnt)
        pruned += cnt
        if j0 + blk < b:
            A = schur_downdate(A, blk)
    return {"W_hat": Wc, "mask": mask, "counts": counts, "lam": lam_abs,
            "k_total": ktot, "pruned": pruned}


def reconstruction_error(W, W_hat, G: np.ndarray):
    """E = ||(W - W_hat) X||_F^2 = sum_k D_k G D_k^T, and E / ||W X||_F^2.

    "Pruning LLMs with Thanos", section "The layer-reconstruction lens": the
    objective is the Frobenius norm of the output change and decomposes over rows.
    """
    W0 = _f64(W)
    D = W0 - _f64(W_hat)
    E = float(np.sum((D @ G) * D))
    base = float(np.sum((W0 @ G) * W0))
    return E, (E / base if base > 0 else 0.0)


def column_sq_norms(X_tok, chunk: int = 8192) -> np.ndarray:
    """G_qq = sum_t X_tq^2 in fp64, rounded to fp32 (the squared input-feature norms
    of the explainer's section "Wanda: Pruning by Weights and Activations").
    Summed over token chunks, so long streams need not exist in fp64 at once."""
    n, b = X_tok.shape
    acc = np.zeros(b, dtype=np.float64)
    for t0 in range(0, n, chunk):
        X = _f64(X_tok[t0:t0 + chunk])
        acc += np.sum(X * X, axis=0)
    return acc.astype(np.float32)


def baseline_keys(W, gdiag=None) -> np.ndarray:
    """Comparator keys in fp32: w^2 (rounded) times g_q (rounded), g = 1 without gdiag.

    "Pruning LLMs with Thanos", section "Why magnitude alone misses important
    weights": W_kq^2 G_qq orders like Wanda's |W_kq| ||X_q||_2; with g = 1 the key
    orders like |W_kq|. The keys are computed in fp32 (the precision in which the
    selection is decided), so both implementations see the same keys.
    """
    w = _f64(W).astype(np.float32)
    k = np.multiply(w, w, dtype=np.float32)
    if gdiag is not None:
        k = np.multiply(k, np.asarray(gdiag, dtype=np.float32)[None, :], dtype=np.float32)
    return k


def prune_baseline(W, method: str, gdiag=None, sparsity: float = 0.5, pattern=None) -> dict:
    """Magnitude or Wanda pruning: zero the lowest keys, no other weight changes.

    The explainer's section "Wanda: Pruning by Weights and Activations": each output
    row loses its lowest fraction of scores and the remaining weights are not
    updated; section "The Failure of Magnitude Pruning in Large Transformers":
    magnitude ranks by |W| (compared per output row here, like Wanda). Section
    "N:M Semi-Structured Sparsity (2:4 Pattern)": with a pattern, the m-n lowest of
    every aligned group of m. Unstructured: round-half-even(p*b) per row. Ties: the
    lower column is pruned first (stable sort).
    """
    W0 = _f64(W)
    c, b = W0.shape
    if method not in ("magnitude", "wanda"):
        raise ValueError(method)
    keys = baseline_keys(W, gdiag if method == "wanda" else None)
    if pattern is None:
        krow = int(np.round(np.float64(sparsity) * b))
        order = np.argsort(keys, axis=1, kind="stable")
        mask = np.zeros((c, b), dtype=bool)
        np.put_along_axis(mask, order[:, :krow], True, axis=1)
    else:
        n_keep, m = pattern
        if not (0 <= n_keep <= m) or b % m:
            raise ValueError("N:M needs 0<=n<=m and m | b")
        mask = select_nm(keys, n_keep, m)
    W_hat = W0.copy()
    W_hat[mask] = 0.0
    return {"W_hat": W_hat, "mask": mask}


def trailing_inverse_rows(H: np.ndarray) -> np.ndarray:
    """T[q, q:] = row q of inv(H restricted to columns q, q+1, ..., b-1); zero below.

    The explainer's section "SparseGPT: Second-Order Reconstruction at Scale": when
    column q is processed the inverse Hessian is that of the columns still active,
    q and everything right of it ("Pruning LLMs with Thanos", section "The scaling
    problem, and what SparseGPT changes": finished columns are frozen). Computed
    from an LU inverse of H by one single-column Schur downdate per column.
    """
    b = H.shape[0]
    A = np.linalg.inv(H)
    T = np.zeros((b, b), dtype=np.float64)
    for q in range(b):
        T[q, q:] = A[0]
        if q + 1 < b:
            A = schur_downdate(A, 1)
    return T


def sparsegpt_column(Wc: np.ndarray, q: int, pruned: np.ndarray, t_row: np.ndarray) -> None:
    """Process column q for every row at once (in place on Wc).

    The explainer's section "SparseGPT: Second-Order Reconstruction at Scale": a
    pruned w_kq (W_hat = 0) has error w_kq / [H^-1]_qq, and that error times row q of
    H^-1 (over the active columns, t_row = [H^-1]_{q, q:}) is subtracted from row k
    at columns q and after; a kept weight has no error and changes nothing. Column q
    is then exactly zero where pruned.
    """
    err = np.where(pruned, Wc[:, q], 0.0) / t_row[0]
    Wc[:, q:] -= np.outer(err, t_row)
    Wc[pruned, q] = 0.0


def prune_sparsegpt(W, G: np.ndarray, sparsity: float = 0.5, pattern=None, block: int = 128,
                    lam: float = 0.01, lam_relative: bool = True, trace: list | None = None) -> dict:
    """Column-sequential pruning on a schedule shared by all rows (the SparseGPT comparator).

    "Pruning LLMs with Thanos", section "The scaling problem, and what SparseGPT
    changes": columns are processed left to right, every row at once; a finished
    column is frozen; compensation goes only into columns still active; pruning
    decisions are refreshed block by block. The explainer's section "SparseGPT:
    Second-Order Reconstruction at Scale" gives the update for column j:
    the error (W_j - W_hat_j) / [H^-1]_jj times row j of H^-1 is subtracted from the
    columns after j, with H^-1 the inverse over the active columns.

    Readings (the pages leave these open):
    * score of w_kq: the OBS cost w_kq^2 / [inv(H_{q:})]_qq of deleting it when
      column q is processed, from the weights at the start of the block;
    * unstructured: every block loses exactly round-half-even(p * c * |J|) weights,
      the lowest (score, flat index) of the block (the equal per-block quota that
      "Contribution two: keep the budget global and the execution local" contrasts
      with the dynamic budget); N:M: the m-n lowest (score, column) of every group;
    * pruned entries are set to exactly 0.0.
    """
    W0 = _f64(W)
    G = np.asarray(G, dtype=np.float64)
    c, b = W0.shape
    if block < 1:
        raise ValueError("block must be >= 1")
    if pattern is not None:
        n_keep, m = pattern
        if not (0 <= n_keep <= m) or block % m or b % m:
            raise ValueError("N:M needs 0<=n<=m, m | block and m | b")
    lam_abs = damping(G, lam, lam_relative)
    H = hessian(G, lam_abs)
    try:
        np.linalg.cholesky(H)
    except np.linalg.LinAlgError as exc:
        raise NotSPDError("damped Hessian is not positive definite") from exc
    T = trailing_inverse_rows(H)
    d = np.diag(T).copy()
    Wc = W0.copy()
    mask = np.zeros((c, b), dtype=bool)
    counts = []
    for j0 in range(0, b, block):
        blk = min(block, b - j0)
        S = Wc[:, j0:j0 + blk] ** 2 / d[None, j0:j0 + blk]
        r = k_total(sparsity, c, blk) if pattern is None else None
        if pattern is None:
            sel = select_unstructured(S, r, blk)
        else:
            sel = select_nm(S, pattern[0], pattern[1])
        if trace is not None:
            trace.append({"j0": j0, "S": S.copy(), "r": r})
        for t in range(blk):
            sparsegpt_column(Wc, j0 + t, sel[:, t], T[j0 + t, j0 + t:])
        mask[:, j0:j0 + blk] = sel
        counts.append(int(sel.sum()))
    return {"W_hat": Wc, "mask": mask, "counts": counts, "lam": lam_abs,
            "pruned": int(sum(counts))}


def silu(z):
    """silu(z) = z * sigmoid(z), with sigmoid(z) = (1 + tanh(z/2)) / 2 (no overflow)."""
    z = np.asarray(z, dtype=np.float64)
    return z * (0.5 * (1.0 + np.tanh(0.5 * z)))


def gated_ffn_input(X_tok, W_gate, W_up) -> np.ndarray:
    """Input of down_proj: Y = silu(X W_gate^T) * (X W_up^T), fp64, token-major [n, f].

    "Pruning LLMs with Thanos", section "The compression target: linear layers": a
    block's feed-forward projections are joined by a nonlinearity. The layer names
    gate_proj / up_proj / down_proj are LLaMA's gated feed-forward, read here as
    down_proj(silu(gate_proj(x)) * up_proj(x)).
    """
    X = _f64(X_tok)
    return silu(X @ _f64(W_gate).T) * (X @ _f64(W_up).T)


def _bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (through fp32, each step to nearest even), as fp64."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    finite = np.isfinite(f)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = np.where(finite, r, u).astype(np.uint32).view(np.float32)
    return out.astype(np.float64)


def prune_mlp_sequential(X_mlp, W_gate, W_up, W_down, sparsity: float = 0.5, pattern=None,
                         block: int = 128, lam: float = 0.01) -> dict:
    """The feed-forward half of a block pruned in order, with propagated activations.

    gate_proj and up_proj share the input X_mlp and so one Hessian; they are pruned
    first. down_proj's calibration input is then produced by the pruned gate and up
    as the layers store them (in their own dtype: bf16 weights rounded to nearest
    even) through gated_ffn_input, kept like every other activation in bf16, and
    down_proj is pruned on its own Hessian ("Pruning LLMs with Thanos", section
    "The layer-reconstruction lens": each linear layer is reconstructed from its
    own inputs).
    """
    G_mlp = gram(X_mlp)
    gate = prune_layer(W_gate, G_mlp, sparsity=sparsity, pattern=pattern, block=block, lam=lam)
    up = prune_layer(W_up, G_mlp, sparsity=sparsity, pattern=pattern, block=block, lam=lam)

    def stored(W, W_hat):
        bf16 = hasattr(W, "dtype") and str(W.dtype) == "torch.bfloat16"
        return _bf16_round(W_hat) if bf16 else W_hat

    X_down = _bf16_round(gated_ffn_input(X_mlp, stored(W_gate, gate["W_hat"]),
                                         stored(W_up, up["W_hat"])))
    G_down = gram(X_down)
    down = prune_layer(W_down, G_down, sparsity=sparsity, pattern=pattern, block=block, lam=lam)
    return {"gate": gate, "up": up, "down": down, "X_down": X_down, "G_mlp": G_mlp,
            "G_down": G_down}


def row_energies(W, gdiag) -> np.ndarray:
    """s_k = sum_q W_kq^2 G_qq, summed in fp64 from G_qq given in fp32 and rounded to
    fp32 (the precision in which the alpha variant ranks rows; see outlier_rows)."""
    W0 = _f64(W)
    g = np.asarray(gdiag, dtype=np.float32).astype(np.float64)
    return ((W0 * W0) @ g).astype(np.float32)


def outlier_rows(W, gdiag, alpha: float) -> np.ndarray:
    """Rows kept dense by the alpha variant (True = dense).

    "Pruning LLMs with Thanos", section "What the experiments show": the alpha = 0.1
    variant keeps 10% of the rows as outliers (50% sparsity becomes 45%). Which rows
    is not stated; read here as the rows with the largest output energy
    s_k = sum_q W_kq^2 G_qq (the diagonal part of ||W_k X||^2, the error of deleting
    the whole row with every column independent), round-half-even(alpha * c) of
    them. s_k is summed in fp64 from G_qq given in fp32 and ranked by its fp32
    value, ties to the higher row index (rows ordered by (s_k, k); the last ones
    stay dense).
    """
    c = _f64(W).shape[0]
    s32 = row_energies(W, gdiag)
    r = int(np.round(np.float64(alpha) * c))
    order = np.lexsort((np.arange(c), s32))
    dense = np.zeros(c, dtype=bool)
    if r > 0:
        dense[order[c - r:]] = True
    return dense


def prune_layer_alpha(W, G: np.ndarray, alpha: float, gdiag=None, **kw) -> dict:
    """The layer step on the rows that are not kept dense (outlier_rows), which form
    a layer of their own: its budget, blocks and solves see only those rows (rows
    are independent given H, "The layer-reconstruction lens"). Dense rows are
    returned unchanged with an all-zero mask. gdiag defaults to diag(G) in fp32."""
    W0 = _f64(W)
    c, b = W0.shape
    if gdiag is None:
        gdiag = np.diag(np.asarray(G, dtype=np.float64)).astype(np.float32)
    dense = outlier_rows(W, gdiag, alpha)
    W_hat = W0.copy()
    mask = np.zeros((c, b), dtype=bool)
    rest = np.flatnonzero(~dense)
    out = {"dense": dense, "counts": [], "pruned": 0, "lam": damping(np.asarray(G), kw.get("lam", 0.01),
                                                                   kw.get("lam_relative", True))}
    if len(rest):
        sub = prune_layer(W0[rest], G, **kw)
        W_hat[rest] = sub["W_hat"]
        mask[rest] = sub["mask"]
        out.update({k: sub[k] for k in ("counts", "pruned", "lam", "k_total")})
    out.update({"W_hat": W_hat, "mask": mask})
    return out


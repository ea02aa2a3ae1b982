"""ctypes binding of libthanos (include/thanos.h): argument marshalling only.

Every step of the pruning path runs in the HIP library. Tensors provide device
memory and the current stream; nothing here computes on the CPU. If the library
has not been built, loading raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libthanos.so")

TH_OK, TH_ERR_INVALID_ARG, TH_ERR_NOT_SPD, TH_ERR_NONFINITE, TH_ERR_WORKSPACE, TH_ERR_HIP = range(6)
TH_F32, TH_BF16 = 0, 1
TH_UNSTRUCTURED, TH_NM = 0, 1
TH_SCORE_OBS, TH_SCORE_WANDA = 0, 1
TH_BASE_MAGNITUDE, TH_BASE_WANDA = 0, 1
STATUS_NAMES = {0: "TH_OK", 1: "TH_ERR_INVALID_ARG", 2: "TH_ERR_NOT_SPD", 3: "TH_ERR_NONFINITE",
                4: "TH_ERR_WORKSPACE", 5: "TH_ERR_HIP"}


class ThanosError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Pattern(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("n", ctypes.c_int32), ("m", ctypes.c_int32)]


class PruneParams(ctypes.Structure):
    _fields_ = [("sparsity", ctypes.c_double), ("pattern", Pattern), ("block", ctypes.c_int64),
                ("lam", ctypes.c_double), ("lambda_is_relative", ctypes.c_int32),
                ("score", ctypes.c_int32)]


class Stats(ctypes.Structure):
    _fields_ = [("lambda_used", ctypes.c_double), ("total_pruned", ctypes.c_int64),
                ("nblocks", ctypes.c_int64)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SIG = {
    "th_hessian_accumulate": [_P, _P, _I32, _I64, _I64, _I64, _P, ctypes.c_size_t, _P],
    "th_hessian_workspace_size": [_I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
    "th_hessian_finalize": [_P, _I64, ctypes.c_double, _I32, ctypes.POINTER(ctypes.c_double), _P],
    "th_prune_layer": [_P, _I32, _I64, _I64, _P, _I32, _I64, _P, ctypes.POINTER(PruneParams), _P,
                       _P, _P, ctypes.c_size_t, ctypes.POINTER(Stats), ctypes.POINTER(_I64), _P],
    "th_prune_layer_workspace_size": [_I64, _I64, _I64, _I32, ctypes.POINTER(PruneParams),
                                      ctypes.POINTER(ctypes.c_size_t)],
    "th_prune_layer_noalloc": [_P, _I32, _I64, _I64, _P, _I32, _I64, _P,
                               ctypes.POINTER(PruneParams), _P, _P, ctypes.POINTER(Stats),
                               ctypes.POINTER(_I64), _P],
    "th_factor": [_P, _I32, _I64, _P, _I64, ctypes.c_double, _I32, _P,
                  ctypes.POINTER(ctypes.c_double), _P, ctypes.c_size_t, _P],
    "th_factor_workspace_size": [_I64, _I64, _I32, ctypes.POINTER(ctypes.c_size_t)],
    "th_prune_layer_factored": [_P, _I32, _I64, _I64, _P, ctypes.POINTER(PruneParams), _P, _P, _P,
                                ctypes.c_size_t, ctypes.POINTER(Stats), ctypes.POINTER(_I64), _P],
    "th_prune_layer_factored_workspace_size": [_I64, _I64, ctypes.POINTER(PruneParams),
                                               ctypes.POINTER(ctypes.c_size_t)],
    "th_prune_layer_alpha": [_P, _I32, _I64, _I64, _P, _I32, _I64, _P, ctypes.POINTER(PruneParams),
                             ctypes.c_double, _P, _P, _P, _P, ctypes.c_size_t, ctypes.POINTER(Stats),
                             ctypes.POINTER(_I64), _P],
    "th_prune_layer_alpha_workspace_size": [_I64, _I64, _I64, _I32, ctypes.POINTER(PruneParams),
                                            ctypes.c_double, ctypes.POINTER(ctypes.c_size_t)],
    "th_gated_ffn_input": [_P, _P, _P, _I32, _I64, _I64, _I64, _P, _P],
    "th_prune_sparsegpt": [_P, _I32, _I64, _I64, _P, _I32, _I64, _P, ctypes.POINTER(PruneParams),
                           _P, _P, _P, ctypes.c_size_t, ctypes.POINTER(Stats),
                           ctypes.POINTER(_I64), _P],
    "th_prune_sparsegpt_workspace_size": [_I64, _I64, _I64, _I32, ctypes.POINTER(PruneParams),
                                          ctypes.POINTER(ctypes.c_size_t)],
    "th_reconstruction_error": [_P, _P, _I32, _I64, _I64, _P, _I32, _I64, _P, _P, ctypes.c_size_t,
                                ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                _P],
    "th_reconstruction_error_workspace_size": [_I64, _I64, _I32, ctypes.POINTER(ctypes.c_size_t)],
    "th_debug_select_nm": [_P, _I64, _I64, _I32, _I32, _P, _P],
    "th_debug_select_global": [_P, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P,
                               ctypes.c_size_t, _P],
    "th_debug_factor": [_P, _I64, _P, _P, ctypes.c_size_t, _P],
    "th_debug_syrk_rect": [_P, _P, _I64, _I64, _I64, _I32, _I32, _P, ctypes.c_size_t, _P],
    "th_debug_far_update": [_P, _I64, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _P,
                            ctypes.c_size_t, _P],
    "th_column_sq_norms_workspace_size": [_I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
    "th_column_sq_norms": [_P, _I32, _I64, _I64, _I64, _P, _P, ctypes.c_size_t, _P],
    "th_prune_baseline": [_P, _I32, _I64, _I64, _I32, _P, ctypes.POINTER(PruneParams), _P, _P],
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libthanos.so from the package directory (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m layer_wise_obs_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIG.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.th_last_error.argtypes = []
        L.th_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != TH_OK:
        raise ThanosError(status, lib().th_last_error().decode())


# ------------------------------------------------------------------ helpers

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return TH_BF16
    if t.dtype == torch.float32:
        return TH_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(device=None):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def make_params(sparsity=0.5, pattern=None, block=128, lam=0.01, relative=True,
                score="obs") -> PruneParams:
    p = PruneParams()
    p.sparsity = float(sparsity)
    if pattern is None:
        p.pattern = Pattern(TH_UNSTRUCTURED, 0, 0)
    else:
        p.pattern = Pattern(TH_NM, int(pattern[0]), int(pattern[1]))
    p.block = int(block)
    p.lam = float(lam)
    p.lambda_is_relative = 1 if relative else 0
    p.score = {"obs": TH_SCORE_OBS, "wanda": TH_SCORE_WANDA}[score]
    return p


def workspace(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- entry points

def hessian_workspace_size(t: int, b: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().th_hessian_workspace_size(t, b, ctypes.byref(out)))
    return out.value


def hessian_accumulate(H, X, ws=None):
    """H (b x b fp32, lower) += 2 X^T X for token-major X [t, b]."""
    _require_cuda(H, X)
    t, b = X.shape
    _check(lib().th_hessian_accumulate(_ptr(H), _ptr(X), _dtype_code(X), t, b, X.stride(0),
                                       _ptr(ws), 0 if ws is None else ws.numel(),
                                       _stream(X.device)))


def hessian_finalize(H, lam=0.01, relative=True) -> float:
    _require_cuda(H)
    out = ctypes.c_double(0.0)
    _check(lib().th_hessian_finalize(_ptr(H), H.shape[0], float(lam), 1 if relative else 0,
                                     ctypes.byref(out), _stream(H.device)))
    return out.value


def prune_layer_workspace_size(c, b, n, have_x, params: PruneParams) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().th_prune_layer_workspace_size(c, b, n, 1 if have_x else 0, ctypes.byref(params),
                                               ctypes.byref(out)))
    return out.value


def _layer_call(entry, size_entry, W, X, H, params, W_out, mask_out, ws) -> dict:
    _require_cuda(W, X, H, W_out, mask_out)
    if params is None:
        params = make_params()
    c, b = W.shape
    n = X.shape[0] if X is not None else 0
    if ws is None:
        out = ctypes.c_size_t(0)
        _check(size_entry(c, b, n, 1 if X is not None else 0, ctypes.byref(params),
                          ctypes.byref(out)))
        ws = workspace(out.value, W.device)
    stats = Stats()
    nblk = -(-b // params.block)
    counts = (_I64 * nblk)()
    _check(entry(_ptr(W), _dtype_code(W), c, b, _ptr(X), _dtype_code(X) if X is not None else 0,
                 n, _ptr(H), ctypes.byref(params), _ptr(W_out), _ptr(mask_out), _ptr(ws),
                 ws.numel(), ctypes.byref(stats), counts, _stream(W.device)))
    return {"lambda": stats.lambda_used, "pruned": stats.total_pruned, "nblocks": stats.nblocks,
            "counts": list(counts)}


def prune_layer(W, X=None, H=None, params: PruneParams | None = None, W_out=None, mask_out=None,
                ws=None) -> dict:
    """Prune W (c x b, bf16/fp32) in place; returns stats and per-block counts."""
    return _layer_call(lib().th_prune_layer, lib().th_prune_layer_workspace_size, W, X, H,
                       params, W_out, mask_out, ws)


NOALLOC_SCRATCH_BYTES = 64 << 20  # TH_NOALLOC_SCRATCH_BYTES in include/thanos.h


def prune_layer_noalloc(W, X=None, H=None, params: PruneParams | None = None, W_out=None,
                        mask_out=None) -> dict:
    """th_prune_layer_noalloc: the layer step in the library's fixed scratch array
    (no workspace, nothing allocated); same results as prune_layer."""
    _require_cuda(W, X, H, W_out, mask_out)
    if params is None:
        params = make_params()
    c, b = W.shape
    n = X.shape[0] if X is not None else 0
    stats = Stats()
    counts = (_I64 * (-(-b // params.block)))()
    _check(lib().th_prune_layer_noalloc(
        _ptr(W), _dtype_code(W), c, b, _ptr(X), _dtype_code(X) if X is not None else 0, n,
        _ptr(H), ctypes.byref(params), _ptr(W_out), _ptr(mask_out), ctypes.byref(stats), counts,
        _stream(W.device)))
    return {"lambda": stats.lambda_used, "pruned": stats.total_pruned, "nblocks": stats.nblocks,
            "counts": list(counts)}


def factor(X=None, H=None, lam=0.01, relative=True, U=None, ws=None):
    """U (b x b fp32, upper) with H^-1 = U^T U from X [n, b] or a damped H; returns (U, lambda)."""
    torch = _torch()
    _require_cuda(X, H, U)
    b = X.shape[1] if X is not None else H.shape[0]
    dev = (X if X is not None else H).device
    n = X.shape[0] if X is not None else 0
    if U is None:
        U = torch.empty((b, b), dtype=torch.float32, device=dev)
    if ws is None:
        out = ctypes.c_size_t(0)
        _check(lib().th_factor_workspace_size(b, n, 1 if X is not None else 0, ctypes.byref(out)))
        ws = workspace(out.value, dev)
    lam_out = ctypes.c_double(0.0)
    _check(lib().th_factor(_ptr(X), _dtype_code(X) if X is not None else 0, n, _ptr(H), b,
                           float(lam), 1 if relative else 0, _ptr(U), ctypes.byref(lam_out),
                           _ptr(ws), ws.numel(), _stream(dev)))
    return U, lam_out.value


def prune_layer_factored(W, U, params: PruneParams | None = None, W_out=None, mask_out=None,
                         ws=None) -> dict:
    """prune_layer from a factor U that layers sharing one input reuse."""
    _require_cuda(W, U, W_out, mask_out)
    if params is None:
        params = make_params()
    c, b = W.shape
    if ws is None:
        out = ctypes.c_size_t(0)
        _check(lib().th_prune_layer_factored_workspace_size(c, b, ctypes.byref(params),
                                                            ctypes.byref(out)))
        ws = workspace(out.value, W.device)
    stats = Stats()
    counts = (_I64 * (-(-b // params.block)))()
    _check(lib().th_prune_layer_factored(_ptr(W), _dtype_code(W), c, b, _ptr(U),
                                         ctypes.byref(params), _ptr(W_out), _ptr(mask_out),
                                         _ptr(ws), ws.numel(), ctypes.byref(stats), counts,
                                         _stream(W.device)))
    return {"lambda": stats.lambda_used, "pruned": stats.total_pruned, "nblocks": stats.nblocks,
            "counts": list(counts)}


def prune_layer_alpha(W, alpha: float, X=None, H=None, params: PruneParams | None = None,
                      W_out=None, mask_out=None, dense_out=None, ws=None) -> dict:
    """prune_layer with round(alpha c) rows of largest output energy kept dense."""
    _require_cuda(W, X, H, W_out, mask_out, dense_out)
    if params is None:
        params = make_params()
    c, b = W.shape
    n = X.shape[0] if X is not None else 0
    if ws is None:
        out = ctypes.c_size_t(0)
        _check(lib().th_prune_layer_alpha_workspace_size(c, b, n, 1 if X is not None else 0,
                                                         ctypes.byref(params), float(alpha),
                                                         ctypes.byref(out)))
        ws = workspace(out.value, W.device)
    stats = Stats()
    counts = (_I64 * (-(-b // params.block)))()
    _check(lib().th_prune_layer_alpha(_ptr(W), _dtype_code(W), c, b, _ptr(X),
                                      _dtype_code(X) if X is not None else 0, n, _ptr(H),
                                      ctypes.byref(params), float(alpha), _ptr(W_out),
                                      _ptr(mask_out), _ptr(dense_out), _ptr(ws), ws.numel(),
                                      ctypes.byref(stats), counts, _stream(W.device)))
    return {"lambda": stats.lambda_used, "pruned": stats.total_pruned, "nblocks": stats.nblocks,
            "counts": list(counts)}


def gated_ffn_input(X, W_gate, W_up, Y=None):
    """Y = silu(X W_gate^T) * (X W_up^T) in bf16 for X [n, d], W [f, d] (bf16)."""
    torch = _torch()
    _require_cuda(X, W_gate, W_up, Y)
    n, d = X.shape
    f = W_gate.shape[0]
    if Y is None:
        Y = torch.empty((n, f), dtype=torch.bfloat16, device=X.device)
    _check(lib().th_gated_ffn_input(_ptr(X), _ptr(W_gate), _ptr(W_up), _dtype_code(X), n, d, f,
                                    _ptr(Y), _stream(X.device)))
    return Y


def prune_sparsegpt_workspace_size(c, b, n, have_x, params: PruneParams) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().th_prune_sparsegpt_workspace_size(c, b, n, 1 if have_x else 0,
                                                   ctypes.byref(params), ctypes.byref(out)))
    return out.value


def prune_sparsegpt(W, X=None, H=None, params: PruneParams | None = None, W_out=None,
                    mask_out=None, ws=None) -> dict:
    """The column-sequential comparator on W (c x b) in place; same arguments as prune_layer."""
    return _layer_call(lib().th_prune_sparsegpt, lib().th_prune_sparsegpt_workspace_size, W, X,
                       H, params, W_out, mask_out, ws)


def reconstruction_error(W, W_hat, X=None, G=None, ws=None):
    _require_cuda(W, W_hat, X, G)
    c, b = W.shape
    if ws is None:
        out = ctypes.c_size_t(0)
        _check(lib().th_reconstruction_error_workspace_size(c, b, 1 if X is not None else 0,
                                                            ctypes.byref(out)))
        ws = workspace(out.value, W.device)
    e = ctypes.c_double(0.0)
    r = ctypes.c_double(0.0)
    _check(lib().th_reconstruction_error(_ptr(W), _ptr(W_hat), _dtype_code(W), c, b, _ptr(X),
                                         _dtype_code(X) if X is not None else 0,
                                         X.shape[0] if X is not None else 0, _ptr(G), _ptr(ws),
                                         ws.numel(), ctypes.byref(e), ctypes.byref(r),
                                         _stream(W.device)))
    return e.value, r.value


def debug_select_nm(scores, n: int, m: int):
    torch = _torch()
    _require_cuda(scores)
    c, blk = scores.shape
    mask = torch.empty((c, blk), dtype=torch.uint8, device=scores.device)
    _check(lib().th_debug_select_nm(_ptr(scores), c, blk, n, m, _ptr(mask), _stream(scores.device)))
    return mask


def debug_select_global(scores, b_full: int, j0: int, blk: int, r: int):
    torch = _torch()
    _require_cuda(scores)
    c, f = scores.shape
    mask = torch.empty((c, blk), dtype=torch.uint8, device=scores.device)
    s_k = torch.empty((c,), dtype=torch.int32, device=scores.device)
    ws = workspace(1 << 16, scores.device)
    _check(lib().th_debug_select_global(_ptr(scores), c, f, b_full, j0, blk, r, _ptr(mask),
                                        _ptr(s_k), _ptr(ws), ws.numel(), _stream(scores.device)))
    return mask, s_k


def debug_syrk_rect(H, X, P, m=0):
    """H (b x b fp32, lower) += 2 X^T X through the rectangles: whole tiles in rounds
    of P workgroups, the rest cut into m pieces each (m = 0: chosen)."""
    _require_cuda(H, X)
    t, b = X.shape
    tiles = -(-b // 384) * -(-b // 256)  # bounds the cut tiles
    ws = workspace(tiles * max(m, 16) * 98304 * 4 + 4 * tiles, H.device)
    _check(lib().th_debug_syrk_rect(_ptr(H), _ptr(X), t, b, X.stride(0), P, m, _ptr(ws),
                                    ws.numel(), _stream(X.device)))


def debug_far_update(W, Z, R, r0, K, col0, col_end):
    """W[:, col0:col_end] -= Z[:, :K] R[r0:r0+K, col0:col_end] (split-bf16 planes, 256 tiles)."""
    _require_cuda(W, Z, R)
    c, b = W.shape
    kp = -(-K // 64) * 64
    ybytes = 3 * kp * (-(-c // 256) + -(-(col_end - col0) // 256)) * 256 * 2
    nbytes = -(-ybytes // 256) * 256 + 256 * 256 * 256 * 4  # planes, then 256 piece slots
    ws = workspace(nbytes, W.device)
    _check(lib().th_debug_far_update(_ptr(W), c, b, _ptr(Z), Z.stride(0), _ptr(R), r0, K, col0,
                                     col_end, _ptr(ws), ws.numel(), _stream(W.device)))
    return ws


def debug_factor(H):
    torch = _torch()
    _require_cuda(H)
    b = H.shape[0]
    U = torch.empty_like(H)
    # b*b fp32, two panel buffers, two split panels (3 planes of 256 x ceil(b/256)*256 bf16)
    nbytes = (4 * b * b + 2 * 4 * (-(-b // 128)) * 128 * 256
              + 2 * 2 * 3 * 256 * (-(-b // 256)) * 256 + (1 << 16))
    ws = workspace(nbytes, H.device)
    _check(lib().th_debug_factor(_ptr(H), b, _ptr(U), _ptr(ws), ws.numel(), _stream(H.device)))
    return U


def column_sq_norms(X):
    """G_qq = sum_t X_tq^2 (fp32, b values) for token-major X [n, b]."""
    torch = _torch()
    _require_cuda(X)
    n, b = X.shape
    out = ctypes.c_size_t(0)
    _check(lib().th_column_sq_norms_workspace_size(n, b, ctypes.byref(out)))
    ws = workspace(out.value, X.device)
    g = torch.empty((b,), dtype=torch.float32, device=X.device)
    _check(lib().th_column_sq_norms(_ptr(X), _dtype_code(X), n, b, X.stride(0), _ptr(g), _ptr(ws),
                                    ws.numel(), _stream(X.device)))
    return g


def prune_baseline(W, method: str, gdiag=None, params: PruneParams | None = None, mask_out=None):
    """Magnitude or Wanda pruning of W (c x b, bf16/fp32) in place, no compensation."""
    _require_cuda(W, gdiag, mask_out)
    if params is None:
        params = make_params()
    c, b = W.shape
    code = {"magnitude": TH_BASE_MAGNITUDE, "wanda": TH_BASE_WANDA}[method]
    _check(lib().th_prune_baseline(_ptr(W), _dtype_code(W), c, b, code, _ptr(gdiag),
                                   ctypes.byref(params), _ptr(mask_out), _stream(W.device)))

"""The C-ABI library builds, loads and exports every entry point include/thanos.h
declares; argument checks answer before anything touches the GPU."""
import ctypes
import os
import re

import pytest

from layer_wise_obs_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "thanos.h")).read()
    return sorted(set(re.findall(r"\b(th_[a-z_]+)\s*\(", src)))


def test_header_declares_the_path():
    names = _declared()
    for must in ("th_hessian_accumulate", "th_hessian_finalize", "th_prune_layer",
                 "th_prune_layer_workspace_size", "th_reconstruction_error", "th_debug_select_nm",
                 "th_debug_select_global", "th_debug_factor", "th_last_error",
                 "th_column_sq_norms", "th_column_sq_norms_workspace_size", "th_prune_baseline",
                 "th_prune_sparsegpt", "th_prune_sparsegpt_workspace_size", "th_factor",
                 "th_factor_workspace_size", "th_prune_layer_factored",
                 "th_prune_layer_factored_workspace_size", "th_gated_ffn_input",
                 "th_prune_layer_alpha", "th_prune_layer_alpha_workspace_size",
                 "th_prune_layer_noalloc", "th_debug_syrk_rect", "th_debug_far_update"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_params_struct_matches_header_layout():
    # double, 3 x int32, (pad), int64, double, int32, int32
    assert ctypes.sizeof(_lib.PruneParams) == 48
    assert _lib.PruneParams.block.offset == 24
    assert ctypes.sizeof(_lib.Stats) == 24


def _status(fn, *args):
    return fn(*args)


def test_invalid_arguments_are_rejected_before_any_launch():
    L = _lib.lib()
    out = ctypes.c_size_t(0)
    ok = _lib.make_params(pattern=(2, 4), block=128)
    assert L.th_prune_layer_workspace_size(4096, 11008, 262144, 1, ctypes.byref(ok), ctypes.byref(out)) == 0
    assert out.value > 2 * 11008 * 11008 * 4
    bad = [
        _lib.make_params(block=0),
        _lib.make_params(block=129),
        _lib.make_params(sparsity=1.5),
        _lib.make_params(pattern=(2, 4), block=126),  # m does not divide B
        _lib.make_params(pattern=(5, 4)),
        _lib.make_params(lam=-1.0),
    ]
    for p in bad:
        assert L.th_prune_layer_workspace_size(64, 128, 10, 1, ctypes.byref(p), ctypes.byref(out)) == 1
    assert "block" in L.th_last_error().decode() or "lambda" in L.th_last_error().decode()
    # N:M with b not a multiple of m
    p = _lib.make_params(pattern=(2, 4), block=8)
    assert L.th_prune_layer_workspace_size(8, 10, 10, 1, ctypes.byref(p), ctypes.byref(out)) == 1
    # prune_layer: both X and H given / neither given
    p = _lib.make_params()
    dummy = ctypes.c_void_p(16)
    args = [dummy, 0, 8, 8, dummy, 0, 8, dummy, ctypes.byref(p), None, None, dummy, 1 << 20,
            None, None, None]
    assert L.th_prune_layer(*args) == 1
    args[4] = None
    args[7] = None
    assert L.th_prune_layer(*args) == 1
    # hessian: ldx < b, misaligned bf16
    assert L.th_hessian_accumulate(dummy, dummy, 1, 10, 16, 8, None, 0, None) == 1
    assert L.th_hessian_accumulate(dummy, ctypes.c_void_p(18), 1, 10, 16, 16, None, 0, None) == 1
    assert L.th_debug_select_nm(dummy, 4, 6, 2, 4, dummy, None) == 1


def test_workspace_size_queries():
    L = _lib.lib()
    out = ctypes.c_size_t(0)
    # 659 rectangles of 384 x 256 (without a device the split assumes 256 compute
    # units): 512 whole in two rounds, the other 147 cut into 5 pieces of 8192 / 5
    # stages, one slot of 384 x 256 floats per piece and one int per cut tile
    assert L.th_hessian_workspace_size(262144, 11008, ctypes.byref(out)) == 0
    assert out.value == (147 * 5 * 384 * 256 + 147) * 4
    assert L.th_hessian_workspace_size(262144, 4096, ctypes.byref(out)) == 0
    assert out.value > 0  # 101 rectangles, all cut into pieces
    assert L.th_hessian_workspace_size(1000, 520, ctypes.byref(out)) == 0
    assert out.value > 0  # 10 square tiles: token split with a fixed-order reduction
    assert L.th_reconstruction_error_workspace_size(4096, 11008, 0, ctypes.byref(out)) == 0
    assert out.value >= 2 * 4096 * 11008 * 4


def test_baseline_arguments_are_rejected_before_any_launch():
    L = _lib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its checks first
    ok = _lib.make_params(sparsity=0.5)
    cases = [
        (None, _lib.TH_BF16, 4, 16, _lib.TH_BASE_MAGNITUDE, None, ok),          # W is NULL
        (fake, 7, 4, 16, _lib.TH_BASE_MAGNITUDE, None, ok),                      # bad dtype
        (fake, _lib.TH_BF16, 0, 16, _lib.TH_BASE_MAGNITUDE, None, ok),           # c = 0
        (fake, _lib.TH_BF16, 4, 16, 5, None, ok),                                # bad method
        (fake, _lib.TH_BF16, 4, 16, _lib.TH_BASE_WANDA, None, ok),               # Wanda without G
        (fake, _lib.TH_BF16, 4, 16, _lib.TH_BASE_MAGNITUDE, None, _lib.make_params(sparsity=1.5)),
        (fake, _lib.TH_BF16, 4, 18, _lib.TH_BASE_MAGNITUDE, None,
         _lib.make_params(pattern=(2, 4), block=16)),                            # m does not divide b
        (fake, _lib.TH_BF16, 4, 16, _lib.TH_BASE_MAGNITUDE, None,
         _lib.make_params(pattern=(5, 4), block=16)),                            # n > m
    ]
    for W, dt, c, b, method, g, p in cases:
        st = L.th_prune_baseline(W, dt, c, b, method, g, ctypes.byref(p), None, None)
        assert st == _lib.TH_ERR_INVALID_ARG, (dt, c, b, method)
    out = ctypes.c_size_t(0)
    assert L.th_column_sq_norms_workspace_size(262144, 11008, ctypes.byref(out)) == 0
    assert out.value == 128 * 11008 * 8
    assert L.th_column_sq_norms(None, _lib.TH_BF16, 10, 8, 8, fake, fake, 1 << 20, None) == 1
    assert L.th_column_sq_norms(fake, _lib.TH_BF16, 10, 8, 8, fake, fake, 8, None) == \
        _lib.TH_ERR_WORKSPACE


def test_sparsegpt_arguments_are_rejected_before_any_launch():
    L = _lib.lib()
    out = ctypes.c_size_t(0)
    ok = _lib.make_params(pattern=(2, 4), block=128)
    assert L.th_prune_sparsegpt_workspace_size(4096, 11008, 262144, 1, ctypes.byref(ok),
                                               ctypes.byref(out)) == 0
    full = ctypes.c_size_t(0)
    L.th_prune_layer_workspace_size(4096, 11008, 262144, 1, ctypes.byref(ok), ctypes.byref(full))
    assert 2 * 11008 * 11008 * 4 < out.value <= full.value  # no slices beside U
    bad = _lib.make_params(pattern=(2, 4), block=126)
    assert L.th_prune_sparsegpt_workspace_size(64, 128, 10, 1, ctypes.byref(bad),
                                               ctypes.byref(out)) == 1
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its checks first
    wanda = _lib.make_params(score="wanda")
    args = [fake, _lib.TH_BF16, 8, 8, fake, _lib.TH_BF16, 8, None, ctypes.byref(wanda), None, None,
            ctypes.c_void_p(0x1000), 1 << 20, None, None, None]
    assert L.th_prune_sparsegpt(*args) == 1  # the comparator takes the OBS score only
    assert "OBS" in L.th_last_error().decode()
    p = _lib.make_params()
    args[8] = ctypes.byref(p)
    args[7] = fake  # both X and H
    assert L.th_prune_sparsegpt(*args) == 1
    args[7] = None
    args[11] = ctypes.c_void_p(0x1010)  # workspace not 256-byte aligned
    assert L.th_prune_sparsegpt(*args) == 1


def test_factor_and_ffn_arguments_are_rejected_before_any_launch():
    L = _lib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its checks first
    ws = ctypes.c_void_p(0x1000)
    lam = ctypes.c_double(0.0)
    # th_factor: both / neither of X and H, negative lambda, misaligned workspace
    assert L.th_factor(fake, _lib.TH_BF16, 8, fake, 8, 0.01, 1, fake, ctypes.byref(lam), ws,
                       1 << 30, None) == 1
    assert L.th_factor(None, _lib.TH_BF16, 8, None, 8, 0.01, 1, fake, ctypes.byref(lam), ws,
                       1 << 30, None) == 1
    assert L.th_factor(None, _lib.TH_BF16, 0, fake, 8, -1.0, 1, fake, ctypes.byref(lam), ws,
                       1 << 30, None) == 1
    assert L.th_factor(None, _lib.TH_BF16, 0, fake, 8, 0.01, 1, fake, ctypes.byref(lam),
                       ctypes.c_void_p(0x1010), 1 << 30, None) == 1
    out = ctypes.c_size_t(0)
    assert L.th_factor(None, _lib.TH_BF16, 0, fake, 8, 0.01, 1, fake, ctypes.byref(lam), ws, 0,
                       None) == 4  # TH_ERR_WORKSPACE
    assert L.th_factor_workspace_size(11008, 262144, 1, ctypes.byref(out)) == 0
    assert out.value >= 11008 * 11008 * 4
    # factored prune: Wanda score rejected; workspace query smaller than the full layer's
    p = _lib.make_params(pattern=(2, 4))
    full = ctypes.c_size_t(0)
    assert L.th_prune_layer_factored_workspace_size(4096, 11008, ctypes.byref(p), ctypes.byref(out)) == 0
    L.th_prune_layer_workspace_size(4096, 11008, 0, 0, ctypes.byref(p), ctypes.byref(full))
    assert out.value < full.value
    wanda = _lib.make_params(score="wanda")
    assert L.th_prune_layer_factored(fake, _lib.TH_BF16, 8, 8, fake, ctypes.byref(wanda), None,
                                     None, ws, 1 << 30, None, None, None) == 1
    assert "OBS" in L.th_last_error().decode()
    # gated ffn: fp32, d % 8, misaligned
    assert L.th_gated_ffn_input(fake, fake, fake, _lib.TH_F32, 4, 8, 4, fake, None) == 1
    assert L.th_gated_ffn_input(fake, fake, fake, _lib.TH_BF16, 4, 12, 4, fake, None) == 1
    assert L.th_gated_ffn_input(ctypes.c_void_p(0x1002), fake, fake, _lib.TH_BF16, 4, 8, 4, fake,
                                None) == 1


def test_alpha_arguments_are_rejected_before_any_launch():
    L = _lib.lib()
    out = ctypes.c_size_t(0)
    p = _lib.make_params(pattern=(2, 4))
    assert L.th_prune_layer_alpha_workspace_size(4096, 11008, 262144, 1, ctypes.byref(p), 0.1,
                                                 ctypes.byref(out)) == 0
    for bad in (-0.1, 1.5, float("nan")):
        assert L.th_prune_layer_alpha_workspace_size(64, 128, 10, 1, ctypes.byref(p), bad,
                                                     ctypes.byref(out)) == 1
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its checks first
    args = [fake, _lib.TH_BF16, 8, 8, fake, _lib.TH_BF16, 8, None, ctypes.byref(p), 2.0, None, None,
            None, fake, 1 << 30, None, None, None]
    assert L.th_prune_layer_alpha(*args) == 1  # alpha > 1
    args[9] = 0.1
    args[7] = fake  # both X and H
    assert L.th_prune_layer_alpha(*args) == 1


def test_noalloc_rejects_layers_beyond_its_scratch_before_any_launch():
    """The allocation-free entry point checks the layer's scratch need against its
    fixed array on the host and answers TH_ERR_WORKSPACE without touching a GPU."""
    L = _lib.lib()
    p = _lib.make_params(pattern=(2, 4))
    dummy = ctypes.c_void_p(256)
    st = L.th_prune_layer_noalloc(dummy, 1, 4096, 4096, None, 1, 0, dummy, ctypes.byref(p), None,
                                  None, None, None, None)
    assert st == 4
    msg = L.th_last_error().decode()
    assert "scratch" in msg and str(_lib.NOALLOC_SCRATCH_BYTES) in msg
    # argument errors come first, as for th_prune_layer
    assert L.th_prune_layer_noalloc(None, 1, 64, 64, None, 1, 0, dummy, ctypes.byref(p), None,
                                    None, None, None, None) == 1


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_present(), reason="calls the layer entry points on fake device pointers")
@pytest.mark.parametrize("pattern,have_x,b", [(None, True, 304), ((2, 4), True, 304),
                                               (None, False, 1000), ((2, 4), False, 11008),
                                               (None, True, 11008)])
def test_workspace_queries_match_the_calls(pattern, have_x, b):
    """Each size query gives exactly what its call carves: with that many bytes the
    call gets past its workspace check (and stops at the first device call, as no
    device is present); one byte fewer is TH_ERR_WORKSPACE before anything runs."""
    L = _lib.lib()
    p = _lib.make_params(sparsity=0.6 if pattern is None else 0.5, pattern=pattern, block=128)
    c, n, alpha = 150, 262144 if b == 11008 else 1000, 0.05
    fake, ws = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x10000000)
    x = fake if have_x else None
    h = None if have_x else fake
    st = _lib.Stats()
    counts = (_lib._I64 * (-(-b // 128)))()
    out = ctypes.c_size_t(0)
    calls = [
        (L.th_prune_layer_workspace_size, (c, b, n if have_x else 0, int(have_x), ctypes.byref(p)),
         lambda nb: L.th_prune_layer(fake, _lib.TH_BF16, c, b, x, _lib.TH_BF16, n if have_x else 0,
                                     h, ctypes.byref(p), None, None, ws, nb, ctypes.byref(st),
                                     counts, None)),
        (L.th_prune_layer_alpha_workspace_size,
         (c, b, n if have_x else 0, int(have_x), ctypes.byref(p), ctypes.c_double(alpha)),
         lambda nb: L.th_prune_layer_alpha(fake, _lib.TH_BF16, c, b, x, _lib.TH_BF16,
                                           n if have_x else 0, h, ctypes.byref(p),
                                           ctypes.c_double(alpha), None, None, None, ws, nb,
                                           ctypes.byref(st), counts, None)),
        (L.th_prune_sparsegpt_workspace_size, (c, b, n if have_x else 0, int(have_x), ctypes.byref(p)),
         lambda nb: L.th_prune_sparsegpt(fake, _lib.TH_BF16, c, b, x, _lib.TH_BF16,
                                         n if have_x else 0, h, ctypes.byref(p), None, None, ws, nb,
                                         ctypes.byref(st), counts, None)),
    ]
    for size_fn, args, call in calls:
        assert size_fn(*args, ctypes.byref(out)) == 0
        assert call(out.value - 1) == _lib.TH_ERR_WORKSPACE
        assert call(out.value) not in (0, _lib.TH_ERR_WORKSPACE, _lib.TH_ERR_INVALID_ARG)

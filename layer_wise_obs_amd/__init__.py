"""MI355X-native block-wise (Thanos-style) pruning of one linear layer.

The pruning path lives in the HIP library libthanos.so (C ABI in include/thanos.h);
this package holds its ctypes binding, the build script and the seeded input
generator.
"""
from ._lib import (  # noqa: F401
    ThanosError, debug_factor, debug_select_global, debug_select_nm, hessian_accumulate,
    hessian_finalize, hessian_workspace_size, lib, make_params, prune_layer,
    prune_layer_workspace_size, reconstruction_error, workspace,
)

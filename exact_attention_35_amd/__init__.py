"""MI355X-native exact attention forward (IO-aware, online softmax, gfx950 HIP kernels).

`forward(q, k, v, bias=None, causal=False)` computes O = softmax(QK^T/sqrt(d) + C) V
and the per-row log-sum-exp through the C-ABI library libfa.so. The library is loaded
on first use; a missing library raises (there is no CPU fallback).
"""

from .capi import (FA_BF16, FA_F32, FA_MASK_CAUSAL, FA_MASK_NONE, FA_OK, FaError,  # noqa: F401
                   fa_fwd, fa_fwd_ex, fa_fwd_workspace_size, fa_shutdown, fa_status_string,
                   fa_version)

forward = fa_fwd

__all__ = [
    "forward", "fa_fwd", "fa_fwd_ex", "fa_fwd_workspace_size", "fa_status_string",
    "fa_version", "fa_shutdown",
    "FaError", "FA_OK", "FA_F32", "FA_BF16", "FA_MASK_NONE", "FA_MASK_CAUSAL",
]

"""Exact tiled attention (FlashAttention forward and backward) for MI355X.

The computation lives in ``libfa.so`` (hand-written gfx950 HIP kernels behind
the C ABI in ``include/fa.h``); :mod:`io_aware_tiled_fwd_amd.binding` is a thin
ctypes layer over it.  Importing this package does not load the library;
the first call does, and fails loudly if it has not been built
(``python -m io_aware_tiled_fwd_amd.build``).
"""
_BINDING_NAMES = ("fa_fwd", "fa_fwd_f32", "fa_fwd_fp8", "fa_bwd", "fa_fwd_gqa", "fa_bwd_gqa", "fa_bwd_gqa_bf16grad",
                  "fa_fwd_dropout", "fa_bwd_dropout", "fa_decode_plan", "fa_decode", "fa_bwd_preprocess",
                  "fa_bwd_dkdv", "fa_bwd_dv", "fa_bwd_dk", "fa_bwd_dq", "fa_status_string", "attention_fwd",
                  "attention_bwd", "attention_decode", "attention_fwd_fp8", "attention_fwd_dropout", "attention_bwd_dropout",
                  "FaError", "load_library")

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)

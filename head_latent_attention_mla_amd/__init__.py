"""MI355X (gfx950) multi-head latent attention: absorbed decode over a
compressed KV cache and the literal wkv_b key/value reconstruction.

The compute lives in ``libmla.so`` (hand-written HIP kernels behind the C ABI
of ``include/mla.h``); ``binding`` marshals torch device tensors into those
calls. Importing the package loads nothing: the library is opened on first
use of a binding function, and a missing library is an error, never a
fallback.
"""
from __future__ import annotations

__all__ = [
    "mla_dequant_fp8_block", "mla_absorb_q", "mla_decode_latent_attn", "mla_out_up",
    "mla_kv_reconstruct", "mla_decode_workspace_bytes", "mla_decode_num_splits",
    "MLAError",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)

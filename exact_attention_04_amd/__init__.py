"""Exact attention for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libattn.so``, built from ``csrc/``); :mod:`exact_attention_04_amd.binding`
is a thin ctypes layer over it that takes torch tensors for device memory and
streams.  The binding is imported on first use so that the seeded input
generator (:mod:`exact_attention_04_amd.synth`) can be used without the
library; every compute entry point raises if the library is missing.
"""

__all__ = ["attn_fwd", "attn_verify", "attn_verify_workspace_bytes", "fwd", "verify"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)

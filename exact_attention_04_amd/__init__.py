"""Exact attention for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libattn.so``, built from ``csrc/``); :mod:`exact_attention_04_amd.binding`
is a thin ctypes layer over it that takes torch tensors for device memory and
streams.  The binding is imported on first use so that the seeded input
generator (:mod:`exact_attention_04_amd.synth`) can be used without the
library; every compute entry point raises if the library is missing.
"""

# the C entry points (raw, device pointers as ints) and the tensor-level calls
__all__ = [
    "attn_fwd", "attn_verify", "attn_verify_noalloc", "attn_verify_tree", "attn_verify_paged",
    "attn_verify_workspace_bytes", "attn_spec_accept", "attn_spec_accept_workspace_bytes", "attn_bwd",
    "attn_bwd_workspace_bytes", "attn_strerror",
    "fwd", "bwd", "verify", "verify_tree", "verify_paged", "spec_accept",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)

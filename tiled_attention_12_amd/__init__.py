"""tiled_attention_12_amd -- tiled fused attention forward for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libtattn.so`` (hand-written HIP
kernels); this package only loads it and marshals torch tensors into it.
The binding is loaded on first attribute access, so ``inputs`` and
``workloads`` stay importable before the library is built; any use of an
entry point without the built library raises ImportError.
"""

_EXPORTS = ("attn_fwd", "attn_fwd_ex", "attn_fwd_f32", "mla_decode", "mla_decode_noalloc", "ssd_scan", "status_str",
            "TattnError", "lib")


def __getattr__(name):
    if name in _EXPORTS:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)


__all__ = list(_EXPORTS)

"""Causal FP8/BF16 prefill attention for AMD MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libattnfwd.so``, declared in ``include/attn_fwd.h``); this package is the thin
ctypes binding above it plus the seeded synthetic workloads.  The binding is
loaded lazily so that ``workloads`` can be used without the built library; any
call into the attention entry points fails loudly if the library is missing.
"""
from . import workloads  # noqa: F401

_BINDING_NAMES = {"attn_fwd_fp8", "attn_fwd_bf16", "rotate_quant_bf16", "attn_last_error", "library_path",
                  "load_library", "P_EXACT", "P_LEAN", "AttnError", "exported_symbols"}


def __getattr__(name):
    if name == "flash_attn_func":
        from .interface import flash_attn_func
        return flash_attn_func
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)

"""Longformer window + global sparse self-attention for AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C-ABI library
``liblfattn.so`` (declared in ``include/lf_attn.h``); this package is a thin
ctypes binding over it plus host-side helpers (seeded workloads, pair counts).

Importing the package loads nothing native; ``forward`` loads the library on
first use and raises if it has not been built.
"""

from __future__ import annotations

__all__ = ["forward", "forward_lse", "backward", "forward_global_proj", "forward_global_proj_lse",
           "backward_global_proj", "layer_forward", "LfAttn", "LfAttnError", "library_path"]


def __getattr__(name):
    if name in __all__ or name == "load_library":
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)

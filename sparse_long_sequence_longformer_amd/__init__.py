"""Longformer window + global sparse self-attention forward for AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C-ABI library
``liblfattn.so`` (declared in ``include/lf_attn.h``); this package is a thin
ctypes binding over it plus host-side helpers (seeded workloads, pair counts).

Importing the package loads nothing native; ``forward`` loads the library on
first use and raises if it has not been built.
"""

from __future__ import annotations

__all__ = ["forward", "forward_lse", "backward", "forward_global_proj", "LfAttn", "LfAttnError", "library_path"]


def __getattr__(name):
    if name in ("forward", "forward_lse", "backward", "forward_global_proj", "LfAttn", "LfAttnError",
                "library_path", "load_library"):
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)

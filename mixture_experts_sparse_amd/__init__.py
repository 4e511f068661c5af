"""Sparse Mixture-of-Experts layer for AMD MI355X (gfx950).

The layer (route -> top-k -> capacity-limited permutation -> grouped SwiGLU
experts -> weighted combine) runs as hand-written HIP kernels in
``libmoe_mi355x.so`` behind the C ABI of ``include/moe.h``; ``_lib`` is its
thin ctypes binding.  ``workloads`` draws the seeded synthetic inputs.

Importing the binding loads the library and fails loudly when it is missing.
"""
from . import workloads  # noqa: F401

__all__ = ["workloads", "load"]


def load():
    """Import and return the C-ABI binding module (raises if the library is not built)."""
    from . import _lib
    return _lib

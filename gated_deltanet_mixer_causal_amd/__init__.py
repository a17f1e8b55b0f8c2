"""Gated DeltaNet causal mixer for AMD Instinct MI355X (gfx950).

The compute path is libgdn.so (hand-written HIP kernels behind the C ABI in
include/gdn.h); `ops` marshals torch tensors into it.  Import of this package
does not load the library; the first call does, and fails loudly if it has
not been built.
"""
import importlib

from ._lib import GdnError, load  # noqa: F401

__all__ = ["GdnError", "load", "ops"]


def __getattr__(name):
    if name == "ops":
        return importlib.import_module(__name__ + ".ops")
    raise AttributeError(name)

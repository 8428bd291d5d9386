"""Fused multi-tensor AdamW for AMD MI355X (gfx950).

The update runs in ``libapexw.so`` (HIP kernels behind the C ABI of
``include/apexw.h``); ``_lib`` is its ctypes binding and ``AdamW`` a torch
wrapper that supplies device memory and the stream.  Importing the package
does not load the library; the first call that needs it does, and raises if
it has not been built.
"""
from . import _lib
from ._lib import ApexwError

__all__ = ["AdamW", "ApexwError", "_lib"]


def __getattr__(name):
    if name == "AdamW":
        from .optim import AdamW
        return AdamW
    raise AttributeError(name)

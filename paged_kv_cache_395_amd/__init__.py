"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

Hand-written HIP kernels behind the C ABI of include/pa.h (libpa.so), a
native host block manager, and thin Python bindings.  Importing the package
loads the library and raises if it has not been built.
"""

from . import _lib
from ._lib import NoSpace, PAError, UnknownSequence  # noqa: F401
from .block_manager import BlockManager  # noqa: F401
from .scheduler import Scheduler  # noqa: F401

_lib.load()

__all__ = ["BlockManager", "Scheduler", "PAError", "NoSpace", "UnknownSequence", "ops"]


def __getattr__(name):
    # torch is only needed for the device entry points
    if name == "ops":
        import importlib
        return importlib.import_module(__name__ + ".ops")
    raise AttributeError(name)

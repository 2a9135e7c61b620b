"""Dynamic top-K sparse decode attention for AMD Instinct MI355X (gfx950).

The computation lives in libstdk.so (hand-written HIP, C ABI in
include/stdk.h); this package only builds it and marshals arguments.
"""

import importlib

from . import native  # noqa: F401

__all__ = ["native", "ops"]


def __getattr__(name):
    if name == "ops":
        return importlib.import_module(__name__ + ".ops")
    raise AttributeError(name)

"""Paged KV cache and paged decode attention for AMD MI355X (gfx950).

The compute lives in ``libpagedkv.so`` (HIP kernels plus a host block
manager, C ABI in ``include/pagedkv.h``); :mod:`.native` is its ctypes
binding. Every public name is re-exported from there on first use, which loads
the library and fails loudly (ImportError) if it has not been built. The build
step itself (:mod:`.build`) does not load it.
"""

import importlib

_native = None


def __getattr__(name):
    global _native
    if name.startswith("__"):
        raise AttributeError(name)
    if _native is None:
        _native = importlib.import_module(".native", __name__)
    try:
        return getattr(_native, name)
    except AttributeError:
        raise AttributeError(f"module {__name__!r} has no attribute {name!r}") from None


def __dir__():
    mod = importlib.import_module(".native", __name__)
    return sorted(set(globals()) | {n for n in dir(mod) if not n.startswith("_")})

"""WildCat weighted-coreset attention on MI355X (gfx950).

The compute path lives in the HIP library ``libwildcat.so`` (C ABI declared in
``include/wildcat.h``); :mod:`nystr_rpcholesky_coreset_amd.wildcat` is a thin
ctypes binding over it.  The binding is imported lazily so that the input
generators can be used on hosts without the built library.
"""

__all__ = ["inputs", "wildcat"]


def __getattr__(name):
    if name == "wildcat":
        from . import wildcat as _w
        return _w
    if name == "inputs":
        from . import inputs as _i
        return _i
    raise AttributeError(name)

"""WildCat weighted-coreset attention on MI355X (gfx950).

The compute path lives in the HIP library ``libwildcat.so`` (C ABI declared in
``include/wildcat.h``); ``nystr_rpcholesky_coreset_amd.wildcat`` is a thin
ctypes binding over it (import it explicitly; it raises if the library has not
been built).  ``nystr_rpcholesky_coreset_amd.inputs`` holds the seeded
synthetic workloads.
"""

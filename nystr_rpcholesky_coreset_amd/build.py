"""Build libwildcat.so (HIP, gfx950) in-tree with hipcc.

    python -m nystr_rpcholesky_coreset_amd.build

Every call recompiles every source.  The library lands next to this file,
with a second build of it for the tests, libwildcat_streamcheck.so: the same
sources, but RPNys takes its non-temporal and kept-column factor loads from
the first round on (cache thresholds of 0 and 2 MiB instead of 256 and
224 MiB), so that small cases exercise those paths.  Only the tests load it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libwildcat.so")
STREAMCHECK_LIB = os.path.join(HERE, "libwildcat_streamcheck.so")
STREAMCHECK_DEFINES = ["-DWILDCAT_SELECT_CACHED_BYTES=0", "-DWILDCAT_SELECT_KEEP_BYTES=(2ull<<20)"]
SOURCES = ["api.hip", "select.hip", "contract.hip", "trsm.hip", "guard.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep a*b and (.)-(.) as separate roundings unless fma() is written out
    "-ffp-contract=on",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    objdir = os.path.join(ROOT, "_build", "obj")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    sc_obj = os.path.join(objdir, "select_streamcheck.o")
    cmds.append([HIPCC, *FLAGS, *STREAMCHECK_DEFINES, "-c", os.path.join(CSRC, "select.hip"), "-o", sc_obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    for lib, lib_objs in ((LIB, objs), (STREAMCHECK_LIB, [sc_obj if o.endswith("select.o") else o for o in objs])):
        tmp = lib + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

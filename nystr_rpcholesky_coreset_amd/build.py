"""Build libwildcat.so (HIP, gfx950) in-tree with hipcc.

    python -m nystr_rpcholesky_coreset_amd.build [--sanitize]

Every call recompiles every source.  The library lands next to this file,
with two test builds of it that only the tests load:
  libwildcat_streamcheck.so  the same sources, but RPNys takes its
      non-temporal and kept-column factor loads from the first round on
      (cache thresholds of 0 and 2 MiB instead of 256 and 224 MiB), so that
      small cases exercise those paths;
  libwildcat_hostsan.so      the host side of the C ABI (argument validation,
      layout and workspace sizing: api.hip) built with AddressSanitizer and
      UndefinedBehaviorSanitizer, linked with the ordinary kernel objects;
      loaded with the sanitizer runtime preloaded (hostsan_env()).
--sanitize builds only the last one (from the existing kernel objects when
they are there).
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
SOURCES = ["api.hip", "select.hip", "contract.hip", "trsm.hip", "guard.hip", "noalloc.hip"]
ARCH = "gfx950"

HOSTSAN_LIB = os.path.join(HERE, "libwildcat_hostsan.so")
# host code only: every -fsanitize= follows -Xarch_host, the device code is unchanged
HOSTSAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-fsanitize=address",
                 "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined"]
HOSTSAN_LINK = ["-shared-libsan", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]

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


def asan_runtime():
    """Path of the clang AddressSanitizer runtime that hipcc links against, or None."""
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def hostsan_env(env=None):
    """Environment for a process that loads libwildcat_hostsan.so."""
    env = dict(os.environ if env is None else env)
    env.update(LD_PRELOAD=asan_runtime() or "", ASAN_OPTIONS="detect_leaks=0", WILDCAT_LIBRARY=HOSTSAN_LIB)
    return env


def _objs(objdir):
    return [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]


def _link(lib, lib_objs, extra=()):
    tmp = lib + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *lib_objs])
    os.replace(tmp, lib)


def _hostsan_cmds(objdir):
    flags = [f for f in FLAGS if f != "-O3"]
    san_obj = os.path.join(objdir, "api_hostsan.o")
    return san_obj, [[HIPCC, *flags, *HOSTSAN_FLAGS, "-c", os.path.join(CSRC, "api.hip"), "-o", san_obj]]


def build(verbose: bool = False, sanitize_only: bool = False) -> str:
    objdir = os.path.join(ROOT, "_build", "obj")
    os.makedirs(objdir, exist_ok=True)
    objs = _objs(objdir)
    san_obj, cmds = _hostsan_cmds(objdir)
    if not sanitize_only or not all(os.path.exists(o) for o in objs):
        cmds += [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    sc_obj = os.path.join(objdir, "select_streamcheck.o")
    if not sanitize_only:
        cmds.append([HIPCC, *FLAGS, *STREAMCHECK_DEFINES, "-c", os.path.join(CSRC, "select.hip"), "-o", sc_obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    _link(HOSTSAN_LIB, [san_obj if o.endswith("api.o") else o for o in objs], HOSTSAN_LINK)
    if sanitize_only:
        return HOSTSAN_LIB
    _link(LIB, objs)
    _link(STREAMCHECK_LIB, [sc_obj if o.endswith("select.o") else o for o in objs])
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize_only="--sanitize" in sys.argv))

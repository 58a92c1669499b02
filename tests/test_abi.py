"""C ABI checks that need no GPU: the library loads, exports every function
include/wildcat.h declares, sizes workspaces, and rejects bad arguments on
the host before anything is launched (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wildcat.h")

wc = pytest.importorskip("nystr_rpcholesky_coreset_amd.wildcat", reason="libwildcat.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wildcat_[a-z_]+)\s*\(", src)))


def test_header_declares_the_three_path_calls():
    names = _declared()
    for n in ("wildcat_select", "wildcat_weights", "wildcat_attend"):
        assert n in names


def test_library_exports_every_declared_function():
    names = _declared()
    assert set(names) == set(wc.EXPORTED)
    for n in names:
        assert hasattr(wc.lib, n), n


def test_streamcheck_build_exports_the_same_functions():
    """The test build with small cache thresholds (used by the GPU tests of the
    factor-load paths) is the same library: it loads and exports every call,
    and sizes workspaces identically."""
    from nystr_rpcholesky_coreset_amd import build as B
    if not os.path.exists(B.STREAMCHECK_LIB):
        pytest.skip("libwildcat_streamcheck.so not built")
    lib = wc.load_library(B.STREAMCHECK_LIB)
    for n in _declared():
        assert hasattr(lib, n), n
    desc = _kv()
    assert lib.wildcat_select_workspace_bytes(ctypes.byref(desc)) == wc.lib.wildcat_select_workspace_bytes(
        ctypes.byref(desc))


FAKE = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: validation fails first


def _kv(**kw):
    base = dict(batch=2, kv_heads=4, n=5000, d=128, r=256, beta=0.1, tau=1.0, recentre=0, dtype=wc.WILDCAT_BF16,
                factor=0)
    base.update(kw)
    return wc.KVDesc(*[base[f] for f, _ in wc.KVDesc._fields_])


def test_workspace_sizes_are_positive_and_grow_with_r():
    a = wc.select_workspace_bytes(_kv(r=128))
    b = wc.select_workspace_bytes(_kv(r=256))
    assert 0 < a < b
    # the factor dominates: U * r * npad * 8 bytes
    assert b >= 8 * 256 * 5120 * 8
    assert wc.weights_workspace_bytes(_kv()) > 0
    assert wc.select_workspace_bytes(_kv(d=100)) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(d=100), wc.WILDCAT_ERR_SHAPE),
    (dict(r=0), wc.WILDCAT_ERR_SHAPE),
    (dict(r=5001), wc.WILDCAT_ERR_SHAPE),
    (dict(n=5000, r=4097), wc.WILDCAT_ERR_SHAPE),
    (dict(n=0, r=1), wc.WILDCAT_ERR_SHAPE),
    (dict(batch=0), wc.WILDCAT_ERR_SHAPE),
    (dict(dtype=7), wc.WILDCAT_ERR_DTYPE),
    (dict(beta=0.0), wc.WILDCAT_ERR_ARG),
    (dict(beta=float("nan")), wc.WILDCAT_ERR_ARG),
    (dict(tau=-1.0), wc.WILDCAT_ERR_ARG),
    (dict(tau=float("inf")), wc.WILDCAT_ERR_ARG),
    (dict(recentre=2), wc.WILDCAT_ERR_ARG),
    (dict(factor=2), wc.WILDCAT_ERR_ARG),
    (dict(factor=-1), wc.WILDCAT_ERR_ARG),
])
def test_select_rejects_bad_descriptors(kw, status):
    d = _kv(**kw)
    assert wc.lib.wildcat_select(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == status
    assert wc.lib.wildcat_weights(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, 1 << 40, None) == status


def test_null_and_misaligned_pointers_and_small_workspace():
    d = _kv()
    assert wc.lib.wildcat_select(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == wc.WILDCAT_ERR_ARG
    assert wc.lib.wildcat_select(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == wc.WILDCAT_ERR_ARG
    assert wc.lib.wildcat_select(ctypes.byref(d), ctypes.c_void_p((1 << 20) + 2), FAKE, FAKE, FAKE, FAKE, FAKE,
                                 1 << 40, None) == wc.WILDCAT_ERR_ARG
    need = wc.select_workspace_bytes(d)
    assert wc.lib.wildcat_select(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == wc.WILDCAT_ERR_WORKSPACE
    assert wc.lib.wildcat_select(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, need, None) == wc.WILDCAT_ERR_WORKSPACE
    needw = wc.weights_workspace_bytes(d)
    assert wc.lib.wildcat_weights(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  needw - 1, None) == wc.WILDCAT_ERR_WORKSPACE


@pytest.mark.parametrize("kw,status", [
    (dict(q_heads=6, kv_heads=4), wc.WILDCAT_ERR_SHAPE),
    (dict(d=48), wc.WILDCAT_ERR_SHAPE),
    (dict(m=0), wc.WILDCAT_ERR_SHAPE),
    (dict(r=5000), wc.WILDCAT_ERR_SHAPE),
    (dict(beta=-1.0), wc.WILDCAT_ERR_ARG),
    (dict(dtype=3), wc.WILDCAT_ERR_DTYPE),
])
def test_attend_rejects_bad_descriptors(kw, status):
    base = dict(batch=1, q_heads=8, kv_heads=4, m=64, d=128, r=256, beta=0.1, dtype=wc.WILDCAT_BF16)
    base.update(kw)
    q = wc.QDesc(*[base[f] for f, _ in wc.QDesc._fields_])
    assert wc.lib.wildcat_attend(ctypes.byref(q), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == status


def _q(**kw):
    base = dict(batch=2, q_heads=8, kv_heads=4, m=64, d=128, r=256, beta=0.1, dtype=wc.WILDCAT_BF16)
    base.update(kw)
    return wc.QDesc(*[base[f] for f, _ in wc.QDesc._fields_])


@pytest.mark.parametrize("kdesc,qdesc,status", [
    (dict(d=100), None, wc.WILDCAT_ERR_SHAPE),
    (dict(beta=-1.0), None, wc.WILDCAT_ERR_ARG),
    (dict(), dict(d=64), wc.WILDCAT_ERR_SHAPE),          # query d differs from the keys'
    (dict(), dict(dtype=wc.WILDCAT_FP32), wc.WILDCAT_ERR_DTYPE),
    (dict(), dict(q_heads=6), wc.WILDCAT_ERR_SHAPE),     # not a multiple of kv_heads
    (dict(), dict(m=0), wc.WILDCAT_ERR_SHAPE),
])
def test_check_range_rejects_bad_descriptors(kdesc, qdesc, status):
    d = _kv(**kdesc)
    q = _q(**qdesc) if qdesc is not None else None
    got = wc.lib.wildcat_check_range(ctypes.byref(d), FAKE, ctypes.byref(q) if q is not None else None,
                                     FAKE if q is not None else None, FAKE, None, None)
    assert got == status


def test_check_range_rejects_bad_pointers():
    d, q = _kv(), _q()
    cr = wc.lib.wildcat_check_range
    assert cr(ctypes.byref(d), None, None, None, FAKE, None, None) == wc.WILDCAT_ERR_ARG
    assert cr(ctypes.byref(d), FAKE, None, None, None, None, None) == wc.WILDCAT_ERR_ARG          # no scratch
    assert cr(ctypes.byref(d), FAKE, None, None, ctypes.c_void_p((1 << 20) + 4), None, None) == wc.WILDCAT_ERR_ARG
    assert cr(ctypes.byref(d), FAKE, ctypes.byref(q), None, FAKE, None, None) == wc.WILDCAT_ERR_ARG  # Q missing
    assert cr(ctypes.byref(d), FAKE, None, FAKE, FAKE, None, None) == wc.WILDCAT_ERR_ARG             # qdesc missing


def test_status_strings():
    for st in (wc.WILDCAT_OK, wc.WILDCAT_ERR_ARG, wc.WILDCAT_ERR_DTYPE, wc.WILDCAT_ERR_SHAPE,
               wc.WILDCAT_ERR_WORKSPACE, wc.WILDCAT_ERR_RANGE, wc.WILDCAT_ERR_HIP, wc.WILDCAT_ERR_SCRATCH):
        assert wc.lib.wildcat_status_string(st) and b"unknown" not in wc.lib.wildcat_status_string(st)
    assert b"unknown" in wc.lib.wildcat_status_string(42)


def test_merge_value_ranges_validation():
    mv = wc.lib.wildcat_merge_value_ranges
    assert mv(0, 4, 128, FAKE, FAKE, FAKE, FAKE, None) == wc.WILDCAT_ERR_SHAPE
    assert mv(8, 0, 128, FAKE, FAKE, FAKE, FAKE, None) == wc.WILDCAT_ERR_SHAPE
    assert mv(8, 4, 100, FAKE, FAKE, FAKE, FAKE, None) == wc.WILDCAT_ERR_SHAPE
    assert mv(40000, 2, 64, FAKE, FAKE, FAKE, FAKE, None) == wc.WILDCAT_ERR_SHAPE
    assert mv(8, 4, 128, None, FAKE, FAKE, FAKE, None) == wc.WILDCAT_ERR_ARG
    assert mv(8, 4, 128, FAKE, FAKE, FAKE, None, None) == wc.WILDCAT_ERR_ARG


@pytest.mark.parametrize("kw,status", [
    (dict(q_heads=6, kv_heads=4), wc.WILDCAT_ERR_SHAPE),
    (dict(d=48), wc.WILDCAT_ERR_SHAPE),
    (dict(m=0), wc.WILDCAT_ERR_SHAPE),
    (dict(r=0), wc.WILDCAT_ERR_SHAPE),
    (dict(beta=float("inf")), wc.WILDCAT_ERR_ARG),
    (dict(dtype=3), wc.WILDCAT_ERR_DTYPE),
])
def test_decode_rejects_bad_descriptors(kw, status):
    q = _q(**kw)
    assert wc.decode_workspace_bytes(q) == 0
    assert wc.lib.wildcat_decode(ctypes.byref(q), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                                 None) == status


def test_decode_rejects_bad_pointers_and_small_workspace():
    q = _q()
    need = wc.decode_workspace_bytes(q)
    # staged operand: U (r + m) (2d + 4(d+1)) bytes, plus the running ranges U m d 8
    U, R = 2 * 4, 256 + 64
    assert need >= U * R * (2 * 128 + 4 * 129) + U * 64 * 128 * 8
    assert wc.decode_workspace_bytes(_q(m=128)) > need
    args = [FAKE] * 9
    for k in range(8):   # Q, K_S, X, vmin, vmax, K_new, V_new, O
        a = list(args)
        a[k] = None
        assert wc.lib.wildcat_decode(ctypes.byref(q), *a, need, None) == wc.WILDCAT_ERR_ARG
    for k in (0, 1, 5, 6):   # Q, K_S, K_new, V_new are read with 16-byte loads
        a = list(args)
        a[k] = ctypes.c_void_p((1 << 20) + 4)
        assert wc.lib.wildcat_decode(ctypes.byref(q), *a, need, None) == wc.WILDCAT_ERR_ARG
    assert wc.lib.wildcat_decode(ctypes.byref(q), *args, need - 1, None) == wc.WILDCAT_ERR_WORKSPACE
    a = list(args)
    a[8] = None
    assert wc.lib.wildcat_decode(ctypes.byref(q), *a, need, None) == wc.WILDCAT_ERR_WORKSPACE
    a[8] = ctypes.c_void_p((1 << 20) + 8)
    assert wc.lib.wildcat_decode(ctypes.byref(q), *a, need, None) == wc.WILDCAT_ERR_WORKSPACE


def test_float32_factor_halves_the_factor_workspace():
    a, b = wc.select_workspace_bytes(_kv(factor=0)), wc.select_workspace_bytes(_kv(factor=1))
    U, npad, r = 8, 5120, 256
    assert a - b >= U * r * npad * 4 - 512
    assert b > U * r * npad * 4
    assert wc.weights_workspace_bytes(_kv(factor=1)) == wc.weights_workspace_bytes(_kv(factor=0))


def test_decode_noalloc_validation_before_any_launch():
    """wildcat_decode_noalloc rejects an invalid descriptor and a call larger
    than its static scratch on the host, before touching the GPU."""
    q = wc.QDesc(1, 32, 8, 1879, 128, 1024, 0.1, wc.WILDCAT_BF16)
    assert wc.decode_workspace_bytes(q) > wc.NOALLOC_SCRATCH_BYTES
    call = wc.lib.wildcat_decode_noalloc
    assert call(ctypes.byref(q), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == wc.WILDCAT_ERR_SCRATCH
    q.m = 1878
    assert wc.decode_workspace_bytes(q) <= wc.NOALLOC_SCRATCH_BYTES
    q.d = 100
    assert call(ctypes.byref(q), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == wc.WILDCAT_ERR_SHAPE
    assert call(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == wc.WILDCAT_ERR_ARG

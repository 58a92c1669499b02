"""Thin ctypes binding over libwildcat.so (C ABI in include/wildcat.h).

Argument marshalling only: torch tensors provide device memory and the
current stream; every step of the computation runs in the HIP library.  If the
library has not been built this module raises at import -- there is no
fallback path.

Shapes (row-major, head dim fastest):
    K, V   [batch][kv_heads][n][d]       Q, O   [batch][q_heads][m][d]
    u      [batch*kv_heads][r] float64   S      [batch*kv_heads][r] int32
    L      [batch*kv_heads][r][r] float64
    K_S    [batch][kv_heads][r][d]       X      [batch][kv_heads][r][d+1] float32
    vmin, vmax [batch][kv_heads][d] float32
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# WILDCAT_LIBRARY may point at another build of the same library (e.g. a
# tuning variant); by default the in-tree build next to this file is used.
LIB_PATH = os.environ.get("WILDCAT_LIBRARY") or os.path.join(_HERE, "libwildcat.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m nystr_rpcholesky_coreset_amd.build`")


WILDCAT_OK = 0
WILDCAT_ERR_ARG = -1
WILDCAT_ERR_DTYPE = -2
WILDCAT_ERR_SHAPE = -3
WILDCAT_ERR_WORKSPACE = -4
WILDCAT_ERR_RANGE = -5
WILDCAT_ERR_HIP = -6
WILDCAT_ERR_SCRATCH = -7
RANGE_LIMIT = 64.0    # WILDCAT_RANGE_LIMIT
NOALLOC_SCRATCH_BYTES = 32 << 20   # WILDCAT_NOALLOC_SCRATCH_BYTES
WILDCAT_FP32 = 0
WILDCAT_BF16 = 1

EXPORTED = (
    "wildcat_select_workspace_bytes", "wildcat_weights_workspace_bytes", "wildcat_select",
    "wildcat_weights", "wildcat_attend", "wildcat_decode_workspace_bytes", "wildcat_decode",
    "wildcat_merge_value_ranges", "wildcat_check_range", "wildcat_status_string", "wildcat_decode_noalloc",
)


class KVDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("n", ctypes.c_int32),
                ("d", ctypes.c_int32), ("r", ctypes.c_int32), ("beta", ctypes.c_double),
                ("tau", ctypes.c_double), ("recentre", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("factor", ctypes.c_int32)]


class QDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("m", ctypes.c_int32), ("d", ctypes.c_int32), ("r", ctypes.c_int32),
                ("beta", ctypes.c_double), ("dtype", ctypes.c_int32)]


_vp = ctypes.c_void_p


def load_library(path: str) -> ctypes.CDLL:
    """Open a build of the library at `path` with the C signatures of
    include/wildcat.h declared (the module's own `lib` is one)."""
    lib = ctypes.CDLL(path)
    lib.wildcat_select_workspace_bytes.argtypes = [ctypes.POINTER(KVDesc)]
    lib.wildcat_select_workspace_bytes.restype = ctypes.c_size_t
    lib.wildcat_weights_workspace_bytes.argtypes = [ctypes.POINTER(KVDesc)]
    lib.wildcat_weights_workspace_bytes.restype = ctypes.c_size_t
    lib.wildcat_select.argtypes = [ctypes.POINTER(KVDesc), _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.wildcat_select.restype = ctypes.c_int
    lib.wildcat_weights.argtypes = [ctypes.POINTER(KVDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    ctypes.c_size_t, _vp]
    lib.wildcat_weights.restype = ctypes.c_int
    lib.wildcat_attend.argtypes = [ctypes.POINTER(QDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.wildcat_attend.restype = ctypes.c_int
    lib.wildcat_decode_workspace_bytes.argtypes = [ctypes.POINTER(QDesc)]
    lib.wildcat_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.wildcat_decode.argtypes = [ctypes.POINTER(QDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                   _vp]
    lib.wildcat_decode.restype = ctypes.c_int
    lib.wildcat_decode_noalloc.argtypes = [ctypes.POINTER(QDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.wildcat_decode_noalloc.restype = ctypes.c_int
    lib.wildcat_merge_value_ranges.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp]
    lib.wildcat_merge_value_ranges.restype = ctypes.c_int
    lib.wildcat_check_range.argtypes = [ctypes.POINTER(KVDesc), _vp, ctypes.POINTER(QDesc), _vp, _vp,
                                        ctypes.POINTER(ctypes.c_double), _vp]
    lib.wildcat_check_range.restype = ctypes.c_int
    lib.wildcat_status_string.argtypes = [ctypes.c_int]
    lib.wildcat_status_string.restype = ctypes.c_char_p
    return lib


lib = load_library(LIB_PATH)


class WildcatError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {lib.wildcat_status_string(status).decode()} (status {status}){detail}")


def _check(status: int, where: str):
    if status != WILDCAT_OK:
        raise WildcatError(status, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return WILDCAT_BF16
    if t.dtype == torch.float32:
        return WILDCAT_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocations made inside belong to the stream the kernels run on, so the
    caching allocator does not hand their memory to work on another stream
    while those kernels may still use it (a workspace is released when the
    call returns, before the kernels have finished)."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


FACTORS = {"f64": 0, "f32": 1}   # wildcat_factor: storage of the RPNys factor


def kv_desc(K: torch.Tensor, r: int, beta: float, tau: float = 1.0, recentre: bool = False,
            factor: str = "f64") -> KVDesc:
    B, H, n, d = K.shape
    if factor not in FACTORS:
        raise ValueError(f"factor must be one of {sorted(FACTORS)}")
    return KVDesc(B, H, n, d, int(r), float(beta), float(tau), int(bool(recentre)), _dtype_code(K), FACTORS[factor])


def select_workspace_bytes(desc: KVDesc) -> int:
    return lib.wildcat_select_workspace_bytes(ctypes.byref(desc))


def weights_workspace_bytes(desc: KVDesc) -> int:
    return lib.wildcat_weights_workspace_bytes(ctypes.byref(desc))


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def select(K, u, r, beta, tau=1.0, recentre=False, workspace=None, stream=None, factor="f64"):
    """wildcat_select: returns (S [U][r] int32, r_eff [U] int32, L [U][r][r] float64).
    factor: "f64" or "f32" storage of the factor (wildcat_factor)."""
    desc = kv_desc(K, r, beta, tau, recentre, factor)
    U = desc.batch * desc.kv_heads
    dev = K.device
    with _on(stream):
        S = torch.empty((U, r), dtype=torch.int32, device=dev)
        r_eff = torch.empty((U,), dtype=torch.int32, device=dev)
        L = torch.empty((U, r, r), dtype=torch.float64, device=dev)
        nbytes = select_workspace_bytes(desc)
        ws = _workspace(nbytes, dev, workspace)
        _check(lib.wildcat_select(ctypes.byref(desc), _ptr(K), _ptr(u), _ptr(S), _ptr(r_eff), _ptr(L),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "wildcat_select")
    return S, r_eff, L


def weights(K, V, S, r_eff, L, r, beta, tau=1.0, recentre=False, workspace=None, stream=None):
    """wildcat_weights: returns (K_S, X, vmin, vmax)."""
    desc = kv_desc(K, r, beta, tau, recentre)
    B, H, n, d = K.shape
    dev = K.device
    with _on(stream):
        K_S = torch.empty((B, H, r, d), dtype=K.dtype, device=dev)
        X = torch.empty((B, H, r, d + 1), dtype=torch.float32, device=dev)
        vmin = torch.empty((B, H, d), dtype=torch.float32, device=dev)
        vmax = torch.empty((B, H, d), dtype=torch.float32, device=dev)
        nbytes = weights_workspace_bytes(desc)
        ws = _workspace(nbytes, dev, workspace)
        _check(lib.wildcat_weights(ctypes.byref(desc), _ptr(K), _ptr(V), _ptr(S), _ptr(r_eff), _ptr(L), _ptr(K_S),
                                   _ptr(X), _ptr(vmin), _ptr(vmax), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "wildcat_weights")
    return K_S, X, vmin, vmax


def attend(Q, K_S, X, vmin, vmax, beta, stream=None, out=None):
    """wildcat_attend: returns O [batch][q_heads][m][d] float32."""
    B, Hq, m, d = Q.shape
    Hkv, r = K_S.shape[1], K_S.shape[2]
    desc = QDesc(B, Hq, Hkv, m, d, r, float(beta), _dtype_code(Q))
    with _on(stream):
        O = out if out is not None else torch.empty((B, Hq, m, d), dtype=torch.float32, device=Q.device)
    _check(lib.wildcat_attend(ctypes.byref(desc), _ptr(Q), _ptr(K_S), _ptr(X), _ptr(vmin), _ptr(vmax), _ptr(O),
                              _stream(stream)), "wildcat_attend")
    return O


def decode_workspace_bytes(desc: QDesc) -> int:
    return lib.wildcat_decode_workspace_bytes(ctypes.byref(desc))


def decode(Q, K_S, X, vmin, vmax, K_new, V_new, beta, workspace=None, stream=None, out=None):
    """wildcat_decode: the m new tokens (K_new, V_new [batch][kv_heads][m][d];
    query row i of Q is token i's query) attend to the cache (K_S, X, vmin,
    vmax) and causally to each other; returns O [batch][q_heads][m][d] float32."""
    B, Hq, m, d = Q.shape
    Hkv, r = K_S.shape[1], K_S.shape[2]
    desc = QDesc(B, Hq, Hkv, m, d, r, float(beta), _dtype_code(Q))
    with _on(stream):
        O = out if out is not None else torch.empty((B, Hq, m, d), dtype=torch.float32, device=Q.device)
        ws = _workspace(decode_workspace_bytes(desc), Q.device, workspace)
        _check(lib.wildcat_decode(ctypes.byref(desc), _ptr(Q), _ptr(K_S), _ptr(X), _ptr(vmin), _ptr(vmax),
                                  _ptr(K_new), _ptr(V_new), _ptr(O), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "wildcat_decode")
    return O


def decode_noalloc(Q, K_S, X, vmin, vmax, K_new, V_new, beta, out, stream=None):
    """wildcat_decode_noalloc: wildcat_decode with the library's static
    scratch instead of a workspace; `out` (O) must be given, nothing is
    allocated.  Calls overlapping on one GPU race on that scratch."""
    B, Hq, m, d = Q.shape
    Hkv, r = K_S.shape[1], K_S.shape[2]
    desc = QDesc(B, Hq, Hkv, m, d, r, float(beta), _dtype_code(Q))
    _check(lib.wildcat_decode_noalloc(ctypes.byref(desc), _ptr(Q), _ptr(K_S), _ptr(X), _ptr(vmin), _ptr(vmax),
                                      _ptr(K_new), _ptr(V_new), _ptr(out), _stream(stream)), "wildcat_decode_noalloc")
    return out


def check_range(K, r, beta, tau=1.0, recentre=False, Q=None, scratch=None, stream=None):
    """wildcat_check_range (host-synchronous): returns the exponent bounds
    (E_k, E_q); raises WildcatError with status WILDCAT_ERR_RANGE when one
    exceeds RANGE_LIMIT."""
    desc = kv_desc(K, r, beta, tau, recentre)
    qd = None
    if Q is not None:
        B, Hq, m, d = Q.shape
        qd = QDesc(B, Hq, K.shape[1], m, d, int(r), float(beta), _dtype_code(Q))
    with _on(stream):
        buf = scratch if scratch is not None else torch.empty(2, dtype=torch.float64, device=K.device)
        bounds = (ctypes.c_double * 2)()
        st = lib.wildcat_check_range(ctypes.byref(desc), _ptr(K), ctypes.byref(qd) if qd is not None else None,
                                     _ptr(Q), _ptr(buf), bounds, _stream(stream))
    if st != WILDCAT_OK:
        raise WildcatError(st, "wildcat_check_range",
                           f": E_k = {bounds[0]:.4g}, E_q = {bounds[1]:.4g}" if st == WILDCAT_ERR_RANGE else "")
    return bounds[0], bounds[1]


def merge_value_ranges(vmin_bins, vmax_bins, bins, stream=None):
    """wildcat_merge_value_ranges: [B][H*bins][d] per-bin ranges -> [B][H][d]."""
    Bt, HB, d = vmin_bins.shape
    H = HB // bins
    with _on(stream):
        vmin = torch.empty((Bt, H, d), dtype=torch.float32, device=vmin_bins.device)
        vmax = torch.empty_like(vmin)
    _check(lib.wildcat_merge_value_ranges(Bt * H, bins, d, _ptr(vmin_bins), _ptr(vmax_bins), _ptr(vmin), _ptr(vmax),
                                          _stream(stream)), "wildcat_merge_value_ranges")
    return vmin, vmax


def bin_view(T, bins):
    """[B][H][n][d] -> the bin-major view [B][H*bins][n/bins][d] (same memory)."""
    Bt, H, n, d = T.shape
    if n % bins:
        raise ValueError(f"n = {n} is not a multiple of bins = {bins}")
    return T.view(Bt, H * bins, n // bins, d)


def forward_binned(Q, K, V, u, r, bins, beta, tau=1.0, recentre=False, stream=None, factor="f64"):
    """Binned WildCat: select and weights on the bin-major view (each bin an
    RPNys problem with r/bins pivots), per-unit value ranges, attend over the
    concatenated coreset.  Returns (O, parts); parts["S"] holds indices local
    to each bin, [B*H*bins][r/bins]."""
    if r % bins:
        raise ValueError(f"r = {r} is not a multiple of bins = {bins}")
    Bt, H, n, d = K.shape
    rb = r // bins
    Kb, Vb = bin_view(K, bins), bin_view(V, bins)
    ub = u.reshape(Bt * H * bins, rb)
    S, r_eff, L = select(Kb, ub, rb, beta, tau, recentre, stream=stream, factor=factor)
    K_S, X, vmin_b, vmax_b = weights(Kb, Vb, S, r_eff, L, rb, beta, tau, recentre, stream=stream)
    vmin, vmax = merge_value_ranges(vmin_b, vmax_b, bins, stream=stream)
    K_S = K_S.view(Bt, H, r, d)
    X = X.view(Bt, H, r, d + 1)
    O = attend(Q, K_S, X, vmin, vmax, beta, stream=stream)
    return O, dict(S=S, r_eff=r_eff, L=L, K_S=K_S, X=X, vmin=vmin, vmax=vmax)


def compress_kv(K, V, u, r, beta, tau=1.0, recentre=True, stream=None, factor="f64"):
    """CompressKV: wildcat_select then wildcat_weights, returning the
    compressed cache dict(S, r_eff, L, K_S, X, vmin, vmax) that attend and
    decode consume.

    [WildCat, recentring paragraph and CompressKV / Alg. 2 paragraph: the
    compression works on the recentred keys k - kbar, kbar the mean of the
    unit's keys, so recentring is on unless turned off; the temperature tau
    is the caller's, its closed form not being recoverable from the pages.]
    Recentring never reaches attend or decode: its per-query factor cancels
    in the ratio of the plug-in estimator, so they take the raw K_S."""
    S, r_eff, L = select(K, u, r, beta, tau, recentre, stream=stream, factor=factor)
    K_S, X, vmin, vmax = weights(K, V, S, r_eff, L, r, beta, tau, recentre, stream=stream)
    return dict(S=S, r_eff=r_eff, L=L, K_S=K_S, X=X, vmin=vmin, vmax=vmax)


def forward(Q, K, V, u, r, beta, tau=1.0, recentre=False, stream=None, factor="f64"):
    """WildCat module: select -> weights -> attend on one stream.  Returns (O, parts)."""
    parts = compress_kv(K, V, u, r, beta, tau, recentre, stream=stream, factor=factor)
    O = attend(Q, parts["K_S"], parts["X"], parts["vmin"], parts["vmax"], beta, stream=stream)
    return O, parts

"""Shared helpers for the parity tests: input marshalling and comparisons.

Nothing here computes any part of the method: the expected values come from
the oracle, the tested values from the HIP library via the C ABI binding.
"""
from __future__ import annotations

import numpy as np

from nystr_rpcholesky_coreset_amd import inputs as I
from oracle import wildcat_oracle as orc

# A draw whose target u*T lies within NEAR_TIE * T0 of a prefix sum (T0 the
# initial residual trace) can flip under fp64 rounding differences in the
# residual diagonal and its prefix sums; the rounding error of those sums is
# ~1e-16..1e-14 * T0, so 1e-11 leaves three orders of margin.
NEAR_TIE = 1e-11


def tol_for(dtype: str) -> float:
    """Output tolerance relative to max|V|: 2e-3 for fp32 inputs, 2e-2 for bf16."""
    return 2e-3 if dtype == "fp32" else 2e-2


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def oracle_units(inp: dict, units, r=None):
    """Oracle CompressKV for the listed units (u = b*Hkv + h)."""
    w = inp["workload"]
    K = I.to_f64(inp["K"], w.dtype)
    V = I.to_f64(inp["V"], w.dtype)
    out = {}
    for u in units:
        b, h = divmod(u, w.kv_heads)
        rr = w.r if r is None else r
        out[u] = orc.compress_unit(K[b, h], V[b, h], inp["u"][u][:rr], rr, w.beta, w.tau, w.recentre)
    return out


def oracle_attend_rows(inp: dict, unit_res, qunit: int, rows=None):
    w = inp["workload"]
    b, h = divmod(qunit, w.q_heads)
    Q = I.to_f64(inp["Q"][b, h], w.dtype)
    if rows is not None:
        Q = Q[rows]
    return orc.plugin_attend(Q, unit_res.K_S, unit_res.X, unit_res.vmin, unit_res.vmax, w.beta)


# With float32 factor storage the two sides' factors can differ by one float32
# rounding where a float64 value falls on a rounding boundary, after which the
# residual diagonals differ at the float32 level (~1e-8 of T0 and below); a
# near tie is then a decision margin below NEAR_TIE_F32.
NEAR_TIE_F32 = 1e-6


# Every draw at which a comparison stopped on a near tie, as
# (context, draw, margin): printed in the session summary (conftest.py), so a
# shortened comparison is always visible.
NEAR_TIE_EXITS: list = []


def check_pivots(S_gpu: np.ndarray, reff_gpu: int, sel, near: float = NEAR_TIE, context: str = "") -> int:
    """Pivots must match the oracle bit for bit.  A mismatch is accepted only
    at a step whose oracle decision margin is below `near` (a near tie); then
    the comparison stops there and the exit is recorded in NEAR_TIE_EXITS.
    Returns the matched length (sel.r_eff when everything matched)."""
    n_or = sel.r_eff
    k = min(n_or, reff_gpu)
    for i in range(k):
        if int(S_gpu[i]) != int(sel.S[i]):
            assert sel.margins[i] < near, (
                f"pivot {i}: gpu {S_gpu[i]} vs oracle {sel.S[i]} with decision margin {sel.margins[i]:.3e}")
            NEAR_TIE_EXITS.append((context, i, float(sel.margins[i])))
            print(f"near tie {context}: pivots diverge at draw {i} (margin {sel.margins[i]:.3e}); "
                  f"comparison stops there", flush=True)
            return i
    assert reff_gpu == n_or, f"r_eff gpu {reff_gpu} vs oracle {n_or}"
    assert np.all(S_gpu[reff_gpu:] == -1)
    return k


def rel_max(a, b, scale):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) / scale

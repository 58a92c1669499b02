"""Parity at the full workload sizes, in the launch configuration bench.py times.

The HIP path runs on every unit of the workload; the oracle recomputes units
completely (pivots bit-exact, L, K_S, value range, outputs of every query head
of those units): sampled units of the ViT-shaped and latent workloads, all
eight units of the 32k KV-cache workload (also with recentring), and one
whole unit of the long-context workload (n = 131072, r = 2048: all 2048
pivots, L, and the 131072 output rows of its query head against the plug-in
estimate on the oracle's own coreset and weights).

A pivot mismatch at a near tie fails these tests: no comparison here may stop
short.
"""
import numpy as np
import pytest

from nystr_rpcholesky_coreset_amd import inputs as I
from oracle import wildcat_oracle as orc

from _helpers import oracle_units, rel_max, tol_for
from test_gpu_parity import _compare_unit, _run_gpu

pytestmark = pytest.mark.gpu

W = I.WORKLOADS
FULL = {
    "vit_b128_n3136_d64_r128_bf16": [0, 64, 127],
    "latent_b8h8_n4096_d64_r256_bf16": [0, 37, 63],
    "kvcache_gqa32x8_n32768_d128_r1024_bf16": list(range(8)),
}


def _check_ranges_and_clip(inp, g):
    w = inp["workload"]
    O = g["O"]
    vmin = g["vmin"].reshape(w.batch, w.kv_heads, 1, w.d).repeat(w.q_heads // w.kv_heads, axis=1)
    vmax = g["vmax"].reshape(w.batch, w.kv_heads, 1, w.d).repeat(w.q_heads // w.kv_heads, axis=1)
    assert np.all(O >= vmin) and np.all(O <= vmax)


@pytest.mark.parametrize("name", list(FULL))
def test_fullsize_units(name):
    w = W[name]
    print(f"workload {name}: generating inputs", flush=True)
    inp = I.make_inputs(w)
    g = _run_gpu(inp)
    assert np.all(g["r_eff"] == w.r)
    _check_ranges_and_clip(inp, g)
    print("running oracle on units", FULL[name], flush=True)
    ref = oracle_units(inp, FULL[name])
    for u, ures in ref.items():
        _compare_unit(inp, g, u, ures)


def test_fullsize_kvcache_recentred():
    """The 32k KV-cache workload with recentring on (every kernel evaluation
    of select and weights on the keys minus their per-unit mean; attend on the
    raw keys): two units against the oracle."""
    w = I.scaled_workload(W["kvcache_gqa32x8_n32768_d128_r1024_bf16"], recentre=True)
    print(f"workload {w.name} (recentred): generating inputs", flush=True)
    inp = I.make_inputs(w)
    g = _run_gpu(inp)
    assert np.all(g["r_eff"] == w.r)
    _check_ranges_and_clip(inp, g)
    units = [2, 6]
    print("running oracle on units", units, flush=True)
    ref = oracle_units(inp, units)
    for u, ures in ref.items():
        _compare_unit(inp, g, u, ures)


def test_fullsize_longctx_whole_unit():
    """One unit of the long-context workload against the full oracle run."""
    w = W["longctx_h8_n131072_d128_r2048_bf16"]
    print(f"workload {w.name}: generating inputs", flush=True)
    inp = I.make_inputs(w)
    g = _run_gpu(inp)
    assert np.all(g["r_eff"] == w.r)
    _check_ranges_and_clip(inp, g)
    unit = 3
    print(f"oracle: unit {unit}, all {w.r} rounds, weights and attend", flush=True)
    ref = oracle_units(inp, [unit])[unit]
    assert ref.sel.r_eff == w.r
    # pivots, L, K_S, value range, and O of every row of the unit's query head
    # (q_heads = kv_heads) against plugin_attend on the oracle's K_S and X
    _compare_unit(inp, g, unit, ref)
    b, h = divmod(unit, w.kv_heads)
    Xg = g["X"][b, h].astype(np.float64)
    xs = max(1e-300, float(np.abs(ref.X).max()))
    print(f"X: max|dX| / max|X| = {rel_max(Xg, ref.X, xs):.3e}", flush=True)

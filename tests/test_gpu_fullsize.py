"""Parity at the full workload sizes, in the launch configuration bench.py times.

The HIP path runs on every unit of the workload; the oracle recomputes a
sample of units completely (pivots bit-exact, L, K_S, value range, outputs of
every query head of those units).  For the long-context workload (n = 131072,
r = 2048) a full oracle run takes minutes, so the oracle runs the first 256
rounds of one unit (with the same uniforms the pivots of a shorter run are a
prefix of the longer run's), and the rest is checked through identities that
hold at any size: L L^T = h(K_S, K_S), (L L^T) X = h(K_S, K)[V, 1] on sampled
rows, the attend output against the plug-in formula on sampled query rows,
and the value-range clip.
"""
import numpy as np
import pytest

from nystr_rpcholesky_coreset_amd import inputs as I
from oracle import wildcat_oracle as orc

from _helpers import check_pivots, oracle_units, rel_max, tol_for
from test_gpu_parity import _compare_unit, _run_gpu

pytestmark = pytest.mark.gpu

W = I.WORKLOADS
FULL = {
    "vit_b128_n3136_d64_r128_bf16": [0, 64, 127],
    "latent_b8h8_n4096_d64_r256_bf16": [0, 37, 63],
    "kvcache_gqa32x8_n32768_d128_r1024_bf16": [5],
}


@pytest.mark.parametrize("name", list(FULL))
def test_fullsize_sampled_units(name):
    w = W[name]
    print(f"workload {name}: generating inputs", flush=True)
    inp = I.make_inputs(w)
    g = _run_gpu(inp)
    assert np.all(g["r_eff"] == w.r)
    Vmax = np.abs(I.to_f64(inp["V"], w.dtype)).max()
    O = g["O"]
    vmin = g["vmin"].reshape(w.batch, w.kv_heads, 1, w.d).repeat(w.q_heads // w.kv_heads, axis=1)
    vmax = g["vmax"].reshape(w.batch, w.kv_heads, 1, w.d).repeat(w.q_heads // w.kv_heads, axis=1)
    assert np.all(O >= vmin) and np.all(O <= vmax)
    print("running oracle on units", FULL[name], flush=True)
    ref = oracle_units(inp, FULL[name])
    for u, ures in ref.items():
        _compare_unit(inp, g, u, ures)


def test_fullsize_longctx_prefix_and_identities():
    w = W["longctx_h8_n131072_d128_r2048_bf16"]
    print(f"workload {w.name}: generating inputs", flush=True)
    inp = I.make_inputs(w)
    g = _run_gpu(inp)
    assert np.all(g["r_eff"] == w.r)
    unit = 3
    b, h = divmod(unit, w.kv_heads)
    K = I.to_f64(inp["K"], w.dtype)[b, h]
    V = I.to_f64(inp["V"], w.dtype)[b, h]
    S = g["S"][unit].astype(np.int64)
    L = g["L"][unit]
    assert len(set(S.tolist())) == w.r and S.min() >= 0 and S.max() < w.n

    # oracle: first 256 rounds with the same uniforms
    rp = 256
    print("oracle prefix run", flush=True)
    sel = orc.rpnys_select(K, inp["u"][unit][:rp], rp, w.beta)
    check_pivots(S[:rp], rp, sel)
    assert rel_max(L[:rp, :rp], sel.L, max(1.0, np.abs(sel.L).max())) < 1e-9

    # L L^T = h(K_S, K_S)
    KS = K[S]
    H = orc.selection_kernel(KS, KS, w.beta)
    assert rel_max(L @ L.T, H, np.abs(H).max()) < 1e-9
    np.testing.assert_array_equal(np.triu(L, 1), 0.0)

    # (L L^T) X = h(K_S, K) [V, 1] on sampled rows: the residual of the
    # computed weights is the bf16 rounding of P in the contraction.
    X = g["X"][b, h].astype(np.float64)
    rows = np.random.default_rng(0).choice(w.r, 8, replace=False)
    V1 = np.hstack([V, np.ones((w.n, 1))])
    P = orc.selection_kernel(KS[rows], K, w.beta)
    Y = P @ V1
    scale = P @ np.abs(V1)
    res = np.abs(H[rows] @ X - Y) / scale
    print(f"weights identity residual (relative to sum |P||V|): {res.max():.3e}")
    assert res.max() < 5e-3

    # attend against the plug-in formula on the GPU's own compressed cache
    KSg = g["K_S"][b, h].astype(np.float64)
    np.testing.assert_array_equal(KSg, KS)
    vmin, vmax = orc.value_range(V)
    np.testing.assert_array_equal(g["vmin"][b, h], vmin.astype(np.float32))
    np.testing.assert_array_equal(g["vmax"][b, h], vmax.astype(np.float32))
    qrows = np.random.default_rng(1).choice(w.m, 256, replace=False)
    Qd = I.to_f64(inp["Q"][b, unit], w.dtype)[qrows]
    Oref = orc.plugin_attend(Qd, KS, X, vmin, vmax, w.beta)
    err = rel_max(g["O"][b, unit][qrows], Oref, np.abs(V).max())
    print(f"attend vs plug-in formula on the compressed cache: {err:.3e}")
    assert err < tol_for(w.dtype)

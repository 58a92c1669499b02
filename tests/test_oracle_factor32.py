"""Pins of the oracle's float32-factor selection (rpnys_select(factor="f32")).

Each pin is fixed by the mathematics or by the float32 format, not by the
oracle itself:
  * every stored factor entry is a float32 value, and L holds exactly those;
  * the first pivot is the float64 mode's (no factor exists before the first
    draw), and the first column is the float32 rounding of
    h(K, k_s) / sqrt(h(k_s, k_s)) (closed form);
  * the residual diagonal is diag(H) minus the squares of the STORED factor
    entries (so a downdate with the unrounded value fails at 1e-12);
  * L L^T reproduces H(S, S) to float32 accuracy;
  * on a benign case every pivot equals the float64 mode's (all decision
    margins far above the float32 perturbation);
  * CompressKV at full rank still gives exact softmax to the accuracy float32
    storage allows.
"""
import numpy as np
import pytest

from oracle import wildcat_oracle as orc


def _keys(seed, n, d, scale=0.6):
    return scale * np.random.default_rng(seed).standard_normal((n, d))


def test_factor_entries_and_pivot_block_are_float32_values():
    K = _keys(1, 300, 8)
    u = np.random.default_rng(2).random(40)
    sel = orc.rpnys_select(K, u, 40, 0.7, factor="f32")
    assert sel.r_eff == 40
    np.testing.assert_array_equal(sel.F, sel.F.astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(sel.L, np.tril(sel.F[:, sel.S].T))
    with pytest.raises(ValueError):
        orc.rpnys_select(K, u, 40, 0.7, factor="f16")


def test_first_pivot_and_first_column_closed_form():
    K = _keys(3, 200, 6)
    u = np.random.default_rng(4).random(5)
    beta, tau = 0.8, 1.3
    a = orc.rpnys_select(K, u, 5, beta, tau, factor="f32")
    b = orc.rpnys_select(K, u, 5, beta, tau, factor="f64")
    assert a.S[0] == b.S[0]
    s = a.S[0]
    col = np.exp(beta * (K @ K[s]) / tau ** 2) / np.sqrt(np.exp(beta * (K[s] @ K[s]) / tau ** 2))
    np.testing.assert_array_equal(a.F[0], col.astype(np.float32).astype(np.float64))


def test_residual_is_the_stored_factors_residual():
    K = _keys(5, 250, 5)
    beta = 0.9
    u = np.random.default_rng(6).random(30)
    sel = orc.rpnys_select(K, u, 30, beta, factor="f32")
    diag = np.exp(beta * np.einsum("ij,ij->i", K, K))
    expect = diag - (sel.F ** 2).sum(axis=0)
    expect[sel.S] = 0.0
    live = np.setdiff1d(np.arange(250), sel.S)
    np.testing.assert_allclose(sel.dres[live], expect[live], rtol=1e-12, atol=1e-12 * diag.max())
    assert np.all(sel.dres[sel.S] == 0.0)
    # the float64 value of the last column would leave a different residual
    sel64 = orc.rpnys_select(K, u, 30, beta, factor="f64")
    assert not np.allclose(sel.dres[live], sel64.dres[live], rtol=1e-12, atol=0)


def test_pivot_block_reproduces_the_pivot_gram_to_float32_accuracy():
    K = _keys(7, 400, 8)
    beta = 0.6
    u = np.random.default_rng(8).random(50)
    sel = orc.rpnys_select(K, u, 50, beta, factor="f32")
    H = np.exp(beta * (K[sel.S] @ K[sel.S].T))
    err = np.max(np.abs(sel.L @ sel.L.T - H)) / np.max(np.abs(H))
    assert 1e-10 < err < 1e-5


def test_benign_case_draws_the_float64_pivots():
    K = _keys(9, 500, 8)
    u = np.random.default_rng(10).random(60)
    a = orc.rpnys_select(K, u, 60, 0.5, factor="f32")
    b = orc.rpnys_select(K, u, 60, 0.5, factor="f64")
    # float32 storage moves the prefix sums of the residual by far less than
    # the smallest decision margin of the float64 run, so no draw can differ
    shift = np.max(np.abs(np.cumsum(a.dres) - np.cumsum(b.dres))) / b.T0
    assert shift < 1e-6 < min(b.margins)
    np.testing.assert_array_equal(a.S, b.S)


def test_full_rank_float32_factor_is_exact_softmax():
    rng = np.random.default_rng(11)
    n, d = 24, 4
    K, V, Q = 0.5 * rng.standard_normal((n, d)), rng.standard_normal((n, d)), 0.5 * rng.standard_normal((9, d))
    c = orc.compress_unit(K, V, rng.random(n), n, 0.8, factor="f32")
    assert c.sel.r_eff == n
    O = orc.plugin_attend(Q, c.K_S, c.X, c.vmin, c.vmax, 0.8)
    ref = orc.exact_attention(Q, K, V, 0.8)
    err = np.max(np.abs(O - ref)) / np.max(np.abs(V))
    assert err < 1e-3

"""Pins for the fp64 oracle against what the pages and the mathematics fix.

Each test compares the oracle with something other than itself: a closed form,
a library routine (numpy/scipy solve, pinv, eigvalsh, cholesky), brute-force
softmax, an independent implementation of the pages' own update rule, or an
invariant the pages state.  Page citations refer to the WildCat paper's method
section (arXiv 2602.10056 HTML) by paragraph.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import lambertw

from oracle import wildcat_oracle as orc


def _keys(seed, n, d, scale=1.0):
    rng = np.random.default_rng(seed)
    return scale * rng.standard_normal((n, d)) / math.sqrt(d)


def _unit(seed, n, d, m=None):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n, d)) / math.sqrt(d)
    V = rng.standard_normal((n, d))
    Q = rng.standard_normal((m or n, d)) / math.sqrt(d)
    return Q, K, V


def _gram(K, beta, tau=1.0):
    return np.exp(beta * (K @ K.T) / tau ** 2)


# ---------------------------------------------------------------- sampling
def test_first_pivot_law_matches_diagonal_on_u_grid():
    """RPNys draws pivot 0 with probability h(k_l,k_l)/sum (RPNys paragraph).

    Sweep u over a fine midpoint grid: the share of u that selects l must equal
    p_l = exp(beta |k_l|^2) / sum_j exp(beta |k_j|^2) to grid resolution.
    """
    K = _keys(1, 5, 3, scale=2.0)
    beta = 0.7
    p = np.exp(beta * (K * K).sum(1))
    p /= p.sum()
    grid = (np.arange(20000) + 0.5) / 20000
    counts = np.zeros(5)
    for u in grid:
        sel = orc.rpnys_select(K, [u], 1, beta)
        counts[sel.S[0]] += 1
    np.testing.assert_allclose(counts / grid.size, p, atol=1.5 / grid.size)


def test_first_pivot_law_statistical():
    """Chi-square check of the first-pivot law over independent seeds."""
    K = _keys(2, 6, 4, scale=2.0)
    beta = 1.0
    p = np.exp(beta * (K * K).sum(1))
    p /= p.sum()
    rng = np.random.default_rng(7)
    N = 20000
    counts = np.zeros(6)
    for u in rng.random(N):
        s, _, _ = orc.draw_pivot(np.exp(beta * (K * K).sum(1)), u)
        counts[s] += 1
    chi2 = ((counts - N * p) ** 2 / (N * p)).sum()
    assert chi2 < 25.0  # 5 dof; P(chi2 > 25) < 2e-4


def test_second_step_residual_is_schur_complement():
    """After pivot s, the residual diagonal is h_ll - h_ls^2 / h_ss (closed form).

    This is the downdate whose formula was lost (RPNys paragraph), derived
    independently as the Schur complement of h(k_s, k_s).
    """
    K = _keys(3, 9, 4, scale=1.5)
    beta = 0.9
    H = _gram(K, beta)
    sel = orc.rpnys_select(K, [0.37], 1, beta)
    s = sel.S[0]
    expect = np.diag(H) - H[:, s] ** 2 / H[s, s]
    expect[s] = 0.0
    np.testing.assert_allclose(sel.dres, expect, rtol=1e-13, atol=1e-15)


def test_draw_pivot_strict_inequality_and_zero_mass():
    d = np.array([1.0, 0.0, 1.0])
    assert orc.draw_pivot(d, 0.5)[0] == 2       # C = [1,1,2], target 1: strict '>'
    assert orc.draw_pivot(d, 0.0)[0] == 0
    assert orc.draw_pivot(np.array([0.0, 1.0, 1.0]), 0.0)[0] == 1
    assert orc.draw_pivot(np.array([1.0, 1.0, 0.0]), 1 - 2.0 ** -53)[0] == 1


def test_draw_pivot_fallback_is_last_positive_index():
    """For u < 1, u*T rounds strictly below T = C[-1], so some prefix sum
    always exceeds the target and the fallback cannot trigger; u = 1 (outside
    the contract) exercises the defined fallback: last index with mass."""
    d = np.array([0.1, 0.2, 0.3, 0.0])
    C = np.cumsum(d)
    for T in (C[-1], 1.0, 3.0, 0.7, 2.0 ** 40 + 3):
        assert (1 - 2.0 ** -53) * T < T
    assert orc.draw_pivot(d, 1 - 2.0 ** -53)[0] == 2
    assert not np.any(C > 1.0 * C[-1])
    assert orc.draw_pivot(d, 1.0)[0] == 2


def test_draw_pivot_matches_brute_force_definition():
    rng = np.random.default_rng(11)
    for _ in range(200):
        d = rng.random(7) * (rng.random(7) < 0.7)
        if d.sum() == 0:
            continue
        u = rng.random()
        T = sum(d)  # python left-to-right sum == prefix order
        acc, pick = 0.0, None
        for l, x in enumerate(d):
            acc += x
            if acc > u * T:
                pick = l
                break
        if pick is None:
            pick = max(l for l in range(7) if d[l] > 0)
        assert orc.draw_pivot(d, u)[0] == pick


# ---------------------------------------------------------------- factor
@pytest.mark.parametrize("recentre,tau", [(False, 1.0), (True, 1.0), (False, 1.7)])
def test_factor_reproduces_nystrom_and_residual_is_psd(recentre, tau):
    """F^T F = H[:,S] H_SS^{-1} H[S,:]; H - F^T F is PSD, vanishes on pivot
    rows, and its diagonal is the maintained residual (Nystroem paragraph:
    orthogonal projection onto span h(., K_S); RPNys paragraph)."""
    K = _keys(4, 64, 6, scale=2.0)
    beta = 0.8
    rng = np.random.default_rng(5)
    sel = orc.rpnys_select(K, rng.random(12), 12, beta, tau, recentre)
    assert sel.r_eff == 12
    Kc = K - K.mean(0) if recentre else K
    H = _gram(Kc, beta, tau)
    S = sel.S
    nys = H[:, S] @ np.linalg.solve(H[np.ix_(S, S)], H[S, :])
    FtF = sel.F.T @ sel.F
    np.testing.assert_allclose(FtF, nys, atol=1e-11 * np.abs(H).max())
    R = H - FtF
    ev = np.linalg.eigvalsh(R)
    assert ev.min() > -1e-11 * np.abs(H).max()
    assert np.abs(R[S, :]).max() < 1e-11 * np.abs(H).max()
    np.testing.assert_allclose(np.diag(R), sel.dres, atol=1e-11 * np.abs(H).max())
    assert len(set(S.tolist())) == len(S)


def test_pivot_block_is_cholesky_of_pivot_gram():
    """L = tril(F[S,:]) is the Cholesky factor of h(K_S, K_S) (numpy cholesky)."""
    K = _keys(6, 80, 8, scale=2.0)
    beta = 1.1
    sel = orc.rpnys_select(K, np.random.default_rng(1).random(20), 20, beta)
    H = _gram(K, beta)
    Lc = np.linalg.cholesky(H[np.ix_(sel.S, sel.S)])
    np.testing.assert_allclose(sel.L, Lc, rtol=1e-9, atol=1e-12)
    upper = np.triu(sel.F[:, sel.S].T, 1)
    assert np.abs(upper).max() < 1e-12


def test_inverse_form_recursion_agrees():
    """The pages' rank-one update of h(K_S,K_S)^{-1} (RPNys paragraph), run as
    a separate implementation, draws the same pivots and reproduces
    inv(L L^T) and the residual diagonal."""
    K = _keys(8, 50, 5, scale=2.0)
    beta = 0.9
    u = np.random.default_rng(9).random(15)
    sel = orc.rpnys_select(K, u, 15, beta)
    S2, G, d2 = orc.rpnys_select_inverse_form(K, u, 15, beta)
    assert S2.tolist() == sel.S.tolist()
    Ginv = np.linalg.inv(sel.L @ sel.L.T)
    np.testing.assert_allclose(G, Ginv, rtol=1e-7, atol=1e-9 * np.abs(Ginv).max())
    np.testing.assert_allclose(d2, sel.dres, atol=1e-10)


def test_nested_prefix_and_monotone_trace():
    """Same u prefix => the shorter run's pivots and pivot block are a prefix
    of the longer run's; the residual trace never increases."""
    K = _keys(10, 120, 8, scale=2.0)
    beta = 1.0
    u = np.random.default_rng(3).random(40)
    a = orc.rpnys_select(K, u[:10], 10, beta)
    b = orc.rpnys_select(K, u, 40, beta)
    assert b.S[:10].tolist() == a.S.tolist()
    np.testing.assert_allclose(b.L[:10, :10], a.L, rtol=0, atol=0)
    traces = [orc.rpnys_select(K, u, k, beta).dres.sum() for k in (1, 5, 10, 20, 40)]
    assert all(t2 <= t1 * (1 + 1e-12) for t1, t2 in zip(traces, traces[1:]))


def test_kernel_evaluation_count_is_linear_in_n():
    """RPNys touches n + n*r_eff entries of H (RPNys paragraph: O(nr))."""
    K = _keys(12, 100, 4)
    sel = orc.rpnys_select(K, np.random.default_rng(0).random(7), 7, 1.0)
    assert sel.kernel_evals == 100 * (1 + sel.r_eff)


# ---------------------------------------------------------------- early stop
def test_zero_keys_stop_after_one_pivot_and_give_mean():
    n, d = 10, 4
    K = np.zeros((n, d))
    V = np.random.default_rng(1).standard_normal((n, d))
    Q = np.random.default_rng(2).standard_normal((3, d))
    O, units = orc.wildcat_forward(Q[None, None], K[None, None], V[None, None],
                                   np.random.default_rng(3).random((1, 5)), 5, 1.0)
    assert units[0].sel.r_eff == 1
    np.testing.assert_allclose(O[0, 0], np.tile(V.mean(0), (3, 1)), rtol=1e-13, atol=1e-14)


def test_duplicate_keys_stop_at_distinct_count_and_are_exact():
    base = _keys(13, 3, 4, scale=2.0)
    K = base[np.array([0, 1, 2, 1, 0, 2, 2, 0])]
    rng = np.random.default_rng(4)
    V = rng.standard_normal((8, 4))
    Q = rng.standard_normal((5, 4))
    O, units = orc.wildcat_forward(Q[None, None], K[None, None], V[None, None],
                                   rng.random((1, 8)), 8, 1.0)
    assert units[0].sel.r_eff == 3
    np.testing.assert_allclose(O[0, 0], orc.exact_attention(Q, K, V, 1.0), rtol=1e-9, atol=1e-12)


def test_rank_deficient_kernel_stops_early():
    """beta -> tiny makes H numerically rank-one-ish: r_eff < r."""
    K = _keys(14, 40, 3)
    sel = orc.rpnys_select(K, np.random.default_rng(5).random(40), 40, 1e-9)
    assert 1 <= sel.r_eff < 40


def test_nonfinite_diagonal_stops_at_zero():
    K = np.full((4, 2), 30.0)  # exp(1800) overflows
    sel = orc.rpnys_select(K, [0.5, 0.5], 2, 1.0)
    assert sel.r_eff == 0


# ---------------------------------------------------------------- weights
def test_weights_match_pinv_route_and_identity_on_pivots():
    """X = pinv(H_SS) H[S,:] [V,1] (numpy pinv) and W[:,S] = I
    (Nystroem paragraph, CompressKV paragraph)."""
    K = _keys(15, 90, 6, scale=2.0)
    rng = np.random.default_rng(6)
    V = rng.standard_normal((90, 6))
    beta = 1.0
    sel = orc.rpnys_select(K, rng.random(14), 14, beta)
    X, K_S = orc.nystrom_weights(K, V, sel.S, sel.L, beta)
    H = _gram(K, beta)
    V1 = np.hstack([V, np.ones((90, 1))])
    Xp = np.linalg.pinv(H[np.ix_(sel.S, sel.S)]) @ H[sel.S, :] @ V1
    np.testing.assert_allclose(X, Xp, rtol=1e-8, atol=1e-9 * np.abs(Xp).max())
    W, _ = orc.nystrom_weights(K, np.eye(90), sel.S, sel.L, beta)
    np.testing.assert_allclose(W[:, :90][:, sel.S], np.eye(14), atol=1e-9)
    np.testing.assert_array_equal(K_S, K[sel.S])


# ---------------------------------------------------------------- outputs
@pytest.mark.parametrize("recentre,tau", [(False, 1.0), (True, 1.0), (True, 2.0), (False, 0.6)])
def test_full_rank_reproduces_exact_softmax(recentre, tau):
    """r = n projects onto the whole feature span, so O_hat is exact softmax
    (Nystroem paragraph); recentring and tau leave it unchanged (recentring
    and temperature paragraphs)."""
    Q, K, V = _unit(16, 16, 16, m=9)
    beta = 0.5
    O, units = orc.wildcat_forward(Q[None, None], K[None, None], V[None, None],
                                   np.random.default_rng(8).random((1, 16)), 16, beta, tau, recentre)
    assert units[0].sel.r_eff == 16
    np.testing.assert_allclose(O[0, 0], orc.exact_attention(Q, K, V, beta), rtol=1e-9, atol=1e-10)


def test_rank_one_gives_pivot_softmax_for_every_query():
    """|S| = 1: O_hat_i = softmax(beta k_s K^T) V for every query i."""
    Q, K, V = _unit(17, 30, 5, m=7)
    beta = 1.3
    O, units = orc.wildcat_forward(Q[None, None], K[None, None], V[None, None],
                                   np.array([[0.42]]), 1, beta)
    s = units[0].sel.S[0]
    a = np.exp(beta * (K @ K[s]))
    expect = (a @ V) / a.sum()
    np.testing.assert_allclose(O[0, 0], np.tile(expect, (7, 1)), rtol=1e-12, atol=1e-13)


def test_clip_to_value_range_and_nan_to_vmin():
    """Lem. 1 paragraph: each output entry is constrained to its column's value
    range; a NaN ratio (0/0) maps to v_min."""
    K_S = np.zeros((2, 2))
    vmin, vmax = np.array([-1.0, -1.0]), np.array([1.0, 1.0])
    Q = np.zeros((3, 2))
    X = np.array([[5.0, -7.0, 1.0], [0.0, 0.0, 0.0]])
    O = orc.plugin_attend(Q, K_S, X, vmin, vmax, 1.0)
    np.testing.assert_array_equal(O, np.tile([1.0, -1.0], (3, 1)))
    X0 = np.zeros((2, 3))
    O0 = orc.plugin_attend(Q, K_S, X0, vmin, vmax, 1.0)
    np.testing.assert_array_equal(O0, np.tile(vmin, (3, 1)))


def test_outputs_lie_in_value_range_and_range_is_columnwise():
    Q, K, V = _unit(18, 60, 4, m=20)
    O, units = orc.wildcat_forward(Q[None, None], K[None, None], V[None, None],
                                   np.random.default_rng(1).random((1, 3)), 3, 2.0)
    vmin, vmax = V.min(0), V.max(0)
    np.testing.assert_array_equal(units[0].vmin, vmin)
    np.testing.assert_array_equal(units[0].vmax, vmax)
    assert np.all(O[0, 0] >= vmin) and np.all(O[0, 0] <= vmax)


def test_normalisation_is_per_query_row():
    """Shifting every coreset key by c multiplies row i of U by
    exp(-beta <q_i, c>); the per-row normaliser must cancel it exactly."""
    Q, K, V = _unit(19, 40, 6, m=11)
    beta = 0.9
    ur = orc.compress_unit(K, V, np.random.default_rng(2).random(8), 8, beta)
    c = np.random.default_rng(3).standard_normal(6)
    O1 = orc.plugin_attend(Q, ur.K_S, ur.X, ur.vmin, ur.vmax, beta)
    O2 = orc.plugin_attend(Q, ur.K_S - c, ur.X, ur.vmin, ur.vmax, beta)
    np.testing.assert_allclose(O1, O2, rtol=1e-11, atol=1e-12)


def test_error_does_not_grow_with_nested_rank():
    """Thm. 1 / Lem. 2 paragraphs: more (nested) pivots cannot worsen the
    approximation; checked against brute-force softmax on a probe-shaped
    input with a doubling ladder."""
    rng = np.random.default_rng(21)

    def ball(rows):
        x = rng.standard_normal((rows, 16))
        return x / np.maximum(1.0, np.linalg.norm(x, axis=1, keepdims=True))
    K, V, Q = ball(256), ball(256), ball(256)
    beta = 0.25
    u = rng.random((1, 256))
    exact = orc.exact_attention(Q, K, V, beta)
    errs = []
    for r in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        O, _ = orc.wildcat_forward(Q[None, None], K[None, None], V[None, None], u[:, :r], r, beta)
        errs.append(np.abs(O[0, 0] - exact).max())
    for e1, e2 in zip(errs, errs[1:]):
        assert e2 <= 1.05 * e1 + 1e-14
    assert errs[-1] < 1e-9


def test_query_residual_decreases_with_nested_pivots():
    """h_res(q, q) = h(q,q) - h(q,K_S) H_SS^{-1} h(K_S,q) is non-increasing in
    the nested coreset for every query (projection onto a growing subspace)."""
    Q, K, _ = _unit(22, 80, 5, m=15)
    beta = 1.0
    u = np.random.default_rng(4).random(30)
    prev = None
    for r in (2, 6, 12, 30):
        sel = orc.rpnys_select(K, u[:r], r, beta)
        hq = np.exp(beta * (Q @ K[sel.S].T))
        Z = np.linalg.solve(sel.L, hq.T)
        res = np.exp(beta * (Q * Q).sum(1)) - (Z * Z).sum(0)
        assert res.min() > -1e-9
        if prev is not None:
            assert np.all(res <= prev + 1e-9)
        prev = res


def test_gqa_mapping_uses_contiguous_groups():
    rng = np.random.default_rng(23)
    B, Hq, Hkv, n, m, d = 1, 4, 2, 20, 3, 4
    Q = rng.standard_normal((B, Hq, m, d))
    K = rng.standard_normal((B, Hkv, n, d)) / 2
    V = rng.standard_normal((B, Hkv, n, d))
    u = rng.random((2, 5))
    O, units = orc.wildcat_forward(Q, K, V, u, 5, 0.7)
    for h in range(Hq):
        ur = units[h // 2]
        np.testing.assert_array_equal(O[0, h], orc.plugin_attend(Q[0, h], ur.K_S, ur.X, ur.vmin, ur.vmax, 0.7))
    Ou, _ = orc.wildcat_forward(Q[:, 2:4], K[:, 1:2], V[:, 1:2], u[1:2], 5, 0.7)
    np.testing.assert_array_equal(O[:, 2:4], Ou)


# ---------------------------------------------------------------- golden
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _closed(expr):
    return float(eval(expr, {"__builtins__": {}}, {"e": math.e, "sqrt": math.sqrt, "exp": math.exp}))


def test_two_key_worked_example():
    with open(os.path.join(GOLDEN, "two_key_worked.json")) as f:
        g = json.load(f)
    K, V, Q = (np.array(g[k], dtype=np.float64) for k in ("K", "V", "Q"))
    for case in g["cases"]:
        u = np.array([case["u"]])
        O, units = orc.wildcat_forward(Q[None, None], K[None, None], V[None, None], u, case["r"], g["beta"])
        assert units[0].sel.S.tolist() == case["S"]
        L = np.array([[_closed(x) for x in row] for row in case["L"]])
        np.testing.assert_allclose(units[0].sel.L, L, rtol=1e-14, atol=1e-15)
        Oexp = np.array([[_closed(x) for x in row] for row in case["O"]])
        np.testing.assert_allclose(O[0, 0], Oexp, rtol=1e-13, atol=1e-14)


def test_rho0_constant_printed_on_the_page():
    with open(os.path.join(GOLDEN, "rho0_constant.json")) as f:
        g = json.load(f)
    w0 = lambertw(2 / math.e ** 2, 0).real
    rho0 = math.sqrt(1 + math.exp(w0 + 2))
    assert round(rho0, g["decimals"]) == g["value"]

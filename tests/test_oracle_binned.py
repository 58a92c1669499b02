"""Pins of the oracle's binned CompressKV (RPNys divide-and-conquer remark).

Each pin is fixed by the mathematics or by a library routine, not by the
oracle itself: bins = 1 is the unbinned path; each bin's first pivot follows
the closed-form law restricted to the bin; the weights equal the
block-diagonal W computed with numpy's pinv; full rank per bin reproduces
exact softmax; the kernel-evaluation count drops by the factor B the pages
state; bins are independent of each other's data.
"""
import numpy as np
import pytest

from oracle import wildcat_oracle as orc


def _kqv(seed, n, d, m=7, scale=1.0):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((n, d)), rng.standard_normal((n, d)),
            scale * rng.standard_normal((m, d)))


def test_one_bin_is_the_unbinned_path():
    K, V, Q = _kqv(1, 60, 4, scale=0.5)
    u = np.random.default_rng(2).random(12)
    a = orc.compress_unit(K, V, u, 12, 0.8)
    b = orc.compress_unit_binned(K, V, u, 12, 1, 0.8)
    np.testing.assert_array_equal(b.bins[0].sel.S, a.sel.S)
    np.testing.assert_array_equal(b.X, a.X)
    np.testing.assert_array_equal(b.K_S, a.K_S)


def test_bins_only_see_their_own_keys_and_uniforms():
    """Pivots of bin b are local indices into its block; changing the data
    or uniforms of another bin changes nothing in bin b (block-diagonal W)."""
    K, V, _ = _kqv(3, 90, 5, scale=0.6)
    u = np.random.default_rng(4).random(15)
    a = orc.compress_unit_binned(K, V, u, 15, 3, 0.5)
    for p in a.bins:
        assert np.all((p.sel.S >= 0) & (p.sel.S < 30)) and p.sel.r_eff == 5
    K2, V2, u2 = K.copy(), V.copy(), u.copy()
    K2[30:60] = np.random.default_rng(5).standard_normal((30, 5))
    V2[30:60] += 1.0
    u2[5:10] = np.random.default_rng(6).random(5)
    b = orc.compress_unit_binned(K2, V2, u2, 15, 3, 0.5)
    for k in (0, 2):
        np.testing.assert_array_equal(a.bins[k].sel.S, b.bins[k].sel.S)
        np.testing.assert_array_equal(a.bins[k].X, b.bins[k].X)
    assert not np.array_equal(a.bins[1].X, b.bins[1].X)


def test_first_pivot_law_within_each_bin():
    """Bin b's first pivot has probability exp(beta |k_l|^2) / sum over the
    bin only (the RPNys law on the bin), swept on a u grid."""
    rng = np.random.default_rng(7)
    K = 1.5 * rng.standard_normal((8, 3))
    V = rng.standard_normal((8, 3))
    beta = 0.6
    for b in range(2):
        blk = K[4 * b:4 * b + 4]
        p = np.exp(beta * (blk * blk).sum(1))
        p /= p.sum()
        grid = (np.arange(4000) + 0.5) / 4000
        counts = np.zeros(4)
        for g in grid:
            u = np.full(2, 0.5)
            u[b] = g
            counts[orc.compress_unit_binned(K, V, u, 2, 2, beta).bins[b].sel.S[0]] += 1
        np.testing.assert_allclose(counts / grid.size, p, atol=1.5 / grid.size)


def test_weights_equal_block_diagonal_pinv():
    """X = blockdiag_b(pinv(H_{S_b S_b}) H_{S_b, K_b}) [V, 1], with numpy's
    pinv (an independent route to the two triangular solves)."""
    K, V, _ = _kqv(8, 80, 4, scale=0.5)
    beta, tau = 0.9, 1.3
    u = np.random.default_rng(9).random(16)
    res = orc.compress_unit_binned(K, V, u, 16, 4, beta, tau)
    rows = []
    for b, p in enumerate(res.bins):
        Kb, Vb = K[20 * b:20 * b + 20], V[20 * b:20 * b + 20]
        S = p.sel.S[:p.sel.r_eff]
        H = np.exp(beta * (Kb @ Kb.T) / tau ** 2)
        W = np.linalg.pinv(H[np.ix_(S, S)]) @ H[S]
        rows.append(W @ np.hstack([Vb, np.ones((20, 1))]))
    np.testing.assert_allclose(res.X, np.vstack(rows), rtol=1e-8, atol=1e-10)


@pytest.mark.parametrize("bins", [2, 4])
def test_full_rank_bins_reproduce_exact_softmax(bins):
    """r = n: every bin keeps all its keys, W_b = I, and the plug-in output
    is exact softmax attention over all n keys (normalised over all bins)."""
    K, V, Q = _kqv(10, 32, 6, scale=0.35)
    u = np.random.default_rng(11).random(32)
    res = orc.compress_unit_binned(K, V, u, 32, bins, 0.5)
    assert all(p.sel.r_eff == 32 // bins for p in res.bins)
    O = orc.plugin_attend(Q, res.K_S, res.X, res.vmin, res.vmax, 0.5)
    np.testing.assert_allclose(O, orc.exact_attention(Q, K, V, 0.5), rtol=1e-9, atol=1e-10)


def test_kernel_evaluations_drop_by_the_bin_factor():
    """Each bin touches n/B + (n/B) r_eff_b kernel entries: n (1 + r/B) in
    all against n (1 + r) unbinned -- the O(nr/B)-entry form of the pages'
    O(nr^2/B^2) count."""
    K, V, _ = _kqv(12, 120, 4, scale=0.4)
    u = np.random.default_rng(13).random(24)
    res = orc.compress_unit_binned(K, V, u, 24, 4, 1.0)
    assert sum(p.sel.kernel_evals for p in res.bins) == 120 * (1 + 24 // 4)


def test_value_range_is_over_the_whole_unit_and_bounds_output():
    K, V, Q = _kqv(14, 40, 3, m=25)
    V[3] += 5.0
    V[37] -= 5.0
    u = np.random.default_rng(15).random(8)
    res = orc.compress_unit_binned(K, V, u, 8, 2, 0.7)
    np.testing.assert_array_equal(res.vmin, V.min(0))
    np.testing.assert_array_equal(res.vmax, V.max(0))
    O = orc.plugin_attend(Q, res.K_S, res.X, res.vmin, res.vmax, 0.7)
    assert np.all(O >= V.min(0)) and np.all(O <= V.max(0))


def test_rejects_sizes_not_divisible_by_bins():
    K, V, _ = _kqv(16, 30, 3)
    with pytest.raises(ValueError):
        orc.compress_unit_binned(K, V, np.zeros(6), 6, 4, 1.0)
    with pytest.raises(ValueError):
        orc.compress_unit_binned(K, V, np.zeros(5), 5, 3, 1.0)

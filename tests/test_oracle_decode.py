"""Pins of the oracle's generation step over a compressed cache (decode_attend).

Each pin is fixed by the mathematics or by a library routine, not by the
oracle itself:
  * a cache that keeps the whole prefix (identity weights) makes the step
    exact causal softmax attention, computed here with scipy's softmax;
  * CompressKV at full rank gives the same, up to the solve's rounding;
  * with an empty prefix the step is causal softmax over the new tokens, and
    the first query returns v_0 exactly (its clip range is the single point);
  * causality: rows after i of K_new / V_new do not change output row i;
  * the clip takes the running range (closed-form cases with all kernel
    values equal to 1);
  * one new token is WtdAttn with that token appended as a weight-1 point;
  * query head h reads kv head h // group;
  * decode_row (one row, for sampling long generations) equals the
    corresponding row of decode_attend.
"""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import wildcat_oracle as orc


def _tokens(seed, n0, m, d, scale=0.5):
    rng = np.random.default_rng(seed)
    Kp, Vp = scale * rng.standard_normal((n0, d)), rng.standard_normal((n0, d))
    Kn, Vn = scale * rng.standard_normal((m, d)), rng.standard_normal((m, d))
    Q = scale * rng.standard_normal((m, d))
    return Kp, Vp, Kn, Vn, Q


def _causal_softmax(Q, Kp, Vp, Kn, Vn, beta):
    """Row i: softmax attention of q_i over the prefix and new tokens 0..i."""
    out = np.empty((Q.shape[0], Vn.shape[1]))
    for i in range(Q.shape[0]):
        K = np.vstack([Kp, Kn[:i + 1]])
        V = np.vstack([Vp, Vn[:i + 1]])
        out[i] = softmax(beta * (K @ Q[i])) @ V
    return out


def test_whole_prefix_cache_gives_exact_causal_attention():
    Kp, Vp, Kn, Vn, Q = _tokens(1, 23, 9, 6)
    beta = 0.7
    X = np.hstack([Vp, np.ones((23, 1))])
    O = orc.decode_attend(Q, Kp, X, Vp.min(0), Vp.max(0), Kn, Vn, beta)
    np.testing.assert_allclose(O, _causal_softmax(Q, Kp, Vp, Kn, Vn, beta), rtol=1e-12, atol=1e-13)


def test_full_rank_compressed_prefix_is_exact():
    Kp, Vp, Kn, Vn, Q = _tokens(2, 20, 7, 5, scale=0.8)
    beta = 0.9
    u = np.random.default_rng(3).random(20)
    c = orc.compress_unit(Kp, Vp, u, 20, beta)
    assert c.sel.r_eff == 20
    O = orc.decode_attend(Q, c.K_S, c.X, c.vmin, c.vmax, Kn, Vn, beta)
    ref = _causal_softmax(Q, Kp, Vp, Kn, Vn, beta)
    assert np.max(np.abs(O - ref)) < 1e-7 * np.max(np.abs(Vp))


def test_empty_prefix_is_causal_softmax_over_new_tokens():
    _, _, Kn, Vn, Q = _tokens(4, 1, 11, 4)
    d = 4
    inf = np.full(d, np.inf)
    O = orc.decode_attend(Q, np.zeros((0, d)), np.zeros((0, d + 1)), inf, -inf, Kn, Vn, 1.3)
    ref = _causal_softmax(Q, np.zeros((0, d)), np.zeros((0, d)), Kn, Vn, 1.3)
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(O[0], Vn[0])


def test_later_tokens_do_not_reach_earlier_queries():
    Kp, Vp, Kn, Vn, Q = _tokens(5, 15, 8, 5)
    X = np.hstack([Vp, np.ones((15, 1))])
    args = (Q, Kp, X, Vp.min(0), Vp.max(0))
    base = orc.decode_attend(*args, Kn, Vn, 0.6)
    for i in range(8):
        K2, V2 = Kn.copy(), Vn.copy()
        rng = np.random.default_rng(10 + i)
        K2[i + 1:] = rng.standard_normal(K2[i + 1:].shape)
        V2[i + 1:] = 5.0 + rng.standard_normal(V2[i + 1:].shape)
        O = orc.decode_attend(*args, K2, V2, 0.6)
        np.testing.assert_array_equal(O[:i + 1], base[:i + 1])
        if i + 1 < 8:
            assert not np.array_equal(O[i + 1:], base[i + 1:])


@pytest.mark.parametrize("x0, expect", [
    # N_i = x0 + sum_{j<=i} v_j over (i + 2); range [min(0, v_0..v_i), max(1, v_0..v_i)]
    (2.0, [1.0, 5.5 / 3.0, 1.5 / 4.0]),       # row 0: 1.25 clipped to hi = 1 (v_1 = 3 not yet seen)
    (-6.0, [0.0, 0.0, -6.5 / 4.0]),           # rows 0, 1: -2.75, -2.5/3 clipped to lo = 0 (v_2 = -4 not yet seen)
])
def test_clip_takes_the_running_range(x0, expect):
    d = 1
    Q, K = np.zeros((3, d)), np.zeros((3, d))            # every kernel value is exp(0) = 1
    Vn = np.array([[0.5], [3.0], [-4.0]])
    O = orc.decode_attend(Q, np.zeros((1, d)), np.array([[x0, 1.0]]), np.array([0.0]), np.array([1.0]), K, Vn, 1.0)
    np.testing.assert_allclose(O[:, 0], expect, rtol=1e-15)


def test_one_new_token_is_wtdattn_with_it_appended():
    Kp, Vp, Kn, Vn, Q = _tokens(6, 12, 1, 3)
    rng = np.random.default_rng(7)
    K_S, X = Kp[:5], np.hstack([rng.standard_normal((5, 3)), rng.random((5, 1))])
    vmin, vmax = Vp.min(0), Vp.max(0)
    O = orc.decode_attend(Q, K_S, X, vmin, vmax, Kn, Vn, 0.8)
    ref = orc.plugin_attend(Q, np.vstack([K_S, Kn]), np.vstack([X, np.hstack([Vn, [[1.0]]])]),
                            np.fmin(vmin, Vn[0]), np.fmax(vmax, Vn[0]), 0.8)
    np.testing.assert_allclose(O, ref, rtol=1e-14, atol=1e-15)


def test_query_heads_read_their_group():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, m, r, d = 2, 4, 2, 5, 6, 3
    Q = rng.standard_normal((B, Hq, m, d))
    K_S = rng.standard_normal((B, Hkv, r, d))
    X = rng.standard_normal((B, Hkv, r, d + 1))
    X[..., d] = rng.random((B, Hkv, r)) + 0.5
    vmin, vmax = -rng.random((B, Hkv, d)), rng.random((B, Hkv, d))
    Kn, Vn = rng.standard_normal((B, Hkv, m, d)), rng.standard_normal((B, Hkv, m, d))
    O = orc.wildcat_decode(Q, K_S, X, vmin, vmax, Kn, Vn, 0.5)
    for b in range(B):
        for h in range(Hq):
            g = h // 2
            np.testing.assert_array_equal(
                O[b, h], orc.decode_attend(Q[b, h], K_S[b, g], X[b, g], vmin[b, g], vmax[b, g], Kn[b, g], Vn[b, g], 0.5))


def test_decode_row_matches_decode_attend():
    Kp, Vp, Kn, Vn, Q = _tokens(12, 30, 17, 6)
    rng = np.random.default_rng(13)
    K_S, X = Kp[:9], np.hstack([rng.standard_normal((9, 6)), 0.5 + rng.random((9, 1))])
    vmin, vmax = Vp.min(0), Vp.max(0)
    O = orc.decode_attend(Q, K_S, X, vmin, vmax, Kn, Vn, 0.7)
    for i in (0, 5, 16):
        np.testing.assert_allclose(orc.decode_row(Q[i], i, K_S, X, vmin, vmax, Kn, Vn, 0.7), O[i],
                                   rtol=1e-13, atol=1e-14)

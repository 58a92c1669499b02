"""fp64 CPU oracle for WildCat weighted-coreset attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the bench's CPU
baseline leg use it.  It shares no code with the HIP library (no kernels,
headers, helpers or constants); both sides receive the same seeded inputs from
the input-generator module, which holds none of the method's arithmetic.

Source: the pages on "WildCat: Near-Linear Attention in Theory and Practice"
(Schroeder & Mackey; arXiv 2602.10056 HTML, and the ICML 2026 poster page).
Citations below name the paragraph of that paper's method section by the
object it introduces (plug-in estimator, Lem. 1, Nystroem approximation,
RPNys / Alg. 1, recentring, temperature eq. (12), CompressKV / Alg. 2,
WtdAttn / Alg. 3, WildCat / Alg. 4).  The HTML lost every display equation and
algorithm box; where a step is missing the reading taken is stated at the
function and listed with the others in the design notes.

Every function works on one (batch, kv-head) unit in float64 with plain numpy
(and scipy's triangular solve), one definition step after another, with no
blocking or fusion.

Pins: every function here is pinned by the CPU tests (closed forms, library
routines, invariants, brute force on tiny inputs); none is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
from scipy.linalg import solve_triangular

STOP_REL = 1e-12  # residual-trace stop threshold, relative to the initial trace


# --------------------------------------------------------------------------
# Kernels
# --------------------------------------------------------------------------
def query_kernel(Q, K, beta):
    """h(q, k) = exp(beta <q, k>) for all pairs.

    [WildCat, Nystroem paragraph: the attention matrix is the exponential
    kernel h evaluated between queries and keys.]
    """
    return np.exp(beta * (np.asarray(Q) @ np.asarray(K).T))


def selection_kernel(X, Y, beta, tau=1.0):
    """h_tau(x, y) = exp(beta <x, y> / tau^2), the kernel RPNys runs on.

    [WildCat, CompressKV / Alg. 2 paragraph: after the temperature choice the
    keys feed RPNys with h_tau; tau = 1 gives h itself.]
    """
    return np.exp(beta * (np.asarray(X) @ np.asarray(Y).T) / tau ** 2)


def prepare_keys(K, recentre):
    """Keys as RPNys and the Nystroem weights see them.

    [WildCat, recentring paragraph: softmax attention does not change when the
    same vector is subtracted from every key; the method subtracts the key
    mean.]  Optional here (default off).
    """
    K = np.asarray(K, dtype=np.float64)
    if recentre:
        return K - K.mean(axis=0)
    return K


# --------------------------------------------------------------------------
# RPNys (randomly pivoted Cholesky with Nystroem weights)
# --------------------------------------------------------------------------
def draw_pivot(dres, u):
    """One pivot draw from the residual diagonal.

    [WildCat, RPNys / Alg. 1 paragraph: each round samples the pivot from the
    diagonal of the current residual kernel.]  The sampling formula itself was
    lost; the reading is p_l = dres_l / sum(dres), realised by the inverse CDF
    in index order: with C the inclusive prefix sums and T = C[-1], the pivot
    is the first l with C_l > u*T (strict, so zero-mass indices are never
    drawn).  If rounding leaves no such l, the last index with positive
    residual is taken.

    Returns (s, T, gap) with gap = min_l |C_l - u T| (a diagnostic: how far
    the draw is from flipping to a neighbouring index).
    """
    C = np.cumsum(dres)
    T = C[-1]
    target = u * T
    hits = np.flatnonzero(C > target)
    if hits.size:
        s = int(hits[0])
    else:
        s = int(np.flatnonzero(dres > 0)[-1])
    gap = float(np.min(np.abs(C - target)))
    return s, T, gap


@dataclass
class SelectResult:
    S: np.ndarray            # pivot indices in draw order, length r_eff
    r_eff: int
    L: np.ndarray            # r_eff x r_eff lower-triangular pivot block
    F: np.ndarray            # r_eff x n partial Cholesky factor (row i = column i of the factor)
    dres: np.ndarray         # residual diagonal after the last step
    T0: float
    margins: list = field(default_factory=list)   # per draw: gap / T0 (see draw_pivot)
    kernel_evals: int = 0    # number of h_tau entries evaluated


def rpnys_select(K, u, r, beta, tau=1.0, recentre=False, factor="f64"):
    """Randomly pivoted partial Cholesky of H = h_tau(K, K).

    [WildCat, RPNys / Alg. 1 paragraph; Nystroem paragraph.]
    The residual diagonal starts at h_tau(k_l, k_l).  Each round draws a pivot
    s (draw_pivot), evaluates the kernel column h_tau(K, k_s), subtracts the
    part already explained by the factor, normalises by the square root of the
    residual at the pivot, and downdates the residual diagonal by the square of
    the new factor column.  The pages state the same step as a rank-one update
    of h(K_S, K_S)^{-1} (see rpnys_select_inverse_form); the two agree in exact
    arithmetic.

    The run stops early (r_eff < r) when the residual trace is no longer above
    STOP_REL times its initial value (or is not finite), or when the residual
    at the drawn pivot is not positive -- the pages only say the residual at
    the pivot stays positive until H is fully approximated.

    Only n + n*r_eff kernel entries are evaluated (the pages: O(nr) entries).

    factor="f32" is the faster selection the pages leave to future work, in
    the reading taken here: the factor is stored in float32 (each new column
    is computed in float64 and rounded once), and everything else stays
    float64 -- the kernel column, the products with the stored factor (exact
    in float64), the sums, the draw.  The residual diagonal is downdated by
    the square of the stored value, and L is taken from the stored values, so
    the diagonal stays the residual of the stored factor.
    """
    if factor not in ("f64", "f32"):
        raise ValueError("factor must be 'f64' or 'f32'")
    Kc = prepare_keys(K, recentre)
    n = Kc.shape[0]
    u = np.asarray(u, dtype=np.float64)
    dres = np.exp(beta * np.einsum("ij,ij->i", Kc, Kc) / tau ** 2)
    evals = n
    T0 = np.cumsum(dres)[-1]
    F = np.zeros((r, n))
    S = []
    margins = []
    for i in range(r):
        T = np.cumsum(dres)[-1]
        if not (T > STOP_REL * T0):
            break
        s, T, gap = draw_pivot(dres, u[i])
        g = selection_kernel(Kc, Kc[s:s + 1], beta, tau)[:, 0] - F[:i].T @ F[:i, s]
        evals += n
        if not (g[s] > 0):
            break
        F[i] = g / np.sqrt(g[s])
        if factor == "f32":
            F[i] = F[i].astype(np.float32).astype(np.float64)
        dres = np.maximum(dres - F[i] ** 2, 0.0)
        dres[s] = 0.0
        S.append(s)
        margins.append(gap / T0)
    r_eff = len(S)
    S = np.asarray(S, dtype=np.int64)
    L = np.tril(F[:r_eff][:, S].T)
    return SelectResult(S=S, r_eff=r_eff, L=L, F=F[:r_eff].copy(), dres=dres,
                        T0=float(T0), margins=margins, kernel_evals=evals)


def rpnys_select_inverse_form(K, u, r, beta, tau=1.0, recentre=False):
    """The same selection, run through the pages' own update rule.

    [WildCat, RPNys / Alg. 1 paragraph.]  Keeps G = h(K_S, K_S)^{-1} and the
    residual diagonal directly: for a new pivot s with residual rho_s,
    g = (h(k_s, K_S) G, -1) / sqrt(rho_s) (the vector the pages give),
    G <- [[G, 0], [0, 0]] + g g^T, and every residual diagonal entry drops by
    (h(k_l, K_S') . g)^2.  The two update formulas were lost in extraction;
    these are the Schur-complement forms that the printed g implies.

    Used only to cross-check rpnys_select.  Returns (S, G, dres).
    """
    Kc = prepare_keys(K, recentre)
    n = Kc.shape[0]
    dres = np.exp(beta * np.einsum("ij,ij->i", Kc, Kc) / tau ** 2)
    T0 = np.cumsum(dres)[-1]
    G = np.zeros((0, 0))
    S = []
    for i in range(r):
        T = np.cumsum(dres)[-1]
        if not (T > STOP_REL * T0):
            break
        s, _, _ = draw_pivot(dres, u[i])
        rho = dres[s]
        if not (rho > 0):
            break
        h_s_S = selection_kernel(Kc[s:s + 1], Kc[S], beta, tau)[0] if S else np.zeros(0)
        gvec = np.concatenate([h_s_S @ G, [-1.0]]) / np.sqrt(rho)
        S.append(s)
        Gn = np.zeros((i + 1, i + 1))
        Gn[:i, :i] = G
        G = Gn + np.outer(gvec, gvec)
        H_lS = selection_kernel(Kc, Kc[S], beta, tau)
        dres = dres - (H_lS @ gvec) ** 2
        dres = np.maximum(dres, 0.0)
        dres[s] = 0.0
    return np.asarray(S, dtype=np.int64), G, dres


# --------------------------------------------------------------------------
# CompressKV: Nystroem weights through the pivot block
# --------------------------------------------------------------------------
def value_range(V):
    """Column-wise value range [v_min j, v_max j] over all n rows.

    [WildCat, Lem. 1 paragraph: every exact output entry O_ij lies in the range
    of column j of V, and the estimate is constrained to it too.]
    """
    V = np.asarray(V, dtype=np.float64)
    return V.min(axis=0), V.max(axis=0)


def nystrom_weights(K, V, S, L, beta, tau=1.0, recentre=False):
    """X = W [V, 1_n] with W = h_tau(K_S, K_S)^{-1} h_tau(K_S, K).

    [WildCat, Nystroem paragraph (optimal weights w_l with a pseudo-inverse);
    CompressKV / Alg. 2 paragraph (V_S = W V, w = W 1_n, inverse).]
    h_tau(K_S, K_S) = L L^T for the pivot block L of the Cholesky factor, so
    W [V, 1] = L^{-T} (L^{-1} (h_tau(K_S, K) [V, 1])): first the contraction,
    then two triangular solves.  W is applied to (V, 1_n) before any query
    touches it (plug-in estimator paragraph).

    Returns (X, K_S) with X of shape r_eff x (d+1): V_S = X[:, :d], w = X[:, d];
    K_S are the raw (not recentred) pivot keys.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Kc = prepare_keys(K, recentre)
    S = np.asarray(S, dtype=np.int64)
    n = K.shape[0]
    if len(S) == 0:
        return np.zeros((0, V.shape[1] + 1)), K[S]
    V1 = np.hstack([V, np.ones((n, 1))])
    Y = selection_kernel(Kc[S], Kc, beta, tau) @ V1
    Z = solve_triangular(L, Y, lower=True)
    X = solve_triangular(L.T, Z, lower=False)
    return X, K[S]


# --------------------------------------------------------------------------
# WtdAttn: the plug-in estimate with the value-range clip
# --------------------------------------------------------------------------
def plugin_attend(Q, K_S, X, vmin, vmax, beta):
    """O_hat = clip(diag(U w)^{-1} U V_S) with U = h(Q, K_S).

    [WildCat, plug-in estimator paragraph; Lem. 1 paragraph (clip to the
    column value range); CompressKV / Alg. 2 paragraph (D_hat_i is the
    w-weighted sum of h(q_i, k_l) over the coreset); WtdAttn / Alg. 3.]
    The division is plain IEEE division; the clip is fmin(fmax(x, lo), hi), so
    a NaN ratio lands on v_min (the pages do not treat a non-positive D_hat).
    """
    Q = np.asarray(Q, dtype=np.float64)
    d = Q.shape[1]
    U = query_kernel(Q, K_S, beta)
    N = U @ X
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = N[:, :d] / N[:, d:d + 1]
    return np.fmin(np.fmax(ratio, vmin[None, :]), vmax[None, :])


def exact_attention(Q, K, V, beta):
    """Exact softmax attention D^{-1} A V with A = exp(beta Q K^T).

    [WildCat, plug-in estimator paragraph (the target O); abstract (quadratic
    cost).]  The per-row maximum is subtracted before exp, which leaves the
    ratio unchanged.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Sc = beta * (Q @ K.T)
    A = np.exp(Sc - Sc.max(axis=1, keepdims=True))
    return (A @ V) / A.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# Generation over a compressed cache
# --------------------------------------------------------------------------
def decode_attend(Q, K_S, X, vmin, vmax, K_new, V_new, beta):
    """Generation over a compressed cache: m new tokens, causal among themselves.

    [WildCat, KV-cache paragraph: after CompressKV the compressed keys and
    values enter later attention computations (the decoding phase) through
    WtdAttn, and m new tokens cost O(rmd + m^2 d) instead of the full prefix;
    WtdAttn / Alg. 3; Lem. 1 paragraph (clip to the value range).]
    Readings (the pages give no formula for this step):
      * new token j joins the weighted attention as one more coreset point
        with weight 1 and value v_j (its row of W is a unit vector: it is kept
        exactly), so N_i = h(q_i, K_S) X + sum_{j <= i} h(q_i, k_j) [v_j, 1];
      * causal: query i (the query of new token i) sees the whole compressed
        prefix and the new tokens 0 .. i;
      * the clip range of query i is the prefix range widened by v_0 .. v_i
        (the values of every key it sees), taken with fmin / fmax so that a
        NaN value leaves the range as it was.
    Q, K_new, V_new: m x d (row i is new token i); K_S: r x d raw coreset keys
    (r may be 0); X: r x (d+1); vmin, vmax: the prefix's column range.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K_new = np.asarray(K_new, dtype=np.float64)
    V_new = np.asarray(V_new, dtype=np.float64)
    m, d = Q.shape
    N = query_kernel(Q, np.asarray(K_S, dtype=np.float64).reshape(-1, d), beta) @ np.asarray(X, dtype=np.float64).reshape(-1, d + 1)
    A = np.tril(query_kernel(Q, K_new, beta))
    N = N + A @ np.hstack([V_new, np.ones((m, 1))])
    lo = np.fmin(np.asarray(vmin, dtype=np.float64)[None, :], np.fmin.accumulate(V_new, axis=0))
    hi = np.fmax(np.asarray(vmax, dtype=np.float64)[None, :], np.fmax.accumulate(V_new, axis=0))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = N[:, :d] / N[:, d:d + 1]
    return np.fmin(np.fmax(ratio, lo), hi)


def decode_row(q, i, K_S, X, vmin, vmax, K_new, V_new, beta):
    """Row i of decode_attend alone (query q of new token i), for sampling
    outputs of long generations: the same definition restricted to one row,
    touching only the cache and the new tokens 0 .. i."""
    q = np.asarray(q, dtype=np.float64)[None, :]
    d = q.shape[1]
    Kn = np.asarray(K_new, dtype=np.float64)[:i + 1]
    Vn = np.asarray(V_new, dtype=np.float64)[:i + 1]
    N = query_kernel(q, np.asarray(K_S, dtype=np.float64).reshape(-1, d), beta) @ \
        np.asarray(X, dtype=np.float64).reshape(-1, d + 1)
    N = N + query_kernel(q, Kn, beta) @ np.hstack([Vn, np.ones((i + 1, 1))])
    lo = np.fmin(np.asarray(vmin, dtype=np.float64), np.fmin.reduce(Vn, axis=0))
    hi = np.fmax(np.asarray(vmax, dtype=np.float64), np.fmax.reduce(Vn, axis=0))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = N[0, :d] / N[0, d]
    return np.fmin(np.fmax(ratio, lo), hi)


def wildcat_decode(Q, K_S, X, vmin, vmax, K_new, V_new, beta):
    """decode_attend over all heads: Q [B][Hq][m][d]; K_S [B][Hkv][r][d];
    X [B][Hkv][r][d+1]; vmin, vmax [B][Hkv][d]; K_new, V_new [B][Hkv][m][d].

    Query head h reads kv head h // (Hq / Hkv), as in wildcat_forward.
    Returns O [B][Hq][m][d].
    """
    Q = np.asarray(Q, dtype=np.float64)
    B, Hq, m, d = Q.shape
    Hkv = K_new.shape[1]
    group = Hq // Hkv
    O = np.empty((B, Hq, m, d))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            O[b, h] = decode_attend(Q[b, h], K_S[b, g], X[b, g], vmin[b, g], vmax[b, g], K_new[b, g], V_new[b, g],
                                    beta)
    return O


# --------------------------------------------------------------------------
# The whole path for one unit and for a batch of units
# --------------------------------------------------------------------------
@dataclass
class UnitResult:
    sel: SelectResult
    X: np.ndarray           # r_eff x (d+1)
    K_S: np.ndarray         # r_eff x d (raw keys)
    vmin: np.ndarray
    vmax: np.ndarray


def compress_unit(K, V, u, r, beta, tau=1.0, recentre=False, factor="f64"):
    """CompressKV for one (batch, kv-head): RPNys, then Nystroem weights.

    [WildCat, CompressKV / Alg. 2 paragraph.]  factor: see rpnys_select.
    """
    sel = rpnys_select(K, u, r, beta, tau, recentre, factor)
    X, K_S = nystrom_weights(K, V, sel.S, sel.L, beta, tau, recentre)
    vmin, vmax = value_range(V)
    return UnitResult(sel=sel, X=X, K_S=K_S, vmin=vmin, vmax=vmax)


@dataclass
class BinnedUnitResult:
    bins: list              # UnitResult of every bin, in bin order (pivots local to the bin)
    X: np.ndarray           # sum_b r_eff_b x (d+1): the bins' weights, concatenated
    K_S: np.ndarray         # the bins' pivot keys (raw), concatenated
    vmin: np.ndarray        # value range over all n rows of the unit
    vmax: np.ndarray


def compress_unit_binned(K, V, u, r, bins, beta, tau=1.0, recentre=False, factor="f64"):
    """Binned CompressKV for one unit.

    [WildCat, RPNys / Alg. 1 paragraph: the divide-and-conquer strategy that
    splits the input into B bins, finds a coreset of size r/B in each bin in
    parallel, and brings the operation count to O(nr^2/B^2 + nrd/B).]
    Readings (the pages give no partition rule and no weight formula for the
    binned case):
      * the bins are B contiguous blocks of n/B keys in index order;
      * bin b runs RPNys on its own keys with r/B pivots and the uniforms
        u[b r/B : (b+1) r/B];
      * bin b's Nystroem weights come from its own keys and values, W_b =
        h_tau(K_Sb, K_Sb)^{-1} h_tau(K_Sb, K_b), i.e. W is block-diagonal --
        the reading the stated O(nrd/B) weight cost implies (weights against
        all n keys would cost nrd);
      * the coreset is the bins' coresets concatenated in bin order, and the
        plug-in estimator normalises over all of it (WtdAttn unchanged);
      * the value range stays over all n rows of the unit (Lem. 1);
      * with recentring each bin subtracts its own key mean (each bin is an
        independent RPNys problem).
    bins = 1 is compress_unit.
    """
    n = K.shape[0]
    if bins < 1 or n % bins or r % bins:
        raise ValueError("n and r must be multiples of the number of bins")
    nb, rb = n // bins, r // bins
    parts = [compress_unit(K[b * nb:(b + 1) * nb], V[b * nb:(b + 1) * nb], u[b * rb:(b + 1) * rb], rb,
                           beta, tau, recentre, factor) for b in range(bins)]
    X = np.concatenate([p.X for p in parts], axis=0)
    K_S = np.concatenate([p.K_S for p in parts], axis=0)
    vmin, vmax = value_range(V)
    return BinnedUnitResult(bins=parts, X=X, K_S=K_S, vmin=vmin, vmax=vmax)


def wildcat_forward(Q, K, V, u, r, beta, tau=1.0, recentre=False, factor="f64"):
    """WildCat over all units: Q [B][Hq][m][d], K, V [B][Hkv][n][d], u [B*Hkv][r].

    [WildCat, WildCat / Alg. 4 paragraph: CompressKV followed by WtdAttn.]
    Query head h reads kv head h // (Hq / Hkv) (contiguous GQA groups; the
    grouping is not on the pages).  Returns (O [B][Hq][m][d], per-unit results).
    """
    Q = np.asarray(Q, dtype=np.float64)
    B, Hq, m, d = Q.shape
    Hkv = K.shape[1]
    group = Hq // Hkv
    units = []
    for b in range(B):
        for h in range(Hkv):
            units.append(compress_unit(K[b, h], V[b, h], u[b * Hkv + h], r, beta, tau, recentre, factor))
    O = np.empty((B, Hq, m, d))
    for b in range(B):
        for h in range(Hq):
            ur = units[b * Hkv + h // group]
            O[b, h] = plugin_attend(Q[b, h], ur.K_S, ur.X, ur.vmin, ur.vmax, beta)
    return O, units

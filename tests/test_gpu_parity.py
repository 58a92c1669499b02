"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Oracle-sized cases compare every output element by element; they span several
workgroups of the selection kernel (512 keys each) with ragged tails, several
64-row contraction tiles, GQA groups, recentring and tau != 1.  Pivots must
match bit for bit, L to 1e-9 of its scale, the value range exactly, and O
within 2e-3 (fp32) or 2e-2 (bf16) of max|V|.  A pivot mismatch at an fp64 near
tie (see _helpers.check_pivots) would stop the comparison of that unit short;
it fails the test unless the caller allows it, and every such exit is listed
in the session summary.
"""
import sys

import numpy as np
import pytest

from nystr_rpcholesky_coreset_amd import inputs as I
from oracle import wildcat_oracle as orc

from _helpers import check_pivots, oracle_attend_rows, oracle_units, rel_max, to_device, tol_for

pytestmark = pytest.mark.gpu

W = I.WORKLOADS
C1, C2, C3, C4, C5 = (W[k] for k in I.WORKLOAD_ORDER)

SMALL_CASES = {
    "probe_full": C1,
    "probe_ragged": I.scaled_workload(C1, n=1000, m=333, r=77, seed=7),
    "vit_b3": I.scaled_workload(C2, batch=3),
    "latent_h2": I.scaled_workload(C3, batch=1, q_heads=2, kv_heads=2),
    "kv_gqa8x2_ragged": I.scaled_workload(C4, q_heads=8, kv_heads=2, n=5000, r=200),
    "sphere_h2": I.scaled_workload(C5, q_heads=2, kv_heads=2, n=3000, m=700, r=150),
    "kv_recentre_tau": I.scaled_workload(C4, q_heads=4, kv_heads=2, n=1500, r=100, recentre=True, tau=1.7),
    "probe_recentre": I.scaled_workload(C1, n=700, m=100, r=40, recentre=True, tau=0.8, seed=9),
    # few query rows and r >= 256: attend splits the pivots over the waves of
    # a workgroup (d = 128: 4 ranges, the last one ragged; d = 64 and 32: 8
    # ranges, some past r and empty, ragged query tiles)
    "kv_keysplit_d128": I.scaled_workload(C4, q_heads=4, kv_heads=2, n=3000, m=64, r=300, seed=21),
    "latent_keysplit_d64": I.scaled_workload(C3, batch=1, q_heads=2, kv_heads=2, n=2000, m=100, r=280, seed=22),
    "kv_keysplit_d32": I.scaled_workload(C4, q_heads=4, kv_heads=1, n=1200, m=50, r=260, d=32, seed=23),
    # 64 or more units: eight unit groups of 8 or 9 units each on the paired
    # streams, fp32 and bf16, recentring and tau, n up to 4096
    "units64_vit_n600": I.scaled_workload(C2, batch=64, n=600, m=40, r=40, seed=24),
    "units64_latent_n3000": I.scaled_workload(C3, batch=8, q_heads=8, kv_heads=8, n=3000, m=64, r=60, seed=25),
    "units64_probe_fp32_recentre": I.scaled_workload(C1, batch=64, n=300, m=20, r=30, recentre=True, tau=0.9,
                                                     seed=26),
    "units64_kv_gqa_d128": I.scaled_workload(C4, batch=8, q_heads=16, kv_heads=8, n=1500, m=32, r=100, seed=27),
    "units72_kv_n4096_tau": I.scaled_workload(C4, batch=9, q_heads=8, kv_heads=8, n=4096, m=16, r=48, tau=1.4,
                                              seed=28),
    # 12 units: the solve's XCD-aware grids round up to 16 units (padding
    # workgroups), with two 256-row solve blocks (r = 300)
    "units12_kv_r300": I.scaled_workload(C4, batch=3, q_heads=8, kv_heads=4, n=2000, m=48, r=300, seed=29),
}


def _run_gpu(inp):
    import torch
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    w = inp["workload"]
    Q = to_device(inp["Q"], w.dtype)
    K = to_device(inp["K"], w.dtype)
    V = to_device(inp["V"], w.dtype)
    u = torch.from_numpy(inp["u"]).cuda()
    O, parts = wc.forward(Q, K, V, u, w.r, w.beta, w.tau, w.recentre)
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in parts.items()}
    out["O"] = O.cpu()
    for k in ("K_S",):
        out[k] = out[k].float() if out[k].dtype == torch.bfloat16 else out[k]
    return {k: v.numpy() for k, v in out.items()}


def _compare_unit(inp, g, u, ures, qrows=None, check_O=True, allow_near_tie=False):
    w = inp["workload"]
    sel = ures.sel
    matched = check_pivots(g["S"][u], int(g["r_eff"][u]), sel, context=f"{w.name} unit {u}")
    full = matched == sel.r_eff
    assert full or allow_near_tie, (
        f"unit {u}: pivots diverge at a near tie at draw {matched}; the comparison of L, X and O "
        f"would stop short")
    re = matched
    L = g["L"][u]
    scale = max(1.0, float(np.abs(sel.L).max()))
    assert rel_max(L[:re, :re], sel.L[:re, :re], scale) < 1e-9
    assert np.all(L[:re][np.triu_indices(re, 1)] == 0.0)
    b, h = divmod(u, w.kv_heads)
    vmin, vmax = g["vmin"][b, h], g["vmax"][b, h]
    np.testing.assert_array_equal(vmin, ures.vmin.astype(np.float32))
    np.testing.assert_array_equal(vmax, ures.vmax.astype(np.float32))
    KS = g["K_S"][b, h]
    np.testing.assert_array_equal(KS[:re], ures.K_S[:re].astype(np.float32))
    if full:
        assert np.all(L[sel.r_eff:] == 0.0) and np.all(KS[sel.r_eff:] == 0) and np.all(g["X"][b, h][sel.r_eff:] == 0)
    if not (check_O and full):
        return
    Vmax = float(np.abs(I.to_f64(inp["V"], w.dtype)).max())
    group = w.q_heads // w.kv_heads
    for hq in range(h * group, (h + 1) * group):
        qu = b * w.q_heads + hq
        Oo = oracle_attend_rows(inp, ures, qu, qrows)
        Og = g["O"][b, hq] if qrows is None else g["O"][b, hq][qrows]
        err = rel_max(Og, Oo, Vmax)
        print(f"unit {u} q-head {hq}: max|dO|/max|V| = {err:.3e}")
        assert err < tol_for(w.dtype), err
        assert np.all(Og >= vmin[None, :]) and np.all(Og <= vmax[None, :])


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_parity_small(name):
    w = SMALL_CASES[name]
    print(f"case {name}: {w}", flush=True)
    inp = I.make_inputs(w)
    g = _run_gpu(inp)
    units = list(range(w.units))
    ref = oracle_units(inp, units)
    for u in units:
        _compare_unit(inp, g, u, ref[u])


def _edge_inputs(K, V, Q, r, beta, dtype="fp32"):
    w = I.Workload("edge", "unit_ball", 1, Q.shape[0], 1, Q.shape[1], K.shape[0], K.shape[1], r, beta, dtype, 0)
    store = (lambda x: x.astype(np.float32)) if dtype == "fp32" else (lambda x: I.bf16_bits_from_f32(x.astype(np.float32)))
    return {"Q": store(Q)[None], "K": store(K)[None, None], "V": store(V)[None, None],
            "u": np.random.default_rng(5).random((1, r)), "workload": w}


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_zero_keys_stop_after_one_pivot(dtype):
    rng = np.random.default_rng(1)
    K = np.zeros((300, 32))
    V = rng.standard_normal((300, 32))
    Q = rng.standard_normal((2, 50, 32)) / 6
    inp = _edge_inputs(K, V, Q, 16, 0.2, dtype)
    g = _run_gpu(inp)
    assert g["r_eff"][0] == 1
    assert np.all(g["S"][0][1:] == -1)
    Vd = I.to_f64(inp["V"], dtype)[0, 0]
    np.testing.assert_allclose(g["O"][0], np.broadcast_to(Vd.mean(0), (2, 50, 32)), atol=tol_for(dtype) * np.abs(Vd).max())


def test_duplicated_keys_stop_at_distinct_count():
    rng = np.random.default_rng(2)
    base = rng.standard_normal((6, 16)) / 2
    K = base[rng.integers(0, 6, 900)]
    K[:6] = base
    V = rng.standard_normal((900, 16))
    Q = rng.standard_normal((1, 64, 16)) / 2
    inp = _edge_inputs(K, V, Q, 20, 0.5)
    g = _run_gpu(inp)
    ref = oracle_units(inp, [0])[0]
    assert ref.sel.r_eff == 6
    _compare_unit(inp, g, 0, ref)
    exact = orc.exact_attention(Q[0], K, V, 0.5)
    assert rel_max(g["O"][0, 0], exact, np.abs(V).max()) < 2e-3


@pytest.mark.parametrize("M,d", [(70, 16), (330, 16), (330, 128)])
def test_early_stop_inside_solve_blocks(M, d):
    """Copies of M distinct keys of one norm stop the selection at r_eff = M
    (equal diagonals: the residual trace falls from at least half a diagonal
    entry to rounding noise once every distinct key is a pivot, far from the
    stop threshold on either side), while r = 600 pads the rank to three
    256-row solve blocks: r_eff falls inside a 64-row block, so the identity
    tail of the block inverses, the guarded doubling tiles and the partial
    sweep tiles all take part."""
    rng = np.random.default_rng(100 + M + d)
    beta = 0.5
    base = rng.standard_normal((M, d))
    base *= np.sqrt(18.0 / beta) / np.linalg.norm(base, axis=1, keepdims=True)
    n = 2000
    K = base[rng.integers(0, M, n)]
    K[:M] = base
    V = rng.standard_normal((n, d))
    Q = rng.standard_normal((1, 64, d)) / np.sqrt(d)
    inp = _edge_inputs(K, V, Q, 600, beta)
    g = _run_gpu(inp)
    ref = oracle_units(inp, [0])[0]
    assert ref.sel.r_eff == M
    assert g["r_eff"][0] == M
    _compare_unit(inp, g, 0, ref)


@pytest.mark.parametrize("n,r", [(64, 64), (1, 1), (513, 1), (600, 600)])
def test_rank_extremes(n, r):
    """Well-conditioned kernels (|k|^2 ~ 16, beta 1/2) so that r = n runs to
    full rank; r = n must then reproduce exact softmax."""
    rng = np.random.default_rng(n + r)
    K = rng.standard_normal((n, 16))
    V = rng.standard_normal((n, 16))
    Q = rng.standard_normal((1, 40, 16)) / 2
    inp = _edge_inputs(K, V, Q, r, 0.5)
    g = _run_gpu(inp)
    ref = oracle_units(inp, [0])[0]
    _compare_unit(inp, g, 0, ref)
    if r == n:
        assert ref.sel.r_eff == n
        exact = orc.exact_attention(Q[0], K, V, 0.5)
        assert rel_max(g["O"][0, 0], exact, np.abs(V).max()) < 2e-3


def test_repeat_calls_are_bitwise_deterministic():
    w = SMALL_CASES["kv_gqa8x2_ragged"]
    inp = I.make_inputs(w)
    a, b = _run_gpu(inp), _run_gpu(inp)
    for k in ("S", "r_eff", "L", "X", "O"):
        np.testing.assert_array_equal(a[k], b[k])


def test_mixed_early_stop_across_unit_groups():
    """Five units run as separate unit groups; units 1 and 3 hold only three
    distinct keys and stop at r_eff = 3 while the others run all r steps."""
    rng = np.random.default_rng(11)
    n, d, r, H = 700, 32, 24, 5
    K = rng.standard_normal((H, n, d)) / 3
    for h in (1, 3):
        base = rng.standard_normal((3, d)) / 3
        K[h] = base[rng.integers(0, 3, n)]
        K[h, :3] = base
    V = rng.standard_normal((H, n, d))
    Q = rng.standard_normal((H, 48, d)) / 3
    w = I.Workload("groups", "unit_ball", 1, H, H, 48, n, d, r, 0.5, "fp32", 0)
    inp = {"Q": Q.astype(np.float32)[None], "K": K.astype(np.float32)[None], "V": V.astype(np.float32)[None],
           "u": np.random.default_rng(12).random((H, r)), "workload": w}
    g = _run_gpu(inp)
    ref = oracle_units(inp, list(range(H)))
    assert [ref[h].sel.r_eff for h in range(H)] == [r, 3, r, 3, r]
    for h in range(H):
        _compare_unit(inp, g, h, ref[h])


def test_check_range_bounds_and_error():
    """wildcat_check_range: the exponent bounds it reports equal the
    Cauchy-Schwarz bounds computed here from the same inputs; inputs scaled
    past the limit, or holding a NaN, give WILDCAT_ERR_RANGE."""
    import torch
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    w = SMALL_CASES["kv_gqa8x2_ragged"]
    inp = I.make_inputs(w)
    K64 = I.to_f64(inp["K"], w.dtype)
    Q64 = I.to_f64(inp["Q"], w.dtype)
    mk = float((K64 ** 2).sum(-1).max())
    mq = float((Q64 ** 2).sum(-1).max())
    K = to_device(inp["K"], w.dtype)
    Q = to_device(inp["Q"], w.dtype)
    ek, eq = wc.check_range(K, w.r, w.beta, Q=Q)
    assert abs(ek - w.beta * mk) <= 1e-12 * max(1.0, ek)
    assert abs(eq - w.beta * np.sqrt(mq) * np.sqrt(mk)) <= 1e-12 * max(1.0, eq)
    ek2, eq2 = wc.check_range(K, w.r, w.beta, tau=2.0, recentre=True)
    assert abs(ek2 - w.beta * mk) <= 1e-12 * max(1.0, ek2) and eq2 == 0.0   # x4 / tau^2 = x1
    big = (K.float() * 40.0).to(K.dtype)
    with pytest.raises(wc.WildcatError) as e:
        wc.check_range(big, w.r, w.beta)
    assert e.value.status == wc.WILDCAT_ERR_RANGE
    bad = K.clone()
    bad.view(-1)[12345] = float("nan")
    with pytest.raises(wc.WildcatError) as e:
        wc.check_range(bad, w.r, w.beta)
    assert e.value.status == wc.WILDCAT_ERR_RANGE
    torch.cuda.synchronize()


def test_concurrent_calls_on_two_streams_match_sequential():
    """Two host threads run the whole path at once, each on its own
    non-default stream (the library's auxiliary streams are shared between
    them); every output must equal, bit for bit, the output of the same call
    made alone on the default stream."""
    import threading

    import torch
    cases = [SMALL_CASES["kv_gqa8x2_ragged"], SMALL_CASES["latent_h2"]]
    inps = [I.make_inputs(w) for w in cases]
    ref = [_run_gpu(inp) for inp in inps]
    out = [None, None]
    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    out[k] = _run_gpu(inps[k])
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(2):
        for key in ("S", "r_eff", "L", "X", "O"):
            np.testing.assert_array_equal(out[k][key], ref[k][key])


def test_many_units_mixed_early_stop():
    """64 units in eight groups; every even unit u has only 3 + u % 7
    distinct keys, so its residual vanishes after that many pivots and it
    stops early (r_eff < r) while the others in its group run to r."""
    rng = np.random.default_rng(31)
    U, n, d, r = 64, 400, 32, 12
    K = np.empty((U, n, d))
    for u in range(U):
        distinct = 3 + u % 7 if u % 2 == 0 else n
        base = 0.3 * rng.standard_normal((min(distinct, n), d))
        K[u] = base[rng.integers(0, len(base), n)] if distinct < n else 0.3 * rng.standard_normal((n, d))
    V = rng.standard_normal((U, n, d))
    Q = 0.3 * rng.standard_normal((U, 8, d))
    w = I.Workload("units64_early", "unit_ball", U, 1, 1, 8, n, d, r, 0.5, "fp32", 0)
    inp = {"Q": Q.astype(np.float32)[:, None], "K": K.astype(np.float32)[:, None], "V": V.astype(np.float32)[:, None],
           "u": np.random.default_rng(32).random((U, r)), "workload": w}
    g = _run_gpu(inp)
    ref = oracle_units(inp, list(range(U)))
    stopped = 0
    for u in range(U):
        _compare_unit(inp, g, u, ref[u])
        stopped += int(g["r_eff"][u] < r)
    assert stopped >= 16


def test_non_current_stream_with_concurrent_allocations():
    """Every call gets stream= a stream that is not the current one.  While
    its kernels run, the current stream allocates and overwrites blocks the
    size of each workspace: memory the binding released to the current
    stream's pool would be handed out and clobbered.  The outputs must equal
    those of plain calls bit for bit."""
    import torch
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    w = I.scaled_workload(C4, q_heads=4, kv_heads=2, n=20000, m=64, r=512, seed=41)
    inp = I.make_inputs(w)
    ref = _run_gpu(inp)
    Q, K, V = (to_device(inp[k], w.dtype) for k in "QKV")
    u = torch.from_numpy(inp["u"]).cuda()
    desc = wc.kv_desc(K, w.r, w.beta)
    nsel, nw = wc.select_workspace_bytes(desc), wc.weights_workspace_bytes(desc)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    S, r_eff, L = wc.select(K, u, w.r, w.beta, stream=s)
    junk = [torch.full((nsel,), 255, dtype=torch.uint8, device="cuda")]
    K_S, X, vmin, vmax = wc.weights(K, V, S, r_eff, L, w.r, w.beta, stream=s)
    junk.append(torch.full((nw,), 255, dtype=torch.uint8, device="cuda"))
    O = wc.attend(Q, K_S, X, vmin, vmax, w.beta, stream=s)
    junk.append(torch.full((O.numel() * 4,), 255, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    got = {"S": S, "r_eff": r_eff, "L": L, "X": X, "vmin": vmin, "vmax": vmax, "O": O}
    for k, v in got.items():
        np.testing.assert_array_equal(v.cpu().numpy(), ref[k], err_msg=k)
    del junk


def test_compress_kv_recentres_by_default():
    """compress_kv with its defaults runs CompressKV on recentred keys: its
    cache equals that of forward(..., recentre=True) bit for bit, and both
    match the oracle's CompressKV with recentring on."""
    import torch
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    w = I.scaled_workload(C4, q_heads=4, kv_heads=2, n=1500, m=40, r=100, recentre=True, tau=1.3, seed=31)
    inp = I.make_inputs(w)
    K = to_device(inp["K"], w.dtype)
    V = to_device(inp["V"], w.dtype)
    u = torch.from_numpy(inp["u"]).cuda()
    cache = wc.compress_kv(K, V, u, w.r, w.beta, w.tau)
    torch.cuda.synchronize()
    g = _run_gpu(inp)   # forward with recentre=True
    for k in ("S", "r_eff", "L", "X", "vmin", "vmax"):
        np.testing.assert_array_equal(cache[k].cpu().numpy(), g[k])
    np.testing.assert_array_equal(cache["K_S"].float().cpu().numpy(), g["K_S"])
    ref = oracle_units(inp, list(range(w.units)))
    for unit in range(w.units):
        _compare_unit(inp, g, unit, ref[unit])

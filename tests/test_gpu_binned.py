"""GPU parity of binned WildCat (the RPNys divide-and-conquer remark) against
the oracle's binned CompressKV, through the C ABI (select and weights on the
bin-major view, wildcat_merge_value_ranges, attend on the concatenated
coreset).  Pivots per bin bit for bit; L per bin to 1e-9; K_S exact; value
ranges exact; Ô within the dtype tolerance of max|V|."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

from nystr_rpcholesky_coreset_amd import inputs as I
from oracle import wildcat_oracle as orc

from _helpers import NEAR_TIE, NEAR_TIE_F32, check_pivots, rel_max, to_device, tol_for

pytestmark = pytest.mark.gpu

W = I.WORKLOADS
CASES = {
    "kv_b4": (I.scaled_workload(W["kvcache_gqa32x8_n32768_d128_r1024_bf16"], q_heads=8, kv_heads=2, n=4096,
                                m=64, r=256, seed=31), 4),
    "latent_b2": (I.scaled_workload(W["latent_b8h8_n4096_d64_r256_bf16"], batch=1, q_heads=2, kv_heads=2, n=2048,
                                    m=300, r=128, seed=32), 2),
    "probe_b4": (I.scaled_workload(W["probe_n256_d16_r32_fp32"], seed=33), 4),
    "vit_b8": (I.scaled_workload(W["vit_b128_n3136_d64_r128_bf16"], batch=2, n=3136, m=500, r=128, seed=34), 8),
    "kv_recentre_b2": (I.scaled_workload(W["kvcache_gqa32x8_n32768_d128_r1024_bf16"], q_heads=4, kv_heads=2,
                                         n=2000, m=40, r=100, recentre=True, tau=1.4, seed=35), 2),
}


def _run(inp, bins, factor="f64"):
    import torch
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    w = inp["workload"]
    Q, K, V = (to_device(inp[k], w.dtype) for k in ("Q", "K", "V"))
    u = torch.from_numpy(inp["u"]).cuda()
    O, parts = wc.forward_binned(Q, K, V, u, w.r, bins, w.beta, w.tau, w.recentre, factor=factor)
    torch.cuda.synchronize()
    out = {k: v.float().cpu().numpy() if v.dtype == torch.bfloat16 else v.cpu().numpy() for k, v in parts.items()}
    out["O"] = O.cpu().numpy()
    return out


def _compare(inp, g, bins, units, factor="f64", allow_near_tie=True):
    w = inp["workload"]
    K = I.to_f64(inp["K"], w.dtype)
    V = I.to_f64(inp["V"], w.dtype)
    Vmax = float(np.abs(V).max())
    rb = w.r // bins
    group = w.q_heads // w.kv_heads
    for u in units:
        b, h = divmod(u, w.kv_heads)
        res = orc.compress_unit_binned(K[b, h], V[b, h], inp["u"][u], w.r, bins, w.beta, w.tau, w.recentre,
                                       factor)
        full = True
        for k, part in enumerate(res.bins):
            ub = u * bins + k
            m = check_pivots(g["S"][ub], int(g["r_eff"][ub]), part.sel,
                             near=NEAR_TIE if factor == "f64" else NEAR_TIE_F32,
                             context=f"{w.name} bins {bins} {factor} unit {u} bin {k}")
            full &= m == part.sel.r_eff
            assert m == part.sel.r_eff or allow_near_tie, f"unit {u} bin {k}: a near tie at draw {m}"
            L = g["L"][ub]
            scale = max(1.0, float(np.abs(part.sel.L).max()))
            assert rel_max(L[:m, :m], part.sel.L[:m, :m], scale) < (1e-9 if factor == "f64" else 2e-6)
            np.testing.assert_array_equal(g["K_S"][b, h][k * rb:k * rb + m], part.K_S[:m].astype(np.float32))
        np.testing.assert_array_equal(g["vmin"][b, h], res.vmin.astype(np.float32))
        np.testing.assert_array_equal(g["vmax"][b, h], res.vmax.astype(np.float32))
        if not full:
            continue
        for hq in range(h * group, (h + 1) * group):
            Qh = I.to_f64(inp["Q"][b, hq], w.dtype)
            Oo = orc.plugin_attend(Qh, res.K_S, res.X, res.vmin, res.vmax, w.beta)
            err = rel_max(g["O"][b, hq], Oo, Vmax)
            print(f"unit {u} q-head {hq}: max|dO|/max|V| = {err:.3e}")
            assert err < tol_for(w.dtype), err


@pytest.mark.parametrize("name", list(CASES))
def test_binned_parity_small(name):
    w, bins = CASES[name]
    print(f"case {name}: bins {bins}, {w}", flush=True)
    inp = I.make_inputs(w)
    g = _run(inp, bins)
    _compare(inp, g, bins, range(w.units))


def test_binned_kvcache_fullsize_all_units():
    """The 32k KV-cache workload with 4 bins (8192 keys and 256 pivots per
    bin): every unit and bin against the oracle."""
    w = W["kvcache_gqa32x8_n32768_d128_r1024_bf16"]
    print(f"workload {w.name}, 4 bins: generating inputs", flush=True)
    inp = I.make_inputs(w)
    g = _run(inp, 4)
    print("running the oracle on all 8 units x 4 bins", flush=True)
    _compare(inp, g, 4, range(w.units), allow_near_tie=False)


def test_binned_rejects_indivisible_sizes():
    import torch
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    K = torch.zeros((1, 1, 100, 16), device="cuda")
    with pytest.raises(ValueError):
        wc.forward_binned(K[:, :, :, :], K, K, torch.zeros((1, 8), dtype=torch.float64, device="cuda"), 8, 3, 0.1)
    with pytest.raises(ValueError):   # n = 100 keys in 8 bins
        wc.forward_binned(K, K, K, torch.zeros((1, 8), dtype=torch.float64, device="cuda"), 8, 8, 0.1)


@pytest.mark.parametrize("name", ["kv_b4", "vit_b8"])
def test_binned_float32_factor(name):
    """Binned selection with the float32 factor against the oracle's binned
    float32-factor CompressKV."""
    w, bins = CASES[name]
    inp = I.make_inputs(w)
    g = _run(inp, bins, factor="f32")
    _compare(inp, g, bins, range(w.units), factor="f32")

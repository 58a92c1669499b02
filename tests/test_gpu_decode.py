"""Parity of wildcat_decode (generation over a compressed cache) with the oracle.

The cache each case decodes over is computed on the CPU: the oracle's
CompressKV of a small workload, or at full size a seeded synthetic weighted
coreset (decode is defined for any cache).  X enters both sides rounded to
float32, the GPU's input type.  The new tokens and their queries come from
the input module.  Every output element is compared, within 2e-3 (fp32) or
2e-2 (bf16) of max |V| over the cache and the new tokens.  The cases cover
every attend kernel (fp32 vector ALU, bf16 d = 16, 32x32 MFMA with and
without the key split), ragged query tiles, several 64-row blocks of the
running range, one new token, and GQA groups.
"""
import numpy as np
import pytest

from nystr_rpcholesky_coreset_amd import inputs as I
from oracle import wildcat_oracle as orc

from _helpers import rel_max, to_device, tol_for

pytestmark = pytest.mark.gpu

W = I.WORKLOADS
C1, C2, C3, C4, C5 = (W[k] for k in I.WORKLOAD_ORDER)

CASES = {
    "probe_fp32_d16": I.scaled_workload(C1, n=300, m=50, r=20, seed=31),
    "probe_fp32_d64_ragged": I.scaled_workload(C1, n=400, m=130, r=33, d=64, seed=32),
    "probe_fp32_d128": I.scaled_workload(C1, q_heads=2, kv_heads=1, n=500, m=70, r=40, d=128, seed=43),
    "probe_fp32_d32_m200": I.scaled_workload(C1, n=350, m=200, r=25, d=32, seed=44),
    "vit_b2_d64": I.scaled_workload(C2, batch=2, n=600, m=100, r=40, seed=33),
    "latent_m300": I.scaled_workload(C3, batch=1, q_heads=2, kv_heads=2, n=800, m=300, r=64, seed=34),
    "kv_gqa8x2_m64": I.scaled_workload(C4, q_heads=8, kv_heads=2, n=2000, m=64, r=200, seed=35),
    "kv_gqa4x2_m200": I.scaled_workload(C4, q_heads=4, kv_heads=2, n=2500, m=200, r=300, seed=36),
    "kv_d32_m70": I.scaled_workload(C4, q_heads=2, kv_heads=1, n=900, m=70, r=50, d=32, seed=37),
    "kv_d16_bf16": I.scaled_workload(C4, q_heads=2, kv_heads=1, n=700, m=90, r=60, d=16, seed=38),
    "sphere_m700": I.scaled_workload(C5, q_heads=2, kv_heads=2, n=1500, m=700, r=150, seed=39),
    # one new token: the dedicated one-workgroup-per-query-head form
    "one_token": I.scaled_workload(C4, q_heads=4, kv_heads=2, n=800, m=1, r=100, seed=40),
    "one_token_fp32_d16": I.scaled_workload(C1, n=300, m=1, r=25, seed=45),
    "one_token_d64_b3": I.scaled_workload(C2, batch=3, n=500, m=1, r=60, seed=46),
    "one_token_d32_r1": I.scaled_workload(C4, q_heads=2, kv_heads=1, n=200, m=1, r=1, d=32, seed=47),
    "rank_one": I.scaled_workload(C2, batch=1, n=300, m=40, r=1, seed=41),
}


def _store(x64, dtype):
    return I.bf16_bits_from_f32(x64.astype(np.float32)) if dtype == "bf16" else x64.astype(np.float32)


def _oracle_cache(inp):
    """CompressKV of every unit on the CPU: K_S (input storage), X (float32),
    vmin, vmax, and the scale max |V| of the cache."""
    w = inp["workload"]
    K = I.to_f64(inp["K"], w.dtype)
    V = I.to_f64(inp["V"], w.dtype)
    B, H, d, r = w.batch, w.kv_heads, w.d, w.r
    K_S = np.zeros((B, H, r, d))
    X = np.zeros((B, H, r, d + 1), np.float32)
    vmin, vmax = np.zeros((B, H, d), np.float32), np.zeros((B, H, d), np.float32)
    for b in range(B):
        for h in range(H):
            c = orc.compress_unit(K[b, h], V[b, h], inp["u"][b * H + h], r, w.beta, w.tau, w.recentre)
            k = c.sel.r_eff
            K_S[b, h, :k], X[b, h, :k] = c.K_S, c.X.astype(np.float32)
            vmin[b, h], vmax[b, h] = c.vmin, c.vmax
    return K_S, X, vmin, vmax, float(np.abs(V).max())


def _run(inp, K_S64, X32, vmin, vmax):
    import torch
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    w = inp["workload"]
    dev = lambda a: to_device(a, w.dtype)
    O = wc.decode(dev(inp["Q"]), dev(_store(K_S64, w.dtype)), torch.from_numpy(X32).cuda(),
                  torch.from_numpy(vmin).cuda(), torch.from_numpy(vmax).cuda(), dev(inp["K_new"]), dev(inp["V_new"]),
                  w.beta)
    torch.cuda.synchronize()
    return O.cpu().numpy()


def _check(O, ref, scale, dtype, what):
    """Element bound relative to max |V| (the contract), plus the relative
    Frobenius error, which also catches outputs that are merely small: the
    outputs are averages, often a few percent of max |V|."""
    assert np.all(np.isfinite(O)), what
    err = rel_max(O, ref, scale)
    assert err < tol_for(dtype), f"{what}: max err {err:.3e} of max|V|"
    fro = float(np.linalg.norm(O - ref) / np.linalg.norm(ref))
    assert fro < (5e-3 if dtype == "fp32" else 5e-2), f"{what}: relative Frobenius error {fro:.3e}"


def _oracle(inp, K_S64, X32, vmin, vmax):
    w = inp["workload"]
    return orc.wildcat_decode(I.to_f64(inp["Q"], w.dtype), K_S64, X32.astype(np.float64), vmin.astype(np.float64),
                              vmax.astype(np.float64), I.to_f64(inp["K_new"], w.dtype), I.to_f64(inp["V_new"], w.dtype),
                              w.beta)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_parity_small(name):
    w = CASES[name]
    print(f"[decode] {name}: {w}", flush=True)
    inp = I.make_inputs(w, new_tokens=True)
    K_S, X, vmin, vmax, vscale = _oracle_cache(inp)
    O = _run(inp, K_S, X, vmin, vmax)
    ref = _oracle(inp, K_S, X, vmin, vmax)
    scale = max(vscale, float(np.abs(I.to_f64(inp["V_new"], w.dtype)).max()))
    _check(O, ref, scale, w.dtype, name)


def test_decode_later_tokens_do_not_reach_earlier_queries():
    import torch
    w = CASES["kv_gqa4x2_m200"]
    inp = I.make_inputs(w, new_tokens=True)
    K_S, X, vmin, vmax, _ = _oracle_cache(inp)
    base = _run(inp, K_S, X, vmin, vmax)
    i = 77
    alt = dict(inp)
    rng = np.random.default_rng(5)
    Kn, Vn = I.to_f64(inp["K_new"], w.dtype), I.to_f64(inp["V_new"], w.dtype)
    Kn[:, :, i + 1:] = 0.1 * rng.standard_normal(Kn[:, :, i + 1:].shape)
    Vn[:, :, i + 1:] += 3.0
    alt["K_new"], alt["V_new"] = _store(Kn, w.dtype), _store(Vn, w.dtype)
    O = _run(alt, K_S, X, vmin, vmax)
    np.testing.assert_array_equal(O[:, :, :i + 1], base[:, :, :i + 1])
    assert not np.array_equal(O[:, :, i + 1:], base[:, :, i + 1:])
    # the same bits on a repeated call
    np.testing.assert_array_equal(_run(inp, K_S, X, vmin, vmax), base)


@pytest.mark.parametrize("m", [64, 1])
def test_decode_full_size_kv_cache(m):
    """The 32k KV-cache workload's decode shape: 32 query heads over 8 kv heads,
    a cache of r = 1024 per kv head, m = 64 new tokens (the key-split attend
    kernel over 1088 rows) or one (the one-token form).  The cache is a seeded
    synthetic weighted coreset: K_S = the first r cached keys, X = w [V_S, 1]
    with weights w in [0.5, 1.5]."""
    w = C4 if m == C4.m else I.scaled_workload(C4, m=m)
    print(f"[decode] full size: {w.name}", flush=True)
    inp = I.make_inputs(w, new_tokens=True)
    K = I.to_f64(inp["K"], w.dtype)
    V = I.to_f64(inp["V"], w.dtype)
    r = w.r
    wt = np.random.default_rng(w.seed + 3000).uniform(0.5, 1.5, (w.batch, w.kv_heads, r, 1))
    K_S = K[:, :, :r]
    X = (wt * np.concatenate([V[:, :, :r], np.ones_like(wt)], axis=3)).astype(np.float32)
    vmin, vmax = V.min(axis=2).astype(np.float32), V.max(axis=2).astype(np.float32)
    O = _run(inp, K_S, X, vmin, vmax)
    ref = _oracle(inp, K_S, X, vmin, vmax)
    scale = max(float(np.abs(V).max()), float(np.abs(I.to_f64(inp["V_new"], w.dtype)).max()))
    _check(O, ref, scale, w.dtype, "full size")


def test_decode_after_gpu_compression_end_to_end():
    """wildcat forward (select, weights) then decode on the GPU, against the
    oracle's CompressKV then decode on the CPU."""
    import torch
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    w = I.scaled_workload(C4, q_heads=4, kv_heads=2, n=1500, m=96, r=120, seed=42)
    inp = I.make_inputs(w, new_tokens=True)
    dev = lambda a: to_device(a, w.dtype)
    K, V = dev(inp["K"]), dev(inp["V"])
    u = torch.from_numpy(inp["u"]).cuda()
    S, r_eff, L = wc.select(K, u, w.r, w.beta)
    K_S, X, vmin, vmax = wc.weights(K, V, S, r_eff, L, w.r, w.beta)
    O = wc.decode(dev(inp["Q"]), K_S, X, vmin, vmax, dev(inp["K_new"]), dev(inp["V_new"]), w.beta)
    torch.cuda.synchronize()
    K_S64, X32, vmn, vmx, vscale = _oracle_cache(inp)
    ref = _oracle(inp, K_S64, X32, vmn, vmx)
    scale = max(vscale, float(np.abs(I.to_f64(inp["V_new"], w.dtype)).max()))
    _check(O.cpu().numpy(), ref, scale, w.dtype, "end to end")


def test_decode_long_context_sampled_rows():
    """The 131k long-context workload's decode shape: 8 heads, a cache of
    r = 2048 per head, m = 131072 new tokens attending causally (the
    many-tile causal form, 2048 blocks of the running range).  The cache is a
    seeded synthetic weighted coreset as above; sampled rows of two heads,
    near the start, the middle and the end, are computed by the oracle one
    by one."""
    w = C5
    print(f"[decode] long context: {w.name}: generating inputs", flush=True)
    inp = I.make_inputs(w, new_tokens=True)
    r = w.r
    K_S = I.to_f64(inp["K"][:, :, :r], w.dtype)
    V_S = I.to_f64(inp["V"][:, :, :r], w.dtype)
    V = I.to_f64(inp["V"], w.dtype)
    wt = np.random.default_rng(w.seed + 3000).uniform(0.5, 1.5, (w.batch, w.kv_heads, r, 1))
    X = (wt * np.concatenate([V_S, np.ones_like(wt)], axis=3)).astype(np.float32)
    vmin, vmax = V.min(axis=2).astype(np.float32), V.max(axis=2).astype(np.float32)
    del V
    print("[decode] long context: GPU", flush=True)
    O = _run(inp, K_S, X, vmin, vmax)
    assert np.all(np.isfinite(O))
    Vn_all = I.to_f64(inp["V_new"], w.dtype)
    scale = max(float(np.abs(V_S).max()), float(np.abs(Vn_all).max()), float(np.abs(vmin).max()),
                float(np.abs(vmax).max()))
    rows = [0, 1, 63, 64, 4097, 65535, 100000, w.m - 1]
    worst = 0.0
    for h in (0, 5):
        Kn = I.to_f64(inp["K_new"][0, h], w.dtype)
        Vn = Vn_all[0, h]
        for i in rows:
            q = I.to_f64(inp["Q"][0, h, i], w.dtype)
            ref = orc.decode_row(q, i, K_S[0, h], X[0, h].astype(np.float64), vmin[0, h].astype(np.float64),
                                 vmax[0, h].astype(np.float64), Kn, Vn, w.beta)
            worst = max(worst, rel_max(O[0, h, i], ref, scale))
    print(f"[decode] long context: max err {worst:.3e} of max|V|", flush=True)
    assert worst < tol_for(w.dtype)

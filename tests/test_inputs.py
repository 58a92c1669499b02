"""Host-side checks of the seeded synthetic input generators."""
import numpy as np
import torch

from nystr_rpcholesky_coreset_amd import inputs as I


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 10000),
                        np.array([1.00390625, 1.01171875, -2.00781250, 0.0, -0.0], np.float32)])
    ours = I.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = I.f64_from_bf16_bits(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_workloads_are_seeded_and_shaped():
    w = I.scaled_workload(I.WORKLOADS["kvcache_gqa32x8_n32768_d128_r1024_bf16"], q_heads=4, kv_heads=2, n=300, m=8, r=16)
    a, b = I.make_inputs(w), I.make_inputs(w)
    for k in "QKVu":
        np.testing.assert_array_equal(a[k], b[k])
    assert a["Q"].shape == (1, 4, 8, 128) and a["K"].shape == (1, 2, 300, 128)
    assert a["u"].shape == (2, 16) and a["u"].dtype == np.float64
    assert np.all((a["u"] >= 0) & (a["u"] < 1))
    K = I.to_f64(a["K"], "bf16")
    # sink keys at rows 0..3 are 8x larger in norm on average
    nr = np.linalg.norm(K[0, 0], axis=1)
    assert nr[:4].mean() > 5 * nr[4:].mean()


def test_recipes_statistics():
    w = I.scaled_workload(I.WORKLOADS["vit_b128_n3136_d64_r128_bf16"], batch=2)
    x = I.make_inputs(w)
    K = I.to_f64(x["K"], "bf16")
    nr = np.linalg.norm(K, axis=-1)
    # 5% outlier keys scaled by 3
    assert abs((nr > 2.0).mean() - 0.05) < 0.01
    w = I.WORKLOADS["probe_n256_d16_r32_fp32"]
    x = I.make_inputs(w)
    for k in "QKV":
        assert np.linalg.norm(x[k], axis=-1).max() <= 1.0 + 1e-6
    w = I.scaled_workload(I.WORKLOADS["longctx_h8_n131072_d128_r2048_bf16"], q_heads=1, kv_heads=1, n=500, m=500)
    x = I.make_inputs(w)
    nr = np.linalg.norm(I.to_f64(x["K"], "bf16"), axis=-1)
    assert np.allclose(nr, 2.0, atol=0.02)


def test_new_tokens_leave_the_cached_inputs_unchanged():
    for name in I.WORKLOAD_ORDER:
        w = I.scaled_workload(I.WORKLOADS[name], batch=1, q_heads=2, kv_heads=1, n=200, m=40, r=8)
        a, b = I.make_inputs(w), I.make_inputs(w, new_tokens=True)
        for k in "QKVu":
            np.testing.assert_array_equal(a[k], b[k])
        assert b["K_new"].shape == b["V_new"].shape == (1, 1, 40, w.d)
        assert b["K_new"].dtype == w.storage_dtype
        kn = I.to_f64(b["K_new"], w.dtype)
        assert np.all(np.isfinite(kn)) and not np.array_equal(kn, I.to_f64(a["K"], w.dtype)[:, :, :40])
    # the sink scaling belongs to the first cached positions only
    w = I.scaled_workload(I.WORKLOADS["kvcache_gqa32x8_n32768_d128_r1024_bf16"], q_heads=1, kv_heads=1, n=64, m=64, r=8)
    b = I.make_inputs(w, new_tokens=True)
    norms = np.linalg.norm(I.to_f64(b["K_new"], w.dtype)[0, 0], axis=1)
    assert norms.max() < 3.0

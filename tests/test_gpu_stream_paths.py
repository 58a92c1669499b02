"""RPNys factor-load paths at small sizes.

A round reads the factor columns j < i with ordinary loads while they fit the
last-level cache, and otherwise streams them with non-temporal loads, except
the oldest columns that fit beside the keys.  At sizes the oracle handles,
every round takes the first path.  libwildcat_streamcheck.so is the same
library built with cache thresholds of 0 and 2 MiB: every round after the
first takes the second path, with a kept-column count that splits a wave's
range inside an unrolled chunk.  The split falls on whole chunks, so the
accumulation order is the same in both builds: S, r_eff and L must agree
bit for bit.  One case per factor type is also checked against the oracle.
"""
import ctypes
import os

import numpy as np
import pytest

from nystr_rpcholesky_coreset_amd import inputs as I
from oracle import wildcat_oracle as orc

from _helpers import NEAR_TIE, NEAR_TIE_F32, check_pivots, rel_max, to_device

pytestmark = pytest.mark.gpu

W = I.WORKLOADS
C2, C4 = W["vit_b128_n3136_d64_r128_bf16"], W["kvcache_gqa32x8_n32768_d128_r1024_bf16"]

# Kept columns with the 2 MiB budget: (2 MiB - key bytes) / (U npad sizeof(factor)).
CASES = {
    # 3 units (odd: one stream per group, separate step and draw launches);
    # keys 768,000 bytes, 27 kept columns (float64) / 54 (float32)
    "vit_u3_n2000": I.scaled_workload(C2, batch=3, n=2000, m=8, r=150, seed=71),
    # 4 units (paired groups on two streams); keys 1,024,000 bytes, 16 / 32 kept
    "vit_u4_n2000": I.scaled_workload(C2, batch=4, n=2000, m=8, r=120, seed=72),
    # keys 2,097,152 bytes: nothing fits beside them, no column is kept
    "kv_u2_n4096": I.scaled_workload(C4, q_heads=2, kv_heads=2, m=8, n=4096, r=100, seed=73),
    # ragged last block, recentred keys; 54 kept (float64), all 90 (float32)
    "kv_u2_ragged_recentre": I.scaled_workload(C4, q_heads=2, kv_heads=2, m=8, n=1500, r=90, recentre=True,
                                              seed=74),
}


def _streamcheck_lib():
    from nystr_rpcholesky_coreset_amd import build as B
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    if not os.path.exists(B.STREAMCHECK_LIB):
        pytest.fail(f"{B.STREAMCHECK_LIB} is missing: build with `python -m nystr_rpcholesky_coreset_amd.build`")
    return wc.load_library(B.STREAMCHECK_LIB)


def _select(lib, K, u, w, factor):
    import torch
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    desc = wc.kv_desc(K, w.r, w.beta, w.tau, w.recentre, factor)
    U = desc.batch * desc.kv_heads
    S = torch.full((U, w.r), -7, dtype=torch.int32, device="cuda")
    r_eff = torch.full((U,), -7, dtype=torch.int32, device="cuda")
    L = torch.full((U, w.r, w.r), float("nan"), dtype=torch.float64, device="cuda")
    nbytes = lib.wildcat_select_workspace_bytes(ctypes.byref(desc))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    status = lib.wildcat_select(ctypes.byref(desc), wc._ptr(K), wc._ptr(u), wc._ptr(S), wc._ptr(r_eff), wc._ptr(L),
                                wc._ptr(ws), nbytes, stream)
    assert status == wc.WILDCAT_OK, lib.wildcat_status_string(status)
    torch.cuda.synchronize()
    return S.cpu().numpy(), r_eff.cpu().numpy(), L.cpu().numpy()


@pytest.mark.parametrize("factor", ["f64", "f32"])
@pytest.mark.parametrize("name", list(CASES))
def test_streaming_paths_match_cached_path(name, factor):
    import torch
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    w = CASES[name]
    inp = I.make_inputs(w)
    print(f"case {name} factor {factor}", flush=True)
    K = to_device(inp["K"], w.dtype)
    u = torch.from_numpy(inp["u"]).cuda()
    S0, r0, L0 = _select(wc.lib, K, u, w, factor)
    S1, r1, L1 = _select(_streamcheck_lib(), K, u, w, factor)
    assert np.array_equal(r0, r1)
    assert np.array_equal(S0, S1)
    assert np.array_equal(L0.view(np.uint64), L1.view(np.uint64))


@pytest.mark.parametrize("factor", ["f64", "f32"])
def test_streaming_paths_against_oracle(factor):
    import torch
    w = CASES["vit_u3_n2000"]
    inp = I.make_inputs(w)
    print(f"case vit_u3_n2000 factor {factor} vs oracle", flush=True)
    K = to_device(inp["K"], w.dtype)
    u = torch.from_numpy(inp["u"]).cuda()
    S, r_eff, L = _select(_streamcheck_lib(), K, u, w, factor)
    Kd = I.to_f64(inp["K"], w.dtype)
    for unit in (0, 2):
        sel = orc.rpnys_select(Kd[unit, 0], inp["u"][unit], w.r, w.beta, w.tau, w.recentre, factor=factor)
        k = check_pivots(S[unit], int(r_eff[unit]), sel, near=NEAR_TIE if factor == "f64" else NEAR_TIE_F32,
                         context=f"streamcheck {factor} unit {unit}")
        if k < sel.r_eff:
            print(f"unit {unit}: pivots match up to a near tie at draw {k}")
        tol = 1e-9 if factor == "f64" else 2e-6
        assert rel_max(L[unit][:k, :k], sel.L[:k, :k], max(1.0, float(np.abs(sel.L).max()))) < tol

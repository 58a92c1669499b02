"""wildcat_decode_noalloc (the library's static scratch, no allocation)
against wildcat_decode with a caller workspace: the same kernels, so the
outputs must agree bit for bit, on calls in a row with shrinking inputs
(general form with range blocks, general form in one block, one new token),
with no allocation made by the call.  Named to be collected last."""
import numpy as np
import pytest

from nystr_rpcholesky_coreset_amd import inputs as I

from _helpers import to_device

pytestmark = pytest.mark.gpu

C4 = I.WORKLOADS["kvcache_gqa32x8_n32768_d128_r1024_bf16"]
C3 = I.WORKLOADS["latent_b8h8_n4096_d64_r256_bf16"]


def _cache(w):
    import torch
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    inp = I.make_inputs(w, new_tokens=True)
    Q, K, V, Kn, Vn = (to_device(inp[k], w.dtype) for k in ("Q", "K", "V", "K_new", "V_new"))
    u = torch.from_numpy(inp["u"]).cuda()
    _, parts = wc.forward(Q, K, V, u, w.r, w.beta)
    torch.cuda.synchronize()
    return Q, (parts["K_S"], parts["X"], parts["vmin"], parts["vmax"]), Kn, Vn


def test_noalloc_matches_decode_on_calls_in_a_row():
    import torch
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    cases = [I.scaled_workload(C4, q_heads=8, kv_heads=2, n=3000, m=200, r=300, seed=61),   # 4 range blocks
             I.scaled_workload(C3, batch=1, q_heads=2, kv_heads=2, n=1500, m=40, r=100, seed=62),
             I.scaled_workload(C4, q_heads=4, kv_heads=1, n=800, m=1, r=64, seed=63)]      # one new token
    data = [_cache(w) for w in cases]
    outs = [torch.empty(Q.shape, dtype=torch.float32, device="cuda") for Q, _, _, _ in data]
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for (Q, cache, Kn, Vn), w, O in zip(data, cases, outs):
        print(f"decode_noalloc: {w.name}", flush=True)
        wc.decode_noalloc(Q, *cache, Kn, Vn, w.beta, out=O)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    for (Q, cache, Kn, Vn), w, O in zip(data, cases, outs):
        ref = wc.decode(Q, *cache, Kn, Vn, w.beta)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(O.cpu().numpy(), ref.cpu().numpy(), err_msg=w.name)


def test_noalloc_rejects_calls_beyond_its_scratch():
    import ctypes
    import torch
    from nystr_rpcholesky_coreset_amd import wildcat as wc
    w = I.scaled_workload(C4, m=1879)   # 1878 new tokens is the most 32 MiB holds at this shape
    q = wc.QDesc(w.batch, w.q_heads, w.kv_heads, w.m, w.d, w.r, w.beta, wc.WILDCAT_BF16)
    assert wc.decode_workspace_bytes(q) > wc.NOALLOC_SCRATCH_BYTES
    t = torch.empty(16, dtype=torch.float32, device="cuda")
    p = ctypes.c_void_p(t.data_ptr())
    st = wc.lib.wildcat_decode_noalloc(ctypes.byref(q), p, p, p, p, p, p, p, p, None)
    assert st == wc.WILDCAT_ERR_SCRATCH
    q.m = 1878
    assert wc.decode_workspace_bytes(q) <= wc.NOALLOC_SCRATCH_BYTES

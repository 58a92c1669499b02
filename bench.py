"""Throughput of the WildCat hot path on one MI355X.

One step = wildcat_select + wildcat_weights + wildcat_attend over the whole
synthetic workload (inputs already resident in HBM).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--bins B] [--factor f64|f32] [--recentre] [--no-cpu-baseline]
                    [--copy-calibration]

Default workload: KV-cache compression with GQA, 32 query heads over 8 kv
heads, n = 32768 keys, d = 128, r = 1024 pivots per kv head, 64 queries per
query head, bf16 inputs.  --bins B > 1 times the binned variant (B contiguous
key bins per kv head, r/B pivots and block-diagonal Nystroem weights per bin);
the default B = 1 is plain RPNys.  --recentre runs select and weights on the
keys minus their per-unit mean (the pages' CompressKV recentring), with the
same inputs and uniforms.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "kvcache_gqa32x8_n32768_d128_r1024_bf16"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_TFLOPS = 2500.0
MFMA_FP32_TFLOPS = 157.3


def select_bytes(w, e, bins=1, fb=8):
    """Algorithmic HBM bytes of RPNys over all units (and bins): per unit (bin)
    and round i the keys (n*d*e), the new factor column (fb*n), the residual
    diagonal read and write (16n) and the previous factor columns (fb*n*i),
    with n/B keys and r/B rounds per bin; fb = 8 (float64 factor) or 4
    (float32 storage)."""
    U, n, d, r = w.units * bins, w.n // bins, w.d, w.r // bins
    return U * n * (r * (d * e + 16 + fb) + fb * r * (r - 1) // 2)


def contraction_flops(w, bins=1):
    """Matrix-core flops: scores and value products of both contractions
    (with bins, each bin's r/B pivots against its n/B keys)."""
    c1 = w.units * bins * (2 * (w.r // bins) * (w.n // bins) * (2 * w.d + 1))
    c2 = w.q_units * (2 * w.m * w.r * w.d + 2 * w.m * w.r * (w.d + 1))
    return c1, c2


def decode_flops(w):
    """Flops of generation over the cache: query i of every head meets the r
    cached points and new tokens 0..i, each with a score (2d) and a value
    product (2(d+1))."""
    return w.q_units * (4 * w.d + 2) * (w.m * w.r + w.m * (w.m + 1) // 2)


TRAFFIC_SUMMARY = {
    "f64": os.path.join(ROOT, "profiles", "rpc_round_hbm_traffic_kvcache_n32768_r1024.md"),
    "f32": os.path.join(ROOT, "profiles", "rpc_round_hbm_traffic_kvcache_n32768_r1024_f32factor.md"),
}


def read_pinned(path, w):
    """Fields of a committed rocprofv3 summary's machine-readable block
    (`key: value` lines), or None unless the summary was taken on workload w
    with the kernel sources it names hashing as they are now."""
    import hashlib
    try:
        fields = {}
        for line in open(path):
            k, sep, v = line.strip().partition(": ")
            if sep:
                fields[k] = v
        if fields.get("workload") != w.name:
            return None
        h = hashlib.sha256()
        for rel in fields["kernel_sources"].split():
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != fields["kernel_sources_sha256"]:
            return None
        return fields
    except (OSError, KeyError, ValueError):
        return None


def measured_traffic(w, factor="f64"):
    """HBM bytes of one RPNys round measured with rocprofv3 FETCH_SIZE and
    WRITE_SIZE (calibrated on a plain 1 GiB elementwise kernel), read from the
    committed counter summary.  None unless that summary was taken on this
    workload with the select kernel sources as they are now."""
    f = read_pinned(TRAFFIC_SUMMARY[factor], w)
    if f is None or f.get("factor") != factor:
        return None
    try:
        return float(f["traffic_bytes_per_round"])
    except (KeyError, ValueError):
        return None


MFMA_SUMMARY = os.path.join(ROOT, "profiles", "contraction_mfma_kvcache_n32768_r1024.md")


def mfma_evidence(w, bins):
    """Matrix-core rate of the two exp-kernel contractions from the committed
    rocprofv3 summary (kernel-trace durations and MFMA counters), only while
    the contraction sources hash as they did when it was taken."""
    if bins != 1:
        return None
    f = read_pinned(MFMA_SUMMARY, w)
    if f is None:
        return None
    out = {"source": os.path.relpath(MFMA_SUMMARY, ROOT), "peak_tflops": MFMA_BF16_TFLOPS}
    try:
        for ph in ("weights", "attend"):
            us, gflop = float(f[f"{ph}_trace_us"]), float(f[f"{ph}_gflop"])
            tflops = gflop / us * 1e3   # GFLOP per microsecond = PFLOP/s
            out[ph] = {"kernel": f[f"{ph}_kernel"], "trace_us": us, "gflop": gflop,
                       "tflops": tflops, "frac": tflops / MFMA_BF16_TFLOPS,
                       "mfma_busy_frac": float(f[f"{ph}_mfma_busy_frac"])}
    except (KeyError, ValueError):
        return None
    return out


def cpu_baseline(w, inp, bins=1, target_s=20.0, factor="f64"):
    """The oracle as it stands, timed on host cores on a bounded sample: whole
    kv units (select + weights + attend for their query heads), as many as fit
    in about target_s seconds (at least one).  Returns the baseline object and
    the oracle's results per unit: (unit, compress result, {q-head: O})."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from nystr_rpcholesky_coreset_amd import inputs as I
    from oracle import wildcat_oracle as orc

    K = I.to_f64(inp["K"], w.dtype)
    V = I.to_f64(inp["V"], w.dtype)
    Qa = inp["Q"]
    group = w.q_heads // w.kv_heads
    rows = 0
    t0 = time.perf_counter()
    units_done = 0
    results = []
    for uidx in range(w.units):
        b, h = divmod(uidx, w.kv_heads)
        if bins == 1:
            ur = orc.compress_unit(K[b, h], V[b, h], inp["u"][uidx], w.r, w.beta, w.tau, w.recentre, factor)
        else:
            ur = orc.compress_unit_binned(K[b, h], V[b, h], inp["u"][uidx], w.r, bins, w.beta, w.tau, w.recentre,
                                          factor)
        outs = {}
        for hq in range(h * group, (h + 1) * group):
            Q = I.to_f64(Qa[b, hq], w.dtype)
            outs[hq] = orc.plugin_attend(Q, ur.K_S, ur.X, ur.vmin, ur.vmax, w.beta)
            rows += Q.shape[0]
        results.append((uidx, ur, outs))
        units_done += 1
        if time.perf_counter() - t0 > target_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {"value": rows / dt, "unit": "query rows/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{units_done} of {w.units} kv units ({rows} query rows), full n={w.n}, r={w.r}; "
                      f"{dt:.1f} s on {threads} BLAS threads (os.cpu_count()={os.cpu_count()})"}, results


def parity_vs_oracle(w, inp, bins, results, S_gpu, O_gpu):
    """The timed path's last outputs against the oracle units of the CPU
    baseline leg (same inputs and uniforms): pivots matched bit for bit (the
    prefix up to the first difference, per unit or bin), the largest output
    error relative to max|V|, and the oracle's smallest decision margin (how
    close any draw came to a near tie)."""
    import numpy as np

    from nystr_rpcholesky_coreset_amd import inputs as I
    Vmax = float(np.abs(I.to_f64(inp["V"], w.dtype)).max())
    matched = total = 0
    err = 0.0
    margin = float("inf")
    for uidx, ur, outs in results:
        sels = [ur.sel] if bins == 1 else [p.sel for p in ur.bins]
        for k, sel in enumerate(sels):
            Sg = S_gpu[uidx * bins + k]
            m = 0
            while m < sel.r_eff and int(Sg[m]) == int(sel.S[m]):
                m += 1
            matched += m
            total += sel.r_eff
            if sel.margins:
                margin = min(margin, min(sel.margins))
        b = uidx // w.kv_heads
        for hq, Oo in outs.items():
            err = max(err, float(np.abs(O_gpu[b, hq].astype(np.float64) - Oo).max()) / Vmax)
    return {"units": len(results), "pivots_matched": matched, "pivots_total": total, "max_err_rel": err,
            "tol": 2e-3 if w.dtype == "fp32" else 2e-2,
            # smallest distance of a draw from flipping to a neighbouring index, relative to the initial trace
            "min_decision_margin": margin}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--bins", type=int, default=1, help="key bins per kv head (1: plain RPNys)")
    ap.add_argument("--factor", choices=("f64", "f32"), default="f64",
                    help="storage of the RPNys factor (f32: the faster selection; all arithmetic stays fp64)")
    ap.add_argument("--recentre", action="store_true",
                    help="select and weights on the keys minus their per-unit mean")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain elementwise kernel over 1 GiB (1 GiB read + 1 GiB write), "
                         "the reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(units would shard across GPUs with no communication; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from nystr_rpcholesky_coreset_amd import inputs as I
    from nystr_rpcholesky_coreset_amd import wildcat as wc

    w = I.WORKLOADS[args.workload]
    if args.recentre:
        w = I.scaled_workload(w, recentre=True)   # same inputs and uniforms (same seed)
    e = 2 if w.dtype == "bf16" else 4
    inp = I.make_inputs(w, new_tokens=True)
    dev = torch.device("cuda:0")

    def to_dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    Q, K, V = to_dev(inp["Q"]), to_dev(inp["K"]), to_dev(inp["V"])
    u = torch.from_numpy(inp["u"]).to(dev)
    B = args.bins
    if B < 1 or w.n % B or w.r % B:
        print(f"--bins {B} must divide n = {w.n} and r = {w.r}", file=sys.stderr)
        sys.exit(2)
    rb = w.r // B
    Kb, Vb = (wc.bin_view(K, B), wc.bin_view(V, B)) if B > 1 else (K, V)
    ub = u.reshape(w.units * B, rb)
    desc = wc.kv_desc(Kb, rb, w.beta, w.tau, w.recentre, args.factor)
    ws_sel = torch.empty(wc.select_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    ws_w = torch.empty(wc.weights_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        S, r_eff, L = wc.select(Kb, ub, rb, w.beta, w.tau, w.recentre, workspace=ws_sel, factor=args.factor)
        if ev:
            ev[1].record(stream)
        K_S, X, vmin, vmax = wc.weights(Kb, Vb, S, r_eff, L, rb, w.beta, w.tau, w.recentre, workspace=ws_w)
        if B > 1:
            vmin, vmax = wc.merge_value_ranges(vmin, vmax, B)
            K_S = K_S.view(w.batch, w.kv_heads, w.r, w.d)
            X = X.view(w.batch, w.kv_heads, w.r, w.d + 1)
        if ev:
            ev[2].record(stream)
        O = wc.attend(Q, K_S, X, vmin, vmax, w.beta)
        if ev:
            ev[3].record(stream)
        return O, r_eff, (K_S, X, vmin, vmax), S

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        O, r_eff, cache, S_last = step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ph = np.array([[evs[k][j].elapsed_time(evs[k][j + 1]) for j in range(3)] for k in range(args.steps)])
    t_sel, t_wts, t_att = (float(np.median(ph[:, j])) for j in range(3))
    ms_step = wall * 1000.0 / args.steps
    reff = r_eff.cpu().numpy()
    assert np.all(reff == rb), f"early stop on the bench workload: r_eff {reff}"
    assert torch.isfinite(O).all().item()

    # generation over the compressed cache: the m new tokens of every kv head
    # (query row i of each head is token i's query), after the timed steps
    Kn, Vn = to_dev(inp["K_new"]), to_dev(inp["V_new"])
    qd = wc.QDesc(w.batch, w.q_heads, w.kv_heads, w.m, w.d, w.r, float(w.beta), wc._dtype_code(Q))
    ws_d = torch.empty(max(wc.decode_workspace_bytes(qd), 1), dtype=torch.uint8, device=dev)
    Od = torch.empty_like(O)
    wc.decode(Q, *cache, Kn, Vn, w.beta, workspace=ws_d, out=Od)
    torch.cuda.synchronize()
    dev_ms = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        wc.decode(Q, *cache, Kn, Vn, w.beta, workspace=ws_d, out=Od)
        e1.record(stream)
        torch.cuda.synchronize()
        dev_ms.append(e0.elapsed_time(e1))
    t_dec = float(np.median(dev_ms))
    assert torch.isfinite(Od).all().item()
    f_dec = decode_flops(w)
    peak = MFMA_BF16_TFLOPS if w.dtype == "bf16" else MFMA_FP32_TFLOPS
    decode = {"new_tokens": w.m, "ms": t_dec, "rows_per_s": w.query_rows / (t_dec * 1e-3), "gflop": f_dec / 1e9,
              "tflops": f_dec / (t_dec * 1e-3) / 1e12, "peak_tflops": peak,
              "frac": f_dec / (t_dec * 1e-3) / 1e12 / peak}
    # one new token per head (token-by-token generation): query row 0, token 0
    Q1, Kn1, Vn1 = (x[:, :, :1].contiguous() for x in (Q, Kn, Vn))
    qd1 = wc.QDesc(w.batch, w.q_heads, w.kv_heads, 1, w.d, w.r, float(w.beta), wc._dtype_code(Q))
    ws_1 = torch.empty(max(wc.decode_workspace_bytes(qd1), 1), dtype=torch.uint8, device=dev)
    O1 = torch.empty_like(Q1, dtype=torch.float32)
    wc.decode(Q1, *cache, Kn1, Vn1, w.beta, workspace=ws_1, out=O1)
    torch.cuda.synchronize()
    tok_ms = []
    for _ in range(20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        wc.decode(Q1, *cache, Kn1, Vn1, w.beta, workspace=ws_1, out=O1)
        e1.record(stream)
        torch.cuda.synchronize()
        tok_ms.append(e0.elapsed_time(e1))
    assert torch.isfinite(O1).all().item()
    decode["one_token_us"] = float(np.median(tok_ms)) * 1e3
    del ws_d, Od, Kn, Vn, Q1, Kn1, Vn1, ws_1, O1

    if args.copy_calibration:
        a = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    # exact softmax attention on the same GPU (comparator only)
    from torch.nn.attention import SDPBackend, sdpa_kernel
    grp = w.q_heads // w.kv_heads
    Ke = K.repeat_interleave(grp, dim=1).contiguous()
    Ve = V.repeat_interleave(grp, dim=1).contiguous()
    exact = {}
    for name, be in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION),
                     ("math", SDPBackend.MATH)):
        try:
            with sdpa_kernel([be]):
                torch.nn.functional.scaled_dot_product_attention(Q, Ke, Ve, scale=w.beta)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(5):
                    torch.nn.functional.scaled_dot_product_attention(Q, Ke, Ve, scale=w.beta)
                e1.record(stream)
                torch.cuda.synchronize()
                exact = {"backend": name, "ms": e0.elapsed_time(e1) / 5}
                break
        except RuntimeError:
            continue
    del Ke, Ve

    fb = 8 if args.factor == "f64" else 4
    sb = select_bytes(w, e, B, fb)
    per_launch_bytes = sb / rb
    avg_launch_ms = t_sel / rb
    achieved = per_launch_bytes / (avg_launch_ms * 1e-3) / 1e9
    c1, c2 = contraction_flops(w, B)
    rows = w.query_rows
    value = rows / (ms_step * 1e-3)
    line = {
        "metric": "WildCat attention query rows/sec at n=32k,r=1k; RPCholesky ms; %HBM/%MFMA peak",
        "value": value,
        "unit": "query rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64+bf16" if w.dtype == "bf16" else "f64+fp32",
        "data": f"synthetic (seeded '{w.recipe}' recipe with the shapes of the {args.workload} workload)",
        "config": {"workload": args.workload, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "n": w.n, "m": w.m, "d": w.d, "r": w.r, "bins": B, "beta": w.beta, "input_dtype": w.dtype,
                   "factor": args.factor, "recentre": bool(w.recentre)},
        "phases_ms": {"select": t_sel, "weights": t_wts, "attend": t_att},
        "rpcholesky_ms": t_sel,
        "select_hbm_frac": sb / (t_sel * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "contraction_gflop": {"weights": c1 / 1e9, "attend": c2 / 1e9},
        "attend_only_rows_per_s": rows / (t_att * 1e-3),
        "decode": decode,
        "exact_attention_gpu": exact,
        "mfma": mfma_evidence(w, B),
        "roofline": {
            "kernel": "one RPNys round over all units" + (f" and their {B} bins" if B > 1 else "")
                      + ": rpc_step (factor/diagonal stream) + rpc_draw (next pivot) "
                      "of every unit group, the groups overlapped on their own streams",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(w, args.factor) if B == 1 else None,
            "traffic_unit": "bytes per round (rocprofv3 FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000)",
            "note": "achieved counts algorithmic bytes; the keys and the oldest factor columns "
                    "(up to 224 MiB together) take ordinary loads so that they can stay in the "
                    "last-level cache from round to round",
            "bytes_per_launch": per_launch_bytes,
            "avg_launch_ms": avg_launch_ms,
        },
    }
    if not args.no_cpu_baseline:
        S_np, O_np = S_last.cpu().numpy(), O.cpu().numpy()
        line["cpu_baseline"], results = cpu_baseline(w, inp, B, factor=args.factor)
        line["parity"] = parity_vs_oracle(w, inp, B, results, S_np, O_np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

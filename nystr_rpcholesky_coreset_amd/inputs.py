"""Seeded synthetic inputs for the WildCat coreset-attention path.

This module is the one piece shared by the HIP path's tests/bench and the CPU
oracle: it draws Q, K, V and the pivot uniforms u, and holds none of the
method's arithmetic (no kernel evaluations, no sampling rule, no solves).

The five workloads stand in for the workloads measured on the pages (image
classification with a ViT-style first layer, latent attention of an image
generator, KV-cache compression of a GQA language model, and a long-context
sweep); the datasets and trained weights behind those measurements are not
available, so each recipe below reproduces only their shapes and value
statistics.

bf16 inputs are produced by drawing in float64, casting to float32, and then
rounding to bfloat16 with round-to-nearest-even on the bit pattern.  Both the
GPU and the oracle receive exactly these values (the oracle upcasts the bf16
bits to float64 exactly).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "WORKLOAD_ORDER", "make_inputs", "make_uniforms",
    "bf16_bits_from_f32", "f64_from_bf16_bits", "to_f64", "scaled_workload",
]


@dataclass(frozen=True)
class Workload:
    name: str
    recipe: str          # generator name: unit_ball, vit_outliers, mixture16, kv_sinks, sphere2
    batch: int
    q_heads: int
    kv_heads: int
    m: int               # queries per query head
    n: int               # keys per kv head
    d: int               # head dimension
    r: int               # requested coreset size
    beta: float
    dtype: str           # "fp32" or "bf16"
    seed: int            # input seed; the uniforms use seed + 1000
    tau: float = 1.0
    recentre: bool = False

    @property
    def units(self) -> int:
        """Number of (batch, kv-head) units that select/weights process."""
        return self.batch * self.kv_heads

    @property
    def q_units(self) -> int:
        return self.batch * self.q_heads

    @property
    def query_rows(self) -> int:
        return self.batch * self.q_heads * self.m

    @property
    def storage_dtype(self):
        """numpy dtype of the stored inputs: fp32 values or bf16 bit patterns."""
        return np.float32 if self.dtype == "fp32" else np.uint16


WORKLOADS = {
    # Correctness probe: one head, unit-ball rows, fp32.
    "probe_n256_d16_r32_fp32": Workload(
        "probe_n256_d16_r32_fp32", "unit_ball", 1, 1, 1, 256, 256, 16, 32,
        1.0 / math.sqrt(16), "fp32", seed=1001),
    # ViT-style first layer: 56x56 patch grid, 5% outlier keys.
    "vit_b128_n3136_d64_r128_bf16": Workload(
        "vit_b128_n3136_d64_r128_bf16", "vit_outliers", 128, 1, 1, 3136, 3136,
        64, 128, 1.0 / math.sqrt(64), "bf16", seed=1002),
    # Image-generator latent attention: 64x64 latent, Gaussian-mixture Q/K.
    "latent_b8h8_n4096_d64_r256_bf16": Workload(
        "latent_b8h8_n4096_d64_r256_bf16", "mixture16", 8, 8, 8, 4096, 4096,
        64, 256, 1.0 / math.sqrt(64), "bf16", seed=1003),
    # KV-cache compression, GQA 32 query heads over 8 kv heads, sink keys.
    "kvcache_gqa32x8_n32768_d128_r1024_bf16": Workload(
        "kvcache_gqa32x8_n32768_d128_r1024_bf16", "kv_sinks", 1, 32, 8, 64,
        32768, 128, 1024, 1.0 / math.sqrt(128), "bf16", seed=1004),
    # Long-context stress: rows on the sphere of radius 2.
    "longctx_h8_n131072_d128_r2048_bf16": Workload(
        "longctx_h8_n131072_d128_r2048_bf16", "sphere2", 1, 8, 8, 131072,
        131072, 128, 2048, 1.0 / math.sqrt(128), "bf16", seed=1005),
}
WORKLOAD_ORDER = list(WORKLOADS)


def scaled_workload(w: Workload, *, batch=None, q_heads=None, kv_heads=None,
                    m=None, n=None, r=None, seed=None, **kw) -> Workload:
    """The same recipe and dtype at other sizes (for oracle-sized parity cases)."""
    ch = {k: v for k, v in dict(batch=batch, q_heads=q_heads, kv_heads=kv_heads,
                                 m=m, n=n, r=r, seed=seed).items() if v is not None}
    ch.update(kw)
    name = w.name + "@" + ",".join(f"{k}={v}" for k, v in sorted(ch.items()))
    return replace(w, name=name, **ch)


# --------------------------------------------------------------------------
# bf16 bit handling (plain IEEE bit manipulation, no method arithmetic)
# --------------------------------------------------------------------------
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs must be finite.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f64_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bfloat16 bit patterns."""
    f32 = (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return f32.astype(np.float64)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of an input tensor stored as fp32 or bf16 bits."""
    if dtype == "bf16":
        return f64_from_bf16_bits(arr)
    if dtype == "fp32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == "fp32":
        return x32
    return bf16_bits_from_f32(x32)


# --------------------------------------------------------------------------
# Recipes.  Each returns Q [B][Hq][m][d], K and V [B][Hkv][n][d] in float64,
# drawing slice by slice so that the largest workload stays within memory.
# --------------------------------------------------------------------------
def _rows_unit_ball(rng, rows, d):
    x = rng.standard_normal((rows, d))
    nrm = np.sqrt((x * x).sum(axis=1, keepdims=True))
    return x / np.maximum(1.0, nrm)


def _rows_sphere(rng, rows, d, radius):
    z = rng.standard_normal((rows, d))
    return radius * z / np.sqrt((z * z).sum(axis=1, keepdims=True))


def _new_rows(w: Workload, rng, mu, rows, d):
    """Keys and values of `rows` tokens that follow the cached sequence: the
    recipe's per-row law, with the unit's own mixture means; the sink scaling
    of the first positions does not apply (those positions are in the cache)."""
    sd = 1.0 / math.sqrt(d)
    if w.recipe == "unit_ball":
        return _rows_unit_ball(rng, rows, d), _rows_unit_ball(rng, rows, d)
    if w.recipe == "vit_outliers":
        k = sd * rng.standard_normal((rows, d))
        v = sd * rng.standard_normal((rows, d))
        idx = rng.choice(rows, size=int(math.floor(0.05 * rows)), replace=False)
        k[idx] *= 3.0
        return k, v
    if w.recipe == "mixture16":
        lab = rng.integers(0, 16, size=rows)
        return mu[lab] + 0.3 * rng.standard_normal((rows, d)), rng.standard_normal((rows, d))
    if w.recipe == "kv_sinks":
        return sd * rng.standard_normal((rows, d)), sd * rng.standard_normal((rows, d))
    if w.recipe == "sphere2":
        return _rows_sphere(rng, rows, d, 2.0), rng.standard_normal((rows, d))
    raise ValueError(w.recipe)


def _gen(w: Workload, rng, rng_new=None):
    B, Hq, Hkv, m, n, d = w.batch, w.q_heads, w.kv_heads, w.m, w.n, w.d
    group = Hq // Hkv
    Q = np.empty((B, Hq, m, d), dtype=w.storage_dtype)
    K = np.empty((B, Hkv, n, d), dtype=w.storage_dtype)
    V = np.empty((B, Hkv, n, d), dtype=w.storage_dtype)
    if rng_new is not None:
        K_new = np.empty((B, Hkv, m, d), dtype=w.storage_dtype)
        V_new = np.empty((B, Hkv, m, d), dtype=w.storage_dtype)
    sd = 1.0 / math.sqrt(d)
    means = {}
    for b in range(B):
        for h in range(Hkv):
            if w.recipe == "unit_ball":
                k = _rows_unit_ball(rng, n, d)
                v = _rows_unit_ball(rng, n, d)
            elif w.recipe == "vit_outliers":
                k = sd * rng.standard_normal((n, d))
                v = sd * rng.standard_normal((n, d))
                n_out = int(math.floor(0.05 * n))
                idx = rng.choice(n, size=n_out, replace=False)
                k[idx] *= 3.0
            elif w.recipe == "mixture16":
                mu = sd * rng.standard_normal((16, d))
                means[(b, h)] = mu
                lab = rng.integers(0, 16, size=n)
                k = mu[lab] + 0.3 * rng.standard_normal((n, d))
                v = rng.standard_normal((n, d))
            elif w.recipe == "kv_sinks":
                k = sd * rng.standard_normal((n, d))
                v = sd * rng.standard_normal((n, d))
                k[:min(4, n)] *= 8.0
            elif w.recipe == "sphere2":
                k = _rows_sphere(rng, n, d, 2.0)
                v = rng.standard_normal((n, d))
            else:
                raise ValueError(w.recipe)
            K[b, h] = _store(k, w.dtype)
            V[b, h] = _store(v, w.dtype)
            if rng_new is not None:
                kn, vn = _new_rows(w, rng_new, means.get((b, h)), m, d)
                K_new[b, h] = _store(kn, w.dtype)
                V_new[b, h] = _store(vn, w.dtype)
    for b in range(B):
        for h in range(Hq):
            if w.recipe == "unit_ball":
                q = _rows_unit_ball(rng, m, d)
            elif w.recipe in ("vit_outliers", "kv_sinks"):
                q = sd * rng.standard_normal((m, d))
            elif w.recipe == "mixture16":
                mu = means[(b, h // group)]
                lab = rng.integers(0, 16, size=m)
                q = mu[lab] + 0.3 * rng.standard_normal((m, d))
            elif w.recipe == "sphere2":
                q = _rows_sphere(rng, m, d, 2.0)
            else:
                raise ValueError(w.recipe)
            Q[b, h] = _store(q, w.dtype)
    if rng_new is not None:
        return Q, K, V, K_new, V_new
    return Q, K, V


def make_uniforms(w: Workload) -> np.ndarray:
    """Pivot uniforms u[U][r], float64 in [0, 1), from their own seed."""
    return np.random.default_rng(w.seed + 1000).random((w.units, w.r))


def make_inputs(w: Workload, new_tokens: bool = False) -> dict:
    """Q, K, V (fp32 values or bf16 bit patterns as uint16) and uniforms u.

    With new_tokens, also K_new, V_new [batch][kv_heads][m][d]: the keys and
    values of m tokens that follow the n cached ones, drawn from their own
    seed (seed + 2000, so Q, K, V and u are the same either way); query row i
    of every query head is then the query of new token i.
    """
    if w.q_heads % w.kv_heads:
        raise ValueError("q_heads must be a multiple of kv_heads")
    rng = np.random.default_rng(w.seed)
    out = {"u": make_uniforms(w), "workload": w}
    if new_tokens:
        out["Q"], out["K"], out["V"], out["K_new"], out["V_new"] = _gen(w, rng, np.random.default_rng(w.seed + 2000))
    else:
        out["Q"], out["K"], out["V"] = _gen(w, rng)
    return out

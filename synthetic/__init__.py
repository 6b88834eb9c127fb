"""Seeded synthetic inputs for the reduced-matrix-multiplication workloads.

This module only draws random numbers and rounds them to the storage
precision.  It holds none of the method's arithmetic (no norms, no ranking,
no products): both the GPU path's tests and the CPU oracle take their inputs
from here, so nothing here may depend on either of them.

The shapes stand in for the activation/weight products of Llama-3.1-8B and
70B layers that the paper "Reduced Matrix Multiplication: Input-Adaptive
Matrix-Product Reduction for LLM Inference" reduces (Sec. 3.1 writes every
product as Y = A B with A the n x d activation block and B the d x m weight or
intermediate; Sec. 3.3 applies it to projections, MLPs and QK^T).  The real
weights and prompts are not available, so the value distributions imitate
what those layers look like: per-column log-normal activation scales with a
few large outlier columns, Gaussian weights with variance 1/d, and a
SwiGLU-like gated activation for the down projection.

Recipe (one numpy ``Generator(PCG64(seed))`` per configuration, float64 draws
rounded to float32 and then, for bf16 configurations, to bf16 with
round-to-nearest-even).  Draw order within a configuration: column scales,
outlier picks, A row-major, B row-major.  Large arrays are drawn in row
chunks; numpy's ``standard_normal`` consumes its stream element by element,
so chunking does not change the values.

Every array is returned as float32 whose values are exactly representable in
the configuration's storage dtype; ``as_bf16_bits`` gives the raw bf16 bit
patterns for the device side.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import numpy as np

__all__ = [
    "Case",
    "round_to_bf16",
    "as_bf16_bits",
    "lognormal_outlier_activations",
    "gated_activations",
    "gaussian_weights",
    "make_case",
    "make_decode_case",
    "attention_weights",
    "quantize_columns",
    "make_attention_case",
    "make_wq_decode_case",
    "make_wq_case",
    "make_pv_case",
    "CONFIGS",
    "sha256_of",
]

_CHUNK_ELEMS = 1 << 24  # rows per draw chunk are chosen so a chunk holds ~16M values


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    bf16 keeps the upper 16 bits of the IEEE-754 binary32 pattern.  Adding
    0x7FFF plus the lowest kept bit and truncating implements
    round-to-nearest-even for finite values.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def as_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) of float32 values that are bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not exactly representable in bf16")
    return (u >> np.uint32(16)).astype(np.uint16)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == "bf16":
        return round_to_bf16(x32)
    if dtype == "f32":
        return x32
    raise ValueError(f"unknown dtype {dtype!r}")


def _rows_per_chunk(cols: int) -> int:
    return max(1, _CHUNK_ELEMS // max(1, cols))


def _column_scales(rng: np.random.Generator, d: int, n_outliers: int, outlier_factor: float) -> np.ndarray:
    """Log-normal per-column scales c_j = exp(N(0,1)) with a few columns boosted."""
    c = np.exp(rng.standard_normal(d))
    if n_outliers > 0:
        picks = rng.choice(d, size=n_outliers, replace=False)
        c[picks] *= outlier_factor
    return c


def lognormal_outlier_activations(rng: np.random.Generator, n: int, d: int, dtype: str,
                                  n_outliers: int, outlier_factor: float = 20.0,
                                  scales: Optional[np.ndarray] = None):
    """A[i, j] = N(0,1) * c_j.  Returns (A, c)."""
    c = _column_scales(rng, d, n_outliers, outlier_factor) if scales is None else scales
    out = np.empty((n, d), dtype=np.float32)
    step = _rows_per_chunk(d)
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        z = rng.standard_normal((r1 - r0, d))
        out[r0:r1] = _store(z * c[None, :], dtype)
    return out, c


def gated_activations(rng: np.random.Generator, n: int, d: int, dtype: str):
    """Post-SwiGLU-like block: A[i,j] = c_j * N(0,1) * sigmoid(N(0,1)).

    The two normals are independent per element (value draw, then gate draw,
    interleaved per row chunk).  Returns (A, c).
    """
    c = np.exp(rng.standard_normal(d))
    out = np.empty((n, d), dtype=np.float32)
    step = _rows_per_chunk(2 * d)
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        v = rng.standard_normal((r1 - r0, d))
        g = rng.standard_normal((r1 - r0, d))
        out[r0:r1] = _store(c[None, :] * v / (1.0 + np.exp(-g)), dtype)
    return out, c


def gaussian_weights(rng: np.random.Generator, d: int, m: int, dtype: str) -> np.ndarray:
    """B ~ N(0, 1/d), d x m row-major."""
    sigma = 1.0 / math.sqrt(d)
    out = np.empty((d, m), dtype=np.float32)
    step = _rows_per_chunk(m)
    for r0 in range(0, d, step):
        r1 = min(d, r0 + step)
        out[r0:r1] = _store(rng.standard_normal((r1 - r0, m)) * sigma, dtype)
    return out


@dataclasses.dataclass
class Case:
    """One workload instance.

    ``A``/``B`` are float32 arrays holding values exact in ``dtype``.
    For the batched attention case ``A`` is (H_q, L, d_h) queries and ``B`` is
    (H_kv, L, d_h) keys; the product is Q_h K_g^T with g = h // group.
    """
    name: str
    dtype: str
    A: np.ndarray
    B: np.ndarray
    rhos: tuple
    alpha: float = 1.0
    transB: bool = False
    group: int = 1
    scales: Optional[np.ndarray] = None

    @property
    def batched(self) -> bool:
        return self.A.ndim == 3


# name -> (seed, description); sizes are the ones the workloads are quoted at.
CONFIGS = {
    "c1": "tiny fp32: A 64x256 lognormal+4 outliers, B 256x128 ~N(0,1/256), rho 0.5",
    "c2": "8B projection: A 4096x4096 lognormal+0.5% outliers, B 4096x4096, bf16, rho .5/.7/.8/1",
    "c3": "8B MLP down: A 2048x14336 gated lognormal, B 14336x4096, bf16, rho .5/.7/.8/1",
    "c4": "QK^T GQA: Q 32x4096x128, K 8x4096x128, per-(head,dim) lognormal, bf16, rho .5 (+1)",
    "c5": "70B MLP up: A 4096x8192 lognormal+4 outliers, B 8192x28672, bf16, rho .8 (+1)",
    "pv": "PV token axis: P 32x4096x4096 causal attention weights, V 8x4096x128, bf16, rho .5/.8 (+1)",
}


def make_case(name: str, scale: Optional[dict] = None) -> Case:
    """Build configuration ``name`` (c1..c5).

    ``scale`` optionally overrides sizes (keys n, d, m, heads, kv_heads, L,
    dh) to get a smaller instance of the same distribution for quick tests;
    the draw order is unchanged.
    """
    s = dict(scale or {})
    if name == "c1":
        rng = np.random.Generator(np.random.PCG64(1))
        n, d, m = s.get("n", 64), s.get("d", 256), s.get("m", 128)
        A, c = lognormal_outlier_activations(rng, n, d, "f32", n_outliers=min(4, d))
        B = gaussian_weights(rng, d, m, "f32")
        return Case("c1", "f32", A, B, (0.5,), scales=c)
    if name == "c2":
        rng = np.random.Generator(np.random.PCG64(2))
        n, d, m = s.get("n", 4096), s.get("d", 4096), s.get("m", 4096)
        A, c = lognormal_outlier_activations(rng, n, d, "bf16", n_outliers=math.ceil(0.005 * d))
        B = gaussian_weights(rng, d, m, "bf16")
        return Case("c2", "bf16", A, B, (0.5, 0.7, 0.8, 1.0), scales=c)
    if name == "c3":
        rng = np.random.Generator(np.random.PCG64(3))
        n, d, m = s.get("n", 2048), s.get("d", 14336), s.get("m", 4096)
        A, c = gated_activations(rng, n, d, "bf16")
        B = gaussian_weights(rng, d, m, "bf16")
        return Case("c3", "bf16", A, B, (0.5, 0.7, 0.8, 1.0), scales=c)
    if name == "c4":
        rng = np.random.Generator(np.random.PCG64(4))
        hq, hkv = s.get("heads", 32), s.get("kv_heads", 8)
        L, dh = s.get("L", 4096), s.get("dh", 128)
        cq = np.exp(rng.standard_normal((hq, dh)))
        ck = np.exp(rng.standard_normal((hkv, dh)))
        Q = np.empty((hq, L, dh), dtype=np.float32)
        K = np.empty((hkv, L, dh), dtype=np.float32)
        for h in range(hq):
            Q[h], _ = lognormal_outlier_activations(rng, L, dh, "bf16", 0, scales=cq[h])
        for g in range(hkv):
            K[g], _ = lognormal_outlier_activations(rng, L, dh, "bf16", 0, scales=ck[g])
        return Case("c4", "bf16", Q, K, (0.5, 1.0), alpha=1.0 / math.sqrt(dh),
                    transB=True, group=hq // hkv, scales=cq)
    if name == "c5":
        rng = np.random.Generator(np.random.PCG64(5))
        n, d, m = s.get("n", 4096), s.get("d", 8192), s.get("m", 28672)
        A, c = lognormal_outlier_activations(rng, n, d, "bf16", n_outliers=min(4, d))
        B = gaussian_weights(rng, d, m, "bf16")
        return Case("c5", "bf16", A, B, (0.8, 1.0), scales=c)
    raise KeyError(name)


@dataclasses.dataclass
class MLPCase:
    """A gated MLP block: x (n x d) and weights Wg, Wu (d x m), Wd (m x d)."""
    x: np.ndarray
    Wg: np.ndarray
    Wu: np.ndarray
    Wd: np.ndarray
    rhos: tuple


def make_mlp_case(scale: Optional[dict] = None, seed: int = 6) -> MLPCase:
    """Llama-3.1-8B-shaped gated MLP block (n = 2048 tokens, d = 4096,
    m = 14336): x from the 8B projection recipe (log-normal column scales,
    0.5% outlier columns x20), then Wg, Wu ~ N(0, 1/d) and Wd ~ N(0, 1/m), all
    bf16, drawn in that order.  ``scale`` overrides n, d, m."""
    s = dict(scale or {})
    rng = np.random.Generator(np.random.PCG64(seed))
    n, d, m = s.get("n", 2048), s.get("d", 4096), s.get("m", 14336)
    x, _ = lognormal_outlier_activations(rng, n, d, "bf16", n_outliers=math.ceil(0.005 * d))
    Wg = gaussian_weights(rng, d, m, "bf16")
    Wu = gaussian_weights(rng, d, m, "bf16")
    Wd = gaussian_weights(rng, m, d, "bf16")
    return MLPCase(x, Wg, Wu, Wd, (0.5, 0.7, 0.8, 1.0))


def attention_weights(rng: np.random.Generator, Lq: int, Lk: int, dtype: str, sinks: int = 4) -> np.ndarray:
    """One head's causal attention weights: an Lq x Lk row-stochastic matrix
    whose row i spreads over the keys t <= i + (Lk - Lq) (the queries are the
    last Lq positions) and is zero past them.

    Logits are drawn, not computed from queries and keys: a per-key salience
    N(0, 1.5^2) with ``sinks`` leading keys raised by 6 (the attention sinks
    of trained models), a per-head recency decay r log(1 + i' - t) with
    r = exp(N(0, 0.5^2)) and i' = i + Lk - Lq, and N(0, 1) noise per entry;
    each row is then exponentiated relative to its maximum over the visible
    keys and divided by its sum.  Draw order: r, salience, noise (row-major).
    """
    if not 0 < Lq <= Lk:
        raise ValueError("causal weights need 0 < Lq <= Lk (every query sees at least one key)")
    r = float(np.exp(0.5 * rng.standard_normal()))
    sal = 1.5 * rng.standard_normal(Lk)
    sal[:min(sinks, Lk)] += 6.0
    z = rng.standard_normal((Lq, Lk), dtype=np.float32)  # float32 arithmetic from here on
    dist = (np.arange(Lq, dtype=np.int64)[:, None] + (Lk - Lq)) - np.arange(Lk)[None, :]
    decay = np.log1p(np.maximum(dist, 0).astype(np.float32))
    decay *= np.float32(r)
    z += sal.astype(np.float32)[None, :]
    z -= decay
    z[dist < 0] = -np.inf
    z -= z.max(axis=1, keepdims=True)
    np.exp(z, out=z)
    z /= z.sum(axis=1, keepdims=True)
    return _store(z, dtype)


def make_pv_case(scale: Optional[dict] = None, seed: int = 7) -> Case:
    """The value product of a Llama-3.1-8B-shaped attention layer at 4096
    tokens: P (32 query heads, 4096 x 4096 causal attention weights from
    ``attention_weights``) and V (8 key/value heads, 4096 x 128, N(0, 1)),
    grouped-query attention with 4 query heads per V head, all bf16.  Draw
    order: P head by head, then V.  ``scale`` overrides heads, kv_heads, Lq,
    Lk, dv."""
    s = dict(scale or {})
    rng = np.random.Generator(np.random.PCG64(seed))
    hq, hkv = s.get("heads", 32), s.get("kv_heads", 8)
    Lk = s.get("Lk", 4096)
    Lq, dv = s.get("Lq", Lk), s.get("dv", 128)
    P = np.empty((hq, Lq, Lk), dtype=np.float32)
    for h in range(hq):
        P[h] = attention_weights(rng, Lq, Lk, "bf16")
    V = np.empty((hkv, Lk, dv), dtype=np.float32)
    for g in range(hkv):
        V[g] = _store(rng.standard_normal((Lk, dv)), "bf16")
    return Case("pv", "bf16", P, V, (0.5, 0.8, 1.0), group=hq // hkv)


def _e4m3_grid() -> np.ndarray:
    """The 127 non-negative finite OCP FP8 E4M3 values in code order 0..126
    (exponent field 0: m 2^-9; else (8 + m) 2^(e-10); code 127 is NaN)."""
    v = []
    for code in range(127):
        e, m = code >> 3, code & 7
        v.append(m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10))
    return np.asarray(v)


def quantize_columns(B: np.ndarray, fmt: str, rows_per_chunk: int = 1024):
    """Weight-only 8-bit quantization with one scale per column: scale_c =
    max_t |B[t, c]| / Q (Q = 448 for FP8 E4M3, 127 for int8), codes =
    round-to-nearest-even(B / scale_c) on the format's grid.  Returns
    (codes uint8 d x m, scale float32 m).  Deterministic (no draws)."""
    B = np.asarray(B, dtype=np.float32)
    top = 448.0 if fmt == "fp8" else 127.0 if fmt == "int8" else None
    if top is None:
        raise ValueError("fmt must be 'fp8' or 'int8'")
    amax = np.abs(B).max(axis=0).astype(np.float64)
    scale = np.where(amax > 0, amax / top, 1.0).astype(np.float32)
    codes = np.empty(B.shape, dtype=np.uint8)
    grid = _e4m3_grid()
    for r0 in range(0, B.shape[0], rows_per_chunk):
        x = B[r0:r0 + rows_per_chunk].astype(np.float64) / scale.astype(np.float64)[None, :]
        if fmt == "int8":
            codes[r0:r0 + rows_per_chunk] = np.clip(np.rint(x), -127, 127).astype(np.int8).view(np.uint8)
            continue
        ax = np.minimum(np.abs(x), 448.0)
        hi = np.clip(np.searchsorted(grid, ax), 1, 126)
        lo = hi - 1
        dlo, dhi = ax - grid[lo], grid[hi] - ax
        pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
        codes[r0:r0 + rows_per_chunk] = (pick | np.where(np.signbit(x) & (pick > 0), 0x80, 0)).astype(np.uint8)
    return codes, scale


@dataclasses.dataclass
class WQCase:
    """Single-row decode over 8-bit weights: a (1 x d bf16 values), codes
    (d x m uint8), scale (m fp32), fmt."""
    a: np.ndarray
    codes: np.ndarray
    scale: np.ndarray
    fmt: str
    rhos: tuple


def make_wq_decode_case(fmt: str, scale: Optional[dict] = None) -> WQCase:
    """The 70B up-projection decode (a 1 x 8192 from the c5 recipe, B 8192 x
    28672 ~ N(0, 1/8192)) with B quantized per column to ``fmt``.  ``scale``
    overrides n, d, m of the underlying case."""
    base = make_case("c5", dict(scale or {}, n=1) if scale else dict(n=1))
    dec = make_decode_case(base)
    codes, sc = quantize_columns(base.B, fmt)
    return WQCase(dec.A, codes, sc, fmt, (0.8, 1.0))


@dataclasses.dataclass
class WQGemmCase:
    """An activation block times 8-bit weights: A (n x d bf16 values), codes
    (d x m uint8), scale (m fp32), fmt."""
    A: np.ndarray
    codes: np.ndarray
    scale: np.ndarray
    fmt: str
    rhos: tuple


def make_wq_case(fmt: str, scale: Optional[dict] = None) -> WQGemmCase:
    """The 70B up projection (A 4096 x 8192 from the c5 recipe, B 8192 x 28672
    ~ N(0, 1/8192)) with B quantized per column to ``fmt``; ``scale``
    overrides n, d, m of the underlying case (same draw order)."""
    base = make_case("c5", scale)
    codes, sc = quantize_columns(base.B, fmt)
    return WQGemmCase(base.A, codes, sc, fmt, (0.5, 0.8, 1.0))


def make_attention_case(scale: Optional[dict] = None, seed: int = 8):
    """Q and K of the QK^T case (c4: per-(head, dim) log-normal scales) and V
    (H_kv x L x 128) ~ N(0, 1) in bf16 from its own seed; ``scale`` as for c4
    (heads, kv_heads, L, dh) plus dv.  Returns (Q, K, V) float32 arrays."""
    s = dict(scale or {})
    dv = s.pop("dv", 128)
    c = make_case("c4", s)
    rng = np.random.Generator(np.random.PCG64(seed))
    hkv, L = c.B.shape[0], c.B.shape[1]
    V = np.empty((hkv, L, dv), dtype=np.float32)
    for g in range(hkv):
        V[g] = _store(rng.standard_normal((L, dv)), "bf16")
    return c.A, c.B, V


def make_decode_case(case: Case, seed: int = 55) -> Case:
    """n = 1 decode row for a linear case: a fresh N(0,1) row times the same c_j."""
    if case.scales is None or case.A.ndim != 2:
        raise ValueError("decode rows need a linear case with column scales")
    rng = np.random.Generator(np.random.PCG64(seed))
    d = case.A.shape[1]
    a = _store(rng.standard_normal((1, d)) * case.scales[None, :], case.dtype)
    return Case(case.name + "_decode", case.dtype, a, case.B, case.rhos, scales=case.scales)


def sha256_of(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()

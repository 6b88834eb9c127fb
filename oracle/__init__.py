"""CPU oracle for Reduced Matrix Multiplication -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import it, and it imports nothing from them: the two sides share only
the seeded inputs of the ``synthetic`` package.

What it computes (fp64 throughout; C code in ``rmm_oracle.c``), following
"Reduced Matrix Multiplication: Input-Adaptive Matrix-Product Reduction for
LLM Inference":

* ``k_of``       -- |I| = ceil(rho d)                       (Sec. 3.2)
* ``colnorm``    -- s_j = ||A[:, j]||_2                     (Sec. 3.2)
* ``topk``       -- I = TopK(s, k), ties to the lower index, listed ascending
* ``reduced_product`` -- alpha * A[:, I] B[I, :]            (Sec. 3.2, 3.3)
* ``rmm``        -- the four steps in the paper's order
* ``attention_scores`` -- per-Q-head selection applied to the matching GQA
  K head, scaled by 1/sqrt(d_h)                             (Sec. 3.3)
* ``attention_pv`` -- the token-axis product of attention: token scores
  a_t = ||P_h[:, t]||_2 over the query rows, T = TopK(a, ceil(rho L_k)), and
  P_h[:, T] V_g[T, :] with g the GQA key/value head of query head h
  (Sec. 3.2, "Attention", and eq. 2 of App. D.1); no renormalisation of the
  kept weights (reading: the paragraph writes the product over T alone).
* ``attention`` -- attention with reduced scores (Sec. 3.2, "Attention"):
  per query head the dimensions I_h from Q_h's column norms, scores
  alpha Q_h[:, I_h] K_g[:, I_h]^T, the causal mask, a row softmax (fp64,
  maximum subtracted) and the product with V_g.
* ``fp8_e4m3_value``, ``int8_value``, ``decode_wq`` -- single-row decode over
  8-bit weights with per-column scales (W8A16; App. B.6 combines RMM with
  INT8 weight quantization): I = TopK(|a_j|, k), y = scale * a[I] q[I, :],
  with the codes decoded from the OCP FP8 E4M3 definition or as int8.
* ``dequantize``, ``reduced_product_wq`` -- the reduced product of an n-row
  activation block with 8-bit weights (codes and one fp32 scale per column,
  the W8A16 combination of App. B.6): the four steps of ``rmm`` on A and the
  dequantized weights value(q) * scale.
* ``diagnostics`` -- retained energy (App. B.4 / eq. 16), the Prop. 1 bound
  (eq. 12), the Cor. 1 bound (eq. 14) and the relative bound (eq. 17).
* ``gated_mlp`` -- the gated MLP block with RMM on its three projections
  (App. D.1 (ii), eqs. 3-4): Up and Gate select from the model dimension of
  their input x, Down from the intermediate dimension of its input h, each
  set from its own input; the gate is SiLU (reading: the Llama block,
  h = SiLU(x W_gate) * (x W_up), y = h W_down), and h is held in bf16
  between the two stages, as the GPU stores it.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, library routines, brute force or invariants that the paper fixes.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rmm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, no BLAS, no intrinsics)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread",
                        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, f64, i32p = ctypes.c_int64, ctypes.c_double, ctypes.POINTER(ctypes.c_int32)
        f64p, i64p = ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)
        lib.oracle_k.argtypes = [f64, i64]
        lib.oracle_k.restype = i64
        lib.oracle_colnorm.argtypes = [f64p, i64, i64, i64, f64p]
        lib.oracle_colnorm.restype = None
        lib.oracle_topk.argtypes = [f64p, i64, i64, i32p]
        lib.oracle_topk.restype = ctypes.c_int
        lib.oracle_reduced_product.argtypes = [f64p, i64, f64p, i64, i64, i32p, i64, f64, i64p, i64,
                                               f64p, ctypes.c_int]
        lib.oracle_reduced_product.restype = ctypes.c_int
        _lib = lib
    return _lib


def host_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def k_of(rho: float, d: int) -> int:
    """|I| = ceil(rho d); 0 for an invalid rho or d (see rmm_oracle.c)."""
    return int(_load().oracle_k(float(rho), int(d)))


def colnorm(A: np.ndarray) -> np.ndarray:
    """Column L2 norms of a 2-D array, fp64."""
    A64 = _f64(A)
    if A64.ndim != 2:
        raise ValueError("colnorm expects a 2-D array")
    n, d = A64.shape
    s = np.empty(d, dtype=np.float64)
    _load().oracle_colnorm(_ptr(A64, ctypes.c_double), n, d, d, _ptr(s, ctypes.c_double))
    return s


def topk(s: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores (ties -> lower index), ascending, int32."""
    s64 = _f64(s)
    idx = np.empty(int(k), dtype=np.int32)
    if _load().oracle_topk(_ptr(s64, ctypes.c_double), s64.size, int(k), _ptr(idx, ctypes.c_int32)) != 0:
        raise ValueError(f"bad topk arguments d={s64.size} k={k}")
    return idx


def reduced_product(A: np.ndarray, B: np.ndarray, idx: np.ndarray, alpha: float = 1.0,
                    rows: Optional[Sequence[int]] = None, threads: Optional[int] = None) -> np.ndarray:
    """alpha * A[rows][:, idx] @ B[idx, :] by the plain triple loop, fp64."""
    A64, B64 = _f64(A), _f64(B)
    n, d = A64.shape
    d2, m = B64.shape
    if d != d2:
        raise ValueError("inner dimensions differ")
    idx32 = np.ascontiguousarray(idx, dtype=np.int32)
    if idx32.size and (idx32.min() < 0 or idx32.max() >= d):
        raise ValueError("index out of range")
    if rows is None:
        rows_arr = None
        nrows = n
        rows_p = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        if rows_arr.size and (rows_arr.min() < 0 or rows_arr.max() >= n):
            raise ValueError("row out of range")
        nrows = rows_arr.size
        rows_p = _ptr(rows_arr, ctypes.c_int64)
    Y = np.empty((nrows, m), dtype=np.float64)
    rc = _load().oracle_reduced_product(_ptr(A64, ctypes.c_double), d, _ptr(B64, ctypes.c_double), m, m,
                                        _ptr(idx32, ctypes.c_int32), idx32.size, float(alpha), rows_p,
                                        nrows, _ptr(Y, ctypes.c_double), int(threads or host_threads()))
    if rc != 0:
        raise RuntimeError("oracle_reduced_product failed")
    return Y


@dataclasses.dataclass
class Result:
    k: int
    s: np.ndarray      # fp64 column norms
    idx: np.ndarray    # int32, ascending
    Y: Optional[np.ndarray]  # fp64 (rows requested) or None


def rmm(A: np.ndarray, B: Optional[np.ndarray], rho: float, alpha: float = 1.0,
        rows: Optional[Sequence[int]] = None, threads: Optional[int] = None) -> Result:
    """RMM_rho(A, B) in the paper's order: score, TopK, gather, reduced product.

    ``B=None`` stops after the selection.
    """
    d = np.shape(A)[1]
    k = k_of(rho, d)
    if k == 0:
        raise ValueError(f"invalid rho={rho!r} for d={d}")
    s = colnorm(A)
    idx = topk(s, k)
    Y = None if B is None else reduced_product(A, B, idx, alpha, rows, threads)
    return Result(k, s, idx, Y)


def attention_scores(Q: np.ndarray, K: np.ndarray, rho: float, alpha: float,
                     heads: Optional[Sequence[int]] = None, rows: Optional[Sequence[int]] = None,
                     threads: Optional[int] = None, with_product: bool = True):
    """Reduced QK^T per query head with grouped-query attention (Sec. 3.3).

    Q is (H_q, L_q, d_h), K is (H_kv, L_k, d_h).  For head h the score is
    computed from Q_h's column norms only and the same dimensions are taken
    from K head g = h // (H_q / H_kv) (reading: contiguous grouping).  The
    product is alpha * Q_h[:, I] K_g[:, I]^T with alpha = 1/sqrt(d_h).
    Returns a list of Result (one per requested head).
    """
    hq, hkv = Q.shape[0], K.shape[0]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of key heads")
    group = hq // hkv
    out = []
    for h in (range(hq) if heads is None else heads):
        Bt = np.ascontiguousarray(np.asarray(K[h // group], dtype=np.float64).T)  # d_h x L_k
        out.append(rmm(Q[h], Bt if with_product else None, rho, alpha, rows, threads))
    return out


def attention_pv(P: np.ndarray, V: np.ndarray, rho: float, heads: Optional[Sequence[int]] = None,
                 rows: Optional[Sequence[int]] = None, threads: Optional[int] = None):
    """Token-axis RMM of attention's value product, per query head.

    P is (H_q, L_q, L_k) attention weights, V is (H_kv, L_k, d_v).  For head h
    the token scores are the column norms of P_h over its L_q rows, the kept
    set T is their TopK of size ceil(rho L_k), and the output is
    P_h[:, T] V_g[T, :] with g = h // (H_q / H_kv) (Sec. 3.2, "Attention").
    The same four steps as ``rmm`` with A = P_h and B = V_g.  Returns a list
    of Result (one per requested head).
    """
    hq, hkv = P.shape[0], V.shape[0]
    if hq % hkv or P.shape[2] != V.shape[1]:
        raise ValueError("P must be (H_q, L_q, L_k) and V (H_kv, L_k, d_v) with H_kv dividing H_q")
    group = hq // hkv
    return [rmm(P[h], V[h // group], rho, 1.0, rows, threads) for h in (range(hq) if heads is None else heads)]


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, rho: float, causal: bool = True,
              heads: Optional[Sequence[int]] = None, rows: Optional[Sequence[int]] = None,
              threads: Optional[int] = None):
    """softmax(alpha Q_h[:, I] K_g[:, I]^T + M) V_g per query head (Sec. 3.2,
    "Attention"), alpha = 1/sqrt(d_h), I from Q_h's column norms, M = -inf on
    keys after the query's position (queries are the last L_q of L_k
    positions) when ``causal``.  Q (H, Lq, dh), K (Hkv, Lk, dh), V (Hkv, Lk,
    dv).  Returns a list of (idx, O) per requested head, O for the requested
    rows (all by default), fp64."""
    hq, Lq, dh = Q.shape
    hkv, Lk, _ = K.shape
    if hq % hkv or V.shape[:2] != (hkv, Lk):
        raise ValueError("Q (H, Lq, dh), K (Hkv, Lk, dh), V (Hkv, Lk, dv) with Hkv dividing H")
    group = hq // hkv
    alpha = 1.0 / np.sqrt(dh)
    rows_arr = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = []
    for h in (range(hq) if heads is None else heads):
        g = h // group
        Kt = np.ascontiguousarray(np.asarray(K[g], dtype=np.float64).T)
        res = rmm(Q[h], Kt, rho, alpha, rows_arr, threads)   # the reduced scores of the requested rows
        S = res.Y
        if causal:
            S = np.where(np.arange(Lk)[None, :] > (rows_arr + (Lk - Lq))[:, None], -np.inf, S)
        S = S - S.max(axis=1, keepdims=True)
        P = np.exp(S)
        P /= P.sum(axis=1, keepdims=True)
        out.append((res.idx, P @ np.asarray(V[g], dtype=np.float64)))
    return out


def fp8_e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes, fp64: sign bit 7, exponent bits 6-3 with
    bias 7, mantissa bits 2-0; exponent 0 is subnormal (m / 8) 2^-6, the code
    S.1111.111 is NaN and there are no infinities (max 448)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def int8_value(codes: np.ndarray) -> np.ndarray:
    """Values of two's-complement int8 codes stored as bytes, fp64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c >= 128, c - 256, c).astype(np.float64)


def decode_wq(a: np.ndarray, codes: np.ndarray, fmt: str, scale: np.ndarray, rho: float, alpha: float = 1.0,
              threads: Optional[int] = None) -> Result:
    """Single-row decode over 8-bit weights: the n = 1 case of ``rmm`` (the
    scores are |a_j|) with B[t, c] = value(q[t, c]) * scale[c]; returns the
    selection and y = alpha * a[I] B[I, :] (1 x m, fp64)."""
    a2 = np.asarray(a, dtype=np.float64).reshape(1, -1)
    return rmm(a2, dequantize(codes, fmt, scale), rho, alpha, None, threads)


def dequantize(codes: np.ndarray, fmt: str, scale: np.ndarray) -> np.ndarray:
    """The weights that 8-bit codes with one fp32 scale per column stand for:
    B[t, c] = value(q[t, c]) * scale[c], fp64 (``fmt`` "fp8" = OCP E4M3,
    "int8" = two's complement)."""
    values = fp8_e4m3_value(codes) if fmt == "fp8" else int8_value(codes) if fmt == "int8" else None
    if values is None:
        raise ValueError("fmt must be 'fp8' or 'int8'")
    return values * np.asarray(scale, dtype=np.float64)[None, :]


def reduced_product_wq(A: np.ndarray, codes: np.ndarray, fmt: str, scale: np.ndarray, rho: float,
                       alpha: float = 1.0, rows: Optional[Sequence[int]] = None,
                       threads: Optional[int] = None) -> Result:
    """RMM with weights stored as 8-bit codes and per-column fp32 scales
    (weight-only quantization, W8A16; App. B.6 runs RMM on INT8-quantized
    weights): the four steps of ``rmm`` on A (n x d) and the dequantized
    weights B = value(q) * scale (``dequantize``).  The selection depends on
    A only (Sec. 3.2), so it is the same as over unquantized weights; the
    product is alpha * A[:, I] B[I, :] by the triple loop, fp64."""
    B = dequantize(codes, fmt, scale)
    if np.shape(A)[1] != B.shape[0]:
        raise ValueError("A's columns must match the code rows")
    return rmm(A, B, rho, alpha, rows, threads)


def diagnostics(A: np.ndarray, B: np.ndarray, idx: np.ndarray) -> dict:
    """Error-bound quantities of App. E for a selection ``idx``.

    retained_energy = sum_{j in I} s_j^2 / sum_j s_j^2 (App. B.4) = 1 - eps_A;
    prop1 = sum_{j not in I} ||A_j|| ||B_j||          (eq. 12);
    cor1  = ||A[:, Ic]||_F ||B[Ic, :]||_F             (eq. 14);
    rel17 = sqrt(eps_A eps_B)                         (eq. 17).
    """
    a = colnorm(A)
    b = colnorm(np.ascontiguousarray(np.asarray(B, dtype=np.float64).T))  # row norms of B
    keep = np.zeros(a.size, dtype=bool)
    keep[np.asarray(idx)] = True
    drop = ~keep
    ea_tot, eb_tot = float(np.sum(a * a)), float(np.sum(b * b))
    ea_drop, eb_drop = float(np.sum(a[drop] ** 2)), float(np.sum(b[drop] ** 2))
    eps_a = ea_drop / ea_tot if ea_tot > 0 else 0.0
    eps_b = eb_drop / eb_tot if eb_tot > 0 else 0.0
    return {
        "retained_energy": 1.0 - eps_a,
        "eps_A": eps_a,
        "eps_B": eps_b,
        "prop1": float(np.sum(a[drop] * b[drop])),
        "cor1": float(np.sqrt(ea_drop) * np.sqrt(eb_drop)),
        "rel17": float(np.sqrt(eps_a * eps_b)),
        "normA_F": float(np.sqrt(ea_tot)),
        "normB_F": float(np.sqrt(eb_tot)),
    }


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 values rounded to the nearest bf16 (ties to even), returned as fp64.

    bf16 keeps the sign, the 8-bit exponent and 7 stored significand bits of
    binary32, so a normal fp64 value keeps its top 7 of 52 significand bits:
    the low 45 bits are rounded away to nearest, ties to the even neighbour.
    Values beyond the largest finite bf16 become infinities; the normal range
    is what the block produces (no bf16 subnormals are modelled)."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    u = a.view(np.uint64).copy()
    keep_lsb = (u >> np.uint64(45)) & np.uint64(1)
    u = (u + np.uint64((1 << 44) - 1) + keep_lsb) & ~np.uint64((1 << 45) - 1)
    r = u.view(np.float64)
    big = np.abs(r) > 3.3895313892515355e38  # largest finite bf16: (2 - 2^-7) * 2^127
    if np.any(big & np.isfinite(a)):
        r = np.where(big & np.isfinite(a), np.copysign(np.inf, a), r)
    return r


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z), fp64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


@dataclasses.dataclass
class MLPResult:
    idx_in: np.ndarray     # kept model-dimension indices (Up and Gate), int32 ascending
    h: np.ndarray          # SiLU(gate) * up, rounded to bf16 (fp64 values), all rows
    idx_h: np.ndarray      # kept intermediate-dimension indices (Down), int32 ascending
    Y: np.ndarray          # fp64 output rows requested


def gated_mlp(x: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray, rho_in: float, rho_h: float,
              rows: Optional[Sequence[int]] = None, threads: Optional[int] = None) -> MLPResult:
    """The gated MLP block with RMM on Up, Gate and Down (App. D.1 (ii)).

    x is N x d, Wg and Wu are d x m, Wd is m x d (B layouts).  Up and Gate
    take ceil(rho_in d) indices of x's columns (both from the same input, so
    the same set); Down takes ceil(rho_h m) indices of h's columns, h being
    computed for every row because its column norms run over all of them."""
    d = np.shape(x)[1]
    m = np.shape(Wg)[1]
    if np.shape(Wu) != (d, m) or np.shape(Wd)[0] != m:
        raise ValueError("gated_mlp expects Wg, Wu of shape (d, m) and Wd with m rows")
    k_in, k_h = k_of(rho_in, d), k_of(rho_h, m)
    if k_in == 0 or k_h == 0:
        raise ValueError("invalid retention ratio")
    idx_in = topk(colnorm(x), k_in)
    g = reduced_product(x, Wg, idx_in, 1.0, None, threads)
    u = reduced_product(x, Wu, idx_in, 1.0, None, threads)
    h = round_bf16(silu(g) * u)
    idx_h = topk(colnorm(h), k_h)
    Y = reduced_product(h, Wd, idx_h, 1.0, rows, threads)
    return MLPResult(idx_in, h, idx_h, Y)

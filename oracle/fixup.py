"""Boundary-gap fix-up of synthetic activations -- TEST INFRASTRUCTURE ONLY.

The GPU ranks fp32 column norms and the oracle ranks fp64 ones.  Both see the
same stored values, but the two sums round differently, so two columns whose
norms agree to ~1e-7 could swap places at the TopK boundary.  To make the
index-set comparison exact by construction, every test input is nudged until,
for every k the test uses, the k-th largest norm exceeds the (k+1)-th by a
relative gap of at least ``rel_gap`` (1e-3, far above either side's rounding
error): the dropped columns that sit inside the gap are multiplied by 0.99
(then re-rounded to the storage precision) and the norms recomputed, until
every boundary passes.

``enforce_gap_mlp`` does the same for the intermediate h of the gated MLP
block, whose columns are computed: it scales columns of the up-projection
weight, which scales the matching columns of h.

The norms come from this package's own fp64 ``colnorm``.  A single row
(n = 1, decode) needs no fix-up: there s_j = |a_j| is exact in both
precisions and both sides break exact ties toward the lower index.
"""
from __future__ import annotations

from typing import Iterable, Tuple

import numpy as np

from synthetic import round_to_bf16

from . import colnorm


def _boundary_ok(s: np.ndarray, order: np.ndarray, k: int, rel_gap: float) -> Tuple[bool, np.ndarray]:
    sk = s[order[k - 1]]
    sk1 = s[order[k]]
    if sk <= 0.0:
        raise ValueError("k-th largest norm is zero; the gap cannot be opened by scaling")
    if (sk - sk1) / sk >= rel_gap:
        return True, order[:0]
    dropped = order[k:]
    inside = dropped[s[dropped] >= sk * (1.0 - rel_gap)]
    return False, inside


def enforce_gap(A: np.ndarray, ks: Iterable[int], dtype: str, rel_gap: float = 1e-3,
                max_iter: int = 1000) -> Tuple[np.ndarray, int]:
    """Return (A', touched) with every TopK boundary in ``ks`` separated.

    ``A`` is a 2-D float32 array of values exact in ``dtype`` ("bf16" or
    "f32"); a copy is modified.  ``touched`` counts column scalings applied.
    """
    A = np.array(A, dtype=np.float32, copy=True)
    if A.ndim != 2:
        raise ValueError("enforce_gap expects a 2-D array")
    d = A.shape[1]
    ks = sorted({int(k) for k in ks if 0 < int(k) < d})
    touched = 0
    for _ in range(max_iter):
        s = colnorm(A)
        order = np.lexsort((np.arange(d), -s))
        bad = []
        for k in ks:
            ok, inside = _boundary_ok(s, order, k, rel_gap)
            if not ok:
                bad.append(inside)
        if not bad:
            return A, touched
        cols = np.unique(np.concatenate(bad))
        scaled = A[:, cols] * np.float32(0.99)
        A[:, cols] = round_to_bf16(scaled) if dtype == "bf16" else scaled.astype(np.float32)
        touched += cols.size
    raise RuntimeError("gap fix-up did not converge")


def enforce_gap_batched(A: np.ndarray, ks: Iterable[int], dtype: str, rel_gap: float = 1e-3):
    """Apply ``enforce_gap`` to every matrix of a (batch, n, d) array."""
    out = np.empty_like(A, dtype=np.float32)
    touched = 0
    ks = list(ks)
    for b in range(A.shape[0]):
        out[b], t = enforce_gap(A[b], ks, dtype, rel_gap)
        touched += t
    return out, touched


def enforce_gap_mlp(x: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, rho_in: float, ks_h: Iterable[int],
                    rel_gap: float = 1e-3, max_iter: int = 200) -> Tuple[np.ndarray, int]:
    """Open the TopK boundary gaps of the gated block's intermediate h.

    h = bf16(SiLU(x_I Wg_I) * (x_I Wu_I)) is computed, so its column norms
    cannot be spaced by nudging x.  Column c of h is proportional to column c
    of the up product x_I Wu_I, so scaling Wu[:, c] by 0.99 (re-rounded to
    bf16) lowers h's column c by about 1%.  Returns (Wu', touched) such that
    the oracle's h (this package's ``colnorm``, ``topk`` and
    ``reduced_product``, the same steps as ``gated_mlp``) has, for every k in
    ``ks_h``, a relative gap of at least ``rel_gap`` between its k-th and
    (k+1)-th largest column norms.  x and Wg are left as they are.

    This only prepares inputs, so the two products use numpy's fp64 matmul
    instead of the oracle's triple loop (many times faster on a large
    block): the sums differ from the oracle's in the last fp64 bits, which
    moves a bf16 rounding of h, and so a norm, by far less than the gap.
    """
    from . import k_of, round_bf16, silu, topk

    x = np.asarray(x, dtype=np.float32)
    Wu = np.array(Wu, dtype=np.float32, copy=True)
    d, m = Wu.shape
    k_in = k_of(rho_in, d)
    idx_in = topk(colnorm(x), k_in)
    xi = np.ascontiguousarray(x[:, idx_in], dtype=np.float64)
    sg = silu(xi @ np.asarray(Wg, dtype=np.float64)[idx_in])
    u = xi @ Wu[idx_in].astype(np.float64)
    ks = sorted({int(k) for k in ks_h if 0 < int(k) < m})
    touched = 0
    for _ in range(max_iter):
        s = colnorm(round_bf16(sg * u))
        order = np.lexsort((np.arange(m), -s))
        bad = []
        for k in ks:
            ok, inside = _boundary_ok(s, order, k, rel_gap)
            if not ok:
                bad.append(inside)
        if not bad:
            return Wu, touched
        cols = np.unique(np.concatenate(bad))
        Wu[:, cols] = round_to_bf16(Wu[:, cols] * np.float32(0.99))
        u[:, cols] = xi @ Wu[np.ix_(idx_in, cols)].astype(np.float64)
        touched += cols.size
    raise RuntimeError("gap fix-up of h did not converge")

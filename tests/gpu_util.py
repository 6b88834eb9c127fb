"""Helpers for the GPU parity tests: moving seeded inputs to the device and
comparing device results with the oracle.

Tolerances (derived from the arithmetic, written out in ``assert_close``):
  * index sets: bit-exact;
  * fp32 outputs (fp32 FMA accumulation of k terms):
        |Y - Y*| <= (k + 4) * u32 * sum_t |a_t b_t| + u32 * |Y*|,  u32 = 2^-24
    and relative Frobenius error <= 1e-5;
  * bf16 outputs (fp32 accumulation, one bf16 rounding of the result):
        |Y - Y*| <= 2^-8 * |Y*| + (k + 68) * u32 * sum_t |a_t b_t| * (1 + 2^-8) + 2^-133
    (2^-8 is bf16's unit roundoff; the +68 covers split-K partial sums and
    the alpha scaling) and relative Frobenius error <= 1e-2.
The elementwise bound is what catches a dropped or duplicated term: a single
missing product is typically far above it, while the Frobenius tolerance
alone could let it through.
"""
from __future__ import annotations

import numpy as np

import synthetic

U32 = 2.0 ** -24
U16 = 2.0 ** -8


def torch_mod():
    import torch
    return torch


def to_device(x: np.ndarray, dtype: str):
    """float32 array (exact in ``dtype``) -> torch tensor on cuda:0, bit-exact."""
    torch = torch_mod()
    if dtype == "bf16":
        bits = synthetic.as_bf16_bits(np.ascontiguousarray(x)).view(np.int16)
        return torch.from_numpy(bits).to("cuda:0").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")


def to_host(t) -> np.ndarray:
    torch = torch_mod()
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def assert_close(Y_gpu: np.ndarray, Y_ref: np.ndarray, absprod: np.ndarray, k: int, dtype: str, what: str = ""):
    """Elementwise bound plus relative Frobenius tolerance (see module doc)."""
    Y_gpu = np.asarray(Y_gpu, np.float64)
    Y_ref = np.asarray(Y_ref, np.float64)
    assert Y_gpu.shape == Y_ref.shape, (what, Y_gpu.shape, Y_ref.shape)
    assert np.all(np.isfinite(Y_gpu)), f"{what}: non-finite output"
    err = np.abs(Y_gpu - Y_ref)
    if dtype == "bf16":
        bound = U16 * np.abs(Y_ref) + (k + 68) * U32 * absprod * (1 + U16) + 2.0 ** -133
        ftol = 1e-2
    else:
        bound = (k + 4) * U32 * absprod + U32 * np.abs(Y_ref) + 2.0 ** -149
        ftol = 1e-5
    bad = err > bound
    if np.any(bad):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside the bound; worst at {i}: "
                             f"gpu={Y_gpu[i]!r} ref={Y_ref[i]!r} bound={bound[i]!r}")
    den = np.linalg.norm(Y_ref)
    rel = np.linalg.norm(Y_gpu - Y_ref) / (den if den > 0 else 1.0)
    assert rel <= ftol, f"{what}: relative Frobenius error {rel:.3e} > {ftol}"
    return rel


def sample_rows(n: int, count: int, seed: int = 0, tile: int = 256):
    """First, last, tile-boundary and random rows (sorted, unique)."""
    rng = np.random.default_rng(seed)
    rows = {0, n - 1}
    for b in range(tile, n, tile * 3):
        rows.update({b - 1, b})
    rows.update(rng.choice(n, size=min(n, count), replace=False).tolist())
    return sorted(r for r in rows if 0 <= r < n)

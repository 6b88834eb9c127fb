"""Pins of the oracle's gated-MLP block (App. D.1 (ii)) and of its two
helpers, bf16 rounding and SiLU, against library routines and closed forms
(numpy's matmul, norms and stable argsort; the generators' own fp32 -> bf16
rounding, an independent implementation)."""
import numpy as np
import pytest

import oracle
import synthetic


def test_round_bf16_hand_values():
    r = oracle.round_bf16(np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -9, 1 + 2.0 ** -7 + 2.0 ** -8, -(1 + 2.0 ** -8 + 2.0 ** -40),
                                    0.0, -0.0, 2.0 ** -126, 3.0e38, 3.4e38, np.inf, -np.inf]))
    want = [1.0, 1.0, 1 + 2.0 ** -7, 1 + 2.0 ** -6, -(1 + 2.0 ** -7), 0.0, -0.0, 2.0 ** -126, 3.00405527e38, np.inf,
            np.inf, -np.inf]
    assert r[:8].tolist() == want[:8]  # ties to even (1 + 2^-8 -> 1, 1 + 3 * 2^-8 -> 1 + 2^-6); sign kept
    assert abs(r[8] - want[8]) < 1e31 and r[9] == np.inf and np.isposinf(r[10]) and np.isneginf(r[11])
    assert np.signbit(r[6])


def test_round_bf16_matches_the_fp32_route_on_fp32_values():
    x = np.random.default_rng(3).standard_normal(200_000).astype(np.float32) * np.float32(37.5)
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), synthetic.round_to_bf16(x).astype(np.float64))


def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0, -1000.0])
    got = oracle.silu(z)
    assert got[0] == 0.0
    assert got[1] == pytest.approx(1.0 / (1.0 + np.exp(-1.0)), rel=1e-15)
    assert got[2] == pytest.approx(-1.0 / (1.0 + np.e), rel=1e-15)
    assert got[3] == pytest.approx(40.0, rel=1e-15) and abs(got[4]) < 1e-15 and got[5] == 0.0
    # SiLU(z) - SiLU(-z) = z
    t = np.linspace(-6, 6, 101)
    assert np.allclose(oracle.silu(t) - oracle.silu(-t), t, rtol=0, atol=1e-14)


def _block(seed, n=48, d=40, m=56):
    rng = np.random.default_rng(seed)
    x = synthetic.round_to_bf16((rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))).astype(np.float32))
    Wg, Wu = (synthetic.round_to_bf16((rng.standard_normal((d, m)) / np.sqrt(d)).astype(np.float32)) for _ in range(2))
    Wd = synthetic.round_to_bf16((rng.standard_normal((m, d)) / np.sqrt(m)).astype(np.float32))
    return [a.astype(np.float64) for a in (x, Wg, Wu, Wd)]


def _topk_np(A, k):
    s = np.linalg.norm(A, axis=0)
    return np.sort(np.argsort(-s, kind="stable")[:k])


def test_gated_mlp_full_retention_is_the_dense_block():
    x, Wg, Wu, Wd = _block(1)
    r = oracle.gated_mlp(x, Wg, Wu, Wd, 1.0, 1.0)
    h = oracle.round_bf16(oracle.silu(x @ Wg) * (x @ Wu))
    assert np.array_equal(r.h, h)
    assert np.allclose(r.Y, h @ Wd, rtol=1e-12, atol=1e-12)
    assert r.idx_in.tolist() == list(range(x.shape[1])) and r.idx_h.tolist() == list(range(Wg.shape[1]))


@pytest.mark.parametrize("rho_in,rho_h", [(0.5, 0.5), (0.8, 0.3), (0.25, 1.0)])
def test_gated_mlp_stages_follow_their_own_inputs(rho_in, rho_h):
    x, Wg, Wu, Wd = _block(2)
    r = oracle.gated_mlp(x, Wg, Wu, Wd, rho_in, rho_h)
    I = _topk_np(x, oracle.k_of(rho_in, x.shape[1]))
    assert np.array_equal(r.idx_in, I)
    h = oracle.round_bf16(oracle.silu(x[:, I] @ Wg[I]) * (x[:, I] @ Wu[I]))
    assert np.allclose(r.h, h, rtol=0, atol=0) or np.max(np.abs(r.h - h)) <= 2.0 ** -7 * np.max(np.abs(h))
    Ih = _topk_np(r.h, oracle.k_of(rho_h, Wg.shape[1]))
    assert np.array_equal(r.idx_h, Ih)
    assert np.allclose(r.Y, r.h[:, Ih] @ Wd[Ih], rtol=1e-12, atol=1e-12)
    rows = [0, 7, 47]
    assert np.allclose(oracle.gated_mlp(x, Wg, Wu, Wd, rho_in, rho_h, rows=rows).Y, r.Y[rows], rtol=0, atol=0)

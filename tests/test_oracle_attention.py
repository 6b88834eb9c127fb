"""Pins of the oracle's attention with reduced scores (``oracle.attention``:
softmax(alpha Q_h[:, I] K_g[:, I]^T + M) V_g, Sec. 3.2 "Attention") against
library routines and closed forms:

* rho = 1 without a mask is textbook attention written with scipy's softmax
  and numpy's matmul;
* queries with all-zero rows score every key 0, so under the causal mask row
  i is the mean of the V rows it sees (a cumulative sum);
* the first of Lq = Lk causal queries sees key 0 only: O[0] = V[0];
* when Q is zero outside the kept dimensions the reduced scores equal the
  full ones (eq. 13 with A[:, I-bar] = 0), so the output equals rho = 1's;
* query head h reads key/value head h // (H / H_kv).
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_full_rho_without_mask_is_textbook_attention():
    Q, K, V = rand((2, 24, 16), 1), rand((1, 40, 16), 2), rand((1, 40, 8), 3)
    for h, (idx, O) in enumerate(oracle.attention(Q, K, V, 1.0, causal=False)):
        assert np.array_equal(idx, np.arange(16))
        want = softmax(Q[h] @ K[0].T / 4.0, axis=1) @ V[0]
        assert np.allclose(O, want, rtol=1e-12, atol=1e-12)


def test_zero_queries_average_the_visible_values():
    Lq, Lk = 20, 32
    Q = np.zeros((1, Lq, 8))
    Q[0, :, 3] = 0.0
    K, V = rand((1, Lk, 8), 4), rand((1, Lk, 6), 5)
    (idx, O), = oracle.attention(Q, K, V, 0.5, causal=True)
    c = np.cumsum(V[0], axis=0)
    vis = np.arange(Lq) + (Lk - Lq)                      # last visible key of each query
    assert np.allclose(O, c[vis] / (vis + 1.0)[:, None], rtol=1e-12, atol=1e-12)


def test_first_causal_query_sees_key_zero_only():
    Q, K, V = rand((3, 16, 8), 6), rand((3, 16, 8), 7), rand((3, 16, 4), 8)
    for h, (_, O) in enumerate(oracle.attention(Q, K, V, 0.5, causal=True)):
        assert np.array_equal(O[0], V[h][0])


def test_dropped_dimensions_that_are_zero_change_nothing():
    Q = rand((2, 30, 16), 9)
    Q[:, :, [0, 1, 4, 5, 6, 9, 10, 11, 13, 14]] = 0.0    # six dimensions carry Q
    K, V = rand((2, 30, 16), 10), rand((2, 30, 8), 11)
    red = oracle.attention(Q, K, V, 6 / 16, causal=True)
    full = oracle.attention(Q, K, V, 1.0, causal=True)
    for (i1, O1), (_, O2) in zip(red, full):
        assert i1.tolist() == [2, 3, 7, 8, 12, 15]
        assert np.allclose(O1, O2, rtol=1e-12, atol=1e-12)


def test_grouped_query_heads_and_rows():
    Q, K, V = rand((4, 12, 8), 12), rand((2, 12, 8), 13), rand((2, 12, 4), 14)
    out = oracle.attention(Q, K, V, 0.5, causal=False)
    for h, (idx, O) in enumerate(out):
        (i2, O2), = oracle.attention(Q[h:h + 1], K[h // 2:h // 2 + 1], V[h // 2:h // 2 + 1], 0.5, causal=False)
        assert np.array_equal(idx, i2) and np.array_equal(O, O2)
    (_, Or), = oracle.attention(Q, K, V, 0.5, causal=True, heads=[3], rows=[0, 7])
    (_, Oa), = oracle.attention(Q, K, V, 0.5, causal=True, heads=[3])
    assert np.allclose(Or, Oa[[0, 7]], rtol=1e-14, atol=1e-14)
    with pytest.raises(ValueError):
        oracle.attention(Q, K[:1], V, 0.5)

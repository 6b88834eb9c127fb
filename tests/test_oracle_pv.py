"""Pins of the oracle's token-axis attention product (``attention_pv``:
a_t = ||P[:, t]||_2, T = TopK(a, ceil(rho L_k)), P[:, T] V[T, :]; Sec. 3.2,
"Attention") against closed forms that hold for special attention patterns,
and of the attention-weight generator the PV workload draws from.

* Uniform causal attention (row i spreads 1/(i+1) over keys 0..i): the token
  scores are a_t^2 = sum_{i>=t} (i+1)^-2 = psi'(t+1) - psi'(L+1) (trigamma),
  strictly decreasing, so T = {0, .., k-1} and output row i is the running
  mean (1/(i+1)) sum_{t<=min(i,k-1)} V[t] (a cumulative sum, no gather).
* One-hot attention (row i puts weight 1 on key pi(i)): a_t = sqrt(#{i:
  pi(i) = t}), T = the most attended keys (ties to the lower index), and
  output row i is V[pi(i)] when pi(i) is kept, else zero.
* rho = 1 is the full product P V (numpy's matmul).
* Query head h reads V head h // (H_q / H_kv).
"""
import numpy as np
import pytest
from scipy.special import polygamma

import oracle
import synthetic


def uniform_causal(L):
    i = np.arange(L)[:, None]
    t = np.arange(L)[None, :]
    return np.where(t <= i, 1.0 / (i + 1.0), 0.0)


def test_uniform_causal_scores_are_trigamma_differences():
    L = 300
    P = uniform_causal(L)
    a = oracle.colnorm(P)
    want = np.sqrt(polygamma(1, np.arange(L) + 1.0) - polygamma(1, L + 1.0))
    assert np.allclose(a, want, rtol=1e-12, atol=0)
    assert np.all(np.diff(a) < 0)


@pytest.mark.parametrize("rho", [0.1, 0.5, 0.8, 1.0])
def test_uniform_causal_keeps_the_earliest_tokens(rho):
    L, dv = 256, 24
    P = uniform_causal(L)[None]
    V = np.random.default_rng(5).standard_normal((1, L, dv))
    res = oracle.attention_pv(P, V, rho)[0]
    k = oracle.k_of(rho, L)
    assert np.array_equal(res.idx, np.arange(k))
    csum = np.cumsum(V[0], axis=0)                         # sum of V[0..t]
    rows = np.arange(L)
    want = csum[np.minimum(rows, k - 1)] / (rows + 1.0)[:, None]
    assert np.allclose(res.Y, want, rtol=1e-12, atol=1e-12)


def test_one_hot_attention_keeps_the_most_attended_keys():
    rng = np.random.default_rng(8)
    L, dv = 200, 16
    # key t attended by a count that falls with t, with ties (equal counts)
    pi = np.concatenate([np.full(c, t) for t, c in enumerate([30, 25, 25, 20, 20, 20, 15, 15, 10, 10, 5, 5])])
    pi = np.concatenate([pi, rng.integers(20, L, size=L - pi.size)])
    rng.shuffle(pi)
    P = np.zeros((1, L, L))
    P[0, np.arange(L), pi] = 1.0
    V = rng.standard_normal((1, L, dv))
    counts = np.bincount(pi, minlength=L)
    for k in (1, 2, 3, 5, 6, 12):
        res = oracle.attention_pv(P, V, k / L)[0]
        assert res.k == k
        order = sorted(range(L), key=lambda t: (-counts[t], t))   # most attended, ties to the lower index
        assert res.idx.tolist() == sorted(order[:k])
        assert np.allclose(res.s, np.sqrt(counts), rtol=1e-15, atol=0)
        kept = np.isin(pi, res.idx)
        want = np.where(kept[:, None], V[0][pi], 0.0)
        assert np.array_equal(res.Y, want)


def test_full_rho_is_the_plain_value_product():
    rng = np.random.default_rng(9)
    P = rng.random((2, 40, 72))
    V = rng.standard_normal((1, 72, 8))
    for h, res in enumerate(oracle.attention_pv(P, V, 1.0)):
        assert np.array_equal(res.idx, np.arange(72))
        assert np.allclose(res.Y, P[h] @ V[0], rtol=1e-13, atol=1e-13)


def test_grouped_query_heads_read_their_value_head():
    rng = np.random.default_rng(10)
    P = rng.random((4, 16, 32))
    V = rng.standard_normal((2, 32, 8))
    out = oracle.attention_pv(P, V, 0.5)
    for h, res in enumerate(out):
        alone = oracle.attention_pv(P[h:h + 1], V[h // 2:h // 2 + 1], 0.5)[0]
        assert np.array_equal(res.idx, alone.idx) and np.array_equal(res.Y, alone.Y)
    # heads 0 and 1 share V head 0: zeroing V head 1 leaves them unchanged and zeroes heads 2, 3
    V0 = V.copy()
    V0[1] = 0.0
    out0 = oracle.attention_pv(P, V0, 0.5)
    assert np.array_equal(out0[1].Y, out[1].Y) and not np.any(out0[3].Y)
    with pytest.raises(ValueError):
        oracle.attention_pv(P, V[:, :16], 0.5)


def test_attention_weight_generator_is_causal_and_row_stochastic():
    case = synthetic.make_pv_case(dict(heads=2, kv_heads=1, Lq=96, Lk=160, dv=32))
    P, V = case.A, case.B
    assert P.shape == (2, 96, 160) and V.shape == (1, 160, 32) and case.group == 2
    assert np.array_equal(synthetic.round_to_bf16(P), P) and np.array_equal(synthetic.round_to_bf16(V), V)
    assert np.all(P >= 0)
    off = 160 - 96
    for i in (0, 50, 95):
        assert not np.any(P[:, i, i + off + 1:])          # no weight on keys after the query's position
        assert np.all(np.abs(P[:, i].sum(axis=1) - 1.0) < 2 ** -7)
    with pytest.raises(ValueError):
        synthetic.make_pv_case(dict(heads=1, kv_heads=1, Lq=200, Lk=160, dv=8))
    again = synthetic.make_pv_case(dict(heads=2, kv_heads=1, Lq=96, Lk=160, dv=32))
    assert np.array_equal(again.A, P) and np.array_equal(again.B, V)

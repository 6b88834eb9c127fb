"""GPU parity of attention with reduced scores and the softmax fused
(``rmm_attention``, Sec. 3.2 "Attention") against the CPU oracle's
``attention``.

* The kept dimensions of every query head bit for bit (Q's TopK boundary gap
  is opened as for the other products).
* O elementwise within a bound from the arithmetic: the probabilities enter
  the value product rounded to bf16 (relative 2^-9 each) and the scores carry
  fp32 accumulation error, so |O - O*| <= 2^-7 sum_t P*_t |V_t| + 2^-8 |O*|
  (the second term: O's own bf16 rounding); relative Frobenius error <= 1e-2.

Cases span several 128-query tiles with a ragged tail, several 64-key blocks
with a ragged last block, queries at the end of a longer context, both
widths of the kept dimensions (64 and 128), with and without the causal
mask, grouped-query heads, and the 32-head 4096-token layer on sampled rows.
"""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import sample_rows, to_device, to_host
from oracle.fixup import enforce_gap_batched

pytestmark = pytest.mark.gpu
_CACHE = {}


@pytest.fixture(scope="module")
def rmm():
    import input_adaptive_reduced_amd as r
    r.load()
    return r


@pytest.fixture(scope="module")
def torch():
    import torch
    return torch


def case(scale, rho, Lq=None):
    key = (tuple(sorted((scale or {}).items())), rho, Lq)
    if key not in _CACHE:
        Q, K, V = synthetic.make_attention_case(scale)
        if Lq is not None:
            Q = np.ascontiguousarray(Q[:, -Lq:])
        dh = Q.shape[2]
        kk = oracle.k_of(rho, dh)
        if kk < dh:
            Q, _ = enforce_gap_batched(Q, [kk], "bf16")
        _CACHE[key] = (Q, K, V)
    return _CACHE[key]


def check(rmm, torch, Q, K, V, rho, causal, heads=None, rows=None):
    O, idx = rmm.attention(to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"), rho, causal=causal)
    torch.cuda.synchronize()
    got_idx = idx.cpu().numpy()
    k = oracle.k_of(rho, Q.shape[2])
    for h in range(Q.shape[0]):
        assert np.array_equal(got_idx[h], oracle.topk(oracle.colnorm(Q[h]), k)), f"head {h}: kept dimensions differ"
    heads = range(Q.shape[0]) if heads is None else heads
    ref = oracle.attention(Q, K, V, rho, causal=causal, heads=heads, rows=rows)
    group = Q.shape[0] // K.shape[0]
    Lq, Lk = Q.shape[1], K.shape[1]
    r = np.arange(Lq) if rows is None else np.asarray(rows)
    for h, (_, Oref) in zip(heads, ref):
        # P* again, for the bound: the oracle's probabilities of the requested rows
        Kt = np.ascontiguousarray(K[h // group].astype(np.float64).T)
        S = oracle.reduced_product(Q[h], Kt, got_idx[h], 1.0 / np.sqrt(Q.shape[2]), r)
        if causal:
            S = np.where(np.arange(Lk)[None, :] > (r + (Lk - Lq))[:, None], -np.inf, S)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        bound = 2.0 ** -7 * (P @ np.abs(V[h // group].astype(np.float64))) + 2.0 ** -8 * np.abs(Oref) + 1e-30
        Og = to_host(O[h])[r]
        assert np.all(np.isfinite(Og))
        err = np.abs(Og - Oref)
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert np.all(err <= bound), f"head {h} at {worst}: {Og[worst]} vs {Oref[worst]} (bound {bound[worst]})"
        assert np.linalg.norm(Og - Oref) <= 1e-2 * np.linalg.norm(Oref)


CASES = [
    # (scale, Lq or None, rho, causal)
    (dict(heads=4, kv_heads=2, L=256, dh=128), None, 0.5, True),      # two query tiles, four key blocks, k = 64
    (dict(heads=2, kv_heads=1, L=328, dh=64), 200, 0.75, True),      # ragged tiles; queries at the end of the keys
    (dict(heads=4, kv_heads=4, L=300, dh=128), None, 1.0, False),    # every dimension (k = 128), no mask
    (dict(heads=8, kv_heads=2, L=192, dh=128), None, 0.6, True),     # k = 77: 128-wide kept dimensions
    (dict(heads=2, kv_heads=2, L=520, dh=64), 130, 0.5, False),      # no mask, Lq < Lk, ragged last key block
    (dict(heads=2, kv_heads=1, L=40, dh=128), None, 0.5, True),      # one partial key block
]


@pytest.mark.parametrize("scale,Lq,rho,causal", CASES,
                         ids=[f"{c[0]['heads']}x{c[1] or c[0]['L']}x{c[0]['L']}-d{c[0]['dh']}-{c[2]}-{'causal' if c[3] else 'full'}"
                              for c in CASES])
def test_attention_against_oracle(rmm, torch, scale, Lq, rho, causal):
    Q, K, V = case(scale, rho, Lq)
    check(rmm, torch, Q, K, V, rho, causal)


def test_attention_full_size(rmm, torch):
    """The 32-head, 4096-token layer (c4's Q and K, GQA 4), causal, rho = 0.5:
    every head's kept dimensions, three heads' outputs on sampled rows."""
    Q, K, V = case(None, 0.5)
    check(rmm, torch, Q, K, V, 0.5, True, heads=[0, 13, 31], rows=sample_rows(4096, 10, seed=6, tile=128))


@pytest.mark.parametrize("rho,Lq", [(0.5, None), (0.8, None), (0.5, 1100)], ids=["k64", "k128", "k64-Lq1100"])
def test_attention_paired_tiles(rmm, torch, rho, Lq):
    """More causal query tiles than two workgroups per CU hold (64 heads x 9
    tiles): each workgroup takes a long and a short tile of one head, the
    middle tile alone; every row of three heads, both kept widths, and queries
    at the end of a longer context with a ragged last tile."""
    Q, K, V = case(dict(heads=64, kv_heads=16, L=1152, dh=128), rho, Lq)
    check(rmm, torch, Q, K, V, rho, True, heads=[0, 37, 63])


def test_attention_rejects_unsupported(rmm, torch):
    q = torch.zeros((2, 64, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 32, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((1, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rmm.RMMError):
        rmm.attention(q, k, v, 0.5, causal=True)                     # causal with Lq > Lk
    v64 = torch.zeros((1, 64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rmm.RMMError):
        rmm.attention(q, torch.zeros((1, 64, 128), dtype=torch.bfloat16, device="cuda"), v64, 0.5)  # dv != 128


def test_attention_repeatable_and_null_index_output(rmm, torch):
    """Two calls give bit-identical outputs, and the C entry point accepts a
    NULL kept-dimension output (the same O)."""
    import ctypes
    Q, K, V = case(dict(heads=4, kv_heads=2, L=256, dh=128), 0.5)
    q, k, v = to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16")
    O1, i1 = rmm.attention(q, k, v, 0.5, causal=True)
    O2, i2 = rmm.attention(q, k, v, 0.5, causal=True)
    L = rmm.load()
    need = L.rmm_attention_workspace_size(4, 2, 256, 256, 128, 0.5)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    O3 = torch.empty_like(O1)
    st = L.rmm_attention(q.data_ptr(), k.data_ptr(), v.data_ptr(), 4, 2, 256, 256, 128, 128, 0.5, 1, O3.data_ptr(),
                         None, ws.data_ptr(), need, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(O1, O2) and torch.equal(i1, i2) and torch.equal(O1, O3)


def test_attention_tied_norms_at_the_boundary(rmm, torch):
    """Exactly tied column norms across the TopK boundary: every odd column of
    Q repeats the even column before it, so the norms come in equal pairs and
    k = 77 (rho = 0.6 of 128) splits one pair; the lower index must be kept.
    The per-head selection runs inside the K pack here (the pack workgroups
    rank the norms themselves), so this pins its tie order to the oracle's."""
    Q, K, V = synthetic.make_attention_case(dict(heads=4, kv_heads=2, L=320, dh=128))
    # the even columns' gaps opened around pair ranks 38 and 39 (so only the
    # exact pair ties decide the boundary), then every pair made equal
    Qe, _ = enforce_gap_batched(np.ascontiguousarray(Q[:, :, 0::2]), [38, 39], "bf16")
    Q = np.array(Q)
    Q[:, :, 0::2] = Qe
    Q[:, :, 1::2] = Qe
    s = oracle.colnorm(Q[0])
    k = oracle.k_of(0.6, 128)
    order = np.argsort(-s, kind="stable")
    assert s[order[k - 1]] == s[order[k]], "the boundary falls inside a tied pair"
    check(rmm, torch, Q, K, V, 0.6, True)


def test_attention_many_row_chunks(rmm, torch):
    """A query block long enough (33024 rows) that its column norms come in
    more row-chunk partials than the pack's own ranking takes: the separate
    norm+select and pack launches run instead; kept dimensions exact, outputs
    on sampled rows."""
    Q, K, V = case(dict(heads=1, kv_heads=1, L=33024, dh=128), 0.5)
    check(rmm, torch, Q, K, V, 0.5, True, rows=sample_rows(33024, 6, seed=8, tile=128))


@pytest.mark.parametrize("dh,L", [(128, 8192), (64, 16384)], ids=["d128-16chunks", "d64-16chunks"])
def test_attention_sixteen_row_chunks(rmm, torch, dh, L):
    """Queries long enough for 16 row-chunk partials per head (more than the
    K pack's ranking loads ahead of its rows, within what it takes): the
    chunks past the eighth are added in order by the pack's own loop; kept
    dimensions exact, outputs on sampled rows."""
    Q, K, V = case(dict(heads=2, kv_heads=1, L=L, dh=dh), 0.5)
    check(rmm, torch, Q, K, V, 0.5, True, rows=sample_rows(L, 6, seed=9, tile=128))

"""GPU parity of the reduced product over a caller-supplied kept set
(``rmm_matmul_indexed``: the static variant of the selection, Sec. 4
"Baselines" of the paper) against the CPU oracle's product over the same set.

The set is any strictly ascending list, not only a TopK; each route the call
can take is covered (operand-block GEMMs, small tiles, batched entries with a
shared B, B stored transposed, the generic fp32 kernel, the decode GEMV).
Entries that break the precondition are dropped by the library; the rule is
restated here on the host and the product compared over what it keeps."""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_close, sample_rows, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rmm():
    import input_adaptive_reduced_amd as r
    r.load()
    return r


@pytest.fixture(scope="module")
def torch():
    import torch
    return torch


def kept(idx, d):
    """The entries the library keeps: in [0, d) and above every earlier in-range entry."""
    out, run = [], -1
    for v in idx:
        if 0 <= v < d:
            if v > run:
                out.append(v)
            run = max(run, v)
    return np.asarray(out, dtype=np.int32)


def random_set(rng, d, k):
    return np.sort(rng.choice(d, size=k, replace=False)).astype(np.int32)


def operands(rng, n, d, m, dtype):
    A = (rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))).astype(np.float32)
    B = (rng.standard_normal((d, m)) / np.sqrt(d)).astype(np.float32)
    if dtype == "bf16":
        A, B = synthetic.round_to_bf16(A), synthetic.round_to_bf16(B)
    return A, B


CASES = [
    # (n, d, m, dtype, k, note): route the call takes
    (3100, 1504, 4000, "bf16", 1203, "operand blocks, 256x256 tiles"),
    (2050, 4200, 3080, "bf16", 3360, "operand blocks, split K"),
    (300, 520, 264, "bf16", 260, "small tiles"),
    (64, 256, 128, "f32", 100, "generic fp32"),
    (1, 8192, 4096, "bf16", 6554, "decode GEMV"),
    (1, 640, 776, "bf16", 1, "decode, k = 1"),
    (512, 1024, 512, "bf16", 1024, "k = d"),
]


@pytest.mark.parametrize("n,d,m,dtype,k,note", CASES, ids=[c[-1] for c in CASES])
def test_indexed_random_sets(rmm, torch, n, d, m, dtype, k, note):
    rng = np.random.default_rng(n + d + m + k)
    A, B = operands(rng, n, d, m, dtype)
    idx = random_set(rng, d, k)
    Y = rmm.matmul_indexed(to_device(A, dtype), to_device(B, dtype), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    rows = sample_rows(n, 16, seed=3) if n > 1024 else None
    Yh = to_host(Y) if rows is None else to_host(Y)[rows]
    B64 = B.astype(np.float64)
    assert_close(Yh, oracle.reduced_product(A, B64, idx, 1.0, rows),
                 oracle.reduced_product(np.abs(A), np.abs(B64), idx, 1.0, rows), k, dtype, note)


def test_indexed_topk_set_gives_the_selected_product_bit_for_bit(rmm, torch):
    """The oracle's TopK set passed in gives exactly rmm_matmul's output (a
    different route: the norm pass writes A^T there, the pack runs here)."""
    case = synthetic.make_case("c2", dict(n=3104, d=1504, m=4000))
    k = oracle.k_of(0.8, 1504)
    from oracle.fixup import enforce_gap
    A, _ = enforce_gap(case.A, [k], "bf16")
    Ad, Bd = to_device(A, "bf16"), to_device(case.B, "bf16")
    Y, idx = rmm.matmul(Ad, Bd, 0.8)
    assert np.array_equal(idx.cpu().numpy(), oracle.topk(oracle.colnorm(A), k))
    Yi = rmm.matmul_indexed(Ad, Bd, idx)
    torch.cuda.synchronize()
    assert torch.equal(Y, Yi)


def test_indexed_batched_shared_b(rmm, torch):
    rng = np.random.default_rng(11)
    batch, group, n, d, m, k = 4, 2, 384, 640, 512, 320
    A = synthetic.round_to_bf16((rng.standard_normal((batch, n, d)) * np.exp(rng.standard_normal((batch, 1, d))))
                                .astype(np.float32))
    B = synthetic.round_to_bf16((rng.standard_normal((batch // group, d, m)) / 25).astype(np.float32))
    idx = np.stack([random_set(rng, d, k) for _ in range(batch)])
    Y = rmm.matmul_indexed(to_device(A, "bf16"), to_device(B, "bf16"), torch.from_numpy(idx).cuda(), b_group=group)
    torch.cuda.synchronize()
    Yh = to_host(Y)
    for b in range(batch):
        B64 = B[b // group].astype(np.float64)
        assert_close(Yh[b], oracle.reduced_product(A[b], B64, idx[b]),
                     oracle.reduced_product(np.abs(A[b]), np.abs(B64), idx[b]), k, "bf16", f"entry {b}")


def test_indexed_transposed_b(rmm, torch):
    rng = np.random.default_rng(12)
    n, d, m, k = 300, 520, 264, 200
    A, Bdm = operands(rng, n, d, m, "bf16")
    Bt = np.ascontiguousarray(Bdm.T)
    idx = random_set(rng, d, k)
    Y = rmm.matmul_indexed(to_device(A, "bf16"), to_device(Bt, "bf16"), torch.from_numpy(idx).cuda(), transB=True,
                           alpha=0.125)
    torch.cuda.synchronize()
    B64 = Bdm.astype(np.float64)
    assert_close(to_host(Y), oracle.reduced_product(A, B64, idx, 0.125),
                 oracle.reduced_product(np.abs(A), np.abs(B64), idx, 0.125), k, "bf16", "transB")


@pytest.mark.parametrize("n", [700, 1])
def test_indexed_drops_entries_that_break_the_precondition(rmm, torch, n):
    """Out-of-range, repeated and descending entries are dropped; the product
    runs over what remains (host restatement of the rule in ``kept``)."""
    rng = np.random.default_rng(13 + n)
    d, m = 1000, 520
    A, B = operands(rng, n, d, m, "bf16")
    raw = np.array([5, 17, 17, -3, 40, 1000, 39, 41, 2 ** 31 - 1, 999, 998, 7, 1200, 500], dtype=np.int32)
    raw = np.concatenate([raw, random_set(rng, d, 300) + 0])  # ascending tail, partly below earlier entries
    want = kept(raw, d)
    assert 0 < want.size < raw.size
    Y = rmm.matmul_indexed(to_device(A, "bf16"), to_device(B, "bf16"), torch.from_numpy(raw).cuda())
    torch.cuda.synchronize()
    B64 = B.astype(np.float64)
    assert_close(to_host(Y).reshape(n, m), oracle.reduced_product(A, B64, want),
                 oracle.reduced_product(np.abs(A), np.abs(B64), want), raw.size, "bf16", f"n={n}")


def test_kept_rule_on_the_host():
    assert kept([3, 1, 4, 1, 5, 9, 2, 6], 10).tolist() == [3, 4, 5, 9]
    assert kept([-1, 12, 0, 11, 2], 10).tolist() == [0, 2]
    assert kept([], 5).size == 0

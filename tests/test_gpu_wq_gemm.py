"""GPU parity of the reduced product over 8-bit weights for n > 1 rows
(``rmm_matmul_wq``: W8A16, OCP FP8 E4M3 or int8 codes with one fp32 scale
per output column) against the CPU oracle's ``reduced_product_wq``.

* Every code of both formats through the GEMM: a one-hot activation row
  keeps one weight row, whose widened codes come back exactly (bf16 holds
  every 8-bit value), times 1 and 1/2.
* Ragged shapes (tiles partly past n and m, K split over several
  workgroups with the scaled partials summed by the reduce) and the 70B up
  projection 4096 x 8192 x 28672 quantized per column, at rho = 0.8 and 1:
  the kept set bit for bit (the activation block's boundary gap opened as
  for the other products) and Y within the bf16 bound of
  ``gpu_util.assert_close`` computed with the dequantized weights.
"""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_close, sample_rows, to_device, to_host
from oracle.fixup import enforce_gap

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


def check(rmm, torch, A, codes, scale, fmt, rho, alpha=1.0, rows=None, expect_splits=None):
    Ad = to_device(A, "bf16")
    Bq, sc = torch.from_numpy(np.ascontiguousarray(codes)).cuda(), torch.from_numpy(scale).cuda()
    Y, idx = rmm.matmul_wq(Ad, Bq, sc, rho, fmt, alpha=alpha)
    torch.cuda.synchronize()
    ref = oracle.reduced_product_wq(A, codes, fmt, scale, rho, alpha, rows)
    assert np.array_equal(idx.cpu().numpy(), ref.idx), f"{fmt} rho={rho}: kept sets differ"
    W = oracle.dequantize(codes, fmt, scale)
    absprod = oracle.reduced_product(np.abs(A), np.abs(W), ref.idx, abs(alpha), rows)
    Yh = to_host(Y) if rows is None else to_host(Y)[rows]
    return assert_close(Yh, ref.Y, absprod, ref.k, "bf16", f"{fmt} {A.shape} rho={rho}")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_every_code_through_the_gemm(rmm, torch, fmt):
    n, d, m = 16, 64, 256
    codes = np.zeros((d, m), np.uint8)
    codes[3] = np.arange(256, dtype=np.uint8)
    codes[5] = 0x38 if fmt == "fp8" else 1   # a second, smaller column norm, dropped at k = 1
    A = np.zeros((n, d), np.float32)
    A[:, 3] = 1.0
    A[1::2, 3] = 0.5
    A[:, 5] = 0.25
    Y, idx = rmm.matmul_wq(to_device(A, "bf16"), torch.from_numpy(codes).cuda(),
                           torch.ones(m, dtype=torch.float32, device="cuda"), 1 / d, fmt)
    torch.cuda.synchronize()
    assert idx.cpu().numpy().tolist() == [3]
    want = oracle.fp8_e4m3_value(codes[3]) if fmt == "fp8" else oracle.int8_value(codes[3])
    Yh = to_host(Y)
    for r in range(n):
        w = want * A[r, 3]
        assert np.array_equal(np.isnan(Yh[r]), np.isnan(w)), r
        assert np.array_equal(Yh[r][~np.isnan(w)], w[~np.isnan(w)]), r


def small(seed, n, d, m, fmt, ks):
    rng = np.random.default_rng(seed)
    c = np.exp(rng.standard_normal(d))
    A = synthetic.round_to_bf16((rng.standard_normal((n, d)) * c).astype(np.float32))
    A, _ = enforce_gap(A, ks, "bf16")
    W = (rng.standard_normal((d, m)) * np.exp(0.5 * rng.standard_normal(m)) / np.sqrt(d)).astype(np.float32)
    codes, scale = synthetic.quantize_columns(W, fmt)
    return A, codes, scale


SHAPES = [
    # (n, d, m, rhos): ragged row and column tiles; one K range
    (264, 520, 1040, (0.5, 1.0)),
    (512, 1024, 2064, (0.8,)),
    # two tiles and 103 K steps: K split over workgroups, scaled partials summed by the reduce
    (256, 8192, 512, (0.8,)),
]


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("n,d,m,rhos", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}" for s in SHAPES])
def test_ragged_and_split(rmm, torch, fmt, n, d, m, rhos):
    A, codes, scale = small(n + d + m, n, d, m, fmt, [oracle.k_of(r, d) for r in rhos])
    for rho in rhos:
        check(rmm, torch, A, codes, scale, fmt, rho, alpha=0.75)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_full_size_70b_up_projection(rmm, torch, fmt):
    """The 70B up projection 4096 x 8192 x 28672 with per-column-quantized
    weights: every index, 64 rows of Y (first and last of every third
    256-row tile plus random rows)."""
    if fmt not in _CACHE:
        c = synthetic.make_wq_case(fmt)
        A, _ = enforce_gap(c.A, [oracle.k_of(r, c.A.shape[1]) for r in c.rhos], "bf16")
        _CACHE[fmt] = (c, A)
    c, A = _CACHE[fmt]
    rows = sample_rows(A.shape[0], 40, seed=11)
    for rho in (0.8, 1.0):
        check(rmm, torch, A, c.codes, c.scale, fmt, rho, rows=rows)


def test_single_row_is_the_decode_route(rmm, torch):
    """n = 1 through rmm_matmul_wq gives rmm_decode_wq's result, bit for bit."""
    rng = np.random.default_rng(21)
    d, m = 2048, 1024
    a = synthetic.round_to_bf16((rng.standard_normal((1, d)) * np.exp(rng.standard_normal(d))).astype(np.float32))
    codes, scale = synthetic.quantize_columns((rng.standard_normal((d, m)) / 40).astype(np.float32), "fp8")
    Bq, sc = torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda()
    ad = to_device(a, "bf16")
    Y1, i1 = rmm.matmul_wq(ad, Bq, sc, 0.7, "fp8")
    y2, i2 = rmm.decode_wq(ad.view(-1), Bq, sc, 0.7, "fp8")
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(Y1.view(-1), y2)


def test_repeatable_and_unsupported(rmm, torch):
    A, codes, scale = small(3, 128, 256, 512, "int8", [oracle.k_of(0.6, 256)])
    Ad, Bq, sc = to_device(A, "bf16"), torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda()
    Y1, i1 = rmm.matmul_wq(Ad, Bq, sc, 0.6, "int8")
    Y2, i2 = rmm.matmul_wq(Ad, Bq, sc, 0.6, "int8")
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(i1, i2)
    with pytest.raises(rmm.RMMError):       # n % 8 != 0
        rmm.matmul_wq(Ad[:100], Bq, sc, 0.6, "int8")
    with pytest.raises(rmm.RMMError):       # m % 16 != 0
        rmm.matmul_wq(Ad, Bq[:, :504].contiguous(), sc[:504].contiguous(), 0.6, "int8")
    with pytest.raises(ValueError):
        rmm.matmul_wq(Ad, Bq, sc, 0.6, "fp4")

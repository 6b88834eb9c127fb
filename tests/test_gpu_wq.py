"""GPU parity of single-row decode over 8-bit weights (``rmm_decode_wq``,
W8A16 with per-column fp32 scales) against the CPU oracle's ``decode_wq``.

* Every FP8 E4M3 and int8 code through the GPU's conversion: a one-hot row
  keeps exactly one weight row, whose codes come back as bf16 (exact: the
  8-bit values are representable) and must equal the oracle's decoded value.
* The 70B up-projection decode (1 x 8192 by 8192 x 28672, quantized per
  column) and ragged shapes: the kept set bit for bit (|a_j| is exact on both
  sides, ties to the lower index), y within the bf16 error bound of
  ``gpu_util.assert_close`` with the dequantized weights.
"""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_close, to_device, to_host

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


def run(rmm, torch, a, codes, scale, fmt, rho, alpha=1.0, ldb=None):
    d, m = codes.shape
    if ldb is not None and ldb > m:
        padded = np.zeros((d, ldb), np.uint8)
        padded[:, :m] = codes
        Bq = torch.from_numpy(padded).cuda()[:, :m]
    else:
        Bq = torch.from_numpy(np.ascontiguousarray(codes)).cuda()
    y, idx = rmm.decode_wq(to_device(a.reshape(-1), "bf16"), Bq, torch.from_numpy(scale).cuda(), rho, fmt,
                           alpha=alpha)
    torch.cuda.synchronize()
    return to_host(y), idx.cpu().numpy()


def check(rmm, torch, a, codes, scale, fmt, rho, alpha=1.0, ldb=None):
    y, idx = run(rmm, torch, a, codes, scale, fmt, rho, alpha, ldb)
    ref = oracle.decode_wq(a, codes, fmt, scale, rho, alpha)
    assert np.array_equal(idx, ref.idx)
    val = oracle.fp8_e4m3_value(codes) if fmt == "fp8" else oracle.int8_value(codes)
    W = val * scale.astype(np.float64)[None, :]
    absprod = oracle.reduced_product(np.abs(a).reshape(1, -1), np.abs(W), ref.idx, abs(alpha))
    assert_close(y.reshape(1, -1), ref.Y, absprod, ref.k, "bf16", f"{fmt} rho={rho}")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_every_code_decodes_exactly(rmm, torch, fmt):
    d, m = 16, 256
    codes = np.zeros((d, m), np.uint8)
    codes[3] = np.arange(256, dtype=np.uint8)
    a = np.zeros(d, np.float32)
    a[3] = 1.0
    a[5] = 0.5
    y, idx = run(rmm, torch, a, codes, np.ones(m, np.float32), fmt, 1 / d)
    assert idx.tolist() == [3]
    want = oracle.fp8_e4m3_value(codes[3]) if fmt == "fp8" else oracle.int8_value(codes[3])
    y = y.reshape(-1)
    assert np.array_equal(np.isnan(y), np.isnan(want))
    assert np.array_equal(y[~np.isnan(want)], want[~np.isnan(want)])


def small_case(seed, d, m, fmt):
    rng = np.random.default_rng(seed)
    a = synthetic.round_to_bf16((rng.standard_normal(d) * np.exp(rng.standard_normal(d))).astype(np.float32))
    B = (rng.standard_normal((d, m)) / np.sqrt(d)).astype(np.float32)
    codes, scale = synthetic.quantize_columns(B, fmt)
    return a, codes, scale


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("d,m,rho,ldb", [(1000, 48, 0.3, None), (640, 1040, 1 / 640, None), (512, 2064, 1.0, None),
                                         (3000, 4096, 0.7, 4160), (16384, 1024, 0.5, None)])
def test_ragged_shapes(rmm, torch, fmt, d, m, rho, ldb):
    a, codes, scale = small_case(d + m, d, m, fmt)
    check(rmm, torch, a, codes, scale, fmt, rho, alpha=0.5, ldb=ldb)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_full_size_decode(rmm, torch, fmt):
    if fmt not in _CACHE:
        _CACHE[fmt] = synthetic.make_wq_decode_case(fmt)
    c = _CACHE[fmt]
    for rho in c.rhos:
        check(rmm, torch, c.a, c.codes, c.scale, fmt, rho)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("d", [1001, 1004])
def test_row_length_not_a_multiple_of_eight(rmm, torch, fmt, d):
    """d % 8 != 0: the row's last 16-byte piece is read element by element;
    the values stored after the row (huge, they would win the TopK if read)
    are never scored."""
    a, codes, scale = small_case(d, d, 64, fmt)
    a[-2:] = np.float32(64.0)
    trap = np.full(d + 15, 3.0e4, np.float32)
    trap[:d] = a
    ad = to_device(synthetic.round_to_bf16(trap), "bf16")[:d]
    for rho in (0.6, 1.0):
        y, idx = rmm.decode_wq(ad, torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda(), rho, fmt)
        torch.cuda.synchronize()
        ref = oracle.decode_wq(a, codes, fmt, scale, rho)
        assert np.array_equal(idx.cpu().numpy(), ref.idx)
        val = oracle.fp8_e4m3_value(codes) if fmt == "fp8" else oracle.int8_value(codes)
        W = val * scale.astype(np.float64)[None, :]
        absprod = oracle.reduced_product(np.abs(a).reshape(1, -1), np.abs(W), ref.idx)
        assert_close(to_host(y).reshape(1, -1), ref.Y, absprod, ref.k, "bf16", f"{fmt} d={d} rho={rho}")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("d,m,rho", [(1001, 24592, 0.6), (16384, 24576, 0.5), (640, 28672, 1.0)])
def test_selection_in_gemv_decode(rmm, torch, fmt, d, m, rho):
    """Wide 8-bit decodes (m >= 14336): every GEMV workgroup selects from |a|
    itself (no select launch): kept set bit for bit, y within the bound."""
    a, codes, scale = small_case(d * 7 + m, d, m, fmt)
    check(rmm, torch, a, codes, scale, fmt, rho, alpha=0.5)


def test_unsupported_shapes(rmm, torch):
    a = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rmm.RMMError):
        rmm.decode_wq(a, torch.zeros((64, 40), dtype=torch.uint8, device="cuda"),
                      torch.ones(40, dtype=torch.float32, device="cuda"), 0.5)      # m % 16 != 0
    with pytest.raises(ValueError):
        rmm.decode_wq(a, torch.zeros((64, 48), dtype=torch.uint8, device="cuda"),
                      torch.ones(48, dtype=torch.float32, device="cuda"), 0.5, "fp4")


def test_repeatable_and_null_index_output(rmm, torch):
    """Two calls give bit-identical outputs, and the C entry point accepts a
    NULL kept-row output (the same y)."""
    import ctypes
    a, codes, scale = small_case(11, 2048, 1024, "fp8")
    ad = to_device(a, "bf16")
    Bq, sc = torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda()
    y1, i1 = rmm.decode_wq(ad, Bq, sc, 0.6, "fp8")
    y2, i2 = rmm.decode_wq(ad, Bq, sc, 0.6, "fp8")
    L = rmm.load()
    need = L.rmm_decode_wq_workspace_size(2048, 1024, 0.6)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y3 = torch.empty_like(y1)
    st = L.rmm_decode_wq(ad.data_ptr(), Bq.data_ptr(), 0, sc.data_ptr(), 2048, 1024, 1024, 0.6, 1.0, y3.data_ptr(),
                         None, ws.data_ptr(), need, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(y1, y2) and torch.equal(i1, i2) and torch.equal(y1, y3)

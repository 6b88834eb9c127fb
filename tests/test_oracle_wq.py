"""Pins of the 8-bit-weight decode pieces: the oracle's OCP FP8 E4M3 and int8
decoders against torch's own float8_e4m3fn / int8 conversions (library
routines) and hand values of the format, the generator's per-column
quantizer against torch's round-to-nearest-even conversion, and the oracle's
``decode_wq`` against the decoded product written out for a hand case."""
import numpy as np
import pytest

import oracle
import synthetic

torch = pytest.importorskip("torch")


def test_fp8_decoder_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.fp8_e4m3_value(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got)) and np.isnan(got).sum() == 2      # 0x7f, 0xff
    assert np.array_equal(ref[~np.isnan(ref)], got[~np.isnan(got)])


def test_fp8_hand_values():
    v = oracle.fp8_e4m3_value(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3c, 0x7e, 0xfe, 0x80, 0xb8], np.uint8))
    assert v.tolist() == [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.5, 448.0, -448.0, -0.0, -1.0]


def test_int8_decoder():
    codes = np.arange(256, dtype=np.uint8)
    assert np.array_equal(oracle.int8_value(codes), codes.view(np.int8).astype(np.float64))


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_quantizer_matches_torch_rounding(fmt):
    rng = np.random.default_rng(4)
    B = (rng.standard_normal((96, 160)) * np.exp(rng.standard_normal(160))).astype(np.float32)
    B[:, 7] = 0.0                                   # an all-zero column keeps scale 1
    codes, scale = synthetic.quantize_columns(B, fmt, rows_per_chunk=40)
    x = B.astype(np.float64) / scale.astype(np.float64)
    if fmt == "fp8":
        want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.abs(oracle.fp8_e4m3_value(codes)).max() == 448.0
    else:
        want = np.clip(np.rint(x), -127, 127).astype(np.int8).view(np.uint8)
        assert np.abs(oracle.int8_value(codes)).max() == 127.0
    assert np.array_equal(codes, want)
    assert scale[7] == 1.0 and not np.any(codes[:, 7] & 0x7f)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_decode_wq_hand_case(fmt):
    rng = np.random.default_rng(6)
    d, m = 40, 48
    a = synthetic.round_to_bf16(rng.standard_normal(d).astype(np.float32))
    codes = rng.integers(0, 256, size=(d, m), dtype=np.uint8)
    if fmt == "fp8":
        codes[(codes & 0x7f) == 0x7f] = 0x3c                   # no NaN codes
    scale = rng.random(m).astype(np.float32) + 0.5
    res = oracle.decode_wq(a, codes, fmt, scale, 0.5, alpha=0.25)
    k = oracle.k_of(0.5, d)
    order = sorted(range(d), key=lambda j: (-abs(float(a[j])), j))[:k]
    assert res.idx.tolist() == sorted(order)
    val = oracle.fp8_e4m3_value if fmt == "fp8" else oracle.int8_value
    want = np.zeros(m)
    for t in sorted(order):
        want += float(a[t]) * val(codes[t]) * scale.astype(np.float64)
    assert np.allclose(res.Y[0], 0.25 * want, rtol=1e-13, atol=1e-13)

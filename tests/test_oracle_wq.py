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


# ---------------------------------------------------------------- reduced product over 8-bit weights (n > 1)

def _golden_codes(fmt):
    """The hand-worked golden B (entries -1, 0, 1, 2, 3) written as 8-bit
    codes: int8 codes are the integers themselves; the FP8 E4M3 codes are
    0x00 = 0, 0x38 = 1, 0x40 = 2, 0x44 = 3 (1.5 * 2), 0xb8 = -1, from the
    format's definition (bias 7, three mantissa bits)."""
    g = __import__("pins").golden()
    B = np.array(g["B"], dtype=np.int64)
    if fmt == "int8":
        return g, B.astype(np.int8).view(np.uint8)
    table = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, -1: 0xB8}
    return g, np.vectorize(table.get)(B).astype(np.uint8)


def _pin_golden(deq, fmt):
    """The golden case's selections and products by hand, with B held as
    codes: scale 1 gives the golden Y, per-column scales (1/2, 2) scale its
    columns, and the selection does not depend on the weights (Sec. 3.2)."""
    g, codes = _golden_codes(fmt)
    A = np.array(g["A"], dtype=np.float64)
    rp = lambda scale, rho, alpha=1.0: oracle.rmm(A, deq(codes, fmt, scale), rho, alpha)  # noqa: E731
    assert np.array_equal(deq(codes, fmt, np.ones(2)), np.array(g["B"], dtype=np.float64))
    for sel in g["selections"]:
        assert rp(np.ones(2, np.float32), sel["rho"]).idx.tolist() == sel["idx"]
    for p in g["products"]:
        assert np.array_equal(rp(np.ones(2, np.float32), p["rho"], p["alpha"]).Y, np.array(p["Y"], dtype=np.float64))
    Y = rp(np.array([0.5, 2.0], np.float32), 0.5).Y
    assert np.array_equal(Y, np.array([[4, 24], [8, 32]], dtype=np.float64))   # [[8,12],[16,16]] * (1/2, 2)


def _pin_numpy(deq, fmt):
    """rho = 1 is numpy's dense product with the weights dequantized from
    torch's own conversion (a library routine); at rho < 1 the dropped rows
    leave exactly A[:, Ic] B[Ic, :] (eq. 13)."""
    rng = np.random.default_rng(12)
    n, d, m = 24, 96, 40
    A = synthetic.round_to_bf16((rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))).astype(np.float32))
    W = (rng.standard_normal((d, m)) / np.sqrt(d)).astype(np.float32)
    codes, scale = synthetic.quantize_columns(W, fmt)
    if fmt == "fp8":
        vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    else:
        vals = codes.view(np.int8).astype(np.float64)
    B = vals * scale.astype(np.float64)[None, :]
    full = oracle.rmm(A, deq(codes, fmt, scale), 1.0)
    assert np.allclose(full.Y, A.astype(np.float64) @ B, rtol=1e-12, atol=1e-12)
    r = oracle.rmm(A, deq(codes, fmt, scale), 0.6, 0.5)
    keep = np.zeros(d, bool)
    keep[r.idx] = True
    drop = A.astype(np.float64)[:, ~keep] @ B[~keep]
    assert np.allclose(0.5 * (A.astype(np.float64) @ B) - r.Y, 0.5 * drop, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_reduced_product_wq_pins(fmt):
    _pin_golden(oracle.dequantize, fmt)
    _pin_numpy(oracle.dequantize, fmt)
    # reduced_product_wq is rmm over the dequantized weights, and one row of it is decode_wq
    g, codes = _golden_codes(fmt)
    A = np.array(g["A"], dtype=np.float64)
    sc = np.array([0.5, 2.0], np.float32)
    r = oracle.reduced_product_wq(A, codes, fmt, sc, 0.5, alpha=0.25)
    assert np.array_equal(r.Y, 0.25 * np.array([[4, 24], [8, 32]], dtype=np.float64))
    assert np.array_equal(oracle.reduced_product_wq(A[1:2], codes, fmt, sc, 0.5).Y,
                          oracle.decode_wq(A[1], codes, fmt, sc, 0.5).Y)


def _deq_with(value_fn):
    return lambda codes, fmt, scale: value_fn(codes, fmt) * np.asarray(scale, np.float64)[None, :]


DEQ_MUTANTS = {
    # plausible dequantization mistakes: each must fail a pin above
    "scale_per_row": lambda codes, fmt, scale: oracle.dequantize(codes, fmt, np.ones(codes.shape[1])) *
    np.resize(np.asarray(scale, np.float64), codes.shape[0])[:, None],
    "scale_divides": lambda codes, fmt, scale: oracle.dequantize(codes, fmt, 1.0 / np.asarray(scale, np.float64)),
    "fp8_bias_8": _deq_with(lambda c, f: oracle.fp8_e4m3_value(c) / 2 if f == "fp8" else oracle.int8_value(c) / 2),
    "codes_unsigned": _deq_with(lambda c, f: np.asarray(c, np.float64)),
    "mantissa_dropped": _deq_with(lambda c, f: np.sign(oracle.dequantize(c, f, np.ones(c.shape[1]))) *
                                  np.exp2(np.floor(np.log2(np.abs(oracle.dequantize(c, f, np.ones(c.shape[1]))) +
                                                            1e-300)))),
}


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("name", sorted(DEQ_MUTANTS))
def test_dequantize_mutant_is_caught(fmt, name):
    failed = False
    for pin in (_pin_golden, _pin_numpy):
        try:
            pin(DEQ_MUTANTS[name], fmt)
        except (AssertionError, ValueError, IndexError):
            failed = True
    assert failed, f"mutant {name} passed every pin for {fmt}"

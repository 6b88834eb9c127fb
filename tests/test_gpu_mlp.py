"""GPU parity of the gated MLP block with RMM on Up, Gate and Down
(``rmm_gated_mlp``, App. D.1 (ii) of the paper) against ``oracle.gated_mlp``.

* The Up/Gate selection from x's column norms is compared bit for bit (the
  inputs' TopK boundary gap is opened as for the other products).
* h = SiLU(x_I Wg_I) * (x_I Wu_I) in bf16 is compared elementwise with the
  oracle's h within a bound from the arithmetic: fp32 accumulation of the two
  products (as for a reduced GEMM), the fp32 SiLU, and one bf16 rounding on
  each side (two values straddling a rounding boundary land one bf16 step,
  at most 2^-7 relative, apart).
* The Down set is compared bit for bit with the oracle's: the up-projection
  weights are nudged by ``oracle.fixup.enforce_gap_mlp`` so that the
  oracle's own h has a relative gap of at least 1e-3 at the TopK boundary,
  far above the effect of the rare one-step rounding differences in h.
* Y is compared with the oracle's Y (relative Frobenius error) and, element
  by element, with the oracle's Down product over the same set taken from
  the GPU's h (the bound of ``gpu_util.assert_close``), which isolates the
  Down GEMM from the rounding of h.
The block's inputs are the seeded synthetic stand-ins of
``synthetic.make_mlp_case`` (a Llama-3.1-8B-shaped block; smaller sizes for
the quick cases), with the TopK boundary gaps of x and h opened."""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_close, sample_rows, to_device, to_host
from oracle.fixup import enforce_gap, enforce_gap_mlp

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


def block(seed, n, d, m, rho_in, rho_h):
    c = synthetic.make_mlp_case(dict(n=n, d=d, m=m), seed=seed)
    x, _ = enforce_gap(c.x, [oracle.k_of(rho_in, d)], "bf16")
    Wu, _ = enforce_gap_mlp(x, c.Wg, c.Wu, rho_in, [oracle.k_of(rho_h, m)])
    return x, c.Wg, Wu, c.Wd


def check_h(h_gpu, x, Wg, Wu, idx, rows):
    """Elementwise bound for h on the given rows (see the module docstring)."""
    k = idx.size
    xa = np.abs(x)
    g = oracle.reduced_product(x, Wg, idx, 1.0, rows)
    u = oracle.reduced_product(x, Wu, idx, 1.0, rows)
    eg = (k + 68) * 2.0 ** -24 * oracle.reduced_product(xa, np.abs(Wg), idx, 1.0, rows) * (1 + 2.0 ** -8)
    eu = (k + 68) * 2.0 ** -24 * oracle.reduced_product(xa, np.abs(Wu), idx, 1.0, rows) * (1 + 2.0 ** -8)
    h_ref = oracle.round_bf16(oracle.silu(g) * u)
    pre = 1.1 * (np.abs(u) + eu) * eg + (np.abs(oracle.silu(g)) + 1.1 * eg) * eu  # product error before rounding
    pre += 2.0 ** -20 * np.abs(oracle.silu(g) * u)                              # fp32 SiLU and product
    bound = 2.0 ** -7 * np.abs(h_ref) + 2 * pre + 2.0 ** -133
    err = np.abs(h_gpu - h_ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"h at {worst}: {h_gpu[worst]} vs {h_ref[worst]} (bound {bound[worst]})"
    rel = np.linalg.norm(h_gpu - h_ref) / max(np.linalg.norm(h_ref), 1e-300)
    assert rel <= 1e-2, rel


def test_gated_weights_layout(rmm, torch):
    rng = np.random.default_rng(1)
    d, m = 72, 96
    Wg = synthetic.round_to_bf16(rng.standard_normal((d, m)).astype(np.float32))
    Wu = synthetic.round_to_bf16(rng.standard_normal((d, m)).astype(np.float32))
    want = np.empty((d, 2 * m), np.float32)
    for c in range(m // 32):
        want[:, 64 * c:64 * c + 32] = Wg[:, 32 * c:32 * c + 32]
        want[:, 64 * c + 32:64 * c + 64] = Wu[:, 32 * c:32 * c + 32]
    got = to_host(rmm.gated_weights(to_device(Wg, "bf16"), to_device(Wu, "bf16")))
    assert np.array_equal(got, want)
    got_t = to_host(rmm.gated_weights(to_device(np.ascontiguousarray(Wg.T), "bf16"),
                                      to_device(np.ascontiguousarray(Wu.T), "bf16"), transposed=True))
    assert np.array_equal(got_t, want)


MLP = [
    # (n, d, m, rho_in, rho_h, every row checked)
    (512, 1024, 2048, 0.8, 0.7, True),
    (264, 520, 1056, 0.5, 0.5, True),       # ragged tiles in every dimension
    (128, 256, 512, 1.0, 1.0, True),        # every index kept
    (64, 1024, 14336, 0.8, 0.8, True),      # a short block: Down over 4 output tiles in 11 K splits
    (512, 4096, 14336, 0.8, 0.8, False),    # the 8B block on 512 tokens: Down in 8 K splits
    (2048, 4096, 14336, 0.8, 0.8, False),   # the 8B MLP block, sampled rows of h and Y (sets in full)
]


@pytest.mark.parametrize("n,d,m,rho_in,rho_h,full", MLP, ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[3]}-{c[4]}" for c in MLP])
def test_gated_mlp_against_oracle(rmm, torch, n, d, m, rho_in, rho_h, full):
    x, Wg, Wu, Wd = block(6 if (n, d, m) == (2048, 4096, 14336) else n + d + m, n, d, m, rho_in, rho_h)
    Wgu = rmm.gated_weights(to_device(Wg, "bf16"), to_device(Wu, "bf16"))
    Y, idx_in, idx_h, h = rmm.gated_mlp(to_device(x, "bf16"), Wgu, to_device(Wd, "bf16"), rho_in, rho_h,
                                        return_h=True)
    torch.cuda.synchronize()
    rows = None if full else sample_rows(n, 12, seed=9)
    ref = oracle.gated_mlp(x, Wg, Wu, Wd, rho_in, rho_h, rows)
    # both selections bit for bit
    assert np.array_equal(idx_in.cpu().numpy(), ref.idx_in)
    assert np.array_equal(idx_h.cpu().numpy(), ref.idx_h)
    # h elementwise within the bound of the arithmetic
    h_gpu = to_host(h).astype(np.float64)
    check_h(h_gpu if rows is None else h_gpu[rows], x, Wg, Wu, ref.idx_in, rows)
    # Y: end to end against the oracle's block ...
    Yh = to_host(Y) if rows is None else to_host(Y)[rows]
    rel = np.linalg.norm(Yh - ref.Y) / np.linalg.norm(ref.Y)
    assert rel <= 1e-2, f"block output: relative Frobenius error {rel:.3e}"
    # ... and element by element against the oracle's Down product over its set, from the GPU's h
    Wd64 = Wd.astype(np.float64)
    assert_close(Yh, oracle.reduced_product(h_gpu, Wd64, ref.idx_h, 1.0, rows),
                 oracle.reduced_product(np.abs(h_gpu), np.abs(Wd64), ref.idx_h, 1.0, rows), ref.idx_h.size, "bf16",
                 "down projection")


def test_gated_mlp_repeatable_and_h_optional(rmm, torch):
    x, Wg, Wu, Wd = block(5, 256, 512, 1024, 0.7, 0.6)
    xd, Wdd = to_device(x, "bf16"), to_device(Wd, "bf16")
    Wgu = rmm.gated_weights(to_device(Wg, "bf16"), to_device(Wu, "bf16"))
    Y1, i1, j1 = rmm.gated_mlp(xd, Wgu, Wdd, 0.7, 0.6)
    Y2, i2, j2, _ = rmm.gated_mlp(xd, Wgu, Wdd, 0.7, 0.6, return_h=True)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(i1, i2) and torch.equal(j1, j2)


def test_gated_mlp_unsupported_shapes(rmm, torch):
    x = torch.zeros((100, 256), dtype=torch.bfloat16, device="cuda")  # n % 8 != 0
    Wgu = torch.zeros((256, 1024), dtype=torch.bfloat16, device="cuda")
    Wd = torch.zeros((512, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rmm.RMMError):
        rmm.gated_mlp(x, Wgu, Wd, 0.5, 0.5)

"""GPU parity of the token-axis attention product (Sec. 3.2, "Attention"):
token scores a_t = ||P_h[:, t]||_2, T = TopK(a, ceil(rho L_k)) and
O_h = P_h[:, T] V_g[T, :], through ``rmm.matmul`` with A = P (query heads)
and B = V (key/value heads, ``b_group`` query heads each), against the CPU
oracle's ``attention_pv``.

These narrow products (m = d_v <= 128) take the in-kernel column gather
(gemm_gcol_kernel): P is read in place in 64-column windows, so the cases
cover several row tiles with a ragged tail, windows cut by d, output widths
below 128, one kept token, every token kept, the caller-supplied set, and the
full 32-head 4096 x 4096 workload on sampled rows.  The kept sets are compared
bit for bit (the inputs' TopK boundary gap is opened as for the other
products); outputs within the bf16 error bound of ``gpu_util.assert_close``.
"""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_close, sample_rows, to_device, to_host
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


def pv_case(scale, rhos):
    key = (tuple(sorted((scale or {}).items())), tuple(rhos))
    if key not in _CACHE:
        case = synthetic.make_pv_case(scale)
        Lk = case.A.shape[2]
        ks = sorted({oracle.k_of(r, Lk) for r in rhos if oracle.k_of(r, Lk) < Lk})
        P = enforce_gap_batched(case.A, ks, "bf16")[0] if ks else case.A
        _CACHE[key] = (case, P)
    return _CACHE[key]


def check_pv(rmm, torch, case, P, rho, heads=None, rows=None, full_path=False):
    V = case.B
    group = case.group
    Pd, Vd = to_device(P, "bf16"), to_device(V, "bf16")
    assert rmm.plan_info(Pd, Vd, rho, b_group=group, full_path=full_path)["gemm"] == "gcol"
    O, idx = rmm.matmul(Pd, Vd, rho, b_group=group, full_path=full_path)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for h, r in enumerate(oracle.attention_pv(P, V, rho, rows=[0])):
        assert np.array_equal(got[h], r.idx), f"head {h}: kept tokens differ"
    for h in (range(P.shape[0]) if heads is None else heads):
        Vg = V[h // group].astype(np.float64)
        Oh = to_host(O[h])
        if rows is not None:
            Oh = Oh[rows]
        assert_close(Oh, oracle.reduced_product(P[h], Vg, got[h], 1.0, rows),
                     oracle.reduced_product(np.abs(P[h]), np.abs(Vg), got[h], 1.0, rows), got[h].size, "bf16",
                     f"pv head {h} rho={rho}")


PV = [
    # (heads, kv_heads, Lq, Lk, dv, rhos)
    (4, 2, 640, 640, 128, (0.5, 0.8)),     # five row tiles, ten windows
    (2, 1, 300, 520, 40, (0.3, 0.7)),      # ragged row tile, window cut by d, narrow output
    (2, 2, 128, 1024, 64, (0.5,)),         # one row tile, queries at the end of the keys
    (8, 2, 192, 200, 128, (0.9,)),         # d below four windows, ragged row tile
]


@pytest.mark.parametrize("hq,hkv,Lq,Lk,dv,rhos", PV, ids=[f"{c[0]}x{c[2]}x{c[3]}x{c[4]}" for c in PV])
def test_pv_against_oracle(rmm, torch, hq, hkv, Lq, Lk, dv, rhos):
    case, P = pv_case(dict(heads=hq, kv_heads=hkv, Lq=Lq, Lk=Lk, dv=dv), rhos)
    for rho in rhos:
        check_pv(rmm, torch, case, P, rho)


def test_pv_one_and_all_tokens(rmm, torch):
    case, P = pv_case(dict(heads=2, kv_heads=1, Lq=384, Lk=576, dv=128), (1 / 576,))
    check_pv(rmm, torch, case, P, 1 / 576)                   # k = 1
    check_pv(rmm, torch, case, P, 1.0)                       # every token, no norms (identity list)
    check_pv(rmm, torch, case, P, 1.0, full_path=True)       # every token through norms and selection


def test_pv_caller_supplied_tokens(rmm, torch):
    """The static variant: any ascending token list per head, dropped entries
    (out of range, repeated) padded at the tail as the library does."""
    case, P = pv_case(dict(heads=4, kv_heads=2, Lq=512, Lk=768, dv=128), ())
    rng = np.random.default_rng(21)
    idx = np.stack([np.sort(rng.choice(768, size=300, replace=False)).astype(np.int32) for _ in range(4)])
    idx[:, [0, 5]] = idx[:, [1, 6]]        # repeats: the kept entries are those above every earlier one
    check = []
    for row in idx:
        out, run = [], -1
        for v in row:
            if 0 <= v < 768 and v > run:
                out.append(v)
            run = max(run, v)
        check.append(np.asarray(out, np.int32))
    assert all(c.size < 300 for c in check)
    Pd, Vd = to_device(P, "bf16"), to_device(case.B, "bf16")
    O = rmm.matmul_indexed(Pd, Vd, torch.from_numpy(idx).cuda(), b_group=2)
    torch.cuda.synchronize()
    for h in range(4):
        Vg = case.B[h // 2].astype(np.float64)
        assert_close(to_host(O[h]), oracle.reduced_product(P[h], Vg, check[h]),
                     oracle.reduced_product(np.abs(P[h]), np.abs(Vg), check[h]), 300, "bf16", f"indexed head {h}")


def test_pv_single_head_takes_the_gather(rmm, torch):
    """One head (batch 1) takes the narrow gather, not the transposed route."""
    case, P = pv_case(dict(heads=1, kv_heads=1, Lq=1024, Lk=2048, dv=128), (0.5,))
    Pd, Vd = to_device(P[0], "bf16"), to_device(case.B[0], "bf16")
    assert rmm.plan_info(Pd, Vd, 0.5)["gemm"] == "gcol"
    O, idx = rmm.matmul(Pd, Vd, 0.5)
    torch.cuda.synchronize()
    ref = oracle.attention_pv(P, case.B, 0.5, rows=[0])[0]
    assert np.array_equal(idx.cpu().numpy(), ref.idx)
    Vg = case.B[0].astype(np.float64)
    assert_close(to_host(O), oracle.reduced_product(P[0], Vg, ref.idx),
                 oracle.reduced_product(np.abs(P[0]), np.abs(Vg), ref.idx), ref.idx.size, "bf16", "single head")


def test_pv_full_size(rmm, torch):
    """The 32-head, 4096-token value product; every head's kept set, outputs
    of four heads (one per pair of value heads) on sampled rows."""
    case, P = pv_case(None, (0.5,))
    check_pv(rmm, torch, case, P, 0.5, heads=[0, 9, 18, 31], rows=sample_rows(4096, 10, seed=4, tile=128))

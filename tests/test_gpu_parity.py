"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Index sets must match bit for bit; outputs must satisfy the elementwise bound
and relative Frobenius tolerance of ``gpu_util.assert_close``.  Inputs are the
seeded synthetic workloads, with the TopK boundary gaps opened by
``oracle.fixup`` so that fp32 (GPU) and fp64 (oracle) norms rank alike.

Every linear case compares every output element (small instances spanning
several tiles plus a ragged tail; the 256x256 kernels with ragged tiles and
split K; the full-size projections c2 at every rho and c3 at rho = 0.8, in
the launch configuration the benchmark times) except c5, whose whole oracle
product (770 G fp64 multiply-adds, twice over with the error bound's |A||B|)
would take minutes: it compares every index and about 200 output rows: 192
seeded random rows plus the first and last rows of every third 256-row tile.  c3 at the other rho
and the attention cases compare sampled rows as well.
"""
import math

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_close, sample_rows, to_device, to_host
from oracle.fixup import enforce_gap, enforce_gap_batched

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rmm():
    import input_adaptive_reduced_amd as r
    r.load()
    return r


_CACHE = {}


def linear_case(name, scale=None, rhos=None):
    key = (name, tuple(sorted((scale or {}).items())), rhos)
    if key not in _CACHE:
        case = synthetic.make_case(name, scale)
        d = case.A.shape[1]
        ks = [oracle.k_of(r, d) for r in (rhos or case.rhos)]
        A, _ = enforce_gap(case.A, ks, case.dtype)
        _CACHE[key] = (case, A, np.ascontiguousarray(case.B, dtype=np.float64))
    return _CACHE[key]


def check_linear(rmm, case, A, B64, rho, rows=None, full_path=False):
    torch = pytest.importorskip("torch")
    d = A.shape[1]
    k = oracle.k_of(rho, d)
    assert rmm.k_of(rho, d) == k
    ref_idx = oracle.topk(oracle.colnorm(A), k)
    Ad, Bd = to_device(A, case.dtype), to_device(case.B, case.dtype)
    Y, idx = rmm.matmul(Ad, Bd, rho, full_path=full_path)
    torch.cuda.synchronize()
    got_idx = idx.cpu().numpy()
    assert np.array_equal(got_idx, ref_idx), f"{case.name} rho={rho}: index sets differ"
    Yh = to_host(Y)
    if rows is not None:
        Yh = Yh[rows]
    Y_ref = oracle.reduced_product(A, B64, ref_idx, 1.0, rows)
    absprod = oracle.reduced_product(np.abs(A), np.abs(B64), ref_idx, 1.0, rows)
    return assert_close(Yh, Y_ref, absprod, k, case.dtype, f"{case.name} rho={rho}")


SMALL = [
    ("c1", None),
    ("c2", dict(n=300, d=520, m=264)),
    ("c2", dict(n=512, d=1024, m=512)),
    ("c3", dict(n=256, d=1792, m=512)),
    ("c5", dict(n=130, d=640, m=776)),
]


@pytest.mark.parametrize("name,scale", SMALL, ids=[f"{n}-{s}" for n, s in SMALL])
def test_small_linear_all_rho(rmm, name, scale):
    case, A, B64 = linear_case(name, scale)
    for rho in case.rhos:
        check_linear(rmm, case, A, B64, rho)
    check_linear(rmm, case, A, B64, 1.0, full_path=True)


RAGGED = [
    # (scale, rho, kernel, split K, full path): the 256x256 kernels with
    # ragged n and m not a multiple of 256.  With n % 8 != 0 the operand-block
    # kernels run (A packed); bdma rounds each split's K steps up to a
    # multiple of three with zero steps: 104 -> 105 steps at d = 8200, and
    # 16 -> 18 in the last of two splits at d = 4200, rho = 0.5.
    (dict(n=3100, d=1504, m=4000), 0.5, "bdma", False, False),
    (dict(n=3100, d=8200, m=4000), 0.8, "bdma", False, False),
    (dict(n=2050, d=4200, m=3080), 0.5, "bdma", True, False),
    (dict(n=2050, d=4200, m=3080), 0.8, "bdma", True, False),
    (dict(n=3100, d=1504, m=4000), 0.8, "adirect", False, False),
    (dict(n=2050, d=4200, m=3080), 0.48, "adirect", True, False),
    # rho = 1 (the identity set, A packed through the index list 0..d-1)
    (dict(n=3100, d=1536, m=4000), 1.0, "bdma", False, False),
    (dict(n=2050, d=4224, m=3080), 1.0, "adirect", True, False),
    # n % 8 == 0: the norm pass writes A^T and both operands are gathered by
    # rows (no pack); the last row tile is partly past n, the last column
    # tile partly past m; two and three K splits (the last split of the
    # rho = 0.5 case runs 16 of 18 steps); the full path at rho = 1
    (dict(n=3104, d=1504, m=4000), 0.5, "tdma", False, False),
    (dict(n=3104, d=8200, m=4000), 0.8, "tdma", False, False),
    (dict(n=2048, d=4200, m=3080), 0.5, "tdma", True, False),
    (dict(n=2048, d=4200, m=3080), 0.8, "tdma", True, False),
    (dict(n=3104, d=1536, m=4000), 1.0, "tdma", False, True),
]


@pytest.mark.parametrize("scale,rho,kernel,split,full", RAGGED,
                         ids=[f"{k}{'-splitk' if s else ''}-d{c['d']}-rho{r}{'-full' if f else ''}"
                              for c, r, k, s, f in RAGGED])
def test_ragged_large_tiles(rmm, scale, rho, kernel, split, full):
    # every output element, including the ragged last row and column tiles
    # and, with split K, every split's partial sums through the reduce
    torch = pytest.importorskip("torch")
    case, A, B64 = linear_case("c2", scale, rhos=(rho,))
    Am = torch.empty(A.shape, dtype=torch.bfloat16, device="meta")
    Bm = torch.empty(case.B.shape, dtype=torch.bfloat16, device="meta")
    info = rmm.plan_info(Am, Bm, rho, full_path=full)
    assert info["gemm"] == kernel and (info["splits"] > 1) == split, info
    check_linear(rmm, case, A, B64, rho, rows=None, full_path=full)


def plan_of(rmm, case, rho):
    torch = pytest.importorskip("torch")
    Am = torch.empty(case.A.shape, dtype=torch.bfloat16, device="meta")
    Bm = torch.empty(case.B.shape, dtype=torch.bfloat16, device="meta")
    return rmm.plan_info(Am, Bm, rho)


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_full_size_linear_every_row(rmm, name):
    """The 8B-shaped projections at full size, every element of Y: c2 at
    rho = 0.5, 0.7, 0.8, 1.0 (the A^T route; rho = 1 takes the shortcut) and
    c3 at rho = 0.8 (the A^T route with split K); c3's other rho on rows."""
    case, A, B64 = linear_case(name)
    for rho in case.rhos:
        if rho < 1.0:
            assert plan_of(rmm, case, rho)["gemm"] == "tdma"
        every = name == "c2" or rho == 0.8
        check_linear(rmm, case, A, B64, rho, rows=None if every else sample_rows(A.shape[0], 12, seed=7))


def test_full_size_linear_c5(rmm):
    case, A, B64 = linear_case("c5")
    n = A.shape[0]
    rows = sorted(set(sample_rows(n, 192, seed=7)) | {n - 2})
    for rho in case.rhos:
        check_linear(rmm, case, A, B64, rho, rows=rows)


def attention_case(scale=None, rhos=None):
    key = ("c4", tuple(sorted((scale or {}).items())), rhos)
    if key not in _CACHE:
        case = synthetic.make_case("c4", scale)
        dh = case.A.shape[2]
        Q, _ = enforce_gap_batched(case.A, [oracle.k_of(r, dh) for r in (rhos or case.rhos)], "bf16")
        _CACHE[key] = (case, Q)
    return _CACHE[key]


def check_attention(rmm, case, Q, rho, heads, rows):
    torch = pytest.importorskip("torch")
    K = case.B
    hq, hkv = Q.shape[0], K.shape[0]
    group = hq // hkv
    dh = Q.shape[2]
    k = oracle.k_of(rho, dh)
    Qd, Kd = to_device(Q, "bf16"), to_device(K, "bf16")
    S, idx = rmm.matmul(Qd, Kd, rho, transB=True, b_group=group, alpha=case.alpha)
    torch.cuda.synchronize()
    got_idx = idx.cpu().numpy()
    for h in range(hq):
        ref = oracle.topk(oracle.colnorm(Q[h]), k)
        assert np.array_equal(got_idx[h], ref), f"head {h}: index sets differ"
    for h in heads:
        g = h // group
        Kt = np.ascontiguousarray(K[g].astype(np.float64).T)
        ref_idx = got_idx[h]
        Y_ref = oracle.reduced_product(Q[h], Kt, ref_idx, case.alpha, rows)
        absprod = oracle.reduced_product(np.abs(Q[h]), np.abs(Kt), ref_idx, abs(case.alpha), rows)
        Sh = to_host(S[h])
        if rows is not None:
            Sh = Sh[rows]
        assert_close(Sh, Y_ref, absprod, k, "bf16", f"c4 head {h} rho={rho}")


def test_small_attention(rmm):
    case, Q = attention_case(dict(heads=8, kv_heads=2, L=300))
    for rho in case.rhos:
        check_attention(rmm, case, Q, rho, heads=range(8), rows=None)


def stream_plan(rmm, case, Q, rho):
    torch = pytest.importorskip("torch")
    Qm = torch.empty(Q.shape, dtype=torch.bfloat16, device="meta")
    Km = torch.empty(case.B.shape, dtype=torch.bfloat16, device="meta")
    return rmm.plan_info(Qm, Km, rho, transB=True, b_group=case.A.shape[0] // case.B.shape[0])


def test_many_heads_ragged_attention(rmm):
    # 128 query heads of 296 tokens (a multiple of 8, so the MFMA route is
    # taken): enough 256x256 tiles (512) for the persistent streaming kernel,
    # with ragged tile edges in both rows and columns
    case, Q = attention_case(dict(heads=128, kv_heads=32, L=296))
    for rho in case.rhos:
        info = stream_plan(rmm, case, Q, rho)
        assert info["gemm"] == "stream", info
        check_attention(rmm, case, Q, rho, heads=range(0, 128, 7), rows=None)


@pytest.mark.parametrize("rho", [0.8, 1.0])
def test_many_heads_two_k_steps(rmm, rho):
    # k = 103 (rho = 0.8, the pages' attention setting) and k = 128 fill two
    # 64-entry K steps: the streaming kernel's 128-row tiles, ragged at L = 296
    case, Q = attention_case(dict(heads=128, kv_heads=32, L=296), rhos=(rho,))
    info = stream_plan(rmm, case, Q, rho)
    assert info["gemm"] == "stream", info
    check_attention(rmm, case, Q, rho, heads=range(0, 128, 9), rows=None)


def test_full_size_attention(rmm):
    case, Q = attention_case()
    rows = sample_rows(Q.shape[1], 6, seed=3)
    for rho in case.rhos:
        check_attention(rmm, case, Q, rho, heads=[0, 3, 4, 17, 31], rows=rows)


@pytest.mark.parametrize("scale", [dict(n=4, d=640, m=776), None], ids=["small", "full"])
def test_decode(rmm, scale):
    torch = pytest.importorskip("torch")
    case, _, B64 = linear_case("c5", scale)
    dec = synthetic.make_decode_case(case)
    a = dec.A  # no gap fix-up: |a_j| is exact on both sides, ties go to the lower index
    d = a.shape[1]
    for rho in dec.rhos:
        k = oracle.k_of(rho, d)
        ref_idx = oracle.topk(oracle.colnorm(a), k)
        Y, idx = rmm.matmul(to_device(a, "bf16"), to_device(case.B, "bf16"), rho)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref_idx)
        Y_ref = oracle.reduced_product(a, B64, ref_idx)
        absprod = oracle.reduced_product(np.abs(a), np.abs(B64), ref_idx)
        assert_close(to_host(Y), Y_ref, absprod, k, "bf16", f"decode rho={rho}")


@pytest.mark.parametrize("d", [1001, 1004])
def test_decode_row_length_not_a_multiple_of_eight(rmm, d):
    """The decode route with d % 8 != 0 (row padded to a multiple of 8): the
    selection reads the row's last 16-byte piece element by element, so the
    last columns keep their values and the padding (huge values here, which
    would win the TopK if read) is never scored."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(d)
    m, ld = 64, 1008
    a = synthetic.round_to_bf16((rng.standard_normal((1, d)) * np.exp(rng.standard_normal(d))).astype(np.float32))
    a[0, -3:] = np.float32(64.0)  # the last columns must be kept
    B = synthetic.round_to_bf16((rng.standard_normal((d, m)) / np.sqrt(d)).astype(np.float32))
    padded = np.full((1, ld), 3.0e4, np.float32)
    padded[:, :d] = a
    Ad = to_device(synthetic.round_to_bf16(padded), "bf16")[:, :d]
    Bd = to_device(B, "bf16")
    assert rmm.plan_info(Ad, Bd, 0.6)["route"] == "decode"
    B64 = B.astype(np.float64)
    for rho in (0.6, 1.0):
        k = oracle.k_of(rho, d)
        ref_idx = oracle.topk(np.abs(a[0]).astype(np.float64), k)
        Y, idx = rmm.matmul(Ad, Bd, rho)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref_idx), rho
        assert_close(to_host(Y), oracle.reduced_product(a, B64, ref_idx),
                     oracle.reduced_product(np.abs(a), np.abs(B64), ref_idx), k, "bf16", f"d={d} rho={rho}")


ONE_LAUNCH = [
    # (d, m, rho): decodes wide enough (m >= 14336) for the selection inside the GEMV
    (1001, 24584, 0.6),    # odd d; the last column block holds 8 columns
    (16384, 24576, 0.5),   # the longest row the selection takes
    (8192, 28672, 1.0),    # every row kept
    (640, 24576, 1 / 640),  # one row kept
]


@pytest.mark.parametrize("d,m,rho", ONE_LAUNCH, ids=[f"d{c[0]}-m{c[1]}-rho{c[2]:.3g}" for c in ONE_LAUNCH])  # noqa
def test_decode_selection_in_gemv(rmm, d, m, rho):
    """Wide single-row decodes (m >= 14336): every GEMV workgroup selects
    from |a| itself, then streams its column block over one split of the kept
    rows (the split sum follows): kept set bit for bit, y within the bound,
    repeat calls identical."""
    import ctypes
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(d + m)
    a = synthetic.round_to_bf16((rng.standard_normal((1, d)) * np.exp(rng.standard_normal(d))).astype(np.float32))
    B = synthetic.round_to_bf16((rng.standard_normal((d, m)) / np.sqrt(d)).astype(np.float32))
    ld = (d + 7) // 8 * 8  # the decode route wants a 16-byte row pitch: pad the row, values after d unused
    padded = np.full((1, ld), 3.0e4, np.float32)
    padded[:, :d] = a
    ad, Bd = to_device(synthetic.round_to_bf16(padded), "bf16")[:, :d], to_device(B, "bf16")
    info = rmm.plan_info(ad, Bd, rho)
    assert info["route"] == "decode", info
    k = oracle.k_of(rho, d)
    ref_idx = oracle.topk(np.abs(a[0]).astype(np.float64), k)
    Y, idx = rmm.matmul(ad, Bd, rho, alpha=0.5)
    Y2, _ = rmm.matmul(ad, Bd, rho, alpha=0.5, return_idx=False)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    assert torch.equal(Y, Y2)
    B64 = B.astype(np.float64)
    assert_close(to_host(Y), oracle.reduced_product(a, B64, ref_idx, 0.5),
                 oracle.reduced_product(np.abs(a), np.abs(B64), ref_idx, 0.5), k, "bf16", f"d={d} m={m}")


def test_decode_selection_in_gemv_ties(rmm):
    """Many equal |a_j| through the selection inside the GEMV: ties -> lower index."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(15)
    d, m = 1000, 24576
    a = synthetic.round_to_bf16(rng.choice([-2.0, -1.0, 0.5, 1.0, 2.0, -0.0], size=(1, d)).astype(np.float32))
    B = synthetic.round_to_bf16(rng.standard_normal((d, m)).astype(np.float32))
    ad, Bd, B64 = to_device(a, "bf16"), to_device(B, "bf16"), B.astype(np.float64)
    for k in (1, 137, 500, 999, 1000):
        rho = k / d
        ref_idx = oracle.topk(np.abs(a[0]).astype(np.float64), k)
        Y, idx = rmm.matmul(ad, Bd, rho)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref_idx), k
        assert_close(to_host(Y), oracle.reduced_product(a, B64, ref_idx),
                     oracle.reduced_product(np.abs(a), np.abs(B64), ref_idx), k, "bf16", f"ties k={k}")


def test_decode_exact_ties(rmm):
    """n = 1 with many equal |a_j| (bf16 has few values): ties -> lower index."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    d, m = 1000, 64
    a = synthetic.round_to_bf16(rng.choice([-2.0, -1.0, 0.5, 1.0, 2.0], size=(1, d)).astype(np.float32))
    B = synthetic.round_to_bf16(rng.standard_normal((d, m)).astype(np.float32))
    for k in (1, 137, 500, 999, 1000):
        rho = k / d
        assert oracle.k_of(rho, d) == k
        ref_idx = oracle.topk(np.abs(a[0]).astype(np.float64), k)
        Y, idx = rmm.matmul(to_device(a, "bf16"), to_device(B, "bf16"), rho)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref_idx), k
        B64 = B.astype(np.float64)
        assert_close(to_host(Y), oracle.reduced_product(a, B64, ref_idx),
                     oracle.reduced_product(np.abs(a), np.abs(B64), ref_idx), k, "bf16", f"ties k={k}")


BATCHED = [
    # (batch, n, d, m, group, rhos, rows sampled per entry or None for all)
    (8, 300, 520, 136, 4, (0.5, 0.8), None),
    (8, 1024, 2048, 1536, 2, (0.5, 0.8), 6),
]


@pytest.mark.parametrize("batch,n,d,m,group,rhos,nrows", BATCHED, ids=["small", "large-tiles"])
def test_batched_grouped_linear(rmm, batch, n, d, m, group, rhos, nrows):
    """Batched products with B shared by `group` consecutive entries and not
    transposed: one selection per entry (the token-axis shape P V of Sec. 3.3,
    with P as A and the GQA value head as B)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(batch * 1000 + d)
    A = np.stack([synthetic.lognormal_outlier_activations(rng, n, d, "bf16", n_outliers=3)[0]
                  for _ in range(batch)])
    B = np.stack([synthetic.gaussian_weights(rng, d, m, "bf16") for _ in range(batch // group)])
    A, _ = enforce_gap_batched(A, [oracle.k_of(r, d) for r in rhos], "bf16")
    Ad, Bd = to_device(A, "bf16"), to_device(B, "bf16")
    for rho in rhos:
        k = oracle.k_of(rho, d)
        info = rmm.plan_info(Ad, Bd, rho, b_group=group)
        assert info["route"] == "mfma", info
        if nrows is not None:
            assert info["gemm"] in ("adirect", "bdma"), info
        Y, idx = rmm.matmul(Ad, Bd, rho, b_group=group)
        torch.cuda.synchronize()
        got_idx = idx.cpu().numpy()
        for b in range(batch):
            ref_idx = oracle.topk(oracle.colnorm(A[b]), k)
            assert np.array_equal(got_idx[b], ref_idx), f"entry {b} rho={rho}: index sets differ"
            rows = None if nrows is None else sample_rows(n, nrows, seed=b)
            B64 = B[b // group].astype(np.float64)
            Yh = to_host(Y[b])
            if rows is not None:
                Yh = Yh[rows]
            assert_close(Yh, oracle.reduced_product(A[b], B64, ref_idx, 1.0, rows),
                         oracle.reduced_product(np.abs(A[b]), np.abs(B64), ref_idx, 1.0, rows), k, "bf16",
                         f"batched entry {b} rho={rho}")


TRANSPOSED = [
    # (n, d, m, rhos, kernel, rows sampled or None): B given as m x d (the
    # nn.Linear weight layout); its kept columns are packed like the keys of
    # Q K^T and contracted with 128x128 or 256x256 tiles
    (300, 520, 264, (0.5, 0.8), "tile128", None),
    (4096, 1024, 3072, (0.5, 0.8), "tile256", 10),
]


@pytest.mark.parametrize("n,d,m,rhos,kernel,nrows", TRANSPOSED, ids=["tile128", "tile256"])
def test_transposed_weights(rmm, n, d, m, rhos, kernel, nrows):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(n + m)
    A, _ = synthetic.lognormal_outlier_activations(rng, n, d, "bf16", n_outliers=3)
    W = synthetic.gaussian_weights(rng, m, d, "bf16")  # m x d: B = W^T
    A, _ = enforce_gap(A, [oracle.k_of(r, d) for r in rhos], "bf16")
    Ad, Wd = to_device(A, "bf16"), to_device(W, "bf16")
    B64 = np.ascontiguousarray(W.astype(np.float64).T)
    rows = None if nrows is None else sample_rows(n, nrows, seed=11)
    for rho in rhos:
        k = oracle.k_of(rho, d)
        info = rmm.plan_info(Ad, Wd, rho, transB=True)
        assert info["gemm"] == kernel, info
        Y, idx = rmm.matmul(Ad, Wd, rho, transB=True)
        torch.cuda.synchronize()
        ref_idx = oracle.topk(oracle.colnorm(A), k)
        assert np.array_equal(idx.cpu().numpy(), ref_idx)
        Yh = to_host(Y)
        if rows is not None:
            Yh = Yh[rows]
        assert_close(Yh, oracle.reduced_product(A, B64, ref_idx, 1.0, rows),
                     oracle.reduced_product(np.abs(A), np.abs(B64), ref_idx, 1.0, rows), k, "bf16",
                     f"transposed rho={rho}")


def test_small_attention_mfma_route(rmm):
    # 296-token heads (a multiple of 8): the MFMA route with 128x128 tiles
    # (too few tiles for the streaming kernel), packed keys
    case, Q = attention_case(dict(heads=8, kv_heads=2, L=296))
    for rho in case.rhos:
        info = stream_plan(rmm, case, Q, rho)
        assert info["route"] == "mfma" and info["gemm"] == "tile128", info
        check_attention(rmm, case, Q, rho, heads=range(8), rows=None)

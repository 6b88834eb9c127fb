"""GPU tests of the single steps and of the boundary: column norms, exact
selection (ties, plateaus, long score vectors), odd shapes and layouts that
take the generic route, argument errors, determinism and stream ordering."""
import ctypes

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_close, to_device, to_host

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


# --------------------------------------------------------------------------- column norms

@pytest.mark.parametrize("n,d,dtype", [(1, 8, "bf16"), (3, 5, "f32"), (64, 256, "f32"), (300, 520, "bf16"),
                                       (4096, 4096, "bf16"), (2048, 14336, "bf16"), (17, 1001, "bf16"),
                                       (1000, 3, "f32"), (5000, 64, "bf16")])
def test_colnorm(rmm, torch, n, d, dtype):
    rng = np.random.default_rng(n * 7 + d)
    A = (rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))).astype(np.float32)
    if dtype == "bf16":
        A = synthetic.round_to_bf16(A)
    s = rmm.colnorm(to_device(A, dtype))
    torch.cuda.synchronize()
    ref = oracle.colnorm(A)
    got = s.cpu().numpy().astype(np.float64)
    rel = np.max(np.abs(got - ref) / ref)
    assert rel <= 1e-5, rel


def test_colnorm_strided_and_unaligned(rmm, torch):
    rng = np.random.default_rng(1)
    W = synthetic.round_to_bf16(rng.standard_normal((70, 203)).astype(np.float32))
    Wd = to_device(W, "bf16")
    for sl in [(slice(None), slice(0, 200)), (slice(None), slice(1, 201)), (slice(3, 70), slice(5, 203))]:
        s = rmm.colnorm(Wd[sl])
        torch.cuda.synchronize()
        ref = oracle.colnorm(W[sl])
        assert np.max(np.abs(s.cpu().numpy() - ref) / ref) <= 1e-5


# --------------------------------------------------------------------------- selection

def _sel_case(rng, d, kind):
    if kind == "random":
        return np.abs(rng.standard_normal(d)).astype(np.float32)
    if kind == "ties":
        v = np.abs(rng.standard_normal(max(1, d // 10))).astype(np.float32)
        return v[rng.integers(0, v.size, size=d)]
    if kind == "bf16":  # bf16-valued scores: the low 16 key bits are zero in every key
        s = (np.abs(rng.standard_normal(d)) * np.exp(rng.standard_normal(d))).astype(np.float32)
        return (s.view(np.uint32) & np.uint32(0xffff0000)).view(np.float32)
    if kind == "const":
        return np.full(d, 3.25, dtype=np.float32)
    if kind == "zeros_and_inf":
        s = np.abs(rng.standard_normal(d)).astype(np.float32)
        s[rng.integers(0, d, size=max(1, d // 7))] = 0.0
        s[rng.integers(0, d, size=max(1, d // 50))] = np.inf
        return s
    if kind == "nan_and_inf":  # NaN ranks above +Inf (any payload or sign), NaNs tie among themselves
        s = np.abs(rng.standard_normal(d)).astype(np.float32)
        s[rng.integers(0, d, size=max(1, d // 40))] = np.inf
        nan_at = rng.integers(0, d, size=max(1, d // 30))
        s[nan_at] = np.nan
        u = s.view(np.uint32)
        u[nan_at[::2]] = np.uint32(0xffc00001)  # a negative NaN with a payload
        return s
    raise KeyError(kind)


@pytest.mark.parametrize("d", [1, 2, 7, 128, 1000, 1024, 2049, 2432, 3008, 4032, 4096, 14336, 30000])
@pytest.mark.parametrize("kind", ["random", "ties", "bf16", "const", "zeros_and_inf", "nan_and_inf"])
def test_select_exact(rmm, torch, d, kind):
    rng = np.random.default_rng(d + len(kind))
    s = _sel_case(rng, d, kind)
    sd = torch.from_numpy(s).to("cuda:0")
    for k in sorted({1, max(1, d // 3), max(1, d // 2), max(1, d - 1), d}):
        got = rmm.select(sd, k)
        torch.cuda.synchronize()
        ref = oracle.topk(s.astype(np.float64), k)
        assert np.array_equal(got.cpu().numpy(), ref), (d, kind, k)


def test_select_batched(rmm, torch):
    rng = np.random.default_rng(9)
    s = np.abs(rng.standard_normal((32, 128))).astype(np.float32)
    s[5] = 1.0  # a whole row of ties
    got = rmm.select(torch.from_numpy(s).to("cuda:0"), 64)
    torch.cuda.synchronize()
    for b in range(32):
        assert np.array_equal(got[b].cpu().numpy(), oracle.topk(s[b].astype(np.float64), 64)), b


# --------------------------------------------------------------------------- odd shapes / generic route

ODD = [
    # (n, d, m, dtype, rho, note)
    (1, 1, 1, "f32", 1.0, "scalar"),
    (5, 37, 13, "bf16", 0.5, "m not a multiple of 8"),
    (7, 9, 3, "f32", 0.2, "k = 2"),
    (257, 300, 24, "bf16", 0.01, "k = 3, n one past a tile"),
    (64, 4096, 64, "bf16", 1 / 4096, "k = 1"),
    (33, 65, 72, "bf16", 0.999, "k = d - 0 (ceil)"),
    (2, 100, 8, "bf16", 0.07, "rho*d just above an integer"),
    # norms finalized in their own launch before the selection: d above the
    # one-workgroup norm+select kernel, and more row chunks (65 x 1024
    # partials) than it takes
    (64, 20480, 64, "bf16", 0.5, "d above the fused selection"),
    (33000, 1024, 64, "bf16", 0.5, "many row chunks"),
    # the one-workgroup norm+select kernel with 8 and 16 keys per thread
    # (4096 < d <= 16384, at most 256 KB of partials: here 1 and 4 row chunks)
    (64, 6000, 64, "bf16", 0.6, "fused selection, 8 keys per thread"),
    (256, 14004, 40, "bf16", 0.3, "fused selection, 16 keys per thread"),
]
SEPARATE_FINALIZE = {"d above the fused selection", "many row chunks"}
FUSED_SELECT = {"fused selection, 8 keys per thread", "fused selection, 16 keys per thread"}


@pytest.mark.parametrize("n,d,m,dtype,rho,note", ODD, ids=[o[-1] for o in ODD])
def test_odd_shapes(rmm, torch, n, d, m, dtype, rho, note):
    rng = np.random.default_rng(n + d + m)
    A = (rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))).astype(np.float32)
    B = rng.standard_normal((d, m)).astype(np.float32)
    if dtype == "bf16":
        A, B = synthetic.round_to_bf16(A), synthetic.round_to_bf16(B)
    k = oracle.k_of(rho, d)
    if n > 1 and k < d:
        A, _ = enforce_gap_2d(A, k, dtype)
    ref_idx = oracle.topk(oracle.colnorm(A), k)
    Ad, Bd = to_device(A, dtype), to_device(B, dtype)
    rmm.timing_enable(True)
    try:
        Y, idx = rmm.matmul(Ad, Bd, rho)
        torch.cuda.synchronize()
        launches = {kind: cnt for kind, (_, cnt) in rmm.timing_collect().items()}
    finally:
        rmm.timing_enable(False)
    if note in SEPARATE_FINALIZE:  # the case reaches the path it is meant to cover
        assert launches["finalize"] == 1, launches
    if note in FUSED_SELECT:
        assert launches["finalize"] == 0 and launches["select"] == 1, launches
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    B64 = B.astype(np.float64)
    assert_close(to_host(Y), oracle.reduced_product(A, B64, ref_idx),
                 oracle.reduced_product(np.abs(A), np.abs(B64), ref_idx), k, dtype, note)


def enforce_gap_2d(A, k, dtype):
    from oracle.fixup import enforce_gap
    return enforce_gap(A, [k], dtype)


def test_strided_views_and_unaligned(rmm, torch):
    """A column slice with lda > d (unaligned start, generic route), B offset by
    one row, and an output with ldy > m: each agrees with the oracle, and the
    untouched output columns keep their NaN fill."""
    from oracle.fixup import enforce_gap
    rng = np.random.default_rng(21)
    n, d, m, rho = 200, 384, 96, 0.7
    k = oracle.k_of(rho, d)
    W = synthetic.round_to_bf16((rng.standard_normal((n, d + 9)) * np.exp(rng.standard_normal(d + 9))).astype(np.float32))
    W[:, 1:1 + d], _ = enforce_gap(W[:, 1:1 + d], [k], "bf16")
    A = np.ascontiguousarray(W[:, 1:1 + d])
    B = synthetic.round_to_bf16(rng.standard_normal((d + 1, m)).astype(np.float32))
    B64 = B[1:].astype(np.float64)
    ref_idx = oracle.topk(oracle.colnorm(A), k)
    ref_Y = oracle.reduced_product(A, B64, ref_idx)
    ref_abs = oracle.reduced_product(np.abs(A), np.abs(B64), ref_idx)
    Wd, Bd = to_device(W, "bf16"), to_device(B, "bf16")
    Ad = Wd[:, 1:1 + d]
    assert Ad.stride(0) == d + 9 and Ad.data_ptr() % 16 != 0
    out = torch.full((n, m + 8), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    for a_t, o in [(Ad, None), (Ad.contiguous(), None), (Ad.contiguous(), out[:, :m])]:
        Y, idx = rmm.matmul(a_t, Bd[1:], rho, out=o)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref_idx)
        assert_close(to_host(Y), ref_Y, ref_abs, k, "bf16", "strided")
    assert torch.isnan(out[:, m:].float()).all(), "columns beyond m must stay untouched"


# --------------------------------------------------------------------------- boundary

def _desc(rmm, n, d, m, dtype=1):
    ds = rmm.Desc()
    rmm.load().rmm_desc_init(ctypes.byref(ds), dtype, n, d, m)
    return ds


def test_invalid_arguments_leave_outputs_untouched(rmm, torch):
    L = rmm.load()
    n, d, m = 64, 128, 64
    A = torch.randn(n, d, device="cuda:0").to(torch.bfloat16)
    B = torch.randn(d, m, device="cuda:0").to(torch.bfloat16)
    Y = torch.full((n, m), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    idx = torch.full((d,), -7, dtype=torch.int32, device="cuda:0")
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda:0")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    good = _desc(rmm, n, d, m)
    assert L.rmm_workspace_size(ctypes.byref(good), 0.5) <= ws.numel()

    def call(ds, rho, a=A.data_ptr(), b=B.data_ptr(), y=Y.data_ptr(), w=ws.data_ptr(), wb=ws.numel()):
        return L.rmm_matmul(ctypes.byref(ds), a, b, rho, y, idx.data_ptr(), w, wb, s)

    for rho in (0.0, -1.0, 1.5, float("nan")):
        assert call(good, rho) == 1
    for field, val in [("n", 0), ("d", 0), ("m", -1), ("lda", 64), ("ldb", 3), ("ldy", 10), ("batch", 0),
                       ("dtype", 7), ("b_group", 0), ("transB", 2), ("flags", 0x100), ("strideA", -1)]:
        bad = _desc(rmm, n, d, m)
        setattr(bad, field, val)
        assert call(bad, 0.5) == 1, field
    assert call(good, 0.5, a=0) == 1
    assert call(good, 0.5, y=0) == 1
    assert call(good, 0.5, y=A.data_ptr()) == 1, "output aliasing an input"
    assert call(good, 0.5, w=0, wb=0) == 3
    assert call(good, 0.5, wb=16) == 3
    torch.cuda.synchronize()
    assert torch.isnan(Y.float()).all()
    assert (idx == -7).all()
    # a valid call after the rejected ones works and writes only k indices
    assert call(good, 0.5) == 0
    torch.cuda.synchronize()
    assert not torch.isnan(Y.float()).any()
    assert (idx[64:] == -7).all() and (idx[:64] >= 0).all()
    # selection and norm entry points
    sc = torch.rand(d, device="cuda:0")
    assert L.rmm_select(sc.data_ptr(), 1, d, 0, idx.data_ptr(), s) == 1
    assert L.rmm_select(sc.data_ptr(), 1, d, d + 1, idx.data_ptr(), s) == 1
    assert L.rmm_colnorm(A.data_ptr(), 1, n, d, d - 1, sc.data_ptr(), ws.data_ptr(), ws.numel(), s) == 1
    assert L.rmm_colnorm(A.data_ptr(), 1, n, d, d, sc.data_ptr(), 0, 0, s) == 3


def test_repeat_calls_are_bitwise_identical(rmm, torch):
    case = synthetic.make_case("c2", scale=dict(n=512, d=1024, m=512))
    Ad, Bd = to_device(case.A, "bf16"), to_device(case.B, "bf16")
    Y0, i0 = rmm.matmul(Ad, Bd, 0.7)
    s0 = rmm.colnorm(Ad)
    for _ in range(20):
        Y, i = rmm.matmul(Ad, Bd, 0.7)
        s = rmm.colnorm(Ad)
        assert torch.equal(Y, Y0) and torch.equal(i, i0) and torch.equal(s, s0)


def test_non_default_streams(rmm, torch):
    case = synthetic.make_case("c2", scale=dict(n=256, d=512, m=256))
    Ad, Bd = to_device(case.A, "bf16"), to_device(case.B, "bf16")
    Y0, i0 = rmm.matmul(Ad, Bd, 0.5)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    A2 = (Ad.float() * 2).to(torch.bfloat16)
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        Y1, i1 = rmm.matmul(Ad, Bd, 0.5)
    with torch.cuda.stream(s2):
        Y2, i2 = rmm.matmul(A2, Bd, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y0) and torch.equal(i1, i0)
    assert torch.equal(i2, i0)  # scaling A by 2 keeps the selection
    assert torch.equal(Y2.float(), (Y0.float() * 2))


GUARDED = [
    # (n, d, m, dtype, rho, route, gemm): every route's stores stay inside Y
    # when Y's rows are a padded pitch apart inside a canary-filled buffer
    (3104, 1504, 4000, "bf16", 0.5, "mfma", "tdma"),
    (2048, 4200, 3080, "bf16", 0.5, "mfma", "tdma"),      # two K splits through the reduce
    (3100, 1504, 4000, "bf16", 0.5, "mfma", "bdma"),
    (3100, 1504, 4000, "bf16", 0.8, "mfma", "adirect"),
    (2050, 4200, 3080, "bf16", 0.48, "mfma", "adirect"),  # split K
    (300, 520, 264, "bf16", 0.5, "mfma", "tile128"),
    (520, 2048, 128, "bf16", 0.5, "mfma", "gcol"),
    (1, 8192, 28680, "bf16", 0.8, "decode", None),        # selection inside the GEMV, ragged last block
    (1, 1000, 264, "bf16", 0.8, "decode", None),          # separate selection, split GEMV and reduce
    (100, 300, 77, "f32", 0.5, "generic", None),
]


@pytest.mark.parametrize("n,d,m,dtype,rho,route,gemm", GUARDED,
                         ids=[f"{g[6] or g[5]}-{g[0]}x{g[1]}x{g[2]}-rho{g[4]}" for g in GUARDED])
def test_stores_stay_inside_a_padded_output(rmm, torch, n, d, m, dtype, rho, route, gemm):
    """Canary guard bands: Y is a view with a row pitch of m + 280 inside a
    buffer with 8 rows above and 256 below it (a whole tile of slack on every
    side), all filled with a canary pattern; the kept-index output sits at
    the start of a longer canary-filled array.  After the call every canary
    outside Y and past k is intact, and Y equals, bit for bit, the output of
    the same call into a contiguous tensor."""
    rng = np.random.default_rng(n + d + m)
    A = (rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))).astype(np.float32)
    B = (rng.standard_normal((d, m)) / np.sqrt(d)).astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Ad = torch.from_numpy(A).to("cuda:0").to(tdt)
    Bd = torch.from_numpy(B).to("cuda:0").to(tdt)
    info = rmm.plan_info(Ad, Bd, rho)
    assert info["route"] == route and info["gemm"] == gemm, info
    Y0, i0 = rmm.matmul(Ad, Bd, rho)
    k = rmm.k_of(rho, d)
    top, bottom, left, right = 8, 256, 16, 264
    itype = torch.int16 if dtype == "bf16" else torch.int32
    canary = 0x5A5A if dtype == "bf16" else 0x5A5A5A5A
    buf = torch.full((top + n + bottom, left + m + right), canary, dtype=itype, device="cuda:0")
    Yv = buf.view(tdt)[top:top + n, left:left + m]
    ibuf = torch.full((k + 256,), -7, dtype=torch.int32, device="cuda:0")
    Y1, i1 = rmm.matmul(Ad, Bd, rho, out=Yv, idx_out=ibuf[:k])
    torch.cuda.synchronize()
    assert torch.equal(Yv.view(itype), Y0.view(itype))
    outside = torch.ones(buf.shape, dtype=torch.bool, device="cuda:0")
    outside[top:top + n, left:left + m] = False
    assert bool((buf[outside] == canary).all())
    assert torch.equal(ibuf[:k], i0) and bool((ibuf[k:] == -7).all())


def _guarded(torch, shape, dtype, front=256, back=8192):
    """A canary-filled 1-D buffer with a contiguous view of `shape` after
    `front` elements (256 two-byte or four-byte elements: 16-byte aligned)."""
    itype = torch.int16 if dtype in (torch.bfloat16,) else torch.int32
    canary = 0x5A5A if itype == torch.int16 else 0x5A5A5A5A
    numel = int(np.prod(shape))
    buf = torch.full((front + numel + back,), canary, dtype=itype, device="cuda:0")
    view = buf[front:front + numel].view(dtype).view(shape)

    def intact():
        return bool((buf[:front] == canary).all()) and bool((buf[front + numel:] == canary).all())

    return view, intact


def test_other_entry_points_stay_inside_their_outputs(rmm, torch):
    """Canary guard bands before and after the outputs of the fused
    attention, the 8-bit decode and GEMM (the GEMM's Y with a padded row
    pitch) and the gated MLP block; each result equals the same call's
    result into freshly allocated outputs, bit for bit."""
    g = torch.Generator(device="cuda:0").manual_seed(11)
    dev = "cuda:0"

    def randn(*shape, scale=1.0):
        return (torch.randn(*shape, device=dev, generator=g) * scale).to(torch.bfloat16)

    # fused attention: 8 query heads over 2 key/value heads, 200 causal queries
    q, kk, v = randn(8, 200, 128), randn(2, 200, 128), randn(2, 200, 128)
    O0, I0 = rmm.attention(q, kk, v, 0.5)
    O, o_ok = _guarded(torch, (8, 200, 128), torch.bfloat16)
    I, i_ok = _guarded(torch, tuple(I0.shape), torch.int32)
    rmm.attention(q, kk, v, 0.5, out=O, idx_out=I)
    torch.cuda.synchronize()
    assert torch.equal(O, O0) and torch.equal(I, I0) and o_ok() and i_ok()

    # 8-bit decode, wide enough for the selection inside the GEMV; ragged last column block
    d, m = 1000, 14352
    a = randn(d)
    codes = torch.randint(-127, 128, (d, m), device=dev, generator=g, dtype=torch.int32).to(torch.int8)
    scale = torch.rand(m, device=dev, generator=g) * 0.01
    y0, j0 = rmm.decode_wq(a, codes, scale, 0.7, "int8")
    y, y_ok = _guarded(torch, (m,), torch.bfloat16)
    j, j_ok = _guarded(torch, tuple(j0.shape), torch.int32)
    rmm.decode_wq(a, codes, scale, 0.7, "int8", out=y, idx_out=j)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(j, j0) and y_ok() and j_ok()

    # 8-bit GEMM (n, d multiples of 8, m of 16; ragged against its tiles) with
    # Y's rows m + 40 apart inside a canary-filled block
    n, d, m = 296, 520, 272
    A = randn(n, d)
    codes = torch.randint(-127, 128, (d, m), device=dev, generator=g, dtype=torch.int32).to(torch.int8)
    scale = torch.rand(m, device=dev, generator=g) * 0.01
    Y0, _ = rmm.matmul_wq(A, codes, scale, 0.6, "int8")
    buf = torch.full((n + 16, m + 40), 0x5A5A, dtype=torch.int16, device=dev)
    Yv = buf.view(torch.bfloat16)[8:8 + n, 16:16 + m]
    rmm.matmul_wq(A, codes, scale, 0.6, "int8", out=Yv)
    torch.cuda.synchronize()
    outside = torch.ones(buf.shape, dtype=torch.bool, device=dev)
    outside[8:8 + n, 16:16 + m] = False
    assert torch.equal(Yv, Y0) and bool((buf[outside] == 0x5A5A).all())

    # gated MLP block
    n, d, m = 64, 256, 512
    x = randn(n, d)
    Wgu = rmm.gated_weights(randn(d, m, scale=d ** -0.5), randn(d, m, scale=d ** -0.5))
    Wd = randn(m, d, scale=m ** -0.5)
    Y0 = rmm.gated_mlp(x, Wgu, Wd, 0.8, 0.8)[0]
    Y, y_ok = _guarded(torch, (n, d), torch.bfloat16)
    rmm.gated_mlp(x, Wgu, Wd, 0.8, 0.8, out=Y)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y0) and y_ok()


RACE_PROBES = [
    # (what, repeats): the hot kernels at their full workload shapes, each call
    # compared bit for bit with the first (an LDS or cross-wave race shows up
    # as a run-to-run difference)
    ("tdma8 4096x4096x4096 rho 0.8", 100),
    ("tdma8 split K 2048x14336x4096 rho 0.8", 50),
    ("fused attention 32 heads x 4096 rho 0.5", 100),
    ("decode 1x8192x28672 rho 0.8", 100),
    ("gated MLP 512x4096x14336 rho 0.8", 30),
]


@pytest.mark.parametrize("what,repeats", RACE_PROBES, ids=[r[0].split()[0] + "-" + r[0].split()[1] for r in RACE_PROBES])
def test_race_probe_repeats(rmm, torch, what, repeats):
    g = torch.Generator(device="cuda:0").manual_seed(21)
    dev = "cuda:0"

    def randn(*shape, scale=1.0):
        return (torch.randn(*shape, device=dev, generator=g) * scale).to(torch.bfloat16)

    if what.startswith("tdma8"):
        n, d, m = (4096, 4096, 4096) if "split" not in what else (2048, 14336, 4096)
        A = (torch.randn(n, d, device=dev, generator=g) * torch.exp(torch.randn(d, device=dev, generator=g))).to(
            torch.bfloat16)
        B = randn(d, m, scale=d ** -0.5)
        info = rmm.plan_info(A, B, 0.8)
        assert info["gemm"] == "tdma" and (info["splits"] > 1) == ("split" in what), info
        call = lambda: rmm.matmul(A, B, 0.8)  # noqa: E731
    elif what.startswith("fused attention"):
        q, k, v = randn(32, 4096, 128), randn(8, 4096, 128), randn(8, 4096, 128)
        call = lambda: rmm.attention(q, k, v, 0.5, causal=True)  # noqa: E731
    elif what.startswith("decode"):
        a = (torch.randn(1, 8192, device=dev, generator=g) * torch.exp(torch.randn(8192, device=dev, generator=g))).to(
            torch.bfloat16)
        B = randn(8192, 28672, scale=8192 ** -0.5)
        assert rmm.plan_info(a, B, 0.8)["route"] == "decode"
        call = lambda: rmm.matmul(a, B, 0.8)  # noqa: E731
    else:
        n, d, m = 512, 4096, 14336
        x = randn(n, d)
        Wgu = rmm.gated_weights(randn(d, m, scale=d ** -0.5), randn(d, m, scale=d ** -0.5))
        Wd = randn(m, d, scale=m ** -0.5)
        call = lambda: rmm.gated_mlp(x, Wgu, Wd, 0.8, 0.8)  # noqa: E731
    first = [t.clone() for t in call()]
    for r in range(repeats - 1):
        got = call()
        for a_, b_ in zip(got, first):
            assert torch.equal(a_, b_), (what, r)
    torch.cuda.synchronize()

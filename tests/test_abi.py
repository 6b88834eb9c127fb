"""The C-ABI library (CPU-only checks): it loads, exports every function that
include/rmm.h declares, and its host-side logic (k, status strings, workspace
sizing, argument validation) behaves as documented.  No GPU work is run."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmm.h")
LIB = os.path.join(ROOT, "input_adaptive_reduced_amd", "librmm.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(rmm_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("librmm.so is not built; run __graft_entry__.build()")
    import input_adaptive_reduced_amd as r
    return r.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("rmm_k", "rmm_colnorm", "rmm_select", "rmm_matmul", "rmm_workspace_size",
                     "rmm_status_string"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_rmm_k_matches_oracle(lib, oracle_mod):
    import pins
    for rho, d, k in pins.K_TABLE:
        assert lib.rmm_k(rho, d) == k == oracle_mod.k_of(rho, d)
    for rho, d in pins.K_INVALID:
        assert lib.rmm_k(rho, d) == 0


def test_status_strings(lib):
    for s in range(5):
        assert lib.rmm_status_string(s)
    assert lib.rmm_status_string(99) == b"unknown status"


def test_workspace_sizing_and_validation_on_host(lib):
    import input_adaptive_reduced_amd as r
    ds = r.Desc()
    lib.rmm_desc_init(ctypes.byref(ds), r.BF16, 4096, 4096, 4096)
    big = lib.rmm_workspace_size(ctypes.byref(ds), 0.5)
    assert 0 < big < (1 << 31)
    assert lib.rmm_workspace_size(ctypes.byref(ds), 0.0) == ctypes.c_size_t(-1).value
    ds.lda = 100
    assert lib.rmm_workspace_size(ctypes.byref(ds), 0.5) == ctypes.c_size_t(-1).value
    ds.lda = 4096
    # argument errors return before any HIP call, so they are safe without a GPU
    assert lib.rmm_matmul(ctypes.byref(ds), None, None, 0.5, None, None, None, 0, None) == 1
    assert lib.rmm_matmul(None, 1, 1, 0.5, 1, None, None, 0, None) == 1
    assert lib.rmm_select(None, 1, 10, 3, None, None) == 1
    assert lib.rmm_colnorm(None, 1, 2, 2, 2, None, None, 0, None) == 1
    # a workspace that is not 256-byte aligned is refused before any launch
    lib.rmm_desc_init(ctypes.byref(ds), r.BF16, 64, 256, 128)
    need = lib.rmm_workspace_size(ctypes.byref(ds), 0.5)
    A, B, Y, W = 1 << 40, 2 << 40, 3 << 40, 4 << 40
    assert lib.rmm_matmul(ctypes.byref(ds), A, B, 0.5, Y, None, W + 16, need, None) == 1
    assert lib.rmm_matmul(ctypes.byref(ds), A, B, 0.5, Y, None, W, need - 1, None) == 3
    # the caller-supplied index variant: sizes, argument checks, alignment
    lib.rmm_workspace_size_indexed.restype = ctypes.c_size_t
    lib.rmm_workspace_size_indexed.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    lib.rmm_matmul_indexed.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                                               ctypes.c_size_t, ctypes.c_void_p]
    bad = ctypes.c_size_t(-1).value
    assert lib.rmm_workspace_size_indexed(ctypes.byref(ds), 0) == bad
    assert lib.rmm_workspace_size_indexed(ctypes.byref(ds), 257) == bad   # k > d
    need_i = lib.rmm_workspace_size_indexed(ctypes.byref(ds), 128)
    assert 0 < need_i <= need                                             # no norm buffers
    I = 5 << 40
    assert lib.rmm_matmul_indexed(ctypes.byref(ds), A, B, None, 128, Y, W, need_i, None) == 1
    assert lib.rmm_matmul_indexed(ctypes.byref(ds), A, B, I, 0, Y, W, need_i, None) == 1
    assert lib.rmm_matmul_indexed(ctypes.byref(ds), A, B, I, 257, Y, W, need_i, None) == 1
    assert lib.rmm_matmul_indexed(ctypes.byref(ds), A, B, I, 128, Y, W + 16, need_i, None) == 1
    assert lib.rmm_matmul_indexed(ctypes.byref(ds), A, B, I, 128, Y, W, need_i - 1, None) == 3
    assert lib.rmm_matmul_indexed(ctypes.byref(ds), A, B, Y, 128, Y, W, need_i, None) == 1  # idx inside Y


def test_plan_info_on_host(lib):
    """rmm_plan_info is host-only: the route and kernel each workload shape
    takes, and its argument checks."""
    import input_adaptive_reduced_amd as r

    def info(dtype, n, d, m, rho, transB=0, batch=1, group=1):
        ds = r.Desc()
        lib.rmm_desc_init(ctypes.byref(ds), dtype, n, d, m)
        ds.transB = transB
        if transB:
            ds.ldb = d
        ds.batch, ds.b_group = batch, group
        if batch > 1:
            ds.strideA, ds.strideB, ds.strideY = n * d, (m * d if transB else d * m), n * m
        out = (ctypes.c_int32 * 3)()
        st = lib.rmm_plan_info(ctypes.byref(ds), rho, out)
        return st, tuple(out)

    # c2 and c3: the norm pass writes A^T, both operands gathered by rows (no pack)
    assert info(r.BF16, 4096, 4096, 4096, 0.8) == (0, (1, 5, 1))
    assert info(r.BF16, 2048, 14336, 4096, 0.8) == (0, (1, 5, 2))      # two K splits
    assert info(r.BF16, 4096, 4096, 4096, 1.0) == (0, (1, 2, 1))       # rho = 1 shortcut: no norms, A packed
    assert info(r.BF16, 4100, 4096, 4096, 0.8) == (0, (1, 2, 1))       # n % 8 != 0: A packed, A-direct kernel
    assert info(r.BF16, 4096, 8192, 28672, 0.8) == (0, (1, 5, 1))      # c5
    assert info(r.BF16, 4096, 8192, 40960, 0.8) == (0, (1, 4, 1))      # wider output keeps the pack; LDS-DMA B
    assert info(r.BF16, 1, 8192, 28672, 0.8) == (0, (2, -1, 4))       # wide decode: 56 column blocks x 4 row splits
    st, (route, gemm, splits) = info(r.BF16, 1, 8192, 4096, 0.8)      # narrower decode: split gathered GEMV
    assert st == 0 and route == 2 and gemm == -1 and splits > 1
    assert info(r.BF16, 4096, 128, 4096, 0.5, transB=1, batch=32, group=4) == (0, (1, 3, 1))  # c4 scores
    # attention's P V (m = d_v): A's kept columns gathered inside the narrow-output kernel
    assert info(r.BF16, 4096, 4096, 128, 0.5, batch=32, group=4) == (0, (1, 6, 1))
    assert info(r.BF16, 1024, 2048, 128, 0.5) == (0, (1, 6, 1))        # one head: not the A^T route
    assert info(r.BF16, 300, 520, 40, 1.0) == (0, (1, 6, 1))           # rho = 1 shortcut reads an identity list
    assert info(r.BF16, 1024, 2048, 136, 0.5)[1][1] != 6                # wider than one 128-column tile
    assert info(r.BF16, 64, 2048, 128, 0.5, batch=8)[1][1] != 6         # fewer rows than one tile
    assert info(r.BF16, 512, 16392, 128, 0.5)[1][1] != 6                # kept list beyond the kernel's LDS copy
    assert info(r.BF16, 512, 1004, 128, 0.5)[1][1] != 6                 # d % 8 != 0
    assert info(r.F32, 64, 256, 128, 0.5)[1][:2] == (0, -1)             # fp32: generic route
    assert info(r.BF16, 300, 520, 300, 0.5)[1][:2] == (0, -1)           # m % 8 != 0: generic route
    assert info(r.BF16, 64, 256, 128, 0.0)[0] == 1                      # invalid rho
    ds = r.Desc()
    lib.rmm_desc_init(ctypes.byref(ds), r.BF16, 64, 256, 128)
    assert lib.rmm_plan_info(ctypes.byref(ds), 0.5, None) == 1          # NULL output


def test_gated_mlp_sizes_on_host(lib):
    """The gated block is supported for short token blocks too: the Down
    stage then splits K so that its LDS row list fits (no GPU call)."""
    SZ_MAX = ctypes.c_size_t(-1).value
    ws = lib.rmm_gated_mlp_workspace_size
    for n in (8, 64, 512, 768, 1024, 2048):
        assert ws(n, 4096, 14336, 0.8, 0.8) != SZ_MAX, n
    assert ws(64, 1024, 14336, 0.8, 0.8) != SZ_MAX
    assert ws(6, 4096, 14336, 0.8, 0.8) == SZ_MAX         # n % 8 != 0
    assert ws(64, 4096, 14330, 0.8, 0.8) == SZ_MAX        # m % 32 != 0


def test_attention_and_decode_wq_host_checks(lib):
    """Workspace sizing and argument checks of rmm_attention and rmm_decode_wq
    are host-only: they return before any GPU call (fake, aligned pointers)."""
    SZ_MAX = ctypes.c_size_t(-1).value
    ws_a = lib.rmm_attention_workspace_size
    assert ws_a(32, 8, 4096, 4096, 128, 0.5) not in (0, SZ_MAX)
    assert ws_a(32, 8, 4096, 4096, 128, 0.5) < ws_a(32, 8, 4096, 4096, 128, 0.8)   # 64 vs 128 kept columns
    assert ws_a(32, 6, 64, 64, 128, 0.5) == SZ_MAX        # H not a multiple of Hkv
    assert ws_a(4, 4, 64, 64, 136, 0.5) == SZ_MAX         # dh > 128
    assert ws_a(4, 4, 64, 64, 100, 0.5) == SZ_MAX         # dh % 8 != 0
    assert ws_a(4, 4, 64, 64, 128, 0.0) == SZ_MAX         # invalid rho
    P = ctypes.c_void_p
    q, k, v, o, w = P(0x10000), P(0x20000), P(0x30000), P(0x40000), P(0x100000)
    need = ws_a(2, 1, 64, 64, 128, 0.5)
    att = lib.rmm_attention
    assert att(None, k, v, 2, 1, 64, 64, 128, 128, 0.5, 1, o, None, w, need, None) == 1   # null q
    assert att(q, k, v, 2, 1, 64, 64, 128, 128, 0.5, 2, o, None, w, need, None) == 1      # causal not 0/1
    assert att(q, k, v, 2, 1, 96, 64, 128, 128, 0.5, 1, o, None, w, need, None) == 1      # causal, Lq > Lk
    assert att(q, k, v, 2, 1, 64, 64, 128, 64, 0.5, 1, o, None, w, need, None) == 2       # dv != 128
    assert att(q, k, v, 2, 1, 64, 64, 128, 128, 0.5, 1, P(0x40008), None, w, need, None) == 2  # misaligned out
    assert att(q, k, v, 2, 1, 64, 64, 128, 128, 0.5, 1, o, None, w, need - 1, None) == 3  # short workspace
    assert att(q, k, v, 2, 1, 64, 64, 128, 128, 0.5, 1, o, None, P(0x100010), need, None) == 1  # unaligned ws
    assert att(q, k, v, 2, 1, 64, 64, 128, 128, 0.5, 1, P(0x10000 + 256), None, w, need, None) == 1  # out over q
    ws_d = lib.rmm_decode_wq_workspace_size
    assert ws_d(8192, 28672, 0.8) == 9 * 28672 * 4        # wide outputs: selection in the GEMV, 9 row splits
    assert ws_d(8192, 4096, 0.8) not in (0, SZ_MAX)       # narrower: select launch, split GEMV and reduce
    assert ws_d(8192, 40, 0.8) == SZ_MAX                  # m % 16 != 0
    assert ws_d(20000, 1024, 0.8) == SZ_MAX               # beyond the fused selection
    a, bq, sc, y = P(0x10000), P(0x200000), P(0x30000), P(0x40000)
    need = ws_d(1024, 256, 0.5)
    dec = lib.rmm_decode_wq
    assert dec(a, bq, 2, sc, 1024, 256, 256, 0.5, 1.0, y, None, w, need, None) == 1     # unknown format
    assert dec(a, bq, 0, sc, 1024, 256, 128, 0.5, 1.0, y, None, w, need, None) == 1     # ldb < m
    assert dec(a, bq, 0, sc, 1024, 256, 264, 0.5, 1.0, y, None, w, need, None) == 2     # ldb % 16 != 0
    assert dec(a, P(0x200008), 0, sc, 1024, 256, 256, 0.5, 1.0, y, None, w, need, None) == 2  # misaligned codes
    assert dec(a, bq, 0, sc, 1024, 256, 256, 0.5, 1.0, y, None, w, need - 1, None) == 3  # short workspace
    assert dec(a, bq, 0, sc, 1024, 256, 256, 0.5, 1.0, P(0x200000 + 512), None, w, need, None) == 1  # y over codes


def test_binding_refuses_wrong_outputs_before_any_launch():
    """The binding validates caller-supplied outputs before it calls the
    library: a tensor of the wrong shape, dtype, layout or device raises
    ValueError (the library would write through the raw pointer)."""
    torch = pytest.importorskip("torch")
    import input_adaptive_reduced_amd as rmm

    meta = torch.device("meta")
    good = torch.empty((4, 128, 128), dtype=torch.bfloat16, device=meta)
    rmm.check_out(good, (4, 128, 128), torch.bfloat16, meta, "out")
    bad = [
        (torch.empty((4, 127, 128), dtype=torch.bfloat16, device=meta), "shape"),
        (torch.empty((4, 128, 128), dtype=torch.float32, device=meta), "float32"),
        (torch.empty((4, 128, 256), dtype=torch.bfloat16, device=meta)[:, :, :128], "contiguous"),
        (torch.empty((4, 128, 128), dtype=torch.bfloat16), "live on"),
    ]
    for t, what in bad:
        with pytest.raises(ValueError, match=what):
            rmm.check_out(t, (4, 128, 128), torch.bfloat16, meta, "out")
    # idx outputs: an int32 tensor one element short is refused
    with pytest.raises(ValueError, match="shape"):
        rmm.check_out(torch.empty(63, dtype=torch.int32, device=meta), (64,), torch.int32, meta, "idx_out")

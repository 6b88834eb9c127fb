"""The entry point that allocates nothing (``rmm_matmul_noalloc``), called
through the C ABI, against the existing entry point ``rmm_matmul`` with a
workspace of its own: the same kernels run on the same inputs, so Y and the
kept set must agree bit for bit.  Two calls in a row, the second smaller, so
the second runs on whatever the first left in the library's scratch array;
a third, at a size whose workspace exceeds the array, must be refused before
anything is launched; a decode-shaped call covers the single-row route."""
import ctypes

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import to_device
from oracle.fixup import enforce_gap

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


def noalloc(rmm, torch, A, B, rho, Y, idx):
    L = rmm.load()
    L.rmm_matmul_noalloc.argtypes = [ctypes.POINTER(rmm.Desc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.rmm_matmul_noalloc.restype = ctypes.c_int
    ds, _ = rmm._desc_for(A, B, False, 1, 1.0, False, Y)
    return L.rmm_matmul_noalloc(ctypes.byref(ds), A.data_ptr(), B.data_ptr(), float(rho), Y.data_ptr(),
                                None if idx is None else idx.data_ptr(),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def compare(rmm, torch, name, scale, rho, with_oracle=False):
    case = synthetic.make_case(name, scale)
    k = oracle.k_of(rho, case.A.shape[1])
    A = case.A if case.A.shape[0] == 1 else enforce_gap(case.A, [k], case.dtype)[0]
    Ad, Bd = to_device(A, "bf16"), to_device(case.B, "bf16")
    Y_ref, idx_ref = rmm.matmul(Ad, Bd, rho)
    Y = torch.full_like(Y_ref, float("nan"))
    idx = torch.full_like(idx_ref, -7)
    st = noalloc(rmm, torch, Ad, Bd, rho, Y, idx)
    torch.cuda.synchronize()
    assert st == 0, rmm.status_string(st)
    assert torch.equal(idx, idx_ref), f"{name} {scale}: kept sets differ"
    assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16)), f"{name} {scale}: outputs differ"
    if with_oracle:
        assert np.array_equal(idx.cpu().numpy(), oracle.topk(oracle.colnorm(A), k))


def test_noalloc_matches_matmul_two_calls_then_refuses_oversize(rmm, torch):
    # first call: the 8B projection 4096 x 4096 x 4096 (workspace ~33.6 MB: A^T and the norm partials)
    compare(rmm, torch, "c2", None, 0.8)
    # second call, smaller: ragged n (operand-block route), checked against the oracle's set too
    compare(rmm, torch, "c2", dict(n=300, d=520, m=264), 0.5, with_oracle=True)
    # a single row (decode route) after them
    compare(rmm, torch, "c5", dict(n=1, d=1024, m=2048), 0.8)
    # 2048 x 4096 x 4096 splits K in two (fp32 partials: ~80 MB of workspace): refused, nothing written
    n, d, m = 2048, 4096, 4096
    A = torch.zeros((n, d), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((d, m), dtype=torch.bfloat16, device="cuda")
    Y = torch.full((n, m), 3.0, dtype=torch.bfloat16, device="cuda")
    assert rmm.workspace_size(A, B, 0.8) > (64 << 20)
    st = noalloc(rmm, torch, A, B, 0.8, Y, None)
    torch.cuda.synchronize()
    assert st == 3, rmm.status_string(st)  # RMM_ERR_WORKSPACE
    assert bool((Y == 3.0).all())

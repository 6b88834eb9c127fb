"""Reduced Matrix Multiplication (RMM) on MI355X (gfx950).

A thin ctypes binding over ``librmm.so`` (C ABI in ``include/rmm.h``).  Every
step of the path -- column norms, TopK selection, gather and the reduced
product -- runs in the library's HIP kernels; this module only marshals
arguments: it reads shapes and strides from torch tensors, allocates outputs
and scratch through torch's caching allocator, and passes device pointers and
the current HIP stream.  There is no CPU fallback: without the built library
every call raises.

The method is the one of "Reduced Matrix Multiplication: Input-Adaptive
Matrix-Product Reduction for LLM Inference" (Sec. 3.2): for Y = A B keep the
ceil(rho d) contraction indices with the largest column norms of A and
compute A[:, I] B[I, :].
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "RMMError", "lib_path", "load", "k_of", "status_string", "version", "colnorm", "select", "matmul",
    "workspace_size", "timing_enable", "timing_collect", "KERNEL_KINDS", "F32", "BF16", "FLAG_FULL_PATH",
    "matmul_indexed", "plan_info", "gated_weights", "gated_mlp", "decode_wq", "WQ_FORMATS", "attention",
    "check_out", "calibrate_mfma", "matmul_wq",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librmm.so")

F32, BF16 = 0, 1
FLAG_FULL_PATH = 0x1
KERNEL_KINDS = ("colnorm", "finalize", "select", "pack", "gemm", "reduce", "gemv", "other")
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "hip"}


class RMMError(RuntimeError):
    def __init__(self, status: int, where: str):
        detail = ""
        if status == 4 and _lib is not None:
            detail = ": " + _lib.rmm_last_hip_error().decode()
        super().__init__(f"{where}: {status_string(status)} (status {status}){detail}")
        self.status = status


class Desc(ctypes.Structure):
    """Mirror of rmm_desc_t (include/rmm.h)."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("transB", ctypes.c_int32),
        ("n", ctypes.c_int64), ("d", ctypes.c_int64), ("m", ctypes.c_int64),
        ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldy", ctypes.c_int64),
        ("batch", ctypes.c_int64),
        ("strideA", ctypes.c_int64), ("strideB", ctypes.c_int64), ("strideY", ctypes.c_int64),
        ("b_group", ctypes.c_int64),
        ("alpha", ctypes.c_float), ("flags", ctypes.c_int32),
    ]


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def _hip_runtimes():
    """Distinct HIP runtime libraries mapped into this process (Linux)."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:  # pragma: no cover
        return []


def load():
    """Load librmm.so (raises if it has not been built).

    torch is imported first: it ships its own HIP runtime, and librmm must
    bind to that same runtime (same soname) so that torch's streams and
    allocations are valid in the library.  Loading librmm first would map a
    second runtime from /opt/rocm next to torch's; that state is refused.
    """
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with input_adaptive_reduced_amd/build.py")
    try:
        import torch  # noqa: F401  (binds the process to torch's HIP runtime)
    except ImportError:
        pass
    L = ctypes.CDLL(_LIB_PATH)
    rts = _hip_runtimes()
    if len(rts) > 1:
        raise RuntimeError("two HIP runtimes are loaded (%s); import torch before anything loads "
                           "librmm.so" % ", ".join(rts))
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.rmm_k.argtypes, L.rmm_k.restype = [ctypes.c_double, i64], i64
    L.rmm_status_string.argtypes, L.rmm_status_string.restype = [ctypes.c_int], ctypes.c_char_p
    L.rmm_version.argtypes, L.rmm_version.restype = [], i32
    L.rmm_last_hip_error.argtypes, L.rmm_last_hip_error.restype = [], ctypes.c_char_p
    L.rmm_colnorm_workspace_size.argtypes, L.rmm_colnorm_workspace_size.restype = [ctypes.c_int, i64, i64], sz
    L.rmm_colnorm.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, sz, vp]
    L.rmm_colnorm.restype = ctypes.c_int
    L.rmm_select.argtypes, L.rmm_select.restype = [vp, i64, i64, i64, vp, vp], ctypes.c_int
    L.rmm_desc_init.argtypes, L.rmm_desc_init.restype = [ctypes.POINTER(Desc), ctypes.c_int, i64, i64, i64], None
    L.rmm_workspace_size.argtypes = [ctypes.POINTER(Desc), ctypes.c_double]
    L.rmm_workspace_size.restype = sz
    L.rmm_matmul.argtypes = [ctypes.POINTER(Desc), vp, vp, ctypes.c_double, vp, vp, vp, sz, vp]
    L.rmm_matmul.restype = ctypes.c_int
    L.rmm_workspace_size_indexed.argtypes = [ctypes.POINTER(Desc), i64]
    L.rmm_workspace_size_indexed.restype = sz
    L.rmm_matmul_indexed.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, i64, vp, vp, sz, vp]
    L.rmm_matmul_indexed.restype = ctypes.c_int
    L.rmm_gated_weights.argtypes = [vp, vp, i64, i64, i32, vp, vp]
    L.rmm_gated_weights.restype = ctypes.c_int
    L.rmm_gated_mlp_workspace_size.argtypes = [i64, i64, i64, ctypes.c_double, ctypes.c_double]
    L.rmm_gated_mlp_workspace_size.restype = sz
    L.rmm_gated_mlp.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_double, ctypes.c_double, vp, vp, vp, vp, vp, sz,
                                vp]
    L.rmm_gated_mlp.restype = ctypes.c_int
    L.rmm_decode_wq_workspace_size.argtypes = [i64, i64, ctypes.c_double]
    L.rmm_decode_wq_workspace_size.restype = sz
    L.rmm_decode_wq.argtypes = [vp, vp, i32, vp, i64, i64, i64, ctypes.c_double, ctypes.c_float, vp, vp, vp, sz, vp]
    L.rmm_decode_wq.restype = ctypes.c_int
    L.rmm_matmul_wq_workspace_size.argtypes = [i64, i64, i64, ctypes.c_double]
    L.rmm_matmul_wq_workspace_size.restype = sz
    L.rmm_matmul_wq.argtypes = [vp, i64, i64, i64, vp, i32, vp, i64, i64, ctypes.c_double, ctypes.c_float, vp, i64,
                                vp, vp, sz, vp]
    L.rmm_matmul_wq.restype = ctypes.c_int
    L.rmm_attention_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_double]
    L.rmm_attention_workspace_size.restype = sz
    L.rmm_attention.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_double, i32, vp, vp, vp, sz, vp]
    L.rmm_attention.restype = ctypes.c_int
    L.rmm_plan_info.argtypes = [ctypes.POINTER(Desc), ctypes.c_double, ctypes.POINTER(i32)]
    L.rmm_plan_info.restype = ctypes.c_int
    L.rmm_timing_enable.argtypes, L.rmm_timing_enable.restype = [i32, i32], ctypes.c_int
    L.rmm_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.rmm_timing_collect.restype = ctypes.c_int
    L.rmm_calibrate_mfma.argtypes, L.rmm_calibrate_mfma.restype = [i64, i32, vp, i64, vp, vp], ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    try:
        return load().rmm_status_string(int(status)).decode()
    except ImportError:
        return _STATUS.get(int(status), "unknown")


def _check(status: int, where: str):
    if status != 0:
        raise RMMError(status, where)


def version() -> int:
    return int(load().rmm_version())


def k_of(rho: float, d: int) -> int:
    """|I| = ceil(rho d) as the library computes it (0 = invalid)."""
    return int(load().rmm_k(float(rho), int(d)))


# ----------------------------------------------------------------------------- torch marshalling

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _stream(t) -> ctypes.c_void_p:
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _require_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _workspace(nbytes: int, device):
    torch = _torch()
    if nbytes == 0:
        return None, 0
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device), int(nbytes)


def _ptr(t):
    """Device address of an optional tensor (None -> NULL)."""
    return None if t is None else t.data_ptr()


def check_out(t, shape, dtype, device, name: str):
    """Raise ValueError unless ``t`` can receive an output of ``shape`` and
    ``dtype`` on ``device``: exact shape and dtype, contiguous, same device.
    The library writes through the raw pointer, so a smaller or strided
    tensor would be written past its end."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must live on {device}, got {t.device}")


def _user_workspace(workspace, need: int, device):
    """The caller's workspace (uint8-sized bytes on ``device``) or a new one."""
    if workspace is None:
        return _workspace(need, device)
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return workspace, workspace.numel() * workspace.element_size()


def colnorm(A) -> "torch.Tensor":
    """s_j = ||A[:, j]||_2 (fp32) of a 2-D bf16/fp32 tensor with unit column stride."""
    torch = _torch()
    _require_gpu(A)
    if A.dim() != 2 or A.stride(1) != 1:
        raise ValueError("A must be 2-D with unit column stride")
    n, d = A.shape
    L = load()
    dt = _dtype_code(A)
    s = torch.empty(d, dtype=torch.float32, device=A.device)
    ws, wsb = _workspace(L.rmm_colnorm_workspace_size(dt, n, d), A.device)
    _check(L.rmm_colnorm(A.data_ptr(), dt, n, d, A.stride(0), s.data_ptr(), _ptr(ws), wsb, _stream(A)),
           "rmm_colnorm")
    return s


def select(s, k: int) -> "torch.Tensor":
    """Indices of the k largest scores (ties -> lower index), ascending int32.

    ``s`` is (d,) or (batch, d) fp32, contiguous.
    """
    torch = _torch()
    _require_gpu(s)
    if s.dtype != torch.float32 or not s.is_contiguous() or s.dim() not in (1, 2):
        raise ValueError("s must be a contiguous fp32 tensor of shape (d,) or (batch, d)")
    batch, d = (1, s.shape[0]) if s.dim() == 1 else s.shape
    out = torch.empty((batch, int(k)), dtype=torch.int32, device=s.device)
    _check(load().rmm_select(s.data_ptr(), batch, d, int(k), out.data_ptr(), _stream(s)), "rmm_select")
    return out[0] if s.dim() == 1 else out


def _desc_for(A, B, transB: bool, b_group: int, alpha: float, full_path: bool, Y=None) -> Tuple[Desc, tuple]:
    if A.dim() not in (2, 3) or B.dim() != A.dim():
        raise ValueError("A and B must both be 2-D, or both 3-D (batched)")
    if A.dtype != B.dtype:
        raise TypeError("A and B must share a dtype")
    if A.stride(-1) != 1 or B.stride(-1) != 1:
        raise ValueError("A and B need unit stride along their last dimension")
    batched = A.dim() == 3
    batch = A.shape[0] if batched else 1
    n, d = A.shape[-2], A.shape[-1]
    if transB:
        m, d2 = B.shape[-2], B.shape[-1]
    else:
        d2, m = B.shape[-2], B.shape[-1]
    if d != d2:
        raise ValueError(f"contraction sizes differ: {d} vs {d2}")
    nb = B.shape[0] if batched else 1
    if batched and batch != nb * b_group:
        raise ValueError(f"batch {batch} must equal B batch {nb} x b_group {b_group}")
    ds = Desc()
    ds.dtype = _dtype_code(A)
    ds.transB = 1 if transB else 0
    ds.n, ds.d, ds.m = n, d, m
    ds.lda, ds.ldb = A.stride(-2), B.stride(-2)
    ds.ldy = m if Y is None else Y.stride(-2)
    ds.batch = batch
    ds.strideA = A.stride(0) if batched else 0
    ds.strideB = B.stride(0) if batched else 0
    ds.strideY = (n * ds.ldy if Y is None else Y.stride(0)) if batched else 0
    ds.b_group = b_group if batched else 1
    ds.alpha = float(alpha)
    ds.flags = FLAG_FULL_PATH if full_path else 0
    shape = (batch, n, m) if batched else (n, m)
    return ds, shape


def workspace_size(A, B, rho: float, transB: bool = False, b_group: int = 1, full_path: bool = False) -> int:
    ds, _ = _desc_for(A, B, transB, b_group, 1.0, full_path)
    w = load().rmm_workspace_size(ctypes.byref(ds), float(rho))
    if w == ctypes.c_size_t(-1).value:
        raise RMMError(1, "rmm_workspace_size")
    return int(w)


ROUTES = ("generic", "mfma", "decode")
GEMM_KERNELS = ("tile256", "tile128", "adirect", "stream", "bdma", "tdma", "gcol")


def plan_info(A, B, rho: float, transB: bool = False, b_group: int = 1, full_path: bool = False) -> dict:
    """The kernels ``matmul`` would run for these operands (host-side, from
    shapes, strides and dtype only: tensors on the ``meta`` device will do)."""
    ds, _ = _desc_for(A, B, transB, b_group, 1.0, full_path)
    info = (ctypes.c_int32 * 3)()
    _check(load().rmm_plan_info(ctypes.byref(ds), float(rho), info), "rmm_plan_info")
    return {"route": ROUTES[info[0]], "gemm": GEMM_KERNELS[info[1]] if info[1] >= 0 else None,
            "splits": int(info[2])}


def matmul(A, B, rho: float, *, transB: bool = False, b_group: int = 1, alpha: float = 1.0,
           out=None, idx_out=None, return_idx: bool = True, full_path: bool = False, workspace=None):
    """Y = alpha * A[:, I] B[I, :] with I = TopK(||A[:, j]||_2, ceil(rho d)).

    A: (n, d) or (batch, n, d).  B: (d, m), or (m, d) with ``transB``; batched
    B has batch / b_group entries, entry b of A pairs with B[b // b_group]
    (grouped-query attention).  Returns (Y, idx) with idx of shape (k,) or
    (batch, k), int32 ascending (None when ``return_idx`` is false and no
    ``idx_out`` was given).
    """
    torch = _torch()
    _require_gpu(A, B)
    L = load()
    ds, shape = _desc_for(A, B, transB, b_group, alpha, full_path, out)
    k = int(L.rmm_k(float(rho), ds.d))
    if k < 1:
        raise RMMError(1, f"rho={rho!r}")
    if out is None:
        out = torch.empty(shape, dtype=A.dtype, device=A.device)
    elif (tuple(out.shape) != shape or out.dtype != A.dtype or out.stride(-1) != 1 or out.device != A.device
          or (A.dim() == 3 and out.stride(0) < shape[1] * out.stride(1))):
        # rows may be padded (ldy = out.stride(-2)); every element must be addressable
        raise ValueError("out has the wrong shape, dtype, layout or device")
    idx_shape = (ds.batch, k) if A.dim() == 3 else (k,)
    if idx_out is None and return_idx:
        idx_out = torch.empty(idx_shape, dtype=torch.int32, device=A.device)
    elif idx_out is not None:
        # any contiguous int32 tensor of batch*k elements (e.g. flat) will do
        check_out(idx_out, tuple(idx_out.shape) if idx_out.numel() == ds.batch * k else idx_shape, torch.int32,
                  A.device, "idx_out")
    need = L.rmm_workspace_size(ctypes.byref(ds), float(rho))
    if need == ctypes.c_size_t(-1).value:
        raise RMMError(1, "rmm_workspace_size")
    ws, wsb = _user_workspace(workspace, need, A.device)
    st = L.rmm_matmul(ctypes.byref(ds), A.data_ptr(), B.data_ptr(), float(rho), out.data_ptr(), _ptr(idx_out),
                      _ptr(ws), wsb, _stream(A))
    _check(st, "rmm_matmul")
    return out, idx_out


def timing_enable(enable: bool = True, capacity: int = 4096):
    _check(load().rmm_timing_enable(1 if enable else 0, int(capacity)), "rmm_timing_enable")


def timing_collect() -> dict:
    """Per kernel kind: (total milliseconds, launches) since the last collect."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(load().rmm_timing_collect(ms, cnt), "rmm_timing_collect")
    return {KERNEL_KINDS[i]: (ms[i], cnt[i]) for i in range(n)}


def calibrate_mfma(workgroups: int = 2048, iters: int = 4096, repeats: int = 5) -> dict:
    """Sustained bf16 matrix-core throughput of this GPU (rmm_calibrate_mfma):
    the probe kernel launched ``repeats`` times back to back on the current
    stream, each launch timed with events.  Returns the TFLOP/s of every
    launch, the flops per launch and the shader clock (MHz) the probe's
    waves measured during each launch (median over workgroups)."""
    torch = _torch()
    L = load()
    out = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    clk = torch.empty((repeats, workgroups, 2), dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(repeats + 1)]
    flops = float(workgroups) * 4 * iters * 8 * 2 * 32 * 32 * 16
    _check(L.rmm_calibrate_mfma(workgroups, iters, out.data_ptr(), out.numel(), None, sp),
           "rmm_calibrate_mfma")  # untimed first launch
    ev[0].record(stream)
    for r in range(repeats):
        _check(L.rmm_calibrate_mfma(workgroups, iters, out.data_ptr(), out.numel(), clk[r].data_ptr(), sp),
               "rmm_calibrate_mfma")
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    ms = [ev[r].elapsed_time(ev[r + 1]) for r in range(repeats)]
    c = clk.cpu().double()
    mhz = (c[:, :, 0] / c[:, :, 1].clamp(min=1) * 100.0).median(dim=1).values.tolist()
    return {"flops_per_launch": flops, "ms": ms, "tflops": [flops / (t * 1e-3) / 1e12 for t in ms],
            "shader_mhz": mhz, "workgroups": workgroups, "iters": iters}


def matmul_indexed(A, B, idx, *, transB: bool = False, b_group: int = 1, alpha: float = 1.0, out=None,
                   workspace=None):
    """Y = alpha * A[:, I] B[I, :] over a given kept set I (rmm_matmul_indexed).

    idx: int32 device tensor of shape (k,), or (batch, k) for a batched A,
    each row strictly ascending in [0, d); entries that break this are
    dropped by the library.  A, B and the other arguments are as for
    ``matmul``.  Returns Y.
    """
    torch = _torch()
    _require_gpu(A, B)
    L = load()
    ds, shape = _desc_for(A, B, transB, b_group, alpha, False, out)
    if idx.dtype != torch.int32 or not idx.is_contiguous() or idx.device != A.device:
        raise ValueError("idx must be a contiguous int32 tensor on A's device")
    if idx.dim() != (2 if A.dim() == 3 else 1) or (A.dim() == 3 and idx.shape[0] != ds.batch):
        raise ValueError("idx must have shape (k,) or (batch, k)")
    k = int(idx.shape[-1])
    if out is None:
        out = torch.empty(shape, dtype=A.dtype, device=A.device)
    elif (tuple(out.shape) != shape or out.dtype != A.dtype or out.stride(-1) != 1 or out.device != A.device
          or (A.dim() == 3 and out.stride(0) < shape[1] * out.stride(1))):
        raise ValueError("out has the wrong shape, dtype, layout or device")
    need = L.rmm_workspace_size_indexed(ctypes.byref(ds), k)
    if need == ctypes.c_size_t(-1).value:
        raise RMMError(1, "rmm_workspace_size_indexed")
    ws, wsb = _user_workspace(workspace, need, A.device)
    st = L.rmm_matmul_indexed(ctypes.byref(ds), A.data_ptr(), B.data_ptr(), idx.data_ptr(), k, out.data_ptr(),
                              _ptr(ws), wsb, _stream(A))
    _check(st, "rmm_matmul_indexed")
    return out


def gated_weights(Wg, Wu, transposed: bool = False):
    """The interleaved Gate/Up operand for ``gated_mlp`` (rmm_gated_weights).

    Wg, Wu: bf16 (d, m), or (m, d) nn.Linear weights with ``transposed``.
    Returns a (d, 2m) bf16 tensor."""
    torch = _torch()
    _require_gpu(Wg, Wu)
    if Wg.dtype != torch.bfloat16 or Wu.dtype != torch.bfloat16 or Wg.shape != Wu.shape or Wg.dim() != 2:
        raise ValueError("Wg and Wu must be bf16 matrices of one shape")
    if not (Wg.is_contiguous() and Wu.is_contiguous()):
        raise ValueError("Wg and Wu must be contiguous")
    d, m = (Wg.shape[1], Wg.shape[0]) if transposed else (Wg.shape[0], Wg.shape[1])
    out = torch.empty((d, 2 * m), dtype=torch.bfloat16, device=Wg.device)
    _check(load().rmm_gated_weights(Wg.data_ptr(), Wu.data_ptr(), d, m, 1 if transposed else 0, out.data_ptr(),
                                    _stream(Wg)), "rmm_gated_weights")
    return out


def attention(q, k, v, rho: float, *, causal: bool = True, out=None, idx_out=None, workspace=None):
    """Attention with reduced scores, softmax fused (rmm_attention).

    q: bf16 (H, Lq, dh); k: bf16 (Hkv, Lk, dh); v: bf16 (Hkv, Lk, 128).
    Returns (O, idx): O bf16 (H, Lq, 128), idx int32 (H, k) the dimensions
    each query head keeps."""
    torch = _torch()
    _require_gpu(q, k, v)
    L = load()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or {q.dtype, k.dtype, v.dtype} != {torch.bfloat16}:
        raise ValueError("expected bf16 q (H, Lq, dh), k (Hkv, Lk, dh), v (Hkv, Lk, dv)")
    H, Lq, dh = q.shape
    Hkv, Lk, dv = v.shape
    if k.shape != (Hkv, Lk, dh):
        raise ValueError("k must be (Hkv, Lk, dh) matching q and v")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("operands must be contiguous")
    need = L.rmm_attention_workspace_size(H, Hkv, Lq, Lk, dh, float(rho))
    if need == ctypes.c_size_t(-1).value:
        raise RMMError(2, "rmm_attention_workspace_size")
    kk = int(L.rmm_k(float(rho), dh))
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must live on one device")
    if out is None:
        out = torch.empty((H, Lq, dv), dtype=torch.bfloat16, device=q.device)
    else:
        check_out(out, (H, Lq, dv), torch.bfloat16, q.device, "out")
    if idx_out is None:
        idx_out = torch.empty((H, kk), dtype=torch.int32, device=q.device)
    else:
        check_out(idx_out, (H, kk), torch.int32, q.device, "idx_out")
    ws, wsb = _user_workspace(workspace, need, q.device)
    st = L.rmm_attention(q.data_ptr(), k.data_ptr(), v.data_ptr(), H, Hkv, Lq, Lk, dh, dv, float(rho),
                         1 if causal else 0, out.data_ptr(), idx_out.data_ptr(), _ptr(ws), wsb, _stream(q))
    _check(st, "rmm_attention")
    return out, idx_out


WQ_FORMATS = {"fp8": 0, "int8": 1}


def decode_wq(a, Bq, scale, rho: float, fmt: str = "fp8", *, alpha: float = 1.0, out=None, idx_out=None,
              workspace=None):
    """Single-row decode over 8-bit weights (rmm_decode_wq).

    a: bf16 (d,) or (1, d); Bq: (d, m) 8-bit codes (uint8, int8 or
    float8_e4m3fn storage; ``fmt`` "fp8" = OCP E4M3, "int8"); scale: fp32
    (m,).  Returns (y, idx): y bf16 of a's shape with m columns, idx int32 (k,)
    ascending."""
    torch = _torch()
    _require_gpu(a, Bq, scale)
    L = load()
    if fmt not in WQ_FORMATS:
        raise ValueError(f"fmt must be one of {sorted(WQ_FORMATS)}")
    d = a.shape[-1]
    if a.dtype != torch.bfloat16 or a.numel() != d or Bq.element_size() != 1 or Bq.dim() != 2 or Bq.shape[0] != d:
        raise ValueError("expected bf16 a with d entries and 8-bit Bq (d, m)")
    m = Bq.shape[1]
    if scale.dtype != torch.float32 or scale.numel() != m or not scale.is_contiguous():
        raise ValueError("scale must be m contiguous fp32 values")
    if not a.is_contiguous() or Bq.stride(1) != 1:
        raise ValueError("a must be contiguous and Bq row-major")
    need = L.rmm_decode_wq_workspace_size(d, m, float(rho))
    if need == ctypes.c_size_t(-1).value:
        raise RMMError(2, "rmm_decode_wq_workspace_size")
    k = int(L.rmm_k(float(rho), d))
    if Bq.device != a.device or scale.device != a.device:
        raise ValueError("a, Bq and scale must live on one device")
    if out is None:
        out = torch.empty(a.shape[:-1] + (m,), dtype=torch.bfloat16, device=a.device)
    else:
        check_out(out, a.shape[:-1] + (m,), torch.bfloat16, a.device, "out")
    if idx_out is None:
        idx_out = torch.empty(k, dtype=torch.int32, device=a.device)
    else:
        check_out(idx_out, (k,), torch.int32, a.device, "idx_out")
    ws, wsb = _user_workspace(workspace, need, a.device)
    st = L.rmm_decode_wq(a.data_ptr(), Bq.data_ptr(), WQ_FORMATS[fmt], scale.data_ptr(), d, m, Bq.stride(0),
                         float(rho), float(alpha), out.data_ptr(), idx_out.data_ptr(), _ptr(ws), wsb, _stream(a))
    _check(st, "rmm_decode_wq")
    return out, idx_out


def matmul_wq(A, Bq, scale, rho: float, fmt: str = "fp8", *, alpha: float = 1.0, out=None, idx_out=None,
              workspace=None):
    """Y = alpha * A[:, I] (value(Bq) * scale)[I, :] with I = TopK(||A[:, j]||, ceil(rho d))
    (rmm_matmul_wq: 8-bit weights with one fp32 scale per column, any n).

    A: bf16 (n, d) with unit column stride; Bq: (d, m) 8-bit codes (uint8,
    int8 or float8_e4m3fn storage; ``fmt`` "fp8" = OCP E4M3, "int8") with
    unit column stride; scale: fp32 (m,).  Returns (Y, idx): Y bf16 (n, m),
    idx int32 (k,) ascending."""
    torch = _torch()
    _require_gpu(A, Bq, scale)
    L = load()
    if fmt not in WQ_FORMATS:
        raise ValueError(f"fmt must be one of {sorted(WQ_FORMATS)}")
    if A.dtype != torch.bfloat16 or A.dim() != 2 or A.stride(1) != 1:
        raise ValueError("A must be a bf16 matrix with unit column stride")
    n, d = A.shape
    if Bq.element_size() != 1 or Bq.dim() != 2 or Bq.shape[0] != d or Bq.stride(1) != 1:
        raise ValueError("Bq must be (d, m) 8-bit codes with unit column stride")
    m = Bq.shape[1]
    if scale.dtype != torch.float32 or scale.numel() != m or not scale.is_contiguous():
        raise ValueError("scale must be m contiguous fp32 values")
    if Bq.device != A.device or scale.device != A.device:
        raise ValueError("A, Bq and scale must live on one device")
    need = L.rmm_matmul_wq_workspace_size(n, d, m, float(rho))
    if need == ctypes.c_size_t(-1).value:
        raise RMMError(2, "rmm_matmul_wq_workspace_size")
    k = int(L.rmm_k(float(rho), d))
    if out is None:
        out = torch.empty((n, m), dtype=torch.bfloat16, device=A.device)
    elif tuple(out.shape) != (n, m) or out.dtype != torch.bfloat16 or out.stride(1) != 1 or out.device != A.device:
        raise ValueError("out has the wrong shape, dtype, layout or device")
    if idx_out is None:
        idx_out = torch.empty(k, dtype=torch.int32, device=A.device)
    else:
        check_out(idx_out, (k,), torch.int32, A.device, "idx_out")
    ws, wsb = _user_workspace(workspace, need, A.device)
    st = L.rmm_matmul_wq(A.data_ptr(), n, d, A.stride(0), Bq.data_ptr(), WQ_FORMATS[fmt], scale.data_ptr(), m,
                         Bq.stride(0), float(rho), float(alpha), out.data_ptr(), out.stride(0), idx_out.data_ptr(),
                         _ptr(ws), wsb, _stream(A))
    _check(st, "rmm_matmul_wq")
    return out, idx_out


def gated_mlp(x, Wgu, Wd, rho_in: float, rho_h: float, *, out=None, return_h: bool = False, workspace=None):
    """The gated MLP block with RMM on Up, Gate and Down (rmm_gated_mlp).

    x: bf16 (n, d); Wgu: from ``gated_weights``; Wd: bf16 (m, d).  Returns
    (Y, idx_in, idx_h) and h when ``return_h``."""
    torch = _torch()
    _require_gpu(x, Wgu, Wd)
    L = load()
    n, d = x.shape
    m = Wd.shape[0]
    if (x.dtype, Wgu.dtype, Wd.dtype) != (torch.bfloat16,) * 3 or Wgu.shape != (d, 2 * m) or Wd.shape != (m, d):
        raise ValueError("expected bf16 x (n, d), Wgu (d, 2m), Wd (m, d)")
    if not (x.is_contiguous() and Wgu.is_contiguous() and Wd.is_contiguous()):
        raise ValueError("operands must be contiguous")
    need = L.rmm_gated_mlp_workspace_size(n, d, m, float(rho_in), float(rho_h))
    if need == ctypes.c_size_t(-1).value:
        raise RMMError(2, "rmm_gated_mlp_workspace_size")
    k_in, k_h = int(L.rmm_k(float(rho_in), d)), int(L.rmm_k(float(rho_h), m))
    if Wgu.device != x.device or Wd.device != x.device:
        raise ValueError("x, Wgu and Wd must live on one device")
    if out is None:
        out = torch.empty((n, d), dtype=torch.bfloat16, device=x.device)
    else:
        check_out(out, (n, d), torch.bfloat16, x.device, "out")
    idx_in = torch.empty(k_in, dtype=torch.int32, device=x.device)
    idx_h = torch.empty(k_h, dtype=torch.int32, device=x.device)
    h = torch.empty((n, m), dtype=torch.bfloat16, device=x.device) if return_h else None
    ws, wsb = _user_workspace(workspace, need, x.device)
    st = L.rmm_gated_mlp(x.data_ptr(), Wgu.data_ptr(), Wd.data_ptr(), n, d, m, float(rho_in), float(rho_h),
                         out.data_ptr(), _ptr(h), idx_in.data_ptr(), idx_h.data_ptr(), _ptr(ws), wsb, _stream(x))
    _check(st, "rmm_gated_mlp")
    return (out, idx_in, idx_h, h) if return_h else (out, idx_in, idx_h)

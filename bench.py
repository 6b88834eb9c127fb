#!/usr/bin/env python3
"""Throughput of the reduced-matrix-multiplication path on one MI355X.

A step is one whole rmm_matmul -- column norms, TopK, gather, reduced product
-- on the largest layer product: the Llama-3.1-70B-shaped MLP up projection
A (4096 x 8192, bf16) x B (8192 x 28672, bf16) at rho = 0.8 (k = 6554), the
retention ratio of the paper's latency experiments.  ``value`` is 2 n k m / t
per step in TFLOP/s with every input resident in HBM: the steps rotate over
enough distinct (A, B) pairs that the working set exceeds the 256 MB Infinity
Cache.  Other workloads (the 8B projections, attention, decode, the gated
MLP block) are selected with --workload.

The same JSON line carries
  * ``median_ms_per_step``: from a second pass of the same K steps, the
    median over ten chunks of each chunk's mean ms per step (``ms_per_step``
    is the mean of the bracketed pass that ``value`` comes from);
  * ``sweep``: the path at each rho of the workload (and rho = 1 with the
    full path forced) with the dense bf16 torch.matmul (hipBLASLt) time and
    the speedup over it;
  * ``roofline``: the reduced-product GEMM kernel (the dominant kernel),
    timed per launch with HIP events recorded around it on its own stream,
    against the bf16 MFMA datasheet peak and against the matrix-core
    throughput measured on this GPU in the same run (``measured_peak``);
    ``traffic`` comes from committed rocprofv3 counters when they were taken
    on the current kernel source, else null;
  * ``clocks``: shader and memory clocks sampled from sysfs during the timed
    pass (null where the files cannot be read);
  * ``inputs_sha256``: digest of the bf16 input bytes;
  * ``cpu_baseline``: the CPU oracle timed on this host on a bounded sample
    (full norms and selection, a sample of output rows, extrapolated), and
    ``parity``: the GPU's kept set and sampled output rows against it.

With ``--jsonl FILE`` every measured (workload, rho) point is also appended
to FILE as a record of its own (the sweep points and the headline, with the
input digest, a digest of the library sources, ROCm and torch versions), and
``--resume`` reuses sweep points already in FILE for the same inputs and
sources instead of timing them again (the headline is always measured).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5]
                       [--jsonl FILE [--resume]]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "RMM layer TFLOP/s (2n⌈ρd⌉m/t) and speedup vs dense GEMM at ρ=0.5–1.0"
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E peak
MALL_BYTES = 256 << 20

WORKLOADS = {
    "c2": dict(case="c2", rho=0.8, sweep=(0.5, 0.7, 0.8, 1.0),
               label="Llama-3.1-8B-shaped projection: A 4096x4096 bf16 x B 4096x4096 bf16"),
    "c3": dict(case="c3", rho=0.8, sweep=(0.5, 0.7, 0.8, 1.0),
               label="Llama-3.1-8B-shaped MLP down projection: A 2048x14336 bf16 x B 14336x4096 bf16"),
    "c5": dict(case="c5", rho=0.8, sweep=(0.5, 0.7, 0.8, 1.0),
               label="Llama-3.1-70B-shaped MLP up projection: A 4096x8192 bf16 x B 8192x28672 bf16"),
    "c5-decode": dict(case="c5", rho=0.8, sweep=(0.8, 1.0), decode=True,
                      label="70B up projection decode: a 1x8192 bf16 x B 8192x28672 bf16"),
    "c4": dict(case="c4", rho=0.5, sweep=(0.5, 0.8, 1.0),
               label="QK^T with head-dim selection: Q 32x4096x128, K 8 GQA heads x4096x128 bf16"),
    "pv": dict(case="pv", rho=0.5, sweep=(0.5, 0.8, 1.0),
               label="attention value product with token selection: P 32x4096x4096 causal weights, "
                     "V 8 GQA heads x4096x128 bf16"),
    "c5-decode-fp8": dict(case="c5", rho=0.8, sweep=(0.8, 1.0), wq="fp8",
                          label="70B up projection decode over FP8 E4M3 weights with per-column scales: "
                                "a 1x8192 bf16 x B 8192x28672 fp8"),
    "c5-decode-int8": dict(case="c5", rho=0.8, sweep=(0.8, 1.0), wq="int8",
                           label="70B up projection decode over int8 weights with per-column scales: "
                                 "a 1x8192 bf16 x B 8192x28672 int8"),
    "c5-fp8": dict(case="c5", rho=0.8, sweep=(0.5, 0.8, 1.0), wqgemm="fp8",
                   label="70B up projection over FP8 E4M3 weights with per-column scales: A 4096x8192 bf16 x "
                         "B 8192x28672 fp8"),
    "c5-int8": dict(case="c5", rho=0.8, sweep=(0.5, 0.8, 1.0), wqgemm="int8",
                    label="70B up projection over int8 weights with per-column scales: A 4096x8192 bf16 x "
                          "B 8192x28672 int8"),
    "attn": dict(case="attn", rho=0.5, sweep=(0.5, 0.8, 1.0), attn=True,
                 label="causal attention with reduced scores, softmax fused: Q 32x4096x128, K/V 8 GQA heads "
                       "x4096x128 bf16"),
    "mlp": dict(case="mlp", rho=0.8, sweep=(0.5, 0.7, 0.8, 1.0), mlp=True,
                label="Llama-3.1-8B-shaped gated MLP block: x 2048x4096, Up/Gate 4096x14336, Down 14336x4096 bf16, "
                      "one rho for all three projections"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def code_text(text):
    """C++/HIP source without its comments and with whitespace runs collapsed:
    what decides the compiled kernels (string literals in these sources hold no
    comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def code_digest(path):
    """sha256 of code_text(path): unchanged by edits to comments or layout only."""
    with open(path, encoding="utf-8") as f:
        return hashlib.sha256(code_text(f.read()).encode()).hexdigest()


def library_digest():
    """sha256 over the library's HIP sources and headers, in name order."""
    import glob
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "input_adaptive_reduced_amd", "csrc")
    for p in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h")) +
                    [os.path.join(ROOT, "include", "rmm.h")]):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_jsonl(path):
    rows = []
    if path and os.path.exists(path):
        with open(path) as f:
            for ln in f:
                ln = ln.strip()
                if ln:
                    try:
                        rows.append(json.loads(ln))
                    except ValueError:
                        log(f"{path}: skipping a line that is not JSON")
    return rows


def reusable_point(rows, workload, rho, full_path, inputs, lib):
    """The last sweep record of FILE for this point, inputs and library sources."""
    if inputs is None:
        return None
    for r in reversed(rows):
        if (r.get("kind") == "sweep" and r.get("workload") == workload and r.get("rho") == rho
                and r.get("full_path") == full_path and r.get("inputs_sha256") == inputs
                and r.get("library_sha256") == lib):
            return r
    return None


# rocprofv3 FETCH_SIZE reads half the bytes a streaming read moves on this chip and
# WRITE_SIZE reads them exactly: factors from a 1 GiB device copy (``--calibrate-copy``)
FETCH_SCALE, WRITE_SCALE = 1.9999496949451407, 1.0
# the dominant kernel of each workload: (roofline key, kernel name fragment, source file)
TRAFFIC_KERNELS = {
    "c2": ("gemm", "gemm_tdma8_kernel", "gemm.hip"),
    "c3": ("gemm", "gemm_tdma8_kernel", "gemm.hip"),
    "c5": ("gemm", "gemm_tdma8_kernel", "gemm.hip"),
    "c5-fp8": ("gemm", "gemm_tdma_kernel", "gemm.hip"),
    "c5-int8": ("gemm", "gemm_tdma_kernel", "gemm.hip"),
    "c4": ("gemm", "gemm_stream_kernel", "gemm.hip"),
    "pv": ("gemm", "gemm_gcol_kernel", "gemm.hip"),
    "attn": ("gemm", "attn_fwd", "attention.hip"),
    "c5-decode": ("gemv", "decode_fused_kernel", "gemv.hip"),
    "c5-decode-fp8": ("gemv", "decode_fused_kernel", "gemv.hip"),
    "c5-decode-int8": ("gemv", "decode_fused_kernel", "gemv.hip"),
}


def short_kernel_name(name):
    """``void rmm::(anonymous namespace)::k<4>(rmm::Args)`` -> ``k<4>``."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):  # the argument list: the first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not name.startswith("(anonymous", i):
            cut = i
            break
    name = name[:cut]
    for ns in ("rmm::(anonymous namespace)::", "rmm::"):
        name = name.replace(ns, "")
    return name


def record_traffic(workload, fetch_csv, write_csv):
    """Average FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over the rows of a
    dispatch) of the workload's dominant kernel from two rocprofv3 --pmc runs of this
    script, scaled by the copy calibration, into profiles/traffic.json with the digests
    of the kernel's source file: the whole file's, and its code's without comments
    (code_digest; a later change of the code retires the record)."""
    import csv
    key, frag, src = TRAFFIC_KERNELS[workload]

    def per_dispatch(path, counter):
        vals, name = {}, None
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter or frag not in r["Kernel_Name"]:
                    continue
                name = short_kernel_name(r["Kernel_Name"])
                vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        if not vals:
            raise SystemExit(f"{path}: no {counter} rows for a kernel named like {frag!r}")
        return sum(vals.values()) / len(vals), len(vals), name

    fetch, nf, name = per_dispatch(fetch_csv, "FETCH_SIZE")
    write, nw, _ = per_dispatch(write_csv, "WRITE_SIZE")
    rel = os.path.join("input_adaptive_reduced_amd", "csrc", src)
    rec = {"kernel": name, "bytes_per_launch": fetch * 1024 * FETCH_SCALE + write * 1024 * WRITE_SCALE,
           "read_bytes": fetch * 1024 * FETCH_SCALE, "write_bytes": write * 1024 * WRITE_SCALE,
           "fetch_kib_raw": fetch, "write_kib_raw": write, "launches": [nf, nw],
           "fetch_scale": FETCH_SCALE, "write_scale": WRITE_SCALE,
           "source": rel, "source_sha256": source_digest(os.path.join(ROOT, rel)),
           "code_sha256": code_digest(os.path.join(ROOT, rel))}
    p = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(p):
        with open(p) as f:
            data = json.load(f)
    data[f"{key}@{workload}"] = rec
    with open(p, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({f"{key}@{workload}": rec}), flush=True)
    return 0


def load_traffic(kernel_key, workload):
    """HBM bytes per launch from committed rocprofv3 counters, if still current."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            rec = json.load(f).get(f"{kernel_key}@{workload}")
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src) or code_digest(src) != rec.get("code_sha256"):
        return None
    return rec.get("bytes_per_launch")


class Runner:
    """Prepared inputs, outputs and workspaces for one workload."""

    def __init__(self, torch, rmm, case, decode, copies):
        import numpy as np
        import synthetic
        self.torch, self.rmm = torch, rmm
        dev = torch.device("cuda:0")
        self.case = case
        self.batched = case.A.ndim == 3
        if decode:
            case = synthetic.make_decode_case(case)
        self.A_host = case.A
        self.B_host = case.B

        def up(x):
            bits = synthetic.as_bf16_bits(np.ascontiguousarray(x)).view(np.int16)
            return torch.from_numpy(bits).to(dev).view(torch.bfloat16)

        A0, B0 = up(case.A), up(case.B)
        self.sha256 = synthetic.sha256_of(synthetic.as_bf16_bits(case.A), synthetic.as_bf16_bits(case.B))
        per_set = A0.numel() * 2 + B0.numel() * 2
        if copies is None:
            copies = max(2, min(16, math.ceil(2 * MALL_BYTES / per_set)))
        self.copies = copies
        self.A = [A0] + [A0.clone() for _ in range(copies - 1)]
        self.B = [B0] + [B0.clone() for _ in range(copies - 1)]
        self.transB = case.transB
        self.group = case.group
        self.alpha = case.alpha
        if self.batched:
            self.n, self.d = case.A.shape[1], case.A.shape[2]
            self.m = case.B.shape[1] if case.transB else case.B.shape[2]
            self.batch = case.A.shape[0]
        else:
            self.n, self.d = case.A.shape
            self.m = case.B.shape[1]
            self.batch = 1
        shape = (self.batch, self.n, self.m) if self.batched else (self.n, self.m)
        self.Y = [torch.empty(shape, dtype=torch.bfloat16, device=dev) for _ in range(copies)]
        self.ws = {}
        self.idx = {}

    def flops(self, rho):
        k = self.rmm.k_of(rho, self.d)
        return 2.0 * self.batch * self.n * k * self.m

    def call(self, i, rho, full_path=False):
        rmm = self.rmm
        key = (rho, full_path)
        if key not in self.ws:
            need = rmm.workspace_size(self.A[0], self.B[0], rho, transB=self.transB, b_group=self.group,
                                      full_path=full_path)
            self.ws[key] = self.torch.empty(max(1, need), dtype=self.torch.uint8, device="cuda:0")
            k = rmm.k_of(rho, self.d)
            self.idx[key] = self.torch.empty(self.batch * k, dtype=self.torch.int32, device="cuda:0")
        rmm.matmul(self.A[i], self.B[i], rho, transB=self.transB, b_group=self.group, alpha=self.alpha,
                   out=self.Y[i], idx_out=self.idx[key], workspace=self.ws[key], full_path=full_path)

    def plan(self, rho):
        """Kernels the library picks for this workload (host-side query)."""
        return self.rmm.plan_info(self.A[0], self.B[0], rho, transB=self.transB, b_group=self.group)

    def dense(self, i):
        """Dense bf16 product of the same shape (hipBLASLt through torch)."""
        torch = self.torch
        if self.batched:
            # the right operand per query head (K^T, or V), materialised once
            # outside the timed region as a plain contiguous tensor
            if not hasattr(self, "_kt"):
                self._kt = [(b.transpose(1, 2) if self.transB else b).repeat_interleave(self.group, dim=0)
                            .contiguous() for b in self.B]
            torch.baddbmm(self.Y[i], self.A[i], self._kt[i], beta=0.0, alpha=self.alpha, out=self.Y[i])
            return
        if self.transB:
            torch.matmul(self.A[i], self.B[i].t(), out=self.Y[i])
        else:
            torch.matmul(self.A[i], self.B[i], out=self.Y[i])


class WQRunner:
    """Single-row decode over 8-bit weights (rmm_decode_wq); the dense
    comparison is the bf16 GEMV over the unquantized weights."""

    def __init__(self, torch, rmm, fmt, copies):
        import numpy as np
        import synthetic
        self.torch, self.rmm, self.fmt = torch, rmm, fmt
        dev = torch.device("cuda:0")
        base = synthetic.make_case("c5", dict(n=1))
        dec = synthetic.make_decode_case(base)
        codes, scale = synthetic.quantize_columns(base.B, fmt)
        self.a_host, self.codes_host, self.scale_host = dec.A, codes, scale
        self.sha256 = synthetic.sha256_of(synthetic.as_bf16_bits(dec.A), codes, scale)

        def up(x):
            bits = synthetic.as_bf16_bits(np.ascontiguousarray(x)).view(np.int16)
            return torch.from_numpy(bits).to(dev).view(torch.bfloat16)

        a0, q0, s0 = up(dec.A.reshape(-1)), torch.from_numpy(codes).to(dev), torch.from_numpy(scale).to(dev)
        self.d, self.m = codes.shape
        if copies is None:
            copies = max(2, min(16, math.ceil(2 * MALL_BYTES / q0.numel())))
        self.copies = copies
        self.a = [a0] + [a0.clone() for _ in range(copies - 1)]
        self.Bq = [q0] + [q0.clone() for _ in range(copies - 1)]
        self.scale = [s0] + [s0.clone() for _ in range(copies - 1)]
        self.B16 = up(base.B)
        self.n, self.batch = 1, 1
        self.Y = [torch.empty(self.m, dtype=torch.bfloat16, device=dev) for _ in range(copies)]
        self.Yd = torch.empty((1, self.m), dtype=torch.bfloat16, device=dev)
        self.ws, self.idx = {}, {}

    def flops(self, rho):
        return 2.0 * self.rmm.k_of(rho, self.d) * self.m

    def call(self, i, rho, full_path=False):
        import ctypes
        torch, rmm = self.torch, self.rmm
        if rho not in self.ws:
            need = rmm.load().rmm_decode_wq_workspace_size(self.d, self.m, rho)
            if need == ctypes.c_size_t(-1).value:
                raise rmm.RMMError(2, "rmm_decode_wq_workspace_size")
            self.ws[rho] = torch.empty(need, dtype=torch.uint8, device="cuda:0")
            self.idx[rho] = torch.empty(rmm.k_of(rho, self.d), dtype=torch.int32, device="cuda:0")
        rmm.decode_wq(self.a[i], self.Bq[i], self.scale[i], rho, self.fmt, out=self.Y[i], idx_out=self.idx[rho],
                      workspace=self.ws[rho])

    def plan(self, rho):
        return {"route": "decode", "gemm": None, "splits": None}

    def dense(self, i):
        # one weight copy: the dense GEMV streams all 470 MB of it, twice the MALL
        self.torch.matmul(self.a[i].view(1, -1), self.B16, out=self.Yd)


class WQGemmRunner:
    """The reduced product over 8-bit weights (rmm_matmul_wq) on the 70B up
    projection; the dense comparison is the bf16 product over the unquantized
    weights (hipBLASLt through torch.matmul)."""

    def __init__(self, torch, rmm, fmt, copies):
        import numpy as np
        import synthetic
        self.torch, self.rmm, self.fmt = torch, rmm, fmt
        dev = torch.device("cuda:0")
        base = synthetic.make_case("c5")
        codes, scale = synthetic.quantize_columns(base.B, fmt)
        self.A_host, self.codes_host, self.scale_host = base.A, codes, scale
        self.sha256 = synthetic.sha256_of(synthetic.as_bf16_bits(base.A), codes, scale)

        def up(x):
            bits = synthetic.as_bf16_bits(np.ascontiguousarray(x)).view(np.int16)
            return torch.from_numpy(bits).to(dev).view(torch.bfloat16)

        A0, q0, s0 = up(base.A), torch.from_numpy(codes).to(dev), torch.from_numpy(scale).to(dev)
        self.n, self.d = base.A.shape
        self.m = codes.shape[1]
        if copies is None:
            copies = max(2, min(16, math.ceil(2 * MALL_BYTES / (A0.numel() * 2 + q0.numel()))))
        self.copies = copies
        self.A = [A0] + [A0.clone() for _ in range(copies - 1)]
        self.Bq = [q0] + [q0.clone() for _ in range(copies - 1)]
        self.scale = [s0] + [s0.clone() for _ in range(copies - 1)]
        self.B16 = up(base.B)  # one copy: 470 MB, above the MALL on its own
        self.batch, self.batched = 1, False
        self.Y = [torch.empty((self.n, self.m), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
        self.ws, self.idx = {}, {}

    def flops(self, rho):
        return 2.0 * self.n * self.rmm.k_of(rho, self.d) * self.m

    def call(self, i, rho, full_path=False):
        import ctypes
        torch, rmm = self.torch, self.rmm
        key = (rho, False)
        if key not in self.ws:
            need = rmm.load().rmm_matmul_wq_workspace_size(self.n, self.d, self.m, rho)
            if need == ctypes.c_size_t(-1).value:
                raise rmm.RMMError(2, "rmm_matmul_wq_workspace_size")
            self.ws[key] = torch.empty(need, dtype=torch.uint8, device="cuda:0")
            self.idx[key] = torch.empty(rmm.k_of(rho, self.d), dtype=torch.int32, device="cuda:0")
        rmm.matmul_wq(self.A[i], self.Bq[i], self.scale[i], rho, self.fmt, out=self.Y[i], idx_out=self.idx[key],
                      workspace=self.ws[key])

    def plan(self, rho):
        return {"route": "mfma", "gemm": "tdma_" + self.fmt, "splits": 1}

    def dense(self, i):
        self.torch.matmul(self.A[i], self.B16, out=self.Y[i])


class AttnRunner:
    """Attention with reduced scores and the softmax fused (rmm_attention);
    the dense comparison is torch's fused attention kernel (flash or
    memory-efficient backend only) over the full head dimension."""

    def __init__(self, torch, rmm, copies):
        import numpy as np
        import synthetic
        self.torch, self.rmm = torch, rmm
        dev = torch.device("cuda:0")
        Q, K, V = synthetic.make_attention_case()
        self.sha256 = synthetic.sha256_of(*(synthetic.as_bf16_bits(x) for x in (Q, K, V)))

        def up(x):
            bits = synthetic.as_bf16_bits(np.ascontiguousarray(x)).view(np.int16)
            return torch.from_numpy(bits).to(dev).view(torch.bfloat16)

        q0, k0, v0 = up(Q), up(K), up(V)
        per_set = (q0.numel() + k0.numel() + v0.numel()) * 2
        if copies is None:
            copies = max(2, min(16, math.ceil(2 * MALL_BYTES / per_set)))
        self.copies = copies
        self.q = [q0] + [q0.clone() for _ in range(copies - 1)]
        self.k = [k0] + [k0.clone() for _ in range(copies - 1)]
        self.v = [v0] + [v0.clone() for _ in range(copies - 1)]
        self.H, self.L, self.dh = Q.shape
        self.Hkv, self.dv = V.shape[0], V.shape[2]
        self.n, self.d, self.m, self.batch = self.L, self.dh, self.dv, self.H
        self.O = [torch.empty((self.H, self.L, self.dv), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
        self.ws, self.idx = {}, {}
        self._kx = None

    def flops(self, rho):
        # causal pairs x (reduced scores + value product), per head
        pairs = self.L * (self.L + 1) / 2
        return 2.0 * self.H * pairs * (self.rmm.k_of(rho, self.dh) + self.dv)

    def call(self, i, rho, full_path=False):
        import ctypes
        torch, rmm = self.torch, self.rmm
        if rho not in self.ws:
            need = rmm.load().rmm_attention_workspace_size(self.H, self.Hkv, self.L, self.L, self.dh, rho)
            if need == ctypes.c_size_t(-1).value:
                raise rmm.RMMError(2, "rmm_attention_workspace_size")
            self.ws[rho] = torch.empty(need, dtype=torch.uint8, device="cuda:0")
            self.idx[rho] = torch.empty((self.H, rmm.k_of(rho, self.dh)), dtype=torch.int32, device="cuda:0")
        rmm.attention(self.q[i], self.k[i], self.v[i], rho, causal=True, out=self.O[i], idx_out=self.idx[rho],
                      workspace=self.ws[rho])

    def plan(self, rho):
        return {"route": "attention", "gemm": "attn_fwd", "splits": 1}

    def dense(self, i):
        torch = self.torch
        from torch.nn.attention import SDPBackend, sdpa_kernel
        if self._kx is None:
            g = self.H // self.Hkv
            self._kx = [kk.repeat_interleave(g, dim=0).contiguous() for kk in self.k]
            self._vx = [vv.repeat_interleave(g, dim=0).contiguous() for vv in self.v]
        # fused kernels only: never the unfused bf16 math path
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            self.O[i].copy_(torch.nn.functional.scaled_dot_product_attention(
                self.q[i].unsqueeze(0), self._kx[i].unsqueeze(0), self._vx[i].unsqueeze(0), is_causal=True)[0])


class MLPRunner:
    """The gated MLP block (rmm_gated_mlp) with its inputs, rotated over copies."""

    def __init__(self, torch, rmm, copies):
        import numpy as np
        import synthetic
        self.torch, self.rmm = torch, rmm
        dev = torch.device("cuda:0")
        c = synthetic.make_mlp_case()
        self.sha256 = synthetic.sha256_of(*(synthetic.as_bf16_bits(x) for x in (c.x, c.Wg, c.Wu, c.Wd)))

        def up(x):
            bits = synthetic.as_bf16_bits(np.ascontiguousarray(x)).view(np.int16)
            return torch.from_numpy(bits).to(dev).view(torch.bfloat16)

        x0, Wg0, Wu0, Wd0 = up(c.x), up(c.Wg), up(c.Wu), up(c.Wd)
        Wgu0 = rmm.gated_weights(Wg0, Wu0)
        per_set = (x0.numel() + Wgu0.numel() + Wd0.numel()) * 2
        if copies is None:
            copies = max(2, min(16, math.ceil(2 * MALL_BYTES / per_set)))
        self.copies = copies
        self.x = [x0] + [x0.clone() for _ in range(copies - 1)]
        self.Wgu = [Wgu0] + [Wgu0.clone() for _ in range(copies - 1)]
        self.Wd = [Wd0] + [Wd0.clone() for _ in range(copies - 1)]
        self.Wg = [Wg0] + [Wg0.clone() for _ in range(copies - 1)]
        self.Wu = [Wu0] + [Wu0.clone() for _ in range(copies - 1)]
        self.n, self.d = c.x.shape
        self.m = c.Wg.shape[1]
        self.batch = 1
        self.Y = [torch.empty((self.n, self.d), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
        self.G = torch.empty((self.n, self.m), dtype=torch.bfloat16, device=dev)
        self.U = torch.empty((self.n, self.m), dtype=torch.bfloat16, device=dev)
        self.ws = {}
        self.idx = {}

    def flops(self, rho):
        k_in, k_h = self.rmm.k_of(rho, self.d), self.rmm.k_of(rho, self.m)
        return 2.0 * self.n * k_in * 2 * self.m + 2.0 * self.n * k_h * self.d

    def call(self, i, rho, full_path=False):
        torch, rmm = self.torch, self.rmm
        if rho not in self.ws:
            import ctypes
            need = rmm.load().rmm_gated_mlp_workspace_size(self.n, self.d, self.m, rho, rho)
            if need == ctypes.c_size_t(-1).value:
                raise rmm.RMMError(2, "rmm_gated_mlp_workspace_size")
            self.ws[rho] = torch.empty(need, dtype=torch.uint8, device="cuda:0")
        rmm.gated_mlp(self.x[i], self.Wgu[i], self.Wd[i], rho, rho, out=self.Y[i], workspace=self.ws[rho])

    def plan(self, rho):
        return {"route": "mfma", "gemm": "tdma", "splits": 1}

    def dense(self, i):
        """The dense block as torch runs it: Gate and Up products, SiLU * up, Down product."""
        torch = self.torch
        torch.matmul(self.x[i], self.Wg[i], out=self.G)
        torch.matmul(self.x[i], self.Wu[i], out=self.U)
        h = torch.nn.functional.silu(self.G)
        h.mul_(self.U)
        torch.matmul(h, self.Wd[i], out=self.Y[i])


def time_steps(torch, fn, steps, warmup, copies, graph, clocks=None, median=False):
    """Mean ms per step over `steps` calls of fn(i) rotating over copies.

    With graphs, each input set's step is captured once (after one eager call
    per set on the capture stream); the `warmup` untimed steps are then replays
    of the same graphs the timed steps replay, so the timed region starts with
    the GPU already running that exact work."""
    if graph:
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(copies):
                fn(i)  # warm the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn(i)
            graphs.append(g)
        run = lambda i: graphs[i % copies].replay()  # noqa: E731
    else:
        run = lambda i: fn(i % copies)  # noqa: E731
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with (clocks if clocks is not None else _Null()):
        start.record()
        for i in range(steps):
            run(i)
        stop.record()
        torch.cuda.synchronize()
    mean = start.elapsed_time(stop) / steps
    if median:
        return mean, step_median(torch, fn, steps, copies, run)
    return mean


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


def step_median(torch, fn, steps, copies, graph_runs=None, chunks=10):
    """Median over ``chunks`` consecutive chunks of the K steps of the mean
    ms per step in each chunk (a separate pass; events sit only between
    chunks, so short steps are not inflated by per-step event records)."""
    run = graph_runs if graph_runs is not None else (lambda i: fn(i % copies))
    chunks = max(1, min(chunks, steps))
    sizes = [steps // chunks + (1 if c < steps % chunks else 0) for c in range(chunks)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(chunks + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    i = 0
    for c, n in enumerate(sizes):
        for _ in range(n):
            run(i)
            i += 1
        ev[c + 1].record()
    torch.cuda.synchronize()
    t = sorted(ev[c].elapsed_time(ev[c + 1]) / n for c, n in enumerate(sizes))
    return t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2])


class ClockSampler:
    """Polls the GPU's current shader and memory clock levels from sysfs
    (pp_dpm_sclk / pp_dpm_mclk of the PCI device torch reports) on a
    background thread while a region runs; the readings are MHz values of
    the level marked current."""

    def __init__(self, torch):
        self.paths = None
        try:
            p = torch.cuda.get_device_properties(0)
            dev = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
            paths = {k: os.path.join(dev, f"pp_dpm_{k}") for k in ("sclk", "mclk")}
            if all(os.access(v, os.R_OK) for v in paths.values()):
                self.paths = paths
                self.device = dev
                with open(paths["sclk"]) as f:  # the driver's level table, as read before the region
                    self.table = " | ".join(ln.strip() for ln in f if ln.strip())
        except Exception:  # noqa: BLE001  (no sysfs, no PCI id: report null)
            self.paths = None
        self.samples = {"sclk": [], "mclk": []}
        self._stop = None

    @staticmethod
    def _current(path):
        with open(path) as f:
            for ln in f:
                if ln.rstrip().endswith("*"):
                    tok = ln.split(":", 1)[1].strip().split()[0]
                    return float(tok.lower().replace("mhz", ""))
        return None

    def __enter__(self):
        import threading
        if self.paths:
            self._stop = threading.Event()

            def poll():
                while not self._stop.is_set():
                    for k, p in self.paths.items():
                        try:
                            v = self._current(p)
                        except (OSError, ValueError, IndexError):
                            v = None
                        if v is not None:
                            self.samples[k].append(v)
                    self._stop.wait(0.002)

            self._thread = threading.Thread(target=poll, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._stop is not None:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if not self.paths or not self.samples["sclk"]:
            return None
        out = {"source": self.device + "/pp_dpm_{sclk,mclk} (the DPM level the driver marks current)",
               "note": "the driver's reported level, polled between launches: it lags the hardware and "
                       "often shows an idle level under load; the shader clock measured inside running "
                       "waves is roofline.measured_peak_shader_mhz (matrix-core probe)",
               "samples": len(self.samples["sclk"]), "sclk_levels": getattr(self, "table", None)}
        for k, v in self.samples.items():
            if v:
                v = sorted(v)
                out[f"{k}_mhz_median"] = v[len(v) // 2]
                out[f"{k}_mhz_min"] = v[0]
                out[f"{k}_mhz_max"] = v[-1]
        return out


def kernel_times(torch, rmm, runner, rho, steps, copies):
    """Per-kernel mean ms from HIP events the library records around each launch."""
    rmm.timing_enable(True, capacity=steps * 64)
    rmm.timing_collect()
    for i in range(steps):
        runner.call(i % copies, rho)
    torch.cuda.synchronize()
    rec = rmm.timing_collect()
    rmm.timing_enable(False)
    return {kname: (ms / cnt if cnt else 0.0, cnt / steps) for kname, (ms, cnt) in rec.items()}


def cpu_baseline(runner, rho, budget_s=12.0, gpu=None):
    """The oracle as it stands, on this host's cores: full norms and selection,
    the product on a sample of output rows, extrapolated to the whole job.

    ``gpu`` (optional) is (idx, Y) of the GPU's own call on the same inputs
    (batch entry 0): its kept set is compared with the oracle's in full and
    its sampled rows with the oracle's rows (``parity`` in the result)."""
    import numpy as np
    import oracle
    threads = oracle.host_threads()
    A = runner.A_host if not runner.batched else runner.A_host[0]
    B = runner.B_host if not runner.batched else np.ascontiguousarray(
        runner.B_host[0].T if runner.transB else runner.B_host[0])
    n, d = A.shape
    m = B.shape[1]
    A64 = np.ascontiguousarray(A, dtype=np.float64)
    B64 = np.ascontiguousarray(B, dtype=np.float64)
    k = oracle.k_of(rho, d)
    t0 = time.perf_counter()
    s = oracle.colnorm(A64)
    idx = oracle.topk(s, k)
    t_sel = time.perf_counter() - t0
    probe = min(n, max(threads, 8))
    t0 = time.perf_counter()
    oracle.reduced_product(A64, B64, idx, 1.0, rows=list(range(probe)), threads=threads)
    t_probe = time.perf_counter() - t0
    rows = int(min(n, max(probe, probe * budget_s / max(t_probe, 1e-6))))
    rows = max(threads, rows // threads * threads) if rows >= threads else rows
    rng = np.random.default_rng(0)
    sample = np.sort(rng.choice(n, size=rows, replace=False))
    t0 = time.perf_counter()
    oracle.reduced_product(A64, B64, idx, 1.0, rows=sample, threads=threads)
    t_rows = time.perf_counter() - t0
    per_matrix = t_sel + t_rows * n / rows
    total = per_matrix * runner.batch
    value = 2.0 * runner.batch * n * k * m / total / 1e12
    parity = None
    if gpu is not None:
        g_idx, g_Y = gpu
        cmp_rows = sample[::max(1, sample.size // 256)][:256]  # spread over the sample
        Y_ref = oracle.reduced_product(A64, B64, idx, 1.0, rows=cmp_rows, threads=threads)
        Y_got = g_Y[cmp_rows].astype(np.float64)
        order = np.sort(s)[::-1]
        parity = {"idx_exact": bool(np.array_equal(g_idx, idx)),
                  "rel_frobenius": float(np.linalg.norm(Y_got - Y_ref) / np.linalg.norm(Y_ref)),
                  "rows_compared": int(cmp_rows.size), "tolerance": 1e-2,
                  "boundary_rel_gap": float((order[k - 1] - order[k]) / order[k - 1]) if k < d else None,
                  "what": "GPU kept set vs the oracle's fp64 full-sort TopK (all of it); GPU output rows vs the "
                          "oracle's fp64 triple-loop rows (relative Frobenius error over the compared rows)"}
    return {"value": value, "unit": "TFLOP/s", "cores": threads, "kind": "oracle", "parity": parity,
            "sample": (f"fp64 oracle: full column norms + full-sort TopK of one {n}x{d} matrix "
                       f"({t_sel:.2f} s) and the reduced product for {rows} of {n} output rows "
                       f"({t_rows:.2f} s)" +
                       (", extrapolated to all rows" if rows < n else " (the whole product)") +
                       (f"; one of {runner.batch} heads, scaled to all" if runner.batch > 1 else "")),
            "seconds_measured": t_sel + t_rows + t_probe}


def cpu_baseline_wqgemm(runner, rho, gpu, budget_s=12.0):
    """The oracle's reduced product over 8-bit weights on this host: the
    per-matrix part (codes decoded and scaled, norms, full-sort TopK) timed
    whole, the triple-loop product on a sample of output rows, extrapolated
    to all rows; plus the GPU's kept set and rows against it."""
    import numpy as np
    import oracle
    threads = oracle.host_threads()
    A, codes, scale = runner.A_host, runner.codes_host, runner.scale_host
    n = A.shape[0]
    t0 = time.perf_counter()
    B = oracle.dequantize(codes, runner.fmt, scale)
    sel = oracle.rmm(A, None, rho)
    t_mat = time.perf_counter() - t0
    k = sel.k
    probe = max(threads, 8)
    t0 = time.perf_counter()
    oracle.reduced_product(A, B, sel.idx, 1.0, rows=list(range(probe)), threads=threads)
    t_probe = time.perf_counter() - t0
    rows = int(min(n, max(probe, probe * budget_s / max(t_probe, 1e-6))))
    rows = max(threads, rows // threads * threads)
    sample = np.sort(np.random.default_rng(0).choice(n, size=rows, replace=False))
    t0 = time.perf_counter()
    Y_ref = oracle.reduced_product(A, B, sel.idx, 1.0, rows=sample, threads=threads)
    t_rows = time.perf_counter() - t0
    total = t_mat + t_rows * n / rows
    value = 2.0 * n * k * runner.m / total / 1e12
    g_idx, g_Y = gpu
    Y_got = g_Y[sample].astype(np.float64)
    order = np.sort(sel.s)[::-1]
    parity = {"idx_exact": bool(np.array_equal(g_idx, sel.idx)),
              "rel_frobenius": float(np.linalg.norm(Y_got - Y_ref) / np.linalg.norm(Y_ref)),
              "rows_compared": int(rows), "tolerance": 1e-2,
              "boundary_rel_gap": float((order[k - 1] - order[k]) / order[k - 1]) if k < order.size else None,
              "what": "GPU kept set vs the oracle's fp64 full-sort TopK; GPU output rows vs the oracle's fp64 "
                      "rows over the dequantized weights"}
    return {"value": value, "unit": "TFLOP/s", "cores": threads, "kind": "oracle", "parity": parity,
            "sample": f"fp64 oracle over {runner.fmt} weights: codes decoded and scaled, norms and full-sort TopK of "
                      f"the {n}x{A.shape[1]} block ({t_mat:.2f} s), the product for {rows} of {n} rows "
                      f"({t_rows:.2f} s), extrapolated to all rows",
            "seconds_measured": t_mat + t_probe + t_rows}


def cpu_baseline_attn(runner, rho, rows=256):
    """The oracle's attention for one head on a row sample (norms, TopK and
    the reduced scores of those rows, softmax, value product), scaled to the
    whole layer by causal pairs."""
    import numpy as np
    import synthetic
    import oracle
    Q, K, V = synthetic.make_attention_case()
    L = Q.shape[1]
    sample = np.sort(np.random.default_rng(0).choice(L, size=rows, replace=False))
    t0 = time.perf_counter()
    oracle.attention(Q, K, V, rho, causal=True, heads=[0], rows=sample)
    t = time.perf_counter() - t0
    pairs_sample = float(np.sum(sample + 1))
    k = oracle.k_of(rho, Q.shape[2])
    flops = 2.0 * pairs_sample * (k + V.shape[2])
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.host_threads(), "kind": "oracle",
            "sample": f"fp64 oracle attention of head 0 for {rows} of {L} query rows (column norms and TopK of the "
                      f"whole head, reduced scores of the sampled rows, causal softmax, value product; {t:.2f} s), "
                      "rate over those rows' causal pairs",
            "seconds_measured": t}


def cpu_baseline_wq(runner, rho):
    """The oracle's whole 8-bit-weight decode (decode, select, product) on this host."""
    import oracle
    t0 = time.perf_counter()
    oracle.decode_wq(runner.a_host, runner.codes_host, runner.fmt, runner.scale_host, rho)
    t = time.perf_counter() - t0
    k = oracle.k_of(rho, runner.d)
    return {"value": 2.0 * k * runner.m / t / 1e12, "unit": "TFLOP/s", "cores": oracle.host_threads(),
            "kind": "oracle",
            "sample": f"the whole fp64 oracle decode: {runner.fmt} codes decoded and scaled ({runner.d}x{runner.m}), "
                      f"|a| TopK, the reduced row product ({t:.2f} s)",
            "seconds_measured": t}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="c5", choices=sorted(WORKLOADS))
    ap.add_argument("--copies", type=int, default=None, help="input sets rotated over (default: > 2x MALL)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--kernel-steps", type=int, default=50, help="steps for per-kernel event timing")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB a few times (the reference kernel "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings) and exit")
    ap.add_argument("--calibrate-mfma", action="store_true",
                    help="only run the matrix-core ceiling probe and print its TFLOP/s")
    ap.add_argument("--no-mfma-ceiling", action="store_true", help="skip the matrix-core ceiling probe")
    ap.add_argument("--jsonl", metavar="FILE", help="also append one record per measured (workload, rho) point")
    ap.add_argument("--resume", action="store_true",
                    help="with --jsonl: reuse sweep points FILE already holds for the same inputs and sources")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: store the HBM bytes of --workload's dominant kernel from the counter_collection "
                         "CSVs of two rocprofv3 runs of this script (--pmc FETCH_SIZE, then --pmc WRITE_SIZE) "
                         "in profiles/traffic.json, and exit")
    args = ap.parse_args(argv)
    if args.resume and not args.jsonl:
        ap.error("--resume needs --jsonl")
    if args.record_traffic:
        return record_traffic(args.workload, *args.record_traffic)

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        return 2
    rank = int(os.environ.get("RANK", "0"))

    import torch
    import input_adaptive_reduced_amd as rmm
    import synthetic
    rmm.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": nbytes, "bytes_written": nbytes,
                          "launches": 5}), flush=True)
        return 0

    if args.calibrate_mfma:
        cal = rmm.calibrate_mfma()
        print(json.dumps({"calibration": "bf16 matrix-core ceiling", **cal}), flush=True)
        return 0

    wl = WORKLOADS[args.workload]
    is_mlp = wl.get("mlp", False)
    is_wq = "wq" in wl
    is_attn = wl.get("attn", False)
    is_wqgemm = "wqgemm" in wl
    if is_wqgemm:
        runner = WQGemmRunner(torch, rmm, wl["wqgemm"], args.copies)
    elif is_mlp:
        runner = MLPRunner(torch, rmm, args.copies)
    elif is_attn:
        runner = AttnRunner(torch, rmm, args.copies)
    elif is_wq:
        runner = WQRunner(torch, rmm, wl["wq"], args.copies)
    else:
        case = synthetic.make_pv_case() if wl["case"] == "pv" else synthetic.make_case(wl["case"])
        runner = Runner(torch, rmm, case, wl.get("decode", False), args.copies)
    rho = wl["rho"]
    graph = not args.no_graph
    log(f"workload {args.workload}: {wl['label']}; copies={runner.copies} graph={graph}")

    inputs_sha = getattr(runner, "sha256", None)
    lib_sha = library_digest()
    previous = read_jsonl(args.jsonl) if args.resume else []
    common = {"workload": args.workload, "n": runner.n, "d": runner.d, "m": runner.m, "batch": runner.batch,
              "inputs_sha256": inputs_sha, "library_sha256": lib_sha, "hip": getattr(torch.version, "hip", None),
              "torch": torch.__version__, "graph": graph, "steps": args.steps, "warmup": args.warmup}

    # the dense comparison and the rho sweep run first: the headline below then starts
    # from a GPU at its working clock, not from the cold-start transient
    sweep = []
    points = [(r, full) for r in wl["sweep"]
              for full in ((False, True) if r == 1.0 and not (is_mlp or is_wq or is_attn or is_wqgemm) else (False,))]
    reused = {pt: reusable_point(previous, args.workload, pt[0], pt[1], inputs_sha, lib_sha) for pt in points}
    if not args.no_sweep and all(reused.values()):
        for pt in points:
            ent = {kk: reused[pt][kk] for kk in ("rho", "k", "full_path", "ms", "tflops", "dense_ms",
                                                  "speedup_vs_dense", "ideal_speedup") if kk in reused[pt]}
            ent["reused"] = True
            sweep.append(ent)
        log(f"sweep: all {len(points)} points reused from {args.jsonl}")
    elif not args.no_sweep:
        try:
            runner.dense(0)
            torch.cuda.synchronize()
        except RuntimeError as e:  # e.g. no fused attention kernel for this GPU in this torch build
            log(f"dense comparison unavailable: {e}")
            dense_ms = None
        else:
            dense_ms = time_steps(torch, runner.dense, args.steps, args.warmup, runner.copies, graph)
            log(f"dense {'fused attention' if is_attn else 'torch.matmul'}: {dense_ms * 1e3:.1f} us/step")
        for r, full in points:
            t = time_steps(torch, lambda i: runner.call(i, r, full), args.steps, args.warmup,
                           runner.copies, graph)
            ent = {"rho": r, "k": rmm.k_of(r, runner.d), "full_path": full, "ms": t,
                   "tflops": runner.flops(r) / (t * 1e-3) / 1e12}
            if dense_ms:
                ent["dense_ms"] = dense_ms
                ent["speedup_vs_dense"] = dense_ms / t
                ent["ideal_speedup"] = 1.0 / (ent["k"] / runner.d)
            sweep.append(ent)
            log(f"  rho={r}{' full' if full else ''}: {t * 1e3:.1f} us, {ent['tflops']:.1f} TFLOP/s"
                + (f", x{ent['speedup_vs_dense']:.2f} vs dense" if dense_ms else ""))

    clocks = ClockSampler(torch)
    ms, med = time_steps(torch, lambda i: runner.call(i, rho), args.steps, args.warmup, runner.copies, graph,
                         clocks=clocks, median=True)
    value = runner.flops(rho) / (ms * 1e-3) / 1e12
    k = rmm.k_of(rho, runner.d)
    log(f"rho={rho} k={k}: {ms * 1e3:.1f} us/step (median {med * 1e3:.1f}), {value:.1f} TFLOP/s; "
        f"clocks {clocks.summary()}")

    kt = kernel_times(torch, rmm, runner, rho, args.kernel_steps, runner.copies)
    log("per-kernel us per step: " + ", ".join(f"{kk}={v[0] * v[1] * 1e3:.1f}" + (f" ({v[1]:g} launches)" if v[1] != 1 else "")
                                           for kk, v in kt.items() if v[1]))
    stream = runner.plan(rho)["gemm"] == "stream"
    if is_attn:
        # the fused attention kernel: reduced scores and value product on the matrix cores
        dom = "gemm"
        gemm_ms = kt["gemm"][0]
        achieved = runner.flops(rho) / (gemm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "attn_fwd", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "algorithmic_flops": runner.flops(rho),
                "kernel_ms": gemm_ms}
    elif runner.n == 1:
        dom, bound = "gemv", "hbm"
        gemv_ms = kt["gemv"][0]
        if is_wq:  # kept 8-bit rows + a + column scales + fp32 partial row
            algo_bytes = k * runner.m + runner.d * 2 + runner.m * 8
        else:      # kept B rows + a + fp32 partial row
            algo_bytes = k * runner.m * 2 + runner.d * 2 + runner.m * 4
        achieved = algo_bytes / (gemv_ms * 1e-3) / 1e9
        # from 28 x 512 output columns on the library selects inside the GEMV (gemv.hip)
        roof = {"bound": "hbm", "kernel": "decode_fused" if runner.m >= 28 * 512 else "gemv_partial",
                "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes": algo_bytes,
                "kernel_ms": gemv_ms}
    elif runner.plan(rho)["gemm"] == "gcol":
        # narrow product (attention's P V): bound by reading the kept entries of A
        dom = "gemm"
        gemm_ms = kt["gemm"][0] * max(1.0, kt["gemm"][1])
        algo_bytes = 2 * runner.batch * (runner.n * k + k * runner.m + runner.n * runner.m)
        achieved = algo_bytes / (gemm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "gemm_gcol", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes": algo_bytes,
                "kernel_ms": gemm_ms}
    elif stream:
        # single-K-step product (scores Q K^T): bound by writing Y; bytes = Y
        # plus both packed operands read once
        dom = "gemm"
        gemm_ms = kt["gemm"][0]
        algo_bytes = 2 * runner.batch * (runner.n * runner.m + (runner.n + runner.m) * k)
        achieved = algo_bytes / (gemm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "gemm_stream", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes": algo_bytes,
                "kernel_ms": gemm_ms}
    else:
        dom = "gemm"
        gemm_ms = kt["gemm"][0] * max(1.0, kt["gemm"][1])  # every GEMM launch of the step (Up/Gate and Down)
        achieved = runner.flops(rho) / (gemm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "gemm_" + runner.plan(rho)["gemm"], "achieved": achieved,
                "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                "algorithmic_flops": runner.flops(rho), "kernel_ms": gemm_ms}
    roof["traffic"] = load_traffic(dom, args.workload)
    roof["per_kernel_ms"] = {kk: v[0] for kk, v in kt.items() if v[1]}
    if roof["bound"] == "mfma" and not args.no_mfma_ceiling:
        cal = rmm.calibrate_mfma()
        ceiling = sorted(cal["tflops"])[len(cal["tflops"]) // 2]
        roof["measured_peak"] = ceiling
        roof["frac_of_measured_peak"] = roof["achieved"] / ceiling
        roof["measured_peak_shader_mhz"] = sorted(cal["shader_mhz"])[len(cal["shader_mhz"]) // 2]
        roof["measured_peak_how"] = ("median of %d back-to-back launches of the matrix-core probe "
                                     "(rmm_calibrate_mfma: %d workgroups x 4 waves, eight independent "
                                     "v_mfma_f32_32x32x16_bf16 chains, no memory traffic); shader clock read "
                                     "in the probe's waves from the cycle counter against the 100 MHz counter"
                                     % (len(cal["tflops"]), cal["workgroups"]))
        log(f"matrix-core ceiling measured: {ceiling:.0f} TFLOP/s; GEMM at {roof['frac_of_measured_peak']:.3f} of it")

    cpu = None
    if rank == 0 and not args.no_cpu_baseline and is_attn:
        cpu = cpu_baseline_attn(runner, rho)
        log(f"cpu oracle: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")
    elif rank == 0 and not args.no_cpu_baseline and is_wqgemm:
        key = (rho, False)
        runner.call(0, rho)
        torch.cuda.synchronize()
        cpu = cpu_baseline_wqgemm(runner, rho, (runner.idx[key].cpu().numpy(), runner.Y[0].float().cpu().numpy()))
        log(f"cpu oracle: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads; parity {cpu['parity']}")
    elif rank == 0 and not args.no_cpu_baseline and is_wq:
        cpu = cpu_baseline_wq(runner, rho)
        log(f"cpu oracle: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")
    elif rank == 0 and not args.no_cpu_baseline and not is_mlp:  # the fp64 block needs every row of h: no bounded sample
        # the GPU's own result on input copy 0, for the parity check against the oracle's
        key = (rho, False)
        runner.call(0, rho)
        torch.cuda.synchronize()
        g_idx = runner.idx[key].view(runner.batch, -1)[0].cpu().numpy()
        g_Y = (runner.Y[0][0] if runner.batched else runner.Y[0]).float().cpu().numpy()
        cpu = cpu_baseline(runner, rho, gpu=(g_idx, g_Y))
        log(f"cpu oracle: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads; parity {cpu['parity']}")

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "median_ms_per_step": med,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {wl['label']}, rho={rho} (k={k})",
                   "n": runner.n, "d": runner.d, "m": runner.m, "batch": runner.batch, "rho": rho, "k": k,
                   "input_copies_rotated": runner.copies, "hip_graph": graph},
        "roofline": roof,
        "clocks": clocks.summary(),
        "inputs_sha256": getattr(runner, "sha256", None),
        "parity": cpu.pop("parity", None) if cpu else None,
        "cpu_baseline": cpu,
        "sweep": sweep,
    }
    if rank == 0:
        print(json.dumps(line), flush=True)
        if args.jsonl:
            now = time.strftime("%Y-%m-%dT%H:%M:%S%z")
            with open(args.jsonl, "a") as f:
                for ent in sweep:
                    if not ent.get("reused"):
                        f.write(json.dumps({"kind": "sweep", **common, **ent, "time": now}) + "\n")
                f.write(json.dumps({"kind": "headline", **common, "rho": rho, "k": k, "full_path": False,
                                    "ms": ms, "median_ms": med, "tflops": value, "roofline": roof,
                                    "clocks": line["clocks"], "parity": line["parity"], "cpu_baseline": cpu,
                                    "time": now}) + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())

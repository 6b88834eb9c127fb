"""Host-side checks of the compiled gfx950 kernels (no GPU is used).

1. No kernel uses flat (generic-address) loads or stores: a pointer that may
   point to either LDS or global memory compiles to flat accesses, which wait
   on both counters and serialise a gather (this once cost the A pack a fifth
   of its time).
2. Ordering arguments the LDS-DMA product kernels rely on.

gemm_bdma_kernel waits for its own LDS-DMA loads of the next K step with
``s_waitcnt vmcnt(28)``: vector-memory loads retire in issue order, so the
wait covers those loads only if at least 28 loads are issued after the last
of them and before the wait.  The kernel fences its sub-steps with scheduling
barriers so that this holds by construction; this test compiles the kernel
to gfx950 assembly and checks it in every loop that contains the wait.

gemm_tdma_kernel and gemm_tdma8_kernel keep two LDS stages per operand:
each wave waits for all of its own LDS-DMA loads (vmcnt(0)) right before
the workgroup barrier, and refills a stage only after that barrier, since
only then has every wave read its last operands from it.  The test checks
that in the compiled loop every barrier directly follows such a wait and
that all LDS-DMA loads of a step (16 per wave with four waves and bf16
weights, 12 with 8-bit weights, 8 with eight waves) come after a barrier
and before the next wait.  No GPU is used.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "input_adaptive_reduced_amd", "csrc")


def loop_sequences(asm: str, kernel: str):
    lines = asm.split("\n")
    start = next(i for i, l in enumerate(lines) if re.match(r"^_Z\S*" + kernel + r"\S*:", l))
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    body = lines[start:end]
    for h, l in enumerate(body):
        if "Loop Header" not in l:
            continue
        stop = next((i for i in range(h + 1, len(body))
                     if body[i].startswith(".LBB") and "in Loop" not in body[i]), len(body))
        seq = []
        for x in body[h:stop]:
            x = x.strip()
            if x.startswith(("buffer_load", "global_load")):
                seq.append("D" if " lds" in x else "A")
            elif x.startswith("s_waitcnt") and "vmcnt(28)" in x:
                seq.append("W")
        if "W" in seq:
            yield seq


def min_younger(seq):
    """Fewest loads issued after the previous step's last DMA load and before
    each wait, around the loop (the sequence repeats)."""
    s2 = seq * 2
    waits = [i for i, c in enumerate(s2) if c == "W"]
    worst = None
    for a, b in zip(waits, waits[1:]):
        dma = [i for i in range(a) if s2[i] == "D"]
        if not dma:
            continue
        n = sum(1 for i in range(dma[-1] + 1, b) if s2[i] in "AD")
        worst = n if worst is None else min(worst, n)
    return worst


def test_min_younger_counts_loads_after_the_previous_steps_dma():
    # each wait needs the DMA loads issued before the previous wait: after
    # the last of them come 3 A loads, 2 DMA loads and 3 A loads
    assert min_younger(list("DDAAAWDDAAAW")) == 8
    # DMA right before each wait: only the next step's two DMA loads follow
    assert min_younger(list("DDWDDW")) == 2


def compile_to_asm(src, out):
    cmd = ["hipcc", "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return out.read_text()


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    return compile_to_asm("gemm.hip", tmp_path_factory.mktemp("asm") / "gemm.s")


@pytest.mark.parametrize("src", ["norm_select.hip", "gemv.hip", "rmm_api.hip"])
def test_no_flat_memory_access(src, tmp_path):
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    asm = compile_to_asm(src, tmp_path / "k.s")
    assert not re.search(r"\bflat_(load|store|atomic)", asm)


def test_no_flat_memory_access_in_gemm(gemm_asm):
    assert not re.search(r"\bflat_(load|store|atomic)", gemm_asm)


def test_bdma_wait_covers_its_dma(gemm_asm):
    asm = gemm_asm
    for split in ("0", "1"):
        seqs = list(loop_sequences(asm, "gemm_bdma_kernelILb" + split))
        assert seqs, "no loop with the DMA wait found"
        for seq in seqs:
            assert seq.count("W") % 3 == 0
            assert min_younger(seq) >= 28, "".join(seq)


def loop_tokens(asm: str, kernel: str):
    """Per loop of `kernel` that contains a barrier: D = LDS-DMA load,
    W = wait for every vector-memory load, B = barrier."""
    lines = asm.split("\n")
    start = next(i for i, l in enumerate(lines) if re.match(r"^_Z\S*" + kernel + r"\S*:", l))
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    body = lines[start:end]
    for h, l in enumerate(body):
        if "Loop Header" not in l:
            continue
        stop = next((i for i in range(h + 1, len(body))
                     if body[i].startswith(".LBB") and "in Loop" not in body[i]), len(body))
        seq = []
        for x in body[h:stop]:
            x = x.strip()
            if x.startswith("buffer_load") and " lds" in x:
                seq.append("D")
            elif x.startswith("s_waitcnt") and "vmcnt(0)" in x:
                seq.append("W")
            elif x.startswith("s_barrier"):
                seq.append("B")
        if "B" in seq:
            yield "".join(seq)


TDMA = [
    # kernel and (split K, epilogue, B format) instantiation, LDS-DMA loads per
    # K step per wave: four waves, SwiGLU epilogue B 8 + A 8, 8-bit B (FP8,
    # int8) 4 + A 8; eight waves (bf16 B, plain or split) B 4 + A 4
    ("gemm_tdma_kernelILb0ELi1ELi0E", 16),
    ("gemm_tdma_kernelILb0ELi0ELi1E", 12), ("gemm_tdma_kernelILb1ELi0ELi1E", 12),
    ("gemm_tdma_kernelILb0ELi0ELi2E", 12), ("gemm_tdma_kernelILb1ELi0ELi2E", 12),
    ("gemm_tdma8_kernelILb0E", 8), ("gemm_tdma8_kernelILb1E", 8),
]


@pytest.mark.parametrize("inst,loads", TDMA, ids=[t[0] for t in TDMA])
def test_tdma_refills_a_stage_only_after_the_barrier(gemm_asm, inst, loads):
    loops = list(loop_tokens(gemm_asm, inst))
    assert loops, "no K loop with a barrier found"
    for seq in loops:
        assert seq.count("B") == 2, seq  # two K steps per iteration, one barrier each
        # rotate to start at a barrier: then B D^loads W B D^loads W
        r = seq[seq.index("B"):] + seq[:seq.index("B")]
        assert re.fullmatch(r"(BD{%d}W){2}" % loads, r), seq

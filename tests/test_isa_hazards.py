"""The prefill GEMM's inline-assembly MFMAs: compile the kernel for gfx950 and
check, on the assembly, that every MFMA keeps its accumulator in place and
that the hazard spacing around it holds on every control-flow path."""
import os
import shutil
import subprocess

import pytest

import isa_hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "w4a8_quantized_linear_amd", "csrc", "gemm_prefill.hip")
KERNELS = ["_ZN4w4a812_GLOBAL__N_119gemm_prefill_kernelILi%dEEEvNS0_11PrefillArgsE" % tm
           for tm in (4, 8, 16)]


@pytest.fixture(scope="module")
def listing(tmp_path_factory):
    from w4a8_quantized_linear_amd import build
    hipcc = build.HIPCC
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("isa") / "gemm_prefill.s")
    flags = [f for f in build.CFLAGS if f != "-fPIC"]
    cmd = [hipcc] + flags + ["-S", "--cuda-device-only", SRC, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return open(out).read()


@pytest.mark.parametrize("kernel", KERNELS)
def test_mfma_accumulators_in_place(listing, kernel):
    insts, _ = isa_hazards.parse_kernel(listing, kernel)
    mfma = [ops for op, ops in insts if op.startswith("v_mfma")]
    assert len(mfma) >= 256
    for ops in mfma:
        assert ops[0].startswith("a[") and ops[0] == ops[3], ops


@pytest.mark.parametrize("kernel", KERNELS)
def test_no_spills_or_accumulator_moves_beside_mfmas(listing, kernel):
    # basic blocks that issue MFMAs hold no scratch traffic and no moves of
    # the accumulation registers the MFMAs use (the accumulators stay put;
    # other values parked in spare AGPRs are allowed)
    insts, labels = isa_hazards.parse_kernel(listing, kernel)
    acc_regs = set()
    for op, ops in insts:
        if op.startswith("v_mfma"):
            acc_regs |= isa_hazards._regs(ops[0])
    starts = sorted(set(labels.values()) | {k + 1 for k, (op, _) in enumerate(insts)
                                             if op.startswith("s_cbranch") or op == "s_branch"})
    bounds = [0] + [s for s in starts if 0 < s < len(insts)] + [len(insts)]
    n_blocks = 0
    for a, b in zip(bounds, bounds[1:]):
        block = insts[a:b]
        if not any(op.startswith("v_mfma") for op, _ in block):
            continue
        n_blocks += 1
        for op, ops in block:
            assert not op.startswith("scratch_"), (a, op, ops)
            if op.startswith("v_accvgpr_"):
                touched = set().union(*(isa_hazards._regs(o) for o in ops))
                assert not (touched & acc_regs), (a, op, ops)
    assert n_blocks > 0


@pytest.mark.parametrize("kernel", KERNELS)
def test_mfma_hazard_spacing(listing, kernel):
    n, found = isa_hazards.check(listing, kernel, valu_mfma=4, mfma_other=19)
    assert n > 0
    assert not found, found[:5]


def test_checker_flags_planted_hazards():
    bad = ("k:\n\tv_xor_b32_e32 v57, 0x80808080, v57\n"
           "\tv_mfma_i32_16x16x64_i8 a[0:3], v[80:83], v[56:59], a[0:3]\n"
           "\ts_nop 1\n\tv_accvgpr_read_b32 v1, a2\n\ts_endpgm\n")
    n, found = isa_hazards.check(bad, "k")
    assert n == 1 and sorted(f[0] for f in found) == ["R1", "R2"]
    # a loop back-edge carries the VALU write into the next iteration's MFMA
    loop = ("k:\n.L1:\n\tv_mfma_i32_16x16x64_i8 a[0:3], v[80:83], v[56:59], a[0:3]\n"
            "\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\tv_xor_b32_e32 v56, 1, v56\n"
            "\ts_cbranch_scc1 .L1\n\ts_endpgm\n")
    n, found = isa_hazards.check(loop, "k")
    assert [f[0] for f in found] == ["R1"]

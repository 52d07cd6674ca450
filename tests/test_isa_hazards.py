"""CPU: the direct-to-LDS loads of the built forward have the wait states the
ISA requires on every path (tests/isa_hazards.py), and the checker finds the
violations it is meant to find on hand-written instruction streams."""

import os
import shutil

import pytest

from tests import isa_hazards as hz

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "temporal_block_sparse_amd",
                   "liblite_attn.so")


def _prog(src):
    """Instruction tuples from lines 'mnemonic operands' with optional 'L<n>:' labels
    and branch targets written as '@L<n>'."""
    insts, labels, pending = [], {}, []
    addr = 0
    for line in src.strip().split("\n"):
        line = line.strip()
        if line.endswith(":"):
            labels[line[:-1]] = addr
            continue
        mn, _, ops = line.partition(" ")
        tgt = None
        if "@" in ops:
            ops, _, lab = ops.partition("@")
            pending.append((len(insts), lab.strip()))
            tgt = 0
        insts.append([addr, mn, ops.strip(), tgt])
        addr += 4
    for i, lab in pending:
        insts[i][3] = labels[lab]
    return [tuple(x) for x in insts]


DMA = "buffer_load_dwordx4 v10, s[8:11], 0 offen lds"


def test_scalar_writes_then_one_wait_state_pass():
    ok = _prog("""
        s_mov_b32 s8, s20
        s_and_b32 s9, s21, 0xffff
        s_add_i32 m0, s22, 0x8000
        s_nop 0
        %s
        s_endpgm""" % DMA)
    assert hz.check_function(ok) == []


def test_m0_without_a_wait_state_fails():
    bad = _prog("""
        s_add_i32 m0, s22, 0x8000
        %s
        s_endpgm""" % DMA)
    v = hz.check_function(bad)
    assert len(v) == 1 and "m0 written 0" in v[0][1]


@pytest.mark.parametrize("writer", ["v_readfirstlane_b32 s9, v3", "v_readlane_b32 s11, v3, 5",
                                    "v_cmp_gt_u32_e64 s[10:11], v1, v2", "v_add_co_u32_e64 v4, s[8:9], v1, v2",
                                    "v_readfirstlane_b32 m0, v3"])
def test_vector_written_sgpr_needs_five(writer):
    for gap in range(0, 7):
        src = "%s\n%s\ns_mov_b32 s30, 0\n%s\ns_endpgm" % (
            writer, "\n".join(["s_nop 0"] * gap), DMA)
        v = hz.check_function(_prog(src))
        # the s_mov adds one wait state: gap + 1 in all
        assert (len(v) > 0) == (gap + 1 < 5), (writer, gap, v)


def test_s_nop_counts_its_argument_plus_one():
    src = "v_readfirstlane_b32 s9, v3\ns_nop 4\n%s\ns_endpgm" % DMA
    assert hz.check_function(_prog(src)) == []            # 5 wait states
    src = "v_readfirstlane_b32 s9, v3\ns_nop 3\n%s\ns_endpgm" % DMA
    assert len(hz.check_function(_prog(src))) == 1        # 4
    src = "v_readfirstlane_b32 s9, v3\ns_nop 2\ns_nop 0\n%s\ns_endpgm" % DMA
    assert len(hz.check_function(_prog(src))) == 1        # 3 + 1


def test_scalar_rewrite_clears_a_vector_write():
    src = "v_readfirstlane_b32 s9, v3\ns_and_b32 s9, s9, 0xffff\n%s\ns_endpgm" % DMA
    assert hz.check_function(_prog(src)) == []


def test_compare_does_not_count_as_a_scalar_write():
    src = "v_readfirstlane_b32 s9, v3\ns_cmp_lt_i32 s9, 0\n%s\ns_endpgm" % DMA
    assert len(hz.check_function(_prog(src))) == 1


def test_violation_through_a_branch_only():
    src = """
        s_cbranch_scc0 @L1
        v_readfirstlane_b32 s10, v3
        s_branch @L2
        L1:
        s_mov_b32 s10, 0
        s_nop 7
        L2:
        %s
        s_endpgm""" % DMA
    v = hz.check_function(_prog(src))
    assert len(v) == 1 and "s10" in v[0][1]


def test_violation_around_a_loop_back_edge():
    src = """
        s_mov_b32 s8, 0
        s_nop 7
        L1:
        %s
        v_readlane_b32 s8, v2, 0
        s_cbranch_scc1 @L1
        s_endpgm""" % DMA
    v = hz.check_function(_prog(src))
    assert len(v) == 1 and "s8" in v[0][1]


def test_address_register_written_by_a_matrix_instruction():
    src = "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0\ns_nop 7\n%s\ns_endpgm" % DMA.replace(
        "v10", "v12")
    v = hz.check_function(_prog(src))
    assert len(v) == 1 and "address v12" in v[0][1]


def test_built_library(tmp_path):
    """Every direct-to-LDS load in the built library passes, and the forward's
    kernels hold such loads (40 at d = 64, 80 at d = 128)."""
    if not os.path.exists(LIB):
        pytest.skip("library not built")
    if not shutil.which(hz.LLVM + "/llvm-objdump"):
        pytest.skip("no llvm-objdump")
    res = hz.check_library(LIB, str(tmp_path))
    fwd = {k: v for k, v in res.items() if "fwd_bf16_kernel" in k}
    assert len(fwd) == 8, sorted(res)
    for name, (n, viol) in res.items():
        assert n > 0
        assert viol == [], (name, viol[:5])

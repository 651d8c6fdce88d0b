"""Two hazards of the built kernels, checked on their gfx950 assembly.

Kernels that issue LDS reads as inline assembly and wait for them by count
are correct only if the compiler never touches a destination register of
such a read before the wait that covers it (a register copy placed there
reads stale data, and the result changes from run to run). And a matrix
instruction's result may only be read by other instructions some slots
after it issues; the hardware does not hold the reader back. The checker
walks every path of each kernel; these tests first show it on small
hand-written listings, then run it on every source with such code.
"""
import concurrent.futures as cf
import os
import shutil

import pytest

from sparse_attention_kv_append_amd import build as sab
from sparse_attention_kv_append_amd import isa_check as ic


def wrap(body):
    """A kernel listing; every LDS read in it is marked as inline assembly
    (the only reads the checker tracks: the compiler waits for its own)."""
    out = []
    for ln in body:
        if ln.startswith("."):
            out.append(ln)
        elif ln.startswith("ds_read"):
            out += ["\t;;#ASMSTART", "\t" + ln, "\t;;#ASMEND"]
        else:
            out.append("\t" + ln)
    return "_Z4testv:\n" + "\n".join(out) + "\n.Lfunc_end0:\n"


def test_copy_before_the_wait_is_flagged():
    asm = wrap(["ds_read_b128 v[4:7], v1",
                "ds_read_b128 v[8:11], v1 offset:1024",
                "v_mov_b64_e32 v[20:21], v[4:5]",
                "s_waitcnt lgkmcnt(0)",
                "s_endpgm"])
    hz = ic.check_asm(asm)
    assert len(hz) == 1 and "v4" in hz[0]


def test_counted_wait_covers_older_reads_only():
    ok = wrap(["ds_read_b128 v[4:7], v1",
               "ds_read_b128 v[8:11], v1 offset:1024",
               "s_waitcnt lgkmcnt(1)",
               "v_mov_b64_e32 v[20:21], v[4:5]",
               "s_waitcnt lgkmcnt(0)",
               "v_mov_b64_e32 v[22:23], v[8:9]",
               "s_endpgm"])
    assert ic.check_asm(ok) == []
    bad = wrap(["ds_read_b128 v[4:7], v1",
                "ds_read_b128 v[8:11], v1 offset:1024",
                "s_waitcnt lgkmcnt(1)",
                "v_mov_b64_e32 v[22:23], v[8:9]",
                "s_endpgm"])
    assert len(ic.check_asm(bad)) == 1


def test_scalar_loads_do_not_retire_lds_reads():
    # an s_load between the read and the wait adds to the count; the LDS read
    # is only known complete once enough later LDS operations are counted
    asm = wrap(["ds_read_b32 v4, v1",
                "s_load_dword s8, s[0:1], 0x0",
                "s_waitcnt lgkmcnt(1)",
                "v_add_u32_e32 v5, v4, v4",
                "s_endpgm"])
    assert len(ic.check_asm(asm)) == 1


def test_pending_read_along_one_branch_is_flagged_at_the_join():
    asm = wrap(["s_cbranch_scc0 .LBB0_2",
                "ds_read_b32 v4, v1",
                ".LBB0_2:",
                "v_add_u32_e32 v5, v4, v4",
                "s_waitcnt lgkmcnt(0)",
                "s_endpgm"])
    assert len(ic.check_asm(asm)) == 1


def test_loop_carried_pending_read_is_flagged():
    asm = wrap([".LBB0_1:",
                "v_add_u32_e32 v5, v4, v4",
                "ds_read_b32 v4, v1",
                "s_cbranch_scc1 .LBB0_1",
                "s_waitcnt lgkmcnt(0)",
                "s_endpgm"])
    assert len(ic.check_asm(asm)) == 1


def test_flag_guarded_paths_that_cannot_both_run_are_kept_apart():
    # the structurizer's pattern: a flag pair set to all-ones on one path and
    # zero on the other selects the successor; the read pending on the first
    # path never reaches the block only the second path enters
    asm = wrap(["ds_read_b32 v4, v1",
                "s_mov_b64 s[8:9], -1",
                "s_cbranch_scc0 .LBB0_3",
                "s_waitcnt lgkmcnt(0)",
                "v_add_u32_e32 v6, v4, v4",
                "s_mov_b64 s[8:9], 0",
                ".LBB0_3:",
                "s_andn2_b64 vcc, exec, s[8:9]",
                "s_cbranch_vccnz .LBB0_5",
                "s_waitcnt lgkmcnt(0)",
                "s_endpgm",
                ".LBB0_5:",
                "v_add_u32_e32 v5, v4, v4",
                "s_endpgm"])
    assert ic.check_asm(asm) == []
    # without the flag the same join is a hazard
    asm2 = asm.replace("s_mov_b64 s[8:9], -1", "s_mov_b64 s[8:9], s[2:3]")
    assert len(ic.check_asm(asm2)) == 1


def test_compiler_reads_and_calls_are_left_to_the_compiler():
    # a read the compiler issued itself (no inline-assembly markers) is its
    # business; a call waits for everything at the callee's entry
    asm = ("_Z4testv:\n\tds_read_b128 v[4:7], v1\n\tv_mov_b32_e32 v20, v4\n"
           "\t;;#ASMSTART\n\tds_read_b128 v[8:11], v1\n\t;;#ASMEND\n"
           "\ts_swappc_b64 s[30:31], s[0:1]\n\tv_mov_b32_e32 v8, v0\n\ts_endpgm\n.Lfunc_end0:\n")
    assert ic.check_asm(asm) == []


def test_matrix_result_read_too_soon_is_flagged_across_a_branch():
    # the consumer sits behind a branch: on the taken path only two slots
    # separate it from the matrix write, which needs eight
    asm = wrap(["v_mfma_f32_16x16x32_bf16 v[8:11], v[0:3], v[4:7], v[8:11]",
                "s_cmp_le_i32 s4, s5",
                "s_cbranch_scc1 .LBB0_2",
                "s_nop 7",
                "s_nop 7",
                ".LBB0_2:",
                "v_mul_f32_e32 v12, v13, v8",
                "s_endpgm"])
    hz = ic.check_asm(asm)
    assert len(hz) == 1 and "v8" in hz[0]


def test_matrix_padding_and_accumulation_chains_pass():
    asm = wrap(["v_mfma_f32_16x16x32_bf16 v[8:11], v[0:3], v[4:7], v[8:11]",
                # the accumulator chain reads the result as C: no padding needed
                "v_mfma_f32_16x16x32_bf16 v[8:11], v[0:3], v[4:7], v[8:11]",
                "s_nop 7",
                "v_mul_f32_e32 v12, v13, v8",
                "v_mfma_f32_32x32x16_bf16 v[16:31], v[0:3], v[4:7], v[16:31]",
                "s_nop 7",
                "v_add_f32_e32 v12, v13, v16",
                "s_endpgm"])
    hz = ic.check_asm(asm)
    # the 32x32 result needs twelve slots; eight plus the nop's own do not cover it
    assert len(hz) == 1 and "v16" in hz[0]
    ok = asm.replace("s_nop 7\n\tv_add_f32", "s_nop 7\n\ts_nop 3\n\tv_add_f32")
    assert ic.check_asm(ok) == []
    # a matrix A/B operand is a reader like any other
    ab = wrap(["v_mfma_f32_16x16x32_bf16 v[8:11], v[0:3], v[4:7], v[8:11]",
               "v_mfma_f32_16x16x32_bf16 v[20:23], v[8:11], v[4:7], v[20:23]",
               "s_endpgm"])
    assert len(ic.check_asm(ab)) == 1


@pytest.mark.skipif(not (os.path.exists(sab.HIPCC) or shutil.which("hipcc")), reason="hipcc not installed")
def test_built_kernels_have_neither_hazard():
    srcs = ic.checked_sources()
    assert {s.name for s in srcs} >= {"k_forward_latent_decode.hip", "k_forward_latent.hip",
                                      "k_csa_attention.hip"}
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        asms = list(ex.map(ic.device_asm, srcs))
    hazards = []
    for s, a in zip(srcs, asms):
        kernels = [n for n, _ in ic._functions(a)]
        assert kernels, f"no kernel found in the assembly of {s.name}"
        hazards += [f"{s.name}: {h}" for h in ic.check_asm(a)]
    assert hazards == [], "\n".join(hazards[:20])

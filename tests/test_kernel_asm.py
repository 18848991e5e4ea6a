"""Static checks of the compiled gfx950 kernels (CPU only: hipcc cross-compiles).

The GEMM kernels issue MFMAs as inline asm, whose operands the compiler's
hazard recognizer does not track, so spills and missing wait states around
them would give wrong results without any error.  These tests compile every
kernel source to assembly and check it with tests/asm_hazards.py; the
synthetic cases first show that each rule of the checker fires.
"""
import glob
import os
import shutil
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import asm_hazards as H  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _wrap(body: str) -> str:
    # every synthetic instruction counts as inline asm, as the kernels' MFMAs are
    out = []
    for ln in body.strip().splitlines():
        ln = ln.strip()
        out.append(ln if ln.startswith(".LBB") else "\t;;#ASMSTART\n\t" + ln + "\n\t;;#ASMEND")
    return "_Zkernel:\n" + "\n".join(out) + "\n.Lfunc_end0:\n"


def _problems(body: str):
    fs = H.parse_functions(_wrap(body))
    assert len(fs) == 1
    return H.check_function(fs[0])


MFMA = "v_mfma_scale_f32_16x16x128_f8f6f4 a[0:3], v[0:7], v[8:15], a[0:3], v16, v17 op_sel_hi:[0,0,0]"


def test_valu_write_then_mfma_read_is_flagged():
    assert _problems("v_lshrrev_b32_e32 v16, 8, v16\n" + MFMA + "\ns_endpgm")
    assert not _problems("v_lshrrev_b32_e32 v16, 8, v16\ns_nop 1\n" + MFMA + "\ns_endpgm")


def test_lds_load_into_mfma_operand_is_not_valu():
    assert not _problems("ds_read_u8 v16, v20\ns_waitcnt lgkmcnt(0)\n" + MFMA + "\ns_endpgm")


def test_accumulator_read_too_early_is_flagged():
    assert _problems(MFMA + "\ns_nop 7\nv_accvgpr_read_b32 v30, a2\ns_endpgm")
    assert not _problems(MFMA + "\ns_nop 15\ns_nop 15\nv_accvgpr_read_b32 v30, a2\ns_endpgm")


def test_accumulator_overwrite_and_store_too_early_are_flagged():
    assert _problems(MFMA + "\nv_accvgpr_write_b32 a1, 0\ns_endpgm")
    assert _problems(MFMA + "\nglobal_store_dwordx4 v[40:41], a[0:3], off\ns_endpgm")


def test_hazard_reached_through_a_branch_is_flagged():
    body = MFMA + "\ns_cbranch_scc1 .LBB0_2\ns_nop 15\ns_nop 15\n.LBB0_2:\nv_accvgpr_read_b32 v30, a0\ns_endpgm"
    assert _problems(body)


def test_accumulation_chain_rules():
    same = MFMA + "\n" + MFMA + "\ns_endpgm"
    assert not _problems(same)
    partial = MFMA + "\nv_mfma_scale_f32_16x16x128_f8f6f4 a[2:5], v[0:7], v[8:15], a[2:5], v16, v17\ns_endpgm"
    assert _problems(partial)
    as_source = MFMA.replace("a[0:3], v[0:7]", "a[0:3], v[20:27]") + \
        "\nv_mfma_f32_16x16x32_f16 a[8:11], a[0:3], v[4:7], a[8:11]\ns_endpgm"
    assert _problems(as_source)


def test_spill_in_mfma_kernel_is_flagged():
    assert _problems(MFMA + "\ns_nop 15\ns_nop 15\nscratch_store_dwordx4 off, a[0:3], off\ns_endpgm")


def test_compiler_generated_pairs_are_left_to_the_compiler():
    asm = "_Zkernel:\n\t" + MFMA + "\n\tv_accvgpr_read_b32 v30, a2\n\ts_endpgm\n.Lfunc_end0:\n"
    assert not H.check_function(H.parse_functions(asm)[0])


def test_checker_sees_the_right_operands():
    ins = H._parse_instr("v_mfma_scale_f32_16x16x128_f8f6f4 a[112:115], v[88:95], v[8:15], a[112:115], v109, "
                         "v107 op_sel:[0,1,0] op_sel_hi:[0,0,0]")
    assert ins.writes == {("a", r) for r in range(112, 116)}
    assert ins.srcc == ins.writes
    assert ("v", 109) in ins.srcab and ("v", 107) in ins.srcab and ("v", 95) in ins.srcab
    ld = H._parse_instr("buffer_load_dwordx4 v98, s[16:19], s6 offen lds")
    assert not ld.writes and ("v", 98) in ld.reads


@pytest.mark.skipif(shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")) is None, reason="hipcc not found")
@pytest.mark.parametrize("src", sorted(glob.glob(os.path.join(ROOT, "block_scaled_precision_mxgemm_amd", "csrc",
                                                              "*.hip"))), ids=os.path.basename)
def test_kernel_source_is_hazard_free(src):
    from block_scaled_precision_mxgemm_amd import build as B
    asm = H.compile_to_asm(src, B.FLAGS, B.HIPCC)
    funcs = H.parse_functions(asm)
    assert funcs, "no functions parsed from " + src
    problems = []
    for f in funcs:
        problems += H.check_function(f)
    assert not problems, "\n".join(problems[:20])


@pytest.mark.skipif(shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")) is None, reason="hipcc not found")
def test_decode_kernel_first_wait_counts_the_issued_loads():
    """The decode kernel's stage waits count the vector-memory instructions
    issued after a stage's copies; in the first fragment these include the
    A operand loads (2 per row block and MFMA: the lo and hi halves of the
    operand), each stage's issued right after that stage's copies, so the
    prologue issues those of the stages it copies: the MFMAs whose operands
    complete in the first AHEAD stages, AHEAD = D - 2 for operands of 64
    bytes or less in a 4-stage ring and for FP6 line stages (K / 1024 a
    multiple of 4: 4 operands of 96 bytes per 3 stages of 128), else D - 1.
    The A scales are loaded before the first copy, so that however the
    compiler merges those loads they are never among the counted ones.
    Between the first copy and the first wait the compiler must issue
    exactly the counted global loads, or the wait lets a stage's copies
    still be in flight.  With two weight operands per stage (E2M1, INT4)
    and K / 1024 odd the kernel has two wave kinds (WK = KW + 1 for waves
    0-3, KW - 1 for waves 4-7) behind one branch on the wave index; the
    prologue of each kind starts at an assembly comment that names WK, MB
    and the count it issues, which must also be the count the rule above
    gives.  Every weight format (E4M3, E2M1, INT4, INT2, E2M3, E3M2) is
    checked."""
    import re
    from block_scaled_precision_mxgemm_amd import build as B
    asm = H.compile_to_asm(os.path.join(ROOT, "block_scaled_precision_mxgemm_amd", "csrc", "gemm_decode.hip"),
                           B.FLAGS, B.HIPCC)

    seen = split = 0
    formats = set()
    op_bytes = {0: 128, 4: 64, 8: 64, 9: 32, 2: 96, 3: 96}   # E4M3, E2M1, INT4, INT2, E2M3, E3M2

    def prologue_a_loads(w, wk, mb, d):
        fp6_line = w in (2, 3) and wk % 4 == 0
        ahead = d - 2 if (fp6_line or (op_bytes[w] <= 64 and d == 4)) else d - 1
        if fp6_line:   # operand u completes in stage (96 u + 95) // 128
            ops = sum(1 for u in range(wk) if (96 * u + 95) // 128 < ahead)
        else:          # 128-byte stages of whole operands (96-byte stages for other FP6)
            per_stage = max(1, 128 // op_bytes[w]) if w not in (2, 3) else 1
            ops = min(wk, ahead * per_stage)
        return 2 * mb * ops

    for m in re.finditer(r"^(_ZN3mxg12_GLOBAL__N_113decode_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)EEEv\S*):", asm,
                         re.M):
        name, w, kw, mb, d = m.group(1), int(m.group(2)), int(m.group(3)), int(m.group(4)), int(m.group(5))
        formats.add(w)
        two_per_stage = w in (4, 8)   # E2M1, INT4: 64-byte operands
        body = asm[m.end():asm.index(".Lfunc_end", m.end())]
        # the prologue of each wave kind starts at its marker comment
        wks = []
        for p in re.finditer(r"; decode prologue wk=(\d+) mb=(\d+) la=(\d+)", body):
            wk, la = int(p.group(1)), int(p.group(3))
            assert int(p.group(2)) == mb, name
            assert la == prologue_a_loads(w, wk, mb, d), (name, wk, la, prologue_a_loads(w, wk, mb, d))
            part = body[p.end():]
            first_wait = re.search(r"s_waitcnt vmcnt\(", part)
            first_copy = re.search(r"^\s*buffer_load_dwordx[34] .* lds", part, re.M)
            assert first_wait and first_copy and first_copy.start() < first_wait.start(), name
            assert re.search(r"^\s*global_load_\w+", part[:first_copy.start()], re.M), name   # the A scales
            loads = re.findall(r"^\s*global_load_\w+", part[first_copy.start():first_wait.start()], re.M)
            assert len(loads) == la, (name, wk, len(loads), la)
            wks.append(wk)
        if two_per_stage and kw % 2 == 1:
            assert sorted(set(wks)) == [kw - 1, kw + 1], (name, wks)
            split += 1
        else:
            assert set(wks) == {kw}, (name, wks)
        seen += 1
    assert seen >= 80 and split >= 12 and formats == {0, 2, 3, 4, 8, 9}

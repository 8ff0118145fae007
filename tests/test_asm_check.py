"""The build-time check of the asynchronous transposing LDS reads
(causal_attention_flash_amd/asm_check.py): planted violations in small assembly
snippets are found, clean code passes, and the shipped sources pass (compiled
to gfx950 device assembly here, no GPU needed)."""
import pytest

from causal_attention_flash_amd import asm_check, build

HEAD = "k:                                      ; @k\n"
TAIL = ".Lfunc_end0:\n"


def asm(*body):
    return HEAD + "\n".join("\t" + b if not b.endswith(":") else b for b in body) + "\n" + TAIL


def tr(dst, addr):
    return [";;#ASMSTART", f"ds_read_b64_tr_b16 {dst}, {addr}", ";;#ASMEND"]


WAIT = [";;#ASMSTART", "s_waitcnt lgkmcnt(0)", ";;#ASMEND"]


def test_clean_read_wait_use():
    a = asm(*tr("v[10:11]", "v4"), *tr("v[12:13]", "v5"), "v_mul_f32_e32 v20, v21, v22", *WAIT,
            "v_mfma_f32_32x32x16_bf16 v[30:45], v[10:13], v[50:53], v[30:45]")
    assert asm_check.check_text(a) == []
    assert asm_check.count_reads(a) == 2


def test_copy_before_wait_found():
    # the failure seen with a register-starved variant: a copy to an AGPR
    a = asm(*tr("v[10:11]", "v4"), "v_accvgpr_write_b32 a5, v11", *WAIT)
    bad = asm_check.check_text(a)
    assert len(bad) == 1 and "v11" in bad[0]


def test_overwrite_before_wait_found():
    a = asm(*tr("v[10:11]", "v4"), "v_mov_b32_e32 v10, 0", *WAIT)
    assert len(asm_check.check_text(a)) == 1


def test_address_from_pending_found():
    a = asm(*tr("v[10:11]", "v4"), *tr("v[12:13]", "v10"), *WAIT)
    assert len(asm_check.check_text(a)) == 1


def test_wait_not_covering_found():
    # a wait that leaves reads outstanding does not count: only lgkmcnt(0) does
    a = asm(*tr("v[10:11]", "v4"), ";;#ASMSTART", "s_waitcnt lgkmcnt(1)", ";;#ASMEND", "v_mov_b32_e32 v1, v10",
            *WAIT)
    assert len(asm_check.check_text(a)) == 1


def test_compiler_wait_does_not_count():
    # a wait the compiler placed (outside inline assembly) is not the pinned one
    a = asm(*tr("v[10:11]", "v4"), "s_waitcnt lgkmcnt(0)", "v_mov_b32_e32 v1, v10", *WAIT)
    assert len(asm_check.check_text(a)) == 1


def test_branches():
    inside = asm(*tr("v[10:11]", "v4"), "s_cbranch_vccz .LBB0_2", "v_mul_f32_e32 v20, v21, v22", ".LBB0_2:",
                 *WAIT)
    assert asm_check.check_text(inside) == []
    leaving = asm(".LBB0_1:", *tr("v[10:11]", "v4"), "s_cbranch_vccz .LBB0_1", *WAIT)
    assert len(asm_check.check_text(leaving)) == 1
    ending = asm(*tr("v[10:11]", "v4"), "s_endpgm")
    assert asm_check.check_text(ending) != []


@pytest.mark.parametrize("src", [s for s in build.sources() if build.uses_async_reads(s)],
                         ids=lambda s: s.rsplit("/", 1)[-1])
def test_shipped_sources_pass(src):
    assert build.check_async_reads(src) > 0

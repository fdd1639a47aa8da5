"""The build's wait-state check of inline-asm matrix instructions (asm_lint),
on small assembly texts in the form hipcc writes them."""
from exact_attention_fwd_amd import asm_lint


def _kernel(*lines):
    body = "\n".join("\t" + ln if not ln.endswith(":") else ln for ln in lines)
    return f"k:\n{body}\n\ts_endpgm\n.Lfunc_end0:\n"


def _asm(ins):
    return [";;#ASMSTART", ins, ";;#ASMEND"]


MFMA32 = "v_mfma_f32_32x32x16_bf16 a[48:63], v[142:145], v[66:69], a[48:63]"
MFMA16 = "v_mfma_f32_16x16x32_bf16 v[50:53], v[90:93], a[12:15], v[50:53]"


def _rules(text):
    return sorted((f.rule, f.distance) for f in asm_lint.check(text))


def test_valu_write_right_before_inline_mfma():
    # a packed B operand written by the instruction just before the MFMA
    text = _kernel("v_cvt_pk_bf16_f32 v66, v66, v92", *_asm(MFMA32))
    assert _rules(text) == [("valu->mfma", 0)]
    text = _kernel("v_cvt_pk_bf16_f32 v67, v67, v93", "s_nop 0", *_asm(MFMA32))
    assert _rules(text) == [("valu->mfma", 1)]


def test_two_wait_states_are_enough():
    assert _rules(_kernel("v_cvt_pk_bf16_f32 v66, v66, v92", "s_nop 1", *_asm(MFMA32))) == []
    assert _rules(_kernel("v_cvt_pk_bf16_f32 v66, v66, v92", "v_add_f32_e32 v1, v2, v3",
                          "s_waitcnt lgkmcnt(0)", *_asm(MFMA32))) == []


def test_unrelated_or_compiler_pairs_pass():
    # a write of another register, and a pair of compiler-emitted instructions
    assert _rules(_kernel("v_cvt_pk_bf16_f32 v70, v66, v92", *_asm(MFMA32))) == []
    assert _rules(_kernel("v_cvt_pk_bf16_f32 v66, v66, v92", MFMA32)) == []


def test_result_read_distance_per_shape():
    # 16x16x32 (4 passes) needs 8, 32x32x16 (8 passes) needs 12
    for mfma, need, dst in ((MFMA16, 8, "v50"), ("v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]", 12, "v3")):
        close = _kernel(*_asm(mfma), f"s_nop {need - 2}", f"v_max_f32_e32 v99, v98, {dst}")
        assert _rules(close) == [("mfma->read", need - 1)]
        far = _kernel(*_asm(mfma), f"s_nop {need - 1}", f"v_max_f32_e32 v99, v98, {dst}")
        assert _rules(far) == []


def test_result_read_by_inline_asm_after_builtin_mfma():
    text = _kernel(MFMA16, "s_nop 3", *_asm("v_max3_f32 v78, v78, v50, v51"))
    assert _rules(text) == [("mfma->read", 4)]


def test_accumulating_chain_and_operand_reuse_pass():
    # the next MFMA accumulating onto the same range, and A/B registers
    # rewritten right after issue (read at issue)
    text = _kernel(*_asm(MFMA16), *_asm(MFMA16), "v_mov_b32_e32 v90, 0", "ds_read_b128 v[90:93], v1")
    assert _rules(text) == []


def test_result_as_operand_of_next_mfma():
    nxt = "v_mfma_f32_16x16x32_bf16 v[60:63], v[50:53], a[12:15], 0"
    assert _rules(_kernel(*_asm(MFMA16), *_asm(nxt))) == [("mfma->mfma", 0)]


def test_srcc_overwritten_early():
    mfma = "v_mfma_f32_16x16x32_bf16 v[0:3], v[8:11], v[12:15], v[4:7]"
    assert _rules(_kernel(*_asm(mfma), "v_mov_b32_e32 v5, 0")) == [("srcc->write", 0)]


def test_branches_are_followed():
    # the reader sits behind a taken branch; the write before a join label
    text = _kernel(*_asm(MFMA16), "s_cbranch_scc1 .LBB0_2", "s_nop 7", ".LBB0_2:", "v_mov_b32_e32 v1, v51")
    assert _rules(text) == [("mfma->read", 1)]
    text = _kernel("s_cbranch_scc1 .LBB0_3", "v_mov_b32_e32 v90, 0", ".LBB0_3:", *_asm(MFMA16))
    assert _rules(text) == [("valu->mfma", 0)]


def test_lds_dma_address_is_not_a_write():
    # the vector operand of a load into LDS is its address, not a result
    text = _kernel(*_asm(MFMA16), "buffer_load_dwordx4 v50, s[20:23], 0 offen lds")
    assert [f.rule for f in asm_lint.check(text)] == ["mfma->read"]  # read of v50 as the address
    assert asm_lint._written(asm_lint._Ins("buffer_load_dwordx4 v50, s[20:23], 0 offen lds",
                                           "buffer_load_dwordx4", ["v50", "s[20:23]", "0 offen lds"], False)) == set()

"""The build's check that no scratch access (register spill or reload) sits
inside a loop of an attention kernel, on hand-written assembly listings."""
from quantized_attention_sage_amd.build import loops_with_scratch, m0_outside_inline_asm

HEAD = "_ZN4sage12_GLOBAL__N_115attn_fwd_kernelEv:\n"
TAIL = ".Lfunc_end0:\n"


def test_spill_outside_the_loop_passes():
    asm = HEAD + """\tscratch_store_dwordx2 off, v[192:193], off ; 8-byte Folded Spill
.LBB0_2:
\tv_add_f32_e32 v1, v2, v3
\ts_cbranch_scc1 .LBB0_2
\tscratch_load_dwordx2 v[192:193], off, off ; 8-byte Folded Reload
\ts_endpgm
""" + TAIL
    assert loops_with_scratch(asm) == []


def test_reload_inside_the_loop_is_found():
    asm = HEAD + """.LBB0_2:
\tv_add_f32_e32 v1, v2, v3
\tscratch_load_dwordx2 v[192:193], off, off ; 8-byte Folded Reload
\ts_branch .LBB0_2
\ts_endpgm
""" + TAIL
    bad = loops_with_scratch(asm)
    assert len(bad) == 1 and bad[0][3] == 1


def test_forward_branch_is_not_a_loop():
    asm = HEAD + """\ts_cbranch_execz .LBB0_4
\tscratch_store_dword off, v7, off
.LBB0_4:
\ts_endpgm
""" + TAIL
    assert loops_with_scratch(asm) == []


def test_layout_back_jump_that_is_no_loop_passes():
    # .LBB0_3 jumps back to .LBB0_2 in the listing, but .LBB0_2 leaves forward
    # for good: no cycle holds the reload.
    asm = HEAD + """\ts_cbranch_scc0 .LBB0_3
.LBB0_2:
\tv_mov_b32_e32 v66, v250
\ts_branch .LBB0_5
.LBB0_3:
\tscratch_load_dwordx2 v[192:193], off, off ; 8-byte Folded Reload
\ts_cbranch_scc1 .LBB0_2
.LBB0_4:
\ts_branch .LBB0_5
.LBB0_5:
\ts_endpgm
""" + TAIL
    assert loops_with_scratch(asm) == []


def test_conditional_back_edge_loop_is_found():
    asm = HEAD + """.LBB0_1:
\tv_add_f32_e32 v1, v2, v3
\ts_cbranch_execz .LBB0_3
\tscratch_store_dword off, v7, off
.LBB0_3:
\ts_cbranch_scc1 .LBB0_1
\ts_endpgm
""" + TAIL
    assert len(loops_with_scratch(asm)) == 1


def test_m0_only_inside_inline_asm():
    ok = HEAD + """\t;;#ASMSTART
\ts_mov_b32 m0, s4
\tbuffer_load_dword v1, s[0:3], 0 offen lds
\t;;#ASMEND
\ts_endpgm
""" + TAIL
    assert m0_outside_inline_asm(ok) == []
    bad = ok.replace("\ts_endpgm", "\ts_mov_b32 m0, -1\n\ts_endpgm")
    assert len(m0_outside_inline_asm(bad)) == 1

"""The build-time check for barrier loops with per-lane exits."""
import glob
import os

import pytest

from tile_pipelined_gemm_amd import isa_check

HEAD = "_Z1kv:\n\ts_mov_b32 s0, 0\n"

# A loop holding a barrier whose exit is a scalar (uniform) branch.
UNIFORM = HEAD + """.LBB0_1:
\ts_barrier
\ts_add_u32 s0, s0, 1
\ts_cmp_lt_u32 s0, 8
\ts_cbranch_scc1 .LBB0_1
\ts_endpgm
"""

# The same loop left one lane at a time: exec shrinks, exit when empty.
PER_LANE = HEAD + """.LBB0_1:
\ts_barrier
\tv_cmp_le_u32_e32 vcc, 8, v1
\ts_or_b64 s[4:5], vcc, s[4:5]
\ts_andn2_b64 exec, exec, s[4:5]
\ts_cbranch_execz .LBB0_2
\ts_branch .LBB0_1
.LBB0_2:
\ts_endpgm
"""

# A divergent if inside a uniform barrier loop (the usual `if (tid == 0)`).
IF_INSIDE = HEAD + """.LBB0_1:
\ts_and_saveexec_b64 s[6:7], s[2:3]
\ts_cbranch_execz .LBB0_3
\tglobal_atomic_add v2, v3, s[8:9]
.LBB0_3:
\ts_or_b64 exec, exec, s[6:7]
\ts_barrier
\ts_add_u32 s0, s0, 1
\ts_cmp_lt_u32 s0, 8
\ts_cbranch_scc1 .LBB0_1
\ts_endpgm
"""

# A per-lane spin loop without a barrier inside a uniform barrier loop.
SPIN_INSIDE = HEAD + """.LBB0_1:
\ts_barrier
.LBB0_2:
\ts_sleep 8
\ts_andn2_b64 exec, exec, s[12:13]
\ts_cbranch_execnz .LBB0_2
\ts_or_b64 exec, exec, s[14:15]
\ts_add_u32 s0, s0, 1
\ts_cmp_lt_u32 s0, 8
\ts_cbranch_scc1 .LBB0_1
\ts_endpgm
"""


def _check(text):
    (name, lines), = list(isa_check.kernels(text))
    return isa_check.divergent_barrier_loops(lines)


def test_uniform_exit_passes():
    assert _check(UNIFORM) == []


def test_per_lane_exit_of_barrier_loop_is_found():
    assert _check(PER_LANE) == [(".LBB0_1", "s_cbranch_execz .LBB0_2")]


def test_divergent_if_and_spin_inside_uniform_loop_pass():
    assert _check(IF_INSIDE) == []
    assert _check(SPIN_INSIDE) == []


def test_built_kernels_are_clean():
    from tile_pipelined_gemm_amd import build
    files = glob.glob(os.path.join(build.BUILD, "*-hip-amdgcn-amd-amdhsa-*.s"))
    if not files:
        pytest.skip("library not built in this tree")
    for f in files:
        assert isa_check.check_file(f) == {}, f


def test_spill_between_mfmas_is_found():
    mf = "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]\n"
    text = HEAD + mf * 3 + "\tscratch_load_dword v9, off, off offset:8\n" + mf * 3 + "\ts_endpgm\n"
    (name, lines), = list(isa_check.kernels(text))
    assert isa_check.spills_among_mfma(lines) == ["scratch_load_dword v9, off, off offset:8"]
    far = HEAD + mf + "\ts_nop 0\n" * 12 + "\tscratch_store_dword off, v1, off\n" + "\ts_endpgm\n"
    (name, lines), = list(isa_check.kernels(far))
    assert isa_check.spills_among_mfma(lines) == []


def test_wide_store_data_rewritten_right_after_is_flagged():
    body = """
        buffer_store_dwordx4 v[36:39], v34, s[60:63], s3 offen
        v_cndmask_b32_e32 v36, v51, v50, vcc
        s_endpgm
    """.splitlines()
    assert len(isa_check.wide_store_data_overwrites(body)) == 1


def test_wide_store_data_rewritten_after_enough_wait_states_passes():
    ok_nop = """
        buffer_store_dwordx4 v[36:39], v34, s[60:63], s3 offen
        s_nop 1
        v_mov_b32_e32 v36, 0
    """.splitlines()
    ok_gap = """
        buffer_store_dwordx4 v[36:39], v34, s[60:63], s3 offen
        s_add_i32 s3, s3, 16
        v_add_u32_e32 v40, s3, v34
        v_mov_b32_e32 v37, 0
    """.splitlines()
    ok_other = """
        buffer_store_dwordx4 v[36:39], v34, s[60:63], s3 offen
        v_mov_b32_e32 v40, 0
    """.splitlines()
    ok_narrow = """
        buffer_store_dwordx2 v[36:37], v34, s[60:63], s3 offen
        v_mov_b32_e32 v36, 0
    """.splitlines()
    for body in (ok_nop, ok_gap, ok_other, ok_narrow):
        assert isa_check.wide_store_data_overwrites(body) == []


def test_wide_store_register_range_overlap():
    body = """
        buffer_store_dwordx3 v[10:12], v0, s[0:3], s4 offen
        v_pk_mov_b32 v[12:13], v[0:1], v[0:1] op_sel:[0,1]
    """.splitlines()
    assert len(isa_check.wide_store_data_overwrites(body)) == 1


def test_lds_dma_right_after_m0_write_is_flagged():
    lines = ["s_mov_b32 m0, s11", "buffer_load_dwordx4 v2, s[56:59], s14 offen lds", "s_endpgm"]
    assert len(isa_check.m0_lds_dma_hazards(lines)) == 1
    lines = ["s_cselect_b32 m0, 0x400, -1", "global_load_lds_dword v[2:3], off lds", "s_endpgm"]
    assert len(isa_check.m0_lds_dma_hazards(lines)) == 1


def test_lds_dma_after_m0_write_and_wait_state_passes():
    lines = ["s_mov_b32 m0, s11", "s_nop 0", "buffer_load_dwordx4 v2, s[56:59], s14 offen lds",
             "s_mov_b32 s4, m0", "buffer_load_dwordx4 v2, s[56:59], s14 offen lds",   # reads M0, no write
             "s_mov_b32 m0, s11", "v_add_u32 v1, v1, v2", "buffer_load_dwordx4 v2, s[56:59], s14 offen lds",
             "s_mov_b32 m0, s11", "buffer_load_dwordx4 v2, s[56:59], s14 offen",      # not an LDS DMA
             "s_endpgm"]
    assert isa_check.m0_lds_dma_hazards(lines) == []

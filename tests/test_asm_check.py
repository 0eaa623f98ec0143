"""The build-time assembly check (`mixture_experts_expert_moe_amd/asm_check.py`)
on small hand-written gfx950 listings: it must flag a use of a load's
destination before a vmcnt wait retires the load, follow in-order retirement
(vmcnt(N) leaves the newest N loads pending) and loop back-edges, and treat
LDS-DMA loads as having no register destination."""
import os
import tempfile


def _check(body: str):
    from mixture_experts_expert_moe_amd import asm_check  # build-time module; imported only when run
    src = "_Z15big_gemm_kernelv:\n" + body + "\n\ts_endpgm\n.Lfunc_end0:\n"
    with tempfile.NamedTemporaryFile("w", suffix=".s", delete=False) as f:
        f.write(src)
    try:
        return asm_check.check_file(f.name)
    finally:
        os.unlink(f.name)


def test_use_before_wait_is_flagged():
    probs = _check("""
	global_load_dwordx4 v[0:3], v[10:11], off
	v_add_u32_e32 v4, v0, v1
	s_waitcnt vmcnt(0)""")
    assert len(probs) == 1 and "v_add_u32_e32 v4, v0, v1" in probs[0]


def test_use_after_wait_is_clean():
    assert _check("""
	global_load_dwordx4 v[0:3], v[10:11], off
	s_waitcnt vmcnt(0)
	v_add_u32_e32 v4, v0, v1""") == []


def test_in_order_retirement():
    # vmcnt(1) retires the older load only: v0 is ready, v20 is not
    ok = _check("""
	global_load_dword v0, v[10:11], off
	global_load_dword v20, v[12:13], off
	s_waitcnt vmcnt(1)
	v_add_u32_e32 v4, v0, v0
	s_waitcnt vmcnt(0)
	v_add_u32_e32 v5, v20, v20""")
    assert ok == []
    bad = _check("""
	global_load_dword v0, v[10:11], off
	global_load_dword v20, v[12:13], off
	s_waitcnt vmcnt(1)
	v_add_u32_e32 v5, v20, v20
	s_waitcnt vmcnt(0)""")
    assert len(bad) == 1 and "v20" in bad[0]


def test_hazard_around_a_loop_back_edge():
    # the load issued at the bottom of the loop is still pending at the top
    probs = _check("""
	s_mov_b32 s0, 4
.LBB0_1:
	v_mov_b32_e32 v7, v0
	global_load_dword v0, v[10:11], off
	s_add_i32 s0, s0, -1
	s_cmp_lg_u32 s0, 0
	s_cbranch_scc1 .LBB0_1
	s_waitcnt vmcnt(0)""")
    assert len(probs) == 1 and "v_mov_b32_e32 v7, v0" in probs[0]


def test_lds_dma_has_no_register_destination():
    # the address register of an LDS DMA load may be reused right away
    assert _check("""
	global_load_lds_dwordx4 v[2:3], off
	v_mov_b32_e32 v2, 0
	s_waitcnt vmcnt(0)""") == []


def test_scratch_traffic_is_rejected():
    probs = _check("""
	scratch_load_dword v1, off, s0
	s_waitcnt vmcnt(0)""")
    assert any("forbidden" in p for p in probs)

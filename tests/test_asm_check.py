"""The static check of hand-timed asm loads (routed_expert_cache_amd/asm_check):
each hazard class planted in small synthetic gfx950 assembly is reported, the
safe forms are not, and the library's own kernels come out clean."""
import os
import shutil

import pytest

from routed_expert_cache_amd import asm_check
from routed_expert_cache_amd import build as B


def fn(body):
    """Wrap instruction lines as one function the way the compiler prints it."""
    return "k:  ; @k\n" + "\n".join(body) + "\n.Lfunc_end0:\n"


def asm(line):
    return [";;#ASMSTART", line, ";;#ASMEND"]


def hazards(body):
    return asm_check.check_asm(fn(body))


def test_wait_then_use_is_clean():
    body = asm("ds_read_b128 v[4:7], v1") + asm("s_waitcnt lgkmcnt(0)") + [
        "v_mfma_f32_16x16x32_bf16 v[8:11], v[4:7], v[12:15], v[8:11]", "s_endpgm"]
    assert hazards(body) == []


def test_copy_before_wait_is_reported():
    body = asm("ds_read_b128 v[4:7], v1") + ["v_mov_b32_e32 v20, v5"] + asm("s_waitcnt lgkmcnt(0)") + ["s_endpgm"]
    h = hazards(body)
    assert len(h) == 1 and "v5" in h[0][3] and h[0][2].startswith("v_mov")


def test_overwrite_before_wait_is_reported():
    body = asm("ds_read_b128 v[4:7], v1") + ["v_mov_b32_e32 v6, 0"] + asm("s_waitcnt lgkmcnt(0)") + ["s_endpgm"]
    assert [x[3] for x in hazards(body)] == ["v6 touched while its asm load is in flight"]


def test_partial_wait_retires_only_older_reads():
    reads = asm("ds_read_b128 v[4:7], v1") + asm("ds_read_b128 v[8:11], v2")
    ok = reads + asm("s_waitcnt lgkmcnt(1)") + ["v_mov_b32_e32 v20, v4", "s_endpgm"]
    assert hazards(ok) == []
    bad = reads + asm("s_waitcnt lgkmcnt(1)") + ["v_mov_b32_e32 v20, v8", "s_endpgm"]
    assert [x[3] for x in hazards(bad)] == ["v8 touched while its asm load is in flight"]


def test_compiler_lds_ops_count_as_younger():
    # a compiler ds_write after the asm read: lgkmcnt(1) then retires the read
    body = asm("ds_read_b128 v[4:7], v1") + ["ds_write_b32 v3, v2"] + asm("s_waitcnt lgkmcnt(1)") + [
        "v_mov_b32_e32 v20, v4", "s_endpgm"]
    assert hazards(body) == []


def test_vmcnt_wait_does_not_retire_lds_reads():
    body = asm("ds_read_b128 v[4:7], v1") + ["s_waitcnt vmcnt(0)", "v_mov_b32_e32 v20, v4", "s_endpgm"]
    assert len(hazards(body)) == 1


def test_combined_wait_and_wait_zero():
    for w in ("s_waitcnt vmcnt(0) lgkmcnt(0)", "s_waitcnt 0"):
        body = asm("ds_read_b128 v[4:7], v1") + [w, "v_mov_b32_e32 v20, v4", "s_endpgm"]
        assert hazards(body) == [], w


def test_scalar_load_needs_wait_zero():
    load = asm("s_load_dword s10, s[2:3], 0x0")
    body = load + asm("ds_read_b128 v[4:7], v1") + asm("s_waitcnt lgkmcnt(1)") + [
        "v_mul_f32_e32 v20, s10, v21", "s_endpgm"]
    assert [x[3] for x in hazards(body)] == ["s10 touched while its asm load is in flight"]
    body = load + asm("s_waitcnt lgkmcnt(0)") + ["v_mul_f32_e32 v20, s10, v21", "s_endpgm"]
    assert hazards(body) == []


def test_one_branch_path_without_wait_is_reported():
    body = asm("ds_read_b128 v[4:7], v1") + [
        "s_cbranch_scc1 .LBB0_2",
        "s_waitcnt lgkmcnt(0)",
        ".LBB0_2:",
        "v_mov_b32_e32 v20, v4",
        "s_endpgm"]
    assert len(hazards(body)) == 1


def test_loop_back_edge_carries_reads_in_flight():
    # the read at the end of the body is in flight when the loop top copies it
    body = [".LBB0_1:", "v_mov_b32_e32 v20, v4"] + asm("ds_read_b128 v[4:7], v1") + [
        "s_cbranch_scc1 .LBB0_1", "s_waitcnt lgkmcnt(0)", "s_endpgm"]
    assert len(hazards(body)) == 1
    body = [".LBB0_1:", "v_mov_b32_e32 v20, v4"] + asm("ds_read_b128 v[4:7], v1") + asm(
        "s_waitcnt lgkmcnt(0)") + ["s_cbranch_scc1 .LBB0_1", "s_endpgm"]
    assert hazards(body) == []


def test_unconditional_branch_ends_the_path():
    body = asm("ds_read_b128 v[4:7], v1") + asm("s_waitcnt lgkmcnt(0)") + [
        "s_branch .LBB0_3", "v_mov_b32_e32 v20, v4", ".LBB0_3:", "s_endpgm"]
    assert hazards(body) == []


def test_compiler_reads_are_not_tracked():
    # a read the compiler issued itself gets its own waits from the compiler
    body = ["ds_read_b128 v[4:7], v1", "v_mov_b32_e32 v20, v4", "s_endpgm"]
    assert hazards(body) == []


@pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None, reason="hipcc not installed")
@pytest.mark.parametrize("src", B.GPU_SOURCES)
def test_library_kernels_are_clean(src):
    text = asm_check.device_asm(os.path.join(B.CSRC, src), B.HIPCC, B.FLAGS)
    assert ".amdhsa_kernel" in text
    assert asm_check.check_asm(text) == []

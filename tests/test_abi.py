"""The C ABI boundary, checked without a GPU: the header parses as C, the
shared library loads and exports every function the header declares, and
the ctypes structures of the binding match the C layouts."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "routed_expert_cache_amd", "libmoe_gfx950.so")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*|int32_t)\s+(moe_\w+)\s*\(", src, flags=re.M)))


def test_header_is_valid_c():
    r = subprocess.run(["gcc", "-std=c99", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        "-x", "c", HEADER], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_library_exports_every_declared_function():
    assert os.path.exists(LIB), "build the library first: python -m routed_expert_cache_amd.build"
    lib = ctypes.CDLL(LIB)
    names = declared_functions()
    assert len(names) >= 18
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_header():
    import routed_expert_cache_amd.binding as b
    assert sorted(b.EXPORTS) == declared_functions()


def test_struct_layouts_match_header():
    import routed_expert_cache_amd.binding as b
    prog = r'''
#include <stdio.h>
#include <stddef.h>
#include "moe.h"
int main(void) {
  printf("%zu %zu %zu %zu\n", sizeof(moe_slots), sizeof(moe_host_pool), sizeof(moe_cache_cfg), sizeof(moe_step_out));
  printf("%zu %zu %zu\n", offsetof(moe_slots, w_gate_up), offsetof(moe_slots, s_down), offsetof(moe_cache_cfg, bh));
  printf("%zu\n", offsetof(moe_step_out, counts));
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(prog)
        exe = os.path.join(d, "t")
        r = subprocess.run(["gcc", "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                            "-I" + os.path.dirname(HEADER), c, "-o", exe], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        out = subprocess.run([exe], capture_output=True, text=True).stdout.split()
    vals = [int(v) for v in out]
    assert vals[:4] == [ctypes.sizeof(b.Slots), ctypes.sizeof(b.HostPool), ctypes.sizeof(b.CacheCfg),
                        ctypes.sizeof(b.StepOutC)]
    assert vals[4:] == [b.Slots.w_gate_up.offset, b.Slots.s_down.offset, b.CacheCfg.bh.offset,
                        b.StepOutC.counts.offset]


def test_status_codes_match_header():
    import routed_expert_cache_amd.binding as b
    src = open(HEADER).read()
    for name, val in re.findall(r"(MOE_(?:OK|ERR_\w+))\s*=\s*(-?\d+)", src):
        assert b.STATUS[int(val)] == name


def test_forward_rejects_internal_modes():
    """The public forward calls take only the three public modes (the wait
    test's internal launch mode among the refused): checked before anything
    else, so no GPU is needed."""
    import routed_expert_cache_amd.binding as b
    for mode in (3, 0x80000000):
        assert b._lib.moe_expert_forward(None, None, None, None, 1, 1, None, None, 0, mode, None) == -1
        assert b._lib.moe_expert_forward_merge(None, None, None, None, 1, 1, None, None, None, None, None, 0,
                                               mode, None) == -1


def test_decode_wait_test_arguments():
    """The wait test's poll count is checked before anything else: no GPU needed."""
    import routed_expert_cache_amd.binding as b
    for bad in (0, (1 << 22) + 1):
        assert b._lib.moe_decode_wait_test(None, None, None, None, 1, 1, None, None, 0, bad, None) == -1   # MOE_ERR_ARG


def test_decode_grid_override_arguments():
    """The decode launch-shape override is host state: checked without a GPU."""
    import routed_expert_cache_amd.binding as b
    for bad in (-1, 4097):
        with pytest.raises(b.MoeError) as ei:
            b.decode_grid_override(bad)
        assert ei.value.status == -1                     # MOE_ERR_ARG
    b.decode_grid_override(4096)
    b.decode_grid_override(0)

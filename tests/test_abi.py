"""The C-ABI library loads on the host and exports every call include/wq.h declares.

No kernel runs here: only calls that return before touching a device.
"""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wq.h")
LIB = os.path.join(ROOT, "fp8_dynamic_quant_amd", "libwq.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libwq.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(wq_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("wq_dynamic_quant", "wq_group_quant_fp8_ue8m0", "wq_quant_matmul", "wq_fused_quant_matmul"):
        assert n in names


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    L = ctypes.CDLL(LIB)
    for n in declared_functions():
        getattr(L, n)


def test_host_only_calls():
    from fp8_dynamic_quant_amd import lib, EXPORTS
    L = lib()
    assert set(EXPORTS) == set(declared_functions())
    assert L.wq_abi_version() == 3
    assert L.wq_workspace_bytes() >= 1 << 20
    for s in range(0, 7):
        assert len(L.wq_status_str(s)) > 0
    # NULL checks return before any device call
    h = ctypes.c_void_p()
    assert L.wq_ctx_create(0, None, 1 << 30, ctypes.byref(h)) == 1
    assert L.wq_ctx_create(0, None, 0, None) == 1
    assert L.wq_dynamic_quant(None, None, 1, 1, 16, 16, None, 0.0, None, None, None, None) == 1
    assert L.wq_group_quant_fp8_ue8m0(None, None, 1, 1, 128, None, None, None) == 1
    assert L.wq_quant_matmul(None, None, None) == 1
    assert L.wq_fused_quant_matmul(None, None, 1, 16, 16, None, None, 16, None, 16, None, None, None, None) == 1
    assert L.wq_moe_sort(None, None, 1, 1, 1, None, None, None, None) == 1
    assert L.wq_pack_weight_i8(None, None, 16, 64, 64, None, None) == 1
    assert L.wq_fused_quant_matmul_packed(None, None, 1, 16, 16, None, None, 16, None, 16, None, None, None,
                                          None) == 1
    assert L.wq_group_quant_mxfp8(None, None, 1, 1, 32, None, None, None) == 1

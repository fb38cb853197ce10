"""The C-ABI library loads on the host and exports every symbol that
include/*.h declares; host-only entry points (workspace sizing, status text,
argument validation that returns before any HIP call) work without a GPU."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quantized_moe_expert_lds_amd", "lib", "libmoe_ffn.so")


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        names |= set(re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s+(moe_\w+)\s*\(", text, re.M))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_qmoe_build", os.path.join(ROOT, "quantized_moe_expert_lds_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build_all()
    return ctypes.CDLL(LIB)


def test_header_declares_the_entry_points():
    assert {"moe_route", "moe_ffn_decode", "moe_ffn_prefill", "moe_workspace_size",
            "moe_residual_rmsnorm", "moe_status_string"} <= _declared()


def test_every_declared_symbol_is_exported(lib):
    for name in sorted(_declared()):
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"


def test_binding_names_match_header():
    import quantized_moe_expert_lds_amd as q
    assert set(q.EXPORTED_SYMBOLS) == _declared()
    for name in q.EXPORTED_SYMBOLS:
        assert callable(getattr(q, name))


def test_workspace_sizes(lib):
    lib.moe_workspace_size.restype = ctypes.c_size_t
    P = 8192 * 10
    pre = lib.moe_workspace_size(2, 8192, 2048, 768, 512, 10)
    # fp16 x, fp16 h per pair, fp32 gated output per pair dominate
    assert pre >= 8192 * 2048 * 2 + P * 768 * 2 + P * 2048 * 4
    assert lib.moe_workspace_size(1, 4, 2048, 768, 512, 10) >= 4 * 10 * 768 * 2
    assert lib.moe_workspace_size(0, 1, 2048, 0, 512, 10) > 0
    assert lib.moe_workspace_size(0, 0, 2048, 0, 512, 10) == 0
    assert lib.moe_workspace_size(9, 1, 2048, 768, 512, 10) == 0


def test_status_strings(lib):
    lib.moe_status_string.restype = ctypes.c_char_p
    assert lib.moe_status_string(0) == b"ok"
    for code in (-1, -2, -3, -4, -5):
        assert lib.moe_status_string(code) not in (b"ok", b"unknown status")


def test_validation_before_any_device_call(lib):
    # null descriptors / pointers are rejected on the host with MOE_ERR_ARG
    assert lib.moe_route(None, None, 0, 1, None, None, None, None, None, ctypes.c_size_t(0), None) == -1
    assert lib.moe_ffn_decode(None, None, 0, 1, None, None, 10, None, None, ctypes.c_size_t(0), None) == -1
    assert lib.moe_ffn_prefill(None, None, 0, 1, None, 10, None, None, None, None, ctypes.c_size_t(0), None) == -1
    lib.moe_residual_rmsnorm.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                                                  ctypes.c_void_p]
    assert lib.moe_residual_rmsnorm(None, None, None, 1, 8, 1e-6, None) == -1

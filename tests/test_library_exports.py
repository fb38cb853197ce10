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


def test_prefill_stack_validation_before_any_device_call(lib):
    """moe_prefill_stack rejects bad arguments on the host: status codes
    only, no pointer is dereferenced on the device."""
    import quantized_moe_expert_lds_amd as q
    P = ctypes.c_void_p
    fake = P(256)          # never dereferenced: validation fails first
    def stack(bits=2, d=2048, f=768, e=512, k=10, layers=2):
        return q._StackT(layers, e, d, f, k, bits, fake, None, fake, fake, fake, fake, fake, fake)
    call = lib.moe_prefill_stack
    call.argtypes = [ctypes.POINTER(q._StackT), P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, P, P,
                     ctypes.c_size_t, P]
    call.restype = ctypes.c_int
    size = lib.moe_prefill_stack_workspace_size
    size.argtypes = [ctypes.POINTER(q._StackT), ctypes.c_int]
    size.restype = ctypes.c_size_t
    st = stack()
    ok_args = lambda s, n=100, chunk=64, dtype=0: (ctypes.byref(s), fake, dtype, n, chunk, 1e-6, fake, fake,
                                                   size(ctypes.byref(s), chunk), None)
    assert size(ctypes.byref(st), 64) > 0
    assert size(ctypes.byref(st), 0) == 0
    assert size(None, 64) == 0
    assert call(*ok_args(st, n=0)) == -1                      # no tokens
    assert call(*ok_args(st, chunk=0)) == -1                  # no chunk
    assert call(*ok_args(st, dtype=7)) == -1                  # unknown dtype
    assert call(*ok_args(stack(bits=3))) == -2                # prefill GEMMs are 2-bit only
    assert call(*ok_args(stack(d=2080))) == -2                # d_model not a multiple of 256
    assert call(*ok_args(stack(f=800))) == -2                 # d_ff not a multiple of 128
    assert call(*ok_args(stack(k=600, e=512))) == -2          # top_k > n_experts
    args = list(ok_args(st))
    args[8] = args[8] - 1                                     # workspace one byte short
    assert call(*args) == -3


def test_prefill_q8_sizes_and_validation(lib):
    """The int8-activation prefill's workspace and host-side argument checks
    (no device call is reached)."""
    import quantized_moe_expert_lds_amd as q
    lib.moe_workspace_size.restype = ctypes.c_size_t
    T, D, F, E, K = 8192, 2048, 768, 512, 10
    P = T * K
    n = lib.moe_workspace_size(3, T, D, F, E, K)
    # int8 x and h, their block scales, fp32 gated output per pair
    assert n >= T * D + T * D // 32 * 4 + P * F + P * F // 32 * 4 + P * D * 4
    assert lib.moe_workspace_size(3, T, D, 0, E, K) == 0
    V = ctypes.c_void_p
    fake = V(256)
    call = lib.moe_ffn_prefill_q8
    call.argtypes = [ctypes.POINTER(q._ExpertsT), V, ctypes.c_int, ctypes.c_int, V, ctypes.c_int, V, V, V, V,
                     ctypes.c_size_t, V]
    call.restype = ctypes.c_int
    def ex(bits=2, d=D, f=F):
        return q._ExpertsT(E, d, f, bits, fake, fake, fake, fake, fake, fake)
    args = lambda e, n_tok=64, ws=n, dtype=1: (ctypes.byref(e), fake, dtype, n_tok, fake, K, fake, fake, fake, fake,
                                               ws, None)
    assert call(None, fake, 1, 64, fake, K, fake, fake, fake, fake, n, None) == -1
    assert call(*args(ex(), n_tok=0)) == -1
    assert call(*args(ex(), dtype=5)) == -1
    assert call(*args(ex(bits=3))) == -2                      # the int8 path covers the 2-bit format
    assert call(*args(ex(d=2080))) == -2
    assert call(*args(ex(f=800))) == -2
    small = lib.moe_workspace_size(3, 64, D, F, E, K)
    assert call(*args(ex(), ws=small - 1)) == -3
    qz = lib.moe_quantize_q8
    qz.argtypes = [V, ctypes.c_int, ctypes.c_int, ctypes.c_int, V, V, V]
    qz.restype = ctypes.c_int
    assert qz(None, 0, 4, 64, fake, fake, None) == -1
    assert qz(fake, 0, 0, 64, fake, fake, None) == -1
    assert qz(fake, 3, 4, 64, fake, fake, None) == -1
    assert qz(fake, 0, 4, 48, fake, fake, None) == -2         # rows cut into blocks of 32

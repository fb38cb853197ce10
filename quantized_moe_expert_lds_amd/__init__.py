"""Python binding of ``libmoe_ffn.so`` (the C ABI in ``include/moe_ffn.h``).

Argument marshalling only: tensors are passed as device pointers with the
current torch stream; every step of the computation runs in the library's
HIP kernels.  Importing the package loads the library and raises if it has
not been built (``python quantized_moe_expert_lds_amd/build.py``): there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import torch

__all__ = [
    "MOE_OK", "MOE_ERR_ARG", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MOE_ERR_NO_DEVICE", "MOE_ERR_HIP",
    "MOE_F32", "MOE_BF16", "MOE_OP_ROUTE", "MOE_OP_DECODE", "MOE_OP_PREFILL", "moe_stack_workspace_size",
    "stack_workspace", "moe_prefill_stack_workspace_size", "prefill_stack_workspace", "moe_prefill_stack",
    "MOE_STACK_ERROR_OFFSET", "MoeError", "Router", "Experts", "Stack", "lib_path", "library",
    "moe_workspace_size", "workspace", "moe_route", "moe_ffn_decode", "moe_ffn_prefill", "moe_decode_stack",
    "moe_residual_rmsnorm", "moe_status_string", "EXPORTED_SYMBOLS", "moe_ffn_decode_noalloc",
    "MOE_OP_PREFILL_Q8", "moe_ffn_prefill_q8", "moe_quantize_q8",
]

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_NO_DEVICE, MOE_ERR_HIP = 0, -1, -2, -3, -4, -5
MOE_F32, MOE_BF16 = 0, 1
MOE_OP_ROUTE, MOE_OP_DECODE, MOE_OP_PREFILL, MOE_OP_PREFILL_Q8 = 0, 1, 2, 3
MOE_STACK_ERROR_OFFSET = 2304

EXPORTED_SYMBOLS = ("moe_workspace_size", "moe_route", "moe_ffn_decode", "moe_ffn_decode_noalloc",
                    "moe_ffn_prefill", "moe_stack_workspace_size", "moe_decode_stack", "moe_prefill_stack_workspace_size",
                    "moe_prefill_stack", "moe_residual_rmsnorm", "moe_status_string", "moe_ffn_prefill_q8",
                    "moe_quantize_q8")

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "lib", "libmoe_ffn.so")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {moe_status_string(status)} (status {status})")
        self.status = status


class _RouterT(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int), ("n_experts", ctypes.c_int), ("top_k", ctypes.c_int),
                ("w", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class _ExpertsT(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int), ("d_model", ctypes.c_int), ("d_ff", ctypes.c_int),
                ("bits", ctypes.c_int),
                ("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
                ("gate_s", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


class _StackT(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("n_experts", ctypes.c_int), ("d_model", ctypes.c_int),
                ("d_ff", ctypes.c_int), ("top_k", ctypes.c_int), ("bits", ctypes.c_int),
                ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
                ("gate_s", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is missing: build it with `python quantized_moe_expert_lds_amd/build.py`")
    lib = ctypes.CDLL(lib_path)
    P, I, Z, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
    lib.moe_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.moe_workspace_size.restype = Z
    lib.moe_route.argtypes = [ctypes.POINTER(_RouterT), P, I, I, P, P, P, P, P, Z, P]
    lib.moe_route.restype = I
    lib.moe_ffn_decode.argtypes = [ctypes.POINTER(_ExpertsT), P, I, I, P, P, I, P, P, Z, P]
    lib.moe_ffn_decode.restype = I
    lib.moe_ffn_decode_noalloc.argtypes = [ctypes.POINTER(_ExpertsT), P, I, I, P, P, I, P, P]
    lib.moe_ffn_decode_noalloc.restype = I
    lib.moe_ffn_prefill.argtypes = [ctypes.POINTER(_ExpertsT), P, I, I, P, I, P, P, P, P, Z, P]
    lib.moe_ffn_prefill.restype = I
    lib.moe_ffn_prefill_q8.argtypes = [ctypes.POINTER(_ExpertsT), P, I, I, P, I, P, P, P, P, Z, P]
    lib.moe_ffn_prefill_q8.restype = I
    lib.moe_quantize_q8.argtypes = [P, I, I, I, P, P, P]
    lib.moe_quantize_q8.restype = I
    lib.moe_stack_workspace_size.argtypes = [ctypes.POINTER(_StackT), I]
    lib.moe_stack_workspace_size.restype = Z
    lib.moe_decode_stack.argtypes = [ctypes.POINTER(_StackT), P, I, I, D, P, P, P, P, P, Z, P]
    lib.moe_decode_stack.restype = I
    lib.moe_prefill_stack_workspace_size.argtypes = [ctypes.POINTER(_StackT), I]
    lib.moe_prefill_stack_workspace_size.restype = Z
    lib.moe_prefill_stack.argtypes = [ctypes.POINTER(_StackT), P, I, I, I, D, P, P, Z, P]
    lib.moe_prefill_stack.restype = I
    lib.moe_residual_rmsnorm.argtypes = [P, P, P, I, I, D, P]
    lib.moe_residual_rmsnorm.restype = I
    lib.moe_status_string.argtypes = [I]
    lib.moe_status_string.restype = ctypes.c_char_p
    return lib


library = _load()


def moe_status_string(status: int) -> str:
    return library.moe_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return MOE_F32
    if x.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {x.dtype}")


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)


@dataclass
class Router:
    """Router of one layer: ``w`` fp32 [n_experts][d_model] (expert-major: row
    e is expert e's router vector), ``bias`` fp32 [n_experts] or None."""
    w: torch.Tensor
    bias: Optional[torch.Tensor]
    top_k: int
    _c: _RouterT = field(init=False, repr=False)

    def __post_init__(self):
        e, d = self.w.shape
        self._c = _RouterT(d, e, self.top_k, self.w.data_ptr(), 0 if self.bias is None else self.bias.data_ptr())

    @property
    def d_model(self) -> int:
        return self.w.shape[1]

    @property
    def n_experts(self) -> int:
        return self.w.shape[0]


@dataclass
class Experts:
    """Stored experts of one layer: codes int32 [E][N][K/32][words] and fp16
    scale bits int16 [E][N][K/32] for gate, up (N = d_ff, K = d_model) and
    down (N = d_model, K = d_ff)."""
    gate_q: torch.Tensor
    up_q: torch.Tensor
    down_q: torch.Tensor
    gate_s: torch.Tensor
    up_s: torch.Tensor
    down_s: torch.Tensor
    bits: int
    _c: _ExpertsT = field(init=False, repr=False)

    def __post_init__(self):
        e, f, nkb = self.gate_s.shape
        self._c = _ExpertsT(e, nkb * 32, f, self.bits,
                            self.gate_q.data_ptr(), self.up_q.data_ptr(), self.down_q.data_ptr(),
                            self.gate_s.data_ptr(), self.up_s.data_ptr(), self.down_s.data_ptr())

    @property
    def n_experts(self) -> int:
        return self._c.n_experts

    @property
    def d_model(self) -> int:
        return self._c.d_model

    @property
    def d_ff(self) -> int:
        return self._c.d_ff


@dataclass
class Stack:
    """All layers of a model, each tensor stored layer-major: router_w fp32
    [L][E][D] (expert-major rows), router_b fp32 [L][E] or None, codes int32
    [L][E][N][K/32][words] and scale bits int16 [L][E][N][K/32] for gate, up
    and down."""
    router_w: torch.Tensor
    router_b: Optional[torch.Tensor]
    gate_q: torch.Tensor
    up_q: torch.Tensor
    down_q: torch.Tensor
    gate_s: torch.Tensor
    up_s: torch.Tensor
    down_s: torch.Tensor
    bits: int
    top_k: int
    _c: _StackT = field(init=False, repr=False)

    def __post_init__(self):
        L, E, D = self.router_w.shape
        F = self.gate_s.shape[2]
        self._c = _StackT(L, E, D, F, self.top_k, self.bits, self.router_w.data_ptr(),
                          0 if self.router_b is None else self.router_b.data_ptr(),
                          self.gate_q.data_ptr(), self.up_q.data_ptr(), self.down_q.data_ptr(),
                          self.gate_s.data_ptr(), self.up_s.data_ptr(), self.down_s.data_ptr())

    @property
    def n_layers(self) -> int:
        return self._c.n_layers

    @property
    def n_experts(self) -> int:
        return self._c.n_experts

    @property
    def d_model(self) -> int:
        return self._c.d_model

    @property
    def d_ff(self) -> int:
        return self._c.d_ff


def moe_workspace_size(op: int, n_tokens: int, d_model: int, d_ff: int, n_experts: int, top_k: int) -> int:
    return int(library.moe_workspace_size(op, n_tokens, d_model, d_ff, n_experts, top_k))


def workspace(op: int, n_tokens: int, d_model: int, d_ff: int, n_experts: int, top_k: int,
              device="cuda") -> torch.Tensor:
    """A zero-filled workspace of the size ``op`` needs (torch allocations are
    256-byte aligned)."""
    n = moe_workspace_size(op, n_tokens, d_model, d_ff, n_experts, top_k)
    if n == 0:
        raise MoeError("moe_workspace_size", MOE_ERR_ARG)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_route(router: Router, x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
              bucket_offsets: Optional[torch.Tensor] = None, bucket_pairs: Optional[torch.Tensor] = None,
              ws: Optional[torch.Tensor] = None, stream=None) -> None:
    st = library.moe_route(ctypes.byref(router._c), _ptr(x), _dtype(x), x.shape[0], _ptr(topk_ids), _ptr(topk_w),
                           _ptr(bucket_offsets), _ptr(bucket_pairs), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream(stream))
    _check("moe_route", st)


def moe_ffn_decode(experts: Experts, x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                   y: torch.Tensor, ws: Optional[torch.Tensor], stream=None) -> None:
    st = library.moe_ffn_decode(ctypes.byref(experts._c), _ptr(x), _dtype(x), x.shape[0], _ptr(topk_ids),
                                _ptr(topk_w), topk_ids.shape[1], _ptr(y), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(stream))
    _check("moe_ffn_decode", st)


def moe_ffn_decode_noalloc(experts: Experts, x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                           y: torch.Tensor, stream=None) -> None:
    """moe_ffn_decode with the library's per-device scratch instead of a
    workspace (no allocation; overlapping calls on one device race)."""
    st = library.moe_ffn_decode_noalloc(ctypes.byref(experts._c), _ptr(x), _dtype(x), x.shape[0], _ptr(topk_ids),
                                        _ptr(topk_w), topk_ids.shape[1], _ptr(y), _stream(stream))
    _check("moe_ffn_decode_noalloc", st)


def moe_ffn_prefill(experts: Experts, x: torch.Tensor, topk_w: torch.Tensor, bucket_offsets: torch.Tensor,
                    bucket_pairs: torch.Tensor, y: torch.Tensor, ws: Optional[torch.Tensor], stream=None) -> None:
    st = library.moe_ffn_prefill(ctypes.byref(experts._c), _ptr(x), _dtype(x), x.shape[0], _ptr(topk_w),
                                 topk_w.shape[1], _ptr(bucket_offsets), _ptr(bucket_pairs), _ptr(y), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(stream))
    _check("moe_ffn_prefill", st)


def moe_ffn_prefill_q8(experts: Experts, x: torch.Tensor, topk_w: torch.Tensor, bucket_offsets: torch.Tensor,
                       bucket_pairs: torch.Tensor, y: torch.Tensor, ws: Optional[torch.Tensor], stream=None) -> None:
    """moe_ffn_prefill with int8 (Q8 block) activations on the int8 matrix
    cores; workspace of op MOE_OP_PREFILL_Q8."""
    st = library.moe_ffn_prefill_q8(ctypes.byref(experts._c), _ptr(x), _dtype(x), x.shape[0], _ptr(topk_w),
                                    topk_w.shape[1], _ptr(bucket_offsets), _ptr(bucket_pairs), _ptr(y), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(stream))
    _check("moe_ffn_prefill_q8", st)


def moe_quantize_q8(x: torch.Tensor, q: torch.Tensor, d: torch.Tensor, stream=None) -> None:
    """Q8 blocks of the rows of x: int8 codes q (x's shape) and fp32 scales d
    [rows][cols / 32]."""
    st = library.moe_quantize_q8(_ptr(x), _dtype(x), x.shape[0], x.shape[1], _ptr(q), _ptr(d), _stream(stream))
    _check("moe_quantize_q8", st)


def moe_stack_workspace_size(stack: Stack, n_tokens: int) -> int:
    return int(library.moe_stack_workspace_size(ctypes.byref(stack._c), n_tokens))


def stack_workspace(stack: Stack, n_tokens: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for moe_decode_stack."""
    n = moe_stack_workspace_size(stack, n_tokens)
    if n == 0:
        raise MoeError("moe_stack_workspace_size", MOE_ERR_ARG)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_decode_stack(stack: Stack, x: torch.Tensor, h_out: torch.Tensor, ws: Optional[torch.Tensor],
                     topk_ids: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                     eps: float = 1e-6, stream=None, h_layers: Optional[torch.Tensor] = None) -> None:
    st = library.moe_decode_stack(ctypes.byref(stack._c), _ptr(x), _dtype(x), x.shape[0], float(eps), _ptr(h_out),
                                  _ptr(topk_ids), _ptr(topk_w), _ptr(h_layers), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(stream))
    _check("moe_decode_stack", st)


def moe_prefill_stack_workspace_size(stack: Stack, chunk_tokens: int) -> int:
    return int(library.moe_prefill_stack_workspace_size(ctypes.byref(stack._c), chunk_tokens))


def prefill_stack_workspace(stack: Stack, chunk_tokens: int, device="cuda") -> torch.Tensor:
    """A workspace for moe_prefill_stack (it keeps no state between calls)."""
    n = moe_prefill_stack_workspace_size(stack, chunk_tokens)
    if n == 0:
        raise MoeError("moe_prefill_stack_workspace_size", MOE_ERR_ARG)
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_prefill_stack(stack: Stack, x: torch.Tensor, h_out: torch.Tensor, chunk_tokens: int,
                      ws: Optional[torch.Tensor], eps: float = 1e-6, stream=None) -> None:
    st = library.moe_prefill_stack(ctypes.byref(stack._c), _ptr(x), _dtype(x), x.shape[0], int(chunk_tokens),
                                   float(eps), _ptr(h_out), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(stream))
    _check("moe_prefill_stack", st)


def moe_residual_rmsnorm(h: torch.Tensor, y: Optional[torch.Tensor], u: torch.Tensor, eps: float = 1e-6,
                         stream=None) -> None:
    st = library.moe_residual_rmsnorm(_ptr(h), _ptr(y), _ptr(u), h.shape[0], h.shape[1], float(eps),
                                      _stream(stream))
    _check("moe_residual_rmsnorm", st)

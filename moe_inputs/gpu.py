"""Device-resident synthetic inputs: expert weights generated in HBM by the
GPU twin of the seeded generator (``csrc/gen.hip``), routers and activations
generated on the host and copied over.  Returns plain torch tensors.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

import moe_inputs as mi

_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libmoe_inputs.so")
_lib = None
_tables = {}


def _library():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise ImportError(f"{_LIB} is missing: build it with `python quantized_moe_expert_lds_amd/build.py`")
        _lib = ctypes.CDLL(_LIB)
        P, I = ctypes.c_void_p, ctypes.c_int
        _lib.moegen_expert_tensors.argtypes = [P, I, I, I, I, ctypes.c_float, P, P, P, P]
        _lib.moegen_expert_tensors.restype = I
    return _lib


def _table(device) -> torch.Tensor:
    key = str(device)
    if key not in _tables:
        _tables[key] = torch.from_numpy(mi.NORMAL_TABLE.copy()).to(device)
    return _tables[key]


def _gen(keys: np.ndarray, n: int, k: int, bits: int, q: torch.Tensor, s: torch.Tensor, device) -> None:
    kt = torch.from_numpy(keys.astype(np.uint64).view(np.int64)).to(device)
    st = _library().moegen_expert_tensors(ctypes.c_void_p(kt.data_ptr()), len(keys), n, k, bits,
                                          ctypes.c_float(0.02), ctypes.c_void_p(_table(device).data_ptr()),
                                          ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(s.data_ptr()),
                                          ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream))
    if st != 0:
        raise RuntimeError(f"moegen_expert_tensors failed with status {st}")


def expert_tensors(wl: mi.Workload, n_layers: int | None = None, bits: int | None = None, device="cuda"):
    """Stored experts of layers 0..n_layers-1, generated on the device.

    Returns a dict with 'gate_q', 'up_q', 'down_q' (int32 [L][E][N][K/32][words])
    and 'gate_s', 'up_s', 'down_s' (int16 [L][E][N][K/32])."""
    L = wl.n_layers if n_layers is None else n_layers
    bits = wl.bits if bits is None else bits
    words = 2 if bits == 2 else 3
    out = {}
    for name, tensor in (("gate", mi.GATE), ("up", mi.UP), ("down", mi.DOWN)):
        n, k = mi.tensor_shape(wl, tensor)
        q = torch.empty((L, wl.n_experts, n, k // 32, words), dtype=torch.int32, device=device)
        s = torch.empty((L, wl.n_experts, n, k // 32), dtype=torch.int16, device=device)
        for layer in range(L):
            keys = np.array([mi.expert_key(wl, layer, tensor, e) for e in range(wl.n_experts)], dtype=np.uint64)
            _gen(keys, n, k, bits, q[layer], s[layer], device)
        out[name + "_q"] = q
        out[name + "_s"] = s
    return out


def routers(wl: mi.Workload, n_layers: int | None = None, device="cuda"):
    """[(w, bias fp32 [E])] per layer on the device, with the router matrix
    stored expert-major: w fp32 [E][D] is the transpose of the host
    generator's [D][E] matrix (same values)."""
    L = wl.n_layers if n_layers is None else n_layers
    out = []
    for layer in range(L):
        w, b = mi.router_host(wl, layer)
        out.append((torch.from_numpy(np.ascontiguousarray(w.T)).to(device), torch.from_numpy(b).to(device)))
    return out


def activations(wl: mi.Workload, n_tokens: int | None = None, stream: int = 0, device="cuda") -> torch.Tensor:
    """Activations on the device: float32, or bfloat16 for bf16 workloads."""
    x = mi.activations_host(wl, n_tokens, stream)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)

"""Shared helpers for the GPU parity tests (device model setup, oracle-side
expert lookup, the row-normalised error metric)."""
from __future__ import annotations

import numpy as np

import moe_inputs as mi
from moe_inputs import host_cache

TOL = 2e-3          # max over rows of max|y_gpu - y_ref| / max|y_ref|


def row_rel_err(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    num = np.max(np.abs(got - want), axis=-1)
    den = np.maximum(np.max(np.abs(want), axis=-1), 1e-30)
    return float(np.max(num / den))


def floored_rel_err(got, want, floor=1e-3) -> float:
    """Elementwise relative error with the denominator floored at
    floor * max|want| of the row (near-zero outputs are not divided by ~0)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.maximum(np.abs(want), floor * np.max(np.abs(want), axis=-1, keepdims=True))
    den = np.maximum(den, 1e-30)
    return float(np.max(np.abs(got - want) / den))


def host_expert(wl_name: str, layer: int, expert: int, bits: int):
    """Stored (gate, up, down) of one expert from the host generator."""
    return host_cache.expert(wl_name, layer, expert, bits)


def oracle_experts(wl: mi.Workload, layer: int, bits: int | None = None):
    return host_cache.experts_of(wl, layer, bits)


def device_layers(wl, n_layers=None, bits=None, device="cuda"):
    """[(Router, Experts)] for the first n_layers layers of a workload."""
    import quantized_moe_expert_lds_amd as q
    import moe_inputs.gpu as g
    bits = wl.bits if bits is None else bits
    ex = g.expert_tensors(wl, n_layers, bits, device)
    rt = g.routers(wl, n_layers, device)
    layers = []
    for l, (w, b) in enumerate(rt):
        layers.append((q.Router(w, b if wl.zipf_bias else None, wl.top_k),
                       q.Experts(ex["gate_q"][l], ex["up_q"][l], ex["down_q"][l],
                                 ex["gate_s"][l], ex["up_s"][l], ex["down_s"][l], bits)))
    return layers, ex, rt


def device_stack(wl, bits=None, n_layers=None, device="cuda"):
    """The whole model of a workload as one Stack (plus the raw tensors)."""
    import torch
    import quantized_moe_expert_lds_amd as q
    import moe_inputs.gpu as g
    bits = wl.bits if bits is None else bits
    ex = g.expert_tensors(wl, n_layers, bits, device)
    rt = g.routers(wl, n_layers, device)
    rw = torch.stack([w for w, _ in rt]).contiguous()
    rb = torch.stack([b for _, b in rt]).contiguous() if wl.zipf_bias else None
    del rt
    st = q.Stack(rw, rb, ex["gate_q"], ex["up_q"], ex["down_q"], ex["gate_s"], ex["up_s"], ex["down_s"],
                 bits, wl.top_k)
    return st, ex, rw, rb

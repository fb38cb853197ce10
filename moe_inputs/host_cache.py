"""Host copies of stored experts, generated on demand and cached in-process.

A stored expert (codes and fp16 scales of gate, up and down) is a pure
function of (workload, layer, expert, bits), so the CPU side regenerates
exactly the experts a computation touches.  Generating one full-size expert
takes ~0.3 s of numpy, so batches of experts go to a spawn pool of numpy
workers (they never touch the GPU).  Nothing here computes any part of the
routed MoE FFN: it only draws and packs weights (``expert_tensor_host``).
"""
from __future__ import annotations

import atexit
import concurrent.futures as cf
import multiprocessing as mp
import os

import moe_inputs as mi

_CACHE: dict = {}
_pool = None
_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _generate(args):
    name, layer, expert, bits = args
    wl = mi.WORKLOADS[name]
    return args, tuple(mi.expert_tensor_host(wl, layer, t, expert, bits) for t in (mi.GATE, mi.UP, mi.DOWN))


def _init_worker(root):
    import sys
    if root not in sys.path:
        sys.path.insert(0, root)


def workers() -> int:
    """Pool size: the process's CPU share, at most 12, leaving two cores."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 2
    return max(1, min(12, n - 2))


def _get_pool():
    global _pool
    if _pool is None:
        _pool = cf.ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn"),
                                       initializer=_init_worker, initargs=(_ROOT,))
    return _pool


def shutdown() -> None:
    """Stop the worker pool (idempotent; also registered at exit)."""
    global _pool
    if _pool is not None:
        _pool.shutdown(wait=True, cancel_futures=True)
        _pool = None


atexit.register(shutdown)


def expert(wl_name: str, layer: int, expert_id: int, bits: int):
    """((gate_q, gate_s), (up_q, up_s), (down_q, down_s)) of one expert."""
    key = (wl_name, int(layer), int(expert_id), int(bits))
    if key not in _CACHE:
        _CACHE[key] = _generate(key)[1]
    return _CACHE[key]


def prefetch(wl_name: str, layer: int, experts, bits: int) -> None:
    """Generate the given experts of one layer into the cache, in parallel."""
    todo = [(wl_name, int(layer), int(e), int(bits)) for e in sorted(set(int(e) for e in experts))]
    todo = [a for a in todo if a not in _CACHE]
    if len(todo) <= 2:
        for a in todo:
            expert(*a)
        return
    for args, val in _get_pool().map(_generate, todo):
        _CACHE[args] = val


def experts_of(wl: mi.Workload, layer: int, bits: int | None = None):
    """Callable e -> stored expert e of ``layer`` (the form the oracle takes)."""
    bits = wl.bits if bits is None else bits
    return lambda e: expert(wl.name, layer, int(e), bits)


def clear() -> None:
    _CACHE.clear()

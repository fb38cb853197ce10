"""Parallel host generation of the experts the oracle needs (a spawn pool of
numpy workers; the workers never touch the GPU)."""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import helpers

_pool = None


def _work(args):
    import moe_inputs as mi
    name, layer, expert, bits = args
    wl = mi.WORKLOADS[name]
    return args, tuple(mi.expert_tensor_host(wl, layer, t, expert, bits) for t in (mi.GATE, mi.UP, mi.DOWN))


def _get_pool():
    global _pool
    if _pool is None:
        n = max(1, min(12, (os.cpu_count() or 2) - 2))
        _pool = cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"),
                                       initializer=_init_path, initargs=(os.path.dirname(os.path.abspath(__file__)),))
    return _pool


def _init_path(tests_dir):
    import sys
    root = os.path.dirname(tests_dir)
    for p in (root, tests_dir):
        if p not in sys.path:
            sys.path.insert(0, p)


def prefetch(wl_name: str, layer: int, experts, bits: int) -> None:
    """Fill helpers.host_expert's cache for the given experts."""
    todo = [(wl_name, layer, int(e), bits) for e in sorted(set(int(e) for e in experts))]
    todo = [a for a in todo if a not in helpers._EXPERT_CACHE]
    if len(todo) <= 2:
        for a in todo:
            helpers.host_expert(*a)
        return
    for args, val in _get_pool().map(_work, todo):
        helpers.host_expert_cache_put(args, val)

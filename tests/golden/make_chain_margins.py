"""Writes chain_margins.json: the oracle's top-k boundary margins, layer by
layer, of single-token streams through the 48-layer workloads.

For every candidate token (``moe_inputs.activations_host(wl, 1, stream=s)``)
it runs the oracle's residual chain (``oracle.moe_chain``) and records, per
layer, the smallest gap between adjacent logits among ranks 1..k+1 of that
layer's routing.  A routing decision whose margin is large cannot be flipped
by rounding differences of the size the GPU path makes, so the GPU parity
tests use this table to pick token streams that must match the oracle at
every layer.  Only ``oracle/`` and the seeded input generators are called.

    python tests/golden/make_chain_margins.py [n_candidates]
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import moe_inputs as mi                      # noqa: E402
from moe_inputs import host_cache            # noqa: E402
import oracle.moe_oracle as O                # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "chain_margins.json")


def boundary_margins(z: np.ndarray, k: int) -> np.ndarray:
    """Per row: min over r < k of (r-th largest - (r+1)-th largest) logit."""
    top = -np.sort(-z, axis=1)[:, :k + 1]
    return np.min(top[:, :-1] - top[:, 1:], axis=1)


def margins_for(wl_name: str, n: int):
    wl = mi.WORKLOADS[wl_name]
    x = np.concatenate([mi.activations_host(wl, 1, stream=s) for s in range(n)])
    routers = {}

    def router_of(l):
        if l not in routers:
            routers.clear()
            routers[l] = mi.router_host(wl, l)
        return routers[l]

    def prepare_of(l):
        def prep(ids):
            host_cache.clear()                 # earlier layers are done with
            host_cache.prefetch(wl.name, l, ids, wl.bits)
        return prep

    t0 = time.time()
    _, recs = O.moe_chain(x, wl.n_layers, router_of, lambda l: host_cache.experts_of(wl, l), wl.top_k, wl.bits,
                          prepare_of=prepare_of)
    out = np.zeros((n, wl.n_layers))
    for l, (u, ids, gates, y, h) in enumerate(recs):
        w, b = mi.router_host(wl, l)
        out[:, l] = boundary_margins(O.router_logits(u, w, b), wl.top_k)
    print(f"{wl_name}: {n} tokens in {time.time() - t0:.0f} s", flush=True)
    host_cache.clear()
    return out


def main():
    n = int(sys.argv[1]) if len(sys.argv) > 1 else 24
    res = {"what": "oracle top-k boundary margin per (token stream, layer): min gap between adjacent logits "
                   "among ranks 1..k+1; token s = moe_inputs.activations_host(wl, 1, stream=s)",
           "script": "tests/golden/make_chain_margins.py"}
    for name in ("decode_48layer", "verify4_3bit"):
        m = margins_for(name, n)
        res[name] = {"streams": list(range(n)), "margins": [[float(v) for v in row] for row in m]}
    with open(OUT, "w") as fh:
        json.dump(res, fh, indent=0)
    host_cache.shutdown()


if __name__ == "__main__":
    main()

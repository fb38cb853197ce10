"""Per-token comparison of a multi-layer GPU decode step with the oracle's
free-running residual chain (``oracle.moe_chain``).

The oracle never consumes a GPU value.  Both sides start from the same
seeded token and run their own chain; the GPU's per-layer residuals
(``moe_decode_stack``'s h_layers output) are compared with the oracle's
layer by layer, token by token.

Where the two chains may legitimately part ways.  The GPU carries the
activations and the SwiGLU intermediate as fp16 (the layer-by-layer calls) or
as two fp16 halves (the whole-step kernel), so its residual drifts from the
oracle's over the layers (~1e-4 and ~1e-7 relative).  Routing then sees logits
z(u_gpu) instead of z(u_oracle); expert e's logit moves by dz_e = (u_gpu -
u_oracle) . w_e (both routers accumulate in fp64, so summation order adds
only ~1e-15).  Two experts a, b can swap ranks only if the oracle's margin
z_a - z_b is below |dz_a| + |dz_b|.  The walk measures dz exactly from the
two u's at every layer and accepts a routing difference only under that
condition; after it, the token's two chains are no longer comparable and its
walk stops.  Tokens listed in ``full`` were chosen by the oracle alone
(tests/golden/chain_margins.json) to have a top-k boundary margin of at
least SELECT_MARGIN at every layer; for them the walk asserts, layer by
layer, that the measured drift 2 max|dz| stays below the oracle's margin
(so no swap is possible) and that they match at every layer, through the
final residual.
"""
from __future__ import annotations

import json
import os

import numpy as np

import moe_inputs as mi
from moe_inputs import host_cache
import oracle.moe_oracle as O
from helpers import TOL, floored_rel_err, row_rel_err

EPS = 1e-6
# Tokens whose oracle margin stays above this at every layer must follow the
# oracle through all layers.  It exceeds the largest logit drift 2 max|dz|
# measured on the 48-layer workloads; the walk re-checks that premise on
# every compared layer of those tokens.
SELECT_MARGIN = 7.5e-4
MARGINS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "chain_margins.json")

_CHAINS: dict = {}


def full_depth_streams(wl_name: str, n: int, skip=()):
    """The first n candidate streams whose oracle margin is >= SELECT_MARGIN at
    every layer (token s = activations_host(wl, 1, stream=s))."""
    with open(MARGINS) as fh:
        tab = json.load(fh)[wl_name]
    good = [s for s, m in zip(tab["streams"], tab["margins"]) if min(m) >= SELECT_MARGIN and s not in skip]
    assert len(good) >= n, f"only {len(good)} full-depth candidates for {wl_name}"
    return good[:n]


def stream_tokens(wl: mi.Workload, streams) -> np.ndarray:
    return np.concatenate([mi.activations_host(wl, 1, stream=s) for s in streams])


def oracle_chain(wl: mi.Workload, bits: int, x: np.ndarray, n_layers: int):
    """Oracle records (u, ids, gates, y, h_next) per layer for tokens x, one
    moe_chain over the tokens not computed before (tokens are independent)."""
    keys = [(wl.name, bits, n_layers, x[t].tobytes()) for t in range(x.shape[0])]
    todo = [t for t in range(x.shape[0]) if keys[t] not in _CHAINS]
    if todo:
        zipf = wl.zipf_bias

        def router_of(l):
            w, b = mi.router_host(wl, l)
            return w, (b if zipf else None)

        def prepare_of(l):
            return lambda ids: host_cache.prefetch(wl.name, l, ids, bits)

        _, recs = O.moe_chain(x[todo], n_layers, router_of, lambda l: host_cache.experts_of(wl, l, bits),
                              wl.top_k, bits, eps=EPS, prepare_of=prepare_of)
        for i, t in enumerate(todo):
            _CHAINS[keys[t]] = [tuple(a[i] for a in rec) for rec in recs]
    return [_CHAINS[k] for k in keys]


def _u_from_h(h: np.ndarray) -> np.ndarray:
    h64 = h.astype(np.float64)
    return (h64 / np.sqrt(np.mean(h64 * h64) + EPS)).astype(np.float32)


def walk(wl: mi.Workload, bits: int, x: np.ndarray, ids_g, gates_g, hl_g, h_out, full=(), label=""):
    """Compare every token of a GPU run with its oracle chain (see module
    doc).  ids_g/gates_g [L][T][k], hl_g [L][T][D], h_out [T][D] are the GPU
    outputs.  Returns per-token layers matched and the largest drift seen."""
    L, T = ids_g.shape[0], ids_g.shape[1]
    chains = oracle_chain(wl, bits, x, L)
    routers = [mi.router_host(wl, l) for l in range(L)]
    matched, worst_drift, worst_err, worst_floor = [], 0.0, 0.0, 0.0
    drift_by_layer = np.zeros(L)

    def margin_of(u, w, b, l):
        z = O.router_logits(u[None], w, b if wl.zipf_bias else None)[0]
        top = -np.sort(-z)[:wl.top_k + 1]
        return float(np.min(top[:-1] - top[1:]))

    for t in range(T):
        rec = chains[t]
        n = 0
        for l in range(L):
            u_o, ids_o, gates_o, y_o, h_o = rec[l]
            w, b = routers[l]
            u_g = O.as_f32_activations(x[t:t + 1])[0] if l == 0 else _u_from_h(hl_g[l - 1, t])
            dz = np.abs((u_g.astype(np.float64) - u_o.astype(np.float64)) @ w.astype(np.float64))
            drift = 2.0 * float(dz.max())
            worst_drift = max(worst_drift, drift)
            drift_by_layer[l] = max(drift_by_layer[l], drift)
            if t in full:
                # the premise of the selection: no swap is possible where the
                # oracle's margin exceeds the measured drift
                m = margin_of(u_o, w, b, l)
                assert drift < m, (f"{label} token {t} layer {l}: logit drift {drift:.2e} reaches the oracle "
                                   f"margin {m:.2e}; the selection margin is too small for this drift")
            ig = np.asarray(ids_g[l, t])
            if not np.array_equal(ig, ids_o):
                j = int(np.nonzero(ig != ids_o)[0][0])
                a, c = int(ids_o[j]), int(ig[j])
                z = O.router_logits(u_o[None], w, b if wl.zipf_bias else None)[0]
                margin = z[a] - z[c]
                print(f"{label} token {t}: routing differs at layer {l} rank {j} (oracle {a}, gpu {c}); "
                      f"oracle margin {margin:.3e}, allowed {dz[a] + dz[c]:.3e}")
                assert 0.0 <= margin <= dz[a] + dz[c] + 1e-9, \
                    f"{label} token {t} layer {l}: routing differs beyond the measured drift"
                assert t not in full, f"{label} token {t} was selected for full depth but diverged at layer {l}"
                break
            gg = np.asarray(gates_g[l, t], dtype=np.float64)
            gate_bound = 2.0 * float(dz.max()) * gates_o.astype(np.float64) + 1e-6
            assert np.all(np.abs(gg - gates_o) <= gate_bound), f"{label} token {t} layer {l}: gates differ"
            err = row_rel_err(hl_g[l, t], h_o)
            worst_err = max(worst_err, err)
            worst_floor = max(worst_floor, floored_rel_err(hl_g[l, t], h_o))
            assert err <= TOL, f"{label} token {t} layer {l}: residual differs by {err:.2e}"
            n += 1
        matched.append(n)
        if n == L:
            assert np.array_equal(np.asarray(h_out[t]), np.asarray(hl_g[L - 1, t]))
            assert row_rel_err(h_out[t], rec[L - 1][4]) <= TOL
        if t in full:
            assert n == L, f"{label} token {t}: {n} of {L} layers"
    print(f"{label}: layers matched per token {matched}; residual row error max {worst_err:.2e} "
          f"(floored elementwise {worst_floor:.2e}); logit drift 2max|dz| max {worst_drift:.2e}", flush=True)
    if L > 1:
        print(f"{label}: drift by layer (max over tokens) " +
              " ".join(f"{l}:{drift_by_layer[l]:.1e}" for l in range(0, L, max(1, L // 12))), flush=True)
    return matched, worst_drift

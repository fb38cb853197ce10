"""CPU oracle of the int8-activation ("MMQ-style") expert FFN variant.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the ``cpu_baseline``
leg of ``bench.py``; never by the library or its binding.  It shares no
code with the HIP path.

The pages run the prefill expert matmuls on quantised operands instead of
first expanding the weights to fp16 (bnskd "Strata：把 125B 大模型塞进 12GB 显
卡", section 工程细节, which names llama.cpp's MMQ kernels).  They do not spell
out the activation format.  The plainest reading, and the one taken here:

* Activations are quantised in blocks of 32 consecutive values along the
  reduction axis (the weight block size) to int8 with one fp32 scale per
  block ("Q8 blocks"): amax = max |v|; inv = 127 / amax and d = amax / 127,
  both fp32 divisions; q = round-half-even(v * inv) in fp32, clipped to
  [-127, 127].  A block whose amax is below 2^-112, zero included, is
  stored as q = 0, d = 0: 127 / amax stays finite and d stays a normal
  fp32 number for every other block.
* Each expert matmul is a sum over blocks b of
      d_act[b] * scale_w[b] * (sum over the 32 k of the block of q[k] * level[k])
  where level is the stored weight level (code - 2 for 2-bit).  The integer
  block sums are exact; the oracle scales and adds them in fp64.
* g and u come from x's Q8 blocks; h = silu(g) * u is evaluated in fp64 and
  rounded to fp32, the precision in which its Q8 quantisation is decided;
  the down projection reads h's Q8 blocks.
* The k expert outputs are rounded to fp32 and combined by the exact-weight
  oracle's ``combine`` (gate-weighted, added in slot order in fp32).

Only the 2-bit format is defined for this variant (the pages' prefill tier,
aiproducthub "Strata Skill", section 功能与原则).
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import as_f32_activations, combine

__all__ = ["Q8_BLOCK", "quantize_q8", "dequantize_q8", "weight_levels", "block_dot_q8",
           "gateup_q8", "down_q8", "swiglu_expert_q8", "moe_layer_q8", "moe_ffn_q8_buckets"]

Q8_BLOCK = 32
_TINY = np.float32(2.0 ** -112)


def quantize_q8(v: np.ndarray):
    """Q8 blocks of ``v`` [..., n] (n a multiple of 32), fp32 arithmetic.

    Returns (q int8 [..., n], d fp32 [..., n/32])."""
    v = np.asarray(v, dtype=np.float32)
    blk = v.reshape(v.shape[:-1] + (-1, Q8_BLOCK))
    amax = np.max(np.abs(blk), axis=-1).astype(np.float32)
    live = amax >= _TINY
    safe = np.where(live, amax, np.float32(1.0)).astype(np.float32)
    inv = (np.float32(127.0) / safe).astype(np.float32)
    d = np.where(live, (safe / np.float32(127.0)).astype(np.float32), np.float32(0.0)).astype(np.float32)
    scaled = (blk * inv[..., None]).astype(np.float32)
    q = np.clip(np.rint(scaled), -127, 127)
    q = np.where(live[..., None], q, 0).astype(np.int8)
    return q.reshape(v.shape), d


def dequantize_q8(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """q * d per block, fp64 (exact)."""
    q = np.asarray(q)
    blk = q.reshape(q.shape[:-1] + (-1, Q8_BLOCK)).astype(np.float64)
    return (blk * np.asarray(d, dtype=np.float64)[..., None]).reshape(q.shape)


def weight_levels(qw: np.ndarray, sw: np.ndarray):
    """Stored 2-bit tensor (codes [N][K/32][2], fp16 scale bits [N][K/32]) ->
    (levels int8 [N][K/32][32], scales fp64 [N][K/32]).

    Weight i of a block sits in word i // 16 at bit 2 (i mod 16); level =
    code - 2."""
    qw = np.asarray(qw, dtype=np.uint32)
    assert qw.shape[-1] == 2, "the int8-activation variant covers the 2-bit format"
    lev = np.empty(qw.shape[:-1] + (Q8_BLOCK,), dtype=np.int8)
    for i in range(Q8_BLOCK):
        lev[..., i] = ((qw[..., i // 16] >> np.uint32(2 * (i % 16))) & np.uint32(3)).astype(np.int8) - 2
    s = np.asarray(sw, dtype=np.uint16).view(np.float16).astype(np.float64)
    return lev, s


def block_dot_q8(aq: np.ndarray, ad: np.ndarray, lev: np.ndarray, ws: np.ndarray) -> np.ndarray:
    """out[n, c] = sum_b ad[n, b] * ws[c, b] * sum_i aq[n, b, i] * lev[c, b, i].

    aq int8 [n][K], ad fp32 [n][K/32]; lev int8 [C][K/32][32], ws fp64
    [C][K/32].  The integer block sums are exact (fp64 products of small
    integers); scaling and the sum over blocks run in fp64, blocks in
    ascending order."""
    n = aq.shape[0]
    nb = lev.shape[1]
    a = np.asarray(aq, dtype=np.float64).reshape(n, nb, Q8_BLOCK)
    l64 = lev.astype(np.float64)
    ad64 = np.asarray(ad, dtype=np.float64)
    out = np.zeros((n, lev.shape[0]), dtype=np.float64)
    for b in range(nb):
        isum = a[:, b, :] @ l64[:, b, :].T                   # exact integers
        out += (ad64[:, b:b + 1] * ws[None, :, b]) * isum
    return out


def gateup_q8(xq, xd, gate, up):
    """(g, u) fp64 [n][F] of Q8 activation rows against stored gate/up
    tensors ((codes, scales) each)."""
    lg, sg = weight_levels(*gate)
    lu, su = weight_levels(*up)
    return block_dot_q8(xq, xd, lg, sg), block_dot_q8(xq, xd, lu, su)


def down_q8(hq, hd, down):
    """Down projection fp64 [n][D] of Q8 rows of h against the stored down
    tensor."""
    ld, sd = weight_levels(*down)
    return block_dot_q8(hq, hd, ld, sd)


def swiglu_expert_q8(xq, xd, gate, up, down) -> np.ndarray:
    """One expert on Q8 activation rows: g, u; h = g * sigmoid(g) * u (fp64,
    rounded to fp32); h -> Q8 blocks; out = down(h), rounded to fp32."""
    g, u = gateup_q8(xq, xd, gate, up)
    h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
    hq, hd = quantize_q8(h)
    return down_q8(hq, hd, down).astype(np.float32)


def moe_ffn_q8_buckets(x, gates, k, offsets, pairs, expert_weights, rows=None):
    """Expert FFN of a chunk given its routing, the way the prefill entry
    point receives it: pairs p = t*k + j grouped by expert (offsets, pairs),
    gates [T][k].  ``expert_weights(e)`` -> ((gq, gs), (uq, us), (dq, ds)).
    ``rows``, if given, restricts the result to those tokens (the others are
    left zero), so large chunks can be checked on a sample.

    y[t] = sum_j gates[t, j] * out_{t,j}, added in slot order in fp32."""
    xf = as_f32_activations(x)
    T = xf.shape[0]
    keep = np.ones(T, dtype=bool) if rows is None else np.isin(np.arange(T), rows)
    xq, xd = quantize_q8(xf)
    outs = np.zeros((T, k, xf.shape[1]), dtype=np.float32)
    offsets = np.asarray(offsets, dtype=np.int64)
    pairs = np.asarray(pairs, dtype=np.int64)
    for e in range(len(offsets) - 1):
        p = pairs[offsets[e]:offsets[e + 1]]
        p = p[keep[p // k]]
        if p.size == 0:
            continue
        t = p // k
        gw, uw, dw = expert_weights(e)
        outs[t, p % k] = swiglu_expert_q8(xq[t], xd[t], gw, uw, dw)
    return combine(np.asarray(gates, dtype=np.float32), outs)


def moe_layer_q8(xf, ids, gates, expert_weights):
    """Int8-activation expert FFN of a layer from its routing (ids, gates
    [T][k]): the per-token form of ``moe_ffn_q8_buckets``."""
    xf = as_f32_activations(xf)
    T, k = ids.shape
    xq, xd = quantize_q8(xf)
    outs = np.zeros((T, k, xf.shape[1]), dtype=np.float32)
    for e in np.unique(ids):
        t, j = np.nonzero(ids == e)
        gw, uw, dw = expert_weights(int(e))
        outs[t, j] = swiglu_expert_q8(xq[t], xd[t], gw, uw, dw)
    return combine(np.asarray(gates, dtype=np.float32), outs)

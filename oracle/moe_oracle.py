"""CPU oracle of the routed mixture-of-experts FFN.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library or its
binding.  It shares no code with the HIP path.

What it computes (the pages' problem statement, made precise):

* Each MoE layer holds 512 experts and each token is sent to 10 of them
  (aiproducthub "Strata Skill", section 介绍: 24,576 experts, 10 per token;
  yudady notes "Strata — 8~12GB 显存跑 125B", section 5 table: 512 experts per
  layer; bnskd "Strata：把 125B 大模型塞进 12GB 显卡", section 投机解码: 48
  layers).  Routing is top-k of a linear router with softmax gates
  renormalised over the chosen k, ties toward the lower expert id.
* Every expert is a SwiGLU FFN whose weights are stored in 2- or 3-bit
  block quantisation (aiproducthub, section 功能与原则: Q2_0 experts); the
  oracle dequantises to fp32 and multiplies in fp32.
* The layer output is the gate-weighted sum of the k expert outputs.
* Chained workloads keep an fp32 residual stream with an RMSNorm between
  layers.

Each function states the plain definition it evaluates.  Precision choices
where the pages are silent: router logits accumulate in fp64 in ascending d
order and the bias is added last; gates are computed in fp64 and rounded to
fp32; expert math is fp32 (dequantise, then matmul); the combine adds the k
weighted outputs in slot order in fp32; RMSNorm takes the mean square in
fp64 with eps = 1e-6 and gamma = 1.

Parity pins live in ``tests/test_oracle_pins.py``.  Nothing here is checked
against a number printed on the pages: the pages print no kernel-level value,
so agreement with the pages themselves is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "unpack_codes", "dequantize", "as_f32_activations", "router_logits",
    "select_experts", "gate_weights", "route", "bucket_pairs",
    "swiglu_expert", "combine", "moe_layer", "rmsnorm", "moe_chain",
]


# ----------------------------------------------------------------- formats

def unpack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Codes of every weight of packed blocks ``q`` [..., words] -> [..., 32].

    2-bit: weight i is in word i // 16 at bit 2 (i mod 16).  3-bit: the three
    words form a little-endian 96-bit string, weight i at bit 3 i."""
    q = np.asarray(q, dtype=np.uint32).astype(np.uint64)
    out = np.empty(q.shape[:-1] + (32,), dtype=np.uint8)
    if bits == 2:
        assert q.shape[-1] == 2
        for i in range(32):
            out[..., i] = (q[..., i // 16] >> np.uint64(2 * (i % 16))) & np.uint64(3)
    elif bits == 3:
        assert q.shape[-1] == 3
        s96 = q[..., 0] | (q[..., 1] << np.uint64(32))          # low 64 bits
        for i in range(32):
            lo = 3 * i
            if lo + 3 <= 64:
                v = (s96 >> np.uint64(lo)) & np.uint64(7)
            else:
                # bits above 63 live in word 2 (bit 64 + m is word-2 bit m)
                v = np.zeros_like(s96)
                for b in range(3):
                    p = lo + b
                    bit = (s96 >> np.uint64(p)) & np.uint64(1) if p < 64 else \
                        (q[..., 2] >> np.uint64(p - 64)) & np.uint64(1)
                    v |= bit << np.uint64(b)
            out[..., i] = v
    else:
        raise ValueError("bits must be 2 or 3")
    return out


def dequantize(q: np.ndarray, s: np.ndarray, bits: int) -> np.ndarray:
    """Stored tensor (codes [N][K/32][words], fp16 scale bits [N][K/32]) ->
    fp32 matrix [N][K] in storage orientation (row n = output n).

    Weight = (code - 2**(bits-1)) * scale, exact in fp32."""
    codes = unpack_codes(q, bits).astype(np.int32)
    levels = (codes - (1 << (bits - 1))).astype(np.float32)
    scale = np.asarray(s, dtype=np.uint16).view(np.float16).astype(np.float32)
    w = levels * scale[..., None]
    return w.reshape(w.shape[0], -1)


def as_f32_activations(x: np.ndarray) -> np.ndarray:
    """fp32 activations; uint16 input is taken as bf16 bit patterns."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return x.astype(np.float32)


# ----------------------------------------------------------------- routing

def router_logits(x: np.ndarray, w: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """z[t, e] = sum_d x[t, d] * w[d, e] + bias[e] in fp64.

    Every product of an fp32 (or bf16) activation and an fp32 weight is exact
    in fp64; the sum runs over d in ascending order, the bias is added last."""
    x64 = as_f32_activations(x).astype(np.float64)
    w64 = np.asarray(w, dtype=np.float32).astype(np.float64)
    t, d = x64.shape
    z = np.zeros((t, w64.shape[1]), dtype=np.float64)
    for i in range(d):
        z += x64[:, i:i + 1] * w64[i:i + 1, :]
    if bias is not None:
        z += np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return z


def select_experts(z: np.ndarray, k: int) -> np.ndarray:
    """The k experts with the largest logits, in rank order; equal logits go
    to the lower expert id (-0.0 and +0.0 are equal)."""
    z = np.asarray(z, dtype=np.float64) + 0.0
    t, e = z.shape
    ids = np.empty((t, k), dtype=np.int32)
    eid = np.arange(e)
    for r in range(t):
        order = np.lexsort((eid, -z[r]))       # primary key -z, then id
        ids[r] = order[:k]
    return ids


def gate_weights(z: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax of the selected logits (equal to softmax over all experts
    renormalised over the chosen k), computed in fp64, rounded to fp32."""
    sel = np.take_along_axis(np.asarray(z, dtype=np.float64), ids.astype(np.int64), axis=1)
    p = np.exp(sel - sel[:, :1])
    return (p / p.sum(axis=1, keepdims=True)).astype(np.float32)


def route(x, w, bias, k):
    """(ids int32 [T][k], gates fp32 [T][k], logits fp64 [T][E])."""
    z = router_logits(x, w, bias)
    ids = select_experts(z, k)
    return ids, gate_weights(z, ids), z


def bucket_pairs(ids: np.ndarray, n_experts: int):
    """Group the (token, slot) pairs p = t*k + j by expert.

    offsets[e] is the exclusive prefix sum of the per-expert counts
    (offsets[E] = T*k); pairs lists the pair ids of expert 0, then expert 1,
    ..., each bucket in ascending pair id (a stable counting sort)."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    pairs = np.argsort(flat, kind="stable")
    return offsets.astype(np.int32), pairs.astype(np.int32)


# ----------------------------------------------------------------- experts

def swiglu_expert(xf: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """SwiGLU expert on fp32 rows ``xf`` [n][D] with dequantised weights in
    storage orientation (wg, wu: [F][D]; wd: [D][F]):
    g = x Wg, u = x Wu, h = g * sigmoid(g) * u, out = h Wd, all fp32."""
    xf = np.asarray(xf, dtype=np.float32)
    g = xf @ wg.T
    u = xf @ wu.T
    h = g * (np.float32(1.0) / (np.float32(1.0) + np.exp(-g))) * u
    return (h @ wd.T).astype(np.float32)


def combine(gates: np.ndarray, outs: np.ndarray) -> np.ndarray:
    """y[t] = sum_j gates[t, j] * outs[t, j] added in slot order j = 0..k-1
    in fp32.  outs: [T][k][D]."""
    t, k, d = outs.shape
    y = np.zeros((t, d), dtype=np.float32)
    for j in range(k):
        y = y + gates[:, j:j + 1] * outs[:, j, :]
    return y


def moe_layer(x, router_w, router_b, k, expert_weights, bits, prepare=None):
    """One routed MoE FFN layer.

    ``expert_weights(e)`` returns the stored ((gate_q, gate_s), (up_q, up_s),
    (down_q, down_s)) of expert e.  ``prepare``, if given, is called once with
    the distinct selected expert ids before any expert is requested (a hook
    for fetching them in bulk; it takes no part in the arithmetic).
    Returns (ids, gates, y fp32 [T][D])."""
    ids, gates, _ = route(x, router_w, router_b, k)
    if prepare is not None:
        prepare(np.unique(ids))
    xf = as_f32_activations(x)
    t = xf.shape[0]
    outs = np.zeros((t, k, xf.shape[1]), dtype=np.float32)
    for e in np.unique(ids):
        rows, slots = np.nonzero(ids == e)
        (gq, gs), (uq, us), (dq, ds) = expert_weights(int(e))
        o = swiglu_expert(xf[rows], dequantize(gq, gs, bits), dequantize(uq, us, bits),
                          dequantize(dq, ds, bits))
        outs[rows, slots] = o
    return ids, gates, combine(gates, outs)


def rmsnorm(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """u = h / sqrt(mean(h^2) + eps), mean square in fp64, gamma = 1,
    result rounded to fp32."""
    h64 = np.asarray(h, dtype=np.float32).astype(np.float64)
    r = np.sqrt(np.mean(h64 * h64, axis=-1, keepdims=True) + eps)
    return (h64 / r).astype(np.float32)


def moe_chain(x, n_layers, router_of, experts_of, k, bits, eps=1e-6, prepare_of=None):
    """Residual chain of MoE layers: h_0 = x; u_l = h_l for l = 0, else
    RMSNorm(h_l); h_{l+1} = h_l + MoE_l(u_l) (fp32 add).

    ``router_of(l)`` -> (w, b); ``experts_of(l)`` -> callable e -> weights;
    ``prepare_of(l)``, if given, -> the ``prepare`` hook of ``moe_layer``.
    Returns (h_L, records) with one record (u, ids, gates, y, h_{l+1}) per
    layer."""
    h = as_f32_activations(x)
    recs = []
    for l in range(n_layers):
        u = h if l == 0 else rmsnorm(h, eps)
        w, b = router_of(l)
        ids, gates, y = moe_layer(u, w, b, k, experts_of(l), bits,
                                  prepare=None if prepare_of is None else prepare_of(l))
        h = (h + y).astype(np.float32)
        recs.append((u, ids, gates, y, h))
    return h, recs

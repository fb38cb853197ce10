"""Pins of the CPU oracle to facts that do not come from the oracle itself.

The pages print no worked example or kernel-level number, so each pin is a
hand-derived value, a closed form, an exact (rational) evaluation, a brute
force on tiny inputs, or an invariant of the definition.  ``PINS`` run on the
real oracle; ``test_planted_mistakes_are_caught`` plants plausible mistakes
in the oracle (on the CPU) and checks that some pin fails for each.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import moe_inputs as mi
import oracle.moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "blocks.txt")


def _parse_golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        bits, words, scale, vals = [p.strip() for p in line.split("|")]
        q = np.array([int(w, 16) for w in words.split()], dtype=np.uint32)
        s = np.array([int(scale, 16)], dtype=np.uint16)
        out = []
        for tok in vals.split():
            v, n = tok.rsplit("*", 1)
            out += [float(v)] * int(n)
        assert len(out) == 32
        rows.append((int(bits), q, s, np.array(out, dtype=np.float64)))
    return rows


def _rng(seed=0):
    return np.random.default_rng(seed)


def _tiny_expert(rng, d, f, bits):
    """Random stored expert (gate, up, down) of shape d_model=d, d_ff=f."""
    out = []
    for n, k in ((f, d), (f, d), (d, f)):
        v = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
        lev, s = mi.quantize_blocks(v, bits)
        out.append((mi.pack_codes(lev, bits), s, lev))
    return out


# ----------------------------------------------------------------- pins

def pin_golden_blocks(O):
    for bits, q, s, want in _parse_golden():
        got = O.dequantize(q[None, None, :], s[None, :], bits).reshape(-1).astype(np.float64)
        assert np.array_equal(got, want), (bits, q, got, want)


def pin_pack_unpack_bijection(O):
    rng = _rng(1)
    for bits in (2, 3):
        words = rng.integers(0, 2**32, size=(257, 2 if bits == 2 else 3), dtype=np.uint64).astype(np.uint32)
        codes = O.unpack_codes(words, bits)
        assert codes.max() < (1 << bits)
        lev = codes.astype(np.int64) - (1 << (bits - 1))
        assert np.array_equal(mi.pack_codes(lev, bits), words)


def pin_quantize_roundtrip(O):
    """Blocks made of levels * s (fp16 s, at least one lowest level) survive
    quantise -> dequantise exactly."""
    rng = _rng(2)
    for bits in (2, 3):
        lo, hi = (-2, 1) if bits == 2 else (-4, 3)
        lev = rng.integers(lo, hi + 1, size=(64, 4, 32))
        lev[:, :, 5] = lo
        s = rng.uniform(1e-3, 10.0, size=(64, 4)).astype(np.float16)
        w = (lev.astype(np.float32) * s.astype(np.float32)[..., None]).reshape(64, 128)
        lq, sq = mi.quantize_blocks(w, bits)
        assert np.array_equal(sq, s.view(np.uint16))
        assert np.array_equal(lq, lev)
        back = O.dequantize(mi.pack_codes(lq, bits), sq, bits)
        assert np.array_equal(back, w)


def pin_quantize_error_bound(O):
    rng = _rng(3)
    for bits in (2, 3):
        hi = 1 if bits == 2 else 3
        w = (0.02 * rng.standard_normal((96, 256))).astype(np.float32)
        lev, s = mi.quantize_blocks(w, bits)
        back = O.dequantize(mi.pack_codes(lev, bits), s, bits).reshape(96, 8, 32)
        sf = s.view(np.float16).astype(np.float64)[..., None]
        wb = w.reshape(96, 8, 32).astype(np.float64)
        err = np.abs(wb - back)
        clip = np.maximum(wb - hi * sf, 0.0)
        assert np.all(err <= np.maximum(sf / 2, clip) * (1 + 1e-6) + 1e-12)


def pin_logits_exact(O):
    """fp64 logits agree with exact rational arithmetic within the fp64
    summation bound."""
    rng = _rng(4)
    t, d, e = 3, 40, 7
    x = rng.standard_normal((t, d)).astype(np.float32)
    w = (0.02 * rng.standard_normal((d, e))).astype(np.float32)
    b = rng.standard_normal(e).astype(np.float32)
    z = O.router_logits(x, w, b)
    for i in range(t):
        for j in range(e):
            exact = sum(Fraction(float(x[i, q])) * Fraction(float(w[q, j])) for q in range(d)) + Fraction(float(b[j]))
            mag = sum(abs(float(x[i, q]) * float(w[q, j])) for q in range(d)) + abs(float(b[j]))
            assert abs(Fraction(z[i, j]) - exact) <= (d + 2) * 2.0**-52 * mag


def pin_logits_bf16_input(O):
    """uint16 activations are bf16 bit patterns: 0x3f80 is 1.0, 0xc000 -2."""
    x = np.array([[0x3F80, 0xC000]], dtype=np.uint16)
    w = np.array([[1.0, 0.5], [0.25, 3.0]], dtype=np.float32)
    z = O.router_logits(x, w, None)
    assert z.tolist() == [[1.0 - 0.5, 0.5 - 6.0]]


def _brute_topk(z, k):
    t, e = z.shape
    ids = np.empty((t, k), dtype=np.int64)
    for r in range(t):
        rank = [sum(1 for q in range(e) if z[r, q] > z[r, p] or (z[r, q] == z[r, p] and q < p)) for p in range(e)]
        for p in range(e):
            if rank[p] < k:
                ids[r, rank[p]] = p
    return ids


def pin_topk_bruteforce(O):
    rng = _rng(5)
    for e in (1, 5, 16, 64):
        z = rng.standard_normal((4, e))
        z[:, e // 2] = z[:, 0]                  # exact ties
        z = np.round(z, 1)                      # more ties
        for k in range(1, e + 1):
            assert np.array_equal(O.select_experts(z, k), _brute_topk(z, k)), (e, k)


def pin_topk_ties_and_zero(O):
    ids = O.select_experts(np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, 2.0]]), 2)
    assert ids.tolist() == [[0, 1], [2, 0]]
    # duplicated router columns give exactly equal logits: lower id wins
    rng = _rng(6)
    x = rng.standard_normal((5, 32)).astype(np.float32)
    w = (0.02 * rng.standard_normal((32, 8))).astype(np.float32)
    w[:, 6] = w[:, 2]
    w[:, 7] = w[:, 2]
    z = O.router_logits(x, w, None)
    ids = O.select_experts(z, 8)
    for r in range(5):
        pos = [list(ids[r]).index(c) for c in (2, 6, 7)]
        assert pos == sorted(pos) and pos[1] == pos[0] + 1 and pos[2] == pos[0] + 2
    # all-equal logits: ids 0..k-1, gates 1/k
    ids, g, _ = O.route(x, np.zeros((32, 8), np.float32), np.zeros(8, np.float32), 3)
    assert np.all(ids == np.arange(3)) and np.allclose(g, 1 / 3, rtol=0, atol=2**-24)


def pin_gate_invariants(O):
    from scipy.special import softmax
    rng = _rng(7)
    z = rng.standard_normal((6, 20)) * 3
    for k in (1, 2, 10, 20):
        ids = O.select_experts(z, k)
        g = O.gate_weights(z, ids).astype(np.float64)
        assert np.all(np.abs(g.sum(1) - 1.0) <= k * 2.0**-24)
        assert np.all(np.diff(g, axis=1) <= 0)
        if k == 1:
            assert np.all(g == 1.0)
    ids = O.select_experts(z, 20)
    g = O.gate_weights(z, ids).astype(np.float64)
    ref = np.take_along_axis(softmax(z, axis=1), ids.astype(np.int64), axis=1)
    assert np.allclose(g, ref, rtol=2**-23, atol=0)
    zz = np.array([[0.3, -1.2, 0.0]])
    ids = O.select_experts(zz, 2)
    g = O.gate_weights(zz, ids)
    assert ids.tolist() == [[0, 2]]
    assert abs(g[0, 0] - 1 / (1 + math.exp(0.0 - 0.3))) <= 2**-24


def pin_buckets(O):
    rng = _rng(8)
    t, k, e = 37, 3, 11
    ids = np.stack([rng.permutation(e)[:k] for _ in range(t)]).astype(np.int32)
    off, pairs = O.bucket_pairs(ids, e)
    flat = ids.reshape(-1)
    want = [p for ex in range(e) for p in range(t * k) if flat[p] == ex]
    assert pairs.tolist() == want
    assert off[0] == 0 and off[-1] == t * k
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=e))
    assert sorted(pairs.tolist()) == list(range(t * k))


def _hand_expert():
    """d_model = d_ff = 32: one block per row.  Gate/up rows read only input
    k = 3; down levels are a fixed asymmetric pattern."""
    lg = np.array([1, -1, -2, 0] * 8)
    lu = np.array([-2, 1, 1, -1, 0, 1, -2, 1] * 4)
    g_lev = np.zeros((32, 1, 32), dtype=np.int64)
    u_lev = np.zeros((32, 1, 32), dtype=np.int64)
    g_lev[:, 0, 3] = lg
    u_lev[:, 0, 3] = lu
    d_lev = ((np.arange(32)[:, None] * 7 + np.arange(32)[None, :] * 3) % 4 - 2).reshape(32, 1, 32)
    sg = np.full((32, 1), 0x3800, np.uint16)      # 0.5
    su = np.full((32, 1), 0x3400, np.uint16)      # 0.25
    sd = np.full((32, 1), 0x3C00, np.uint16)      # 1.0
    stored = ((mi.pack_codes(g_lev, 2), sg), (mi.pack_codes(u_lev, 2), su), (mi.pack_codes(d_lev, 2), sd))
    gv = lg * 0.5
    uv = lu * 0.25
    h = [gv[f] / (1 + math.exp(-gv[f])) * uv[f] for f in range(32)]
    y = [sum(h[f] * d_lev[d, 0, f] for f in range(32)) for d in range(32)]
    return stored, np.array(y)


def pin_expert_hand(O):
    stored, y_want = _hand_expert()
    x = np.zeros((1, 32), np.float32)
    x[0, 3] = 1.0
    (gq, gs), (uq, us), (dq, ds) = stored
    o = O.swiglu_expert(x, O.dequantize(gq, gs, 2), O.dequantize(uq, us, 2), O.dequantize(dq, ds, 2))
    assert np.allclose(o[0], y_want, rtol=1e-6, atol=1e-7)
    # through the layer: one expert, k = 1, gate 1.0
    ids, g, y = O.moe_layer(x, np.zeros((32, 1), np.float32), None, 1, lambda e: stored, 2)
    assert ids.tolist() == [[0]] and g.tolist() == [[1.0]]
    assert np.allclose(y[0], y_want, rtol=1e-6, atol=1e-7)
    # g = 0 everywhere (x orthogonal to the gate rows): output exactly 0
    x0 = np.zeros((1, 32), np.float32)
    x0[0, 7] = 1.0
    _, _, y0 = O.moe_layer(x0, np.zeros((32, 1), np.float32), None, 1, lambda e: stored, 2)
    assert np.all(y0 == 0)


def pin_dense_fp64(O):
    """E = 1, k = 1 is a dense SwiGLU MLP; compare with an fp64 evaluation
    built from the quantiser's own levels (not the oracle's unpacking)."""
    rng = _rng(9)
    for bits in (2, 3):
        d, f = 96, 64
        ex = _tiny_expert(rng, d, f, bits)
        x = rng.standard_normal((5, d)).astype(np.float32)
        stored = tuple((q, s) for q, s, _ in ex)
        _, _, y = O.moe_layer(x, np.zeros((d, 1), np.float32), None, 1, lambda e: stored, bits)
        w64 = [(lev.astype(np.float64) * s.view(np.float16).astype(np.float64)[..., None]).reshape(lev.shape[0], -1)
               for _, s, lev in ex]
        x64 = x.astype(np.float64)
        g = np.einsum("td,fd->tf", x64, w64[0])
        u = np.einsum("td,fd->tf", x64, w64[1])
        h = g / (1 + np.exp(-g)) * u
        ref = np.einsum("tf,df->td", h, w64[2])
        assert np.max(np.abs(y - ref)) <= 1e-5 * np.max(np.abs(ref))


def pin_combine_and_slots(O):
    y = O.combine(np.array([[0.25, 0.75]], np.float32), np.array([[[1, 2], [3, 4]]], np.float32))
    assert y.tolist() == [[2.5, 3.5]]
    # two experts, each token uses both: y = g0 * o(e0) + g1 * o(e1)
    rng = _rng(10)
    d, f = 64, 32
    exps = [_tiny_expert(rng, d, f, 2) for _ in range(2)]
    stored = [tuple((q, s) for q, s, _ in ex) for ex in exps]
    x = rng.standard_normal((4, d)).astype(np.float32)
    wr = (0.3 * rng.standard_normal((d, 2))).astype(np.float32)
    ids, g, y = O.moe_layer(x, wr, None, 2, lambda e: stored[e], 2)
    deq = [[O.dequantize(q, s, 2) for q, s in st] for st in stored]
    for t in range(4):
        o = [O.swiglu_expert(x[t:t + 1], *deq[ids[t, j]])[0] for j in range(2)]
        want = np.float32(0) + g[t, 0] * o[0] + g[t, 1] * o[1]
        # rows batched through BLAS may round differently from one row alone
        assert np.allclose(y[t], want, rtol=1e-5, atol=1e-6 * np.abs(want).max())


def pin_rmsnorm(O):
    h = np.array([[3e-3, 4e-3]], np.float32)
    u = O.rmsnorm(h, 1e-6)
    want = np.array([3e-3, 4e-3]) / math.sqrt((9e-6 + 16e-6) / 2 + 1e-6)
    assert np.allclose(u[0], want, rtol=1e-6)
    rng = _rng(11)
    h = rng.standard_normal((7, 300)).astype(np.float32) * np.arange(1, 8)[:, None]
    u = O.rmsnorm(h).astype(np.float64)
    ms = np.mean(h.astype(np.float64) ** 2, axis=1)
    assert np.allclose(np.mean(u * u, axis=1), 1 / (1 + 1e-6 / ms), rtol=1e-6)


def pin_chain(O):
    rng = _rng(12)
    d, f, e = 64, 32, 3
    exps = [tuple((q, s) for q, s, _ in _tiny_expert(rng, d, f, 2)) for _ in range(e)]
    wr = [(0.3 * rng.standard_normal((d, e))).astype(np.float32) for _ in range(2)]
    x = rng.standard_normal((3, d)).astype(np.float32)
    h1, recs = O.moe_chain(x, 1, lambda l: (wr[l], None), lambda l: (lambda i: exps[i]), 2, 2)
    _, _, y = O.moe_layer(x, wr[0], None, 2, lambda i: exps[i], 2)
    assert np.array_equal(h1, x + y)
    # two layers: the second layer reads the normalised residual and its
    # output is added to the residual (not to its own input)
    h2, recs = O.moe_chain(x, 2, lambda l: (wr[l], None), lambda l: (lambda i: exps[i]), 2, 2)
    u1 = O.rmsnorm(h1)
    _, _, y1 = O.moe_layer(u1, wr[1], None, 2, lambda i: exps[i], 2)
    assert np.array_equal(recs[0][4], h1) and np.array_equal(recs[1][0], u1)
    assert np.array_equal(h2, (h1 + y1).astype(np.float32)) and np.array_equal(recs[1][4], h2)
    m = np.mean(recs[1][0].astype(np.float64) ** 2, axis=1)
    assert np.allclose(m, 1.0, rtol=1e-4)


def pin_chain_hand(O):
    """Two layers of the hand-built expert (E = 1, k = 1, gate 1) on a one-hot
    token, evaluated in closed form with Python floats: layer 1 sees the
    RMS-normalised residual h1 = x + y0, and h2 = h1 + y1."""
    stored, y0 = _hand_expert()
    lg = np.array([1, -1, -2, 0] * 8) * 0.5
    lu = np.array([-2, 1, 1, -1, 0, 1, -2, 1] * 4) * 0.25
    d_lev = (np.arange(32)[:, None] * 7 + np.arange(32)[None, :] * 3) % 4 - 2
    x = np.zeros((1, 32), np.float32)
    x[0, 3] = 1.0
    h1 = [float(x[0, i]) + float(y0[i]) for i in range(32)]
    rms = math.sqrt(sum(v * v for v in h1) / 32 + 1e-6)
    a = h1[3] / rms                                  # the only input the gate/up rows read
    h = [(a * lg[j]) / (1 + math.exp(-(a * lg[j]))) * (a * lu[j]) for j in range(32)]
    h2 = [h1[i] + sum(h[j] * d_lev[i, j] for j in range(32)) for i in range(32)]
    got, recs = O.moe_chain(x, 2, lambda l: (np.zeros((32, 1), np.float32), None), lambda l: (lambda e: stored), 1, 2)
    assert np.allclose(recs[0][4][0], h1, rtol=1e-6, atol=1e-6)
    assert np.allclose(got[0], h2, rtol=1e-5, atol=1e-5 * max(abs(v) for v in h2))


def pin_token_independence(O):
    rng = _rng(13)
    d, f, e = 64, 32, 4
    exps = [tuple((q, s) for q, s, _ in _tiny_expert(rng, d, f, 3)) for _ in range(e)]
    wr = (0.3 * rng.standard_normal((d, e))).astype(np.float32)
    x = rng.standard_normal((5, d)).astype(np.float32)
    ids, g, y = O.moe_layer(x, wr, None, 2, lambda i: exps[i], 3)
    for t in range(5):
        i1, g1, y1 = O.moe_layer(x[t:t + 1], wr, None, 2, lambda i: exps[i], 3)
        assert np.array_equal(i1[0], ids[t]) and np.array_equal(g1[0], g[t])
        assert np.allclose(y1[0], y[t], rtol=1e-6, atol=1e-7)


PINS = [pin_golden_blocks, pin_pack_unpack_bijection, pin_quantize_roundtrip, pin_quantize_error_bound,
        pin_logits_exact, pin_logits_bf16_input, pin_topk_bruteforce, pin_topk_ties_and_zero,
        pin_gate_invariants, pin_buckets, pin_expert_hand, pin_dense_fp64, pin_combine_and_slots,
        pin_rmsnorm, pin_chain, pin_chain_hand, pin_token_independence]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(O)


# ------------------------------------------------------ planted mistakes

def _mut_unpack2_reversed(orig):
    def f(q, bits):
        c = orig(q, bits)
        return c[..., ::-1].copy() if bits == 2 else c
    return "unpack_codes", f


def _mut_unpack3_straddle(orig):
    def f(q, bits):
        c = orig(q, bits)
        if bits == 3:
            c = c.copy()
            c[..., 10] = (np.asarray(q)[..., 0] >> np.uint32(30)) & np.uint32(3)
        return c
    return "unpack_codes", f


def _mut_dequant_offset(orig):
    def f(q, s, bits):
        # level = code - (bias - 1): every weight moves up by one scale step
        sc = np.asarray(s, np.uint16).view(np.float16).astype(np.float32)
        return orig(q, s, bits) + np.repeat(sc, 32, axis=-1).reshape(sc.shape[0], -1)
    return "dequantize", f


def _mut_logits_no_bias(orig):
    return "router_logits", lambda x, w, b: orig(x, w, None)


def _mut_logits_fp32(orig):
    def f(x, w, b):
        z = O.as_f32_activations(x) @ np.asarray(w, np.float32)
        if b is not None:
            z = z + b
        return z.astype(np.float64)
    return "router_logits", f


def _mut_topk_high_id(orig):
    def f(z, k):
        z = np.asarray(z, np.float64)
        e = z.shape[1]
        flipped = orig(z[:, ::-1], k)
        return (e - 1 - flipped).astype(np.int32)
    return "select_experts", f


def _mut_gates_all_experts(orig):
    def f(z, ids):
        z = np.asarray(z, np.float64)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        return np.take_along_axis(p, ids.astype(np.int64), axis=1).astype(np.float32)
    return "gate_weights", f


def _mut_buckets_descending(orig):
    def f(ids, e):
        off, pairs = orig(ids, e)
        pairs = pairs.copy()
        for i in range(e):
            pairs[off[i]:off[i + 1]] = pairs[off[i]:off[i + 1]][::-1]
        return off, pairs
    return "bucket_pairs", f


def _mut_swiglu_swapped(orig):
    return "swiglu_expert", lambda x, wg, wu, wd: orig(x, wu, wg, wd)


def _mut_combine_unweighted(orig):
    return "combine", lambda g, o: orig(np.ones_like(g), o)


def _mut_rmsnorm_no_eps(orig):
    return "rmsnorm", lambda h, eps=1e-6: orig(h, 0.0)


def _mut_combine_slot_shift(orig):
    return "combine", lambda g, o: orig(np.roll(g, 1, axis=1), o)


def _chain_variant(update, norm_first=False, norm_rest=True):
    """A moe_chain built from the oracle's own layer and norm but composed
    wrongly: ``update(h, u, y)`` forms the next residual."""
    def chain(x, n_layers, router_of, experts_of, k, bits, eps=1e-6, prepare_of=None):
        h = O.as_f32_activations(x)
        recs = []
        for l in range(n_layers):
            u = O.rmsnorm(h, eps) if (norm_first if l == 0 else norm_rest) else h
            w, b = router_of(l)
            ids, gates, y = O.moe_layer(u, w, b, k, experts_of(l), bits)
            h = update(h, u, y).astype(np.float32)
            recs.append((u, ids, gates, y, h))
        return h, recs
    return chain


def _mut_chain_residual_on_u(orig):
    return "moe_chain", _chain_variant(lambda h, u, y: u + y)


def _mut_chain_norm_first_layer(orig):
    return "moe_chain", _chain_variant(lambda h, u, y: h + y, norm_first=True)


def _mut_chain_no_norm(orig):
    return "moe_chain", _chain_variant(lambda h, u, y: h + y, norm_rest=False)


MUTATIONS = [_mut_chain_residual_on_u, _mut_chain_norm_first_layer, _mut_chain_no_norm, _mut_unpack2_reversed, _mut_unpack3_straddle, _mut_dequant_offset, _mut_logits_no_bias,
             _mut_logits_fp32, _mut_topk_high_id, _mut_gates_all_experts, _mut_buckets_descending,
             _mut_swiglu_swapped, _mut_combine_unweighted, _mut_rmsnorm_no_eps, _mut_combine_slot_shift]


@pytest.mark.parametrize("mut", MUTATIONS, ids=[m.__name__ for m in MUTATIONS])
def test_planted_mistakes_are_caught(mut, monkeypatch):
    name, bad = mut(getattr(O, name_of(mut)))
    monkeypatch.setattr(O, name, bad)
    failed = []
    for pin in PINS:
        try:
            pin(O)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"planted mistake in {name} went unnoticed"


def name_of(mut):
    return mut(lambda *a, **k: None)[0]

"""Pins of the int8-activation oracle variant to facts outside the oracle.

The pages leave the activation format of their quantised prefill matmuls
open (bnskd "Strata：把 125B 大模型塞进 12GB 显卡", section 工程细节); the
reading pinned here is Q8 blocks of 32 with an fp32 scale.  Each pin is a
hand-derived value (``tests/golden/q8_blocks.txt``), an exact rational
evaluation, a special case that reduces to a plain fp64 matmul, a grid
property, or a derived error bound against the exact-weight oracle.
``test_planted_mistakes_are_caught`` plants plausible mistakes in the
variant (on the CPU) and checks that some pin fails for each.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import moe_inputs as mi
import oracle.moe_oracle as O
import oracle.moe_oracle_q8 as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q8_blocks.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        e, ns, qs = [p.strip() for p in line.split("|")]
        n = [Fraction(v) for v in ns.split()]
        q = np.array([int(v) for v in qs.split()], dtype=np.int8)
        assert len(n) == 32 and q.size == 32
        x = np.array([float(v * Fraction(2) ** int(e)) for v in n], dtype=np.float32)
        assert all(Fraction(float(a)) == v * Fraction(2) ** int(e) for a, v in zip(x, n))   # exact inputs
        rows.append((x, q))
    return rows


def _nearest_f32(r: Fraction) -> np.float32:
    """The fp32 value nearest to the rational r (no tie occurs in the pins)."""
    f = np.float32(float(r))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: abs(Fraction(float(c)) - r))


def _expert(rng, d, f):
    out = []
    for n, k in ((f, d), (f, d), (d, f)):
        v = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
        lev, s = mi.quantize_blocks(v, 2)
        out.append((mi.pack_codes(lev, 2), s))
    return tuple(out)


def _dense64(q, s):
    """fp64 [N][K] of a stored 2-bit tensor, through the exact-weight oracle's
    (separately pinned) dequantiser."""
    return O.dequantize(q, s, 2).astype(np.float64)


# ----------------------------------------------------------------- pins

def pin_q8_golden(Q):
    for x, want in _golden():
        q, d = Q.quantize_q8(x[None, :])
        assert np.array_equal(q[0], want), (x, q[0], want)
        amax = max(abs(Fraction(float(v))) for v in x)
        if amax < Fraction(2) ** -112:
            assert d[0, 0] == 0.0
        else:
            assert d[0, 0] == _nearest_f32(amax / 127), (d[0, 0], float(amax / 127))


def pin_q8_rational(Q):
    """Random blocks against exact rational rounding: q = round(x * 127 / amax)
    wherever the fp32 product cannot sit on the other side of a half."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((40, 64)) * np.exp(rng.uniform(-8, 8, size=(40, 1)))).astype(np.float32)
    q, d = Q.quantize_q8(x)
    checked = 0
    for r in range(x.shape[0]):
        for b in range(2):
            blk = x[r, 32 * b:32 * b + 32]
            amax = max(abs(Fraction(float(v))) for v in blk)
            assert d[r, b] == _nearest_f32(amax / 127)
            for i, v in enumerate(blk):
                exact = Fraction(float(v)) * 127 / amax
                frac = exact - (exact.numerator // exact.denominator)
                if abs(frac - Fraction(1, 2)) < Fraction(1, 2 ** 14):
                    continue                                    # too close to a tie to decide exactly
                want = round(exact)
                assert q[r, 32 * b + i] == want, (v, exact, q[r, 32 * b + i])
                checked += 1
    assert checked > 2500


def pin_q8_invariants(Q):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((50, 96)).astype(np.float32)
    q, d = Q.quantize_q8(x)
    qn, dn = Q.quantize_q8(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d)           # odd symmetry, ties included
    blk = x.reshape(50, 3, 32)
    qb = q.reshape(50, 3, 32).astype(np.int32)
    j = np.argmax(np.abs(blk), axis=-1)
    top = np.take_along_axis(qb, j[..., None], axis=-1)[..., 0]
    assert np.array_equal(np.abs(top), np.full_like(top, 127))       # the largest value maps to +-127
    err = np.abs(Q.dequantize_q8(q, d) - x.astype(np.float64)).reshape(50, 3, 32)
    assert np.all(err <= d[..., None].astype(np.float64) * (0.5 + 1e-6))   # round-trip within half a step


def pin_q8_levels(Q):
    """Levels times scales equal the exact oracle's dequantised weights."""
    rng = np.random.default_rng(13)
    words = rng.integers(0, 2 ** 32, size=(9, 4, 2), dtype=np.uint64).astype(np.uint32)
    s = rng.integers(0x0400, 0x7800, size=(9, 4)).astype(np.uint16)
    lev, sc = Q.weight_levels(words, s)
    got = (lev.astype(np.float64) * sc[..., None]).reshape(9, -1)
    assert np.array_equal(got, _dense64(words, s))


def pin_q8_gateup_exact(Q):
    """With activations on their Q8 grid (x = n * 2^-4, one |n| = 127 per
    block) quantisation is exact, and g, u equal the plain fp64 matmul."""
    rng = np.random.default_rng(14)
    d, f = 128, 64
    gw, uw, _ = _expert(rng, d, f)
    n = rng.integers(-126, 127, size=(7, d)).astype(np.float64)
    n[:, ::32] = np.where(rng.random((7, d // 32)) < 0.5, -127.0, 127.0)
    x = (n * 2.0 ** -4).astype(np.float32)
    xq, xd = Q.quantize_q8(x)
    assert np.array_equal(xq.astype(np.float64), n) and np.all(xd == np.float32(2.0 ** -4))
    g, u = Q.gateup_q8(xq, xd, gw, uw)
    x64 = x.astype(np.float64)
    for got, (wq, ws) in ((g, gw), (u, uw)):
        want = x64 @ _dense64(wq, ws).T
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def pin_q8_down_exact(Q):
    rng = np.random.default_rng(15)
    d, f = 96, 128
    _, _, dw = _expert(rng, d, f)
    n = rng.integers(-127, 128, size=(5, f)).astype(np.float64)
    n[:, 5::32] = 127.0
    h = (n * 2.0 ** 3).astype(np.float32)
    hq, hd = Q.quantize_q8(h)
    got = Q.down_q8(hq, hd, dw)
    want = h.astype(np.float64) @ _dense64(*dw).T
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def pin_q8_h_on_grid(Q):
    """The down projection sees h on its Q8 grid: with a down matrix that
    copies h (level 1, scale 1 on the diagonal, level 0 elsewhere) the
    expert's output is q * d per block, so out / (blockmax / 127) is an
    integer within fp32 rounding."""
    rng = np.random.default_rng(16)
    d = f = 64
    gw, uw, _ = _expert(rng, d, f)
    lev = np.zeros((d, f // 32, 32), dtype=np.int8)
    for i in range(d):
        lev[i, i // 32, i % 32] = 1
    dq = mi.pack_codes(lev, 2)
    ds = np.full((d, f // 32), 0x3C00, dtype=np.uint16)
    x = rng.standard_normal((6, d)).astype(np.float32)
    xq, xd = Q.quantize_q8(x)
    out = Q.swiglu_expert_q8(xq, xd, gw, uw, (dq, ds)).astype(np.float64).reshape(6, 2, 32)
    step = np.abs(out).max(axis=-1, keepdims=True) / 127.0
    r = out / step
    assert np.all(np.abs(r - np.rint(r)) < 1e-4), np.abs(r - np.rint(r)).max()
    g, u = Q.gateup_q8(xq, xd, gw, uw)
    h = (g / (1 + np.exp(-g)) * u).reshape(6, 2, 32)
    off = np.abs(h / step - np.rint(h / step)).max()
    assert off > 0.05                                           # unquantised h is off the grid


def _layer_case(seed, T=24, d=256, f=128, E=6, k=2):
    rng = np.random.default_rng(seed)
    experts = [_expert(rng, d, f) for _ in range(E)]
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = (0.05 * rng.standard_normal((d, E))).astype(np.float32)
    ids, gates, _ = O.route(x, wr, None, k)
    return x, ids, gates, experts


def pin_q8_error_bound(Q):
    """Against the exact-weight oracle (fp32 activations), the variant's
    per-row error max|dy| / max|y| stays below 3e-2 and is not zero.

    Derivation: Q8 rounding of a Gaussian block leaves a relative rms error
    of about (amax / 127) / sqrt(12) / rms ~ 2.4 / 127 / 3.46 ~ 5.5e-3 on
    each dot product (x for gate/up, h for down, independently); through
    SwiGLU (h ~ g * u, both perturbed) and the down projection that is
    ~1.1e-2 rms relative per output, and the largest of d_model outputs of a
    row sits ~3 sigma out, relative to a row maximum ~3.5 rms: ~1e-2.  The
    bound is 3x that."""
    x, ids, gates, experts = _layer_case(21)
    outs = np.zeros((x.shape[0], ids.shape[1], x.shape[1]), dtype=np.float32)
    for e in np.unique(ids):
        t, j = np.nonzero(ids == e)
        gw, uw, dw = experts[e]
        outs[t, j] = O.swiglu_expert(x[t], O.dequantize(*gw, 2), O.dequantize(*uw, 2), O.dequantize(*dw, 2))
    y = O.combine(gates, outs)
    yq = Q.moe_layer_q8(x, ids, gates, lambda e: experts[e])
    err = np.abs(yq - y).max(axis=1) / np.abs(y).max(axis=1)
    assert err.max() < 3e-2, err.max()
    assert np.median(err) > 1e-3, np.median(err)


def pin_q8_bucket_form(Q):
    """The bucket form (pairs grouped by expert) gives the per-token form's
    result bit for bit, and a sampled subset of rows equals those rows."""
    x, ids, gates, experts = _layer_case(22)
    off, pairs = O.bucket_pairs(ids, len(experts))
    yb = Q.moe_ffn_q8_buckets(x, gates, ids.shape[1], off, pairs, lambda e: experts[e])
    yl = Q.moe_layer_q8(x, ids, gates, lambda e: experts[e])
    assert np.array_equal(yb, yl)
    rows = np.array([1, 7, 20])
    ys = Q.moe_ffn_q8_buckets(x, gates, ids.shape[1], off, pairs, lambda e: experts[e], rows=rows)
    assert np.array_equal(ys[rows], yl[rows])
    assert not np.any(np.delete(ys, rows, axis=0))


def pin_q8_bf16_input(Q):
    """bf16 bit patterns quantise like the fp32 values they encode."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    b = (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    xf = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    _, ids, gates, experts = _layer_case(24, T=4, d=64, f=64, E=3, k=2)
    assert np.array_equal(Q.moe_layer_q8(b, ids, gates, lambda e: experts[e]),
                          Q.moe_layer_q8(xf, ids, gates, lambda e: experts[e]))


PINS = [pin_q8_golden, pin_q8_rational, pin_q8_invariants, pin_q8_levels, pin_q8_gateup_exact,
        pin_q8_down_exact, pin_q8_h_on_grid, pin_q8_error_bound, pin_q8_bucket_form, pin_q8_bf16_input]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(Q)


# ------------------------------------------------------ planted mistakes

def _mut_trunc(orig):
    def f(v):
        v = np.asarray(v, dtype=np.float32)
        blk = v.reshape(v.shape[:-1] + (-1, 32))
        amax = np.max(np.abs(blk), axis=-1).astype(np.float32)
        safe = np.where(amax > 0, amax, np.float32(1)).astype(np.float32)
        q = np.trunc(blk * (np.float32(127) / safe)[..., None]).astype(np.int8)
        return q.reshape(v.shape), np.where(amax > 0, safe / np.float32(127), 0).astype(np.float32)
    return "quantize_q8", f


def _mut_scale_128(orig):
    def f(v):
        q, d = orig(np.asarray(v, np.float32) * np.float32(127.0 / 128.0))
        return q, (d * np.float32(128.0 / 127.0)).astype(np.float32)
    return "quantize_q8", f


def _mut_half_away(orig):
    def f(v):
        v = np.asarray(v, dtype=np.float32)
        q, d = orig(v)
        blk = v.reshape(v.shape[:-1] + (-1, 32))
        inv = np.where(d > 0, np.float32(127) / np.where(d > 0, d * np.float32(127), 1), 0).astype(np.float32)
        s = blk * inv[..., None]
        q2 = np.clip(np.sign(s) * np.floor(np.abs(s) + 0.5), -127, 127).astype(np.int8)
        return q2.reshape(v.shape), d
    return "quantize_q8", f


def _mut_level_offset(orig):
    def f(qw, sw):
        lev, s = orig(qw, sw)
        return (lev + 1).astype(np.int8), s
    return "weight_levels", f


def _mut_level_reversed(orig):
    def f(qw, sw):
        lev, s = orig(qw, sw)
        return lev[..., ::-1].copy(), s
    return "weight_levels", f


def _mut_no_act_scale(orig):
    return "block_dot_q8", lambda aq, ad, lev, ws: orig(aq, np.ones_like(ad), lev, ws)


def _mut_block_scale_shift(orig):
    return "block_dot_q8", lambda aq, ad, lev, ws: orig(aq, ad, lev, np.roll(ws, 1, axis=1))


def _mut_h_unquantised(orig):
    def f(xq, xd, gate, up, down):
        g, u = Q.gateup_q8(xq, xd, gate, up)
        h = (g / (1.0 + np.exp(-g)) * u)
        ld, sd = Q.weight_levels(*down)
        w = (ld.astype(np.float64) * sd[..., None]).reshape(ld.shape[0], -1)
        return (h @ w.T).astype(np.float32)
    return "swiglu_expert_q8", f


def _mut_gate_up_swapped(orig):
    def f(xq, xd, gate, up):
        g, u = orig(xq, xd, gate, up)
        return u, g
    return "gateup_q8", f


MUTATIONS = [_mut_trunc, _mut_scale_128, _mut_half_away, _mut_level_offset, _mut_level_reversed,
             _mut_no_act_scale, _mut_block_scale_shift, _mut_h_unquantised, _mut_gate_up_swapped]


def name_of(mut):
    return mut(lambda *a, **k: None)[0]


@pytest.mark.parametrize("mut", MUTATIONS, ids=[m.__name__ for m in MUTATIONS])
def test_planted_mistakes_are_caught(mut, monkeypatch):
    name, bad = mut(getattr(Q, name_of(mut)))
    monkeypatch.setattr(Q, name, bad)
    failed = []
    for pin in PINS:
        try:
            pin(Q)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"planted mistake in {name} went unnoticed"

"""Edge cases of the block format through every HIP path.

Hand-picked blocks of the 2-bit and 3-bit formats (zero scale, the smallest
subnormal scale 2^-24, the largest scales, and the 3-bit weights that
straddle a word boundary, as in tests/golden/blocks.txt) are written into
otherwise random experts and sent through moe_ffn_decode (2- and 3-bit),
moe_ffn_prefill and moe_decode_stack; outputs are compared with the oracle.

The prefill path feeds level * scale to the fp16 matrix cores, so its
largest scale is 32752 (0x77FF: -2 * 32752 = -65504 is the most negative
fp16); the decode and stack paths apply the scale in fp32 and take the
largest fp16 scale 65504 (0x7BFF)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import moe_inputs as mi
import oracle.moe_oracle as O
from helpers import TOL, floored_rel_err, row_rel_err

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

E, D, F, T = 4, 256, 128, 5
BIG_ROWS = 16          # down rows 0..15 carry the largest-scale block


def _say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def q(need_gpu):
    import quantized_moe_expert_lds_amd as q
    return q


def _block_words(bits, levels):
    return mi.pack_codes(np.asarray(levels, dtype=np.int64)[None, :], bits)[0]


def edge_experts(bits: int, big_scale: int):
    """Stored experts [E] (codes, scales per tensor) with edge blocks planted.
    Returns dict name -> (q [E][N][K/32][W] uint32, s [E][N][K/32] uint16)."""
    key = mi.derive_key(7, 99, bits)
    out = {}
    for ti, (name, (n, k)) in enumerate((("gate", (F, D)), ("up", (F, D)), ("down", (D, F)))):
        v = mi.normal(mi.derive_key(key, ti), E * n * k, 0.02).reshape(E * n, k)
        lev, s = mi.quantize_blocks(v, bits)
        qw = mi.pack_codes(lev, bits).reshape(E, n, k // 32, -1)
        out[name] = [qw, s.reshape(E, n, k // 32).copy()]
    lo, hi = (-2, 1) if bits == 2 else (-4, 3)
    mixed = np.array([lo, hi] * 16)
    gq, gs = out["gate"]
    uq, us = out["up"]
    dq, ds = out["down"]
    gs[0, 0:4, 0] = 0x0000                     # zero scale (codes left random)
    gs[1, 5, 2] = 0x0001                       # smallest subnormal scale
    gq[1, 5, 2] = _block_words(bits, mixed)
    us[2, 7, 1] = 0x0001
    us[3, 0, :] = 0x0000                       # a whole zero row
    gs[2, 9, 5] = big_scale                    # largest scale, on a block whose inputs are tiny
    gq[2, 9, 5] = _block_words(bits, mixed)
    ds[0, :BIG_ROWS, 0] = big_scale            # largest scale on the down projection
    dq[0, :BIG_ROWS, 0] = _block_words(bits, [lo] * 16 + [hi] * 16)
    ds[1, 3, 3] = 0x0001
    if bits == 3:
        # weights 10 and 21 straddle word boundaries: the only non-lowest codes
        for r, i in ((4, 10), (5, 21)):
            levs = np.full(32, lo)
            levs[i] = hi
            dq[1, r, 1] = _block_words(3, levs)
            ds[1, r, 1] = 0x3C00
    return out


def tokens():
    x = mi.normal(mi.derive_key(7, 98), T * D, 1.0).reshape(T, D)
    # inputs of gate block 5 (largest scale) are small, so that h stays in the
    # fp16 range, but mostly above the fp16 subnormal range (6.1e-5)
    x[:, 160:192] *= np.float32(3e-3)
    return x.astype(np.float32)


def oracle_y(ex, x, bits, k):
    wr = np.zeros((D, E), np.float32)          # all experts chosen; gates from the bias
    bias = np.array([0.5, 0.25, -0.25, 0.0], np.float32)
    stored = lambda e: tuple((ex[n][0][e], ex[n][1][e]) for n in ("gate", "up", "down"))
    ids, gates, y = O.moe_layer(x, wr, bias, k, stored, bits)
    return wr, bias, ids, gates, y


def dev(ex):
    return {n: (torch.from_numpy(ex[n][0].view(np.int32)).cuda(), torch.from_numpy(ex[n][1].view(np.int16)).cuda())
            for n in ex}


def experts_obj(q, d, bits):
    return q.Experts(d["gate"][0], d["up"][0], d["down"][0], d["gate"][1], d["up"][1], d["down"][1], bits)


def magnitude(ex, x, bits, gates, ids):
    """Per output element, the sum of the absolute values of the terms that
    form it: sum_j gate_j sum_f |h_jf| |Wd_jdf| (fp64).  The GPU rounds h (and
    the activations) to fp16, so its error is bounded by a small multiple of
    2^-11 times this, whatever cancellation the sum has."""
    deq = lambda n, e: O.dequantize(ex[n][0][e], ex[n][1][e], bits).astype(np.float64)
    x64 = x.astype(np.float64)
    m = np.zeros((x.shape[0], D))
    with np.errstate(over="ignore"):
        for t in range(x.shape[0]):
            for j, e in enumerate(ids[t]):
                g = x64[t] @ deq("gate", e).T
                u = x64[t] @ deq("up", e).T
                h = g / (1 + np.exp(-g)) * u
                m[t] += float(gates[t, j]) * (np.abs(h) @ np.abs(deq("down", e)).T)
    return m


def check(y, y_o, m, label):
    y = np.asarray(y, np.float64)
    cond = float(np.max(np.abs(y - y_o) / np.maximum(m, 1e-30)))
    rest = row_rel_err(y[:, BIG_ROWS:], y_o[:, BIG_ROWS:])
    print(f"{label}: error / term magnitude {cond:.2e}; row error of the rows without the largest scale "
          f"{rest:.2e} (floored {floored_rel_err(y[:, BIG_ROWS:], y_o[:, BIG_ROWS:]):.2e}); "
          f"max |y| {np.abs(y_o).max():.3g}")
    assert np.all(np.isfinite(y))
    assert cond <= TOL and rest <= TOL


def _premise(ex, x, bits):
    """The SwiGLU intermediate must be fp16-representable on every path."""
    deq = lambda n, e: O.dequantize(ex[n][0][e], ex[n][1][e], bits)
    with np.errstate(over="ignore"):
        for e in range(E):
            g = x @ deq("gate", e).T
            u = x @ deq("up", e).T
            h = g / (1 + np.exp(-g)) * u
            assert np.abs(h).max() < 6e4


@pytest.mark.parametrize("bits", [2, 3])
def test_edge_blocks_decode(q, bits):
    _say(f"moe_ffn_decode, {bits}-bit edge blocks (scales 0, 2^-24, 65504; straddling 3-bit weights)")
    ex = edge_experts(bits, 0x7BFF)
    x = tokens()
    _premise(ex, x, bits)
    wr, bias, ids_o, gates_o, y_o = oracle_y(ex, x, bits, E)
    d = dev(ex)
    ids = torch.from_numpy(ids_o).cuda()
    gates = torch.from_numpy(gates_o).cuda()
    y = torch.empty((T, D), device="cuda")
    q.moe_ffn_decode(experts_obj(q, d, bits), torch.from_numpy(x).cuda(), ids, gates, y,
                     q.workspace(q.MOE_OP_DECODE, T, D, F, E, E))
    torch.cuda.synchronize()
    check(y.cpu().numpy(), y_o, magnitude(ex, x, bits, gates_o, ids_o), f"decode {bits}-bit")


def test_edge_blocks_prefill(q):
    _say("route + moe_ffn_prefill, 2-bit edge blocks (scales 0, 2^-24, 32752)")
    ex = edge_experts(2, 0x77FF)
    x = tokens()
    _premise(ex, x, 2)
    wr, bias, ids_o, gates_o, y_o = oracle_y(ex, x, 2, E)
    d = dev(ex)
    router = q.Router(torch.from_numpy(np.ascontiguousarray(wr.T)).cuda(), torch.from_numpy(bias).cuda(), E)
    xd = torch.from_numpy(x).cuda()
    ids = torch.empty((T, E), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, E), device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    prs = torch.empty(T * E, dtype=torch.int32, device="cuda")
    q.moe_route(router, xd, ids, gates, off, prs, q.workspace(q.MOE_OP_ROUTE, T, D, F, E, E))
    y = torch.empty((T, D), device="cuda")
    q.moe_ffn_prefill(experts_obj(q, d, 2), xd, gates, off, prs, y, q.workspace(q.MOE_OP_PREFILL, T, D, F, E, E))
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    check(y.cpu().numpy(), y_o, magnitude(ex, x, 2, gates_o, ids_o), "prefill 2-bit")


@pytest.mark.parametrize("bits", [2, 3])
def test_edge_blocks_stack(q, bits):
    _say(f"moe_decode_stack (1 layer), {bits}-bit edge blocks")
    ex = edge_experts(bits, 0x7BFF)
    x = tokens()
    _premise(ex, x, bits)
    wr, bias, ids_o, gates_o, y_o = oracle_y(ex, x, bits, E)
    d = dev(ex)
    st = q.Stack(torch.from_numpy(np.ascontiguousarray(wr.T))[None].contiguous().cuda(),
                 torch.from_numpy(bias)[None].contiguous().cuda(),
                 d["gate"][0][None], d["up"][0][None], d["down"][0][None],
                 d["gate"][1][None], d["up"][1][None], d["down"][1][None], bits, E)
    h = torch.empty((T, D), device="cuda")
    ids = torch.empty((1, T, E), dtype=torch.int32, device="cuda")
    g = torch.empty((1, T, E), device="cuda")
    ws = q.stack_workspace(st, T)
    q.moe_decode_stack(st, torch.from_numpy(x).cuda(), h, ws, ids, g)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy()[0], ids_o)
    check(h.cpu().numpy() - x, y_o, magnitude(ex, x, bits, gates_o, ids_o), f"stack {bits}-bit")   # h = x + y

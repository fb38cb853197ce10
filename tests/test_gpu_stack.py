"""moe_decode_stack: whole decode / verify steps (every layer in one
persistent launch) against the oracle's free-running chain, token by token
and layer by layer (chain_walk), plus batch invariance (a batch equals its
tokens run alone, bitwise), determinism across launches and argument checks.

Token streams that must match the oracle through all 48 layers are picked by
the oracle alone (tests/golden/chain_margins.json)."""
from __future__ import annotations

import copy
import ctypes
import sys

import numpy as np
import pytest

import moe_inputs as mi
import oracle.moe_oracle as O
from chain_walk import full_depth_streams, stream_tokens, walk
from helpers import TOL, device_stack, oracle_experts, row_rel_err
import oracle_pool

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def q(need_gpu):
    import quantized_moe_expert_lds_amd as q
    return q


def to_device(x: np.ndarray):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x).cuda()


def run_stack(q, st, x, ws=None):
    """One moe_decode_stack launch; returns (h_out, ids, gates, h_layers) on
    the host and the workspace."""
    T = x.shape[0]
    L, K, D = st.n_layers, st.top_k, st.d_model
    h = torch.empty((T, D), device="cuda")
    ids = torch.empty((L, T, K), dtype=torch.int32, device="cuda")
    g = torch.empty((L, T, K), device="cuda")
    hl = torch.empty((L, T, D), device="cuda")
    ws = q.stack_workspace(st, T) if ws is None else ws
    q.moe_decode_stack(st, x, h, ws, ids, g, h_layers=hl)
    torch.cuda.synchronize()
    err = int(ws[q.MOE_STACK_ERROR_OFFSET:q.MOE_STACK_ERROR_OFFSET + 4].view(torch.int32).item())
    assert err == 0, "grid barrier timed out"
    return h.cpu().numpy(), ids.cpu().numpy(), g.cpu().numpy(), hl.cpu().numpy(), ws


def check_batch_invariance(q, st, xd, out):
    """Every token of a batch run equals the same token run alone, bitwise."""
    h, ids, g, hl, _ = out
    for t in range(xd.shape[0]):
        h1, ids1, g1, hl1, _ = run_stack(q, st, xd[t:t + 1].contiguous())
        assert np.array_equal(h1[0], h[t]), f"token {t}: batch result differs from the token alone"
        assert np.array_equal(ids1[:, 0], ids[:, t]) and np.array_equal(g1[:, 0], g[:, t])
        assert np.array_equal(hl1[:, 0], hl[:, t])


@pytest.fixture(scope="module")
def stack2(q):
    wl = mi.WORKLOADS["decode_48layer"]
    st, ex, rw, rb = device_stack(wl)
    yield st
    del st, ex, rw, rb
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def stack3(q, stack2):
    wl = mi.WORKLOADS["verify4_3bit"]
    st, ex, rw, rb = device_stack(wl)
    yield st
    del st, ex, rw, rb
    torch.cuda.empty_cache()


def test_stack_tiny_single_layer(q):
    _say("moe_decode_stack, tiny workload (1 layer, 16 experts, T=8)")
    wl = mi.WORKLOADS["tiny"]
    st, ex, rw, rb = device_stack(wl)
    x = mi.activations_host(wl)
    out = run_stack(q, st, torch.from_numpy(x).cuda())
    matched, _ = walk(wl, 2, x, out[1], out[2], out[3], out[0], full=range(8), label="tiny")
    assert matched == [1] * 8


def test_stack_decode_48_layers(q, stack2):
    _say("moe_decode_stack, 48 layers x 512 experts, T=1, 2-bit: stream 0 and two full-depth streams")
    wl = mi.WORKLOADS["decode_48layer"]
    st = stack2
    x = mi.activations_host(wl)
    xd = torch.from_numpy(x).cuda()
    out = run_stack(q, st, xd)
    # the same workspace again (the kernel resets its counters): identical bits
    h2, _, _, _, _ = run_stack(q, st, xd, ws=out[4])
    assert np.array_equal(out[0], h2)
    walk(wl, 2, x, out[1], out[2], out[3], out[0], label="decode_48layer stream 0")
    for s in full_depth_streams(wl.name, 2):
        xs = stream_tokens(wl, [s])
        o = run_stack(q, st, torch.from_numpy(xs).cuda())
        walk(wl, 2, xs, o[1], o[2], o[3], o[0], full=[0], label=f"decode_48layer stream {s}")
    # the layer-by-layer router agrees on the first layer
    router = q.Router(st.router_w[0], st.router_b[0], wl.top_k)
    ids1 = torch.empty((1, wl.top_k), dtype=torch.int32, device="cuda")
    w1 = torch.empty((1, wl.top_k), device="cuda")
    q.moe_route(router, xd, ids1, w1, None, None, q.workspace(q.MOE_OP_ROUTE, 1, 2048, 768, 512, 10))
    torch.cuda.synchronize()
    assert np.array_equal(ids1.cpu().numpy()[0], out[1][0, 0])


def test_stack_verify_4_tokens_3bit(q, stack3):
    _say("moe_decode_stack, 48 layers, T=4, 3-bit: the seeded batch, and a batch of 4 full-depth tokens")
    wl = mi.WORKLOADS["verify4_3bit"]
    st = stack3
    x = mi.activations_host(wl)
    xd = torch.from_numpy(x).cuda()
    out = run_stack(q, st, xd)
    check_batch_invariance(q, st, xd, out)
    walk(wl, 3, x, out[1], out[2], out[3], out[0], label="verify4_3bit seeded batch")
    xs = stream_tokens(wl, full_depth_streams(wl.name, 4))
    xsd = torch.from_numpy(xs).cuda()
    o = run_stack(q, st, xsd)
    check_batch_invariance(q, st, xsd, o)
    matched, _ = walk(wl, 3, xs, o[1], o[2], o[3], o[0], full=range(4), label="verify4_3bit full-depth batch")
    assert matched == [48] * 4


@pytest.mark.parametrize("bits", [2, 3])
def test_stack_verify_6_tokens(q, stack2, stack3, bits):
    _say(f"moe_decode_stack, 48 layers, T=6 (1 + 5 drafts), {bits}-bit, full depth, vs 6 x T=1")
    wl = mi.WORKLOADS["decode_48layer" if bits == 2 else "verify4_3bit"]
    st = stack2 if bits == 2 else stack3
    xs = stream_tokens(wl, full_depth_streams(wl.name, 6))
    xd = torch.from_numpy(xs).cuda()
    out = run_stack(q, st, xd)
    check_batch_invariance(q, st, xd, out)
    matched, _ = walk(wl, bits, xs, out[1], out[2], out[3], out[0], full=range(6), label=f"T=6 {bits}-bit")
    assert matched == [48] * 6


@pytest.mark.parametrize("T", [2, 8])
def test_stack_3bit_batches(q, stack3, T):
    _say(f"moe_decode_stack, 48 layers, 3-bit, T={T}: per-token oracle walk and batch invariance")
    wl = mi.WORKLOADS["verify4_3bit"]
    st = stack3
    streams = full_depth_streams(wl.name, min(T, 6))
    streams += [100 + i for i in range(T - len(streams))]          # seeded tokens with no margin guarantee
    xs = stream_tokens(wl, streams)
    xd = torch.from_numpy(xs).cuda()
    out = run_stack(q, st, xd)
    check_batch_invariance(q, st, xd, out)
    walk(wl, 3, xs, out[1], out[2], out[3], out[0], full=range(min(T, 6)), label=f"3-bit T={T}")


def test_stack_batch_of_8(q, stack2):
    _say("moe_decode_stack, 48 layers, T=8 (largest batch), 2-bit")
    wl = mi.WORKLOADS["decode_48layer"]
    st = stack2
    x = mi.activations_host(wl, 8, stream=11)
    xd = torch.from_numpy(x).cuda()
    out = run_stack(q, st, xd)
    check_batch_invariance(q, st, xd, out)
    walk(wl, 2, x, out[1], out[2], out[3], out[0], label="2-bit T=8")


def test_stack_single_layer_bf16_matches_layer_calls(q):
    _say("moe_decode_stack, single-layer decode (bf16 token, 512 experts) vs oracle and vs moe_route + moe_ffn_decode")
    wl = mi.WORKLOADS["decode_1layer"]
    st, ex, rw, rb = device_stack(wl)
    x = mi.activations_host(wl)                       # bf16 bit patterns
    xd = to_device(x)
    h, ids, g, hl, _ = run_stack(q, st, xd)
    walk(wl, 2, x, ids, g, hl, h, full=[0], label="decode_1layer")
    # the layer-by-layer calls agree on routing, and on the layer output to rounding
    router = q.Router(rw[0], rb[0], wl.top_k)
    experts = q.Experts(ex["gate_q"][0], ex["up_q"][0], ex["down_q"][0], ex["gate_s"][0], ex["up_s"][0],
                        ex["down_s"][0], 2)
    ids1 = torch.empty((1, wl.top_k), dtype=torch.int32, device="cuda")
    w1 = torch.empty((1, wl.top_k), device="cuda")
    q.moe_route(router, xd, ids1, w1, None, None, q.workspace(q.MOE_OP_ROUTE, 1, 2048, 768, 512, 10))
    y1 = torch.empty((1, 2048), device="cuda")
    q.moe_ffn_decode(experts, xd, ids1, w1, y1, q.workspace(q.MOE_OP_DECODE, 1, 2048, 768, 512, 10))
    torch.cuda.synchronize()
    assert np.array_equal(ids1.cpu().numpy()[0], ids[0, 0])
    assert np.max(np.abs(w1.cpu().numpy()[0] - g[0, 0])) <= 1e-6
    h_layers = (xd.float() + y1).cpu().numpy()
    assert row_rel_err(h, h_layers) <= TOL
    del st, ex, rw, rb
    torch.cuda.empty_cache()


def test_stack_256_experts(q):
    _say("moe_decode_stack, 4 layers x 256 experts (one router expert per workgroup), T=2 and T=6")
    wl = mi.WORKLOADS["coder_256"]
    st, ex, rw, rb = device_stack(wl)
    for T, stream in ((2, 0), (6, 1)):
        x = mi.activations_host(wl, T, stream=stream)
        xd = torch.from_numpy(x).cuda()
        out = run_stack(q, st, xd)
        check_batch_invariance(q, st, xd, out)
        walk(wl, 2, x, out[1], out[2], out[3], out[0], label=f"256 experts T={T}")
    del st, ex, rw, rb
    torch.cuda.empty_cache()


def test_stack_batch_of_3(q):
    _say("moe_decode_stack, 4 layers, T=3 (odd batch) equals three batch-1 runs")
    wl = mi.WORKLOADS["decode_48layer"]
    st, ex, rw, rb = device_stack(wl, n_layers=4)
    x = mi.activations_host(wl, 3, stream=7)
    xd = torch.from_numpy(x).cuda()
    out = run_stack(q, st, xd)
    check_batch_invariance(q, st, xd, out)
    walk(wl, 2, x, out[1], out[2], out[3], out[0], label="T=3, 4 layers")
    del st, ex, rw, rb
    torch.cuda.empty_cache()


def test_stack_abi_errors(q):
    _say("moe_decode_stack argument checks (before any launch)")
    wl = mi.WORKLOADS["tiny"]
    st, ex, rw, rb = device_stack(wl)
    x = torch.from_numpy(mi.activations_host(wl)).cuda()
    h = torch.empty((8, 256), device="cuda")
    ws = q.stack_workspace(st, 8)
    lib = q.library

    def call(stack, xx, n, hh, w, nbytes, ids=None, gates=None):
        return lib.moe_decode_stack(ctypes.byref(stack._c), q._ptr(xx), q._dtype(xx), n, 1e-6, q._ptr(hh),
                                    q._ptr(ids), q._ptr(gates), None, q._ptr(w), nbytes, None)

    assert call(st, x, 8, h, ws, ws.numel()) == q.MOE_OK
    torch.cuda.synchronize()
    assert call(st, x, 0, h, ws, ws.numel()) == q.MOE_ERR_ARG
    assert call(st, x, 9, h, ws, ws.numel()) == q.MOE_ERR_UNSUPPORTED          # more than 8 tokens
    assert call(st, x, 8, h, None, 0) == q.MOE_ERR_WORKSPACE
    assert call(st, x, 8, h, ws, 4096) == q.MOE_ERR_WORKSPACE                   # far below any grid's need
    ids = torch.empty((1, 8, 2), dtype=torch.int32, device="cuda")
    assert call(st, x, 8, h, ws, ws.numel(), ids=ids) == q.MOE_ERR_ARG           # ids without gates
    bad = copy.copy(st)
    bad._c = q._StackT.from_buffer_copy(st._c)
    bad._c.bits = 4
    assert call(bad, x, 8, h, ws, ws.numel()) == q.MOE_ERR_UNSUPPORTED
    bad._c.bits = 2
    bad._c.top_k = 17                                                           # k > experts
    assert call(bad, x, 8, h, ws, ws.numel()) == q.MOE_ERR_UNSUPPORTED
    bad._c.top_k = 2
    bad._c.d_model = 250                                                        # not a multiple of 32
    assert call(bad, x, 8, h, ws, ws.numel()) == q.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    err = int(ws[q.MOE_STACK_ERROR_OFFSET:q.MOE_STACK_ERROR_OFFSET + 4].view(torch.int32).item())
    assert err == 0

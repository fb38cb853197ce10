"""moe_decode_stack: a whole decode/verify step (every layer, one persistent
launch) against the free-running CPU oracle, plus batch invariance,
determinism across launches and the barrier error word."""
from __future__ import annotations

import copy
import ctypes
import sys

import numpy as np
import pytest

import moe_inputs as mi
import oracle.moe_oracle as O
from helpers import TOL, device_stack, oracle_experts, row_rel_err
import oracle_pool

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

NEAR_TIE = 2e-3


def _say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def q(need_gpu):
    import quantized_moe_expert_lds_amd as q
    return q


def run_stack(q, st, x, T, record=True):
    L, K, D = st.n_layers, st.top_k, st.d_model
    h = torch.empty((T, D), device="cuda")
    ids = torch.empty((L, T, K), dtype=torch.int32, device="cuda") if record else None
    g = torch.empty((L, T, K), device="cuda") if record else None
    ws = q.stack_workspace(st, T)
    q.moe_decode_stack(st, x, h, ws, ids, g)
    torch.cuda.synchronize()
    err = int(ws[q.MOE_STACK_ERROR_OFFSET:q.MOE_STACK_ERROR_OFFSET + 4].view(torch.int32).item())
    assert err == 0, "grid barrier timed out"
    return h, ids, g, ws


def oracle_walk(wl, x, ids_g, gates_g, h_gpu, bits):
    """Free-running oracle chain; returns layers matched.  A routing
    difference is accepted only at a near-tie, after which the streams are no
    longer comparable."""
    h = O.as_f32_activations(x)
    L = ids_g.shape[0]
    for l in range(L):
        u = h if l == 0 else O.rmsnorm(h)
        wh, bh = mi.router_host(wl, l)
        ids_o, gates_o, z_o = O.route(u, wh, bh if wl.zipf_bias else None, wl.top_k)
        ig = ids_g[l]
        if not np.array_equal(ig, ids_o):
            margins = []
            for t in range(ids_o.shape[0]):
                diff = np.nonzero(ig[t] != ids_o[t])[0]
                if diff.size:
                    j = diff[0]
                    margins.append(z_o[t, ids_o[t, j]] - z_o[t, ig[t, j]])
            print(f"layer {l}: routing differs at a near-tie, oracle margins {margins}")
            assert max(margins) < NEAR_TIE, f"routing differs at layer {l} beyond a near-tie"
            return l
        assert np.max(np.abs(gates_g[l] - gates_o)) <= TOL
        oracle_pool.prefetch(wl.name, l, np.unique(ids_o), bits)
        _, _, y_o = O.moe_layer(u, wh, bh if wl.zipf_bias else None, wl.top_k, oracle_experts(wl, l, bits), bits)
        h = (h + y_o).astype(np.float32)
    err = row_rel_err(h_gpu, h)
    print(f"all {L} layers matched; final residual row_rel_err={err:.2e}")
    assert err <= TOL
    return L


def test_stack_tiny_single_layer(q):
    _say("moe_decode_stack, tiny workload (1 layer, 16 experts, T=8)")
    wl = mi.WORKLOADS["tiny"]
    st, ex, rw, rb = device_stack(wl)
    x = mi.activations_host(wl)
    h, ids, g, _ = run_stack(q, st, torch.from_numpy(x).cuda(), wl.n_tokens)
    matched = oracle_walk(wl, x, ids.cpu().numpy(), g.cpu().numpy(), h.cpu().numpy(), 2)
    assert matched == 1


def test_stack_decode_48_layers(q):
    _say("moe_decode_stack, 48 layers x 512 experts, T=1, 2-bit")
    wl = mi.WORKLOADS["decode_48layer"]
    st, ex, rw, rb = device_stack(wl)
    x = mi.activations_host(wl)
    xd = torch.from_numpy(x).cuda()
    h, ids, g, ws = run_stack(q, st, xd, 1)
    # the same workspace again (counters were reset by the kernel): identical bits
    h2 = torch.empty_like(h)
    q.moe_decode_stack(st, xd, h2, ws)
    torch.cuda.synchronize()
    assert torch.equal(h, h2)
    matched = oracle_walk(wl, x, ids.cpu().numpy(), g.cpu().numpy(), h.cpu().numpy(), 2)
    assert matched >= 8
    # a second token: stream 0 meets a genuine near-tie at layer 13
    x1 = mi.activations_host(wl, 1, stream=1)
    h1, ids1s, g1s, _ = run_stack(q, st, torch.from_numpy(x1).cuda(), 1)
    matched1 = oracle_walk(wl, x1, ids1s.cpu().numpy(), g1s.cpu().numpy(), h1.cpu().numpy(), 2)
    print(f"token stream 1: {matched1} layers matched")
    assert matched1 >= 8
    # the layer-by-layer entry points agree on routing for the first layer
    router = q.Router(rw[0], rb[0], wl.top_k)
    ids1 = torch.empty((1, wl.top_k), dtype=torch.int32, device="cuda")
    w1 = torch.empty((1, wl.top_k), device="cuda")
    q.moe_route(router, xd, ids1, w1, None, None, q.workspace(q.MOE_OP_ROUTE, 1, 2048, 768, 512, 10))
    torch.cuda.synchronize()
    assert torch.equal(ids1[0], ids[0, 0])
    del st, ex, rw, rb
    torch.cuda.empty_cache()


def test_stack_verify_4_tokens_3bit(q):
    _say("moe_decode_stack, 48 layers, T=4, 3-bit; batch invariance vs T=1")
    wl = mi.WORKLOADS["verify4_3bit"]
    st, ex, rw, rb = device_stack(wl)
    x = mi.activations_host(wl)
    xd = torch.from_numpy(x).cuda()
    h, ids, g, _ = run_stack(q, st, xd, 4)
    for t in range(4):
        h1, ids1, g1, _ = run_stack(q, st, xd[t:t + 1].contiguous(), 1)
        assert torch.equal(h1[0], h[t]), f"token {t}: T=4 differs from T=1"
        assert torch.equal(ids1[:, 0], ids[:, t]) and torch.equal(g1[:, 0], g[:, t])
    matched = oracle_walk(wl, x, ids.cpu().numpy(), g.cpu().numpy(), h.cpu().numpy(), 3)
    assert matched >= 8
    del st, ex, rw, rb
    torch.cuda.empty_cache()


def test_stack_batch_of_8(q):
    _say("moe_decode_stack, 4 layers, T=8 (largest batch), 2-bit")
    wl = mi.WORKLOADS["decode_48layer"]
    st, ex, rw, rb = device_stack(wl, n_layers=4)
    x = mi.activations_host(wl, 8, stream=11)
    xd = torch.from_numpy(x).cuda()
    h, ids, g, _ = run_stack(q, st, xd, 8)
    h1, ids1, _, _ = run_stack(q, st, xd[5:6].contiguous(), 1)
    assert torch.equal(h1[0], h[5])
    matched = oracle_walk(wl, x, ids.cpu().numpy(), g.cpu().numpy(), h.cpu().numpy(), 2)
    assert matched >= 1


def test_stack_single_layer_bf16_matches_layer_calls(q):
    _say("moe_decode_stack, single-layer decode (bf16 token, 512 experts) vs oracle and vs moe_route + moe_ffn_decode")
    wl = mi.WORKLOADS["decode_1layer"]
    st, ex, rw, rb = device_stack(wl)
    x = mi.activations_host(wl)                       # bf16 bit patterns
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    h, ids, g, _ = run_stack(q, st, xd, 1)
    # oracle: one layer, no norm before it: h = x + y
    wh, bh = mi.router_host(wl, 0)
    ids_o, gates_o, y_o = O.moe_layer(O.as_f32_activations(x), wh, bh, wl.top_k, oracle_experts(wl, 0, 2), 2)
    assert np.array_equal(ids.cpu().numpy()[0], ids_o)
    assert np.max(np.abs(g.cpu().numpy()[0] - gates_o)) <= TOL
    want = (O.as_f32_activations(x) + y_o).astype(np.float32)
    assert row_rel_err(h.cpu().numpy(), want) <= TOL
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
    assert torch.equal(ids1[0], ids[0, 0])
    assert torch.max(torch.abs(w1[0] - g[0, 0])).item() <= 1e-6
    h_layers = (xd.float() + y1).cpu().numpy()
    assert row_rel_err(h.cpu().numpy(), h_layers) <= TOL
    del st, ex, rw, rb
    torch.cuda.empty_cache()


def test_stack_256_experts_two_tokens(q):
    _say("moe_decode_stack, 4 layers x 256 experts (one router expert per workgroup), T=2, batch invariance")
    wl = mi.WORKLOADS["coder_256"]
    st, ex, rw, rb = device_stack(wl)
    x = mi.activations_host(wl)
    xd = torch.from_numpy(x).cuda()
    h, ids, g, _ = run_stack(q, st, xd, 2)
    for t in range(2):
        h1, ids1, g1, _ = run_stack(q, st, xd[t:t + 1].contiguous(), 1)
        assert torch.equal(h1[0], h[t]) and torch.equal(ids1[:, 0], ids[:, t]) and torch.equal(g1[:, 0], g[:, t])
    matched = oracle_walk(wl, x, ids.cpu().numpy(), g.cpu().numpy(), h.cpu().numpy(), 2)
    assert matched >= 1
    del st, ex, rw, rb
    torch.cuda.empty_cache()


def test_stack_batch_of_3(q):
    _say("moe_decode_stack, 4 layers, T=3 (odd batch) equals three batch-1 runs")
    wl = mi.WORKLOADS["decode_48layer"]
    st, ex, rw, rb = device_stack(wl, n_layers=4)
    x = mi.activations_host(wl, 3, stream=7)
    xd = torch.from_numpy(x).cuda()
    h, ids, g, _ = run_stack(q, st, xd, 3)
    for t in range(3):
        h1, ids1, g1, _ = run_stack(q, st, xd[t:t + 1].contiguous(), 1)
        assert torch.equal(h1[0], h[t]) and torch.equal(ids1[:, 0], ids[:, t]) and torch.equal(g1[:, 0], g[:, t])
    matched = oracle_walk(wl, x, ids.cpu().numpy(), g.cpu().numpy(), h.cpu().numpy(), 2)
    assert matched >= 1
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
                                    q._ptr(ids), q._ptr(gates), q._ptr(w), nbytes, None)

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

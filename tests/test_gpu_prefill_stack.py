"""moe_prefill_stack: a prompt cut into chunks through every layer of a
stack, against the CPU oracle's layer chain (tiny shapes), against the
layer-by-layer entry points (full shapes, bit for bit) and across chunk
sizes (bit for bit)."""
from __future__ import annotations

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


def run_prefill_stack(q, st, x, chunk):
    h = torch.full((x.shape[0], st.d_model), float("nan"), device="cuda")
    ws = q.prefill_stack_workspace(st, chunk)
    q.moe_prefill_stack(st, x, h, chunk, ws)
    torch.cuda.synchronize()
    return h


def test_prefill_stack_tiny_vs_oracle_chain(q):
    _say("moe_prefill_stack, 3 tiny layers, 40 tokens in chunks of 16 (16, 16, 8)")
    wl = mi.WORKLOADS["tiny_stack"]
    st, ex, rw, rb = device_stack(wl)
    x = mi.activations_host(wl)
    h_g = run_prefill_stack(q, st, torch.from_numpy(x).cuda(), 16).cpu().numpy()
    # the oracle chain over all tokens at once (tokens do not interact)
    h = O.as_f32_activations(x)
    close = np.ones(wl.n_tokens, dtype=bool)        # tokens with no near-tie at the top-k boundary
    for l in range(wl.n_layers):
        u = h if l == 0 else O.rmsnorm(h)
        wh, bh = mi.router_host(wl, l)
        _, _, z = O.route(u, wh, bh, wl.top_k)
        zs = -np.sort(-z, axis=1)
        close &= (zs[:, wl.top_k - 1] - zs[:, wl.top_k]) >= NEAR_TIE
        _, _, y = O.moe_layer(u, wh, bh, wl.top_k, oracle_experts(wl, l, 2), 2)
        h = (h + y).astype(np.float32)
    n = int(close.sum())
    print(f"{n} of {wl.n_tokens} tokens have no near-tie at the top-k boundary in any layer")
    assert n >= wl.n_tokens // 2
    err = row_rel_err(h_g[close], h[close])
    print(f"final residual row_rel_err={err:.2e}")
    assert err <= TOL
    assert np.isfinite(h_g).all()


def test_prefill_stack_matches_layer_calls_and_chunking(q):
    _say("moe_prefill_stack, first 2 layers of the 48-layer model, 300 tokens: vs layer calls, chunks 128 / 300")
    wl = mi.WORKLOADS["decode_48layer"]
    L = 2
    st, ex, rw, rb = device_stack(wl, n_layers=L)
    T, D, F, E, K = 300, wl.d_model, wl.d_ff, wl.n_experts, wl.top_k
    x = mi.activations_host(mi.WORKLOADS["prefill_8192"], T, stream=5)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    h128 = run_prefill_stack(q, st, xd, 128)
    h300 = run_prefill_stack(q, st, xd, 300)
    assert torch.equal(h128, h300), "result depends on the chunk size"
    # the same chain through the layer-by-layer entry points
    h = xd.float()
    u = torch.empty_like(h)
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    prs = torch.empty(T * K, dtype=torch.int32, device="cuda")
    y = torch.empty((T, D), device="cuda")
    ws_r = q.workspace(q.MOE_OP_ROUTE, T, D, F, E, K)
    ws_p = q.workspace(q.MOE_OP_PREFILL, T, D, F, E, K)
    for l in range(L):
        router = q.Router(rw[l], rb[l], K)
        experts = q.Experts(ex["gate_q"][l], ex["up_q"][l], ex["down_q"][l], ex["gate_s"][l], ex["up_s"][l],
                            ex["down_s"][l], 2)
        inp = xd if l == 0 else u
        q.moe_route(router, inp, ids, w, off, prs, ws_r)
        q.moe_ffn_prefill(experts, inp, w, off, prs, y, ws_p)
        q.moe_residual_rmsnorm(h, y, u)
    torch.cuda.synchronize()
    assert torch.equal(h128, h), "moe_prefill_stack differs from the layer-by-layer calls"
    del st, ex, rw, rb
    torch.cuda.empty_cache()


def test_prefill_stack_abi_errors(q):
    _say("moe_prefill_stack argument validation")
    wl = mi.WORKLOADS["tiny_stack"]
    st, ex, rw, rb = device_stack(wl)
    x = torch.zeros((4, wl.d_model), device="cuda")
    h = torch.empty_like(x)
    ws = q.prefill_stack_workspace(st, 4)
    lib = q.library
    P = ctypes.c_void_p
    c = ctypes.byref(st._c)
    args = lambda n, chunk, wsb: (c, P(x.data_ptr()), 0, n, chunk, 1e-6, P(h.data_ptr()), P(ws.data_ptr()), wsb, None)
    assert lib.moe_prefill_stack(*args(0, 4, ws.numel())) == q.MOE_ERR_ARG
    assert lib.moe_prefill_stack(*args(4, 0, ws.numel())) == q.MOE_ERR_ARG
    assert lib.moe_prefill_stack(*args(8, 8, ws.numel())) == q.MOE_ERR_WORKSPACE    # sized for chunks of 4
    assert lib.moe_prefill_stack(c, P(x.data_ptr()), 7, 4, 4, 1e-6, P(h.data_ptr()), P(ws.data_ptr()),
                                 ws.numel(), None) == q.MOE_ERR_ARG
    assert lib.moe_prefill_stack(*args(4, 4, ws.numel())) == q.MOE_OK
    torch.cuda.synchronize()
    assert lib.moe_prefill_stack_workspace_size(c, 0) == 0

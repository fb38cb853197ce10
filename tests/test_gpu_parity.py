"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.  Routing ids and bucket layouts must match bit for
bit; floating outputs within TOL (max over rows of max|err| / max|ref|)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import moe_inputs as mi
import oracle.moe_oracle as O
from helpers import TOL, device_layers, floored_rel_err, oracle_experts, row_rel_err
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


# ------------------------------------------------------------- helpers

def gpu_route(q, router, x, buckets=True):
    T, K, E = x.shape[0], router.top_k, router.n_experts
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda") if buckets else None
    prs = torch.empty(T * K, dtype=torch.int32, device="cuda") if buckets else None
    ws = q.workspace(q.MOE_OP_ROUTE, T, router.d_model, 0, E, K)
    q.moe_route(router, x, ids, w, off, prs, ws)
    torch.cuda.synchronize()
    return ids, w, off, prs


def gpu_decode(q, ex, x, ids, w):
    T, K = ids.shape
    y = torch.empty((T, ex.d_model), dtype=torch.float32, device="cuda")
    ws = q.workspace(q.MOE_OP_DECODE, T, ex.d_model, ex.d_ff, ex.n_experts, K)
    q.moe_ffn_decode(ex, x, ids, w, y, ws)
    torch.cuda.synchronize()
    return y


def gpu_prefill(q, ex, x, w, off, prs):
    T, K = w.shape
    y = torch.empty((T, ex.d_model), dtype=torch.float32, device="cuda")
    ws = q.workspace(q.MOE_OP_PREFILL, T, ex.d_model, ex.d_ff, ex.n_experts, K)
    q.moe_ffn_prefill(ex, x, w, off, prs, y, ws)
    torch.cuda.synchronize()
    return y


def np_x(x: "torch.Tensor") -> np.ndarray:
    """Device activations back to the oracle's input convention (bf16 as
    uint16 bit patterns).  Used only on tensors built from the host
    generator, never on kernel outputs."""
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def oracle_layer(wl, layer, xh, router_w, router_b, bits, k=None):
    k = wl.top_k if k is None else k
    ids, gates, z = O.route(xh, router_w, router_b, k)
    oracle_pool.prefetch(wl.name, layer, np.unique(ids), bits)
    _, _, y = O.moe_layer(xh, router_w, router_b, k, oracle_experts(wl, layer, bits), bits)
    return ids, gates, z, y


def check_routing(ids_g, w_g, off_g, prs_g, ids_o, gates_o, E):
    assert np.array_equal(ids_g.cpu().numpy(), ids_o), "routing ids differ"
    assert np.max(np.abs(w_g.cpu().numpy() - gates_o)) <= TOL * 1e-2
    if off_g is not None:
        off_o, prs_o = O.bucket_pairs(ids_o, E)
        assert np.array_equal(off_g.cpu().numpy(), off_o), "bucket offsets differ"
        assert np.array_equal(prs_g.cpu().numpy(), prs_o), "bucket pairs differ"


# ------------------------------------------------------------- tiny workload

@pytest.fixture(scope="module")
def tiny(q):
    wl = mi.WORKLOADS["tiny"]
    layers, ex, rt = device_layers(wl)
    return wl, layers, ex, rt


def test_generator_twin_tiny(tiny):
    _say("generator twin, tiny, all experts")
    wl, layers, ex, rt = tiny
    for e in range(wl.n_experts):
        for name, t in (("gate", mi.GATE), ("up", mi.UP), ("down", mi.DOWN)):
            qh, sh = mi.expert_tensor_host(wl, 0, t, e)
            assert np.array_equal(ex[name + "_q"][0, e].cpu().numpy().view(np.uint32), qh)
            assert np.array_equal(ex[name + "_s"][0, e].cpu().numpy().view(np.uint16), sh)


def test_route_and_buckets_tiny(q, tiny):
    _say("moe_route tiny T=8 k=2 E=16")
    wl, layers, ex, rt = tiny
    router, experts = layers[0]
    x = mi.activations_host(wl)
    ids, w, off, prs = gpu_route(q, router, torch.from_numpy(x).cuda())
    wh, bh = mi.router_host(wl, 0)
    ids_o, gates_o, _ = O.route(x, wh, bh, wl.top_k)
    check_routing(ids, w, off, prs, ids_o, gates_o, wl.n_experts)


@pytest.mark.parametrize("k", [1, 5, 16])
def test_route_k_range_tiny(q, tiny, k):
    _say(f"moe_route tiny k={k}")
    wl, layers, ex, rt = tiny
    router0, _ = layers[0]
    router = q.Router(router0.w, None, k)
    x = mi.activations_host(wl)
    ids, w, off, prs = gpu_route(q, router, torch.from_numpy(x).cuda())
    wh, _ = mi.router_host(wl, 0)
    ids_o, gates_o, _ = O.route(x, wh, None, k)
    check_routing(ids, w, off, prs, ids_o, gates_o, wl.n_experts)


def test_route_ties(q):
    _say("moe_route constructed ties: duplicated columns, all-zero router")
    rng = np.random.default_rng(0)
    D, E, T, K = 64, 32, 6, 8
    w = (0.02 * rng.standard_normal((D, E))).astype(np.float32)
    w[:, 9] = w[:, 3]
    w[:, 21] = w[:, 3]
    x = rng.standard_normal((T, D)).astype(np.float32)
    for wmat in (w, np.zeros_like(w)):
        router = q.Router(torch.from_numpy(np.ascontiguousarray(wmat.T)).cuda(), None, K)
        ids, g, off, prs = gpu_route(q, router, torch.from_numpy(x).cuda())
        ids_o, gates_o, _ = O.route(x, wmat, None, K)
        check_routing(ids, g, off, prs, ids_o, gates_o, E)


def test_decode_tiny(q, tiny):
    _say("moe_ffn_decode tiny T=8")
    wl, layers, ex, rt = tiny
    router, experts = layers[0]
    x = mi.activations_host(wl)
    wh, bh = mi.router_host(wl, 0)
    ids_o, gates_o, _, y_o = oracle_layer(wl, 0, x, wh, bh, wl.bits)
    y = gpu_decode(q, experts, torch.from_numpy(x).cuda(), torch.from_numpy(ids_o).cuda(),
                   torch.from_numpy(gates_o).cuda())
    err = row_rel_err(y.cpu().numpy(), y_o)
    print(f"tiny decode row_rel_err={err:.2e}")
    assert err <= TOL


def test_prefill_tiny(q, tiny):
    _say("moe_ffn_prefill tiny T=8")
    wl, layers, ex, rt = tiny
    router, experts = layers[0]
    x = mi.activations_host(wl)
    wh, bh = mi.router_host(wl, 0)
    ids_o, gates_o, _, y_o = oracle_layer(wl, 0, x, wh, bh, wl.bits)
    off_o, prs_o = O.bucket_pairs(ids_o, wl.n_experts)
    y = gpu_prefill(q, experts, torch.from_numpy(x).cuda(), torch.from_numpy(gates_o).cuda(),
                    torch.from_numpy(off_o).cuda(), torch.from_numpy(prs_o).cuda())
    err = row_rel_err(y.cpu().numpy(), y_o)
    print(f"tiny prefill row_rel_err={err:.2e}")
    assert err <= TOL


# ------------------------------------------------------------- full shapes, one layer

@pytest.fixture(scope="module")
def full1(q):
    wl = mi.WORKLOADS["decode_1layer"]
    layers, ex, rt = device_layers(wl, 1)
    yield wl, layers, ex, rt
    del layers, ex, rt
    torch.cuda.empty_cache()


def test_generator_twin_full_sampled(full1):
    _say("generator twin, full shapes, sampled experts")
    wl, layers, ex, rt = full1
    for e in (0, 1, 255, 511):
        for name, t in (("gate", mi.GATE), ("down", mi.DOWN)):
            qh, sh = mi.expert_tensor_host(wl, 0, t, e)
            assert np.array_equal(ex[name + "_q"][0, e].cpu().numpy().view(np.uint32), qh)
            assert np.array_equal(ex[name + "_s"][0, e].cpu().numpy().view(np.uint16), sh)
    import moe_inputs.gpu as g
    ex3 = g.expert_tensors(wl, 1, 3)
    for e in (3, 400):
        qh, sh = mi.expert_tensor_host(wl, 0, mi.UP, e, bits=3)
        assert np.array_equal(ex3["up_q"][0, e].cpu().numpy().view(np.uint32), qh)
        assert np.array_equal(ex3["up_s"][0, e].cpu().numpy().view(np.uint16), sh)


def test_decode_single_layer_bs1(q, full1):
    _say("route + decode, single layer, T=1 bf16, 512 experts top-10")
    wl, layers, ex, rt = full1
    router, experts = layers[0]
    x = mi.activations_host(wl)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    ids, w, off, prs = gpu_route(q, router, xd)
    wh, bh = mi.router_host(wl, 0)
    ids_o, gates_o, _, y_o = oracle_layer(wl, 0, x, wh, bh, 2)
    check_routing(ids, w, off, prs, ids_o, gates_o, wl.n_experts)
    y = gpu_decode(q, experts, xd, ids, w)
    err = row_rel_err(y.cpu().numpy(), y_o)
    print(f"decode T=1 row_rel_err={err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("T", [2, 8])
def test_decode_single_layer_batches(q, full1, T):
    _say(f"route + decode, single layer, T={T} fp32")
    wl, layers, ex, rt = full1
    router, experts = layers[0]
    x = mi.activations_host(mi.WORKLOADS["decode_48layer"], T, stream=7)
    xd = torch.from_numpy(x).cuda()
    ids, w, off, prs = gpu_route(q, router, xd)
    wh, bh = mi.router_host(wl, 0)
    ids_o, gates_o, _, y_o = oracle_layer(wl, 0, x, wh, bh, 2)
    check_routing(ids, w, off, prs, ids_o, gates_o, wl.n_experts)
    y = gpu_decode(q, experts, xd, ids, w)
    err = row_rel_err(y.cpu().numpy(), y_o)
    print(f"decode T={T} row_rel_err={err:.2e}")
    assert err <= TOL
    # batch invariance: each token alone gives the same bits
    for t in range(T):
        i1, w1, _, _ = gpu_route(q, router, xd[t:t + 1].contiguous(), buckets=False)
        y1 = gpu_decode(q, experts, xd[t:t + 1].contiguous(), i1, w1)
        assert torch.equal(i1[0], ids[t]) and torch.equal(w1[0], w[t])
        assert torch.equal(y1[0], y[t])


def test_decode_top64(q, full1):
    _say("route + decode, single layer, top-64 (largest k), T=2")
    wl, layers, ex, rt = full1
    router0, experts = layers[0]
    router = q.Router(router0.w, router0.bias, 64)
    x = mi.activations_host(mi.WORKLOADS["decode_48layer"], 2, stream=9)
    xd = torch.from_numpy(x).cuda()
    ids, w, off, prs = gpu_route(q, router, xd)
    wh, bh = mi.router_host(wl, 0)
    ids_o, gates_o, _, y_o = oracle_layer(wl, 0, x, wh, bh, 2, k=64)
    check_routing(ids, w, off, prs, ids_o, gates_o, wl.n_experts)
    y = gpu_decode(q, experts, xd, ids, w)
    assert row_rel_err(y.cpu().numpy(), y_o) <= TOL


def test_decode_single_layer_3bit_T4(q, full1):
    _say("decode, single layer, 3-bit experts, T=4")
    wl, layers, ex, rt = full1
    import moe_inputs.gpu as g
    ex3 = g.expert_tensors(wl, 1, 3)
    experts3 = q.Experts(ex3["gate_q"][0], ex3["up_q"][0], ex3["down_q"][0],
                         ex3["gate_s"][0], ex3["up_s"][0], ex3["down_s"][0], 3)
    router, _ = layers[0]
    wl5 = mi.WORKLOADS["verify4_3bit"]
    x = mi.activations_host(wl5)
    xd = torch.from_numpy(x).cuda()
    wh, bh = mi.router_host(wl, 0)
    ids_o, gates_o, _, y_o = oracle_layer(wl5, 0, x, wh, bh, 3)
    ids, w, _, _ = gpu_route(q, router, xd, buckets=False)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    y = gpu_decode(q, experts3, xd, ids, w)
    err = row_rel_err(y.cpu().numpy(), y_o)
    print(f"decode 3-bit T=4 row_rel_err={err:.2e}")
    assert err <= TOL
    for t in range(4):
        y1 = gpu_decode(q, experts3, xd[t:t + 1].contiguous(), ids[t:t + 1].contiguous(), w[t:t + 1].contiguous())
        assert torch.equal(y1[0], y[t])


def test_prefill_ragged_small(q, full1):
    _say("route + prefill, full shapes, T=37 (ragged tiles), and decode equivalence")
    wl, layers, ex, rt = full1
    router, experts = layers[0]
    x = mi.activations_host(mi.WORKLOADS["prefill_8192"], 37)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    ids, w, off, prs = gpu_route(q, router, xd)
    wh, bh = mi.router_host(wl, 0)
    ids_o, gates_o, _, y_o = oracle_layer(wl, 0, x, wh, bh, 2)
    check_routing(ids, w, off, prs, ids_o, gates_o, wl.n_experts)
    y = gpu_prefill(q, experts, xd, w, off, prs)
    err = row_rel_err(y.cpu().numpy(), y_o)
    print(f"prefill T=37 row_rel_err={err:.2e}")
    assert err <= TOL


def test_prefill_one_hot_expert_set(q, full1):
    _say("prefill, T=300, router forcing every token onto experts 0..9")
    wl, layers, ex, rt = full1
    _, experts = layers[0]
    D, E, K = wl.d_model, wl.n_experts, wl.top_k
    wmat = np.zeros((D, E), np.float32)
    bias = np.full(E, -10.0, np.float32)
    bias[:K] = np.linspace(1.0, 0.1, K, dtype=np.float32)
    router = q.Router(torch.from_numpy(np.ascontiguousarray(wmat.T)).cuda(), torch.from_numpy(bias).cuda(), K)
    x = mi.activations_host(mi.WORKLOADS["prefill_8192"], 300, stream=3)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    ids, w, off, prs = gpu_route(q, router, xd)
    ids_o, gates_o, _, y_o = oracle_layer(wl, 0, x, wmat, bias, 2)
    check_routing(ids, w, off, prs, ids_o, gates_o, E)
    assert np.all(np.diff(off.cpu().numpy())[:K] == 300)
    y = gpu_prefill(q, experts, xd, w, off, prs)
    assert row_rel_err(y.cpu().numpy(), y_o) <= TOL


def test_prefill_chunk_8192(q, full1):
    _say("route + buckets + prefill, 8,192-token chunk: every row against the oracle")
    wl = mi.WORKLOADS["prefill_8192"]
    _, layers, _, _ = full1
    router, experts = layers[0]
    x = mi.activations_host(wl)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    ids, w, off, prs = gpu_route(q, router, xd)
    y = gpu_prefill(q, experts, xd, w, off, prs)
    y2 = gpu_prefill(q, experts, xd, w, off, prs)
    assert torch.equal(y, y2), "prefill is not deterministic"
    wh, bh = mi.router_host(wl, 0)
    ids_o, gates_o, y_o = O.moe_layer(x, wh, bh, wl.top_k, oracle_experts(wl, 0, 2), 2,
                                      prepare=lambda e: oracle_pool.prefetch(wl.name, 0, e, 2))
    check_routing(ids, w, off, prs, ids_o, gates_o, wl.n_experts)
    load = np.bincount(ids_o.reshape(-1), minlength=wl.n_experts)
    print(f"bucket load: max {load.max()} mean {load.mean():.1f} non-empty {(load > 0).sum()}")
    yg = y.cpu().numpy()
    err = row_rel_err(yg, y_o)
    print(f"prefill 8192, all rows: row_rel_err={err:.2e} floored elementwise {floored_rel_err(yg, y_o):.2e}")
    assert err <= TOL


def test_prefill_chunk_256_experts(q):
    _say("route + buckets + prefill, 2,048 tokens through one 256-expert layer: every row against the oracle")
    wl = mi.WORKLOADS["coder_256"]
    layers, ex, rt = device_layers(wl, 1)
    router, experts = layers[0]
    x = mi.activations_host(wl, 2048, stream=5)
    xd = torch.from_numpy(x).cuda()
    ids, w, off, prs = gpu_route(q, router, xd)
    y = gpu_prefill(q, experts, xd, w, off, prs)
    wh, bh = mi.router_host(wl, 0)
    ids_o, gates_o, y_o = O.moe_layer(x, wh, bh, wl.top_k, oracle_experts(wl, 0, 2), 2,
                                      prepare=lambda e: oracle_pool.prefetch(wl.name, 0, e, 2))
    check_routing(ids, w, off, prs, ids_o, gates_o, wl.n_experts)
    load = np.bincount(ids_o.reshape(-1), minlength=wl.n_experts)
    print(f"bucket load: max {load.max()} mean {load.mean():.1f} non-empty {(load > 0).sum()}")
    err = row_rel_err(y.cpu().numpy(), y_o)
    print(f"prefill, 256 experts, 2048 tokens: row_rel_err={err:.2e}")
    assert err <= TOL
    del layers, ex, rt
    torch.cuda.empty_cache()


def test_route_logits_bit_exact_8192(q, full1):
    _say("moe_route, 8,192 tokens: fp64 logits bit for bit against the ascending-d definition (sampled tokens)")
    wl = mi.WORKLOADS["prefill_8192"]
    _, layers, _, _ = full1
    router, _ = layers[0]
    T, K, E, D = wl.n_tokens, wl.top_k, wl.n_experts, wl.d_model
    x = mi.activations_host(wl)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    ws = q.workspace(q.MOE_OP_ROUTE, T, D, 0, E, K)
    q.moe_route(router, xd, ids, w, None, None, ws)
    torch.cuda.synchronize()
    # the route workspace starts with the [T][E] fp64 logits (route_ws_layout)
    z = ws[: T * E * 8].view(torch.float64).reshape(T, E).cpu().numpy()
    wh, bh = mi.router_host(wl, 0)
    sample = np.array([0, 1, 2, 3, 15, 16, 17, 127, 128, 1000, 4095, 4096, 6001, 8190, 8191])
    z_o = O.router_logits(x[sample], wh, bh)
    assert np.array_equal(z[sample], z_o), f"{np.mean(z[sample] != z_o):.3f} of the sampled logits differ"


@pytest.mark.parametrize("T", [9, 63, 64, 65, 129])
def test_route_gemm_tile_boundaries(q, full1, T):
    """The matrix-core router GEMM works on 64-token x 64-expert tiles: token
    counts just below, at and above a tile edge (and 9, the smallest count
    that takes this path) give the oracle's ids, gates and buckets, and every
    fp64 logit of every token bit for bit, for bf16 and fp32 activations."""
    _say(f"moe_route T={T}: 64-token router GEMM tiles, bf16 and fp32 inputs")
    wl = mi.WORKLOADS["prefill_8192"]
    _, layers, _, _ = full1
    router, _ = layers[0]
    K, E, D = wl.top_k, wl.n_experts, wl.d_model
    wh, bh = mi.router_host(wl, 0)
    xb = mi.activations_host(wl, T)
    xf = xb.astype(np.uint32) << 16
    xf = xf.view(np.float32)                   # the same values as fp32
    for x_host, x_dev in ((xb, torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)),
                          (xf, torch.from_numpy(np.ascontiguousarray(xf)).cuda())):
        ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
        w = torch.empty((T, K), dtype=torch.float32, device="cuda")
        off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        prs = torch.empty(T * K, dtype=torch.int32, device="cuda")
        ws = q.workspace(q.MOE_OP_ROUTE, T, D, 0, E, K)
        q.moe_route(router, x_dev, ids, w, off, prs, ws)
        torch.cuda.synchronize()
        z = ws[: T * E * 8].view(torch.float64).reshape(T, E).cpu().numpy()
        z_o = O.router_logits(x_host, wh, bh)
        assert np.array_equal(z, z_o), f"{np.mean(z != z_o):.4f} of the logits differ"
        ids_o, gates_o, _ = O.route(x_host, wh, bh, K)
        check_routing(ids, w, off, prs, ids_o, gates_o, E)


@pytest.mark.parametrize("E", [16, 100, 200])
def test_route_gemm_ragged_experts(q, E):
    """The router GEMM's last 64-expert tile partly empty (and a bias): 70
    tokens (two token tiles, the second ragged) on seeded random routers whose
    expert count is not a multiple of 64; logits bit for bit, ids, gates and
    buckets against the oracle."""
    _say(f"moe_route T=70 E={E}: ragged expert tiles of the router GEMM, with bias")
    rng = np.random.default_rng(1000 + E)
    D, T, K = 256, 70, min(8, E)
    w = (0.02 * rng.standard_normal((D, E))).astype(np.float32)
    b = (0.01 * rng.standard_normal(E)).astype(np.float32)
    x = rng.standard_normal((T, D)).astype(np.float32)
    router = q.Router(torch.from_numpy(np.ascontiguousarray(w.T)).cuda(), torch.from_numpy(b).cuda(), K)
    ids, g, off, prs = gpu_route(q, router, torch.from_numpy(x).cuda())
    ws = q.workspace(q.MOE_OP_ROUTE, T, D, 0, E, K)
    q.moe_route(router, torch.from_numpy(x).cuda(), torch.empty_like(ids), torch.empty_like(g), None, None, ws)
    torch.cuda.synchronize()
    z = ws[: T * E * 8].view(torch.float64).reshape(T, E).cpu().numpy()
    assert np.array_equal(z, O.router_logits(x, w, b)), "router logits differ"
    ids_o, gates_o, _ = O.route(x, w, b, K)
    check_routing(ids, g, off, prs, ids_o, gates_o, E)


# ------------------------------------------------------------- errors

def test_abi_errors(q, tiny):
    _say("C ABI argument validation")
    import ctypes
    wl, layers, ex, rt = tiny
    router, experts = layers[0]
    lib = q.library
    x = torch.zeros((4, wl.d_model), device="cuda")
    ids = torch.zeros((4, 2), dtype=torch.int32, device="cuda")
    w = torch.zeros((4, 2), device="cuda")
    y = torch.zeros((4, wl.d_model), device="cuda")
    ws = q.workspace(q.MOE_OP_ROUTE, 4, wl.d_model, 0, wl.n_experts, 2)
    P = ctypes.c_void_p
    s = P(torch.cuda.current_stream().cuda_stream)
    rc = ctypes.byref(router._c)
    assert lib.moe_route(None, P(x.data_ptr()), 0, 4, P(ids.data_ptr()), P(w.data_ptr()), None, None,
                         P(ws.data_ptr()), ws.numel(), s) == q.MOE_ERR_ARG
    assert lib.moe_route(rc, P(x.data_ptr()), 0, 0, P(ids.data_ptr()), P(w.data_ptr()), None, None,
                         P(ws.data_ptr()), ws.numel(), s) == q.MOE_ERR_ARG
    assert lib.moe_route(rc, P(x.data_ptr()), 7, 4, P(ids.data_ptr()), P(w.data_ptr()), None, None,
                         P(ws.data_ptr()), ws.numel(), s) == q.MOE_ERR_ARG
    assert lib.moe_route(rc, P(x.data_ptr()), 0, 4, P(ids.data_ptr()), P(w.data_ptr()), None, None,
                         P(ws.data_ptr()), 16, s) == q.MOE_ERR_WORKSPACE
    assert lib.moe_route(rc, P(x.data_ptr()), 0, 4, P(ids.data_ptr()), P(w.data_ptr()), None, None,
                         P(ws.data_ptr() + 4), ws.numel() - 4, s) == q.MOE_ERR_WORKSPACE
    bad = q.Router(router.w, None, 17)       # k > E
    assert lib.moe_route(ctypes.byref(bad._c), P(x.data_ptr()), 0, 4, P(ids.data_ptr()), P(w.data_ptr()),
                         None, None, P(ws.data_ptr()), ws.numel(), s) == q.MOE_ERR_UNSUPPORTED
    wsd = q.workspace(q.MOE_OP_DECODE, 4, wl.d_model, wl.d_ff, wl.n_experts, 2)
    ec = ctypes.byref(experts._c)
    assert lib.moe_ffn_decode(ec, P(x.data_ptr()), 0, 9, P(ids.data_ptr()), P(w.data_ptr()), 2,
                              P(y.data_ptr()), P(wsd.data_ptr()), wsd.numel(), s) == q.MOE_ERR_UNSUPPORTED
    assert lib.moe_ffn_decode(ec, P(x.data_ptr()), 0, 4, None, P(w.data_ptr()), 2,
                              P(y.data_ptr()), P(wsd.data_ptr()), wsd.numel(), s) == q.MOE_ERR_ARG
    ex3 = q.Experts(experts.gate_q, experts.up_q, experts.down_q, experts.gate_s, experts.up_s,
                    experts.down_s, 3)
    wsp = q.workspace(q.MOE_OP_PREFILL, 4, wl.d_model, wl.d_ff, wl.n_experts, 2)
    assert lib.moe_ffn_prefill(ctypes.byref(ex3._c), P(x.data_ptr()), 0, 4, P(w.data_ptr()), 2,
                               P(ids.data_ptr()), P(ids.data_ptr()), P(y.data_ptr()), P(wsp.data_ptr()),
                               wsp.numel(), s) == q.MOE_ERR_UNSUPPORTED
    with pytest.raises(q.MoeError):
        q.moe_residual_rmsnorm(y, None, y[:, :0], eps=-1.0)
    torch.cuda.synchronize()

"""GPU parity of the int8-activation prefill (moe_quantize_q8 and
moe_ffn_prefill_q8, through the C ABI) against the int8 oracle variant on
the same seeded inputs.

- Q8 codes and scales: bit for bit (both sides take the rounding decision in
  fp32 with correctly rounded divisions).
- Expert FFN: within TOL (max over rows of max|err| / max|ref|).  The x
  codes are identical on both sides; the rest differs by fp32 accumulation
  order (~1e-6 of a row's largest value) and by h: the kernel's h (fp32
  accumulation, fast exp) and the oracle's (fp64, rounded to fp32) can fall
  on different sides of a rounding tie of their Q8 grid, which moves one
  term of one down-projection dot product by one grid step (a few 1e-4 of
  the row maximum at most; such flips are rare).
The error against the exact-weight oracle (int8 rounding of x and h, ~1e-2)
is printed for information; the oracle pins bound it.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import moe_inputs as mi
import oracle.moe_oracle as O
import oracle.moe_oracle_q8 as Q
from helpers import TOL, device_layers, oracle_experts, row_rel_err
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


@pytest.fixture(scope="module")
def full1(q):
    wl = mi.WORKLOADS["decode_1layer"]
    layers, ex, rt = device_layers(wl, 1)
    yield wl, layers
    del layers, ex, rt
    torch.cuda.empty_cache()


def gpu_quantize(q, x):
    T, D = x.shape
    qq = torch.empty((T, D), dtype=torch.int8, device="cuda")
    d = torch.empty((T, D // 32), dtype=torch.float32, device="cuda")
    q.moe_quantize_q8(x, qq, d)
    torch.cuda.synchronize()
    return qq.cpu().numpy(), d.cpu().numpy()


def gpu_route(q, router, x):
    T, K, E = x.shape[0], router.top_k, router.n_experts
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    prs = torch.empty(T * K, dtype=torch.int32, device="cuda")
    q.moe_route(router, x, ids, w, off, prs, q.workspace(q.MOE_OP_ROUTE, T, router.d_model, 0, E, K))
    torch.cuda.synchronize()
    return ids, w, off, prs


def gpu_prefill_q8(q, ex, x, w, off, prs):
    T, K = w.shape
    y = torch.empty((T, ex.d_model), dtype=torch.float32, device="cuda")
    ws = q.workspace(q.MOE_OP_PREFILL_Q8, T, ex.d_model, ex.d_ff, ex.n_experts, K)
    q.moe_ffn_prefill_q8(ex, x, w, off, prs, y, ws)
    torch.cuda.synchronize()
    return y


def _bf16(x):
    return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)


# ----------------------------------------------------------------- Q8 codes

def test_quantize_q8_bit_exact(q):
    _say("moe_quantize_q8: fp32 rows over 60 binades, golden blocks, zero and tiny blocks, bf16")
    rng = np.random.default_rng(40)
    x = (rng.standard_normal((300, 512)) * np.exp2(rng.integers(-30, 30, size=(300, 1)))).astype(np.float32)
    # rows built on exact grids so that many products land on rounding ties
    n = rng.integers(-254, 255, size=(40, 512)).astype(np.float32) / 2
    n[:, ::32] = 127.0
    x[:40] = n * np.float32(2.0 ** -5)
    x[40, :] = 0.0                                         # zero blocks
    x[41, :] = np.float32(2.0 ** -120)                     # below the live threshold
    x[42, :32] = np.float32(2.0 ** -112)                   # exactly at it
    x[43] = -np.abs(x[43])
    for dt in ("f32", "bf16"):
        if dt == "f32":
            xg, xo = torch.from_numpy(x).cuda(), x
        else:
            xo = (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
            xg = _bf16(xo)
        qg, dg = gpu_quantize(q, xg)
        qo, do = Q.quantize_q8(O.as_f32_activations(xo))
        assert np.array_equal(dg.view(np.uint32), do.view(np.uint32)), f"{dt}: scales differ"
        assert np.array_equal(qg, qo), f"{dt}: codes differ in {(qg != qo).sum()} places"


# ----------------------------------------------------------------- expert FFN

def _check(yg, yo, exact=None):
    err = row_rel_err(yg, yo)
    msg = f"int8 prefill: row_rel_err vs int8 oracle {err:.2e}"
    if exact is not None:
        msg += f", vs exact-weight oracle {row_rel_err(yg, exact):.2e}"
    print(msg)
    assert err <= TOL


def test_prefill_q8_tiny(q):
    _say("moe_ffn_prefill_q8 tiny T=8 (16 experts, d_model 256, d_ff 128)")
    wl = mi.WORKLOADS["tiny"]
    layers, ex, rt = device_layers(wl)
    _, experts = layers[0]
    x = mi.activations_host(wl)
    wh, bh = mi.router_host(wl, 0)
    ids, gates, _ = O.route(x, wh, bh, wl.top_k)
    off, prs = O.bucket_pairs(ids, wl.n_experts)
    oracle_pool.prefetch(wl.name, 0, np.unique(ids), wl.bits)
    y = gpu_prefill_q8(q, experts, torch.from_numpy(x).cuda(), torch.from_numpy(gates).cuda(),
                       torch.from_numpy(off).cuda(), torch.from_numpy(prs).cuda())
    yo = Q.moe_ffn_q8_buckets(x, gates, wl.top_k, off, prs, oracle_experts(wl, 0, 2))
    _check(y.cpu().numpy(), yo)


def test_prefill_q8_ragged(q, full1):
    _say("route + moe_ffn_prefill_q8, full shapes, T=37 (ragged tiles)")
    wl, layers = full1
    router, experts = layers[0]
    x = mi.activations_host(mi.WORKLOADS["prefill_8192"], 37)
    ids, w, off, prs = gpu_route(q, router, _bf16(x))
    wh, bh = mi.router_host(wl, 0)
    ids_o, gates_o, _ = O.route(x, wh, bh, wl.top_k)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    off_o, prs_o = O.bucket_pairs(ids_o, wl.n_experts)
    assert np.array_equal(off.cpu().numpy(), off_o) and np.array_equal(prs.cpu().numpy(), prs_o)
    oracle_pool.prefetch(wl.name, 0, np.unique(ids_o), 2)
    y = gpu_prefill_q8(q, experts, _bf16(x), w, off, prs)
    _, _, y_exact = O.moe_layer(x, wh, bh, wl.top_k, oracle_experts(wl, 0, 2), 2)
    yo = Q.moe_ffn_q8_buckets(x, gates_o, wl.top_k, off_o, prs_o, oracle_experts(wl, 0, 2))
    _check(y.cpu().numpy(), yo, exact=y_exact)


def test_prefill_q8_one_hot_expert_set(q, full1):
    _say("moe_ffn_prefill_q8, T=300 all on experts 0..9 (300-row buckets: 2 full tiles + 44 rows)")
    wl, layers = full1
    _, experts = layers[0]
    D, E, K = wl.d_model, wl.n_experts, wl.top_k
    x = mi.activations_host(mi.WORKLOADS["prefill_8192"], 300, stream=3)
    ids = np.tile(np.arange(K, dtype=np.int32), (300, 1))
    rng = np.random.default_rng(41)
    g = rng.random((300, K)).astype(np.float32)
    gates = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
    off, prs = O.bucket_pairs(ids, E)
    oracle_pool.prefetch(wl.name, 0, np.arange(K), 2)
    y = gpu_prefill_q8(q, experts, _bf16(x), torch.from_numpy(gates).cuda(), torch.from_numpy(off).cuda(),
                       torch.from_numpy(prs).cuda())
    _check(y.cpu().numpy(), Q.moe_ffn_q8_buckets(x, gates, K, off, prs, oracle_experts(wl, 0, 2)))


def test_prefill_q8_chunk_8192_sampled(q, full1):
    _say("route + moe_ffn_prefill_q8, 8,192-token chunk, 128 sampled rows against the oracle")
    wl = mi.WORKLOADS["prefill_8192"]
    _, layers = full1
    router, experts = layers[0]
    x = mi.activations_host(wl)
    xd = _bf16(x)
    ids, w, off, prs = gpu_route(q, router, xd)
    y = gpu_prefill_q8(q, experts, xd, w, off, prs)
    y2 = gpu_prefill_q8(q, experts, xd, w, off, prs)
    assert torch.equal(y, y2), "int8 prefill is not deterministic"
    rows = np.sort(np.random.default_rng(42).choice(wl.n_tokens, 128, replace=False))
    rows = np.unique(np.concatenate([rows, [0, wl.n_tokens - 1]]))
    _sampled(wl, x, rows, ids, y)


def _sampled(wl, x, rows, ids_gpu, y_gpu):
    """Route the sampled tokens on the CPU (routing is per token), check the
    kernel's ids for them, and compare their rows with the per-token form of
    the int8 oracle."""
    wh, bh = mi.router_host(wl, 0)
    ids_o, gates_o, _ = O.route(x[rows], wh, bh, wl.top_k)
    assert np.array_equal(ids_gpu.cpu().numpy()[rows], ids_o)
    oracle_pool.prefetch(wl.name, 0, np.unique(ids_o), 2)
    yo = Q.moe_layer_q8(x[rows], ids_o, gates_o, oracle_experts(wl, 0, 2))
    _check(y_gpu.cpu().numpy()[rows], yo)


def test_prefill_q8_256_experts_sampled(q):
    _say("route + moe_ffn_prefill_q8, 2,048 fp32 tokens through one 256-expert layer, 128 sampled rows")
    wl = mi.WORKLOADS["coder_256"]
    layers, ex, rt = device_layers(wl, 1)
    router, experts = layers[0]
    x = mi.activations_host(wl, 2048, stream=5)
    ids, w, off, prs = gpu_route(q, router, torch.from_numpy(x).cuda())
    y = gpu_prefill_q8(q, experts, torch.from_numpy(x).cuda(), w, off, prs)
    rows = np.sort(np.random.default_rng(43).choice(2048, 128, replace=False))
    _sampled(wl, x, rows, ids, y)
    del layers, ex, rt
    torch.cuda.empty_cache()


def test_prefill_q8_abi_errors(q, full1):
    _say("moe_ffn_prefill_q8 / moe_quantize_q8 argument errors")
    wl, layers = full1
    _, experts = layers[0]
    x = torch.zeros((4, wl.d_model), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((4, wl.top_k), device="cuda")
    off = torch.zeros(wl.n_experts + 1, dtype=torch.int32, device="cuda")
    prs = torch.zeros(4 * wl.top_k, dtype=torch.int32, device="cuda")
    y = torch.empty((4, wl.d_model), device="cuda")
    ws = q.workspace(q.MOE_OP_PREFILL_Q8, 4, wl.d_model, wl.d_ff, wl.n_experts, wl.top_k)
    with pytest.raises(q.MoeError) as e:
        q.moe_ffn_prefill_q8(experts, x, w, off, prs, y, ws[:-256])
    assert e.value.status == q.MOE_ERR_WORKSPACE
    qq = torch.empty((4, 48), dtype=torch.int8, device="cuda")
    d = torch.empty((4, 2), device="cuda")
    with pytest.raises(q.MoeError) as e:
        q.moe_quantize_q8(torch.zeros((4, 48), device="cuda"), qq, d)
    assert e.value.status == q.MOE_ERR_UNSUPPORTED

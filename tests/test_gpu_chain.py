"""Chained decode through the layer-by-layer entry points: 48 layers of
moe_route + moe_ffn_decode + moe_residual_rmsnorm with the residual stream
and RMSNorm between layers, compared token by token and layer by layer with
the oracle's free-running chain (chain_walk).  Batch invariance (4 tokens
together vs each alone) is checked bitwise, and a HIP graph of the 48 layers
replays bit-identically."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import moe_inputs as mi
from chain_walk import full_depth_streams, stream_tokens, walk
from helpers import device_layers

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def q(need_gpu):
    import quantized_moe_expert_lds_amd as q
    return q


class ChainRunner:
    """Runs route -> decode -> residual+RMSNorm for every layer on one stream."""

    def __init__(self, q, layers, T):
        self.q, self.layers, self.T = q, layers, T
        r0, e0 = layers[0]
        D, F, E, K = e0.d_model, e0.d_ff, e0.n_experts, r0.top_k
        self.h = torch.empty((T, D), device="cuda")
        self.u = torch.empty((T, D), device="cuda")
        self.y = torch.empty((T, D), device="cuda")
        self.ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
        self.w = torch.empty((T, K), device="cuda")
        self.ws_r = q.workspace(q.MOE_OP_ROUTE, T, D, F, E, K)
        self.ws_d = q.workspace(q.MOE_OP_DECODE, T, D, F, E, K)

    def run(self, x, record=False):
        """Returns (ids, gates, h after each layer) stacked over the layers
        when record is set."""
        q = self.q
        self.h.copy_(x)
        ids, gates, hs = [], [], []
        for l, (router, experts) in enumerate(self.layers):
            inp = self.h if l == 0 else self.u
            q.moe_route(router, inp, self.ids, self.w, None, None, self.ws_r)
            q.moe_ffn_decode(experts, inp, self.ids, self.w, self.y, self.ws_d)
            q.moe_residual_rmsnorm(self.h, self.y, self.u, 1e-6)
            if record:
                ids.append(self.ids.clone())
                gates.append(self.w.clone())
                hs.append(self.h.clone())
        if not record:
            return None
        return (torch.stack(ids).cpu().numpy(), torch.stack(gates).cpu().numpy(), torch.stack(hs).cpu().numpy())


def test_chain_decode_48_layers(q):
    _say("48-layer decode chain, T=1, 2-bit, fp32 residual stream")
    wl = mi.WORKLOADS["decode_48layer"]
    layers, ex, rt = device_layers(wl)
    x = mi.activations_host(wl)
    runner = ChainRunner(q, layers, 1)
    ids, gates, hl = runner.run(torch.from_numpy(x).cuda(), record=True)
    torch.cuda.synchronize()
    h_gpu = runner.h.cpu().numpy()
    # second run is bit-identical (deterministic kernels, self-resetting counters)
    runner.run(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(runner.h.cpu().numpy(), h_gpu)
    walk(wl, 2, x, ids, gates, hl, h_gpu, label="layer calls, stream 0")
    s = full_depth_streams(wl.name, 1)[0]
    xs = stream_tokens(wl, [s])
    o = runner.run(torch.from_numpy(xs).cuda(), record=True)
    torch.cuda.synchronize()
    walk(wl, 2, xs, *o, runner.h.cpu().numpy(), full=[0], label=f"layer calls, stream {s}")
    # the same 48 layers captured once in a graph and replayed
    g = torch.cuda.CUDAGraph()
    xd = torch.from_numpy(x).cuda()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        runner.run(xd)          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        runner.run(xd)
    for rep in range(3):
        runner.h.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(runner.h.cpu().numpy(), h_gpu), f"graph replay {rep} differs"
        _ = (torch.ones(1024, device="cuda") * rep).sum().item()    # eager work between replays
    del layers, ex, rt, g
    torch.cuda.empty_cache()


def test_chain_verify_4_tokens_3bit(q):
    _say("48-layer verify chain, T=4, 3-bit experts; batch invariance vs 4 x T=1; full-depth tokens")
    wl = mi.WORKLOADS["verify4_3bit"]
    layers, ex, rt = device_layers(wl)
    xs = stream_tokens(wl, full_depth_streams(wl.name, 4))
    xd = torch.from_numpy(xs).cuda()
    runner = ChainRunner(q, layers, 4)
    ids, gates, hl = runner.run(xd, record=True)
    torch.cuda.synchronize()
    h_gpu = runner.h.cpu().numpy()
    one = ChainRunner(q, layers, 1)
    for t in range(4):
        i1, g1, hl1 = one.run(xd[t:t + 1], record=True)
        torch.cuda.synchronize()
        assert np.array_equal(one.h.cpu().numpy()[0], h_gpu[t]), f"token {t}: T=4 differs from T=1"
        assert np.array_equal(i1[:, 0], ids[:, t]) and np.array_equal(hl1[:, 0], hl[:, t])
    uniq = [len(np.unique(ids[l])) for l in range(ids.shape[0])]
    print(f"distinct experts per layer: mean {np.mean(uniq):.1f} min {min(uniq)} max {max(uniq)}")
    matched, _ = walk(wl, 3, xs, ids, gates, hl, h_gpu, full=range(4), label="layer calls, 3-bit T=4")
    assert matched == [48] * 4
    del layers, ex, rt
    torch.cuda.empty_cache()

"""moe_ffn_decode_noalloc (no workspace, library-owned per-device scratch)
against moe_ffn_decode with a caller workspace, through the C ABI: two calls
in a row, the second with a smaller batch, each bitwise equal to the
workspace variant on the same inputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import moe_inputs as mi
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


def test_noalloc_matches_workspace_variant(q):
    wl = mi.WORKLOADS["decode_1layer"]
    layers, ex, rt = device_layers(wl, 1)
    router, experts = layers[0]
    D, F, E, K = wl.d_model, wl.d_ff, wl.n_experts, wl.top_k
    src = mi.WORKLOADS["decode_48layer"]
    for T, stream in ((8, 21), (3, 22)):
        _say(f"moe_ffn_decode_noalloc vs moe_ffn_decode, single layer, T={T}")
        x = torch.from_numpy(mi.activations_host(src, T, stream=stream)).cuda()
        ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
        w = torch.empty((T, K), device="cuda")
        q.moe_route(router, x, ids, w, None, None, q.workspace(q.MOE_OP_ROUTE, T, D, F, E, K))
        y_ws = torch.full((T, D), float("nan"), device="cuda")
        q.moe_ffn_decode(experts, x, ids, w, y_ws, q.workspace(q.MOE_OP_DECODE, T, D, F, E, K))
        y_na = torch.full((T, D), float("nan"), device="cuda")
        q.moe_ffn_decode_noalloc(experts, x, ids, w, y_na)
        torch.cuda.synchronize()
        assert torch.isfinite(y_ws).all()
        assert torch.equal(y_na, y_ws), f"T={T}: the allocation-free variant differs"
    del layers, ex, rt
    torch.cuda.empty_cache()

"""Guard bands around every output buffer and workspace of every entry point.

Each output (and each workspace) is the middle of a larger device buffer
whose leading and trailing GUARD bytes, plus the tail padding up to the next
256-byte boundary, hold a fixed byte pattern.  After each call (and a device
synchronisation) the guards must still hold the pattern, byte for byte, and
the output itself must have been written (it no longer holds the pattern).
Shapes are small and deliberately ragged (5 and 37 tokens, 3 tokens through
the stack) so that partial tiles and tail lanes are exercised."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import moe_inputs as mi
from helpers import device_layers, device_stack

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

GUARD = 4096          # bytes before and after each buffer (keeps the buffer 256-byte aligned)
PATTERN = 0xA5


def _say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def q(need_gpu):
    import quantized_moe_expert_lds_amd as q
    return q


class Guarded:
    """A device buffer of `shape` and `dtype` inside guard bands."""

    def __init__(self, name, shape, dtype, zero=False):
        self.name = name
        itemsize = torch.empty((), dtype=dtype).element_size()
        self.n = int(np.prod(shape)) * itemsize
        padded = (self.n + 255) // 256 * 256
        self.raw = torch.full((GUARD + padded + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD:GUARD + self.n].view(dtype).view(shape)
        if zero:
            self.t.zero_()

    def check(self, written=True):
        torch.cuda.synchronize()
        raw = self.raw.cpu().numpy()
        head, tail = raw[:GUARD], raw[GUARD + self.n:]
        bad_h = np.flatnonzero(head != PATTERN)
        bad_t = np.flatnonzero(tail != PATTERN)
        assert bad_h.size == 0, f"{self.name}: {bad_h.size} bytes before the buffer overwritten (first at -{GUARD - bad_h[0]})"
        assert bad_t.size == 0, f"{self.name}: {bad_t.size} bytes after the buffer overwritten (first at +{bad_t[0]})"
        if written:
            inner = raw[GUARD:GUARD + self.n]
            assert np.any(inner != PATTERN), f"{self.name}: output never written"


def _workspace(q, name, op, T, D, F, E, K):
    return Guarded(name, (q.moe_workspace_size(op, T, D, F, E, K),), torch.uint8, zero=True)


def test_canaries_route_decode_prefill(q):
    wl = mi.WORKLOADS["tiny"]
    (router, experts), = device_layers(wl)[0]
    D, F, E, K = wl.d_model, wl.d_ff, wl.n_experts, wl.top_k
    for T in (5, 37):
        _say(f"guard bands: moe_route, moe_ffn_decode(_noalloc), moe_ffn_prefill(_q8), moe_quantize_q8, "
             f"moe_residual_rmsnorm; tiny workload, {T} tokens")
        x = torch.from_numpy(mi.activations_host(wl, T, stream=3)).cuda()
        ids = Guarded("route ids", (T, K), torch.int32)
        w = Guarded("route gates", (T, K), torch.float32)
        off = Guarded("bucket offsets", (E + 1,), torch.int32)
        prs = Guarded("bucket pairs", (T * K,), torch.int32)
        ws = _workspace(q, "route workspace", q.MOE_OP_ROUTE, T, D, 0, E, K)
        q.moe_route(router, x, ids.t, w.t, off.t, prs.t, ws.t)
        for g in (ids, w, off, prs):
            g.check()
        ws.check(written=False)

        if T <= 8:
            y = Guarded("decode y", (T, D), torch.float32)
            ws = _workspace(q, "decode workspace", q.MOE_OP_DECODE, T, D, F, E, K)
            q.moe_ffn_decode(experts, x, ids.t, w.t, y.t, ws.t)
            y.check()
            ws.check(written=False)
            y2 = Guarded("decode_noalloc y", (T, D), torch.float32)
            q.moe_ffn_decode_noalloc(experts, x, ids.t, w.t, y2.t)
            y2.check()

        y = Guarded("prefill y", (T, D), torch.float32)
        ws = _workspace(q, "prefill workspace", q.MOE_OP_PREFILL, T, D, F, E, K)
        q.moe_ffn_prefill(experts, x, w.t, off.t, prs.t, y.t, ws.t)
        y.check()
        ws.check(written=False)

        y = Guarded("prefill_q8 y", (T, D), torch.float32)
        ws = _workspace(q, "prefill_q8 workspace", q.MOE_OP_PREFILL_Q8, T, D, F, E, K)
        q.moe_ffn_prefill_q8(experts, x, w.t, off.t, prs.t, y.t, ws.t)
        y.check()
        ws.check(written=False)

        qc = Guarded("q8 codes", (T, D), torch.int8)
        dq = Guarded("q8 scales", (T, D // 32), torch.float32)
        q.moe_quantize_q8(x, qc.t, dq.t)
        qc.check()
        dq.check()

        h = Guarded("residual h", (T, D), torch.float32)
        h.t.copy_(x)
        u = Guarded("rmsnorm u", (T, D), torch.float32)
        q.moe_residual_rmsnorm(h.t, y.t, u.t)
        h.check()
        u.check()


def test_canaries_decode_stack(q):
    wl = mi.WORKLOADS["tiny"]
    st, ex, rw, rb = device_stack(wl)
    L, D, K = st.n_layers, st.d_model, wl.top_k
    T = 3
    _say(f"guard bands: moe_decode_stack, tiny stack, {T} tokens, with per-layer outputs")
    x = torch.from_numpy(mi.activations_host(wl, T, stream=5)).cuda()
    h = Guarded("stack h_out", (T, D), torch.float32)
    ids = Guarded("stack ids", (L, T, K), torch.int32)
    g = Guarded("stack gates", (L, T, K), torch.float32)
    hl = Guarded("stack h_layers", (L, T, D), torch.float32)
    ws = Guarded("stack workspace", (q.moe_stack_workspace_size(st, T),), torch.uint8, zero=True)
    q.moe_decode_stack(st, x, h.t, ws.t, ids.t, g.t, h_layers=hl.t)
    for b in (h, ids, g, hl):
        b.check()
    ws.check(written=False)
    err = int(ws.t[q.MOE_STACK_ERROR_OFFSET:q.MOE_STACK_ERROR_OFFSET + 4].view(torch.int32).item())
    assert err == 0


def test_canaries_prefill_stack(q):
    wl = mi.WORKLOADS["tiny_stack"]
    st, ex, rw, rb = device_stack(wl)
    _say("guard bands: moe_prefill_stack, 3 tiny layers, 40 tokens in chunks of 16")
    x = torch.from_numpy(mi.activations_host(wl)).cuda()
    h = Guarded("prefill stack h_out", (x.shape[0], st.d_model), torch.float32)
    ws = Guarded("prefill stack workspace", (q.moe_prefill_stack_workspace_size(st, 16),), torch.uint8)
    q.moe_prefill_stack(st, x, h.t, 16, ws.t)
    h.check()
    ws.check(written=False)

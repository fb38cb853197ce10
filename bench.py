"""Benchmark of the routed MoE FFN hot path on one MI355X.

Headline workload: one 48-layer decode step at batch 1 (512 experts per
layer, d_model 2048, d_ff 768, top-10, 2-bit block-quantised experts, fp32
residual stream with RMSNorm between layers).  A step is, for every layer:
router logits + top-k + gates, the expert FFN with the weighted combine, and
the residual update + RMSNorm -- all on the GPU in one persistent kernel
launch (moe_decode_stack).
Inputs (all 24,576 experts, ~36 GB) are resident in HBM before timing; each
step consumes a different synthetic token.

Also measured in the same run (reported under "also"): the 8,192-token
prefill chunk (route + buckets + grouped GEMMs + combine) and the 4-token
3-bit verify step over 48 layers.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-FFN tokens/s: 48-layer decode (bs1, bs4) + 8192-tok prefill; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
# HBM traffic of decode_stack_kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes (see profiles/), valid only for the kernel source it was taken on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_stack_traffic.json")
KERNEL_SOURCES = ("quantized_moe_expert_lds_amd/csrc/stack.hip", "quantized_moe_expert_lds_amd/csrc/common.hpp")
COPY_BYTES = 1 << 30


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_stack(q, torch, wl, bits=None):
    """Every layer of a workload as one Stack, generated in HBM."""
    import moe_inputs.gpu as g
    bits = wl.bits if bits is None else bits
    ex = g.expert_tensors(wl, None, bits)
    rt = g.routers(wl)
    rw = torch.stack([w for w, _ in rt]).contiguous()
    rb = torch.stack([b for _, b in rt]).contiguous() if wl.zipf_bias else None
    del rt
    st = q.Stack(rw, rb, ex["gate_q"], ex["up_q"], ex["down_q"], ex["gate_s"], ex["up_s"], ex["down_s"],
                 bits, wl.top_k)
    return st, (ex, rw, rb)


def bench_stack(q, torch, wl, steps, warmup, bits=None, built=None):
    """Time `steps` decode steps (one moe_decode_stack launch each, a new
    token batch per step) after `warmup` steps.  Returns wall seconds per step,
    the average kernel duration from HIP events on the launch stream, and the
    algorithmic HBM bytes per launch (packed codes + scales of the distinct
    experts each layer selects, the router matrices, activations).  `built`
    is a (Stack, tensors) pair from build_stack to reuse; it is not freed."""
    import moe_inputs.gpu as g
    st, keep = build_stack(q, torch, wl, bits) if built is None else built
    T, L, K, D, E = wl.n_tokens, st.n_layers, wl.top_k, wl.d_model, wl.n_experts
    n_tok = steps + warmup
    xs = torch.stack([g.activations(wl, stream=s) for s in range(n_tok)])
    h = torch.empty((T, D), device="cuda")
    ws = q.stack_workspace(st, T)
    ids = torch.empty((steps, L, T, K), dtype=torch.int32, device="cuda")
    gw = torch.empty((steps, L, T, K), device="cuda")
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        q.moe_decode_stack(st, xs[i], h, ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        q.moe_decode_stack(st, xs[warmup + i], h, ws, ids[i], gw[i])
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    kern = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    err = int(ws[q.MOE_STACK_ERROR_OFFSET:q.MOE_STACK_ERROR_OFFSET + 4].view(torch.int32).item())
    if err:
        raise RuntimeError("moe_decode_stack reported a barrier timeout")
    ids_np = ids.cpu().numpy()
    uniq = np.array([[len(np.unique(ids_np[i, l])) for l in range(L)] for i in range(steps)])
    bits_ = st._c.bits
    per_expert = 3 * D * wl.d_ff // 32 * (4 * (2 if bits_ == 2 else 3) + 2)
    nbytes = float(uniq.sum(axis=1).mean()) * per_expert + L * E * D * 4 + (E * 4 * L if wl.zipf_bias else 0) \
        + 2 * T * D * 4
    del xs, ws
    if built is None:
        del st, keep
    torch.cuda.empty_cache()
    return wall, kern, nbytes, float(uniq.mean())


def bench_prefill_stack(q, torch, st, steps=2, warmup=1):
    """A 32,768-token prompt in 4 chunks of 8,192 through every layer of the
    48-layer stack (moe_prefill_stack: router, buckets, expert FFN, residual +
    RMSNorm per chunk and layer)."""
    import moe_inputs as mi
    import moe_inputs.gpu as g
    wl = mi.WORKLOADS["prefill_8192"]
    chunk = wl.n_tokens
    T = 4 * chunk
    x = torch.cat([g.activations(wl, stream=s) for s in range(4)])
    h = torch.empty((T, st.d_model), device="cuda")
    ws = q.prefill_stack_workspace(st, chunk)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        q.moe_prefill_stack(st, x, h, chunk, ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        q.moe_prefill_stack(st, x, h, chunk, ws)
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    gpu_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    L, K, D, F = st.n_layers, st.top_k, st.d_model, wl.d_ff
    flops = 2.0 * T * K * 3 * D * F * L
    res = {"workload": "prefill_32k_48layer", "tokens": T, "chunk": chunk, "layers": L,
           "tokens_per_s": T / wall, "ms_per_prompt": wall * 1e3, "gpu_ms_per_prompt": gpu_s * 1e3,
           "ffn_tflops_incl_routing": flops / gpu_s / 1e12}
    del x, h, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(n_layers_sample=12):
    """The oracle (numpy) on the host cores: the first n layers of the 48-layer
    bs1 chain; expert generation (input preparation) is done before timing."""
    import moe_inputs as mi
    from moe_inputs import host_cache
    import oracle.moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    wl = mi.WORKLOADS["decode_48layer"]
    x = mi.activations_host(wl)
    # input preparation: route through the sample once to learn which experts
    # are touched and generate them (untimed)
    h = x.copy()
    routers = [mi.router_host(wl, l) for l in range(n_layers_sample)]
    for l in range(n_layers_sample):
        u = h if l == 0 else O.rmsnorm(h)
        ids, _, _ = O.route(u, routers[l][0], routers[l][1], wl.top_k)
        host_cache.prefetch(wl.name, l, np.unique(ids), wl.bits)
        _, _, y = O.moe_layer(u, routers[l][0], routers[l][1], wl.top_k, host_cache.experts_of(wl, l), wl.bits)
        h = (h + y).astype(np.float32)
    t0 = time.perf_counter()
    O.moe_chain(x, n_layers_sample, lambda l: routers[l], lambda l: host_cache.experts_of(wl, l), wl.top_k,
                wl.bits)
    dt = time.perf_counter() - t0
    per_token = dt * wl.n_layers / n_layers_sample
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": int(blas_threads),
            "host_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"first {n_layers_sample} of 48 layers of one bs1 decode step, scaled to 48 layers "
                      f"({dt:.1f} s measured; expert generation excluded)"}


def bench_prefill(q, torch, steps=5, warmup=2):
    import moe_inputs as mi
    import moe_inputs.gpu as g
    wl = mi.WORKLOADS["prefill_8192"]
    ex = g.expert_tensors(wl, 1)
    (w, b), = g.routers(wl, 1)
    router = q.Router(w, b, wl.top_k)
    experts = q.Experts(ex["gate_q"][0], ex["up_q"][0], ex["down_q"][0], ex["gate_s"][0], ex["up_s"][0],
                        ex["down_s"][0], 2)
    T, K, E, D, F = wl.n_tokens, wl.top_k, wl.n_experts, wl.d_model, wl.d_ff
    x = g.activations(wl)
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gw = torch.empty((T, K), device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    prs = torch.empty(T * K, dtype=torch.int32, device="cuda")
    y = torch.empty((T, D), device="cuda")
    ws_r = q.workspace(q.MOE_OP_ROUTE, T, D, F, E, K)
    ws_p = q.workspace(q.MOE_OP_PREFILL, T, D, F, E, K)
    stream = torch.cuda.current_stream()

    def step():
        q.moe_route(router, x, ids, gw, off, prs, ws_r)
        q.moe_ffn_prefill(experts, x, gw, off, prs, y, ws_p)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, m, b in ev:
        a.record(stream)
        q.moe_route(router, x, ids, gw, off, prs, ws_r)
        m.record(stream)
        q.moe_ffn_prefill(experts, x, gw, off, prs, y, ws_p)
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    route_s = float(np.mean([a.elapsed_time(m) for a, m, b in ev])) * 1e-3
    ffn_s = float(np.mean([m.elapsed_time(b) for a, m, b in ev])) * 1e-3
    flops = 2.0 * T * K * 3 * D * F
    res = {"workload": "prefill_8192", "tokens_per_s": T / wall, "ms_per_step": wall * 1e3,
           "route_ms": route_s * 1e3, "ffn_ms": ffn_s * 1e3,
           "ffn_tflops": flops / ffn_s / 1e12, "ffn_mfma_frac": flops / ffn_s / 1e12 / MFMA_F16_PEAK_TFLOPS}
    del ex, ws_p
    torch.cuda.empty_cache()
    return res


def bench_verify(q, torch, steps=10, warmup=3):
    import moe_inputs as mi
    wl = mi.WORKLOADS["verify4_3bit"]
    wall, kern, nbytes, uniq = bench_stack(q, torch, wl, steps, warmup)
    return {"workload": "verify4_3bit", "tokens_per_s": wl.n_tokens / wall, "ms_per_step": wall * 1e3,
            "kernel_ms": kern * 1e3, "distinct_experts_per_layer": uniq,
            "hbm_gbs": nbytes / kern / 1e9, "hbm_frac": nbytes / kern / 1e9 / HBM_PEAK_GBS}


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode_stack_kernel launch from the committed counter
    passes, or None when the kernel source changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def profile_pass(q, torch):
    """A short run for hardware-counter passes: 3 decode steps of the 48-layer
    batch-1 workload, then a plain elementwise copy of COPY_BYTES (read once,
    written once) that calibrates the counters."""
    import moe_inputs as mi
    wl = mi.WORKLOADS["decode_48layer"]
    bench_stack(q, torch, wl, 3, 1)
    src = torch.ones(COPY_BYTES // 4, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"profile_pass": "decode_48layer x3 + copy", "copy_bytes": COPY_BYTES,
                      "kernel_source_sha256": kernel_source_hash()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-also", action="store_true", help="skip the prefill and verify workloads")
    ap.add_argument("--profile-pass", action="store_true",
                    help="only 3 decode steps and a calibration copy, for rocprofv3 counter passes")
    ap.add_argument("--prefill-pass", action="store_true",
                    help="only the 8,192-token prefill chunk (3 timed calls), for rocprofv3 passes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the MoE FFN path is built and measured on a single MI355X "
              "(all experts resident in its HBM); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_inputs as mi
    import moe_inputs.gpu as g
    import quantized_moe_expert_lds_amd as q

    torch.cuda.set_device(0)
    if args.profile_pass:
        profile_pass(q, torch)
        return
    if args.prefill_pass:
        print(json.dumps(bench_prefill(q, torch, steps=3, warmup=1)), flush=True)
        return
    wl = mi.WORKLOADS["decode_48layer"]
    log("48-layer decode, batch 1: generating 48 x 512 experts in HBM and timing")
    built = build_stack(q, torch, wl)
    dt, kern, nbytes, uniq = bench_stack(q, torch, wl, args.steps, args.warmup, built=built)
    achieved = nbytes / kern / 1e9
    log(f"decode step {dt * 1e6:.1f} us wall, kernel {kern * 1e6:.1f} us, {achieved:.0f} GB/s")

    also = {}
    if not args.no_also:
        log("prefill of a 32,768-token prompt through the 48 layers")
        also["prefill_stack"] = bench_prefill_stack(q, torch, built[0])
    del built
    torch.cuda.empty_cache()
    if not args.no_also:
        log("prefill 8192")
        also["prefill"] = bench_prefill(q, torch)
        log("verify 4 tokens 3-bit")
        also["verify"] = bench_verify(q, torch)

    cpu = None
    if not args.no_cpu:
        log("CPU oracle baseline")
        cpu = cpu_baseline()

    out = {
        "metric": METRIC,
        "value": 1.0 / dt,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights quantised to 2-bit blocks, "
                "Zipf-biased router)",
        "config": {"workload": "decode_48layer", "layers": 48, "experts_per_layer": 512, "d_model": 2048,
                   "d_ff": 768, "top_k": 10, "batch": 1, "weight_bits": 2, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "decode_stack_kernel (all 48 layers, one launch)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "bytes_per_launch": nbytes, "kernel_us": kern * 1e6,
                     "distinct_experts_per_layer": uniq},
        "cpu_baseline": cpu,
        "also": also,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

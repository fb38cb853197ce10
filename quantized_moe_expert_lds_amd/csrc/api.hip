// C ABI entry points: argument validation, workspace layout, kernel choice.
// Nothing here allocates device memory or synchronises; all work is enqueued
// on the caller's stream.
#include <atomic>
#include <cstring>

#include "prefill_q8.hpp"

namespace qmoe {
bool decode_supported(int T, int K, int F);
}

namespace {

using namespace qmoe;

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return MOE_ERR_NO_DEVICE;
    }
    if (dev >= kMaxDevices) return MOE_ERR_NO_DEVICE;
    int ok = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (ok == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return MOE_ERR_NO_DEVICE;
        }
        ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_arch_ok[dev].store(ok, std::memory_order_relaxed);
    }
    return ok == 1 ? MOE_OK : MOE_ERR_NO_DEVICE;
}

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return MOE_OK;
    if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

int check_experts(const moe_experts_t* ex) {
    if (!ex || !ex->gate_q || !ex->up_q || !ex->down_q || !ex->gate_s || !ex->up_s || !ex->down_s)
        return MOE_ERR_ARG;
    if (ex->n_experts <= 0 || ex->d_model <= 0 || ex->d_ff <= 0) return MOE_ERR_ARG;
    if (ex->bits != 2 && ex->bits != 3) return MOE_ERR_UNSUPPORTED;
    if (ex->d_model % 32 || ex->d_ff % 32) return MOE_ERR_UNSUPPORTED;
    if (ex->d_model > kMaxDModel || ex->d_ff > kMaxDff || ex->n_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int dtype_flag(int x_dtype) {
    if (x_dtype == MOE_F32) return 0;
    if (x_dtype == MOE_BF16) return 1;
    return -1;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

size_t decode_ws_bytes(int T, int F, int K) { return decode_ws_layout(T, F, K).total; }

std::atomic<int> g_cus[kMaxDevices];       // compute units per device, 0 = unknown

int device_cus() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        int coop = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) {
            (void)hipGetLastError();
            return 0;
        }
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(int op, int n_tokens, int d_model, int d_ff, int n_experts, int top_k) {
    if (n_tokens <= 0 || d_model <= 0 || n_experts <= 0 || top_k <= 0) return 0;
    switch (op) {
        case MOE_OP_ROUTE:
            return route_ws_layout(n_tokens, d_model, n_experts, top_k).total;
        case MOE_OP_DECODE:
            if (d_ff <= 0) return 0;
            return decode_ws_bytes(n_tokens, d_ff, top_k);
        case MOE_OP_PREFILL:
            if (d_ff <= 0) return 0;
            return prefill_ws_layout(n_tokens, d_model, d_ff, n_experts, top_k).total;
        case MOE_OP_PREFILL_Q8:
            if (d_ff <= 0) return 0;
            return prefill_q8_ws_layout(n_tokens, d_model, d_ff, n_experts, top_k).total;
        default:
            return 0;
    }
}

int moe_route(const moe_router_t* router, const void* x, int x_dtype, int n_tokens, int32_t* topk_ids,
              float* topk_w, int32_t* bucket_offsets, int32_t* bucket_pairs, void* ws, size_t ws_bytes,
              void* stream) {
    if (!router || !router->w || !x || !topk_ids || !topk_w || n_tokens <= 0) return MOE_ERR_ARG;
    const int xf = dtype_flag(x_dtype);
    if (xf < 0) return MOE_ERR_ARG;
    const int D = router->d_model, E = router->n_experts, K = router->top_k;
    if (D <= 0 || E <= 0 || K <= 0) return MOE_ERR_ARG;
    if (D % 32 || D > kMaxDModel || E > kMaxExperts || K > E || K > kMaxTopK) return MOE_ERR_UNSUPPORTED;
    if ((long long)n_tokens * K > (1LL << 30)) return MOE_ERR_UNSUPPORTED;
    const bool buckets = bucket_offsets && bucket_pairs;
    const RouteWs L = route_ws_layout(n_tokens, D, E, K);
    int st = check_ws(ws, ws_bytes, L.total);
    if (st) return st;
    if ((st = check_device())) return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (n_tokens <= kMaxDecodeTokens)
        e = launch_route_small(*router, x, xf, n_tokens, topk_ids, topk_w, (char*)ws, L, s);
    else
        e = launch_route_large(*router, x, xf, n_tokens, topk_ids, topk_w, (char*)ws, L, s);
    if (e == hipSuccess && buckets)
        e = launch_buckets(topk_ids, n_tokens, K, E, bucket_offsets, bucket_pairs, (char*)ws, L, s);
    return hip_status(e);
}

int moe_ffn_decode(const moe_experts_t* experts, const void* x, int x_dtype, int n_tokens,
                   const int32_t* topk_ids, const float* topk_w, int top_k, float* y, void* ws,
                   size_t ws_bytes, void* stream) {
    int st = check_experts(experts);
    if (st) return st;
    if (!x || !topk_ids || !topk_w || !y || n_tokens <= 0 || top_k <= 0) return MOE_ERR_ARG;
    const int xf = dtype_flag(x_dtype);
    if (xf < 0) return MOE_ERR_ARG;
    if (n_tokens > kMaxDecodeTokens || top_k > kMaxTopK || top_k > experts->n_experts)
        return MOE_ERR_UNSUPPORTED;
    if (!decode_supported(n_tokens, top_k, experts->d_ff)) return MOE_ERR_UNSUPPORTED;
    const DecodeWs L = decode_ws_layout(n_tokens, experts->d_ff, top_k);
    if ((st = check_ws(ws, ws_bytes, L.total))) return st;
    if ((st = check_device())) return st;
    return hip_status(launch_decode(*experts, x, xf, n_tokens, topk_ids, topk_w, top_k, y, (char*)ws, L,
                                    (hipStream_t)stream));
}

int moe_ffn_decode_noalloc(const moe_experts_t* experts, const void* x, int x_dtype, int n_tokens,
                           const int32_t* topk_ids, const float* topk_w, int top_k, float* y, void* stream) {
    int st = check_experts(experts);
    if (st) return st;
    if (!x || !topk_ids || !topk_w || !y || n_tokens <= 0 || top_k <= 0) return MOE_ERR_ARG;
    const int xf = dtype_flag(x_dtype);
    if (xf < 0) return MOE_ERR_ARG;
    if (n_tokens > kMaxDecodeTokens || top_k > kMaxTopK || top_k > experts->n_experts)
        return MOE_ERR_UNSUPPORTED;
    if (!decode_supported(n_tokens, top_k, experts->d_ff)) return MOE_ERR_UNSUPPORTED;
    const DecodeWs L = decode_ws_layout(n_tokens, experts->d_ff, top_k);
    if (L.total > kDecodeScratchBytes) return MOE_ERR_UNSUPPORTED;
    if ((st = check_device())) return st;
    char* scratch = nullptr;
    if (decode_noalloc_scratch(&scratch) != hipSuccess) {
        (void)hipGetLastError();
        return MOE_ERR_HIP;
    }
    return hip_status(launch_decode(*experts, x, xf, n_tokens, topk_ids, topk_w, top_k, y, scratch, L,
                                    (hipStream_t)stream));
}

int moe_ffn_prefill(const moe_experts_t* experts, const void* x, int x_dtype, int n_tokens, const float* topk_w,
                    int top_k, const int32_t* bucket_offsets, const int32_t* bucket_pairs, float* y, void* ws,
                    size_t ws_bytes, void* stream) {
    int st = check_experts(experts);
    if (st) return st;
    if (!x || !topk_w || !bucket_offsets || !bucket_pairs || !y || n_tokens <= 0 || top_k <= 0) return MOE_ERR_ARG;
    const int xf = dtype_flag(x_dtype);
    if (xf < 0) return MOE_ERR_ARG;
    if (experts->bits != 2 || experts->d_model % kDownBN || experts->d_ff % kGateUpBN || top_k > kMaxTopK ||
        top_k > experts->n_experts)
        return MOE_ERR_UNSUPPORTED;
    if ((long long)n_tokens * top_k > (1LL << 28)) return MOE_ERR_UNSUPPORTED;
    const PrefillWs L = prefill_ws_layout(n_tokens, experts->d_model, experts->d_ff, experts->n_experts, top_k);
    if ((st = check_ws(ws, ws_bytes, L.total))) return st;
    if ((st = check_device())) return st;
    return hip_status(launch_prefill(*experts, x, xf, n_tokens, topk_w, top_k, bucket_offsets, bucket_pairs, y,
                                     (char*)ws, L, (hipStream_t)stream));
}

int moe_ffn_prefill_q8(const moe_experts_t* experts, const void* x, int x_dtype, int n_tokens, const float* topk_w,
                       int top_k, const int32_t* bucket_offsets, const int32_t* bucket_pairs, float* y, void* ws,
                       size_t ws_bytes, void* stream) {
    int st = check_experts(experts);
    if (st) return st;
    if (!x || !topk_w || !bucket_offsets || !bucket_pairs || !y || n_tokens <= 0 || top_k <= 0) return MOE_ERR_ARG;
    const int xf = dtype_flag(x_dtype);
    if (xf < 0) return MOE_ERR_ARG;
    if (experts->bits != 2 || experts->d_model % kDownBN || experts->d_ff % kGateUpBN || top_k > kMaxTopK ||
        top_k > experts->n_experts)
        return MOE_ERR_UNSUPPORTED;
    if ((long long)n_tokens * top_k > (1LL << 28)) return MOE_ERR_UNSUPPORTED;
    const PrefillQ8Ws L = prefill_q8_ws_layout(n_tokens, experts->d_model, experts->d_ff, experts->n_experts, top_k);
    if ((st = check_ws(ws, ws_bytes, L.total))) return st;
    if ((st = check_device())) return st;
    return hip_status(launch_prefill_q8(*experts, x, xf, n_tokens, topk_w, top_k, bucket_offsets, bucket_pairs, y,
                                        (char*)ws, L, (hipStream_t)stream));
}

int moe_quantize_q8(const void* x, int x_dtype, int n_rows, int n_cols, int8_t* q, float* d, void* stream) {
    if (!x || !q || !d || n_rows <= 0 || n_cols <= 0) return MOE_ERR_ARG;
    const int xf = dtype_flag(x_dtype);
    if (xf < 0) return MOE_ERR_ARG;
    if (n_cols % 32) return MOE_ERR_UNSUPPORTED;
    const size_t nblocks = (size_t)n_rows * (size_t)(n_cols / 32);
    if (nblocks > (size_t(1) << 36)) return MOE_ERR_UNSUPPORTED;
    int st = check_device();
    if (st) return st;
    return hip_status(launch_quantize_q8(x, xf, nblocks, q, d, (hipStream_t)stream));
}

size_t moe_stack_workspace_size(const moe_stack_t* m, int n_tokens) {
    if (!m || n_tokens <= 0 || m->n_layers <= 0 || m->n_experts <= 0 || m->d_model <= 0 || m->d_ff <= 0 ||
        m->top_k <= 0)
        return 0;
    return stack_ws_layout(n_tokens, m->d_model, m->d_ff, m->n_experts, m->top_k, kStackMaxGrid, m->n_layers).total;
}

int moe_decode_stack(const moe_stack_t* m, const void* x, int x_dtype, int n_tokens, double eps, float* h_out,
                     int32_t* ids_out, float* gates_out, float* h_layers_out, void* ws, size_t ws_bytes,
                     void* stream) {
    if (!m || !x || !h_out || n_tokens <= 0 || !(eps >= 0.0)) return MOE_ERR_ARG;
    if (!m->router_w || !m->gate_q || !m->up_q || !m->down_q || !m->gate_s || !m->up_s || !m->down_s)
        return MOE_ERR_ARG;
    if ((ids_out == nullptr) != (gates_out == nullptr)) return MOE_ERR_ARG;
    const int xf = dtype_flag(x_dtype);
    if (xf < 0) return MOE_ERR_ARG;
    const int L = m->n_layers, E = m->n_experts, D = m->d_model, F = m->d_ff, K = m->top_k;
    if (L <= 0 || E <= 0 || D <= 0 || F <= 0 || K <= 0) return MOE_ERR_ARG;
    if (m->bits != 2 && m->bits != 3) return MOE_ERR_UNSUPPORTED;
    if (n_tokens > kMaxDecodeTokens || D % 32 || F % 32 || D > kStackMaxD || F > kMaxDff || E > kMaxExperts ||
        K > E || K > kMaxTopK)
        return MOE_ERR_UNSUPPORTED;
    if (!ws) return MOE_ERR_WORKSPACE;
    int st = check_device();
    if (st) return st;
    const int G = device_cus();
    if (G <= 0 || G > kStackMaxGrid) return MOE_ERR_NO_DEVICE;
    const StackWs Lw = stack_ws_layout(n_tokens, D, F, E, K, G, L);
    if ((st = check_ws(ws, ws_bytes, Lw.total))) return st;
    // router experts and d_model rows per workgroup
    if ((E + G - 1) / G > 4 || (D + G - 1) / G > 16) return MOE_ERR_UNSUPPORTED;
    if (stack_lds_bytes(n_tokens, D, F, E, K, G, m->bits) > kStackLdsLimit)
        return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_decode_stack(*m, x, xf, n_tokens, h_out, ids_out, gates_out, h_layers_out, eps,
                                          (char*)ws, Lw, G,
                                          (hipStream_t)stream));
}

int moe_residual_rmsnorm(float* h, const float* y, float* u, int n_tokens, int d, double eps, void* stream) {
    if (!h || !u || n_tokens <= 0 || d <= 0 || !(eps >= 0.0)) return MOE_ERR_ARG;
    int st = check_device();
    if (st) return st;
    return hip_status(launch_residual_rmsnorm(h, y, u, n_tokens, d, eps, (hipStream_t)stream));
}

size_t moe_prefill_stack_workspace_size(const moe_stack_t* m, int chunk_tokens) {
    if (!m || chunk_tokens <= 0 || m->n_layers <= 0 || m->n_experts <= 0 || m->d_model <= 0 || m->d_ff <= 0 ||
        m->top_k <= 0)
        return 0;
    return prefill_stack_ws_layout(chunk_tokens, m->d_model, m->d_ff, m->n_experts, m->top_k).total;
}

int moe_prefill_stack(const moe_stack_t* m, const void* x, int x_dtype, int n_tokens, int chunk_tokens, double eps,
                      float* h_out, void* ws, size_t ws_bytes, void* stream) {
    if (!m || !x || !h_out || n_tokens <= 0 || chunk_tokens <= 0 || !(eps >= 0.0)) return MOE_ERR_ARG;
    if (!m->router_w || !m->gate_q || !m->up_q || !m->down_q || !m->gate_s || !m->up_s || !m->down_s)
        return MOE_ERR_ARG;
    const int xf = dtype_flag(x_dtype);
    if (xf < 0) return MOE_ERR_ARG;
    const int L = m->n_layers, E = m->n_experts, D = m->d_model, F = m->d_ff, K = m->top_k;
    if (L <= 0 || E <= 0 || D <= 0 || F <= 0 || K <= 0) return MOE_ERR_ARG;
    if (m->bits != 2 || D % kDownBN || F % kGateUpBN || D > kMaxDModel || F > kMaxDff || E > kMaxExperts ||
        K > E || K > kMaxTopK)
        return MOE_ERR_UNSUPPORTED;
    if ((long long)chunk_tokens * K > (1LL << 28)) return MOE_ERR_UNSUPPORTED;
    const PrefillStackWs W = prefill_stack_ws_layout(chunk_tokens, D, F, E, K);
    int st = check_ws(ws, ws_bytes, W.total);
    if (st) return st;
    if ((st = check_device())) return st;
    hipStream_t s = (hipStream_t)stream;
    char* b = (char*)ws;
    int32_t* ids = (int32_t*)(b + W.ids);
    float* gates = (float*)(b + W.gates);
    int32_t* offsets = (int32_t*)(b + W.offsets);
    int32_t* pairs = (int32_t*)(b + W.pairs);
    float* y = (float*)(b + W.y);
    float* u = (float*)(b + W.u);
    const size_t x_row = (size_t)D * (xf ? 2 : 4);
    const size_t gu_words = (size_t)E * F * (D / 32) * 2, d_words = (size_t)E * D * (F / 32) * 2;
    const size_t gu_blocks = (size_t)E * F * (D / 32), d_blocks = (size_t)E * D * (F / 32);
    // chunk-major: every chunk passes through all layers before the next starts
    for (int c0 = 0; c0 < n_tokens; c0 += chunk_tokens) {
        const int Tc = n_tokens - c0 < chunk_tokens ? n_tokens - c0 : chunk_tokens;
        const void* xc = (const char*)x + (size_t)c0 * x_row;
        float* h = h_out + (size_t)c0 * D;
        hipError_t e = launch_to_f32(xc, xf, (size_t)Tc * D, h, s);
        for (int l = 0; l < L && e == hipSuccess; ++l) {
            const moe_router_t r{D, E, K, m->router_w + (size_t)l * E * D, m->router_b ? m->router_b + (size_t)l * E : nullptr};
            moe_experts_t ex{};
            ex.n_experts = E;
            ex.d_model = D;
            ex.d_ff = F;
            ex.bits = 2;
            ex.gate_q = m->gate_q + l * gu_words;
            ex.up_q = m->up_q + l * gu_words;
            ex.down_q = m->down_q + l * d_words;
            ex.gate_s = m->gate_s + l * gu_blocks;
            ex.up_s = m->up_s + l * gu_blocks;
            ex.down_s = m->down_s + l * d_blocks;
            const void* ul = l == 0 ? xc : (const void*)u;
            const int uf = l == 0 ? xf : 0;
            e = Tc <= kMaxDecodeTokens ? launch_route_small(r, ul, uf, Tc, ids, gates, b + W.route, W.rl, s)
                                       : launch_route_large(r, ul, uf, Tc, ids, gates, b + W.route, W.rl, s);
            if (e == hipSuccess) e = launch_buckets(ids, Tc, K, E, offsets, pairs, b + W.route, W.rl, s);
            if (e == hipSuccess)
                e = launch_prefill(ex, ul, uf, Tc, gates, K, offsets, pairs, y, b + W.prefill, W.pl, s);
            // h += y; u = RMSNorm(h), the next layer's input
            if (e == hipSuccess) e = launch_residual_rmsnorm(h, y, u, Tc, D, eps, s);
        }
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    return MOE_OK;
}

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_ARG: return "invalid argument (null pointer, non-positive size or unknown dtype)";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or format";
        case MOE_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
        case MOE_ERR_NO_DEVICE: return "no HIP device, or the current device is not gfx950";
        case MOE_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

}  // extern "C"

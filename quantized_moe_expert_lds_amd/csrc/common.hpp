// Internal declarations shared by the HIP sources of the MoE FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_ffn.h"

namespace qmoe {

// ------------------------------------------------------------------ limits
constexpr int kMaxDecodeTokens = 8;
constexpr int kMaxTopK = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxDModel = 16384;
constexpr int kMaxDff = 4096;

// bucketing: pairs per block
constexpr int kBucketBlock = 256;
// prefill grouped GEMM tile
constexpr int kGemmBM = 128;
constexpr int kGemmBK = 64;
constexpr int kGateUpBN = 128;    // d_ff columns per gate/up tile (x2 for gate and up)
constexpr int kDownBN = 256;      // d_model columns per down tile

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// ------------------------------------------------------------ workspace map
struct RouteWs {
    size_t zfull, hist, rank, counter, total;
};
struct DecodeWs {
    size_t h, total;
};
struct PrefillWs {
    size_t x16, hbuf, obuf, tiles, ntiles, total;
};
struct StackWs {
    size_t hdr, rows, logits, flags, hp, total;
};
constexpr int kStackMaxGrid = 1024;      // workspace sized for up to this many workgroups
constexpr int kStackMaxD = 2048;
constexpr size_t kStackLdsLimit = 160 * 1024;
StackWs stack_ws_layout(int T, int D, int F, int E, int K, int G, int L);
size_t stack_lds_bytes(int T, int D, int F, int E, int K, int G, int bits);

inline RouteWs route_ws_layout(int T, int D, int E, int K) {
    RouteWs w{};
    size_t off = 0;
    (void)D;
    w.zfull = off;
    off += align256(sizeof(double) * (size_t)T * E);
    const size_t P = (size_t)T * K;
    const size_t nb = (P + kBucketBlock - 1) / kBucketBlock;
    w.hist = off;
    off += align256(sizeof(int) * nb * E);
    w.rank = off;
    off += align256(sizeof(int) * P);
    w.counter = off;                     // small-batch router: workgroups done (zero between calls)
    off += 256;
    w.total = off;
    return w;
}

// chunked prefill through a stack: per-chunk buffers, then the route and
// prefill workspaces of one chunk
struct PrefillStackWs {
    size_t ids, gates, offsets, pairs, y, u, route, prefill, total;
    RouteWs rl;
    PrefillWs pl;
};

// the SwiGLU intermediate as two fp16 halves (hi, then lo) per value
inline DecodeWs decode_ws_layout(int T, int F, int K) {
    DecodeWs w{};
    w.h = 0;
    w.total = align256(2 * sizeof(uint16_t) * (size_t)T * K * F);
    return w;
}

// moe_ffn_decode_noalloc: the per-device scratch that replaces the decode
// workspace (8 MiB: the SwiGLU intermediate of 8 tokens x 64 slots x 4096
// d_ff values, kept as two fp16 halves each) and its device address on the
// current device.
constexpr size_t kDecodeScratchBytes = size_t(8) << 20;
hipError_t decode_noalloc_scratch(char** ptr);

inline int prefill_max_tiles(int T, int E, int K) {
    const long long P = (long long)T * K;
    const long long nonempty = P < E ? P : E;
    return (int)((P + kGemmBM - 1) / kGemmBM + nonempty);
}

inline PrefillWs prefill_ws_layout(int T, int D, int F, int E, int K) {
    PrefillWs w{};
    size_t off = 0;
    const size_t P = (size_t)T * K;
    w.x16 = off;
    off += align256(sizeof(uint16_t) * (size_t)T * D);
    w.hbuf = off;
    off += align256(sizeof(uint16_t) * P * F);
    w.obuf = off;
    off += align256(sizeof(float) * P * D);
    w.tiles = off;
    off += align256(sizeof(int4) * (size_t)prefill_max_tiles(T, E, K));
    w.ntiles = off;
    off += align256(sizeof(int) * 4);
    w.total = off;
    return w;
}

inline PrefillStackWs prefill_stack_ws_layout(int Tc, int D, int F, int E, int K) {
    PrefillStackWs w{};
    const size_t P = (size_t)Tc * K;
    size_t off = 0;
    w.ids = off;
    off += align256(sizeof(int32_t) * P);
    w.gates = off;
    off += align256(sizeof(float) * P);
    w.offsets = off;
    off += align256(sizeof(int32_t) * ((size_t)E + 1));
    w.pairs = off;
    off += align256(sizeof(int32_t) * P);
    w.y = off;
    off += align256(sizeof(float) * (size_t)Tc * D);
    w.u = off;
    off += align256(sizeof(float) * (size_t)Tc * D);
    w.rl = route_ws_layout(Tc, D, E, K);
    w.route = off;
    off += w.rl.total;
    w.pl = prefill_ws_layout(Tc, D, F, E, K);
    w.prefill = off;
    off += w.pl.total;
    w.total = off;
    return w;
}

// -------------------------------------------------------- kernel launchers
// Each returns hipGetLastError() of its launches.
hipError_t launch_route_small(const moe_router_t& r, const void* x, int x_bf16, int T, int32_t* ids,
                              float* gates, char* ws, const RouteWs& L, hipStream_t s);
hipError_t launch_route_large(const moe_router_t& r, const void* x, int x_bf16, int T, int32_t* ids,
                              float* gates, char* ws, const RouteWs& L, hipStream_t s);
hipError_t launch_buckets(const int32_t* ids, int T, int K, int E, int32_t* offsets, int32_t* pairs,
                          char* ws, const RouteWs& L, hipStream_t s);
hipError_t launch_decode(const moe_experts_t& ex, const void* x, int x_bf16, int T, const int32_t* ids,
                         const float* gates, int K, float* y, char* ws, const DecodeWs& L, hipStream_t s);
hipError_t launch_prefill(const moe_experts_t& ex, const void* x, int x_bf16, int T, const float* gates,
                          int K, const int32_t* offsets, const int32_t* pairs, float* y, char* ws,
                          const PrefillWs& L, hipStream_t s);
hipError_t launch_decode_stack(const moe_stack_t& m, const void* x, int x_bf16, int T, float* h_out,
                               int32_t* ids_out, float* gates_out, float* h_layers, double eps, char* ws,
                               const StackWs& L, int G, hipStream_t s);
hipError_t launch_residual_rmsnorm(float* h, const float* y, float* u, int T, int d, double eps,
                                   hipStream_t s);
hipError_t launch_to_f32(const void* x, int x_bf16, size_t n, float* out, hipStream_t s);

}  // namespace qmoe

// ------------------------------------------------------------ device helpers
namespace qmoe_dev {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Position of weight i (0..31) of a block after the pair-interleaving used
// by the fp16 unpack: weights (m, m+8) of each 16-weight half are adjacent.
__device__ __forceinline__ int perm32(int i) {
    return (i & 16) | ((i & 7) << 1) | ((i >> 3) & 1);
}

__device__ __forceinline__ half2_t as_half2(uint32_t v) {
    return __builtin_bit_cast(half2_t, v);
}
__device__ __forceinline__ uint32_t as_u32(half2_t v) {
    return __builtin_bit_cast(uint32_t, v);
}

// Two 2-bit codes -> fp16 pair (1024 + code) by placing each code in the low
// mantissa bits of 1024.0 (0x6400); the caller subtracts 1024 + bias.
__device__ __forceinline__ uint32_t codes2_pair(uint32_t word, int shift) {
    return ((word >> shift) & 0x00030003u) | 0x64006400u;
}

// Codes of a 3-bit block (96-bit little-endian string) for weights m and
// m+8 of half h (weights 16h+m and 16h+m+8) as an fp16 pair (1024 + code).
__device__ __forceinline__ uint32_t code3(uint32_t w0, uint32_t w1, uint32_t w2, int i) {
    const int pos = 3 * i;
    uint64_t lo = ((uint64_t)w1 << 32) | w0;
    if (pos + 3 <= 64) return (uint32_t)(lo >> pos) & 7u;
    if (pos >= 64) return (w2 >> (pos - 64)) & 7u;
    return (uint32_t)((lo >> pos) | ((uint64_t)w2 << (64 - pos))) & 7u;
}
__device__ __forceinline__ uint32_t codes3_pair(uint32_t w0, uint32_t w1, uint32_t w2, int i) {
    return (code3(w0, w1, w2, i) | (code3(w0, w1, w2, i + 8) << 16)) | 0x64006400u;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ bool better(double a, int ia, double b, int ib) {
    return a > b || (a == b && ia < ib);
}

// One wavefront selects the top-k of z[0..E) (E <= 1024) and writes ids and
// gates.  Ranks by (z descending, id ascending); -0.0 == +0.0 by IEEE compare.
__device__ inline void wave_topk(const double* z, int E, int K, int32_t* ids, float* gates) {
    const int lane = threadIdx.x & 63;
    constexpr int kPer = qmoe::kMaxExperts / 64;
    double v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? z[e] + 0.0 : -INFINITY;
    }
    uint32_t taken = 0;
    double my_sel = 0.0;
    for (int j = 0; j < K; ++j) {
        double bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !(taken >> i & 1u) && better(v[i], e, bv, bi)) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const double ov = __shfl_xor(bv, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            if (better(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (lane == j) {
            my_sel = bv;
            ids[j] = bi;
        }
    }
    // gates: softmax over the selected logits, fp64
    const double m = __shfl(my_sel, 0, 64);
    double p = lane < K ? exp(my_sel - m) : 0.0;
    double sum = p;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    // every lane holds the same sum only if the butterfly is order-symmetric;
    // take lane 0's value so all gates divide by one number
    sum = __shfl(sum, 0, 64);
    if (lane < K) gates[lane] = (float)(p / sum);
}

}  // namespace qmoe_dev

// Router: logits z = x W + b in fp64, top-k selection (ties -> lower id) and
// softmax gates over the selected logits.
//
// The Strata pages name a dedicated router kernel (bnskd "Strata：把 125B 大模型
// 塞进 12GB 显卡", section 代码结构) and state that each token is sent to 10 of
// the experts (same page, section 核心思路); the kernels here are this
// library's own design for gfx950.
//
// Two paths:
//  * small batches (T <= 8, decode and verify): reading the router matrix is
//    the whole cost.  The router is stored expert-major ([E][d_model]), so
//    each workgroup reads the contiguous rows of two experts (16 KB) with
//    128-bit loads and produces complete logits; a second small kernel (one
//    wavefront per token) selects the top-k.  No cross-workgroup
//    synchronisation inside a kernel.
//  * large batches (prefill): a tiled fp64 GEMM in which every logit is
//    accumulated by one thread over d in ascending order with fused
//    multiply-adds (each fp32 x fp32 product is exact in fp64, so this is the
//    same rounding sequence as the plain definition), then one wavefront per
//    token selects the top-k.
#include "common.hpp"

#include <math.h>

namespace {

using namespace qmoe;
using namespace qmoe_dev;

__device__ __forceinline__ double load_x(const void* x, int x_bf16, size_t i) {
    if (x_bf16) return (double)bf16_to_f32(((const uint16_t*)x)[i]);
    return (double)((const float*)x)[i];
}

// ---------------------------------------------------------------- small T
// grid ceil(E/2), block 256: workgroup w computes the full logits of experts
// 2w and 2w+1 for every token.  Wave v covers expert 2w + (v & 1) and half
// (v >> 1) of the d range; lane l owns 16 consecutive d of that half (an
// expert row is contiguous in the expert-major router layout).
template <int T>
__global__ __launch_bounds__(256) void route_logits_kernel(moe_router_t r, const void* __restrict__ x, int x_bf16,
                                                           double* __restrict__ z) {
    const int E = r.n_experts, D = r.d_model;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e = blockIdx.x * 2 + (wave & 1);
    const int half = wave >> 1;
    const int dh = D / 2;                        // D is a multiple of 32
    __shared__ double red[2][2][T];
    double acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.0;
    if (e < E) {
        const float* wr = r.w + (size_t)e * D + half * dh;
        for (int d0 = 16 * lane; d0 < dh; d0 += 16 * 64) {
            float4 wv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) wv[q] = *reinterpret_cast<const float4*>(wr + d0 + 4 * q);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const size_t xo = (size_t)t * D + half * dh + d0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[t] = fma(load_x(x, x_bf16, xo + 4 * q), (double)wv[q].x, acc[t]);
                    acc[t] = fma(load_x(x, x_bf16, xo + 4 * q + 1), (double)wv[q].y, acc[t]);
                    acc[t] = fma(load_x(x, x_bf16, xo + 4 * q + 2), (double)wv[q].z, acc[t]);
                    acc[t] = fma(load_x(x, x_bf16, xo + 4 * q + 3), (double)wv[q].w, acc[t]);
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        double v = acc[t];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) red[wave & 1][half][t] = v;
    }
    __syncthreads();
    if (tid < 2 * T) {
        const int ee = blockIdx.x * 2 + (tid & 1), t = tid >> 1;
        if (ee < E) {
            double s = red[tid & 1][0][t] + red[tid & 1][1][t];
            if (r.bias) s += (double)r.bias[ee];
            z[(size_t)t * E + ee] = s;
        }
    }
}

// ---------------------------------------------------------------- large T
// grid: (ceil(E/64), ceil(T/64)), block 256: thread (ty = tid/16, tx = tid%16)
// owns tokens t0 + 4 ty .. +3 and experts e0 + 4 tx .. +3.
__global__ __launch_bounds__(256) void route_gemm_kernel(moe_router_t r, const void* __restrict__ x,
                                                         int x_bf16, int T, double* __restrict__ z) {
    const int E = r.n_experts, D = r.d_model;
    const int e0 = blockIdx.x * kRouteTileE, t0 = blockIdx.y * kRouteTileT;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    __shared__ double xs[kRouteTileD][kRouteTileT + 2];
    __shared__ double ws_[kRouteTileD][kRouteTileE + 2];

    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;

    for (int d0 = 0; d0 < D; d0 += kRouteTileD) {
        // x tile: 64 tokens x 32 d -> transposed into xs[d][t]
        for (int i = tid; i < kRouteTileT * kRouteTileD; i += 256) {
            const int t = i / kRouteTileD, dd = i % kRouteTileD;
            const int tt = t0 + t, d = d0 + dd;
            xs[dd][t] = (tt < T && d < D) ? load_x(x, x_bf16, (size_t)tt * D + d) : 0.0;
        }
        for (int i = tid; i < kRouteTileD * kRouteTileE; i += 256) {
            const int ee = i / kRouteTileD, dd = i % kRouteTileD;
            const int d = d0 + dd, e = e0 + ee;
            ws_[dd][ee] = (d < D && e < E) ? (double)r.w[(size_t)e * D + d] : 0.0;
        }
        __syncthreads();
#pragma unroll 4
        for (int dd = 0; dd < kRouteTileD; ++dd) {
            double xv[4], wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[i] = xs[dd][4 * ty + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) wv[j] = ws_[dd][4 * tx + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fma(xv[i], wv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * ty + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + 4 * tx + j;
            if (e >= E) continue;
            double s = acc[i][j];
            if (r.bias) s += (double)r.bias[e];
            z[(size_t)t * E + e] = s;
        }
    }
}

// grid: ceil(T/4), block 256: one wavefront per token
__global__ __launch_bounds__(256) void topk_kernel(const double* __restrict__ z, int T, int E, int K,
                                                   int32_t* __restrict__ ids, float* __restrict__ gates) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    wave_topk(z + (size_t)t * E, E, K, ids + (size_t)t * K, gates + (size_t)t * K);
}

}  // namespace

namespace qmoe {

hipError_t launch_route_small(const moe_router_t& r, const void* x, int x_bf16, int T, int32_t* ids,
                              float* gates, char* ws, const RouteWs& L, hipStream_t s) {
    double* z = (double*)(ws + L.zfull);
    const unsigned grid = (unsigned)cdiv(r.n_experts, 2);
    switch (T) {
#define QMOE_CASE(N)                                                         \
    case N:                                                                  \
        route_logits_kernel<N><<<grid, 256, 0, s>>>(r, x, x_bf16, z); \
        break;
        QMOE_CASE(1) QMOE_CASE(2) QMOE_CASE(3) QMOE_CASE(4) QMOE_CASE(5) QMOE_CASE(6) QMOE_CASE(7) QMOE_CASE(8)
#undef QMOE_CASE
        default:
            return hipErrorInvalidValue;
    }
    topk_kernel<<<cdiv(T, 4), 256, 0, s>>>(z, T, r.n_experts, r.top_k, ids, gates);
    return hipGetLastError();
}

hipError_t launch_route_large(const moe_router_t& r, const void* x, int x_bf16, int T, int32_t* ids,
                              float* gates, char* ws, const RouteWs& L, hipStream_t s) {
    double* z = (double*)(ws + L.zfull);
    dim3 grid(cdiv(r.n_experts, kRouteTileE), cdiv(T, kRouteTileT));
    route_gemm_kernel<<<grid, 256, 0, s>>>(r, x, x_bf16, T, z);
    topk_kernel<<<cdiv(T, 4), 256, 0, s>>>(z, T, r.n_experts, r.top_k, ids, gates);
    return hipGetLastError();
}

}  // namespace qmoe

// Router: logits z = x W + b in fp64, top-k selection (ties -> lower id) and
// softmax gates over the selected logits.
//
// The Strata pages name a dedicated router kernel (bnskd "Strata：把 125B 大模型
// 塞进 12GB 显卡", section 代码结构) and state that each token is sent to 10 of
// the experts (same page, section 核心思路); the kernels here are this
// library's own design for gfx950.
//
// Two paths:
//  * small batches (T <= 8, decode and verify): the 4 MB router matrix is the
//    whole cost, so it is split over 64x64 (expert x d) tiles, one per
//    workgroup, each reading 16 KB with 128-bit loads.  Partial sums are
//    reduced by the last workgroup of each expert column ("last block done"
//    counters), and the last column finisher selects the top-k.
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

__device__ __forceinline__ bool better(double a, int ia, double b, int ib) {
    return a > b || (a == b && ia < ib);
}

// One wavefront selects the top-k of z[0..E) (E <= 1024) and writes ids and
// gates.  Ranks by (z descending, id ascending); -0.0 == +0.0 by IEEE compare.
__device__ void wave_topk(const double* z, int E, int K, int32_t* ids, float* gates) {
    const int lane = threadIdx.x & 63;
    constexpr int kPer = kMaxExperts / 64;
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

// ---------------------------------------------------------------- small T
// grid: (ceil(E/64), ceil(D/64)), block 256.  Thread (rg = tid/16, c = tid%16)
// handles experts e0 + 4c .. +3 for rows d0 + rg + 16 i, i < 4.
template <int T>
__global__ __launch_bounds__(256) void route_small_kernel(moe_router_t r, const void* __restrict__ x,
                                                          int x_bf16, int32_t* __restrict__ ids,
                                                          float* __restrict__ gates,
                                                          double* __restrict__ zpart,
                                                          double* __restrict__ zfull,
                                                          int* __restrict__ counters) {
    const int E = r.n_experts, D = r.d_model;
    const int ec = blockIdx.x, dc = blockIdx.y;
    const int ndc = gridDim.y, nec = gridDim.x;
    const int e0 = ec * kRouteSmallE, d0 = dc * kRouteSmallD;
    const int tid = threadIdx.x;
    const int rg = tid >> 4, c = tid & 15;

    __shared__ double xs[T][kRouteSmallD];
    __shared__ double red[4][T][kRouteSmallE];
    __shared__ int s_last;

    // issue the weight loads first (16 KB per workgroup, 4 x 16 B per thread)
    float4 wv[4];
    const bool full_e = (e0 + kRouteSmallE <= E) && (E % 4 == 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int d = d0 + rg + 16 * i;
        if (d < D && full_e) {
            wv[i] = *reinterpret_cast<const float4*>(r.w + (size_t)d * E + e0 + 4 * c);
        } else {
            float t4[4];
            for (int q = 0; q < 4; ++q) {
                const int e = e0 + 4 * c + q;
                t4[q] = (d < D && e < E) ? r.w[(size_t)d * E + e] : 0.0f;
            }
            wv[i] = make_float4(t4[0], t4[1], t4[2], t4[3]);
        }
    }
    for (int i = tid; i < T * kRouteSmallD; i += 256) {
        const int t = i / kRouteSmallD, dd = i % kRouteSmallD;
        const int d = d0 + dd;
        xs[t][dd] = d < D ? load_x(x, x_bf16, (size_t)t * D + d) : 0.0;
    }
    __syncthreads();

    double acc[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[t][q] = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double w4[4] = {(double)wv[i].x, (double)wv[i].y, (double)wv[i].z, (double)wv[i].w};
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const double xv = xs[t][rg + 16 * i];
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[t][q] = fma(xv, w4[q], acc[t][q]);
        }
    }
    // reduce the 4 row groups of a wavefront (lanes 16 apart), then the 4 waves
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            double v = acc[t][q];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc[t][q] = v;
        }
    const int wave = tid >> 6;
    if ((tid & 63) < 16) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) red[wave][t][4 * c + q] = acc[t][q];
    }
    __syncthreads();
    for (int i = tid; i < T * kRouteSmallE; i += 256) {
        const int t = i / kRouteSmallE, ee = i % kRouteSmallE;
        if (e0 + ee >= E) continue;
        const double sum = ((red[0][t][ee] + red[1][t][ee]) + red[2][t][ee]) + red[3][t][ee];
        zpart[((size_t)dc * T + t) * E + e0 + ee] = sum;
    }

    // last d-chunk of this expert column reduces the partials in d order
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&counters[ec], 1) == ndc - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int i = tid; i < T * kRouteSmallE; i += 256) {
        const int t = i / kRouteSmallE, e = e0 + i % kRouteSmallE;
        if (e >= E) continue;
        double s = 0.0;
        for (int k = 0; k < ndc; ++k) s += zpart[((size_t)k * T + t) * E + e];
        if (r.bias) s += (double)r.bias[e];
        zfull[(size_t)t * E + e] = s;
    }
    if (tid == 0) counters[ec] = 0;
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&counters[nec], 1) == nec - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (tid == 0) counters[nec] = 0;
    for (int t = wave; t < T; t += 4)
        wave_topk(zfull + (size_t)t * E, E, r.top_k, ids + (size_t)t * r.top_k, gates + (size_t)t * r.top_k);
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
            const int dd = i / kRouteTileE, ee = i % kRouteTileE;
            const int d = d0 + dd, e = e0 + ee;
            ws_[dd][ee] = (d < D && e < E) ? (double)r.w[(size_t)d * E + e] : 0.0;
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
    dim3 grid(cdiv(r.n_experts, kRouteSmallE), cdiv(r.d_model, kRouteSmallD));
    double* zpart = (double*)(ws + L.zpart);
    double* zfull = (double*)(ws + L.zfull);
    int* counters = (int*)(ws + L.counters);
    switch (T) {
#define QMOE_CASE(N)                                                                                       \
    case N:                                                                                                \
        route_small_kernel<N><<<grid, 256, 0, s>>>(r, x, x_bf16, ids, gates, zpart, zfull, counters); \
        break;
        QMOE_CASE(1) QMOE_CASE(2) QMOE_CASE(3) QMOE_CASE(4) QMOE_CASE(5) QMOE_CASE(6) QMOE_CASE(7) QMOE_CASE(8)
#undef QMOE_CASE
        default:
            return hipErrorInvalidValue;
    }
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

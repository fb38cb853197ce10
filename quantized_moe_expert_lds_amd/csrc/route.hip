// Router: logits z = x W + b in fp64, top-k selection (ties -> lower id) and
// softmax gates over the selected logits.
//
// The Strata pages name a dedicated router kernel (bnskd "Strata：把 125B 大模型
// 塞进 12GB 显卡", section 代码结构) and state that each token is sent to 10 of
// the experts (same page, section 核心思路); the kernels here are this
// library's own design for gfx950.
//
// Two paths:
//  * small batches (T <= 8, decode and verify): one launch.  Reading the
//    router matrix is the whole cost of the logits.  The router is stored
//    expert-major ([E][d_model]), so each workgroup reads the contiguous rows
//    of two experts (16 KB) with 128-bit loads and produces complete logits;
//    the last workgroup to finish (a counter in the workspace) selects the
//    top-k of every token, one wavefront per token, with the selections of
//    the decode-step kernel.
//  * large batches (prefill): an fp64 GEMM on the matrix cores
//    (v_mfma_f64_16x16x4_f64) in which every logit is accumulated over d in
//    ascending order, one fused multiply-add per d (each fp32 x fp32 product
//    is exact in fp64, so this is the same rounding sequence as the plain
//    definition; a GPU test checks the logits bit for bit), then one
//    wavefront per token selects the top-k.
#include "wave_ops.hpp"

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
//
// Then the workgroups count themselves out on a counter in the workspace
// (the pattern of a fence by every writer, a barrier and one atomic add per
// workgroup); the one that brings it to the grid size has every logit in
// view after its own fence, selects the top-k of each token (wave v takes
// tokens v, v + 4: the histogram selection, or the round-by-round one when
// it declines) and resets the counter to zero for the next call.
template <int T, int KPER>
__global__ __launch_bounds__(256) void route_small_kernel(moe_router_t r, const void* __restrict__ x, int x_bf16,
                                                          double* __restrict__ z, unsigned* __restrict__ counter,
                                                          int32_t* __restrict__ ids, float* __restrict__ gates) {
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
        __threadfence();
    }
    __shared__ int s_last;
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(counter, 1u) == gridDim.x - 1;
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // the last workgroup: the selections, reading the logits from memory
    const int K = r.top_k;
    __shared__ double s_cv[4][128];
    __shared__ int s_ci[4][128];
    __shared__ unsigned s_ck[4][64];
    __shared__ int s_hist[4][128];
    __shared__ double s_sv[4][64];
    __shared__ int s_si[4][64];
    for (int t = wave; t < T; t += 4) {
        const double* zt = z + (size_t)t * E;
        if (!wave_topk_hist<KPER>(zt, E, K, s_sv[wave], s_si[wave], s_hist[wave], s_cv[wave], s_ci[wave]))
            wave_topk_core<KPER>(zt, 0, E, K, s_sv[wave], s_si[wave], s_ck[wave]);
        __builtin_amdgcn_wave_barrier();
        wave_gates(s_sv[wave], s_si[wave], K, ids + (size_t)t * K, gates + (size_t)t * K);
        __builtin_amdgcn_wave_barrier();
    }
    if (tid == 0) *counter = 0u;
}

// ---------------------------------------------------------------- large T
// fp64 matrix cores (v_mfma_f64_16x16x4_f64).  A block of 256 threads
// computes a 64-token x 64-expert tile of z; d runs in chunks of 32 through
// LDS, where x and w sit as fp64, transposed ([d][token], [d][expert]) so a
// fragment read is 16 consecutive doubles.  Wave v owns tokens
// 32 (v & 1) .. +32 and experts 32 (v >> 1) .. +32: 2 x 2 MFMA tiles, each
// accumulating over d in ascending groups of 4.  The next chunk is loaded
// into registers while the current one multiplies.  An 8,192-token chunk
// over 512 experts gives 1,024 blocks, four per CU (four waves per SIMD to
// cover the barriers and loads); 128-token tiles (two per CU) took ~30 us
// more per chunk, 32-token tiles ~15 us more.
typedef double double4_t __attribute__((ext_vector_type(4)));
constexpr int kR64T = 64, kR64E = 64, kR64K = 32;

__global__ __launch_bounds__(256, 4) void route_gemm_kernel(moe_router_t r, const void* __restrict__ x,
                                                            int x_bf16, int T, double* __restrict__ z) {
    const int E = r.n_experts, D = r.d_model;
    const int e0 = blockIdx.x * kR64E, t0 = blockIdx.y * kR64T;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int kTI = kR64T / 32, kXL = kR64T * kR64K / 4 / 256;   // token tiles per wave, x loads per thread
    const int wt = (kR64T / 2) * (wave & 1), we = 32 * (wave >> 1);
    __shared__ double xs[kR64K][kR64T + 1];
    __shared__ double ws_[kR64K][kR64E + 1];

    // staging: float4 f = tid + 256 i of a chunk holds d 4 (f & 7) .. +3 of
    // token (or expert) f >> 3
    float4 xr[kXL], wr[2];
    auto load = [&](int d0) {
#pragma unroll
        for (int i = 0; i < kXL; ++i) {
            const int f = tid + 256 * i, t = t0 + (f >> 3), d = d0 + 4 * (f & 7);
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (t < T) {
                const size_t o = (size_t)t * D + d;
                if (x_bf16) {
                    const uint2 b = *reinterpret_cast<const uint2*>((const uint16_t*)x + o);
                    v = make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u),
                                    __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xffff0000u));
                } else {
                    v = *reinterpret_cast<const float4*>((const float*)x + o);
                }
            }
            xr[i] = v;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int f = tid + 256 * i, e = e0 + (f >> 3), d = d0 + 4 * (f & 7);
            wr[i] = e < E ? *reinterpret_cast<const float4*>(r.w + (size_t)e * D + d) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < kXL; ++i) {
            const int f = tid + 256 * i, t = f >> 3, dd = 4 * (f & 7);
            xs[dd][t] = xr[i].x;
            xs[dd + 1][t] = xr[i].y;
            xs[dd + 2][t] = xr[i].z;
            xs[dd + 3][t] = xr[i].w;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int f = tid + 256 * i, e = f >> 3, dd = 4 * (f & 7);
            ws_[dd][e] = wr[i].x;
            ws_[dd + 1][e] = wr[i].y;
            ws_[dd + 2][e] = wr[i].z;
            ws_[dd + 3][e] = wr[i].w;
        }
    };

    double4_t acc[kTI][2];
#pragma unroll
    for (int i = 0; i < kTI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = double4_t{0.0, 0.0, 0.0, 0.0};
    load(0);
    for (int d0 = 0; d0 < D; d0 += kR64K) {
        store();
        __syncthreads();
        load(min(d0 + kR64K, D - kR64K));                // the last reload is unused
#pragma unroll
        for (int kk = 0; kk < kR64K / 4; ++kk) {
            const int k = 4 * kk + (lane >> 4);
            double a[kTI], b[2];
#pragma unroll
            for (int i = 0; i < kTI; ++i) a[i] = xs[k][wt + 16 * i + (lane & 15)];
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = ws_[k][we + 16 * j + (lane & 15)];
#pragma unroll
            for (int i = 0; i < kTI; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    // lane l holds rows (l >> 4) + 4 v, v = 0..3, of column l & 15 of each tile
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = e0 + we + 16 * j + (lane & 15);
        if (e >= E) continue;
        const double bias = r.bias ? (double)r.bias[e] : 0.0;
#pragma unroll
        for (int i = 0; i < kTI; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + wt + 16 * i + (lane >> 4) + 4 * v;
                if (t < T) z[(size_t)t * E + e] = r.bias ? acc[i][j][v] + bias : acc[i][j][v];
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

template <int KPER>
hipError_t launch_route_small_k(const moe_router_t& r, const void* x, int x_bf16, int T, int32_t* ids,
                                float* gates, double* z, unsigned* counter, hipStream_t s) {
    const unsigned grid = (unsigned)cdiv(r.n_experts, 2);
    switch (T) {
#define QMOE_CASE(N)                                                                                  \
    case N:                                                                                           \
        route_small_kernel<N, KPER><<<grid, 256, 0, s>>>(r, x, x_bf16, z, counter, ids, gates); \
        break;
        QMOE_CASE(1) QMOE_CASE(2) QMOE_CASE(3) QMOE_CASE(4) QMOE_CASE(5) QMOE_CASE(6) QMOE_CASE(7) QMOE_CASE(8)
#undef QMOE_CASE
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_route_small(const moe_router_t& r, const void* x, int x_bf16, int T, int32_t* ids,
                              float* gates, char* ws, const RouteWs& L, hipStream_t s) {
    double* z = (double*)(ws + L.zfull);
    unsigned* counter = (unsigned*)(ws + L.counter);
    // logits per lane in the selections: a compile-time bound on n_experts
    if (r.n_experts <= 128) return launch_route_small_k<2>(r, x, x_bf16, T, ids, gates, z, counter, s);
    if (r.n_experts <= 512) return launch_route_small_k<8>(r, x, x_bf16, T, ids, gates, z, counter, s);
    return launch_route_small_k<16>(r, x, x_bf16, T, ids, gates, z, counter, s);
}

hipError_t launch_route_large(const moe_router_t& r, const void* x, int x_bf16, int T, int32_t* ids,
                              float* gates, char* ws, const RouteWs& L, hipStream_t s) {
    double* z = (double*)(ws + L.zfull);
    dim3 grid(cdiv(r.n_experts, kR64E), cdiv(T, kR64T));
    route_gemm_kernel<<<grid, 256, 0, s>>>(r, x, x_bf16, T, z);
    topk_kernel<<<cdiv(T, 4), 256, 0, s>>>(z, T, r.n_experts, r.top_k, ids, gates);
    return hipGetLastError();
}

}  // namespace qmoe

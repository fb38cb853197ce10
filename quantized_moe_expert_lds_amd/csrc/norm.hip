// Residual update and RMSNorm between chained MoE layers:
//   h += y;  u = h / sqrt(mean(h^2) + eps)   (mean square in fp64, gamma = 1)
// The pages chain 48 layers per forward (bnskd "Strata：把 125B 大模型塞进 12GB
// 显卡", section 投机解码); the norm between layers is this library's plain
// reading of a residual stream with a pre-norm.
// One workgroup per token; the fp64 sum uses a fixed tree, so the result is
// deterministic and independent of the batch.
#include "common.hpp"

namespace {

__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(float* __restrict__ h, const float* __restrict__ y,
                                                               float* __restrict__ u, int d, double eps) {
    const int t = blockIdx.x, tid = threadIdx.x;
    float* hr = h + (size_t)t * d;
    float* ur = u + (size_t)t * d;
    double ss = 0.0;
    for (int i = tid; i < d; i += 256) {
        float v = hr[i];
        if (y) {
            v = v + y[(size_t)t * d + i];
            hr[i] = v;
        }
        ss += (double)v * (double)v;
    }
    __shared__ double red[256];
    red[tid] = ss;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (tid < off) red[tid] += red[tid + off];
        __syncthreads();
    }
    const double r = sqrt(red[0] / (double)d + eps);
    for (int i = tid; i < d; i += 256) ur[i] = (float)((double)hr[i] / r);
}

// x (fp32 or bf16) -> fp32, the first residual of a chunk
__global__ __launch_bounds__(256) void to_f32_kernel(const void* __restrict__ x, int x_bf16, size_t n,
                                                     float* __restrict__ out) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    out[i] = x_bf16 ? __uint_as_float((uint32_t)((const uint16_t*)x)[i] << 16) : ((const float*)x)[i];
}

}  // namespace

namespace qmoe {

hipError_t launch_to_f32(const void* x, int x_bf16, size_t n, float* out, hipStream_t s) {
    to_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(x, x_bf16, n, out);
    return hipGetLastError();
}

hipError_t launch_residual_rmsnorm(float* h, const float* y, float* u, int T, int d, double eps, hipStream_t s) {
    residual_rmsnorm_kernel<<<T, 256, 0, s>>>(h, y, u, d, eps);
    return hipGetLastError();
}

}  // namespace qmoe

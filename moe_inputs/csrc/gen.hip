// GPU twin of the seeded expert-weight generator of moe_inputs/__init__.py.
//
// Input preparation only (the weights a model would load from disk): draws
// N(0, sigma) values from the SplitMix64 counter stream of each expert, maps
// 16-bit lanes through the normal-quantile table, quantises each 32-weight
// block (absmax scale in fp16, round-half-even levels) and packs the codes.
// Every step after the table lookup is an IEEE-exact or correctly rounded
// fp32 operation, so the bytes equal the host generator's (checked by test).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kM1 = 0xBF58476D1CE4E5B9ull;
constexpr uint64_t kM2 = 0x94D049BB133111EBull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * kM1;
    z = (z ^ (z >> 27)) * kM2;
    return z ^ (z >> 31);
}

// one thread per (expert, row, block)
template <int BITS>
__global__ __launch_bounds__(256) void gen_kernel(const uint64_t* __restrict__ keys, int n_experts, int N, int K,
                                                  float sigma, const float* __restrict__ table,
                                                  uint32_t* __restrict__ q, uint16_t* __restrict__ s) {
    const int nkb = K >> 5;
    const size_t per_expert = (size_t)N * nkb;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= per_expert * n_experts) return;
    const int e = (int)(idx / per_expert);
    const size_t rb = idx - (size_t)e * per_expert;
    const int n = (int)(rb / nkb), kb = (int)(rb - (size_t)n * nkb);
    const uint64_t key = keys[e];
    const uint64_t c0 = ((uint64_t)n * K + 32ull * kb) >> 2;    // first stream output of the block
    float w[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint64_t h = mix64(key + (c0 + i + 1) * kGamma);
#pragma unroll
        for (int l = 0; l < 4; ++l) w[4 * i + l] = sigma * table[(h >> (16 * l)) & 0xFFFF];
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(w[i]));
    const float half = BITS == 2 ? 2.0f : 4.0f;
    const _Float16 s16 = (_Float16)(a / half);
    const float sf = (float)s16;
    const int lo = BITS == 2 ? -2 : -4, hi = BITS == 2 ? 1 : 3;
    uint32_t code[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        int lev = 0;
        if (sf > 0.0f) {
            const float r = rintf(w[i] / sf);
            lev = (int)fminf(fmaxf(r, (float)lo), (float)hi);
        }
        code[i] = (uint32_t)(lev - lo);
    }
    const size_t blk = (size_t)e * per_expert + rb;
    if (BITS == 2) {
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            w0 |= code[i] << (2 * i);
            w1 |= code[16 + i] << (2 * i);
        }
        q[blk * 2] = w0;
        q[blk * 2 + 1] = w1;
    } else {
        uint32_t ww[3] = {0, 0, 0};
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int pos = 3 * i, wd = pos >> 5, off = pos & 31;
            ww[wd] |= code[i] << off;
            if (off > 29) ww[wd + 1] |= code[i] >> (32 - off);
        }
        q[blk * 3] = ww[0];
        q[blk * 3 + 1] = ww[1];
        q[blk * 3 + 2] = ww[2];
    }
    s[blk] = __builtin_bit_cast(uint16_t, s16);
}

}  // namespace

extern "C" int moegen_expert_tensors(const uint64_t* keys, int n_experts, int N, int K, int bits, float sigma,
                                     const float* table, uint32_t* q, uint16_t* s, void* stream) {
    if (!keys || !table || !q || !s || n_experts <= 0 || N <= 0 || K <= 0 || K % 32) return -1;
    if (bits != 2 && bits != 3) return -2;
    const size_t total = (size_t)n_experts * N * (K / 32);
    const unsigned grid = (unsigned)((total + 255) / 256);
    hipStream_t st = (hipStream_t)stream;
    if (bits == 2)
        gen_kernel<2><<<grid, 256, 0, st>>>(keys, n_experts, N, K, sigma, table, q, s);
    else
        gen_kernel<3><<<grid, 256, 0, st>>>(keys, n_experts, N, K, sigma, table, q, s);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

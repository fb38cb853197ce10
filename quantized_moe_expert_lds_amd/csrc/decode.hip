// Decode / verify expert FFN: fused dequantisation + gate/up GEMV + SwiGLU,
// then dequantisation + down GEMV + slot-ordered weighted combine.
//
// The pages call decode bandwidth-limited and stream the experts of every
// token from memory (bnskd "Strata：把 125B 大模型塞进 12GB 显卡", section 核心
// 思路); each token uses 10 experts (same section).  On one MI355X every
// expert is resident in HBM, so the kernels are built to stream the packed
// blocks of the selected experts once per call:
//
//  * gate/up (grid: pair slot x 16 d_ff rows): one wavefront owns 4 gate and
//    4 up rows; lane l owns 32-weight block l (and l + 64, ...) of every row,
//    so a wavefront load of one row is one contiguous 512-byte segment.  Codes
//    are unpacked two at a time into fp16 pairs by OR-ing them into the
//    mantissa of 1024.0, the bias is removed with one packed fp16 add (exact),
//    and v_dot2_f32_f16 multiplies them with the fp16 activations, fp32
//    accumulation; the block scale is applied once per block.  Each expert is
//    handled by the first slot that names it, for every token that chose it.
//  * down (grid: 8 output rows per workgroup): thread (slot, block) streams
//    its block of the 8 rows, partial sums go to LDS, and one thread per
//    (token, row) adds the blocks in order and the k slots in order with
//    their gates.
//
// Every per-token quantity is computed by the same instruction sequence for
// any batch size, so results do not depend on n_tokens (bitwise).
#include <atomic>

#include "common.hpp"

namespace {

using namespace qmoe;
using namespace qmoe_dev;

constexpr int kGuRowsPerWave = 4;                 // f values per wavefront
constexpr int kGuRowsPerBlock = 4 * kGuRowsPerWave;  // f values per workgroup
constexpr int kDownRowsMax = 8;                   // output rows per workgroup (fewer when LDS is short)
constexpr size_t kDownLdsLimit = 64 * 1024;

__device__ __forceinline__ float half_bits_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// x values of block kb of token row xrow -> 16 fp16 pairs in the unpack
// order (pair m = (x[m], x[m+8]), pair 8+m = (x[16+m], x[24+m])), as two
// halves: xp[0..15] = fp16(x), xp[16..31] = fp16(x - fp16(x)).  Together
// they carry ~22 significant bits of x into the dot products.
__device__ __forceinline__ void load_x_pairs(const void* x, int x_bf16, size_t row_off, int kb,
                                             uint32_t* xp) {
    float v[32];
    if (x_bf16) {
        const uint4* p = reinterpret_cast<const uint4*>((const uint16_t*)x + row_off + 32 * kb);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 u = p[q];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[8 * q + 2 * h] = __uint_as_float(w[h] << 16);
                v[8 * q + 2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
            }
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>((const float*)x + row_off + 32 * kb);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float4 f = p[q];
            v[4 * q] = f.x;
            v[4 * q + 1] = f.y;
            v[4 * q + 2] = f.z;
            v[4 * q + 3] = f.w;
        }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int ia[4] = {m, m + 8, 16 + m, 24 + m};
        _Float16 hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            hi[i] = (_Float16)v[ia[i]];
            lo[i] = (_Float16)(v[ia[i]] - (float)hi[i]);
        }
        xp[m] = as_u32(half2_t{hi[0], hi[1]});
        xp[8 + m] = as_u32(half2_t{hi[2], hi[3]});
        xp[16 + m] = as_u32(half2_t{lo[0], lo[1]});
        xp[24 + m] = as_u32(half2_t{lo[2], lo[3]});
    }
}

// Levels of one block as 16 fp16 pairs, same pair order as load_x_pairs.
template <int BITS>
__device__ __forceinline__ void block_levels(const uint32_t* w, uint32_t* lv) {
    if constexpr (BITS == 2) {
        const half2_t bias = {(_Float16)-1026.0f, (_Float16)-1026.0f};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            lv[m] = as_u32(as_half2(codes2_pair(w[0], 2 * m)) + bias);
            lv[8 + m] = as_u32(as_half2(codes2_pair(w[1], 2 * m)) + bias);
        }
    } else {
        const half2_t bias = {(_Float16)-1028.0f, (_Float16)-1028.0f};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            lv[m] = as_u32(as_half2(codes3_pair(w[0], w[1], w[2], m)) + bias);
            lv[8 + m] = as_u32(as_half2(codes3_pair(w[0], w[1], w[2], 16 + m)) + bias);
        }
    }
}

// levels . (hi + lo) with the operand halves as load_x_pairs lays them out;
// the small lo terms are summed first
__device__ __forceinline__ float dot32(const uint32_t* lv, const uint32_t* xp) {
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < 16; ++m) acc = __builtin_amdgcn_fdot2(as_half2(lv[m]), as_half2(xp[16 + m]), acc, false);
#pragma unroll
    for (int m = 0; m < 16; ++m) acc = __builtin_amdgcn_fdot2(as_half2(lv[m]), as_half2(xp[m]), acc, false);
    return acc;
}

// ------------------------------------------------------------- gate / up
// grid (T*K, F/16), block 256.  hbuf: fp16 [2][T*K][F]: hbuf[0] holds
// fp16(h), hbuf[1] fp16(h - fp16(h)), each 32-block stored in the unpack pair
// order (position perm32(i) holds element i).
template <int T, int BITS>
__global__ __launch_bounds__(256) void decode_gateup_kernel(moe_experts_t ex, const void* __restrict__ x,
                                                            int x_bf16, const int32_t* __restrict__ ids,
                                                            int K, uint16_t* __restrict__ hbuf) {
    constexpr int W = BITS == 2 ? 2 : 3;
    const int D = ex.d_model, F = ex.d_ff;
    const int nkb = D >> 5;
    const int slot = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ int s_pair[T];
    __shared__ int s_skip;

    const int e = ids[slot];
    if (tid == 0) {
        int dup = (e < 0 || e >= ex.n_experts);      // out-of-range ids are skipped
        for (int p = 0; p < slot; ++p) dup |= (ids[p] == e);
        s_skip = dup;
    }
    if (tid < T) {
        int pr = -1;
        for (int j = 0; j < K; ++j)
            if (ids[tid * K + j] == e) pr = tid * K + j;
        s_pair[tid] = pr;
    }
    __syncthreads();
    if (s_skip) return;

    const int f0 = blockIdx.y * kGuRowsPerBlock + wave * kGuRowsPerWave;
    // rows 0..3: gate rows f0..f0+3, rows 4..7: up rows f0..f0+3
    const uint32_t* qrow[2 * kGuRowsPerWave];
    const uint16_t* srow[2 * kGuRowsPerWave];
#pragma unroll
    for (int r = 0; r < kGuRowsPerWave; ++r) {
        const size_t rg = ((size_t)e * F + f0 + r) * nkb;
        qrow[r] = ex.gate_q + rg * W;
        srow[r] = ex.gate_s + rg;
        qrow[kGuRowsPerWave + r] = ex.up_q + rg * W;
        srow[kGuRowsPerWave + r] = ex.up_s + rg;
    }

    float acc[2 * kGuRowsPerWave][T];
#pragma unroll
    for (int r = 0; r < 2 * kGuRowsPerWave; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t) acc[r][t] = 0.0f;

    for (int kb = lane; kb < nkb; kb += 64) {
        uint32_t q[2 * kGuRowsPerWave][W];
        float sc[2 * kGuRowsPerWave];
#pragma unroll
        for (int r = 0; r < 2 * kGuRowsPerWave; ++r) {
            if constexpr (W == 2) {
                const uint2 v = *reinterpret_cast<const uint2*>(qrow[r] + (size_t)kb * 2);
                q[r][0] = v.x;
                q[r][1] = v.y;
            } else {
                const uint32_t* p = qrow[r] + (size_t)kb * 3;
                q[r][0] = p[0];
                q[r][1] = p[1];
                q[r][2] = p[2];
            }
            sc[r] = half_bits_to_f32(srow[r][kb]);
        }
        uint32_t xp[T][32];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (s_pair[t] >= 0) load_x_pairs(x, x_bf16, (size_t)t * D, kb, xp[t]);
        }
#pragma unroll
        for (int r = 0; r < 2 * kGuRowsPerWave; ++r) {
            uint32_t lv[16];
            block_levels<BITS>(q[r], lv);
#pragma unroll
            for (int t = 0; t < T; ++t)
                if (s_pair[t] >= 0) acc[r][t] = fmaf(sc[r], dot32(lv, xp[t]), acc[r][t]);
        }
    }
    // wavefront sums (same butterfly for every row and token)
#pragma unroll
    for (int r = 0; r < 2 * kGuRowsPerWave; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t) {
            float v = acc[r][t];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            acc[r][t] = v;
        }
    // lane (r, t) writes h for f0 + r and token t
#pragma unroll
    for (int r = 0; r < kGuRowsPerWave; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (lane == r * T + t && s_pair[t] >= 0) {
                const float h = silu_mul(acc[r][t], acc[kGuRowsPerWave + r][t]);
                const int f = f0 + r;
                const _Float16 hh = (_Float16)h;
                const _Float16 hl = (_Float16)(h - (float)hh);
                const size_t hi = (size_t)s_pair[t] * F + (f & ~31) + perm32(f & 31);
                hbuf[hi] = __builtin_bit_cast(uint16_t, hh);
                hbuf[(size_t)T * K * F + hi] = __builtin_bit_cast(uint16_t, hl);
            }
        }
}

// ----------------------------------------------------------------- down
// grid D/R, block 256, dynamic LDS: part[T*K][R][nkbF] floats.
template <int T, int BITS, int kDownRows>
__global__ __launch_bounds__(256) void decode_down_kernel(moe_experts_t ex, const int32_t* __restrict__ ids,
                                                          const float* __restrict__ gates, int K,
                                                          const uint16_t* __restrict__ hbuf,
                                                          float* __restrict__ y) {
    constexpr int W = BITS == 2 ? 2 : 3;
    const int D = ex.d_model, F = ex.d_ff;
    const int nkb = F >> 5;
    const int P = T * K;
    const int d0 = blockIdx.x * kDownRows;
    const int tid = threadIdx.x;
    // dynamic LDS: part [P][kDownRows][nkb] floats | s_e [P] ints |
    // s_pair [P][T] shorts (pair of token t using slot p's expert, or -1) |
    // s_first [P] bytes (slot p is the first that names its expert)
    extern __shared__ float part[];
    int* s_e = reinterpret_cast<int*>(part + (size_t)P * kDownRows * nkb);
    short* s_pair = reinterpret_cast<short*>(s_e + P);
    signed char* s_first = reinterpret_cast<signed char*>(s_pair + (size_t)P * T);

    for (int p = tid; p < P; p += 256) s_e[p] = ids[p];
    __syncthreads();
    for (int p = tid; p < P; p += 256) {
        const int e = s_e[p];
        int first = (e >= 0 && e < ex.n_experts);     // out-of-range ids are skipped
        for (int q = 0; q < p; ++q) first &= (s_e[q] != e);
        s_first[p] = (signed char)first;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            int pr = -1;
            for (int j = 0; j < K; ++j)
                if (s_e[t * K + j] == e) pr = t * K + j;
            s_pair[p * T + t] = (short)pr;
        }
    }
    __syncthreads();

    for (int it = tid; it < P * nkb; it += 256) {
        const int p = it / nkb, kb = it - p * nkb;
        if (!s_first[p]) continue;
        const int e = s_e[p];
        uint32_t q[kDownRows][W];
        float sc[kDownRows];
#pragma unroll
        for (int r = 0; r < kDownRows; ++r) {
            const size_t rg = ((size_t)e * D + d0 + r) * nkb + kb;
            if constexpr (W == 2) {
                const uint2 v = *reinterpret_cast<const uint2*>(ex.down_q + rg * 2);
                q[r][0] = v.x;
                q[r][1] = v.y;
            } else {
                const uint32_t* pq = ex.down_q + rg * 3;
                q[r][0] = pq[0];
                q[r][1] = pq[1];
                q[r][2] = pq[2];
            }
            sc[r] = half_bits_to_f32(ex.down_s[rg]);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int pr = s_pair[p * T + t];
            if (pr < 0) continue;
            uint32_t hp[32];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const uint4* hs = reinterpret_cast<const uint4*>(hbuf + (size_t)half * P * F + (size_t)pr * F + 32 * kb);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint4 u = hs[v];
                    hp[16 * half + 4 * v] = u.x;
                    hp[16 * half + 4 * v + 1] = u.y;
                    hp[16 * half + 4 * v + 2] = u.z;
                    hp[16 * half + 4 * v + 3] = u.w;
                }
            }
#pragma unroll
            for (int r = 0; r < kDownRows; ++r) {
                uint32_t lv[16];
                block_levels<BITS>(q[r], lv);
                part[((size_t)pr * kDownRows + r) * nkb + kb] = sc[r] * dot32(lv, hp);
            }
        }
    }
    __syncthreads();
    for (int o = tid; o < T * kDownRows; o += 256) {
        const int t = o / kDownRows, r = o - t * kDownRows;
        float yv = 0.0f;
        for (int j = 0; j < K; ++j) {
            const float* pp = part + ((size_t)(t * K + j) * kDownRows + r) * nkb;
            float oj = 0.0f;
            for (int kb = 0; kb < nkb; ++kb) oj += pp[kb];
            yv = yv + gates[t * K + j] * oj;
        }
        y[(size_t)t * D + d0 + r] = yv;
    }
}

size_t down_lds_bytes(int T, int K, int F, int R) {
    const size_t P = (size_t)T * K;
    return sizeof(float) * P * R * (F / 32) + sizeof(int) * P + sizeof(short) * P * T + P;
}

// rows per down workgroup: the most (<= 8) whose partials fit in LDS, 0 if none
int down_rows(int T, int K, int F) {
    for (int R = kDownRowsMax; R >= 1; R >>= 1)
        if (down_lds_bytes(T, K, F, R) <= kDownLdsLimit) return R;
    return 0;
}

template <int T, int BITS>
hipError_t launch_decode_t(const moe_experts_t& ex, const void* x, int x_bf16, const int32_t* ids,
                           const float* gates, int K, float* y, uint16_t* hbuf, hipStream_t s) {
    dim3 g1(T * K, ex.d_ff / kGuRowsPerBlock);
    decode_gateup_kernel<T, BITS><<<g1, 256, 0, s>>>(ex, x, x_bf16, ids, K, hbuf);
    const int R = down_rows(T, K, ex.d_ff);
    const size_t lds = down_lds_bytes(T, K, ex.d_ff, R);
    switch (R) {
        case 8: decode_down_kernel<T, BITS, 8><<<ex.d_model / 8, 256, lds, s>>>(ex, ids, gates, K, hbuf, y); break;
        case 4: decode_down_kernel<T, BITS, 4><<<ex.d_model / 4, 256, lds, s>>>(ex, ids, gates, K, hbuf, y); break;
        case 2: decode_down_kernel<T, BITS, 2><<<ex.d_model / 2, 256, lds, s>>>(ex, ids, gates, K, hbuf, y); break;
        case 1: decode_down_kernel<T, BITS, 1><<<ex.d_model, 256, lds, s>>>(ex, ids, gates, K, hbuf, y); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

namespace qmoe {
bool decode_supported(int T, int K, int F) { return down_rows(T, K, F) > 0; }
}  // namespace qmoe

// ------------------------------------------------ allocation-free variant
// moe_ffn_decode_noalloc keeps the SwiGLU intermediate in this file-scope
// array instead of a caller workspace.  Each device holds its own copy until
// the process ends.  On the host, `scratch` names only a stand-in for the
// symbol: host code passes kernels the device address hipGetSymbolAddress
// returns for the current device, looked up once per device.
namespace {

constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[qmoe::kDecodeScratchBytes];
std::atomic<char*> g_scratch_ptr[kScratchDevices];

}  // namespace

namespace qmoe {

hipError_t decode_noalloc_scratch(char** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    char* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        p = static_cast<char*>(a);
        // two threads racing here store the same address
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace qmoe

namespace qmoe {

hipError_t launch_decode(const moe_experts_t& ex, const void* x, int x_bf16, int T, const int32_t* ids,
                         const float* gates, int K, float* y, char* ws, const DecodeWs& L, hipStream_t s) {
    uint16_t* hbuf = (uint16_t*)(ws + L.h);
#define QMOE_DEC(N)                                                                              \
    case N:                                                                                      \
        return ex.bits == 2 ? launch_decode_t<N, 2>(ex, x, x_bf16, ids, gates, K, y, hbuf, s) \
                            : launch_decode_t<N, 3>(ex, x, x_bf16, ids, gates, K, y, hbuf, s);
    switch (T) {
        QMOE_DEC(1) QMOE_DEC(2) QMOE_DEC(3) QMOE_DEC(4) QMOE_DEC(5) QMOE_DEC(6) QMOE_DEC(7) QMOE_DEC(8)
        default:
            return hipErrorInvalidValue;
    }
#undef QMOE_DEC
}

}  // namespace qmoe

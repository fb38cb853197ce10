// Prefill expert FFN with int8 activations ("MMQ-style"): the expert matmuls
// run on the int8 matrix cores (v_mfma_i32_16x16x32_i8) with the 2-bit
// weights as int8 levels and the activations quantised to int8.
//
// The pages run their prefill matmuls on quantised operands instead of
// first expanding the weights to fp16 (bnskd "Strata：把 125B 大模型塞进 12GB 显
// 卡", section 工程细节).  Activation format (the pages leave it open): blocks
// of 32 consecutive values along the reduction axis, int8 codes
// q = round-half-even(v * (127 / amax)) and one fp32 scale d = amax / 127
// per block; blocks with amax < 2^-112 are stored as zeros.  A matmul is
//   out[r][c] = sum over blocks b of  d[r][b] * s[c][b] * I[r][c][b],
//   I[r][c][b] = sum over the block's 32 k of q[r][k] * level[c][k]
// with I exact in int32 (one MFMA over K = 32 per block) and the scaling and
// the sum over blocks in fp32.
//
// Pipeline (all on the caller's stream):
//  1. x -> Q8 blocks (codes and scales).
//  2. tile list, as for the fp16 prefill.
//  3. gate/up GEMM: 128 bucket rows x (128 d_ff columns of gate and the same
//     128 of up); epilogue h = silu(g) * u, then h -> Q8 blocks, stored in
//     bucket-row order.
//  4. down GEMM: 128 rows of h x 256 d_model columns; the epilogue scales by
//     the pair's gate and stores the row under its pair id.
//  5. combine, as for the fp16 prefill.
//
// Cost model: per output element and block the MFMA does 32 multiply-adds
// and the vector unit three instructions (int -> float, scale product,
// fused multiply-add); at 16 lanes per clock per SIMD against ~1,000 int8
// multiply-adds, the block scaling and not the matrix core bounds these
// kernels.
#include "prefill_q8.hpp"

namespace {

using namespace qmoe;
using namespace qmoe_dev;

typedef int int4_t __attribute__((ext_vector_type(4)));

constexpr int kQ8Row = kGemmBK + 8;        // bytes per LDS row of int8 operands: 8-byte aligned, and the
                                           // 16 rows of a fragment read fall in distinct bank pairs
constexpr float kQ8Tiny = 0x1p-112f;       // blocks below this amax are stored as zeros

// Q8 of 32 fp32 values held by one thread: codes packed 4 per word (little
// endian), scale returned.
__device__ __forceinline__ float q8_block(const float (&v)[32], uint32_t (&o)[8]) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0u;
    if (!(amax >= kQ8Tiny)) return 0.f;
    const float inv = __fdiv_rn(127.0f, amax);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const float s = v[i] * inv;
        const int q = min(127, max(-127, (int)__builtin_rintf(s)));
        o[i >> 2] |= ((uint32_t)q & 0xffu) << (8 * (i & 3));
    }
    return __fdiv_rn(amax, 127.0f);
}

// ------------------------------------------------------------ 1. x -> Q8
__global__ __launch_bounds__(256) void quantize_q8_kernel(const void* __restrict__ x, int x_bf16, size_t nblocks,
                                                          int8_t* __restrict__ q, float* __restrict__ d) {
    const size_t b = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    float v[32];
    if (x_bf16) {
        const uint4* p = reinterpret_cast<const uint4*>((const uint16_t*)x + b * 32);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 u = p[c];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[8 * c + 2 * h] = __uint_as_float(w[h] << 16);
                v[8 * c + 2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
            }
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>((const float*)x + b * 32);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float4 f = p[c];
            v[4 * c] = f.x;
            v[4 * c + 1] = f.y;
            v[4 * c + 2] = f.z;
            v[4 * c + 3] = f.w;
        }
    }
    uint32_t o[8];
    const float s = q8_block(v, o);
    uint4* dst = reinterpret_cast<uint4*>(q + b * 32);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    d[b] = s;
}

// 16 2-bit codes of a word -> 16 int8 levels (code - 2), 4 per output word:
// the 4 codes of a byte are spread to one byte each by two shift-ors and a
// mask, then v_perm_b32 maps each code to its level byte through a 4-entry
// table (0xFE, 0xFF, 0x00, 0x01).
__device__ __forceinline__ void levels16(uint32_t w, uint32_t (&o)[4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t v = (w >> (8 * g)) & 0xffu;
        uint32_t t = v | (v << 6);
        t = (t | (t << 12)) & 0x03030303u;
        o[g] = __builtin_amdgcn_perm(0u, 0x0100FFFEu, t);
    }
}

__device__ __forceinline__ void tile_coords(int n_ntiles, int& mt, int& nt) {
    const int b = blockIdx.x, xcd = b & 7, s = b >> 3;
    mt = (s / n_ntiles) * 8 + xcd;
    nt = s % n_ntiles;
}

// ---------------------------------------------------- 3./4. grouped GEMMs
// Both GEMMs: 256 threads (4 waves) compute a 128-row x 256-column tile, K
// in steps of 64 (two Q8 blocks) through LDS.  Wave w owns rows 64 (w & 1)
// .. +64 and LDS B rows 128 (w >> 1) .. +128: 4 x 8 MFMA tiles of 16 x 16,
// one int8 MFMA per tile and block, then the block's scaling in fp32.  The
// next step's operands are loaded into registers while the current step
// multiplies.  Thread t stages A row t >> 1 (32 of its 64 bytes and one of
// its two block scales) and B row t (codes and scales of both blocks).
struct Q8Stage {
    uint4 a[2];       // 32 bytes of A row (tid >> 1)
    float sa;         // its scale of block (tid & 1)
    uint4 b;          // codes of both blocks of B row tid
    uint32_t sb;      // their fp16 scales
};

struct Q8Src {
    const int8_t* a;      // A row + (tid & 1) * 32, or null for rows past the bucket
    const float* sa;      // A row scales + (tid & 1), or null
    const uint32_t* bq;   // B row codes
    const uint16_t* bs;   // B row scales
};

__device__ __forceinline__ void q8_load(Q8Stage& st, const Q8Src& src, int ks) {
    const int k0 = ks * kGemmBK;
    if (src.a) {
        const uint4* p = reinterpret_cast<const uint4*>(src.a + k0);
        st.a[0] = p[0];
        st.a[1] = p[1];
        st.sa = src.sa[2 * ks];
    } else {
        st.a[0] = st.a[1] = make_uint4(0, 0, 0, 0);
        st.sa = 0.f;
    }
    st.b = *reinterpret_cast<const uint4*>(src.bq + (size_t)ks * 4);
    st.sb = *reinterpret_cast<const uint32_t*>(src.bs + (size_t)ks * 2);
}

__device__ __forceinline__ void q8_store(const Q8Stage& st, int8_t (*As)[kQ8Row], int8_t (*Bs)[kQ8Row],
                                         float (*SA)[kGemmBM], float (*SB)[256], int b_lds_row) {
    const int tid = threadIdx.x;
    const int ar = tid >> 1, ah = tid & 1;
    uint2* a = reinterpret_cast<uint2*>(&As[ar][32 * ah]);
    a[0] = make_uint2(st.a[0].x, st.a[0].y);
    a[1] = make_uint2(st.a[0].z, st.a[0].w);
    a[2] = make_uint2(st.a[1].x, st.a[1].y);
    a[3] = make_uint2(st.a[1].z, st.a[1].w);
    SA[ah][ar] = st.sa;
    uint2* b = reinterpret_cast<uint2*>(&Bs[b_lds_row][0]);
    const uint32_t w[4] = {st.b.x, st.b.y, st.b.z, st.b.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t o[4];
        levels16(w[q], o);
        b[2 * q] = make_uint2(o[0], o[1]);
        b[2 * q + 1] = make_uint2(o[2], o[3]);
    }
    SB[0][b_lds_row] = (float)__builtin_bit_cast(_Float16, (uint16_t)(st.sb & 0xffffu));
    SB[1][b_lds_row] = (float)__builtin_bit_cast(_Float16, (uint16_t)(st.sb >> 16));
}

template <bool kFull>
__device__ __forceinline__ void q8_kloop(const Q8Src& src, int b_lds_row, int nsteps, int wm, int wn, int ni,
                                         int8_t (*As)[kQ8Row], int8_t (*Bs)[kQ8Row], float (*SA)[kGemmBM],
                                         float (*SB)[256], float4_t (&acc)[4][8]) {
    const int lane = threadIdx.x & 63;
    Q8Stage st;
    q8_load(st, src, 0);
    for (int ks = 0; ks < nsteps; ++ks) {
        q8_store(st, As, Bs, SA, SB, b_lds_row);
        __syncthreads();
        q8_load(st, src, min(ks + 1, nsteps - 1));   // the last reload is unused
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int kofs = kk * 32 + 8 * (lane >> 4);
            long a[4], b[8];
            float4_t sa[4];
            float sb[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = *reinterpret_cast<const long*>(&As[64 * wm + 16 * i + (lane & 15)][kofs]);
                sa[i] = *reinterpret_cast<const float4_t*>(&SA[kk][64 * wm + 16 * i + 4 * (lane >> 4)]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                b[j] = *reinterpret_cast<const long*>(&Bs[128 * wn + 16 * j + (lane & 15)][kofs]);
                sb[j] = SB[kk][128 * wn + 16 * j + (lane & 15)];
            }
            // products and their scaling at raised wave priority, as in the
            // fp16 GEMMs
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (!kFull && i >= ni) continue;            // slice beyond the bucket
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int4_t r = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[i], b[j], int4_t{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[i][j][v] = __builtin_fmaf((float)r[v], sa[i][v] * sb[j], acc[i][j][v]);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
        __syncthreads();
    }
}

// gate/up: B rows 0..127 are gate rows f0.., 128..255 the up rows f0..
__global__ __launch_bounds__(256, 2) void gemm_gateup_q8_kernel(moe_experts_t ex, const int8_t* __restrict__ xq,
                                                                const float* __restrict__ xd,
                                                                const int4* __restrict__ tiles,
                                                                const int* __restrict__ ntiles,
                                                                const int32_t* __restrict__ pairs, int K, int P,
                                                                int8_t* __restrict__ hq, float* __restrict__ hd) {
    const int D = ex.d_model, F = ex.d_ff;
    const int nkb = D >> 5, nfb = F >> 5;
    const int n_ntiles = F / kGateUpBN;
    int mt, nt;
    tile_coords(n_ntiles, mt, nt);
    if (mt >= ntiles[0]) return;
    const int4 tile = tiles[mt];
    const int e = tile.x, r0 = tile.y, r1 = tile.z;
    const int f0 = nt * kGateUpBN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = __builtin_amdgcn_readfirstlane(wave & 1), wn = __builtin_amdgcn_readfirstlane(wave >> 1);
    const int ni = __builtin_amdgcn_readfirstlane(min(4, max(0, (r1 - r0 - 64 * wm + 15) >> 4)));

    __shared__ __align__(16) int8_t As[kGemmBM][kQ8Row];
    __shared__ __align__(16) int8_t Bs[2 * kGateUpBN][kQ8Row];
    __shared__ __align__(16) float SA[2][kGemmBM];
    __shared__ __align__(16) float SB[2][256];

    Q8Src src;
    {
        const int q = r0 + (tid >> 1);
        const int p = q < r1 ? pairs[q] : -1;
        const bool ok = p >= 0 && p < P;
        const size_t t = ok ? (size_t)(p / K) : 0;
        src.a = ok ? xq + t * D + (tid & 1) * 32 : nullptr;
        src.sa = ok ? xd + t * nkb + (tid & 1) : nullptr;
    }
    const int b_row = tid;
    const int wf = f0 + (b_row & (kGateUpBN - 1));
    const size_t b_rowidx = ((size_t)e * F + wf) * nkb;
    src.bq = (b_row < kGateUpBN ? ex.gate_q : ex.up_q) + b_rowidx * 2;
    src.bs = (b_row < kGateUpBN ? ex.gate_s : ex.up_s) + b_rowidx;
    // wave wn needs gate rows 64 wn .. and up rows 128 + 64 wn ..: they are
    // made contiguous (LDS rows 128 wn .. +128) by permuting the row order;
    // tiles j < 4 are gate columns, j >= 4 the same up columns
    const int b_lds_row = 128 * ((b_row & 127) >> 6) + (b_row >= kGateUpBN ? 64 : 0) + (b_row & 63);

    float4_t acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
    if (ni == 4) q8_kloop<true>(src, b_lds_row, D / kGemmBK, wm, wn, ni, As, Bs, SA, SB, acc);
    else q8_kloop<false>(src, b_lds_row, D / kGemmBK, wm, wn, ni, As, Bs, SA, SB, acc);

    // epilogue: h = silu(g) * u, then Q8 blocks of h.  The wave's 64 d_ff
    // columns are two blocks (tiles 2c, 2c + 1); a row's block is spread over
    // the 16 lanes with the same lane >> 4, two values each.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int q = r0 + 64 * wm + 16 * i + 4 * (lane >> 4) + v;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const float h0 = silu_mul(acc[i][2 * c][v], acc[i][4 + 2 * c][v]);
                const float h1 = silu_mul(acc[i][2 * c + 1][v], acc[i][4 + 2 * c + 1][v]);
                float amax = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
                for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
                int q0 = 0, q1 = 0;
                float dq = 0.f;
                if (amax >= kQ8Tiny) {
                    const float inv = __fdiv_rn(127.0f, amax);
                    q0 = min(127, max(-127, (int)__builtin_rintf(h0 * inv)));
                    q1 = min(127, max(-127, (int)__builtin_rintf(h1 * inv)));
                    dq = __fdiv_rn(amax, 127.0f);
                }
                if (q < r1) {
                    const int f = f0 + 64 * wn + 32 * c + (lane & 15);
                    int8_t* row = hq + (size_t)q * F;
                    row[f] = (int8_t)q0;
                    row[f + 16] = (int8_t)q1;
                    if ((lane & 15) == 0) hd[(size_t)q * nfb + (f >> 5)] = dq;
                }
            }
        }
}

// down: B rows are d_model rows n0 ..
__global__ __launch_bounds__(256, 2) void gemm_down_q8_kernel(moe_experts_t ex, const int8_t* __restrict__ hq,
                                                              const float* __restrict__ hd,
                                                              const int4* __restrict__ tiles,
                                                              const int* __restrict__ ntiles,
                                                              const int32_t* __restrict__ pairs,
                                                              const float* __restrict__ gates, int P,
                                                              float* __restrict__ obuf) {
    const int D = ex.d_model, F = ex.d_ff;
    const int nfb = F >> 5;
    const int n_ntiles = D / kDownBN;
    int mt, nt;
    tile_coords(n_ntiles, mt, nt);
    if (mt >= ntiles[0]) return;
    const int4 tile = tiles[mt];
    const int e = tile.x, r0 = tile.y, r1 = tile.z;
    const int n0 = nt * kDownBN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = __builtin_amdgcn_readfirstlane(wave & 1), wn = __builtin_amdgcn_readfirstlane(wave >> 1);
    const int ni = __builtin_amdgcn_readfirstlane(min(4, max(0, (r1 - r0 - 64 * wm + 15) >> 4)));

    __shared__ __align__(16) int8_t As[kGemmBM][kQ8Row];
    __shared__ __align__(16) int8_t Bs[kDownBN][kQ8Row];
    __shared__ __align__(16) float SA[2][kGemmBM];
    __shared__ __align__(16) float SB[2][256];

    Q8Src src;
    {
        const int q = r0 + (tid >> 1);
        src.a = q < r1 ? hq + (size_t)q * F + (tid & 1) * 32 : nullptr;
        src.sa = q < r1 ? hd + (size_t)q * nfb + (tid & 1) : nullptr;
    }
    const int b_row = tid;
    const size_t b_rowidx = ((size_t)e * D + n0 + b_row) * nfb;
    src.bq = ex.down_q + b_rowidx * 2;
    src.bs = ex.down_s + b_rowidx;

    float4_t acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
    if (ni == 4) q8_kloop<true>(src, b_row, F / kGemmBK, wm, wn, ni, As, Bs, SA, SB, acc);
    else q8_kloop<false>(src, b_row, F / kGemmBK, wm, wn, ni, As, Bs, SA, SB, acc);

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int q = r0 + 64 * wm + 16 * i + 4 * (lane >> 4) + v;
            if (q >= r1) continue;
            const int p = pairs[q];
            if (p < 0 || p >= P) continue;
            const float g = gates[p];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int n = n0 + 128 * wn + 16 * j + (lane & 15);
                obuf[(size_t)p * D + n] = g * acc[i][j][v];
            }
        }
}

}  // namespace

namespace qmoe {

hipError_t launch_quantize_q8(const void* x, int x_bf16, size_t nblocks, int8_t* q, float* d, hipStream_t s) {
    if (nblocks == 0) return hipSuccess;
    quantize_q8_kernel<<<(unsigned)((nblocks + 255) / 256), 256, 0, s>>>(x, x_bf16, nblocks, q, d);
    return hipGetLastError();
}

hipError_t launch_prefill_q8(const moe_experts_t& ex, const void* x, int x_bf16, int T, const float* gates, int K,
                             const int32_t* offsets, const int32_t* pairs, float* y, char* ws,
                             const PrefillQ8Ws& L, hipStream_t s) {
    const int D = ex.d_model, F = ex.d_ff, E = ex.n_experts;
    int8_t* xq = (int8_t*)(ws + L.xq);
    float* xd = (float*)(ws + L.xd);
    int8_t* hq = (int8_t*)(ws + L.hq);
    float* hd = (float*)(ws + L.hd);
    float* obuf = (float*)(ws + L.obuf);
    int4* tiles = (int4*)(ws + L.tiles);
    int* ntiles = (int*)(ws + L.ntiles);
    hipError_t e = launch_quantize_q8(x, x_bf16, (size_t)T * D / 32, xq, xd, s);
    if (e != hipSuccess) return e;
    const int max_tiles = prefill_max_tiles(T, E, K);
    const int P = T * K;
    if ((e = launch_prefill_tiles(offsets, E, P, max_tiles, tiles, ntiles, s)) != hipSuccess) return e;
    const int mt8 = cdiv(max_tiles, 8) * 8;
    gemm_gateup_q8_kernel<<<mt8 * (F / kGateUpBN), 256, 0, s>>>(ex, xq, xd, tiles, ntiles, pairs, K, P, hq, hd);
    gemm_down_q8_kernel<<<mt8 * (D / kDownBN), 256, 0, s>>>(ex, hq, hd, tiles, ntiles, pairs, gates, P, obuf);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_prefill_combine(obuf, T, K, D, y, s);
}

}  // namespace qmoe

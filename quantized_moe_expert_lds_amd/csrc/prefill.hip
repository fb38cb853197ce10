// Prefill expert FFN: grouped GEMMs over the expert buckets on the matrix
// cores (v_mfma_f32_16x16x32_f16), with the 2-bit weights dequantised into
// fp16 tiles in LDS.
//
// The pages process prompts in chunks of up to 8,192 tokens and run the
// expert matmuls on quantised weights (bnskd "Strata：把 125B 大模型塞进 12GB 显
// 卡", section 工程细节).  Their kernel keeps activations quantised; here the
// dequantised 2-bit weights are exact in fp16 (level x fp16 scale with
// |level| <= 2), so the only rounding on the operands is that of the
// activations (bf16 -> fp16 is exact in range) and of the SwiGLU
// intermediate h (fp16).  Accumulation is fp32.
//
// Pipeline (all on the caller's stream):
//  1. x -> fp16, each 32-block permuted into the pair order the weight unpack
//     produces (any permutation of k inside a block leaves the dot product
//     unchanged as long as both operands share it).
//  2. tile list: every bucket is cut into 128-row tiles (expert, first row,
//     end row).
//  3. gate/up GEMM: tile (128 rows) x (128 d_ff columns of gate and the same
//     128 of up); rows are gathered from the token list of the bucket; the
//     epilogue applies SwiGLU and stores h (fp16, bucket order).
//  4. down GEMM: tile (128 rows of h) x (256 d_model columns); the epilogue
//     scales by the pair's gate and stores the row under its pair id.
//  5. combine: y[t] = sum over slots j of the gated rows of pairs t*K + j,
//     in slot order.
// Workgroups map to tiles so that the 8 XCDs take interleaved m-tiles and
// each XCD sweeps all column tiles of an m-tile back to back (the gathered
// activation rows stay in that XCD's L2).
#include "prefill_q8.hpp"

namespace {

using namespace qmoe;
using namespace qmoe_dev;

constexpr int kLdsStride = kGemmBK + 8;   // halves per LDS row (144 B)

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// -------------------------------------------------------------- 1. x -> fp16
__global__ __launch_bounds__(256) void x_to_f16_kernel(const void* __restrict__ x, int x_bf16, size_t nblocks,
                                                       uint16_t* __restrict__ x16) {
    const size_t b = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    float v[32];
    if (x_bf16) {
        const uint4* p = reinterpret_cast<const uint4*>((const uint16_t*)x + b * 32);
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
        const float4* p = reinterpret_cast<const float4*>((const float*)x + b * 32);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float4 f = p[q];
            v[4 * q] = f.x;
            v[4 * q + 1] = f.y;
            v[4 * q + 2] = f.z;
            v[4 * q + 3] = f.w;
        }
    }
    uint32_t o[16];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        o[m] = (uint32_t)f32_to_f16_bits(v[m]) | ((uint32_t)f32_to_f16_bits(v[m + 8]) << 16);
        o[8 + m] = (uint32_t)f32_to_f16_bits(v[16 + m]) | ((uint32_t)f32_to_f16_bits(v[24 + m]) << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(x16 + b * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
}

// ------------------------------------------------------------ 2. tile list
// Offsets are clamped to [0, P] and tiles beyond max_tiles dropped, so an
// inconsistent bucket table cannot send the GEMMs out of bounds.
__global__ __launch_bounds__(1024) void tiles_kernel(const int32_t* __restrict__ offsets, int E, int P,
                                                     int max_tiles, int4* __restrict__ tiles,
                                                     int* __restrict__ ntiles) {
    __shared__ int cnt[1024];
    const int tid = threadIdx.x;
    int n = 0, lo = 0, hi = 0;
    if (tid < E) {
        lo = min(max(offsets[tid], 0), P);
        hi = min(max(offsets[tid + 1], lo), P);
        n = (hi - lo + kGemmBM - 1) / kGemmBM;
    }
    cnt[tid] = n;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int add = tid >= off ? cnt[tid - off] : 0;
        __syncthreads();
        cnt[tid] += add;
        __syncthreads();
    }
    const int base = cnt[tid] - n;
    for (int m = 0; m < n && base + m < max_tiles; ++m) {
        const int r0 = lo + m * kGemmBM;
        tiles[base + m] = make_int4(tid, r0, min(r0 + kGemmBM, hi), 0);
    }
    if (tid == 1023) ntiles[0] = min(cnt[1023], max_tiles);
}

// Dequantise one 2-bit block (codes w0, w1; fp16 scale bits sb) into 16 fp16
// pairs in unpack order: level * scale, exact in fp16.  Pair m < 8 of a word
// holds its weights (m, m + 8), whose codes sit at bits 2m of the word's low
// and high halves.  OR-ing the masked word (shifted by 10 for m >= 5, so the
// bits stay inside the 10-bit mantissa) into 1024.0 gives 1024 + code * 4^m';
// one fused multiply-add by 4^-m' and -(1024 * 4^-m' + 2) yields the level
// exactly, and one multiply the scaled weight.  The mask and the magic are
// kept in registers (DequantConsts) so the and-or is one v_and_or_b32: a
// three-operand instruction takes no literal on gfx9.
struct DequantConsts {
    uint32_t magic;      // 0x64006400, in a VGPR
    uint32_t mask[5];    // 0x00030003 << 2m', in SGPRs
};

__device__ __forceinline__ DequantConsts make_dequant_consts() {
    DequantConsts k;
    k.magic = 0x64006400u;
    asm("" : "+v"(k.magic));
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        k.mask[j] = 0x00030003u << (2 * j);
        asm("" : "+s"(k.mask[j]));
    }
    return k;
}

__device__ __forceinline__ void dequant_block2(uint32_t w0, uint32_t w1, uint16_t sb, uint32_t* out,
                                               const DequantConsts& k) {
    const _Float16 s = __builtin_bit_cast(_Float16, sb);
    const half2_t s2 = {s, s};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t w = h ? w1 : w0, w10 = w >> 10;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int mm = m < 5 ? m : m - 5;
            const uint32_t v = ((m < 5 ? w : w10) & k.mask[mm]) | k.magic;
            const _Float16 mul = (_Float16)(1.0f / (float)(1 << (2 * mm)));
            const _Float16 add = (_Float16)(-(1024.0f / (float)(1 << (2 * mm)) + 2.0f));
            const half2_t lev = __builtin_elementwise_fma(as_half2(v), half2_t{mul, mul}, half2_t{add, add});
            out[8 * h + m] = as_u32(lev * s2);
        }
    }
}

__device__ __forceinline__ void tile_coords(int n_ntiles, int& mt, int& nt) {
    const int b = blockIdx.x, xcd = b & 7, s = b >> 3;
    mt = (s / n_ntiles) * 8 + xcd;
    nt = s % n_ntiles;
}

__device__ __forceinline__ half8_t lds_frag(const _Float16* base) {
    return *reinterpret_cast<const half8_t*>(base);
}

// ---------------------------------------------------- 3./4. grouped GEMMs
// Both GEMMs: a block of 256 threads (4 waves) computes a 128-row x 256-column
// tile (rows = pairs of one bucket; columns = 128 d_ff columns of gate plus
// the same 128 of up, or 256 d_model columns), K in steps of 64 through LDS.
// Wave w owns rows 64 (w & 1) .. +64 and LDS B rows 128 (w >> 1) .. +128: a
// 64 x 128 patch of 4 x 8 MFMA 16x16x32 tiles, so each fragment read from
// LDS feeds 4 or 8 MFMAs.  16-row slices holding no pair of the bucket skip
// their MFMAs.  B rows are dequantised from 2-bit blocks: thread t owns B
// row t, both blocks of a step.  The next step's operands are loaded into
// registers while the current step multiplies.
struct GemmStage {
    uint4 a[4];        // A rows (tid >> 3) + 32 i, 16-byte column chunk tid & 7
    uint4 b;           // codes of the two blocks of B row tid in this step
    uint32_t s;        // their fp16 scales
};

__device__ __forceinline__ void gemm_load(GemmStage& st, const uint16_t* const* a_src, const uint32_t* b_q,
                                          const uint16_t* b_s, int ks) {
    const int k0 = ks * kGemmBK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        st.a[i] = a_src[i] ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
    st.b = *reinterpret_cast<const uint4*>(b_q + (size_t)ks * 4);
    st.s = *reinterpret_cast<const uint32_t*>(b_s + (size_t)ks * 2);
}

__device__ __forceinline__ void gemm_store(const GemmStage& st, _Float16 (*As)[kLdsStride],
                                           _Float16 (*Bs)[kLdsStride], int b_lds_row, const DequantConsts& k) {
    const int tid = threadIdx.x;
    const int a_col = (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&As[(tid >> 3) + 32 * i][a_col]) = st.a[i];
    uint32_t o[16];
    uint4* dst = reinterpret_cast<uint4*>(&Bs[b_lds_row][0]);
    dequant_block2(st.b.x, st.b.y, (uint16_t)(st.s & 0xffff), o, k);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    dequant_block2(st.b.z, st.b.w, (uint16_t)(st.s >> 16), o, k);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[4 + q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
}

// the K loop shared by both GEMMs; ni = 16-row slices of the wave that hold
// pairs.  Full tiles (ni == 4) take a copy without the per-slice branches, so
// the MFMAs of a step form one block the scheduler can interleave with the
// fragment reads.
template <bool kFull>
__device__ __forceinline__ void gemm_kloop(const uint16_t* const* a_src, const uint32_t* b_q, const uint16_t* b_s,
                                           int b_lds_row, int nsteps, int wm, int wn, int ni,
                                           _Float16 (*As)[kLdsStride], _Float16 (*Bs)[kLdsStride],
                                           float4_t (&acc)[4][8]) {
    const int lane = threadIdx.x & 63;
    const DequantConsts dk = make_dequant_consts();
    GemmStage st;
    gemm_load(st, a_src, b_q, b_s, 0);
    for (int ks = 0; ks < nsteps; ++ks) {
        gemm_store(st, As, Bs, b_lds_row, dk);
        __syncthreads();
        gemm_load(st, a_src, b_q, b_s, min(ks + 1, nsteps - 1));   // the last reload is unused
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int kofs = kk * 32 + 8 * (lane >> 4);
            half8_t a[4], b[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = lds_frag(&As[64 * wm + 16 * i + (lane & 15)][kofs]);
#pragma unroll
            for (int j = 0; j < 8; ++j) b[j] = lds_frag(&Bs[128 * wn + 16 * j + (lane & 15)][kofs]);
            // the matrix-core block runs at raised wave priority, so the other
            // workgroup on the CU issues its dequant and LDS work meanwhile
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (!kFull && i >= ni) continue;            // slice beyond the bucket
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
        }
        __syncthreads();
    }
}

// gate/up: B rows 0..127 are gate rows f0.., 128..255 the up rows f0..
__global__ __launch_bounds__(256, 2) void gemm_gateup_kernel(moe_experts_t ex, const uint16_t* __restrict__ x16,
                                                             const int4* __restrict__ tiles,
                                                             const int* __restrict__ ntiles,
                                                             const int32_t* __restrict__ pairs, int K, int P,
                                                             uint16_t* __restrict__ hbuf) {
    const int D = ex.d_model, F = ex.d_ff;
    const int nkb = D >> 5;
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

    __shared__ _Float16 As[kGemmBM][kLdsStride];
    __shared__ _Float16 Bs[2 * kGateUpBN][kLdsStride];

    const uint16_t* a_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = r0 + (tid >> 3) + 32 * i;
        const int p = q < r1 ? pairs[q] : -1;
        a_src[i] = (p >= 0 && p < P) ? x16 + (size_t)(p / K) * D + (tid & 7) * 8 : nullptr;
    }
    const int b_row = tid;
    const int wf = f0 + (b_row & (kGateUpBN - 1));
    const size_t b_rowidx = ((size_t)e * F + wf) * nkb;
    const uint32_t* b_q = (b_row < kGateUpBN ? ex.gate_q : ex.up_q) + b_rowidx * 2;
    const uint16_t* b_s = (b_row < kGateUpBN ? ex.gate_s : ex.up_s) + b_rowidx;
    // wave wn needs gate rows 64 wn .. and up rows 128 + 64 wn ..: they are
    // made contiguous (LDS rows 128 wn .. +128) by permuting the row order;
    // tiles j < 4 are gate columns, j >= 4 the same up columns
    const int b_lds_row = 128 * ((b_row & 127) >> 6) + (b_row >= kGateUpBN ? 64 : 0) + (b_row & 63);

    float4_t acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
    if (ni == 4) gemm_kloop<true>(a_src, b_q, b_s, b_lds_row, D / kGemmBK, wm, wn, ni, As, Bs, acc);
    else gemm_kloop<false>(a_src, b_q, b_s, b_lds_row, D / kGemmBK, wm, wn, ni, As, Bs, acc);

    // epilogue: h = silu(g) * u -> fp16, stored in bucket-row order, each
    // 32-block of d_ff in unpack pair order
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int f = f0 + 64 * wn + 16 * j + (lane & 15);
            const int fpos = (f & ~31) + perm32(f & 31);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int q = r0 + 64 * wm + 16 * i + 4 * (lane >> 4) + v;
                if (q < r1) hbuf[(size_t)q * F + fpos] = f32_to_f16_bits(silu_mul(acc[i][j][v], acc[i][4 + j][v]));
            }
        }
}

// down: B rows are d_model rows n0 ..
__global__ __launch_bounds__(256, 2) void gemm_down_kernel(moe_experts_t ex, const uint16_t* __restrict__ hbuf,
                                                           const int4* __restrict__ tiles,
                                                           const int* __restrict__ ntiles,
                                                           const int32_t* __restrict__ pairs,
                                                           const float* __restrict__ gates, int P,
                                                           float* __restrict__ obuf) {
    const int D = ex.d_model, F = ex.d_ff;
    const int nkb = F >> 5;
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

    __shared__ _Float16 As[kGemmBM][kLdsStride];
    __shared__ _Float16 Bs[kDownBN][kLdsStride];

    const uint16_t* a_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = r0 + (tid >> 3) + 32 * i;
        a_src[i] = q < r1 ? hbuf + (size_t)q * F + (tid & 7) * 8 : nullptr;
    }
    const int b_row = tid;
    const size_t b_rowidx = ((size_t)e * D + n0 + b_row) * nkb;
    const uint32_t* b_q = ex.down_q + b_rowidx * 2;
    const uint16_t* b_s = ex.down_s + b_rowidx;

    float4_t acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
    if (ni == 4) gemm_kloop<true>(a_src, b_q, b_s, b_row, F / kGemmBK, wm, wn, ni, As, Bs, acc);
    else gemm_kloop<false>(a_src, b_q, b_s, b_row, F / kGemmBK, wm, wn, ni, As, Bs, acc);

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

// ------------------------------------------------------------ 5. combine
// The per-pair rows are read once and y is written once: non-temporal
// accesses keep them from evicting other lines (152 -> 117 us for an
// 8,192-token chunk).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ obuf, int T, int K, int D,
                                                      float* __restrict__ y) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;     // float4 index
    const size_t n4 = (size_t)T * D / 4;
    if (i >= n4) return;
    const size_t t = i / (D / 4), c = i % (D / 4);
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < K; ++j) {
        const float4_t* row = reinterpret_cast<const float4_t*>(obuf + ((size_t)t * K + j) * D);
        acc = acc + __builtin_nontemporal_load(row + c);
    }
    __builtin_nontemporal_store(acc, reinterpret_cast<float4_t*>(y + t * D) + c);
}

}  // namespace

namespace qmoe {

hipError_t launch_prefill_tiles(const int32_t* offsets, int E, int P, int max_tiles, int4* tiles, int* ntiles,
                                hipStream_t s) {
    tiles_kernel<<<1, 1024, 0, s>>>(offsets, E, P, max_tiles, tiles, ntiles);
    return hipGetLastError();
}

hipError_t launch_prefill_combine(const float* obuf, int T, int K, int D, float* y, hipStream_t s) {
    const size_t n4 = (size_t)T * D / 4;
    combine_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(obuf, T, K, D, y);
    return hipGetLastError();
}

hipError_t launch_prefill(const moe_experts_t& ex, const void* x, int x_bf16, int T, const float* gates, int K,
                          const int32_t* offsets, const int32_t* pairs, float* y, char* ws, const PrefillWs& L,
                          hipStream_t s) {
    const int D = ex.d_model, F = ex.d_ff, E = ex.n_experts;
    uint16_t* x16 = (uint16_t*)(ws + L.x16);
    uint16_t* hbuf = (uint16_t*)(ws + L.hbuf);
    float* obuf = (float*)(ws + L.obuf);
    int4* tiles = (int4*)(ws + L.tiles);
    int* ntiles = (int*)(ws + L.ntiles);
    const size_t nblocks = (size_t)T * D / 32;
    x_to_f16_kernel<<<(unsigned)((nblocks + 255) / 256), 256, 0, s>>>(x, x_bf16, nblocks, x16);
    const int max_tiles = prefill_max_tiles(T, E, K);
    const int P = T * K;
    tiles_kernel<<<1, 1024, 0, s>>>(offsets, E, P, max_tiles, tiles, ntiles);
    const int mt8 = cdiv(max_tiles, 8) * 8;
    gemm_gateup_kernel<<<mt8 * (F / kGateUpBN), 256, 0, s>>>(ex, x16, tiles, ntiles, pairs, K, P, hbuf);
    gemm_down_kernel<<<mt8 * (D / kDownBN), 256, 0, s>>>(ex, hbuf, tiles, ntiles, pairs, gates, P, obuf);
    const size_t n4 = (size_t)T * D / 4;
    combine_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(obuf, T, K, D, y);
    return hipGetLastError();
}

}  // namespace qmoe

// Whole decode (or verify) step over a stack of MoE layers in one persistent
// kernel launch.
//
// Each token visits all layers of the model in order (bnskd "Strata：把 125B 大
// 模型塞进 12GB 显卡", section 投机解码: one forward pass runs all 48 layers; each
// token is sent to 10 experts, section 核心思路).  At batch 1 a layer moves
// ~15 MB, about 2 us of HBM time on MI355X, while a kernel launch with 256
// workgroups costs ~3-4 us and a dependent launch in a graph ~1.6 us, so a
// step is one cooperative launch with one workgroup per CU that stays
// resident for all layers; grid barriers replace kernel boundaries.
//
// Per layer l, three phases separated by grid barriers:
//   ROUTE : u_l = h_l (l = 0) or RMSNorm(h_l), computed redundantly by every
//           workgroup from the residual slices and sums of squares the
//           workgroups published; workgroup w then computes the fp64 logits
//           of experts w*EPW .. from router rows it loaded during the previous
//           layer.
//   FFN   : every workgroup reads all logits, selects the top-k per token
//           (ties to the lower id), derives the distinct experts of the batch
//           and processes its share of (expert, 16-row d_ff chunk) items:
//           2-/3-bit unpack, fp16 dot products with fp32 accumulation,
//           SwiGLU, fp16 h per (token, slot) pair.  While wave 0 waits at the
//           next barrier, waves 1-3 copy the down-projection rows the
//           workgroup needs next into LDS.
//   DOWN  : workgroup w owns d_model rows w*DPW ..; it combines those rows of
//           every distinct expert (blocks in order, slots in order with their
//           gates), adds the residual and publishes its slice of h and its
//           sum of squares.
//
// Coherence.  Every buffer shared between workgroups exists once per layer,
// so it is written once per launch, and every 128-byte line of it is written
// by a single workgroup.  Writers use agent-scope (write-through) stores;
// after a barrier readers use ordinary cached vector loads: a line can only
// enter an L2 after its writer finished it, and kernel boundaries invalidate
// the L2s.  A barrier is a relaxed agent-scope atomic add on one of 8
// counters (one per XCD slot, 256 B apart) after each thread's stores have
// completed, and a poll of the 8 counters by 8 lanes.  Every wait is bounded
// by a wall-clock timeout: on expiry the kernel records an error flag and
// exits instead of hanging.
#include "common.hpp"
//
// This header holds the kernel template; each stack_t<T>.hip instantiates it
// for one batch size, so the instantiations compile in parallel.
#pragma once

#include <atomic>

#include "stack.hpp"

namespace {

using namespace qmoe;
using namespace qmoe_dev;
using namespace qmoe::stk;

constexpr int kMaxDevices = 64;

typedef __attribute__((address_space(3))) void lds_void_t;

// One direct-to-LDS chunk: lane i copies GRAN bytes from src + off + i*GRAN
// to dst + off + i*GRAN (LDS address = M0 base + lane id * GRAN); lanes past
// `bytes` are masked off.  The data is in LDS once the issuing wave has
// waited for vmcnt(0).
__device__ __forceinline__ void dma_chunk(const char* src, char* dst, int off, int bytes, int gran) {
    const int lane = threadIdx.x & 63;
    if (gran == 16) {
        if (off + lane * 16 < bytes)
            __builtin_amdgcn_global_load_lds(src + off + lane * 16, (lds_void_t*)(dst + off), 16, 0, 0);
    } else {
        if (off + lane * 4 < bytes)
            __builtin_amdgcn_global_load_lds(src + off + lane * 4, (lds_void_t*)(dst + off), 4, 0, 0);
    }
}

// Copy `bytes` (a multiple of 16, 16-byte aligned) to LDS, 1 KB chunks spread
// over waves w0 .. w0+nw-1.
__device__ __forceinline__ void dma_to_lds(const void* src, void* dst, int bytes, int w0, int nw) {
    const int wave = (threadIdx.x >> 6) - w0;
    for (int off = wave * 1024; off < bytes; off += nw * 1024)
        dma_chunk((const char*)src, (char*)dst, off, bytes, 16);
}

struct LdsCopy {
    const void* src;
    void* dst;
    int bytes;
};

struct NoSideWork {
    __device__ void operator()() const {}
};

// ------------------------------------------------------- coherent stores
__device__ __forceinline__ void st_f32(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_f64(double* p, double v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------- DPP wavefront reductions
// Fixed-order reductions to lane 63 (row_shr 1, 2, 4, 8 inside each row of
// 16 lanes, then row_bcast 15 and 31 across rows), broadcast by readlane.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp0(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xf, false);
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_addf(float v) {
    return v + __int_as_float(dpp0<CTRL, ROWMASK>(__float_as_int(v)));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
    v = dpp_addf<0x111, 0xf>(v);
    v = dpp_addf<0x112, 0xf>(v);
    v = dpp_addf<0x114, 0xf>(v);
    v = dpp_addf<0x118, 0xf>(v);
    v = dpp_addf<0x142, 0xa>(v);
    v = dpp_addf<0x143, 0xc>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_addd(double v) {
    const int lo = dpp0<CTRL, ROWMASK>(__double2loint(v));
    const int hi = dpp0<CTRL, ROWMASK>(__double2hiint(v));
    return v + __hiloint2double(hi, lo);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
    v = dpp_addd<0x111, 0xf>(v);
    v = dpp_addd<0x112, 0xf>(v);
    v = dpp_addd<0x114, 0xf>(v);
    v = dpp_addd<0x118, 0xf>(v);
    v = dpp_addd<0x142, 0xa>(v);
    v = dpp_addd<0x143, 0xc>(v);
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 63),
                            __builtin_amdgcn_readlane(__double2loint(v), 63));
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_maxd(double v) {
    const int lo = __builtin_amdgcn_update_dpp(__double2loint(v), __double2loint(v), CTRL, ROWMASK, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(__double2hiint(v), __double2hiint(v), CTRL, ROWMASK, 0xf, false);
    return fmax(v, __hiloint2double(hi, lo));
}
__device__ __forceinline__ double wave_max_f64(double v) {
    v = dpp_maxd<0x111, 0xf>(v);
    v = dpp_maxd<0x112, 0xf>(v);
    v = dpp_maxd<0x114, 0xf>(v);
    v = dpp_maxd<0x118, 0xf>(v);
    v = dpp_maxd<0x142, 0xa>(v);
    v = dpp_maxd<0x143, 0xc>(v);
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 63),
                            __builtin_amdgcn_readlane(__double2loint(v), 63));
}
// identity "old" values with bound_ctrl let each step fold into one DPP op
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp_mini(int v) {
    return min(v, __builtin_amdgcn_update_dpp(0x7fffffff, v, CTRL, ROWMASK, 0xf, true));
}
__device__ __forceinline__ int wave_min_i32(int v) {
    v = dpp_mini<0x111, 0xf>(v);
    v = dpp_mini<0x112, 0xf>(v);
    v = dpp_mini<0x114, 0xf>(v);
    v = dpp_mini<0x118, 0xf>(v);
    v = dpp_mini<0x142, 0xa>(v);
    v = dpp_mini<0x143, 0xc>(v);
    return __builtin_amdgcn_readlane(v, 63);
}

template <int CTRL, int ROWMASK>
__device__ __forceinline__ unsigned dpp_maxu(unsigned v) {
    return max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWMASK, 0xf, true));
}
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
    v = dpp_maxu<0x111, 0xf>(v);
    v = dpp_maxu<0x112, 0xf>(v);
    v = dpp_maxu<0x114, 0xf>(v);
    v = dpp_maxu<0x118, 0xf>(v);
    v = dpp_maxu<0x142, 0xa>(v);
    v = dpp_maxu<0x143, 0xc>(v);
    return (unsigned)__builtin_amdgcn_readlane((int)v, 63);
}

// High 32 bits of an unsigned key that orders doubles like their values
// (-0 is normalised to +0 beforehand).
__device__ __forceinline__ unsigned order_hi(double v) {
    const unsigned hi = (unsigned)__double2hiint(v);
    return (hi & 0x80000000u) ? ~hi : (hi | 0x80000000u);
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
}

// Top-k of z[e_lo..e_hi) (at most 64 * kPer values) by one wavefront,
// ranked by (z desc, id asc), written in rank order to out_v / out_i (and
// the 32-bit order keys to out_k).  Each lane sorts its kPer values (ids
// ascending; a stable sort on value keeps equal values in id order), so a
// lane's head is its best element.  Each round takes the largest 32-bit
// order key over the heads (one DPP max per step); when a single lane holds
// it, that lane writes its head and pops it.  A tie on the key bits is
// settled by the fp64 values and then the ids of the tied lanes.
template <int kPer>
__device__ void wave_topk_core(const double* z, int e_lo, int e_hi, int K, double* out_v, int* out_i,
                               unsigned* out_k) {
    const int lane = threadIdx.x & 63;
    double v[kPer];
    int id[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = e_lo + lane + 64 * i;
        v[i] = e < e_hi ? z[e] + 0.0 : -INFINITY;
        id[i] = e < e_hi ? e : 0x7fffffff;
    }
#pragma unroll
    for (int a = 1; a < kPer; ++a)
#pragma unroll
        for (int b = a; b > 0; --b) {
            const bool sw = v[b] > v[b - 1];
            const double tv = v[b];
            const int ti = id[b];
            v[b] = sw ? v[b - 1] : tv;
            id[b] = sw ? id[b - 1] : ti;
            v[b - 1] = sw ? tv : v[b - 1];
            id[b - 1] = sw ? ti : id[b - 1];
        }
    for (int j = 0; j < K; ++j) {
        const unsigned key = order_hi(v[0]);
        const unsigned mk = wave_max_u32(key);
        bool win = key == mk;
        if (__popcll(__ballot(win)) > 1) {
            // tie on the high key bits: exact value, then lowest id
            const double M = wave_max_f64(win ? v[0] : -INFINITY);
            const int wid = wave_min_i32(win && v[0] == M ? id[0] : 0x7fffffff);
            win = win && id[0] == wid;
        }
        if (win) {
            out_v[j] = v[0];
            out_i[j] = id[0];
            out_k[j] = key;
#pragma unroll
            for (int i = 0; i < kPer - 1; ++i) {
                v[i] = v[i + 1];
                id[i] = id[i + 1];
            }
            v[kPer - 1] = -INFINITY;
            id[kPer - 1] = 0x7fffffff;
        }
    }
}

// softmax gates over K sorted logits (LDS, rank order)
__device__ __forceinline__ void wave_gates(const double* sv, const int* si, int K, int* ids, float* gates) {
    const int lane = threadIdx.x & 63;
    const double mine = lane < K ? sv[lane] : 0.0;
    const double m0 = sv[0];
    const double p = lane < K ? exp(mine - m0) : 0.0;
    const double sum = wave_sum_f64(p);
    if (lane < K) {
        ids[lane] = si[lane];
        gates[lane] = (float)(p / sum);
    }
}

// Merge C <= 64 candidates (value, id, key; C a multiple of 4) into the top
// K by rank counting: a candidate's rank is the number of candidates ranked
// before it; distinct 32-bit order keys decide alone, ties on them use the
// exact values and ids.  Writes rank order to out_v / out_i.
__device__ void wave_merge_topk(const double* cv, const int* ci, const unsigned* ck, int C, int K, double* out_v,
                                int* out_i) {
    const int lane = threadIdx.x & 63;
    const bool valid = lane < C;
    const double v = valid ? cv[lane] : -INFINITY;
    const int id = valid ? ci[lane] : 0x7fffffff;
    const unsigned key = valid ? ck[lane] : 0u;
    int rank = 0, eq = 0;
    for (int q = 0; q < C; q += 4) {
        const uint4 kq = *reinterpret_cast<const uint4*>(ck + q);          // same address in every lane
        rank += (kq.x > key) + (kq.y > key) + (kq.z > key) + (kq.w > key);
        eq += (kq.x == key) + (kq.y == key) + (kq.z == key) + (kq.w == key);
    }
    if (__ballot(valid && eq > 1)) {
        rank = 0;
        for (int q = 0; q < C; ++q) {
            const double vq = cv[q];
            const int iq = ci[q];
            rank += (vq > v) || (vq == v && iq < id);
        }
    }
    if (valid && rank < K) {
        out_v[rank] = v;
        out_i[rank] = id;
    }
}

// Grid barrier number `epoch` (1-based).  Returns false if it timed out or
// another workgroup reported an error.
// Waves 1..3 may start an LDS copy (`cp`) while wave 0 waits; it completes
// by the next barrier.
// Waves 1-3 run `side` (copies into LDS) while wave 0 waits for the grid.
template <typename Side = NoSideWork>
__device__ bool grid_barrier(const StackParams& P, int epoch, int* s_flag, Side side = Side{}) {
    // every thread waits until its own stores have completed (gfx9 counts
    // stores in vmcnt; a workgroup-scope release fence emits no wait)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int* sync = P.sync;
    if (threadIdx.x >= 64) side();
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        if (lane == 0)
            __hip_atomic_fetch_add(&sync[(blockIdx.x & 7) * kLine], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int ok = 1;
        if (lane < 8) {
            const int need = epoch * ((P.G - lane + 7) >> 3);
            const long long t0 = wall_clock64();
            int n = 0;
            while (__hip_atomic_load(&sync[lane * kLine], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
                if ((++n & 63) == 0 &&
                    (__hip_atomic_load(&sync[9 * kLine], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 ||
                     wall_clock64() - t0 > kTimeoutTicks)) {
                    ok = 0;
                    break;
                }
            }
        }
        const unsigned long long bad = __ballot(lane < 8 && !ok);
        if (lane == 0) {
            if (bad) __hip_atomic_store(&sync[9 * kLine], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *s_flag = bad ? 0 : 1;
        }
    }
    __syncthreads();
    return *s_flag != 0;
}

// NB bits of the 96-bit string w[0] | w[1] << 32 | w[2] << 64 from bit p
// (compile-time p after unrolling); bits past 96 read as zero
template <int NB>
__device__ __forceinline__ uint32_t bits96(const uint32_t* w, int p) {
    const int k = p >> 5, off = p & 31;
    const uint32_t lo = w[k];
    const uint32_t hi = k + 1 < 3 ? w[k + 1] : 0u;
    const uint32_t x = off + NB <= 32 ? (lo >> off) : __builtin_amdgcn_alignbit(hi, lo, off);
    return x & ((1u << NB) - 1u);
}

// Levels of a block as 16 fp16 pairs in unpack order: pair m < 8 holds
// weights (m, m + 8), pair 8 + m weights (16 + m, 24 + m).
// 2-bit: the code of weight m sits at bits 2m of the word's low half and the
// code of weight m + 8 at bits 2m of its high half.  OR-ing the masked word
// into the mantissa of 1024.0 gives 1024 + code * 4^m' (m' = m, or m - 5
// after one shift by 10 so the bits stay inside the 10-bit mantissa); one
// fused multiply-add by 4^-m' and -(1024 * 4^-m' + 2) yields code - 2,
// exactly, in both halves.
//
// The and-or is one v_and_or_b32 only when its two constants sit in
// registers (a three-operand instruction takes no literal on gfx9), so the
// constants are made once per kernel and hidden from constant folding.
struct UnpackConsts {
    uint32_t magic;      // 0x64006400 (1024.0 in both halves), in a VGPR
    uint32_t mask[5];    // code masks, in SGPRs
};

template <int BITS>
__device__ __forceinline__ UnpackConsts make_unpack_consts() {
    UnpackConsts k;
    k.magic = 0x64006400u;
    asm("" : "+v"(k.magic));
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        k.mask[j] = BITS == 2 ? 0x00030003u << (2 * j) : (j < 3 ? 0x00070007u << (3 * j) : 0u);
        asm("" : "+s"(k.mask[j]));
    }
    return k;
}

template <int BITS>
__device__ __forceinline__ void levels16(const uint32_t* w, uint32_t* lv, const UnpackConsts& k) {
    if constexpr (BITS == 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t w0 = w[h], w10 = w[h] >> 10;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int mm = m < 5 ? m : m - 5;
                const uint32_t v = ((m < 5 ? w0 : w10) & k.mask[mm]) | k.magic;
                const _Float16 mul = (_Float16)(1.0f / (float)(1 << (2 * mm)));
                const _Float16 add = (_Float16)(-(1024.0f / (float)(1 << (2 * mm)) + 2.0f));
                lv[8 * h + m] = as_u32(__builtin_elementwise_fma(as_half2(v), half2_t{mul, mul}, half2_t{add, add}));
            }
        }
    } else {
        // 3-bit: weight i sits at bits 3i of the 96-bit string w0 | w1 << 32
        // | w2 << 64.  Pairs (m, m + 8) are built three at a time: the 9 bits
        // of weights m0 .. m0+2 go to the low half of X and those of weights
        // m0+8 .. m0+10 to the high half; pair j then is an and-or of the
        // codes at bits 3j into the mantissa of 1024.0 (1024 + code * 8^j)
        // and one fused multiply-add by 8^-j and -(1024 * 8^-j + 4).
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int g = 0; g < 3; ++g) {
                const int m0 = 3 * g, nj = g < 2 ? 3 : 2;
                const uint32_t lo = bits96<9>(w, 48 * h + 3 * m0);
                const uint32_t hi = bits96<9>(w, 48 * h + 3 * m0 + 24);
                const uint32_t X = lo | (hi << 16);
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    if (j >= nj) continue;
                    const uint32_t v = (X & k.mask[j]) | k.magic;
                    const _Float16 mul = (_Float16)(1.0f / (float)(1 << (3 * j)));
                    const _Float16 add = (_Float16)(-(1024.0f / (float)(1 << (3 * j)) + 4.0f));
                    lv[8 * h + m0 + j] = as_u32(__builtin_elementwise_fma(as_half2(v), half2_t{mul, mul}, half2_t{add, add}));
                }
            }
    }
}

__device__ __forceinline__ float dot16h(const uint32_t* lv, const uint32_t* xp) {
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < 16; ++m) acc = __builtin_amdgcn_fdot2(as_half2(lv[m]), as_half2(xp[m]), acc, false);
    return acc;
}

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// u as fp16 in unpack order, one 17-word row per 32-element block (16 pair
// words + 1 pad word, so lane-per-block reads hit distinct banks).  Element
// i of a block sits in pair word (i & 16) / 2 + (i & 7), half (i >> 3) & 1.
__device__ __forceinline__ int xh_half_index(int t, int nkb, int d) {
    const int kb = d >> 5, i = d & 31;
    return ((t * nkb + kb) * kXhWords + ((i >> 4) << 3) + (i & 7)) * 2 + ((i >> 3) & 1);
}

template <int W>
__device__ __forceinline__ void load_block(const uint32_t* qb, size_t blk, uint32_t* q) {
    if constexpr (W == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(qb + blk * 2);
        q[0] = v.x;
        q[1] = v.y;
    } else {
        q[0] = qb[blk * 3];
        q[1] = qb[blk * 3 + 1];
        q[2] = qb[blk * 3 + 2];
    }
}


template <int T, int BITS, int KPER>
__global__ __launch_bounds__(kThreads, 1) void decode_stack_kernel(StackParams P) {
    constexpr int W = BITS == 2 ? 2 : 3;
    extern __shared__ __align__(16) unsigned char lds[];
    const moe_stack_t& m = P.m;
    const int L = m.n_layers, E = m.n_experts, D = m.d_model, F = m.d_ff, K = m.top_k;
    const int G = P.G, w = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const UnpackConsts uk = make_unpack_consts<BITS>();
    const int nkbD = D >> 5, nkbF = F >> 5, nch = F >> 4;
    const int PT = T * K;
    const int EPW = (E + G - 1) / G;
    const int DPW = (D + G - 1) / G;
    const int d_lo = min(w * DPW, D), d_hi = min(d_lo + DPW, D);
    const int nrows = d_hi - d_lo;

    _Float16* xh = reinterpret_cast<_Float16*>(lds + P.lds_xh);           // [T][D/32][17 words]
    const uint32_t* xhw = reinterpret_cast<const uint32_t*>(lds + P.lds_xh);
    float* part = reinterpret_cast<float*>(lds + P.lds_part);             // [PT][DPW][nkbF]
    double* s_z = reinterpret_cast<double*>(lds + P.lds_part);            // [T][E] (dead before part is used)
    float* s_z_f = reinterpret_cast<float*>(lds + P.lds_us);              // [PT][DPW] per-pair sums in DOWN
    uint32_t* pre = reinterpret_cast<uint32_t*>(lds + P.lds_pre);         // prefetched down blocks
    unsigned char* misc = lds + P.lds_misc;
    int* s_ids = reinterpret_cast<int*>(misc);                            // [PT]
    float* s_gates = reinterpret_cast<float*>(s_ids + PT);                // [PT]
    int* s_uniq = reinterpret_cast<int*>(s_gates + PT);                   // [PT]
    int* s_first = s_uniq + PT;                                           // [PT]
    short* s_upair = reinterpret_cast<short*>(s_first + PT);              // [PT][T]
    double* s_red = reinterpret_cast<double*>(misc + misc_head_bytes(PT, T));   // [4][kMaxEPW][T]
    float* s_hloc = reinterpret_cast<float*>(s_red + 4 * kMaxEPW * T);    // see hloc_floats
    int* s_misc = reinterpret_cast<int*>(s_hloc + hloc_floats(DPW, T));   // [0] = U, [1] = flag
    double* s_r = reinterpret_cast<double*>(s_misc + 4);                  // [4][T] per-wave sums of squares
    float* s_hres = reinterpret_cast<float*>(s_r + 4 * T);                // [T][DPW] own residual rows
    double* s_cand_v = reinterpret_cast<double*>(misc + misc_tail_offset(PT, T, DPW));   // [256] top-k lists
    int* s_cand_i = reinterpret_cast<int*>(s_cand_v + 256);               // [256]
    unsigned* s_cand_k = reinterpret_cast<unsigned*>(s_cand_i + 256);     // [256]

    const size_t zb_layer = (size_t)G * T * kZW;
    const size_t hb_layer = (size_t)G * T * kHW;
    const size_t sb_layer = (size_t)G * 16;
    const size_t hp_layer = (size_t)PT * nch * kHBW;

    // router rows of this workgroup's experts live in LDS, copied by DMA one
    // layer ahead (expert-major rows are contiguous)
    float* wr_lds = reinterpret_cast<float*>(lds + P.lds_wr);             // [EPW][D]
    const int e_first = w * EPW;
    const int my_experts = max(0, min(EPW, E - e_first));
    auto router_copy = [&](int layer) {
        return LdsCopy{m.router_w + ((size_t)layer * E + e_first) * D, wr_lds, my_experts * D * 4};
    };
    if (my_experts > 0) {
        const LdsCopy c = router_copy(0);
        dma_to_lds(c.src, c.dst, c.bytes, 0, 4);
    }
    for (int i = tid; i < T * nrows; i += kThreads) {
        const int t = i / nrows, r = i - t * nrows;
        const size_t xi = (size_t)t * D + d_lo + r;
        s_hres[t * DPW + r] = P.x_bf16 ? bf16_to_f32(((const uint16_t*)P.x)[xi]) : ((const float*)P.x)[xi];
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    int epoch = 0;
    for (int l = 0; l < L; ++l) {
        // ------------------------------------------------------------- ROUTE
        float bias_v = 0.0f;           // bias of (expert j, token t) for thread j*T + t
        if (m.router_b && tid < kMaxEPW * T) {
            const int j = tid / T, e = w * EPW + j;
            if (j < EPW && e < E) bias_v = m.router_b[(size_t)l * E + e];
        }
        {
            // Thread tid owns elements d = tid + 256 k of every token: it loads
            // them (x, or the residual slices the workgroups published), forms
            // u, stores u's fp16 pairs for the expert phase and accumulates its
            // share of this workgroup's logits, with no barrier in between.
            const float* hbp = P.hb + (size_t)(l > 0 ? l - 1 : 0) * hb_layer;
            constexpr int KR = T >= 16 ? 1 : 16 / T;      // elements per token per round of loads
            float hv[KR][T];
            auto load_round = [&](int k0) {
#pragma unroll
                for (int kr = 0; kr < KR; ++kr) {
                    const int d = min(tid + (k0 + kr) * kThreads, D - 1);
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        if (l == 0) {
                            const size_t xi = (size_t)t * D + d;
                            hv[kr][t] = P.x_bf16 ? bf16_to_f32(((const uint16_t*)P.x)[xi]) : ((const float*)P.x)[xi];
                        } else {
                            const int g = d / DPW;
                            hv[kr][t] = hbp[((size_t)g * T + t) * kHW + (d - g * DPW)];
                        }
                    }
                }
            };
            load_round(0);                                // in flight during the sums of squares
            double rr[T], inv[T];
            if (l > 0) {
                // sums of squares: thread g loads workgroup g's sum (threads
                // over workgroups, then DPP, then the 4 waves in order); every
                // thread then forms the same rms from the 4 wave sums
                const double* sbp = P.sb + (size_t)(l - 1) * sb_layer;
                double ss[T];
#pragma unroll
                for (int t = 0; t < T; ++t) ss[t] = tid < G ? sbp[(size_t)tid * 16 + t] : 0.0;
                for (int g = tid + kThreads; g < G; g += kThreads)
#pragma unroll
                    for (int t = 0; t < T; ++t) ss[t] += sbp[(size_t)g * 16 + t];
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const double v = wave_sum_f64(ss[t]);
                    if (lane == 0) s_r[wave * T + t] = v;
                }
                __syncthreads();
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const double tot = ((s_r[t] + s_r[T + t]) + s_r[2 * T + t]) + s_r[3 * T + t];
                    rr[t] = sqrt(tot / (double)D + P.eps);
                    inv[t] = 1.0 / rr[t];
                }
            }
            double acc[kMaxEPW][T];
#pragma unroll
            for (int j = 0; j < kMaxEPW; ++j)
#pragma unroll
                for (int t = 0; t < T; ++t) acc[j][t] = 0.0;
            for (int k0 = 0; k0 * kThreads < D; k0 += KR) {
                if (k0 > 0) load_round(k0);
#pragma unroll
                for (int kr = 0; kr < KR; ++kr) {
                    const int d = tid + (k0 + kr) * kThreads;
                    if (d >= D) continue;
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        float uv = hv[kr][t];
                        if (l > 0) {
                            // h / r correctly rounded: reciprocal, then one
                            // remainder correction (Markstein)
                            const double hd = (double)uv;
                            const double q0 = hd * inv[t];
                            uv = (float)fma(fma(-q0, rr[t], hd), inv[t], q0);
                        }
                        xh[xh_half_index(t, nkbD, d)] = (_Float16)uv;
#pragma unroll
                        for (int j = 0; j < kMaxEPW; ++j)
                            if (j < my_experts) acc[j][t] = fma((double)uv, (double)wr_lds[j * D + d], acc[j][t]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kMaxEPW; ++j) {
                if (j >= EPW) break;
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const double v = wave_sum_f64(acc[j][t]);
                    if (lane == 0) s_red[(wave * kMaxEPW + j) * T + t] = v;
                }
            }
            __syncthreads();
            if (tid < kMaxEPW * T) {
                const int j = tid / T, t = tid - j * T;
                const int e = w * EPW + j;
                if (j < EPW && e < E) {
                    double s = ((s_red[(0 * kMaxEPW + j) * T + t] + s_red[(1 * kMaxEPW + j) * T + t]) +
                                s_red[(2 * kMaxEPW + j) * T + t]) + s_red[(3 * kMaxEPW + j) * T + t];
                    s += (double)bias_v;
                    st_f64(&P.zb[(size_t)l * zb_layer + ((size_t)w * T + t) * kZW + j], s);
                }
            }
        }
        // the next layer's router rows stream in while this barrier waits
        // (every wave is done reading wr_lds once the barrier's entry
        // __syncthreads has passed)
        if (!grid_barrier(P, ++epoch, &s_misc[1], [&]() {
                if (l + 1 < L && my_experts > 0) {
                    const LdsCopy c = router_copy(l + 1);
                    dma_to_lds(c.src, c.dst, c.bytes, 1, 3);
                }
            }))
            return;

        // --------------------------------------------------------------- FFN
        {
            // logit lines (workgroup g, token t), all loads of a round in flight
            const double* zbp = P.zb + (size_t)l * zb_layer;
            const int nz = G * T;
            for (int i0 = 0; i0 < nz; i0 += 4 * kThreads) {
                double2 v[4][2];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int i = min(i0 + tid + a * kThreads, nz - 1);
                    const double2* src = reinterpret_cast<const double2*>(zbp + (size_t)i * kZW);
                    v[a][0] = src[0];
                    v[a][1] = src[1];
                }
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int i = i0 + tid + a * kThreads;
                    if (i < nz) {
                        const int g = i / T, t = i - g * T;
                        const double vv[4] = {v[a][0].x, v[a][0].y, v[a][1].x, v[a][1].y};
#pragma unroll
                        for (int j = 0; j < kMaxEPW; ++j) {
                            const int e = g * EPW + j;
                            if (j < EPW && e < E) s_z[t * E + e] = vv[j];
                        }
                    }
                }
            }
        }
        __syncthreads();
        constexpr bool kSplitTopk = T == 1 && KPER >= 4;
        const bool split_topk = kSplitTopk && 4 * K <= 64;
        if (split_topk) {
            // batch 1: each wave selects the top K of a quarter of the
            // experts, then wave 0 merges the 4 K candidates.  With one token
            // the distinct experts are the selected ones in rank order; the
            // gates are formed later, while the expert weight loads are in
            // flight.
            constexpr int kq = KPER >= 4 ? KPER / 4 : 1;
            wave_topk_core<kq>(s_z, 64 * kq * wave, min(E, 64 * kq * (wave + 1)), K, s_cand_v + wave * K,
                               s_cand_i + wave * K, s_cand_k + wave * K);
            __syncthreads();
            if (wave == 0) {
                wave_merge_topk(s_cand_v, s_cand_i, s_cand_k, 4 * K, K, s_cand_v + 64, s_cand_i + 64);
                if (lane < K) {
                    const int e = s_cand_i[64 + lane];
                    s_ids[lane] = e;
                    s_uniq[lane] = e;
                    s_upair[lane] = (short)lane;
                }
                if (lane == 0) s_misc[0] = K;
            }
        } else {
            for (int t = wave; t < T; t += 4) {
                double* ov = s_cand_v + 64 * wave;
                int* oi = s_cand_i + 64 * wave;
                wave_topk_core<KPER>(s_z + (size_t)t * E, 0, E, K, ov, oi, s_cand_k + 64 * wave);
                wave_gates(ov, oi, K, s_ids + t * K, s_gates + t * K);
            }
        }
        __syncthreads();
        // gates of the batch-1 path (wave 0), and the routing outputs
        auto finish_gates = [&]() {
            if constexpr (kSplitTopk) {
                wave_gates(s_cand_v + 64, s_cand_i + 64, K, s_ids, s_gates);
                if (w == 0 && P.ids_out && lane < K) {
                    P.ids_out[(size_t)l * PT + lane] = s_cand_i[64 + lane];
                    P.gates_out[(size_t)l * PT + lane] = s_gates[lane];
                }
            }
        };
        bool gates_pending = split_topk;
        if (!split_topk && w == 0 && P.ids_out) {
            for (int i = tid; i < PT; i += kThreads) {
                P.ids_out[(size_t)l * PT + i] = s_ids[i];
                P.gates_out[(size_t)l * PT + i] = s_gates[i];
            }
        }
        // distinct experts of the batch, in slot order of first appearance
        if (split_topk) {
            // set above
        } else if (PT <= 64) {
            if (wave == 0) {
                // lane p holds pair p; its expert's first pair is the lowest q
                // with the same id; first pairs are numbered by a ballot
                const int e = lane < PT ? s_ids[lane] : -1;
                int firstq = lane;
                for (int q = PT - 1; q >= 0; --q)
                    if (__builtin_amdgcn_readlane(e, q) == e) firstq = q;
                const bool first = lane < PT && firstq == lane;
                const unsigned long long fm = __ballot(first);
                const int idx = __popcll(fm & ((1ull << lane) - 1ull));
                const int U = __popcll(fm);
                if (first) s_uniq[idx] = e;
                for (int i = lane; i < U * T; i += 64) s_upair[i] = (short)-1;
                const int my_u = __shfl(idx, firstq);             // distinct-expert number of pair p
                if (lane < PT) s_upair[my_u * T + lane / K] = (short)lane;
                if (lane == 0) s_misc[0] = U;
            }
        } else {
            for (int p = tid; p < PT; p += kThreads) {
                const int e = s_ids[p];
                int first = 1;
                for (int q = 0; q < p; ++q) first &= (s_ids[q] != e);
                s_first[p] = first;
            }
            __syncthreads();
            for (int p = tid; p < PT; p += kThreads) {
                if (!s_first[p]) continue;
                int idx = 0;
                for (int q = 0; q < p; ++q) idx += s_first[q];
                const int e = s_ids[p];
                s_uniq[idx] = e;
                for (int t = 0; t < T; ++t) {
                    int pr = -1;
                    for (int j = 0; j < K; ++j)
                        if (s_ids[t * K + j] == e) pr = t * K + j;
                    s_upair[idx * T + t] = (short)pr;
                }
            }
            if (tid == 0) {
                int U = 0;
                for (int p = 0; p < PT; ++p) U += s_first[p];
                s_misc[0] = U;
            }
        }
        __syncthreads();
        const int U = s_misc[0];

        const size_t lstrideD = (size_t)E * D * nkbF;
        const int uid = lane < U ? s_uniq[lane] : 0;     // distinct expert `lane` (first 64)
        const int n_pre = min(U, P.pre_cap);
        // copy this workgroup's down-projection rows d_lo .. d_hi of the first
        // n_pre distinct experts into LDS.  Waves 1-3 issue the copies while
        // wave 0 waits at the next grid barrier, so they do not compete with
        // the gate/up weight loads; chunks are dealt to the three waves
        // round-robin.  Wave-uniform control flow only: every lane of the
        // wave takes part in a chunk.
        auto issue_down_prefetch = [&]() {
            if (nrows <= 0) return;
            const int cbytes = nrows * nkbF * W * 4, sbytes = nrows * nkbF * 2;
            int ci = 0;
            for (int u = 0; u < n_pre; ++u) {
                const int e = u < 64 ? __builtin_amdgcn_readlane(uid, u) : s_uniq[u];
                const size_t row0 = ((size_t)l * E + e) * D + d_lo;
                const char* csrc = reinterpret_cast<const char*>(m.down_q + row0 * nkbF * W);
                const char* ssrc = reinterpret_cast<const char*>(m.down_s + row0 * nkbF);
                char* cdst = reinterpret_cast<char*>(pre) + (size_t)u * (P.pre_cstride + P.pre_sstride);
                for (int off = 0; off < cbytes; off += 64 * P.pre_cgran, ++ci)
                    if (ci % 3 == wave - 1) dma_chunk(csrc, cdst, off, cbytes, P.pre_cgran);
                for (int off = 0; off < sbytes; off += 64 * P.pre_sgran, ++ci)
                    if (ci % 3 == wave - 1) dma_chunk(ssrc, cdst + P.pre_cstride, off, sbytes, P.pre_sgran);
            }
        };

        {
            const int n_items = U * nch;
            const size_t lstrideGU = (size_t)E * F * nkbD;
            uint32_t xp0[T][16];                    // x pairs of block kb = lane (clamped), read once
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int mm = 0; mm < 16; ++mm) xp0[t][mm] = xhw[(t * nkbD + min(lane, nkbD - 1)) * kXhWords + mm];
            for (int it0 = w; it0 < n_items; it0 += G * kMaxItemsInFlight) {
                float acc[kMaxItemsInFlight][8][T];
                int tmask[kMaxItemsInFlight];       // tokens that chose the item's expert
                int ie[kMaxItemsInFlight];          // the item's expert
#pragma unroll
                for (int a = 0; a < kMaxItemsInFlight; ++a) {
                    const int it = it0 + a * G;
                    int msk = 0, e = 0;
                    if (it < n_items) {
                        const int u = it / nch;
#pragma unroll
                        for (int t = 0; t < T; ++t) msk |= (s_upair[u * T + t] >= 0) << t;
                        e = s_uniq[u];
                    }
                    tmask[a] = __builtin_amdgcn_readfirstlane(msk);
                    ie[a] = __builtin_amdgcn_readfirstlane(e);
                }
#pragma unroll
                for (int a = 0; a < kMaxItemsInFlight; ++a)
#pragma unroll
                    for (int r = 0; r < 8; ++r)
#pragma unroll
                        for (int t = 0; t < T; ++t) acc[a][r][t] = 0.0f;
                for (int kb0 = 0; kb0 < nkbD; kb0 += 64) {        // wave-uniform loop
                    const int kb = kb0 + lane;
                    const bool kact = kb < nkbD;
                    const int kbc = kact ? kb : nkbD - 1;         // loads stay in bounds
                    uint32_t q[kMaxItemsInFlight][8][W];
                    uint16_t sr[kMaxItemsInFlight][8];
#pragma unroll
                    for (int a = 0; a < kMaxItemsInFlight; ++a) {
                        const int it = it0 + a * G;
                        if (it >= n_items) continue;
                        const int c = it - (it / nch) * nch;
                        const int f0 = 16 * c + 4 * wave;
#pragma unroll
                        for (int r = 0; r < 8; ++r) {
                            const size_t blk = (size_t)l * lstrideGU + ((size_t)ie[a] * F + f0 + (r & 3)) * nkbD + kbc;
                            load_block<W>(r < 4 ? m.gate_q : m.up_q, blk, q[a][r]);
                            sr[a][r] = (r < 4 ? m.gate_s : m.up_s)[blk];
                        }
                    }
                    if (gates_pending) {
                        gates_pending = false;
                        if (wave == 0) finish_gates();
                    }
                    uint32_t xpk[T][16];
                    if (kb0 > 0) {
#pragma unroll
                        for (int t = 0; t < T; ++t)
#pragma unroll
                            for (int mm = 0; mm < 16; ++mm) xpk[t][mm] = xhw[(t * nkbD + kbc) * kXhWords + mm];
                    }
                    // every loaded register is consumed on every path (lanes past
                    // the last block add 0), so no load is left in flight at the
                    // loop's back edge
#pragma unroll
                    for (int a = 0; a < kMaxItemsInFlight; ++a) {
                        if (it0 + a * G >= n_items) continue;
#pragma unroll
                        for (int r = 0; r < 8; ++r) {
                            uint32_t lv[16];
                            levels16<BITS>(q[a][r], lv, uk);
                            const float sc = kact ? h2f(sr[a][r]) : 0.0f;
#pragma unroll
                            for (int t = 0; t < T; ++t)        // (one token: it chose every item's expert)
                                if (T == 1 || ((tmask[a] >> t) & 1))
                                    acc[a][r][t] = fmaf(sc, dot16h(lv, kb0 == 0 ? xp0[t] : xpk[t]), acc[a][r][t]);
                        }
                    }
                }
                // wave sums, gathered so lane j = (a T + t) 4 + r holds the
                // gate and up sums of (item a, token t, row r); one SwiGLU
                // evaluation then covers all of them
                static_assert(4 * T * kMaxItemsInFlight <= 64, "one lane per (item, token, row)");
                float gv = 0.0f, uv = 0.0f;
#pragma unroll
                for (int a = 0; a < kMaxItemsInFlight; ++a) {
                    const int it = it0 + a * G;
                    if (it >= n_items) continue;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int t = 0; t < T; ++t) {
                            if (T > 1 && !((tmask[a] >> t) & 1)) continue;
                            const float g = wave_sum_f32(acc[a][r][t]);
                            const float uu = wave_sum_f32(acc[a][4 + r][t]);
                            if (lane == (a * T + t) * 4 + r) {
                                gv = g;
                                uv = uu;
                            }
                        }
                }
                {
                    const int a = lane / (4 * T), t = (lane >> 2) % T, r = lane & 3;
                    int tm = 0;
#pragma unroll
                    for (int b = 0; b < kMaxItemsInFlight; ++b)
                        if (a == b && it0 + b * G < n_items) tm = tmask[b];
                    const float hv = silu_mul(gv, uv);
                    if (a < kMaxItemsInFlight && ((tm >> t) & 1)) s_hloc[(a * T + t) * 16 + 4 * wave + r] = hv;
                }
                __syncthreads();
                if (tid < 8 * T * kMaxItemsInFlight) {
                    const int a = tid / (8 * T), rem = tid - a * 8 * T, t = rem >> 3, mm = rem & 7;
                    const int it = it0 + a * G;
                    if (it < n_items) {
                        const int u = it / nch, c = it - u * nch;
                        const int pr = s_upair[u * T + t];
                        if (pr >= 0) {
                            half2_t hv = {(_Float16)s_hloc[(a * T + t) * 16 + mm], (_Float16)s_hloc[(a * T + t) * 16 + mm + 8]};
                            st_u32(&P.hp[(size_t)l * hp_layer + ((size_t)pr * nch + c) * kHBW + mm], as_u32(hv));
                        }
                    }
                }
                __syncthreads();
            }
        }
        if (gates_pending && wave == 0) finish_gates();   // workgroups without gate/up items
        // the copies must have landed before any wave reads them after the barrier
        if (!grid_barrier(P, ++epoch, &s_misc[1], [&]() {
                issue_down_prefetch();
                __builtin_amdgcn_s_waitcnt(0);
            }))
            return;

        // -------------------------------------------------------------- DOWN
        {
            const uint32_t* hpp = P.hp + (size_t)l * hp_layer;
            for (int it = tid; it < U * nkbF; it += kThreads) {
                const int u = it / nkbF, kb = it - u * nkbF;
                const int e = s_uniq[u];
                uint32_t hv[T][16];
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int pr = s_upair[u * T + t];
                    if (pr < 0) continue;
                    // block kb of d_ff = 16-row chunks 2kb (pairs 0..7) and 2kb+1 (pairs 8..15)
                    const uint4* s0 = reinterpret_cast<const uint4*>(hpp + ((size_t)pr * nch + 2 * kb) * kHBW);
                    const uint4* s1 = reinterpret_cast<const uint4*>(hpp + ((size_t)pr * nch + 2 * kb + 1) * kHBW);
                    const uint4 a0 = s0[0], a1 = s0[1], b0 = s1[0], b1 = s1[1];
                    hv[t][0] = a0.x; hv[t][1] = a0.y; hv[t][2] = a0.z; hv[t][3] = a0.w;
                    hv[t][4] = a1.x; hv[t][5] = a1.y; hv[t][6] = a1.z; hv[t][7] = a1.w;
                    hv[t][8] = b0.x; hv[t][9] = b0.y; hv[t][10] = b0.z; hv[t][11] = b0.w;
                    hv[t][12] = b1.x; hv[t][13] = b1.y; hv[t][14] = b1.z; hv[t][15] = b1.w;
                }
                if (u < n_pre) {
                    // rows from LDS (nrows <= 8 whenever experts are prefetched)
                    const char* cb = reinterpret_cast<const char*>(pre) + (size_t)u * (P.pre_cstride + P.pre_sstride);
                    const uint32_t* cw = reinterpret_cast<const uint32_t*>(cb);
                    const uint16_t* sw = reinterpret_cast<const uint16_t*>(cb + P.pre_cstride);
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        if (r >= nrows) continue;
                        uint32_t qv[W];
#pragma unroll
                        for (int k = 0; k < W; ++k) qv[k] = cw[(r * nkbF + kb) * W + k];
                        const float sc = h2f(sw[r * nkbF + kb]);
                        uint32_t lv[16];
                        levels16<BITS>(qv, lv, uk);
#pragma unroll
                        for (int t = 0; t < T; ++t) {
                            const int pr = s_upair[u * T + t];
                            if (pr < 0) continue;
                            part[((size_t)pr * DPW + r) * nkbF + kb] = sc * dot16h(lv, hv[t]);
                        }
                    }
                } else {
                    for (int r0 = 0; r0 < nrows; r0 += 8) {
                        uint32_t q[8][W];
                        uint16_t sr[8];
#pragma unroll
                        for (int r = 0; r < 8; ++r) {      // clamped rows: every load is issued unconditionally
                            const int rr = min(r0 + r, nrows - 1);
                            const size_t blk = (size_t)l * lstrideD + ((size_t)e * D + d_lo + rr) * nkbF + kb;
                            load_block<W>(m.down_q, blk, q[r]);
                            sr[r] = m.down_s[blk];
                        }
#pragma unroll
                        for (int r = 0; r < 8; ++r) {
                            if (r0 + r >= nrows) continue;
                            uint32_t lv[16];
                            levels16<BITS>(q[r], lv, uk);
                            const float sc = h2f(sr[r]);
#pragma unroll
                            for (int t = 0; t < T; ++t) {
                                const int pr = s_upair[u * T + t];
                                if (pr < 0) continue;
                                part[((size_t)pr * DPW + r0 + r) * nkbF + kb] = sc * dot16h(lv, hv[t]);
                            }
                        }
                    }
                }
            }
            __syncthreads();
            // o[p][r] = sum of blocks in order, one thread per (pair, row)
            float* s_o = s_z_f;                                          // [PT][DPW], reuses the logit area
            for (int o = tid; o < PT * nrows; o += kThreads) {
                const int p = o / nrows, r = o - p * nrows;
                const float* pp = part + ((size_t)p * DPW + r) * nkbF;
                // blocks added in order; reads issued 8 at a time
                float oj = 0.0f;
                int kb = 0;
                for (; kb + 8 <= nkbF; kb += 8) {
                    float v[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[i] = pp[kb + i];
#pragma unroll
                    for (int i = 0; i < 8; ++i) oj += v[i];
                }
                for (; kb < nkbF; ++kb) oj += pp[kb];
                s_o[p * DPW + r] = oj;
            }
            __syncthreads();
            // y rows (slots in order with their gates), residual, sums of squares
            for (int o = tid; o < T * nrows; o += kThreads) {
                const int t = o / nrows, r = o - t * nrows;
                // slots added in order with their gates; reads issued 8 at a time
                float yv = 0.0f;
                int j = 0;
                for (; j + 8 <= K; j += 8) {
                    float gv[8], ov[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        gv[i] = s_gates[t * K + j + i];
                        ov[i] = s_o[(t * K + j + i) * DPW + r];
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) yv = yv + gv[i] * ov[i];
                }
                for (; j < K; ++j) yv = yv + s_gates[t * K + j] * s_o[(t * K + j) * DPW + r];
                const int d = d_lo + r;
                const float hn = s_hres[t * DPW + r] + yv;
                s_hres[t * DPW + r] = hn;
                if (l + 1 < L) st_f32(&P.hb[(size_t)l * hb_layer + ((size_t)w * T + t) * kHW + r], hn);
                else P.h_out[(size_t)t * D + d] = hn;
                if (P.h_layers) P.h_layers[((size_t)l * T + t) * D + d] = hn;
                s_hloc[t * nrows + r] = hn;
            }
            __syncthreads();
            if (l + 1 < L && tid < T) {
                double ss = 0.0;
                for (int r = 0; r < nrows; ++r) {
                    const double v = (double)s_hloc[tid * nrows + r];
                    ss += v * v;
                }
                st_f64(&P.sb[(size_t)l * sb_layer + (size_t)w * 16 + tid], ss);
            }
        }
        if (l + 1 < L) {
            if (!grid_barrier(P, ++epoch, &s_misc[1])) return;
        }
    }
    // last arrival resets the counters for the next launch
    __syncthreads();
    if (tid == 0) {
        const int prev = __hip_atomic_fetch_add(&P.sync[8 * kLine], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == G - 1) {
            for (int x = 0; x < 9; ++x)
                __hip_atomic_store(&P.sync[x * kLine], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int T, int BITS, int KPER>
hipError_t launch_stack_t(StackParams& P, size_t lds, hipStream_t s) {
    auto fn = decode_stack_kernel<T, BITS, KPER>;
    // the dynamic LDS limit is raised once per device; two threads making
    // their first call at the same time both set the same value
    static std::atomic<int> attr_done[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!attr_done[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_done[dev].store(1, std::memory_order_release);
    }
    void* args[] = {&P};
    return hipLaunchCooperativeKernel((const void*)fn, dim3(P.G), dim3(kThreads), args, (unsigned)lds, s);
}

template <int T, int BITS>
hipError_t launch_stack_e(StackParams& P, size_t lds, hipStream_t s) {
    const int E = P.m.n_experts;
    if (E <= 128) return launch_stack_t<T, BITS, 2>(P, lds, s);
    if (E <= 512) return launch_stack_t<T, BITS, 8>(P, lds, s);
    return launch_stack_t<T, BITS, 16>(P, lds, s);
}

}  // namespace

// Defines launch_stack_T<N> (both weight formats) in a stack_t<N>.hip file.
#define QMOE_DEFINE_STACK_LAUNCH(N)                                                                  \
    namespace qmoe {                                                                                 \
    namespace stk {                                                                                  \
    template <>                                                                                      \
    hipError_t launch_stack_T<N>(StackParams & P, size_t lds, hipStream_t s) {                       \
        return P.m.bits == 2 ? launch_stack_e<N, 2>(P, lds, s) : launch_stack_e<N, 3>(P, lds, s);    \
    }                                                                                                \
    }                                                                                                \
    }

// Whole decode (or verify) step over a stack of MoE layers in one persistent
// kernel launch.
//
// Each token visits all layers of the model in order (bnskd "Strata：把 125B 大
// 模型塞进 12GB 显卡", section 投机解码: one forward pass runs all 48 layers; each
// token is sent to 10 experts, section 核心思路).  At batch 1 a layer moves
// ~15 MB, about 2 us of HBM time on MI355X, while a kernel launch with 256
// workgroups costs ~3-4 us and a dependent launch in a graph ~1.6 us, so a
// step is one launch with one workgroup per CU that stays resident for all
// layers.
//
// Per layer l, three phases; each hands its results to the next through
// device memory:
//   ROUTE : u_l = h_l (l = 0) or RMSNorm(h_l), computed redundantly by every
//           workgroup from the residual rows and sums of squares the
//           workgroups published; workgroup w then computes the fp64 logits
//           of experts w*EPW .. from router rows it copied into LDS during the
//           previous layer, and publishes them.
//   FFN   : every workgroup gathers all logits, selects the top-k per token
//           (ties to the lower id), derives the distinct experts of the batch
//           and processes its share of (expert, 16-row d_ff chunk) items:
//           2-/3-bit unpack, dot products with fp32 accumulation, SwiGLU,
//           h per (token, slot) pair; then it raises its flag.
//   DOWN  : workgroup w owns d_model rows w*DPW ..; once every flag is up it
//           combines those rows of every distinct expert (blocks in order,
//           slots in order with their gates), adds the residual and
//           publishes its rows of h and their sum of squares.
//
// Precision.  The activations u and the SwiGLU output h enter the packed
// fp16 dot products as two fp16 halves (hi = fp16(v), lo = fp16(v - hi));
// the levels are exact small integers and the accumulation is fp32, so the
// dot products carry ~22 bits of u and h, close to an fp32 evaluation.
//
// Hand-over.  Logits and residual rows travel as tagged 64-bit words
// (payload + epoch, one agent-scope atomic each; see ll_store): a reader
// spins on exactly the words it needs until they carry this layer's epoch,
// so no grid-wide barrier is needed and the data arrive with the signal.
// Every 128-byte line of these buffers has a single writer workgroup.
// Lines shared by words of several writers (workgroups on different XCDs)
// returned wrong logits in tests, without any wait timing out, while the
// same exchange over single-writer lines was exact.
// The SwiGLU rows (many words read by every workgroup) are stored once per
// layer and launch with write-through agent-scope stores into a buffer of
// their own per layer, followed by the writer's tagged flag; readers load
// them with ordinary cached loads after seeing every flag.  That relies on
// the hardware rather than on the HIP memory model: a line of that buffer
// enters a workgroup's L2 only after its writer's stores have completed,
// and a kernel launch starts with invalidated L2s.  Every wait is bounded
// by a wall-clock timeout: on expiry the kernel records an error word and
// exits instead of hanging.
//
// This header holds the kernel template; each stack_t<T>.hip instantiates it
// for one batch size, so the instantiations compile in parallel.
#pragma once

#include <atomic>

#include "stack.hpp"
#include "wave_ops.hpp"

namespace {

using namespace qmoe;
using namespace qmoe_dev;
using namespace qmoe::stk;

constexpr int kMaxDevices = 64;

// ------------------------------------------------------- coherent stores
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup barrier that orders LDS only.  Outstanding global loads and
// stores stay in flight: __syncthreads() also waits for every one of them,
// and a write-through store is acknowledged only after a round trip to
// memory, which put that latency on every barrier that followed a
// hand-over store.  Global data is never shared between the threads of a
// workgroup except through the SwiGLU-row protocol, which waits for its
// stores explicitly.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------ tagged exchanges
// A shared value travels as a 64-bit word: the 32-bit payload in the low
// half and the epoch it belongs to in the high half, stored and loaded with
// agent-scope atomics.  A reader waits until the word carries the epoch it
// expects; payload and tag arrive together (one single-copy-atomic word), so
// no fence or separate flag is needed, and the tag also tells this layer's
// value from one left by an earlier layer or launch.  Every word of token
// slot t is tagged with that slot's epoch base[t] + layer + 1; the bases
// advance by L at the end of every launch that uses the slot, so a word
// never carries a current tag before it is written in the current launch.
__device__ __forceinline__ void ll_store(u64* p, uint32_t tag, uint32_t payload) {
    __hip_atomic_store(p, ((u64)tag << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ll_load(const u64* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// p, hidden from the optimiser's view (kept in scalar registers)
template <typename Ptr>
__device__ __forceinline__ Ptr opaque_ptr(Ptr p) {
    asm volatile("" : "+s"(p));
    return p;
}

// true once the wait must end: the wall-clock limit passed, or another
// workgroup reported an error
__device__ __forceinline__ bool stack_should_stop(const StackParams& P, long long t0) {
    return __hip_atomic_load(&P.hdr[kHdrErr], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 ||
           wall_clock64() - t0 > kTimeoutTicks;
}

// Waits until the first n of the N words addr(i) carry tag tg(i) and returns
// their payloads in out.  All loads are issued before any wait.  Returns
// false if the wait had to stop (stack_should_stop).
template <int N, typename Addr, typename Tag>
__device__ __forceinline__ bool ll_wait(Addr addr, Tag tg, uint32_t (&out)[N], int n, const StackParams& P) {
    u64 v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = i < n ? ll_load(addr(i)) : 0ull;
    uint64_t pend = 0;
#pragma unroll
    for (int i = 0; i < N; ++i)
        if (i < n && (uint32_t)(v[i] >> 32) != tg(i)) pend |= 1ull << i;
    if (pend) {
        const long long t0 = wall_clock64();
        int it = 0;
        while (pend) {
            if ((++it & 15) == 0 && stack_should_stop(P, t0)) return false;
            __builtin_amdgcn_s_sleep(2);
#pragma unroll
            for (int i = 0; i < N; ++i)
                if ((pend >> i) & 1) v[i] = ll_load(addr(i));
#pragma unroll
            for (int i = 0; i < N; ++i)
                if (((pend >> i) & 1) && (uint32_t)(v[i] >> 32) == tg(i)) pend &= ~(1ull << i);
        }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = (uint32_t)v[i];
    return true;
}

// Ends the kernel for the whole workgroup when any of its threads had to stop
// waiting; the first such workgroup records the error for the caller.  The
// workgroup's verdict goes through an LDS word that starts at zero and is
// only ever set (a workgroup that sees it set exits).
#define STACK_CHECK_OK(ok)                                                                           \
    do {                                                                                             \
        if (!(ok)) s_misc[1] = 1;                                                                    \
        lds_barrier();                                                                               \
        if (s_misc[1]) {                                                                             \
            if (threadIdx.x == 0)                                                                    \
                __hip_atomic_store(&P.hdr[kHdrErr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); \
            return;                                                                                  \
        }                                                                                            \
    } while (0)

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

// Dot product of a block's levels with an operand split into fp16 halves v =
// hi + lo (hi = fp16(v), lo = fp16(v - hi)): the levels are exact small
// integers, so this carries ~22 significant bits of v into the fp32
// accumulation.  The small lo terms are summed first.
__device__ __forceinline__ float dot32h(const uint32_t* lv, const uint32_t* hi, const uint32_t* lo) {
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < 16; ++m) acc = __builtin_amdgcn_fdot2(as_half2(lv[m]), as_half2(lo[m]), acc, false);
#pragma unroll
    for (int m = 0; m < 16; ++m) acc = __builtin_amdgcn_fdot2(as_half2(lv[m]), as_half2(hi[m]), acc, false);
    return acc;
}

// v = hi + lo with hi = fp16(v) and lo = fp16(v - hi) (v - hi is exact in fp32)
__device__ __forceinline__ void split_f16(float v, _Float16& hi, _Float16& lo) {
    hi = (_Float16)v;
    lo = (_Float16)(v - (float)hi);
}

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// u in LDS as fp16 halves in unpack order, one kXhWords-word row per
// (token, 32-element block): words 0..15 hold the hi pairs, 16..31 the lo
// pairs.  The 144-byte row stride keeps the 16-byte reads of a lane per block
// on distinct banks.  Element i of a block sits in pair word
// (i & 16) / 2 + (i & 7), half (i >> 3) & 1; this returns the half index of
// its hi part (the lo part is 32 halves further).
__device__ __forceinline__ int xh_half_index(int t, int nkb, int d) {
    const int kb = d >> 5, i = d & 31;
    return ((t * nkb + kb) * kXhWords + ((i >> 4) << 3) + (i & 7)) * 2 + ((i >> 3) & 1);
}

// Expert codes and scales are read once per step: the loads carry the
// non-temporal hint, so this stream of ~0.7 GB per batch-1 step does not
// evict what the step reads again (the router rows of every layer, the
// exchange lines).  48-layer batch-1 step: 1,069 -> 1,016 us (same box,
// alternating runs); the 4-token 3-bit step is unchanged.
template <int W>
__device__ __forceinline__ void load_block(const uint32_t* qb, size_t blk, uint32_t* q) {
    if constexpr (W == 2) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(qb + blk * 2));
        q[0] = v.x;
        q[1] = v.y;
    } else {
        q[0] = __builtin_nontemporal_load(qb + blk * 3);
        q[1] = __builtin_nontemporal_load(qb + blk * 3 + 1);
        q[2] = __builtin_nontemporal_load(qb + blk * 3 + 2);
    }
}

__device__ __forceinline__ uint16_t ld_scale(const uint16_t* p) { return __builtin_nontemporal_load(p); }

template <int T, int BITS, int KPER, int EPWM>
__global__ __launch_bounds__(kThreads, 1) void decode_stack_kernel(StackParams P) {
    constexpr int W = BITS == 2 ? 2 : 3;
    extern __shared__ __align__(16) unsigned char lds[];
    const moe_stack_t& m = P.m;
    const int L = m.n_layers, E = m.n_experts, D = m.d_model, F = m.d_ff, K = m.top_k;
    const int G = P.G, w = blockIdx.x;
    const int tid = threadIdx.x;
    const UnpackConsts uk = make_unpack_consts<BITS>();
    const int nkbD = D >> 5, nkbF = F >> 5, nch = F >> 4;
    const int PT = T * K;
    const int EPW = (E + G - 1) / G;
    const int DPW = (D + G - 1) / G;
    const int d_lo = min(w * DPW, D), d_hi = min(d_lo + DPW, D);
    const int nrows = d_hi - d_lo;

    _Float16* xh = reinterpret_cast<_Float16*>(lds + P.lds_xh);           // [T][D/32][kXhWords]
    const uint32_t* xhw = reinterpret_cast<const uint32_t*>(lds + P.lds_xh);
    float* part = reinterpret_cast<float*>(lds + P.lds_part);             // [PT][DPW][nkbF]
    double* s_z = reinterpret_cast<double*>(lds + P.lds_part);            // [T][E] (dead before part is used)
    float* s_z_f = reinterpret_cast<float*>(lds + P.lds_us);              // [PT][DPW] per-pair sums in DOWN
    unsigned char* misc = lds + P.lds_misc;
    int* s_ids = reinterpret_cast<int*>(misc);                            // [PT]
    float* s_gates = reinterpret_cast<float*>(s_ids + PT);                // [PT]
    int* s_uniq = reinterpret_cast<int*>(s_gates + PT);                   // [PT]
    int* s_first = s_uniq + PT;                                           // [PT]
    short* s_upair = reinterpret_cast<short*>(s_first + PT);              // [PT][T]
    double* s_red = reinterpret_cast<double*>(misc + misc_head_bytes(PT, T));   // [4][EPWM][T]
    float* s_hloc = reinterpret_cast<float*>(s_red + 4 * EPWM * T);    // see hloc_floats
    int* s_misc = reinterpret_cast<int*>(s_hloc + hloc_floats(DPW, T));   // [0] = U
    double* s_r = reinterpret_cast<double*>(s_misc + 4);                  // [4][T] per-wave sums of squares
    float* s_hres = reinterpret_cast<float*>(s_r + 4 * T);                // [T][DPW] own residual rows
    float* s_gu = s_hres + T * DPW;                                       // see gu_floats
    double* s_cand_v = reinterpret_cast<double*>(misc + misc_tail_offset(PT, T, DPW));   // [4][128] top-k candidates
    int* s_cand_i = reinterpret_cast<int*>(s_cand_v + 512);               // [4][128]
    unsigned* s_cand_k = reinterpret_cast<unsigned*>(s_cand_i + 512);     // [4][64]
    double* s_sel_v = reinterpret_cast<double*>(s_cand_k + 256);          // [4][64] selected, rank order
    int* s_sel_i = reinterpret_cast<int*>(s_sel_v + 256);                 // [4][64]
    int* s_hist = s_sel_i + 256;                                          // [4][128]

    const size_t hp_layer = (size_t)PT * nch * kHBW;

    // epoch of token slot t at layer l; flags of a layer carry slot 0's epoch
    uint32_t base[T];
#pragma unroll
    for (int t = 0; t < T; ++t) base[t] = P.hdr[kHdrBase + t];

    // router rows of this workgroup's experts: each thread multiplies only
    // the elements d = tid + 256 k of them, which it loads into registers at
    // the start of the layer's ROUTE phase, ahead of its waits
    const int e_first = w * EPW;
    const int my_experts = max(0, min(EPW, E - e_first));
    constexpr int kDK = kStackMaxD / kThreads;                            // d elements per thread
    if (tid == 0) s_misc[1] = 0;
    for (int i = tid; i < T * nrows; i += kThreads) {
        const int t = i / nrows, r = i - t * nrows;
        const size_t xi = (size_t)t * D + d_lo + r;
        s_hres[t * DPW + r] = P.x_bf16 ? bf16_to_f32(((const uint16_t*)P.x)[xi]) : ((const float*)P.x)[xi];
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int l = 0; l < L; ++l) {
        // For batches of two or more tokens the exchange and input pointers
        // and the thread's element offset are made opaque to the optimiser
        // every layer, so the addresses derived from them are formed where
        // they are used.  Hoisted out of the layer loop they stayed live for
        // its whole length and were spilled to scratch memory, and every
        // phase then waited for their reloads (a 4-token 3-bit step took
        // 4.4 ms instead of 3.5 ms).  At one token nothing spills and the
        // hoisted addresses are faster.
        u64* sl_ = P.sl;
        u64* lg_ = P.lg;
        u64* fl_ = P.fl;
        const void* x_ = P.x;
        int tid_ = tid;
        if constexpr (T > 1) {
            sl_ = opaque_ptr(sl_);
            lg_ = opaque_ptr(lg_);
            fl_ = opaque_ptr(fl_);
            x_ = opaque_ptr(x_);
            asm volatile("" : "+v"(tid_));
        }
        // the thread's indices inside the layer derive from the opaque copy
        const int tid = tid_, lane = tid_ & 63, wave = tid_ >> 6;
        // ------------------------------------------------------------- ROUTE
        float bias_v = 0.0f;           // bias of (expert j, token t) for thread j*T + t
        if (m.router_b && tid < EPWM * T) {
            const int j = tid / T, e = w * EPW + j;
            if (j < EPW && e < E) bias_v = m.router_b[(size_t)l * E + e];
        }
        // this thread's router elements, clamped in bounds (every load is
        // issued, so later waits count them at compile time); loads return
        // in order, so they arrive during the waits below
        float wr[EPWM][kDK];
        {
            const float* rw = m.router_w + ((size_t)l * E + min(e_first, E - 1)) * D;
#pragma unroll
            for (int j = 0; j < EPWM; ++j)
#pragma unroll
                for (int k = 0; k < kDK; ++k)
                    wr[j][k] = rw[(size_t)min(j, max(my_experts - 1, 0)) * D + min(tid + k * kThreads, D - 1)];
        }
        {
            // Thread tid owns elements d = tid + 256 k of every token: it waits
            // for them (x, or the residual rows the workgroups published),
            // forms u, stores u's fp16 halves for the expert phase and
            // accumulates its share of this workgroup's logits.
            constexpr int KR = T >= 5 ? 2 : (T >= 3 ? 4 : 8);   // elements per token per round of waits
            float hv[KR][T];
            bool ok = true;
            // tagged words of the residual rows (written by layer l - 1)
            auto row_word = [&](int k0, int i) -> const u64* {
                const int kr = i / T, t = i - kr * T;
                const int d = min(tid_ + (k0 + kr) * kThreads, D - 1);
                const int g = d / DPW;
                return sl_ + ((size_t)g * kSlots + t) * kSLW + (d - g * DPW);
            };
            auto row_tag = [&](int i) { return base[i % T] + (uint32_t)l; };
            auto take_rows = [&](const uint32_t* pay) {
#pragma unroll
                for (int kr = 0; kr < KR; ++kr)
#pragma unroll
                    for (int t = 0; t < T; ++t) hv[kr][t] = __uint_as_float(pay[kr * T + t]);
            };
            auto load_x = [&](int k0) {
#pragma unroll
                for (int kr = 0; kr < KR; ++kr) {
                    const int d = min(tid_ + (k0 + kr) * kThreads, D - 1);
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        const size_t xi = (size_t)t * D + d;
                        hv[kr][t] = P.x_bf16 ? bf16_to_f32(((const uint16_t*)x_)[xi]) : ((const float*)x_)[xi];
                    }
                }
            };
            double rr[T], inv[T];
            if (l > 0) {
                // sums of squares: thread g waits for workgroup g's (threads
                // over workgroups, then DPP, then the 4 waves in order), in
                // the same wait as its first round of rows; every thread then
                // forms the same rms from the 4 wave sums
                double ss[T];
                {
                    const int g = tid;
                    const int nss = g < G ? 2 * T : 0;
                    uint32_t pay[2 * T + KR * T];
                    ok = ll_wait<2 * T + KR * T>(
                        [&](int i) -> const u64* {
                            if (i < 2 * T) return sl_ + ((size_t)min(g, G - 1) * kSlots + (i >> 1)) * kSLW + kSSWord + (i & 1);
                            return row_word(0, i - 2 * T);
                        },
                        [&](int i) { return i < 2 * T ? base[i >> 1] + (uint32_t)l : row_tag(i - 2 * T); },
                        pay, 2 * T + KR * T, P);
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        ss[t] = nss ? __hiloint2double((int)pay[2 * t + 1], (int)pay[2 * t]) : 0.0;
                    take_rows(pay + 2 * T);
                }
                for (int g = tid + kThreads; g < G; g += kThreads) {
                    uint32_t pay[2 * T];
                    ok = ok && ll_wait<2 * T>(
                        [&](int i) -> const u64* { return sl_ + ((size_t)g * kSlots + (i >> 1)) * kSLW + kSSWord + (i & 1); },
                        [&](int i) { return base[i >> 1] + (uint32_t)l; }, pay, 2 * T, P);
#pragma unroll
                    for (int t = 0; t < T; ++t) ss[t] += __hiloint2double((int)pay[2 * t + 1], (int)pay[2 * t]);
                }
                STACK_CHECK_OK(ok);
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const double v = wave_sum_f64(ss[t]);
                    if (lane == 0) s_r[wave * T + t] = v;
                }
                lds_barrier();
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const double tot = ((s_r[t] + s_r[T + t]) + s_r[2 * T + t]) + s_r[3 * T + t];
                    rr[t] = sqrt(tot / (double)D + P.eps);
                    inv[t] = 1.0 / rr[t];
                }
            } else {
                load_x(0);
            }
            double acc[EPWM][T];
#pragma unroll
            for (int j = 0; j < EPWM; ++j)
#pragma unroll
                for (int t = 0; t < T; ++t) acc[j][t] = 0.0;
#pragma unroll
            for (int k0 = 0; k0 < kDK; k0 += KR) {
                if (k0 * kThreads >= D) break;
                if (k0 > 0) {
                    if (l == 0) {
                        load_x(k0);
                    } else {
                        uint32_t pay[KR * T];
                        ok = ll_wait<KR * T>([&](int i) { return row_word(k0, i); }, row_tag, pay, KR * T, P);
                        STACK_CHECK_OK(ok);
                        take_rows(pay);
                    }
                }
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
                        _Float16 uh, ul;
                        split_f16(uv, uh, ul);
                        const int xi = xh_half_index(t, nkbD, d);
                        xh[xi] = uh;
                        xh[xi + 32] = ul;
#pragma unroll
                        for (int j = 0; j < EPWM; ++j)
                            if (j < my_experts) acc[j][t] = fma((double)uv, (double)wr[j][k0 + kr], acc[j][t]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < EPWM; ++j) {
                if (j >= EPW) break;
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const double v = wave_sum_f64(acc[j][t]);
                    if (lane == 0) s_red[(wave * EPWM + j) * T + t] = v;
                }
            }
            lds_barrier();
            if (tid < EPWM * T) {
                const int j = tid / T, t = tid - j * T;
                const int e = w * EPW + j;
                if (j < EPW && e < E) {
                    double s = ((s_red[(0 * EPWM + j) * T + t] + s_red[(1 * EPWM + j) * T + t]) +
                                s_red[(2 * EPWM + j) * T + t]) + s_red[(3 * EPWM + j) * T + t];
                    s += (double)bias_v;
                    u64* q = lg_ + ((size_t)w * kSlots + t) * kLGW + 2 * j;
                    const uint32_t tg = base[t] + (uint32_t)l + 1u;
                    ll_store(q, tg, (uint32_t)__double2loint(s));
                    ll_store(q + 1, tg, (uint32_t)__double2hiint(s));
                }
            }
        }

        // --------------------------------------------------------------- FFN
        {
            // logits of every expert: thread g waits for workgroup g's line,
            // two experts (four words) per token at a time
            bool ok = true;
            for (int g = tid; g < G; g += kThreads) {
                const int ne = min(EPW, E - g * EPW);
                for (int j0 = 0; j0 < ne; j0 += 2) {
                    const int nj = min(2, ne - j0);
                    uint32_t pay[4 * T];
                    ok = ok && ll_wait<4 * T>(
                        [&](int i) -> const u64* {
                            const int t = i >> 2, k4 = min(i & 3, 2 * nj - 1);
                            return lg_ + ((size_t)g * kSlots + t) * kLGW + 2 * j0 + k4;
                        },
                        [&](int i) { return base[i >> 2] + (uint32_t)l + 1u; }, pay, 4 * T, P);
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        for (int j = 0; j < nj; ++j)
                            s_z[t * E + g * EPW + j0 + j] =
                                __hiloint2double((int)pay[4 * t + 2 * j + 1], (int)pay[4 * t + 2 * j]);
                }
            }
            STACK_CHECK_OK(ok);
        }
        // top-k and gates per token, one wave per token: the histogram
        // selection, or the round-by-round one
        for (int t = wave; t < T; t += 4) {
            double* ov = s_sel_v + 64 * wave;
            int* oi = s_sel_i + 64 * wave;
            // the histogram selection runs faster alone; with four waves
            // at once their LDS adds collide and the rounds win
            if (T > 2 || !wave_topk_hist<KPER>(s_z + (size_t)t * E, E, K, ov, oi, s_hist + 128 * wave,
                                               s_cand_v + 128 * wave, s_cand_i + 128 * wave))
                wave_topk_core<KPER>(s_z + (size_t)t * E, 0, E, K, ov, oi, s_cand_k + 64 * wave);
            wave_gates(ov, oi, K, s_ids + t * K, s_gates + t * K);
        }
        lds_barrier();
        if (w == 0 && P.ids_out) {
            for (int i = tid; i < PT; i += kThreads) {
                P.ids_out[(size_t)l * PT + i] = s_ids[i];
                P.gates_out[(size_t)l * PT + i] = s_gates[i];
            }
        }
        // distinct experts of the batch, in slot order of first appearance
        if (T == 1) {
            // one token: the distinct experts are its selected ones, in rank order
            if (tid < K) {
                s_uniq[tid] = s_ids[tid];
                s_upair[tid] = (short)tid;
            }
            if (tid == 0) s_misc[0] = K;
        } else if (PT <= 64) {
            if (wave == 0) {
                // lane p holds pair p; its expert's first pair is the lowest q
                // with the same id, found by an atomic minimum in a table over
                // the experts (the logits' LDS area, free after the top-k;
                // the wave's LDS operations run in order); first pairs are
                // numbered by a ballot
                int* first_of = reinterpret_cast<int*>(s_z);
                const int e = lane < PT ? s_ids[lane] : -1;
                if (lane < PT) first_of[e] = 0x7fffffff;
                if (lane < PT) atomicMin(&first_of[e], lane);
                const int firstq = lane < PT ? first_of[e] : lane;
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
            lds_barrier();
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
        lds_barrier();
        const int U = s_misc[0];
        // For five or more tokens an item's cost grows with the number of
        // tokens that chose its expert, so the items are dealt by weight: the
        // distinct experts ranked by that number (descending, ties to the
        // lower index; s_order[rank] = distinct index), their chunks in rank
        // order, one pass over the workgroups forward, the next backward.
        // Which workgroup computes an item does not change its arithmetic.
        // (At 2-4 tokens the extra registers cost more than the balance gains.)
        constexpr bool kBal = T >= 5;
        int* s_order = s_first;
        if constexpr (kBal) {
            if (tid < U) {
                int n = 0;
#pragma unroll
                for (int t = 0; t < T; ++t) n += s_upair[tid * T + t] >= 0;
                int rank = 0;
                for (int v = 0; v < U; ++v) {
                    int nv = 0;
#pragma unroll
                    for (int t = 0; t < T; ++t) nv += s_upair[v * T + t] >= 0;
                    rank += nv > n || (nv == n && v < tid);
                }
                s_order[rank] = tid;
            }
            lds_barrier();
        }

        const size_t lstrideD = (size_t)E * D * nkbF;
        // The down rows of this thread's first (expert, block) item, which
        // the DOWN phase needs whatever the flags say, are loaded right after
        // each batch of item loads and land during the SwiGLU dot products.
        // Loads return in order: issued before the item loads they would hold
        // up the item products, issued before the flag wait every poll of it.
        uint32_t qd0[8][W];
        uint16_t scd0[8];           // raw fp16 scales: converting them here would wait for the loads
        auto issue_down_prefetch = [&]() {
            // unconditional and clamped in bounds (only the rows of a real
            // first item are used), so later waits count them at compile time
            const int it = min(tid, U * nkbF - 1);
            const int u = it / nkbF, kb = it - u * nkbF;
            const int e = s_uniq[u];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int d = min(d_lo + min(r, nrows - 1), D - 1);
                const size_t blk = (size_t)l * lstrideD + ((size_t)e * D + d) * nkbF + kb;
                load_block<W>(m.down_q, blk, qd0[r]);
                scd0[r] = ld_scale(m.down_s + blk);
            }
        };
        {
            const int n_items = U * nch;
            const size_t lstrideGU = (size_t)E * F * nkbD;
            const bool kact = lane < nkbD;                    // d_model <= 2048: one block per lane
            const int kbc = kact ? lane : nkbD - 1;           // loads stay in bounds
            // item a of the round starting at it0 (pass (it0 - w) / G + a): w,
            // or G - 1 - w on odd passes of the weighted order; valid below
            // n_items
            auto ita = [&](int it0, int a) {
                if constexpr (kBal) {
                    const int p = (it0 - w) / G + a;
                    return p * G + ((p & 1) ? G - 1 - w : w);
                }
                return it0 + a * G;
            };
            // distinct expert of item it: by rank when dealt by weight
            auto item_expert = [&](int it) { return kBal ? s_order[it / nch] : it / nch; };
            for (int it0 = w; it0 < n_items; it0 += G * kMaxItemsInFlight) {
                int tmask[kMaxItemsInFlight];       // tokens that chose the item's expert
                int ie[kMaxItemsInFlight];          // the item's expert
#pragma unroll
                for (int a = 0; a < kMaxItemsInFlight; ++a) {
                    const int it = ita(it0, a);
                    int msk = 0, e = 0;
                    if (it < n_items) {
                        const int u = item_expert(it);
#pragma unroll
                        for (int t = 0; t < T; ++t) msk |= (s_upair[u * T + t] >= 0) << t;
                        e = s_uniq[u];
                    }
                    tmask[a] = __builtin_amdgcn_readfirstlane(msk);
                    ie[a] = __builtin_amdgcn_readfirstlane(e);
                }
                uint32_t q[kMaxItemsInFlight][8][W];
                uint16_t sr[kMaxItemsInFlight][8];
#pragma unroll
                for (int a = 0; a < kMaxItemsInFlight; ++a) {
                    const int it = ita(it0, a);
                    if (it >= n_items) continue;
                    const int c = it - (it / nch) * nch;
                    const int f0 = 16 * c + 4 * wave;
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const size_t blk = (size_t)l * lstrideGU + ((size_t)ie[a] * F + f0 + (r & 3)) * nkbD + kbc;
                        load_block<W>(r < 4 ? m.gate_q : m.up_q, blk, q[a][r]);
                        sr[a][r] = ld_scale((r < 4 ? m.gate_s : m.up_s) + blk);
                    }
                }
                issue_down_prefetch();       // the same rows every batch
                // Gate and up sums of (item a, token t, row r) are formed one
                // token at a time by the same instruction sequence for every
                // batch size (the block products rounded on their own, never
                // fused into a later add), so a token's sums do not depend on
                // the batch.  They are gathered so lane (a T + t) 4 + r holds
                // the pair for row r, and one SwiGLU evaluation covers them
                // all.  Lanes past the last block use a zero scale.
                static_assert(4 * T * kMaxItemsInFlight <= 64, "one lane per (item, token, row)");
                float gv = 0.0f, uv = 0.0f;
                {
                    // token by token: its u halves from LDS (8 16-byte reads
                    // per lane), the levels unpacked for each token that chose
                    // the item's expert; sums staged in LDS
                    float* gu = s_gu + wave * (kMaxItemsInFlight * T * 8);
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        bool any = false;
#pragma unroll
                        for (int a = 0; a < kMaxItemsInFlight; ++a)
                            any = any || (ita(it0, a) < n_items && ((tmask[a] >> t) & 1));
                        if (!any) continue;
                        uint32_t xt[32];
#pragma unroll
                        for (int q4 = 0; q4 < 8; ++q4) {
                            const uint4 v = *reinterpret_cast<const uint4*>(xhw + (t * nkbD + kbc) * kXhWords + 4 * q4);
                            xt[4 * q4] = v.x;
                            xt[4 * q4 + 1] = v.y;
                            xt[4 * q4 + 2] = v.z;
                            xt[4 * q4 + 3] = v.w;
                        }
#pragma unroll
                        for (int a = 0; a < kMaxItemsInFlight; ++a) {
                            if (ita(it0, a) >= n_items || !((tmask[a] >> t) & 1)) continue;
#pragma unroll
                            for (int r = 0; r < 8; ++r) {
                                uint32_t lv[16];
                                levels16<BITS>(q[a][r], lv, uk);
                                const float sc = kact ? h2f(sr[a][r]) : 0.0f;
                                const float s = wave_sum_f32(__fmul_rn(sc, dot32h(lv, xt, xt + 16)));
                                if (lane == 0) gu[(a * T + t) * 8 + r] = s;
                            }
                        }
                    }
                    const int a = lane / (4 * T), t = (lane >> 2) % T, r = lane & 3;
                    bool take;
                    if constexpr (kBal) {
                        int tm = 0;                 // tokens of this lane's item (none past the last)
#pragma unroll
                        for (int b = 0; b < kMaxItemsInFlight; ++b)
                            if (a == b && ita(it0, b) < n_items) tm = tmask[b];
                        take = a < kMaxItemsInFlight && ((tm >> t) & 1);
                    } else {
                        take = a < kMaxItemsInFlight && it0 + a * G < n_items && ((tmask[a] >> t) & 1);
                    }
                    if (take) {
                        gv = gu[(a * T + t) * 8 + r];
                        uv = gu[(a * T + t) * 8 + 4 + r];
                    }
                }
                {
                    const int a = lane / (4 * T), t = (lane >> 2) % T, r = lane & 3;
                    int tm = 0;
#pragma unroll
                    for (int b = 0; b < kMaxItemsInFlight; ++b)
                        if (a == b && ita(it0, b) < n_items) tm = tmask[b];
                    const float hv = silu_mul(gv, uv);
                    if (a < kMaxItemsInFlight && ((tm >> t) & 1)) s_hloc[(a * T + t) * 16 + 4 * wave + r] = hv;
                }
                lds_barrier();
                if (tid < 8 * T * kMaxItemsInFlight) {
                    const int a = tid / (8 * T), rem = tid - a * 8 * T, t = rem >> 3, mm = rem & 7;
                    const int it = ita(it0, a);
                    if (it < n_items) {
                        const int u = item_expert(it), c = it - (kBal ? it / nch : u) * nch;
                        const int pr = s_upair[u * T + t];
                        if (pr >= 0) {
                            _Float16 h0, l0, h1, l1;
                            split_f16(s_hloc[(a * T + t) * 16 + mm], h0, l0);
                            split_f16(s_hloc[(a * T + t) * 16 + mm + 8], h1, l1);
                            uint32_t* dst = P.hp + (size_t)l * hp_layer + ((size_t)pr * nch + c) * kHBW;
                            st_u32(dst + mm, as_u32(half2_t{h0, h1}));
                            st_u32(dst + 8 + mm, as_u32(half2_t{l0, l1}));
                        }
                    }
                }
                lds_barrier();
            }
        }
        // this workgroup's SwiGLU rows of layer l are stored (every thread's
        // write-through stores have completed): raise its flag
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) ll_store(fl_ + (size_t)w * kFLW, base[0] + (uint32_t)l + 1u, 1u);
        if (w >= U * nch) issue_down_prefetch();     // no items in this workgroup

        // -------------------------------------------------------------- DOWN
        {
            // every workgroup's flag: thread g waits for workgroup g's
            bool ok = true;
            for (int g = tid; g < G; g += kThreads) {
                uint32_t pay[1];
                ok = ok && ll_wait<1>([&](int) -> const u64* { return fl_ + (size_t)g * kFLW; },
                                      [&](int) { return base[0] + (uint32_t)l + 1u; }, pay, 1, P);
            }
            STACK_CHECK_OK(ok);
            const uint32_t* hpp = P.hp + (size_t)l * hp_layer;
            constexpr int kTG = T <= 4 ? T : 2;     // tokens whose h halves are held at once
            for (int it = tid; it < U * nkbF; it += kThreads) {
                const int u = it / nkbF, kb = it - u * nkbF;
                const int e = s_uniq[u];
#pragma unroll 1
                for (int t0 = 0; t0 < T; t0 += kTG) {
                    int prs[kTG];
                    bool any = false;
#pragma unroll
                    for (int tt = 0; tt < kTG; ++tt) {
                        prs[tt] = t0 + tt < T ? s_upair[u * T + t0 + tt] : -1;
                        any = any || prs[tt] >= 0;
                    }
                    if (!any) continue;
                    uint32_t hv[kTG][32];               // hi pairs 0..15, lo pairs 16..31
#pragma unroll
                    for (int tt = 0; tt < kTG; ++tt) {
                        if (prs[tt] < 0) continue;
                        // block kb of d_ff = 16-row chunks 2kb (pairs 0..7) and 2kb+1 (pairs 8..15)
#pragma unroll
                        for (int hc = 0; hc < 2; ++hc) {
                            const uint4* s0 =
                                reinterpret_cast<const uint4*>(hpp + ((size_t)prs[tt] * nch + 2 * kb + hc) * kHBW);
                            const uint4 a0 = s0[0], a1 = s0[1], b0 = s0[2], b1 = s0[3];
                            const uint32_t v[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                                                    b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                hv[tt][8 * hc + i] = v[i];
                                hv[tt][16 + 8 * hc + i] = v[8 + i];
                            }
                        }
                    }
                    for (int r0 = 0; r0 < nrows; r0 += 8) {
                        uint32_t qd[8][W];
                        float scd[8];
                        if (it == tid && r0 == 0) {
                            // the rows loaded before the wait
#pragma unroll
                            for (int r = 0; r < 8; ++r) {
#pragma unroll
                                for (int k = 0; k < W; ++k) qd[r][k] = qd0[r][k];
                                scd[r] = h2f(scd0[r]);
                            }
                        } else {
#pragma unroll
                            for (int r = 0; r < 8; ++r) {  // clamped rows: every load is issued
                                const int rr = min(r0 + r, nrows - 1);
                                const size_t blk = (size_t)l * lstrideD + ((size_t)e * D + d_lo + rr) * nkbF + kb;
                                load_block<W>(m.down_q, blk, qd[r]);
                                scd[r] = h2f(ld_scale(m.down_s + blk));
                            }
                        }
#pragma unroll
                        for (int r = 0; r < 8; ++r) {
                            if (r0 + r >= nrows) continue;
                            uint32_t lv[16];
                            levels16<BITS>(qd[r], lv, uk);
#pragma unroll
                            for (int tt = 0; tt < kTG; ++tt) {
                                if (prs[tt] < 0) continue;
                                part[((size_t)prs[tt] * DPW + r0 + r) * nkbF + kb] =
                                    __fmul_rn(scd[r], dot32h(lv, hv[tt], hv[tt] + 16));
                            }
                        }
                    }
                }
            }
            lds_barrier();
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
            lds_barrier();
            // y rows (slots in order with their gates), residual, sums of squares
            for (int o = tid; o < T * nrows; o += kThreads) {
                const int t = o / nrows, r = o - t * nrows;
                // slots added in order with their gates; reads issued 8 at a time
                float yv = 0.0f;
                int j = 0;
                for (; j + 8 <= K; j += 8) {
                    float gv8[8], ov[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        gv8[i] = s_gates[t * K + j + i];
                        ov[i] = s_o[(t * K + j + i) * DPW + r];
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) yv = yv + gv8[i] * ov[i];
                }
                for (; j < K; ++j) yv = yv + s_gates[t * K + j] * s_o[(t * K + j) * DPW + r];
                const int d = d_lo + r;
                const float hn = s_hres[t * DPW + r] + yv;
                s_hres[t * DPW + r] = hn;
                if (l + 1 < L) ll_store(sl_ + ((size_t)w * kSlots + t) * kSLW + r, base[t] + (uint32_t)l + 1u,
                                        __float_as_uint(hn));
                else P.h_out[(size_t)t * D + d] = hn;
                if (P.h_layers) P.h_layers[((size_t)l * T + t) * D + d] = hn;
                s_hloc[t * nrows + r] = hn;
            }
            lds_barrier();
            if (l + 1 < L && tid < T) {
                double ss = 0.0;
                for (int r = 0; r < nrows; ++r) {
                    const double v = (double)s_hloc[tid * nrows + r];
                    ss += v * v;
                }
                u64* q = sl_ + ((size_t)w * kSlots + tid) * kSLW + kSSWord;
                const uint32_t tg = base[tid] + (uint32_t)l + 1u;
                ll_store(q, tg, (uint32_t)__double2loint(ss));
                ll_store(q + 1, tg, (uint32_t)__double2hiint(ss));
            }
        }
    }
    // the last workgroup to finish advances the epoch bases of the slots this
    // launch used and resets the completion counter for the next launch
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(&P.hdr[kHdrDone], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == (uint32_t)G - 1) {
            for (int t = 0; t < T; ++t)
                __hip_atomic_store(&P.hdr[kHdrBase + t], base[t] + (uint32_t)L, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&P.hdr[kHdrDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// A plain launch of G <= (compute units) workgroups, which must all be
// resident at once (they wait for each other's words).  A compute unit holds
// one: checked once per device with the occupancy API at the largest
// dynamic LDS size, and the LDS plan never asks for more.  A cooperative
// launch would guarantee residency too, but its dispatch costs more than
// several layers of this kernel (measured).  Should other work hold compute
// units for longer than the kernel's wall-clock limit, the waits end there
// with the error word set.
template <int T, int BITS, int KPER, int EPWM>
hipError_t launch_stack_t(StackParams& P, size_t lds, hipStream_t s) {
    auto fn = decode_stack_kernel<T, BITS, KPER, EPWM>;
    // the dynamic LDS limit is raised and residency checked once per device;
    // two threads making their first call at the same time do the same work
    static std::atomic<int> attr_done[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!attr_done[dev].load(std::memory_order_acquire)) {
        // all of LDS the kernel's own (static) allocation leaves
        hipFuncAttributes fa{};
        e = hipFuncGetAttributes(&fa, (const void*)fn);
        if (e != hipSuccess) return e;
        const size_t dyn_max = kStackLdsLimit - fa.sharedSizeBytes;
        e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn_max);
        if (e != hipSuccess) return e;
        int per_cu = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fn, kThreads, dyn_max);
        if (e != hipSuccess) return e;
        if (per_cu < 1) return hipErrorCooperativeLaunchTooLarge;
        attr_done[dev].store(1, std::memory_order_release);
    }
    void* args[] = {&P};
    return hipLaunchKernel((const void*)fn, dim3(P.G), dim3(kThreads), args, (unsigned)lds, s);
}

template <int T, int BITS>
hipError_t launch_stack_e(StackParams& P, size_t lds, hipStream_t s) {
    // logits per lane in the top-k (KPER) and router experts per workgroup
    // (EPWM) are compile-time bounds
    const int E = P.m.n_experts, epw = (E + P.G - 1) / P.G;
    if (E <= 128 && epw <= 2) return launch_stack_t<T, BITS, 2, 2>(P, lds, s);
    if (E <= 512 && epw <= 2) return launch_stack_t<T, BITS, 8, 2>(P, lds, s);
    return launch_stack_t<T, BITS, 16, kMaxEPW>(P, lds, s);
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

// Declarations shared by the persistent decode-step kernel (stack_kernel.hpp,
// instantiated per batch size in stack_t1.hip .. stack_t8.hip) and its host
// side (stack.hip): kernel parameters, constants and the layouts of the
// workspace and of LDS.
#pragma once

#include "common.hpp"

namespace qmoe {
namespace stk {

typedef unsigned long long u64;

constexpr int kThreads = 256;
constexpr int kSlots = 8;              // token slots of the tagged buffers (their layout never depends on T)
constexpr int kMaxEPW = 4;             // router experts per workgroup
constexpr long long kTimeoutTicks = 400000000LL;   // 4 s of the 100 MHz wall clock
constexpr int kHBW = 32;               // words per (pair, 16-row chunk) h line (8 hi pairs, 8 lo pairs)
constexpr int kSLW = 32;               // tagged words per (workgroup, token) residual line
constexpr int kSSWord = 16;            // word of that line holding the sum of squares (2 words)
constexpr int kLGW = 8;                // tagged words per (workgroup, token) logit line
constexpr int kFLW = 16;               // words per workgroup flag: one 128-byte line each
constexpr int kMaxItemsInFlight = 2;   // gate/up items whose loads are issued together
constexpr int kXhWords = 36;           // words per u block row in LDS: 16 hi pairs, 16 lo pairs, 4 pad
constexpr int kMaxDPW = 16;            // d_model rows per workgroup
// bytes of the per-wave top-k scratch at the end of the misc area:
// candidates (value, id) 128 per wave, keys 64, selections (value, id) 64,
// histogram 128
constexpr int kTopkScratchBytes = 4 * (128 * (8 + 4) + 64 * 4 + 64 * (8 + 4) + 128 * 4);
// workspace header (uint32 words): epoch bases of the 8 token slots, the
// launch-completion counter and the error word
constexpr int kHdrBase = 0;
constexpr int kHdrDone = 64;
constexpr int kHdrErr = MOE_STACK_ERROR_OFFSET / 4;
constexpr size_t kHdrBytes = 4096;

struct StackParams {
    moe_stack_t m;
    const void* x;
    int x_bf16;
    int T;
    float* h_out;
    int32_t* ids_out;
    float* gates_out;
    float* h_layers;    // [L][T][D] residual after each layer, or null
    double eps;
    int G;
    uint32_t* hdr;      // workspace header (see kHdr*)
    u64* sl;            // [G][kSlots][kSLW]  residual rows of workgroup g (+ sum of squares), tagged
    u64* lg;            // [G][kSlots][kLGW]  fp64 logits of workgroup g's experts (lo, hi words), tagged
    u64* fl;            // [G][kFLW]          flag: workgroup g's SwiGLU rows of this layer are stored
    uint32_t* hp;       // [L][T*K][F/16][kHBW] SwiGLU h as fp16 pairs: 8 hi words, then 8 lo words
    int lds_us, lds_part, lds_misc, lds_xh;
};

__host__ __device__ inline int misc_head_bytes(int PT, int T) { return (16 * PT + 2 * PT * T + 15) & ~15; }
__host__ __device__ inline int hloc_floats(int DPW, int T) {
    const int a = (DPW > 16 ? DPW : 16) * T;
    const int b = 16 * T * kMaxItemsInFlight;
    return a > b ? a : b;
}
// floats of the per-(wave, item, token, row) gate/up sums staged in LDS
__host__ __device__ inline int gu_floats(int T) { return kMaxItemsInFlight * T * 4 * 8; }
// byte offset (from the misc base) of the top-k candidate arrays, past
// s_ids .. s_gu, 16-byte aligned
__host__ __device__ inline int misc_tail_offset(int PT, int T, int DPW) {
    const int end = misc_head_bytes(PT, T) + 8 * 4 * kMaxEPW * T + 4 * hloc_floats(DPW, T) + 16 + 8 * 4 * T +
                    4 * T * DPW + 4 * gu_floats(T);
    return (end + 15) & ~15;
}

// Launches decode_stack_kernel for batch size T (2- or 3-bit weights by
// P.m.bits); defined in stack_t<T>.hip.
template <int T>
hipError_t launch_stack_T(StackParams& P, size_t lds, hipStream_t s);

}  // namespace stk
}  // namespace qmoe

// Declarations shared by the persistent decode-step kernel (stack_kernel.hpp,
// instantiated per batch size in stack_t1.hip .. stack_t8.hip) and its host
// side (stack.hip): kernel parameters, constants and the LDS sub-layout.
#pragma once

#include "common.hpp"

namespace qmoe {
namespace stk {


constexpr int kThreads = 256;
constexpr int kMaxEPW = 4;             // router experts per workgroup
constexpr int kLine = 64;              // ints between barrier counters (256 B)
constexpr long long kTimeoutTicks = 400000000LL;   // 4 s of the 100 MHz wall clock
constexpr int kZW = 16;                // doubles per (workgroup, token) logit line
constexpr int kHW = 32;                // floats per (workgroup, token) residual line
constexpr int kHBW = 32;               // words per (pair, 16-row chunk) h line
constexpr int kMaxItemsInFlight = 2;   // gate/up items whose loads are issued together
constexpr int kXhWords = 17;           // words per fp16 u block row in LDS (16 pairs + 1 pad)

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
    int* sync;          // 8 counters (256 B apart), done counter, error flag
    double* zb;         // [L][G][T][kZW]      logits of the workgroup's experts
    float* hb;          // [L][G][T][kHW]      residual rows of the workgroup
    double* sb;         // [L][G][16]          sums of squares per token
    uint32_t* hp;       // [L][T*K][F/16][kHBW] SwiGLU h, fp16 pairs in unpack order
    int lds_us, lds_part, lds_misc, lds_pre, lds_wr, lds_xh;
    // down-projection rows prefetched into LDS: up to pre_cap distinct
    // experts, each [rows][blocks][W] codes (pre_cstride bytes) followed by
    // [rows][blocks] fp16 scales (pre_sstride bytes); copy granules in bytes
    int pre_cap, pre_cstride, pre_sstride, pre_cgran, pre_sgran;
};

__host__ __device__ inline int misc_head_bytes(int PT, int T) { return (16 * PT + 2 * PT * T + 15) & ~15; }
__host__ __device__ inline int hloc_floats(int DPW, int T) {
    const int a = (DPW > 16 ? DPW : 16) * T;
    const int b = 16 * T * kMaxItemsInFlight;
    return a > b ? a : b;
}
// byte offset (from the misc base) of the top-k candidate arrays, past
// s_ids .. s_hres, 16-byte aligned
__host__ __device__ inline int misc_tail_offset(int PT, int T, int DPW) {
    const int end = misc_head_bytes(PT, T) + 8 * 4 * kMaxEPW * T + 4 * hloc_floats(DPW, T) + 16 + 8 * 4 * T +
                    4 * T * DPW;
    return (end + 15) & ~15;
}

// Launches decode_stack_kernel for batch size T (2- or 3-bit weights by
// P.m.bits); defined in stack_t<T>.hip.
template <int T>
hipError_t launch_stack_T(StackParams& P, size_t lds, hipStream_t s);

}  // namespace stk
}  // namespace qmoe

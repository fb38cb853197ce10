// Host side of the persistent decode-step kernel: workspace layout, LDS plan
// and the dispatch by batch size (the kernel itself is in stack_kernel.hpp).
#include "stack.hpp"

using namespace qmoe::stk;

namespace qmoe {

// Workspace: header, then the tagged exchange buffers (sized for
// kStackMaxGrid workgroups and kSlots token slots, so their layout is the
// same for every batch size and device), then the per-layer SwiGLU rows.
// Every 128-byte line of the exchange buffers is written by one workgroup
// only (residual lines 256 B, logit lines of two slots, one flag line each).
StackWs stack_ws_layout(int T, int D, int F, int E, int K, int G, int L) {
    StackWs w{};
    size_t off = 0;
    w.hdr = off;
    off += kHdrBytes;
    w.rows = off;                                              // residual rows + sums of squares
    off += align256(sizeof(u64) * (size_t)kStackMaxGrid * kSlots * kSLW);
    w.logits = off;
    off += align256(sizeof(u64) * (size_t)kStackMaxGrid * kSlots * kLGW);
    w.flags = off;
    off += align256(sizeof(u64) * (size_t)kStackMaxGrid * kFLW);
    w.hp = off;
    off += align256(sizeof(uint32_t) * (size_t)L * T * K * (F / 16) * kHBW);
    w.total = off;
    (void)D;
    (void)E;
    (void)G;
    return w;
}

// LDS plan of one workgroup.
struct StackLds {
    size_t us, part, xh, misc, total;
};

static StackLds stack_lds_plan(int T, int D, int F, int E, int K, int G, int bits) {
    StackLds p{};
    const int DPW = (D + G - 1) / G;
    const int PT = T * K;
    const int nkbF = F / 32;
    (void)bits;
    size_t off = 0;
    p.us = off;                        // per-pair sums [PT][DPW] of the DOWN phase
    off += align256(sizeof(float) * (size_t)PT * DPW);
    // ROUTE and FFN: logits [T][E] doubles, then u as fp16 halves (padded
    // rows); DOWN: per-block partial sums [PT][DPW][F/32] floats
    p.part = off;
    const size_t part_bytes = sizeof(float) * (size_t)PT * DPW * nkbF;
    const size_t z_bytes = align256(sizeof(double) * (size_t)T * E);
    const size_t xh_bytes = sizeof(uint32_t) * (size_t)T * (D / 32) * kXhWords;
    p.xh = off + z_bytes;
    off += align256(part_bytes > z_bytes + xh_bytes ? part_bytes : z_bytes + xh_bytes);
    p.misc = off;
    off += align256((size_t)misc_tail_offset(PT, T, DPW) + kTopkScratchBytes);
    p.total = off;
    return p;
}

size_t stack_lds_bytes(int T, int D, int F, int E, int K, int G, int bits) {
    return stack_lds_plan(T, D, F, E, K, G, bits).total;
}

hipError_t launch_decode_stack(const moe_stack_t& m, const void* x, int x_bf16, int T, float* h_out,
                               int32_t* ids_out, float* gates_out, float* h_layers, double eps, char* ws, const StackWs& L, int G,
                               hipStream_t s) {
    StackParams P{};
    P.m = m;
    P.x = x;
    P.x_bf16 = x_bf16;
    P.T = T;
    P.h_out = h_out;
    P.ids_out = ids_out;
    P.gates_out = gates_out;
    P.h_layers = h_layers;
    P.eps = eps;
    P.G = G;
    P.hdr = (uint32_t*)(ws + L.hdr);
    P.sl = (u64*)(ws + L.rows);
    P.lg = (u64*)(ws + L.logits);
    P.fl = (u64*)(ws + L.flags);
    P.hp = (uint32_t*)(ws + L.hp);
    const StackLds pl = stack_lds_plan(T, m.d_model, m.d_ff, m.n_experts, m.top_k, G, m.bits);
    P.lds_us = (int)pl.us;
    P.lds_part = (int)pl.part;
    P.lds_xh = (int)pl.xh;
    P.lds_misc = (int)pl.misc;
    const size_t lds = pl.total;
#define QMOE_ST(N) \
    case N:           \
        return launch_stack_T<N>(P, lds, s);
    switch (T) {
        QMOE_ST(1) QMOE_ST(2) QMOE_ST(3) QMOE_ST(4) QMOE_ST(5) QMOE_ST(6) QMOE_ST(7) QMOE_ST(8)
        default:
            return hipErrorInvalidValue;
    }
#undef QMOE_ST
}

}  // namespace qmoe

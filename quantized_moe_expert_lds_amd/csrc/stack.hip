// Host side of the persistent decode-step kernel: workspace layout, LDS plan
// and the dispatch by batch size (the kernel itself is in stack_kernel.hpp).
#include "stack.hpp"

using namespace qmoe::stk;

namespace qmoe {

// Workspace: header, then the tagged residual-row, logit and flag buffers
// (sized for kStackMaxGrid workgroups and kSlots token slots, so their
// layout is the same for every batch size and device), then the per-layer
// SwiGLU rows.
StackWs stack_ws_layout(int T, int D, int F, int E, int K, int G, int L) {
    StackWs w{};
    size_t off = 0;
    w.sync = off;
    off += kHdrBytes;
    w.zbuf = off;                                              // residual rows + sums of squares
    off += align256(sizeof(u64) * (size_t)kStackMaxGrid * kSlots * kSLW);
    w.hres = off;                                              // logits
    off += align256(sizeof(u64) * (size_t)kStackMaxGrid * kSlots * kLGW);
    w.ssp = off;                                               // flags
    off += align256(sizeof(u64) * (size_t)kStackMaxGrid * kFLW);
    w.hbuf = off;
    off += align256(sizeof(uint32_t) * (size_t)L * T * K * (F / 16) * kHBW);
    w.total = off;
    (void)D;
    (void)E;
    (void)G;
    return w;
}

// LDS plan of one workgroup.  Whatever the fixed regions leave of the LDS
// limit holds prefetched down-projection rows, whole experts at a time.
struct StackLds {
    size_t us, part, wr, xh, misc, pre, total;
    int pre_cap, cstride, sstride, cgran, sgran;
};

static StackLds stack_lds_plan(int T, int D, int F, int E, int K, int G, int bits) {
    StackLds p{};
    const int DPW = (D + G - 1) / G;
    const int EPW = (E + G - 1) / G;
    const int PT = T * K;
    const int W = bits == 2 ? 2 : 3;
    const int nkbF = F / 32;
    size_t off = 0;
    p.us = off;                        // per-pair sums [PT][DPW] of the DOWN phase
    off += align256(sizeof(float) * (size_t)PT * DPW);
    // ROUTE and FFN: logits [T][E] doubles, then u in fp16 pair order
    // (padded); DOWN: per-block partial sums [PT][DPW][F/32] floats
    p.part = off;
    const size_t part_bytes = sizeof(float) * (size_t)PT * DPW * nkbF;
    const size_t z_bytes = align256(sizeof(double) * (size_t)T * E);
    const size_t xh_bytes = sizeof(uint32_t) * (size_t)T * (D / 32) * kXhWords;
    p.xh = off + z_bytes;
    off += align256(part_bytes > z_bytes + xh_bytes ? part_bytes : z_bytes + xh_bytes);
    p.wr = off;                        // router rows
    off += align256(sizeof(float) * (size_t)EPW * D);
    p.misc = off;
    size_t mb = (size_t)misc_head_bytes(PT, T);
    mb = (size_t)misc_tail_offset(PT, T, DPW) + 256 * (sizeof(double) + 2 * sizeof(int));
    off += align256(mb);
    p.pre = off;
    p.total = off;
    // prefetch: at most 8 rows per workgroup; copy granule 16 B where rows of
    // codes / scales are multiples of 16 B, else 4 B; odd block counts are
    // not prefetched
    p.cstride = (int)((sizeof(uint32_t) * (size_t)DPW * nkbF * W + 15) & ~(size_t)15);
    p.sstride = (int)((sizeof(uint16_t) * (size_t)DPW * nkbF + 15) & ~(size_t)15);
    p.cgran = (nkbF * W) % 4 == 0 ? 16 : 4;
    p.sgran = nkbF % 8 == 0 ? 16 : 4;
    if (DPW <= 8 && nkbF % 2 == 0 && off < (size_t)kStackLdsLimit) {
        const size_t per = (size_t)p.cstride + p.sstride;
        size_t cap = ((size_t)kStackLdsLimit - off) / per;
        if (cap > (size_t)PT) cap = PT;
        p.pre_cap = (int)cap;
        p.total = off + cap * per;
    }
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
    P.hdr = (uint32_t*)(ws + L.sync);
    P.sl = (u64*)(ws + L.zbuf);
    P.lg = (u64*)(ws + L.hres);
    P.fl = (u64*)(ws + L.ssp);
    P.hp = (uint32_t*)(ws + L.hbuf);
    const StackLds pl = stack_lds_plan(T, m.d_model, m.d_ff, m.n_experts, m.top_k, G, m.bits);
    P.lds_us = (int)pl.us;
    P.lds_part = (int)pl.part;
    P.lds_wr = (int)pl.wr;
    P.lds_xh = (int)pl.xh;
    P.lds_misc = (int)pl.misc;
    P.lds_pre = (int)pl.pre;
    // prefetch needs 16-byte aligned rows for the 16-byte granule
    const bool al = ((uintptr_t)m.down_q % 16 == 0) && ((uintptr_t)m.down_s % 16 == 0);
    P.pre_cap = al ? pl.pre_cap : 0;
    P.pre_cstride = pl.cstride;
    P.pre_sstride = pl.sstride;
    P.pre_cgran = pl.cgran;
    P.pre_sgran = pl.sgran;
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

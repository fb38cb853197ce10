// Declarations of the int8-activation prefill (prefill_q8.hip) and of the
// pieces of the fp16 prefill it shares (prefill.hip).
#pragma once

#include "common.hpp"

namespace qmoe {

// workspace: Q8 codes and scales of x and of h, per-pair rows, the tile list
struct PrefillQ8Ws {
    size_t xq, xd, hq, hd, obuf, tiles, ntiles, total;
};

inline PrefillQ8Ws prefill_q8_ws_layout(int T, int D, int F, int E, int K) {
    PrefillQ8Ws w{};
    size_t off = 0;
    const size_t P = (size_t)T * K;
    w.xq = off;
    off += align256((size_t)T * D);
    w.xd = off;
    off += align256(sizeof(float) * (size_t)T * (D / 32));
    w.hq = off;
    off += align256(P * F);
    w.hd = off;
    off += align256(sizeof(float) * P * (F / 32));
    w.obuf = off;
    off += align256(sizeof(float) * P * D);
    w.tiles = off;
    off += align256(sizeof(int4) * (size_t)prefill_max_tiles(T, E, K));
    w.ntiles = off;
    off += align256(sizeof(int) * 4);
    w.total = off;
    return w;
}

hipError_t launch_prefill_q8(const moe_experts_t& ex, const void* x, int x_bf16, int T, const float* gates,
                             int K, const int32_t* offsets, const int32_t* pairs, float* y, char* ws,
                             const PrefillQ8Ws& L, hipStream_t s);
hipError_t launch_quantize_q8(const void* x, int x_bf16, size_t nblocks, int8_t* q, float* d, hipStream_t s);
// pieces of the fp16 prefill shared with the int8 one
hipError_t launch_prefill_tiles(const int32_t* offsets, int E, int P, int max_tiles, int4* tiles, int* ntiles,
                                hipStream_t s);
hipError_t launch_prefill_combine(const float* obuf, int T, int K, int D, float* y, hipStream_t s);

}  // namespace qmoe

// Host-side driver of the C ABI for the sanitizer build (AddressSanitizer and
// UndefinedBehaviorSanitizer on the library's host code).  Every call here
// either fails argument validation or, with valid arguments, stops at the
// device check (this runs on a machine without a GPU); no kernel is launched
// and no pointer handed to the library is dereferenced.  Exits non-zero on
// the first unexpected status; the sanitizers abort on any error they find.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "../include/moe_ffn.h"

static int g_fail = 0;

static void expect(const char* what, int got, int want, int want2 = 1) {
    if (got != want && got != want2) {
        fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
        g_fail = 1;
    }
}

int main() {
    // fake device addresses: validation rejects the calls before any use
    void* fake = (void*)(uintptr_t)4096;
    const uint32_t* fq = (const uint32_t*)fake;
    const uint16_t* fs = (const uint16_t*)fake;
    const float* ff = (const float*)fake;

    // status strings, including unknown codes
    for (int c = -8; c <= 2; ++c) {
        const char* s = moe_status_string(c);
        if (!s || !strlen(s)) { fprintf(stderr, "FAIL status string %d\n", c); g_fail = 1; }
    }

    // workspace sizes: every op, valid and invalid shapes
    const int ops[] = {MOE_OP_ROUTE, MOE_OP_DECODE, MOE_OP_PREFILL, MOE_OP_PREFILL_Q8, 7, -1};
    for (int op : ops)
        for (int T : {0, 1, 8, 37, 8192})
            for (int K : {0, 1, 10, 65})
                (void)moe_workspace_size(op, T, 2048, 768, 512, K);
    if (moe_workspace_size(MOE_OP_ROUTE, 0, 2048, 0, 512, 10) != 0) { fprintf(stderr, "FAIL ws T=0\n"); g_fail = 1; }
    if (moe_workspace_size(MOE_OP_PREFILL, 8192, 2048, 768, 512, 10) == 0) { fprintf(stderr, "FAIL ws prefill\n"); g_fail = 1; }

    moe_router_t rt = {2048, 512, 10, ff, nullptr};
    moe_experts_t ex = {512, 2048, 768, 2, fq, fq, fq, fs, fs, fs};
    moe_stack_t st = {48, 512, 2048, 768, 10, 2, ff, ff, fq, fq, fq, fs, fs, fs};
    const size_t big = (size_t)1 << 40;

    // moe_route
    expect("route null router", moe_route(nullptr, fake, MOE_F32, 4, (int32_t*)fake, (float*)fake, nullptr, nullptr, fake, big, nullptr), MOE_ERR_ARG);
    expect("route no tokens", moe_route(&rt, fake, MOE_F32, 0, (int32_t*)fake, (float*)fake, nullptr, nullptr, fake, big, nullptr), MOE_ERR_ARG);
    expect("route bad dtype", moe_route(&rt, fake, 9, 4, (int32_t*)fake, (float*)fake, nullptr, nullptr, fake, big, nullptr), MOE_ERR_ARG);
    moe_router_t rk = rt; rk.top_k = 600;
    expect("route k > E", moe_route(&rk, fake, MOE_F32, 4, (int32_t*)fake, (float*)fake, nullptr, nullptr, fake, big, nullptr), MOE_ERR_ARG, MOE_ERR_UNSUPPORTED);
    moe_router_t rd = rt; rd.d_model = 2050;
    expect("route d % 32", moe_route(&rd, fake, MOE_F32, 4, (int32_t*)fake, (float*)fake, nullptr, nullptr, fake, big, nullptr), MOE_ERR_ARG, MOE_ERR_UNSUPPORTED);
    expect("route small ws", moe_route(&rt, fake, MOE_F32, 4, (int32_t*)fake, (float*)fake, nullptr, nullptr, fake, 16, nullptr), MOE_ERR_WORKSPACE);
    expect("route valid (no device)", moe_route(&rt, fake, MOE_F32, 4, (int32_t*)fake, (float*)fake, nullptr, nullptr, fake, big, nullptr), MOE_ERR_NO_DEVICE, MOE_ERR_HIP);

    // moe_ffn_decode and its no-allocation variant
    expect("decode null", moe_ffn_decode(nullptr, fake, MOE_F32, 1, (int32_t*)fake, ff, 10, (float*)fake, fake, big, nullptr), MOE_ERR_ARG);
    expect("decode T > 8", moe_ffn_decode(&ex, fake, MOE_F32, 9, (int32_t*)fake, ff, 10, (float*)fake, fake, big, nullptr), MOE_ERR_UNSUPPORTED, MOE_ERR_ARG);
    moe_experts_t eb = ex; eb.bits = 4;
    expect("decode bits 4", moe_ffn_decode(&eb, fake, MOE_F32, 1, (int32_t*)fake, ff, 10, (float*)fake, fake, big, nullptr), MOE_ERR_UNSUPPORTED);
    expect("decode k > 64", moe_ffn_decode(&ex, fake, MOE_F32, 1, (int32_t*)fake, ff, 65, (float*)fake, fake, big, nullptr), MOE_ERR_UNSUPPORTED, MOE_ERR_ARG);
    expect("decode no ws", moe_ffn_decode(&ex, fake, MOE_F32, 1, (int32_t*)fake, ff, 10, (float*)fake, nullptr, 0, nullptr), MOE_ERR_WORKSPACE);
    expect("decode valid (no device)", moe_ffn_decode(&ex, fake, MOE_BF16, 4, (int32_t*)fake, ff, 10, (float*)fake, fake, big, nullptr), MOE_ERR_NO_DEVICE, MOE_ERR_HIP);
    expect("noalloc null", moe_ffn_decode_noalloc(&ex, nullptr, MOE_F32, 1, (int32_t*)fake, ff, 10, (float*)fake, nullptr), MOE_ERR_ARG);
    expect("noalloc valid (no device)", moe_ffn_decode_noalloc(&ex, fake, MOE_F32, 1, (int32_t*)fake, ff, 10, (float*)fake, nullptr), MOE_ERR_NO_DEVICE, MOE_ERR_HIP);

    // moe_ffn_prefill and the int8 variant
    expect("prefill null", moe_ffn_prefill(&ex, nullptr, MOE_F32, 8, ff, 10, (int32_t*)fake, (int32_t*)fake, (float*)fake, fake, big, nullptr), MOE_ERR_ARG);
    expect("prefill 3-bit", moe_ffn_prefill(&eb, fake, MOE_F32, 8, ff, 10, (int32_t*)fake, (int32_t*)fake, (float*)fake, fake, big, nullptr), MOE_ERR_UNSUPPORTED);
    moe_experts_t ed = ex; ed.d_model = 2080;
    expect("prefill d % 256", moe_ffn_prefill(&ed, fake, MOE_F32, 8, ff, 10, (int32_t*)fake, (int32_t*)fake, (float*)fake, fake, big, nullptr), MOE_ERR_UNSUPPORTED);
    expect("prefill small ws", moe_ffn_prefill(&ex, fake, MOE_F32, 8, ff, 10, (int32_t*)fake, (int32_t*)fake, (float*)fake, fake, 64, nullptr), MOE_ERR_WORKSPACE);
    expect("prefill valid (no device)", moe_ffn_prefill(&ex, fake, MOE_F32, 8192, ff, 10, (int32_t*)fake, (int32_t*)fake, (float*)fake, fake, big, nullptr), MOE_ERR_NO_DEVICE, MOE_ERR_HIP);
    expect("prefill_q8 3-bit", moe_ffn_prefill_q8(&eb, fake, MOE_F32, 8, ff, 10, (int32_t*)fake, (int32_t*)fake, (float*)fake, fake, big, nullptr), MOE_ERR_UNSUPPORTED);
    expect("prefill_q8 valid (no device)", moe_ffn_prefill_q8(&ex, fake, MOE_BF16, 37, ff, 10, (int32_t*)fake, (int32_t*)fake, (float*)fake, fake, big, nullptr), MOE_ERR_NO_DEVICE, MOE_ERR_HIP);
    expect("quantize_q8 cols % 32", moe_quantize_q8(fake, MOE_F32, 4, 48, (int8_t*)fake, (float*)fake, nullptr), MOE_ERR_UNSUPPORTED);
    expect("quantize_q8 null", moe_quantize_q8(nullptr, MOE_F32, 4, 64, (int8_t*)fake, (float*)fake, nullptr), MOE_ERR_ARG);
    expect("quantize_q8 valid (no device)", moe_quantize_q8(fake, MOE_F32, 4, 64, (int8_t*)fake, (float*)fake, nullptr), MOE_ERR_NO_DEVICE, MOE_ERR_HIP);

    // residual + RMSNorm
    expect("rmsnorm null", moe_residual_rmsnorm(nullptr, ff, (float*)fake, 1, 2048, 1e-6, nullptr), MOE_ERR_ARG);
    expect("rmsnorm eps < 0", moe_residual_rmsnorm((float*)fake, ff, (float*)fake, 1, 2048, -1.0, nullptr), MOE_ERR_ARG);
    expect("rmsnorm valid (no device)", moe_residual_rmsnorm((float*)fake, ff, (float*)fake, 3, 2048, 1e-6, nullptr), MOE_ERR_NO_DEVICE, MOE_ERR_HIP);

    // whole-stack calls
    for (int T : {0, 1, 4, 9}) (void)moe_stack_workspace_size(&st, T);
    (void)moe_stack_workspace_size(nullptr, 1);
    const size_t sws = moe_stack_workspace_size(&st, 4);
    if (!sws) { fprintf(stderr, "FAIL stack workspace size\n"); g_fail = 1; }
    expect("stack null", moe_decode_stack(nullptr, fake, MOE_F32, 4, 1e-6, (float*)fake, nullptr, nullptr, nullptr, fake, sws, nullptr), MOE_ERR_ARG);
    expect("stack T=9", moe_decode_stack(&st, fake, MOE_F32, 9, 1e-6, (float*)fake, nullptr, nullptr, nullptr, fake, big, nullptr), MOE_ERR_UNSUPPORTED, MOE_ERR_ARG);
    expect("stack ids w/o gates", moe_decode_stack(&st, fake, MOE_F32, 4, 1e-6, (float*)fake, (int32_t*)fake, nullptr, nullptr, fake, sws, nullptr), MOE_ERR_ARG);
    moe_stack_t sd = st; sd.d_model = 4096;
    expect("stack d > 2048", moe_decode_stack(&sd, fake, MOE_F32, 4, 1e-6, (float*)fake, nullptr, nullptr, nullptr, fake, big, nullptr), MOE_ERR_UNSUPPORTED);
    expect("stack no ws", moe_decode_stack(&st, fake, MOE_F32, 4, 1e-6, (float*)fake, nullptr, nullptr, nullptr, nullptr, 0, nullptr), MOE_ERR_WORKSPACE);
    expect("stack valid (no device)", moe_decode_stack(&st, fake, MOE_F32, 4, 1e-6, (float*)fake, nullptr, nullptr, nullptr, fake, sws, nullptr), MOE_ERR_NO_DEVICE, MOE_ERR_HIP);
    const size_t pws = moe_prefill_stack_workspace_size(&st, 8192);
    if (!pws) { fprintf(stderr, "FAIL prefill stack workspace size\n"); g_fail = 1; }
    (void)moe_prefill_stack_workspace_size(&st, 0);
    (void)moe_prefill_stack_workspace_size(nullptr, 64);
    expect("prefill stack no chunk", moe_prefill_stack(&st, fake, MOE_F32, 100, 0, 1e-6, (float*)fake, fake, pws, nullptr), MOE_ERR_ARG);
    expect("prefill stack small ws", moe_prefill_stack(&st, fake, MOE_F32, 100, 8192, 1e-6, (float*)fake, fake, pws - 1, nullptr), MOE_ERR_WORKSPACE);
    expect("prefill stack valid (no device)", moe_prefill_stack(&st, fake, MOE_BF16, 32768, 8192, 1e-6, (float*)fake, fake, pws, nullptr), MOE_ERR_NO_DEVICE, MOE_ERR_HIP);

    if (g_fail) return 1;
    printf("host ABI driver: ok\n");
    return 0;
}

/*
 * moe_ffn.h -- C ABI of the routed mixture-of-experts FFN library (gfx950).
 *
 * The library computes one routed MoE FFN layer of a large sparse LLM: a
 * linear router picks the top-k of E experts per token, each chosen expert is
 * a SwiGLU FFN whose weights are stored in 2- or 3-bit block quantisation, and
 * the layer output is the gate-weighted sum of the k expert outputs.
 *
 * Sources: the Strata write-ups describe a model with 24,576 experts of which
 * each token uses 10 (aiproducthub "Strata Skill", section 介绍; bnskd "Strata：
 * 把 125B 大模型塞进 12GB 显卡", section 核心思路), 512 experts per layer over 48
 * layers (yudady notes "Strata — 8~12GB 显存跑 125B", section 5 table; bnskd,
 * section 投机解码), experts served from 2-bit "Q2_0" weights (aiproducthub,
 * section 功能与原则) and prefill processed in chunks of up to 8,192 tokens
 * (bnskd, section 工程细节).  The pages give no kernel interface; the calls
 * below follow that problem statement.
 *
 * Conventions common to every call
 * --------------------------------
 * - Pointers marked "device" must point to device memory of the current HIP
 *   device.  The caller owns every buffer; the library allocates and frees
 *   nothing and keeps nothing between calls except what the caller hands in.
 * - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *   enqueues asynchronous work on it; outputs are valid once the stream has
 *   reached that point.  Nothing synchronises.
 * - Return value: MOE_OK (0) or a negative MOE_ERR_* code.  Arguments are
 *   validated before anything is launched; on an error nothing is enqueued
 *   (except MOE_ERR_HIP, reported when a launch itself fails).  Nothing throws.
 * - Workspaces: `ws` is device scratch of at least moe_workspace_size(...)
 *   bytes, 256-byte aligned.  It must be zero-filled once before its first
 *   use; every call leaves the synchronisation counters it uses at zero
 *   again, so one zeroed workspace serves any number of calls.  Calls that
 *   run concurrently need distinct workspaces.
 * - Inputs are assumed finite; NaN logits give unspecified routing.
 *
 * Stored expert weights
 * ---------------------
 * Each matrix applied as x @ W with W of shape [K x N] is stored output-major:
 * row n holds its K reduction weights in blocks of 32 consecutive k.
 *   codes  uint32 [E][N][K/32][words]   words = 2 (2-bit) or 3 (3-bit)
 *   scales uint16 [E][N][K/32]          IEEE binary16 bit patterns
 * gate and up use K = d_model, N = d_ff; down uses K = d_ff, N = d_model.
 * 2-bit: code = level + 2 (levels -2..1), weight i of a block in word i/16 at
 * bits [2(i mod 16), +2).  3-bit: code = level + 4 (levels -4..3), the three
 * words are one little-endian 96-bit string, weight i at bits [3i, 3i+3).
 * Dequantised weight = level * scale, exact in fp32 for every fp16 scale
 * (the decode and stack paths apply the scale in fp32).  The prefill path
 * feeds level * scale to the fp16 matrix cores, which is exact as long as it
 * is representable in fp16: |level * scale| <= 65504, i.e. 2-bit scales up to
 * 32752 (bits 0x77FF), which quantising any fp16-representable weights
 * always gives; a larger scale makes a level -2 weight overflow to -inf in
 * prefill only.  Subnormal and zero scales are exact on every path.  The
 * SwiGLU intermediate h = silu(g) * u enters the down projection as fp16 on
 * every path, so |h| must stay below 65504.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK               0
#define MOE_ERR_ARG         -1  /* null pointer, non-positive size, bad dtype       */
#define MOE_ERR_UNSUPPORTED -2  /* shape/format outside what the kernels handle     */
#define MOE_ERR_WORKSPACE   -3  /* workspace missing, too small or misaligned       */
#define MOE_ERR_NO_DEVICE   -4  /* no HIP device, or the device is not gfx950       */
#define MOE_ERR_HIP         -5  /* a kernel launch failed (hipGetLastError)         */

/* activation dtypes */
#define MOE_F32  0
#define MOE_BF16 1

/* operations for moe_workspace_size */
#define MOE_OP_ROUTE   0
#define MOE_OP_DECODE  1
#define MOE_OP_PREFILL 2
#define MOE_OP_PREFILL_Q8 3

/* byte offset in a moe_decode_stack workspace of the int that becomes
 * nonzero if a grid barrier timed out (see moe_decode_stack) */
#define MOE_STACK_ERROR_OFFSET 2304

/* Linear router of one layer.
 *   w    device fp32 [n_experts][d_model]: expert-major, row e is the router
 *        vector of expert e (the transpose of the [d_model x n_experts]
 *        matrix in z = x W)
 *   bias device fp32 [n_experts], or NULL for no bias
 * Supported: d_model multiple of 32 and <= 16384, 1 <= top_k <= min(n_experts, 64),
 * n_experts <= 1024. */
typedef struct {
    int d_model;
    int n_experts;
    int top_k;
    const float* w;
    const float* bias;
} moe_router_t;

/* Stored experts of one layer (layout above).  All pointers device.
 * Supported: bits 2 or 3; d_model and d_ff multiples of 32, d_model <= 16384,
 * d_ff <= 4096.  Prefill additionally needs bits == 2, d_model % 256 == 0 and
 * d_ff % 128 == 0. */
typedef struct {
    int n_experts;
    int d_model;
    int d_ff;
    int bits;
    const uint32_t* gate_q;
    const uint32_t* up_q;
    const uint32_t* down_q;
    const uint16_t* gate_s;
    const uint16_t* up_s;
    const uint16_t* down_s;
} moe_experts_t;

/* A stack of MoE layers whose tensors are stored back to back, layer-major
 * (layer l of each tensor starts at l times that tensor's per-layer size).
 *   router_w device fp32 [L][n_experts][d_model] (expert-major rows)
 *   router_b device fp32 [L][n_experts], or NULL
 *   *_q, *_s device, [L] x the per-layer layouts of moe_experts_t */
typedef struct {
    int n_layers;
    int n_experts;
    int d_model;
    int d_ff;
    int top_k;
    int bits;
    const float* router_w;
    const float* router_b;
    const uint32_t* gate_q;
    const uint32_t* up_q;
    const uint32_t* down_q;
    const uint16_t* gate_s;
    const uint16_t* up_s;
    const uint16_t* down_s;
} moe_stack_t;

/* Bytes of workspace `op` needs for n_tokens tokens (0 if the arguments are
 * invalid).  For MOE_OP_ROUTE, d_ff is ignored. */
size_t moe_workspace_size(int op, int n_tokens, int d_model, int d_ff, int n_experts, int top_k);

/* Router logits, top-k selection, gates and (optionally) expert buckets.
 *
 *   z[t][e]  = sum_d x[t][d] * w[e][d] + bias[e], accumulated in fp64
 *   ids[t]   = the top_k experts by z in rank order; equal logits go to the
 *              lower expert id
 *   gates[t] = softmax over the selected logits (= softmax over all experts
 *              renormalised over the chosen k), fp64, stored as fp32
 *   buckets  = pairs p = t*top_k + j grouped by expert: bucket_offsets[e] is
 *              the exclusive prefix sum of per-expert counts, with
 *              bucket_offsets[n_experts] = n_tokens*top_k, and bucket_pairs
 *              lists the pair ids of expert 0, expert 1, ..., each bucket in
 *              ascending pair id.
 *
 *   x              device [n_tokens][d_model], fp32 or bf16 (x_dtype)
 *   topk_ids       device int32 [n_tokens][top_k]            (output)
 *   topk_w         device fp32  [n_tokens][top_k]            (output)
 *   bucket_offsets device int32 [n_experts + 1] or NULL      (output)
 *   bucket_pairs   device int32 [n_tokens * top_k] or NULL   (output)
 * Buckets are produced only when both bucket pointers are non-NULL. */
int moe_route(const moe_router_t* router, const void* x, int x_dtype, int n_tokens,
              int32_t* topk_ids, float* topk_w, int32_t* bucket_offsets, int32_t* bucket_pairs,
              void* ws, size_t ws_bytes, void* stream);

/* Expert FFN and combine for a small batch (decode / speculative verify).
 *
 *   y[t] = sum_{j < top_k} topk_w[t][j] * FFN_{topk_ids[t][j]}(x[t])
 *   FFN_e(v) = (silu(v Wg_e) * (v Wu_e)) Wd_e,  silu(g) = g / (1 + exp(-g))
 * with weights dequantised exactly, fp32 accumulation, and the slot sum in
 * ascending j.  Each distinct expert's weights are read once per call and
 * shared by the tokens that chose it.  Results for a token do not depend on
 * n_tokens or on the other tokens (bitwise).
 *
 *   x        device [n_tokens][d_model], fp32 or bf16
 *   topk_ids device int32 [n_tokens][top_k], each id in [0, n_experts), no
 *            id repeated within a token
 *   topk_w   device fp32 [n_tokens][top_k]
 *   y        device fp32 [n_tokens][d_model] (output)
 * Supported: 1 <= n_tokens <= 8, top_k <= 64. */
int moe_ffn_decode(const moe_experts_t* experts, const void* x, int x_dtype, int n_tokens,
                   const int32_t* topk_ids, const float* topk_w, int top_k, float* y,
                   void* ws, size_t ws_bytes, void* stream);

/* moe_ffn_decode without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation.  Same arguments (minus ws), limits and
 * results (bitwise) as moe_ffn_decode; the SwiGLU intermediate lives in a
 * library-owned 8 MiB array of device memory per device, held until the
 * process ends, and nothing is allocated or freed.  Every call on a device
 * shares that array, so calls that overlap on one device (different streams
 * or threads) race and give undefined results; serialise them. */
int moe_ffn_decode_noalloc(const moe_experts_t* experts, const void* x, int x_dtype, int n_tokens,
                           const int32_t* topk_ids, const float* topk_w, int top_k, float* y, void* stream);

/* Expert FFN and combine for a prefill chunk, as grouped GEMMs over the
 * expert buckets produced by moe_route.  Same result as moe_ffn_decode
 * (within fp16-operand rounding: activations and the SwiGLU intermediate
 * enter the matrix cores as fp16, accumulation is fp32).
 *
 *   x              device [n_tokens][d_model], fp32 or bf16
 *   topk_w         device fp32 [n_tokens][top_k], indexed by pair id
 *   bucket_offsets device int32 [n_experts + 1]   (from moe_route)
 *   bucket_pairs   device int32 [n_tokens*top_k]  (from moe_route)
 *   y              device fp32 [n_tokens][d_model] (output)
 * Supported: n_tokens >= 1, bits == 2 (see moe_experts_t). */
int moe_ffn_prefill(const moe_experts_t* experts, const void* x, int x_dtype, int n_tokens,
                    const float* topk_w, int top_k, const int32_t* bucket_offsets,
                    const int32_t* bucket_pairs, float* y, void* ws, size_t ws_bytes, void* stream);

/* Q8 blocks of activations, the int8 format of moe_ffn_prefill_q8 (a
 * reading of the quantised prefill matmuls of bnskd, section 工程细节, whose
 * activation format the pages leave open).  Each row is cut into blocks of
 * 32 consecutive values; per block, in fp32:
 *   amax = max |v|;  if amax < 2^-112:  q = 0, d = 0
 *   else:  q[i] = round_half_even(v[i] * (127 / amax)) in [-127, 127],
 *          d = amax / 127      (both divisions correctly rounded)
 * so v[i] ~ q[i] * d within d / 2.
 *
 *   x  device [n_rows][n_cols], fp32 or bf16 (x_dtype)
 *   q  device int8 [n_rows][n_cols] (output)
 *   d  device fp32 [n_rows][n_cols / 32] (output)
 * Supported: n_cols a multiple of 32.  No workspace. */
int moe_quantize_q8(const void* x, int x_dtype, int n_rows, int n_cols, int8_t* q, float* d, void* stream);

/* Expert FFN and combine for a prefill chunk with int8 activations on the
 * int8 matrix cores, the pages' way of running prefill matmuls on quantised
 * operands (bnskd, section 工程细节).  Same arguments and routing inputs as
 * moe_ffn_prefill, workspace moe_workspace_size(MOE_OP_PREFILL_Q8, ...).
 *   x -> Q8 blocks (moe_quantize_q8);  for each pair (t, j) of expert e:
 *     g, u = sum over blocks b of d_x[t][b] * s[f][b] * sum_k q_x[t][k] * level[f][k]
 *     h = silu(g) * u  -> Q8 blocks (d_h, q_h)
 *     o = sum over blocks b of d_h[b] * s_down[n][b] * sum_k q_h[k] * level_down[n][k]
 *   y[t] = sum_j topk_w[t][j] * o(t, j), in ascending j
 * The block sums are exact int32 products of int8 codes and 2-bit levels;
 * scaling and the sums over blocks are fp32.  The result differs from
 * moe_ffn_prefill's by the int8 rounding of x and h (about 1e-2 of a row's
 * largest value).
 * Supported: as moe_ffn_prefill (bits == 2, d_model % 256 == 0,
 * d_ff % 128 == 0). */
int moe_ffn_prefill_q8(const moe_experts_t* experts, const void* x, int x_dtype, int n_tokens,
                       const float* topk_w, int top_k, const int32_t* bucket_offsets,
                       const int32_t* bucket_pairs, float* y, void* ws, size_t ws_bytes, void* stream);

/* Residual update and RMSNorm between chained layers:
 *   h[t] += y[t];  u[t] = h[t] / sqrt(mean(h[t]^2) + eps)
 * with the mean square in fp64 and gamma = 1.  h, y, u: device fp32
 * [n_tokens][d]; y may be NULL (norm only); u may alias nothing. */
int moe_residual_rmsnorm(float* h, const float* y, float* u, int n_tokens, int d, double eps, void* stream);

/* Bytes of workspace moe_decode_stack needs for `model` and n_tokens tokens
 * (sized for up to 1024 compute units; 0 if the arguments are invalid). */
size_t moe_stack_workspace_size(const moe_stack_t* model, int n_tokens);

/* One decode (or speculative-verify) step through every layer of a stack:
 *   h_0 = x;  for l = 0 .. L-1:
 *     u_l = h_l if l == 0, else h_l / sqrt(mean(h_l^2) + eps)   (fp64 mean)
 *     ids_l, gates_l = moe_route(layer l, u_l)
 *     h_{l+1} = h_l + moe_ffn_decode(layer l, u_l, ids_l, gates_l)   (fp32)
 *   h_out = h_L
 * Routing follows moe_route (fp64 logits, ties to the lower id; the logits
 * are summed in a different order than in moe_route, so a logit can differ
 * in its last bits) and the expert math follows moe_ffn_decode (u and the
 * SwiGLU intermediate enter the fp16 dot products as two fp16 halves each,
 * ~22 significant bits, with fp32 accumulation).  Results for a token do not
 * depend on n_tokens or on the other tokens (bitwise).
 *
 * Runs as one launch with one workgroup per compute unit that stays
 * resident for all layers; the workgroups hand logits, residual rows and
 * SwiGLU rows to each other through the workspace, tagged with per-token-
 * slot epochs kept in its header (a workspace can serve any sequence of
 * launches and batch sizes).  If a compute unit cannot hold a workgroup the
 * call fails with MOE_ERR_HIP.  The workgroups must run at the same time:
 * should other work keep compute units busy, or should a wait last longer
 * than a few seconds for any other reason, the kernel stops, the int at byte
 * offset MOE_STACK_ERROR_OFFSET of ws becomes nonzero, the outputs are
 * undefined and ws must be zero-filled again before reuse.
 *
 *   x            device [n_tokens][d_model], fp32 or bf16 (|x| < 65504)
 *   h_out        device fp32 [n_tokens][d_model] (output)
 *   topk_ids_out device int32 [L][n_tokens][top_k] or NULL (output)
 *   topk_w_out   device fp32  [L][n_tokens][top_k] or NULL (output; both or neither)
 *   h_layers_out device fp32  [L][n_tokens][d_model] or NULL (output): h_{l+1}
 *                after every layer l (its last row block equals h_out)
 *   ws           device, moe_stack_workspace_size(model, n_tokens) bytes,
 *                256-byte aligned, zero-filled before its first use
 * Supported: 1 <= n_tokens <= 8, d_model and d_ff multiples of 32,
 * d_model <= 2048, d_ff <= 4096, n_experts <= min(1024, 4 x compute units),
 * top_k <= min(n_experts, 64). */
int moe_decode_stack(const moe_stack_t* model, const void* x, int x_dtype, int n_tokens, double eps,
                     float* h_out, int32_t* topk_ids_out, float* topk_w_out, float* h_layers_out, void* ws,
                     size_t ws_bytes, void* stream);

/* Bytes of workspace moe_prefill_stack needs for `model` and chunks of at
 * most chunk_tokens tokens (0 if the arguments are invalid).  It does not
 * depend on the prompt length. */
size_t moe_prefill_stack_workspace_size(const moe_stack_t* model, int chunk_tokens);

/* Chunked prefill of a prompt through every layer of a stack, the way the
 * pages process long prompts (chunks of up to 8,192 tokens; bnskd, section
 * 工程细节).  The prompt is cut into chunks of chunk_tokens tokens (the last
 * may be shorter); each chunk runs through all layers before the next one
 * starts:
 *   h_0 = x;  for l = 0 .. L-1:
 *     u_l = h_l if l == 0, else moe_residual_rmsnorm's u of h_l
 *     ids_l, gates_l, buckets_l = moe_route(layer l, u_l)
 *     h_{l+1} = h_l + moe_ffn_prefill(layer l, u_l, gates_l, buckets_l)
 *   h_out = h_L
 * Tokens do not interact, so a token's result does not depend on the chunk
 * size; each layer matches moe_route and moe_ffn_prefill called one by one.
 * Work is enqueued on `stream` as one sequence of kernel launches per
 * (chunk, layer); nothing synchronises.
 *
 *   x     device [n_tokens][d_model], fp32 or bf16
 *   h_out device fp32 [n_tokens][d_model] (output; also the residual stream)
 *   ws    device scratch of moe_prefill_stack_workspace_size(model,
 *         chunk_tokens) bytes, 256-byte aligned; holds no state between calls
 * Supported: bits == 2, d_model a multiple of 256, d_ff a multiple of 128,
 * the moe_route limits on n_experts and top_k, chunk_tokens * top_k <= 2^28. */
int moe_prefill_stack(const moe_stack_t* model, const void* x, int x_dtype, int n_tokens, int chunk_tokens,
                      double eps, float* h_out, void* ws, size_t ws_bytes, void* stream);

/* Static English text for a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FFN_H */

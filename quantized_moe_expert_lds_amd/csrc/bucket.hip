// Bucketing of (token, slot) pairs by expert: a stable counting sort.
//
// Pair p = t*K + j goes to expert ids[p].  Output: offsets[e] = exclusive
// prefix sum of the per-expert counts (offsets[E] = T*K) and pairs[] = pair
// ids grouped by expert, ascending pair id inside each bucket.  The grouped
// GEMM of the prefill path walks these buckets.  (The pages give no bucket
// format; prefill of up to 8,192-token chunks is from bnskd "Strata：把 125B
// 大模型塞进 12GB 显卡", section 工程细节.)
//
// Everything is integer: results are exact and independent of scheduling.
//  * P <= 1024 (decode, verify): one workgroup does histogram, ranks, scan
//    and scatter in LDS.
//  * larger P: per-block LDS histograms and in-block ranks (256 pairs per
//    block) -> one workgroup turns the block histograms into per-block
//    bases (column prefix over blocks) and scans the counts -> scatter.
#include "common.hpp"

namespace {

using namespace qmoe;

// Inclusive Hillis-Steele scan of v[0..1024) in LDS by 1024 threads.
__device__ void block_scan_1024(int* v) {
    const int tid = threadIdx.x;
    for (int off = 1; off < 1024; off <<= 1) {
        const int add = tid >= off ? v[tid - off] : 0;
        __syncthreads();
        v[tid] += add;
        __syncthreads();
    }
}

__global__ __launch_bounds__(1024) void bucket_small_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ pairs) {
    __shared__ int es[1024];
    __shared__ int cnt[1024];
    const int tid = threadIdx.x;
    int e = -1;
    if (tid < P) {
        e = ids[tid];
        if (e < 0 || e >= E) e = -1;
    }
    es[tid] = e;
    cnt[tid] = 0;
    __syncthreads();
    int rank = 0;
    if (e >= 0) {
        atomicAdd(&cnt[e], 1);
        for (int i = 0; i < tid; ++i) rank += (es[i] == e);
    }
    __syncthreads();
    const int mine = cnt[tid];
    block_scan_1024(cnt);
    const int excl = cnt[tid] - mine;     // exclusive prefix of expert tid
    __syncthreads();
    es[tid] = excl;                       // reuse as offsets
    __syncthreads();
    if (tid < E) offsets[tid] = excl;
    if (tid == 0) offsets[E] = cnt[E - 1];
    if (e >= 0) pairs[es[e] + rank] = tid;
}

__global__ __launch_bounds__(kBucketBlock) void bucket_hist_kernel(const int32_t* __restrict__ ids, int P,
                                                                   int E, int* __restrict__ hist,
                                                                   int* __restrict__ rank) {
    __shared__ int es[kBucketBlock];
    __shared__ int h[kMaxExperts];
    const int tid = threadIdx.x, b = blockIdx.x;
    const int p = b * kBucketBlock + tid;
    int e = -1;
    if (p < P) {
        e = ids[p];
        if (e < 0 || e >= E) e = -1;
    }
    es[tid] = e;
    for (int i = tid; i < E; i += kBucketBlock) h[i] = 0;
    __syncthreads();
    if (e >= 0) {
        int r = 0;
        for (int i = 0; i < tid; ++i) r += (es[i] == e);
        rank[p] = r;
        atomicAdd(&h[e], 1);
    }
    __syncthreads();
    for (int i = tid; i < E; i += kBucketBlock) hist[(size_t)b * E + i] = h[i];
}

// one workgroup of 1024 threads; thread e owns expert column e and walks it
// in batches of 32 blocks whose loads are all in flight together
__global__ __launch_bounds__(1024) void bucket_scan_kernel(int* __restrict__ hist, int NB, int E, int P,
                                                           int32_t* __restrict__ offsets) {
    __shared__ int cnt[1024];
    const int tid = threadIdx.x;
    int run = 0;
    if (tid < E) {
        for (int b0 = 0; b0 < NB; b0 += 32) {
            int c[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) c[i] = b0 + i < NB ? hist[(size_t)(b0 + i) * E + tid] : 0;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if (b0 + i < NB) hist[(size_t)(b0 + i) * E + tid] = run;
                run += c[i];
            }
        }
    }
    cnt[tid] = run;
    __syncthreads();
    block_scan_1024(cnt);
    if (tid < E) offsets[tid] = cnt[tid] - run;
    if (tid == 0) offsets[E] = P;
}

__global__ __launch_bounds__(256) void bucket_scatter_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                             const int* __restrict__ hist,
                                                             const int* __restrict__ rank,
                                                             const int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ pairs) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= P) return;
    const int e = ids[p];
    if (e < 0 || e >= E) return;
    const int b = p / kBucketBlock;
    pairs[offsets[e] + hist[(size_t)b * E + e] + rank[p]] = p;
}

}  // namespace

namespace qmoe {

hipError_t launch_buckets(const int32_t* ids, int T, int K, int E, int32_t* offsets, int32_t* pairs,
                          char* ws, const RouteWs& L, hipStream_t s) {
    const int P = T * K;
    if (P <= 1024) {
        bucket_small_kernel<<<1, 1024, 0, s>>>(ids, P, E, offsets, pairs);
        return hipGetLastError();
    }
    const int NB = cdiv(P, kBucketBlock);
    int* hist = (int*)(ws + L.hist);
    int* rank = (int*)(ws + L.rank);
    bucket_hist_kernel<<<NB, kBucketBlock, 0, s>>>(ids, P, E, hist, rank);
    bucket_scan_kernel<<<1, 1024, 0, s>>>(hist, NB, E, P, offsets);
    bucket_scatter_kernel<<<cdiv(P, 256), 256, 0, s>>>(ids, P, E, hist, rank, offsets, pairs);
    return hipGetLastError();
}

}  // namespace qmoe

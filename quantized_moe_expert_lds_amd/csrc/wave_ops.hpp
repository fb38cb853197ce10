// Wavefront-level building blocks shared by the decode-step kernel and the
// small-batch router: fixed-order DPP reductions and scans, and exact top-k
// selections of fp64 logits ranked by (value descending, id ascending).
#pragma once

#include "common.hpp"

namespace {

using namespace qmoe_dev;

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

// Inclusive prefix sum over the 64 lanes (row_shr 1, 2, 4, 8 inside each
// row of 16 lanes, then row_bcast 15 and 31 carry the row totals across).
__device__ __forceinline__ int wave_scan_add(int v) {
    v += dpp0<0x111, 0xf>(v);
    v += dpp0<0x112, 0xf>(v);
    v += dpp0<0x114, 0xf>(v);
    v += dpp0<0x118, 0xf>(v);
    v += dpp0<0x142, 0xa>(v);
    v += dpp0<0x143, 0xc>(v);
    return v;
}

// Top-k of z[0..E) (E <= 64 * kPer) by one wavefront, exact, ranked by
// (z desc, id asc) and written in rank order to out_v / out_i.  With m the
// largest logit, logit v falls in bin floor((m - v) * kHistScale), or in the
// overflow bin kHistBins when it lies farther than the range.  Rounding is
// monotone, so the K-th largest value tau lies in the first bin b* whose
// cumulative count reaches K: every logit >= tau lies in a bin <= b*, every
// logit in a bin < b* is larger than tau.  The histogram is built with LDS
// adds, its prefix sum with DPP, b* with one ballot; the C logits in bins
// <= b* are compacted into LDS (ballot + mbcnt; lanes with nothing to write
// store to a discard area instead of branching) and each is ranked against
// all C by broadcast reads, issued together for up to 16 candidates.  One
// wave runs this straight-line code, so its time is the length of its
// dependency chain, LDS round trips above all (VALU-to-scalar hand-offs cost
// about as much: a ballot-count binary search over the bins measured
// slower).  Returns false, with nothing written, when fewer than K logits
// lie in range or more than 64 are candidates (clustered logits); the
// caller then takes the round-by-round selection.  LDS private to the wave:
// hist[kHistBins + 1] (128 reserved), cand_v / cand_i[128] (64 candidates,
// then the discard area).
constexpr int kHistBins = 64;
constexpr double kHistScale = 16.0;

template <int kPer>
__device__ bool wave_topk_hist(const double* z, int E, int K, double* out_v, int* out_i, int* hist,
                               double* cand_v, int* cand_i) {
    const int lane = threadIdx.x & 63;
    hist[lane] = 0;
    hist[64 + lane] = 0;
    double v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        const double x = z[min(e, E - 1)];
        v[i] = e < E ? x + 0.0 : -INFINITY;
    }
    double mx = v[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i) mx = fmax(mx, v[i]);
    const double m = wave_max_f64(mx);
    int bin[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const double dd = (m - v[i]) * kHistScale;
        bin[i] = dd < (double)kHistBins ? (int)dd : kHistBins;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < kPer; ++i) atomicAdd(&hist[bin[i]], 1);
    __builtin_amdgcn_wave_barrier();
    const int c = wave_scan_add(hist[lane]);
    const unsigned long long reach = __ballot(c >= K);
    if (!reach) return false;
    const int bstar = __ffsll((unsigned long long)reach) - 1;
    const int C = __builtin_amdgcn_readlane(c, bstar);
    if (C > 64) return false;
    int base = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const bool cnd = bin[i] <= bstar;
        const unsigned long long bal = __ballot(cnd);
        const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
        const int p = cnd ? pos : 64 + lane;
        cand_v[p] = v[i];
        cand_i[p] = lane + 64 * i;
        base += __popcll(bal);
    }
    const int C4 = (C + 3) & ~3;
    {
        const int p = lane >= C && lane < C4 ? lane : 64 + lane;   // sentinels rank after every candidate
        cand_v[p] = -INFINITY;
        cand_i[p] = 0x7fffffff;
    }
    __builtin_amdgcn_wave_barrier();
    const int me = lane < C ? lane : 0;
    const double cv = cand_v[me];
    const int ci = cand_i[me];
    auto before4 = [&](int q) {
        const double2 a = *reinterpret_cast<const double2*>(cand_v + q);
        const double2 b = *reinterpret_cast<const double2*>(cand_v + q + 2);
        const int4 ii = *reinterpret_cast<const int4*>(cand_i + q);
        return ((a.x > cv) || (a.x == cv && ii.x < ci)) + ((a.y > cv) || (a.y == cv && ii.y < ci)) +
               ((b.x > cv) || (b.x == cv && ii.z < ci)) + ((b.y > cv) || (b.y == cv && ii.w < ci));
    };
    int rank = 0;
    if (C4 <= 16) {
        // the reads of the first 16 entries are issued together; entries
        // past C4 hold stale data and are left out
        int r4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) r4[j] = before4(4 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j) rank += 4 * j < C4 ? r4[j] : 0;
    } else {
        for (int q = 0; q < C4; q += 4) rank += before4(q);
    }
    if (lane < C && rank < K) {
        out_v[rank] = cv;
        out_i[rank] = ci;
    }
    __builtin_amdgcn_wave_barrier();
    return true;
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

}  // namespace

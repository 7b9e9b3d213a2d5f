// Exact top-k selection of one wavefront over double logits (ties to the
// lower index) and the softmax over the selected values; shared by the router
// kernels and the decode gate/up kernel that selects its slot's expert itself.
#pragma once
#include <float.h>

#include "common.hpp"
#include "wave.hpp"

namespace moe {

// ---------------------------------------------------------------- top-k ----

// Iterative wave argmax: k rounds of (lane best, wave best).  Exact; used when
// the threshold filter below leaves more than 64 candidates.
template <int NPL>
__device__ void topk_iterative(double (&v)[NPL], int E, int k, int32_t* zi, double* zv) {
    const int lane = threadIdx.x & 63;
    for (int j = 0; j < k; ++j) {
        double bv = -DBL_MAX;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            const int e = lane + 64 * i;
            if (e < E && (v[i] > bv || (v[i] == bv && e < bi))) { bv = v[i]; bi = e; }
        }
        wave_argmax(bv, bi);
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (lane + 64 * i == bi) v[i] = -DBL_MAX;
        if (lane == 0) { zi[j] = bi; zv[j] = bv; }
    }
}

// LDS-only synchronisation: orders LDS accesses without waiting for global
// stores still in flight (a plain barrier would also wait for those).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}
__device__ __forceinline__ void block_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Order-preserving 64-bit key of a finite double: a larger value has a larger
// key; -0.0 is folded onto +0.0 so that equal values have equal keys.
__device__ __forceinline__ uint64_t order_key(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v + 0.0);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ __forceinline__ double key_value(uint64_t k) {
    const uint64_t b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
    return __longlong_as_double((long long)b);
}
// (k1, i1) ranks before (k2, i2): larger key, then lower index
__device__ __forceinline__ bool key_before(uint64_t k1, int i1, uint64_t k2, int i2) {
    return k1 > k2 || (k1 == k2 && i1 < i2);
}

// per-wavefront LDS scratch of the top-k
struct RankScratch {
    uint64_t k[64];
    int32_t i[64];
    double v[64];
};

// One wavefront selects the top-k of z[0..E) by (value desc, index asc) and
// forms the softmax over the selected values.  Every rank is found by counting
// (how many entries rank before this one), which needs no sorting network:
//  1. every lane's maximum over its values; tau = the k-th largest of the 16
//     maxima of four-lane groups (or, for k > 16 or E < 64, the kk-th largest
//     lane maximum).  Those maxima are distinct entries, so every value of the
//     top k ranks at or before tau;
//  2. the entries ranking at or before tau (usually 10..20) are compacted into LDS;
//  3. each candidate counts the candidates ranking before it, which is its rank;
//     lane r then holds the entry of rank r.
// More than 64 candidates (heavy ties) fall back to k rounds of wave argmax.
// topk_select leaves rank r's value and index in S.v[r], S.i[r] (r < k) and,
// if s_ids is given, the index in s_ids[r]; topk_gates then forms the softmax
// from S and writes ids and gates, so that a caller can take the selection
// alone first and the gates later.
// topk_select_regs: the same selection over values already in registers
// (entry lane + 64 i in v[i]; entries at or past E must hold -DBL_MAX).
template <int NPL>
__device__ __forceinline__ void topk_select_regs(double (&v)[NPL], int E, int k, int32_t* s_ids, RankScratch& S) {
    const int lane = threadIdx.x & 63;
    uint64_t key[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) key[i] = order_key(v[i]);
    uint64_t lk = key[0];  // lane maximum; equal keys keep the lower index
    int li = lane;
#pragma unroll
    for (int i = 1; i < NPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E && key[i] > lk) { lk = key[i]; li = e; }
    }
    if (lane >= E) { lk = 0; li = 0x40000000 + lane; }  // lanes without values rank last
    const int nlanes = E < 64 ? E : 64;
    uint64_t tk;
    int ti;
    if (k <= 16 && nlanes == 64) {
        // maxima of the 16 groups of four lanes; tau = the k-th largest of them
#pragma unroll
        for (int J = 1; J <= 2; J <<= 1) {
            const uint32_t ohi = J == 1 ? lane_xor<1>((uint32_t)(lk >> 32)) : lane_xor<2>((uint32_t)(lk >> 32));
            const uint32_t olo = J == 1 ? lane_xor<1>((uint32_t)lk) : lane_xor<2>((uint32_t)lk);
            const int oi = (int)(J == 1 ? lane_xor<1>((uint32_t)li) : lane_xor<2>((uint32_t)li));
            const uint64_t ok = ((uint64_t)ohi << 32) | olo;
            if (key_before(ok, oi, lk, li)) { lk = ok; li = oi; }
        }
        if ((lane & 3) == 0) { S.k[lane >> 2] = lk; S.i[lane >> 2] = li; }
        wave_lds_sync();
        int r = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) r += key_before(S.k[j], S.i[j], lk, li) ? 1 : 0;
        const unsigned long long tb = __ballot((lane & 3) == 0 && r == k - 1);
        const int tl = __builtin_ctzll(tb);
        tk = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(lk >> 32), tl) << 32) |
             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lk, tl);
        ti = __builtin_amdgcn_readlane(li, tl);
    } else {
        S.k[lane] = lk;
        S.i[lane] = li;
        wave_lds_sync();
        int r = 0;
#pragma unroll 8
        for (int j = 0; j < 64; ++j) r += key_before(S.k[j], S.i[j], lk, li) ? 1 : 0;
        const int kk = k < nlanes ? k : nlanes;  // with fewer lanes than k, the weakest lane maximum
        const unsigned long long tb = __ballot(r == kk - 1);
        const int tl = __builtin_ctzll(tb);
        tk = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(lk >> 32), tl) << 32) |
             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lk, tl);
        ti = __builtin_amdgcn_readlane(li, tl);
    }
    __builtin_amdgcn_wave_barrier();
    const unsigned long long lt = (1ull << lane) - 1ull;
    int base = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        const bool c = e < E && !key_before(tk, ti, key[i], e);
        const unsigned long long b = __ballot(c);
        const int pos = base + __popcll(b & lt);
        if (c && pos < 64) { S.k[pos] = key[i]; S.i[pos] = e; }
        base += __popcll(b);
    }
    wave_lds_sync();
    if (base <= 64) {
        const uint64_t ck = lane < base ? S.k[lane] : 0;
        const int ci = lane < base ? S.i[lane] : 0x40000000 + lane;
        if (lane >= base) { S.k[lane] = 0; S.i[lane] = 0x40000000 + lane; }  // rank after every candidate
        wave_lds_sync();
        int cr = 0;
        for (int j = 0; j < base; j += 4) {
#pragma unroll
            for (int q = 0; q < 4; ++q) cr += key_before(S.k[j + q], S.i[j + q], ck, ci) ? 1 : 0;
        }
        wave_lds_sync();
        if (lane < base && cr < 64) { S.v[cr] = key_value(ck); S.i[cr] = ci; }
    } else {
        topk_iterative<NPL>(v, E, k, S.i, S.v);
    }
    wave_lds_sync();
    if (s_ids && lane < k) s_ids[lane] = S.i[lane];
}

template <int NPL>
__device__ __forceinline__ void topk_select(const double* __restrict__ z, int E, int k, int32_t* s_ids,
                                            RankScratch& S, int planes = 1, size_t plane_stride = 0) {
    const int lane = threadIdx.x & 63;
    double v[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) v[i] = z[min(lane + 64 * i, E - 1)];
    // split-k logits: the partial sums of the k planes are added in plane order
    for (int p = 1; p < planes; ++p)
#pragma unroll
        for (int i = 0; i < NPL; ++i) v[i] += z[p * plane_stride + min(lane + 64 * i, E - 1)];
#pragma unroll
    for (int i = 0; i < NPL; ++i)
        if (lane + 64 * i >= E) v[i] = -DBL_MAX;
    topk_select_regs<NPL>(v, E, k, s_ids, S);
}

// softmax over the k selected values of S (rank order) and the global writes
__device__ __forceinline__ void topk_gates(const RankScratch& S, int k, int32_t* __restrict__ ids,
                                           float* __restrict__ gates) {
    const int lane = threadIdx.x & 63;
    const double sv = lane < k ? S.v[lane] : -DBL_MAX;
    const int si = lane < k ? S.i[lane] : 0;
    // lane r holds rank r: the softmax terms are summed in rank order
    const double z0 = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(sv), 0),
                                       __builtin_amdgcn_readlane(__double2loint(sv), 0));
    const double p = lane < k ? exp(sv - z0) : 0.0;
    const double ssum = wave_sum_xor_d(p);
    if (lane < k) {
        ids[lane] = si;
        gates[lane] = (float)(p / ssum);
    }
}

template <int NPL>
__device__ __forceinline__ void topk_rank(const double* __restrict__ z, int E, int k, int32_t* __restrict__ ids,
                                          float* __restrict__ gates, int32_t* s_ids, RankScratch& S, int planes = 1,
                                          size_t plane_stride = 0) {
    topk_select<NPL>(z, E, k, s_ids, S, planes, plane_stride);
    topk_gates(S, k, ids, gates);
}

// values per lane for E experts (E <= 1024)
inline int topk_npl(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16; }

}  // namespace moe

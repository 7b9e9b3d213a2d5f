// Router: logits in double (exact products of fp32/bf16 inputs, double sums),
// then one wavefront per token selects the top-k by (logit desc, index asc)
// and forms the softmax over the selected logits.  Selection on logits, not
// probabilities, follows the router description of the Strata pages ("single
// RTX 5090 runs a 125B model": a light gating network picks the top-K
// experts per token; the others do not compute).
//
// Small and moderate batches: every wavefront computes one router row against
// a group of up to 8 tokens staged in LDS; for small batches a single
// workgroup then selects the top-k of every token and, when asked, also groups
// the routing slots by expert (the moe_permute outputs), so decode routing is
// two launches.  A device-wide last-workgroup election would need an
// agent-scope release per workgroup, which on this multi-die part writes back
// the L2 each time; the kernel boundary is cheaper.
#include <float.h>

#include <algorithm>

#include "common.hpp"
#include "wave.hpp"

namespace moe {

template <typename XT>
__device__ __forceinline__ float load_xf(const XT* x, size_t i);
template <>
__device__ __forceinline__ float load_xf<float>(const float* x, size_t i) { return x[i]; }
template <>
__device__ __forceinline__ float load_xf<uint16_t>(const uint16_t* x, size_t i) { return bf16_bits_to_float(x[i]); }

// ---------------------------------------------------------------- top-k ----
constexpr int kMaxPerLane = 16;  // E <= 1024

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

// (v1, i1) ranks before (v2, i2): larger logit, then lower index
__device__ __forceinline__ bool ranks_before(double v1, int i1, double v2, int i2) {
    return v1 > v2 || (v1 == v2 && i1 < i2);
}

// One compare-exchange step of a bitonic sort across the wavefront (lane pairs
// l, l ^ J inside blocks of SIZE lanes; the last stage sorts all 64 into rank order).
template <int SIZE, int J>
__device__ __forceinline__ void bitonic_step(double& v, int& i) {
    const int lane = threadIdx.x & 63;
    const double pv = lane_xor_d<J>(v);
    const int pi = (int)lane_xor<J>((uint32_t)i);
    const bool first = (lane & J) == 0;
    const bool best_first = SIZE == 64 || (lane & SIZE) == 0;
    if ((first == best_first) == ranks_before(pv, pi, v, i)) {
        v = pv;
        i = pi;
    }
}

// Sort one (value, index) pair per lane into rank order (lane 0 = best); indices distinct.
__device__ __forceinline__ void wave_rank_sort(double& v, int& i) {
    bitonic_step<2, 1>(v, i);
    bitonic_step<4, 2>(v, i); bitonic_step<4, 1>(v, i);
    bitonic_step<8, 4>(v, i); bitonic_step<8, 2>(v, i); bitonic_step<8, 1>(v, i);
    bitonic_step<16, 8>(v, i); bitonic_step<16, 4>(v, i); bitonic_step<16, 2>(v, i); bitonic_step<16, 1>(v, i);
    bitonic_step<32, 16>(v, i); bitonic_step<32, 8>(v, i); bitonic_step<32, 4>(v, i); bitonic_step<32, 2>(v, i);
    bitonic_step<32, 1>(v, i);
    bitonic_step<64, 32>(v, i); bitonic_step<64, 16>(v, i); bitonic_step<64, 8>(v, i); bitonic_step<64, 4>(v, i);
    bitonic_step<64, 2>(v, i); bitonic_step<64, 1>(v, i);
}

// One wavefront selects the top-k of z[0..E) by (value desc, index asc).
//  1. every lane's maximum over its values; the lane maxima are sorted across
//     the wavefront and tau = the kk-th of them, so that every value of the
//     top k ranks at or before tau;
//  2. the values ranking at or before tau (usually k..2k) are compacted into LDS;
//  3. they are sorted across the wavefront; lanes 0..k-1 hold the result.
// More than 64 candidates (heavy ties) fall back to k rounds of wave argmax.
// scratch: LDS for 64 (value, index) pairs plus k selected pairs.
template <int NPL>
__device__ void topk_wave(const double* __restrict__ z, int E, int k, int32_t* __restrict__ ids,
                          float* __restrict__ gates, int32_t* s_ids, double* cv, int32_t* ci) {
    const int lane = threadIdx.x & 63;
    double v[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? z[e] : -DBL_MAX;
    }
    double lm = v[0];
    int li = lane;
#pragma unroll
    for (int i = 1; i < NPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E && v[i] > lm) { lm = v[i]; li = e; }  // strict: equal values keep the lower index
    }
    if (lane >= E) { lm = -DBL_MAX; li = 0x40000000 + lane; }  // lanes without values rank last
    wave_rank_sort(lm, li);
    const int nlanes = E < 64 ? E : 64;
    const int kk = k < nlanes ? k : nlanes;  // with fewer lanes than k, take the weakest lane maximum
    const double tau = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(lm), kk - 1),
                                        __builtin_amdgcn_readlane(__double2loint(lm), kk - 1));
    const int taui = __builtin_amdgcn_readlane(li, kk - 1);
    const unsigned long long lt = (1ull << lane) - 1ull;
    int base = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        const bool c = e < E && (e == taui || ranks_before(v[i], e, tau, taui));
        const unsigned long long b = __ballot(c);
        const int pos = base + __popcll(b & lt);
        if (c && pos < 64) { cv[pos] = v[i]; ci[pos] = e; }
        base += __popcll(b);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0);
    double sv;
    int si;
    if (base <= 64) {
        sv = lane < base ? cv[lane] : -DBL_MAX;
        si = lane < base ? ci[lane] : 0x40000000 + lane;
        wave_rank_sort(sv, si);
    } else {
        double* zv = cv + 64;  // selected values [k]
        int32_t* zi = ci + 64; // selected indices [k]
        topk_iterative<NPL>(v, E, k, zi, zv);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_s_waitcnt(0);
        sv = lane < k ? zv[lane] : -DBL_MAX;
        si = lane < k ? zi[lane] : 0;
    }
    const double z0 = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(sv), 0),
                                       __builtin_amdgcn_readlane(__double2loint(sv), 0));
    const double p = lane < k ? exp(sv - z0) : 0.0;
    const double ssum = wave_sum_xor_d(p);
    if (lane < k) {
        ids[lane] = si;
        gates[lane] = (float)(p / ssum);
        if (s_ids) s_ids[lane] = si;
    }
}

// per-wavefront LDS scratch of topk_wave: 64 + 64 candidates/selected pairs
struct TopkScratch {
    double v[128];
    int32_t i[128];
};

template <int NPL>
__device__ void topk_token(const double* z, int E, int k, int32_t* ids, float* gates, int32_t* s_ids,
                           TopkScratch& S) {
    topk_wave<NPL>(z, E, k, ids, gates, s_ids, S.v, S.i);
}

__device__ void topk_dispatch(const double* z, int E, int k, int32_t* ids, float* gates, int32_t* s_ids,
                              TopkScratch& S) {
    if (E <= 64) topk_token<1>(z, E, k, ids, gates, s_ids, S);
    else if (E <= 128) topk_token<2>(z, E, k, ids, gates, s_ids, S);
    else if (E <= 256) topk_token<4>(z, E, k, ids, gates, s_ids, S);
    else if (E <= 512) topk_token<8>(z, E, k, ids, gates, s_ids, S);
    else topk_token<16>(z, E, k, ids, gates, s_ids, S);
}

__global__ __launch_bounds__(256) void route_topk(const double* __restrict__ logits, int T, int E, int k,
                                                  int32_t* __restrict__ ids, float* __restrict__ gates) {
    __shared__ TopkScratch sc[4];
    const int wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    topk_dispatch(logits + (size_t)t * E, E, k, ids + (size_t)t * k, gates + (size_t)t * k, nullptr, sc[wave]);
}

// ------------------------------------------------- block-level permutation ----
// Stable grouping of n <= kSmallSlots slots held in LDS (s_ids) by one
// 256-thread workgroup.  Same outputs as the multi-workgroup path.
constexpr int kSmallSlots = 512;

__device__ void block_permute(const int32_t* s_ids, int n, int E, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_idx, int32_t* dest, int32_t* active, int32_t* s_cnt, int32_t* s_part,
                              int32_t* s_flag) {
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 256) s_cnt[e] = 0;
    __syncthreads();
    for (int f = tid; f < n; f += 256) {
        const int id = s_ids[f];
        if ((unsigned)id < (unsigned)E) atomicAdd(&s_cnt[id], 1);
    }
    __syncthreads();
    // exclusive scan of counts (and of active flags): 4 experts per thread, then 256 partials
    int c4[4], p = 0, fl = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid * 4 + i;
        c4[i] = e < E ? s_cnt[e] : 0;
        p += c4[i];
        fl += c4[i] > 0;
    }
    s_part[tid] = p;
    s_flag[tid] = fl;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int a = tid >= off ? s_part[tid - off] : 0;
        const int b = tid >= off ? s_flag[tid - off] : 0;
        __syncthreads();
        s_part[tid] += a;
        s_flag[tid] += b;
        __syncthreads();
    }
    int run = s_part[tid] - p, frun = s_flag[tid] - fl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid * 4 + i;
        if (e < E) {
            counts[e] = c4[i];
            offsets[e] = run;
            s_cnt[e] = run;  // becomes the running position of expert e
            if (c4[i] > 0) active[1 + frun++] = e;
            run += c4[i];
        }
    }
    if (tid == 255) {
        offsets[E] = s_part[255];
        active[0] = s_flag[255];
    }
    __syncthreads();
    // stable scatter by wavefront 0, slots in ascending order
    if (tid < 64) {
        const int lane = tid;
        int nbits = 0;
        while ((1 << nbits) < E) ++nbits;
        const unsigned long long lt = (1ull << lane) - 1ull;
        for (int f0 = 0; f0 < n; f0 += 64) {
            const int f = f0 + lane;
            const int raw = f < n ? s_ids[f] : -1;
            const bool valid = (unsigned)raw < (unsigned)E;
            const int id = valid ? raw : 0;
            unsigned long long peers = __ballot(valid);
            for (int b = 0; b < nbits; ++b) {
                const unsigned long long on = __ballot(valid && ((id >> b) & 1));
                peers &= ((id >> b) & 1) ? on : ~on;
            }
            const int rank = __popcll(peers & lt);
            const int cnt = __popcll(peers);
            const int pos = valid ? s_cnt[id] + rank : 0;
            __builtin_amdgcn_wave_barrier();
            if (valid && rank == 0) s_cnt[id] += cnt;
            __builtin_amdgcn_wave_barrier();
            if (valid) {
                sorted_idx[pos] = f;
                dest[f] = pos;
            }
        }
    }
}

// ------------------------------------------------------ row-dot logits ----
// grid = (ceil(E / 4), ceil(T / kTG)); wavefront w of workgroup (b, g) computes
// router row e = 4b + w for the kTG tokens of group g, staged in LDS as fp32.
// Wr rows are read with coalesced 16-byte loads, all issued before any math.
constexpr int kTG = 8;
template <typename XT>
__global__ __launch_bounds__(256) void route_logits_rows(const XT* __restrict__ x, int T, int d,
                                                         const float* __restrict__ Wr, const float* __restrict__ bias,
                                                         int E, double* __restrict__ logits) {
    extern __shared__ __align__(16) float xs[];  // [kTG][d]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.y * kTG;
    const int nt = min(kTG, T - t0);
    const int e = blockIdx.x * 4 + wave;
    // router row loads first (8 x 16 bytes per lane per 2048 features)
    const float4* w = reinterpret_cast<const float4*>(Wr + (size_t)(e < E ? e : 0) * d);
    const int nq = d / 4;
    // stage x (8 elements per thread-iteration, loads issued before the stores)
    const int n8 = nt * d / 8;
    for (int i0 = tid; i0 < n8; i0 += 256 * 4) {
        float v[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * 256;
            if (i < n8) {
                const size_t g = (size_t)t0 * d + (size_t)i * 8;
                if constexpr (sizeof(XT) == 4) {
                    const float4 a = reinterpret_cast<const float4*>(x + g)[0];
                    const float4 b = reinterpret_cast<const float4*>(x + g)[1];
                    v[u][0] = a.x; v[u][1] = a.y; v[u][2] = a.z; v[u][3] = a.w;
                    v[u][4] = b.x; v[u][5] = b.y; v[u][6] = b.z; v[u][7] = b.w;
                } else {
                    const uint4 r = *reinterpret_cast<const uint4*>(x + g);
                    const uint32_t wv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        v[u][2 * j] = __uint_as_float(wv[j] << 16);
                        v[u][2 * j + 1] = __uint_as_float(wv[j] & 0xFFFF0000u);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * 256;
            if (i < n8) {
                float4* dst = reinterpret_cast<float4*>(xs + (size_t)i * 8);
                dst[0] = make_float4(v[u][0], v[u][1], v[u][2], v[u][3]);
                dst[1] = make_float4(v[u][4], v[u][5], v[u][6], v[u][7]);
            }
        }
    }
    __syncthreads();
    if (e >= E) return;
    double acc[kTG];
#pragma unroll
    for (int t = 0; t < kTG; ++t) acc[t] = 0.0;
    for (int q0 = 0; q0 < nq; q0 += 64 * 8) {
        float4 wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int q = q0 + u * 64 + lane;
            wv[u] = q < nq ? w[q] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int q = q0 + u * 64 + lane;
            if (q >= nq) break;
#pragma unroll
            for (int t = 0; t < kTG; ++t) {
                if (t >= nt) break;
                const float4 xv = reinterpret_cast<const float4*>(xs + (size_t)t * d)[q];
                acc[t] = fma((double)xv.x, (double)wv[u].x, acc[t]);
                acc[t] = fma((double)xv.y, (double)wv[u].y, acc[t]);
                acc[t] = fma((double)xv.z, (double)wv[u].z, acc[t]);
                acc[t] = fma((double)xv.w, (double)wv[u].w, acc[t]);
            }
        }
    }
    const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
    for (int t = 0; t < kTG; ++t) {
        if (t >= nt) break;
        const double s = wave_sum_d(acc[t]);
        if (lane == 0) logits[(size_t)(t0 + t) * E + e] = s + b;
    }
}

// ascending bitonic sort of one 32-bit key per lane
template <int SIZE, int J>
__device__ __forceinline__ void bitonic_step_u(uint32_t& v) {
    const int lane = threadIdx.x & 63;
    const uint32_t pv = lane_xor<J>(v);
    const bool first = (lane & J) == 0;
    const bool asc = SIZE == 64 || (lane & SIZE) == 0;
    const uint32_t lo = pv < v ? pv : v, hi = pv < v ? v : pv;
    v = (first == asc) ? lo : hi;
}
__device__ __forceinline__ void wave_sort_u32(uint32_t& v) {
    bitonic_step_u<2, 1>(v);
    bitonic_step_u<4, 2>(v); bitonic_step_u<4, 1>(v);
    bitonic_step_u<8, 4>(v); bitonic_step_u<8, 2>(v); bitonic_step_u<8, 1>(v);
    bitonic_step_u<16, 8>(v); bitonic_step_u<16, 4>(v); bitonic_step_u<16, 2>(v); bitonic_step_u<16, 1>(v);
    bitonic_step_u<32, 16>(v); bitonic_step_u<32, 8>(v); bitonic_step_u<32, 4>(v); bitonic_step_u<32, 2>(v);
    bitonic_step_u<32, 1>(v);
    bitonic_step_u<64, 32>(v); bitonic_step_u<64, 16>(v); bitonic_step_u<64, 8>(v); bitonic_step_u<64, 4>(v);
    bitonic_step_u<64, 2>(v); bitonic_step_u<64, 1>(v);
}

// Stable grouping of n <= 64 slots (ids in LDS) by one 256-thread workgroup:
// wavefront 0 sorts the keys (id << 10 | slot), which yields sorted_idx, dest
// and the active list directly; then every thread counts, for its experts, the
// sorted keys below each expert's key range (offsets) and inside it (counts).
// Ids outside [0, E) are ignored.  Same outputs as block_permute.
__device__ void small_permute64(const int32_t* s_ids, int n, int E, int32_t* counts, int32_t* offsets,
                                int32_t* sorted_idx, int32_t* dest, int32_t* active, uint32_t* s_keys) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int id = lane < n ? s_ids[lane] : -1;
        const bool valid = (unsigned)id < (unsigned)E;
        uint32_t key = valid ? ((uint32_t)id << 10) | (uint32_t)lane : 0xFFFFFFFFu;
        wave_sort_u32(key);
        s_keys[lane] = key;
        const bool kv = key != 0xFFFFFFFFu;
        if (kv) {
            const int slot = (int)(key & 1023u);
            sorted_idx[lane] = slot;
            dest[slot] = lane;
        }
        const int kid = (int)(key >> 10);
        const int pid = __shfl_up(kid, 1);
        const bool first = kv && (lane == 0 || pid != kid);
        const unsigned long long fb = __ballot(first);
        if (first) active[1 + __popcll(fb & ((1ull << lane) - 1ull))] = kid;
        if (lane == 0) active[0] = __popcll(fb);
    }
    __syncthreads();
    uint32_t keys[64];
#pragma unroll
    for (int q = 0; q < 64; q += 4) {
        const uint4 kv = *reinterpret_cast<const uint4*>(&s_keys[q]);
        keys[q] = kv.x; keys[q + 1] = kv.y; keys[q + 2] = kv.z; keys[q + 3] = kv.w;
    }
    for (int e = threadIdx.x; e < E; e += 256) {
        const uint32_t lo = (uint32_t)e << 10, hi = (uint32_t)(e + 1) << 10;
        int below = 0, upto = 0;
#pragma unroll
        for (int q = 0; q < 64; ++q) {
            below += keys[q] < lo;
            upto += keys[q] < hi;
        }
        counts[e] = upto - below;
        offsets[e] = below;
        if (e == E - 1) offsets[E] = upto;
    }
}

// One workgroup: top-k of every token (T <= kSmallSlots / k) and, when asked,
// the grouping of the routing slots by expert.
__global__ __launch_bounds__(256) void route_select_small(const double* __restrict__ logits, int T, int E, int k,
                                                          int32_t* __restrict__ ids, float* __restrict__ gates,
                                                          int do_permute, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_idx,
                                                          int32_t* __restrict__ dest, int32_t* __restrict__ active) {
    __shared__ TopkScratch sc[4];
    __shared__ int32_t s_ids[kSmallSlots];
    __shared__ int32_t s_cnt[1024];
    __shared__ int32_t s_part[256], s_flag[256];
    __shared__ __align__(16) uint32_t s_keys[64];
    const int wave = threadIdx.x >> 6;
    for (int t = wave; t < T; t += 4)
        topk_dispatch(logits + (size_t)t * E, E, k, ids + (size_t)t * k, gates + (size_t)t * k, s_ids + t * k,
                      sc[wave]);
    __syncthreads();
    if (do_permute) {
        if (T * k <= 64)
            small_permute64(s_ids, T * k, E, counts, offsets, sorted_idx, dest, active, s_keys);
        else
            block_permute(s_ids, T * k, E, counts, offsets, sorted_idx, dest, active, s_cnt, s_part, s_flag);
    }
}

// General T: 64 tokens x 64 experts per workgroup, 4x4 outputs per thread,
// operands staged in LDS as double.
constexpr int RT = 64, RE = 64, RK = 16;
template <typename XT>
__global__ __launch_bounds__(256) void route_logits_tiled(const XT* __restrict__ x, int T, int d,
                                                          const float* __restrict__ Wr,
                                                          const float* __restrict__ bias, int E,
                                                          double* __restrict__ logits) {
    __shared__ double xs[RK][RT + 1];
    __shared__ double ws[RK][RE + 1];
    const int t0 = blockIdx.y * RT, e0 = blockIdx.x * RE;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    for (int k0 = 0; k0 < d; k0 += RK) {
        for (int idx = threadIdx.x; idx < RK * RT; idx += 256) {
            const int kk = idx % RK, r = idx / RK;
            const int t = t0 + r, e = e0 + r;
            xs[kk][r] = t < T ? (double)load_xf(x, (size_t)t * d + k0 + kk) : 0.0;
            ws[kk][r] = e < E ? (double)Wr[(size_t)e * d + k0 + kk] : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < RK; ++kk) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + ty * 4 + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + tx * 4 + j;
            if (e < E) logits[(size_t)t * E + e] = acc[i][j] + (bias ? (double)bias[e] : 0.0);
        }
    }
}

bool route_small_ok(int T, int d, int k) { return T <= 64 && (size_t)T * k <= kSmallSlots && (size_t)kTG * d * 4 <= 64 * 1024; }

// ------------------------------------------------ wavefront per row (T <= 8) ----
// Decode batches: grid = E wavefronts, each computes one router row against all
// T <= 8 tokens.  The lane's router values (float4 q = u * 64 + lane) and the
// matching token values are loaded straight from global memory, all before any
// arithmetic; no LDS and no barrier, so every wavefront runs on its own.
template <typename XT, int TT, int NU>
__global__ __launch_bounds__(64) void route_logits_wave(const XT* __restrict__ x, int T, int d,
                                                        const float* __restrict__ Wr,
                                                        const float* __restrict__ bias, int E,
                                                        double* __restrict__ logits) {
    const int lane = threadIdx.x;
    const int e = blockIdx.x;
    const int nq = d / 4;
    const float4* w = reinterpret_cast<const float4*>(Wr + (size_t)e * d);
    float4 wv[NU];
    float4 xv[TT][NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) wv[u] = w[min(u * 64 + lane, nq - 1)];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const int tt = min(t, T - 1);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int q = min(u * 64 + lane, nq - 1);
            if constexpr (sizeof(XT) == 4) {
                xv[t][u] = reinterpret_cast<const float4*>(x + (size_t)tt * d)[q];
            } else {
                const uint2 r = reinterpret_cast<const uint2*>(x + (size_t)tt * d)[q];
                xv[t][u] = make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u),
                                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xFFFF0000u));
            }
        }
    }
    double acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        if (u * 64 + lane >= nq) continue;
        const double w0 = wv[u].x, w1 = wv[u].y, w2 = wv[u].z, w3 = wv[u].w;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            acc[t] = fma((double)xv[t][u].x, w0, acc[t]);
            acc[t] = fma((double)xv[t][u].y, w1, acc[t]);
            acc[t] = fma((double)xv[t][u].z, w2, acc[t]);
            acc[t] = fma((double)xv[t][u].w, w3, acc[t]);
        }
    }
    const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const double sm = wave_sum_xor_d(acc[t]);
        if (lane == 0 && t < T) logits[(size_t)t * E + e] = sm + b;
    }
}

template <typename XT, int NU>
static bool launch_logits_wave(const XT* x, int T, int d, const float* Wr, const float* bias, int E, double* logits,
                               hipStream_t s) {
    if (T <= 1) route_logits_wave<XT, 1, NU><<<E, 64, 0, s>>>(x, T, d, Wr, bias, E, logits);
    else if (T <= 2) route_logits_wave<XT, 2, NU><<<E, 64, 0, s>>>(x, T, d, Wr, bias, E, logits);
    else if (T <= 4) route_logits_wave<XT, 4, NU><<<E, 64, 0, s>>>(x, T, d, Wr, bias, E, logits);
    else if (T <= 8) route_logits_wave<XT, 8, NU><<<E, 64, 0, s>>>(x, T, d, Wr, bias, E, logits);
    else return false;
    return true;
}

static int launch_logits(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E,
                         double* logits, hipStream_t s) {
    if (T <= 8 && d <= 2048) {
        // one wavefront per router row; NU float4 per lane cover d
        const int nu = (d / 4 + 63) / 64;
        bool ok;
        if (x_dtype == MOE_DT_F32)
            ok = nu <= 2 ? launch_logits_wave<float, 2>((const float*)x, T, d, Wr, bias, E, logits, s)
                         : launch_logits_wave<float, 8>((const float*)x, T, d, Wr, bias, E, logits, s);
        else
            ok = nu <= 2 ? launch_logits_wave<uint16_t, 2>((const uint16_t*)x, T, d, Wr, bias, E, logits, s)
                         : launch_logits_wave<uint16_t, 8>((const uint16_t*)x, T, d, Wr, bias, E, logits, s);
        if (ok) return check_launch();
    }
    if (T <= 256 && (size_t)kTG * d * 4 <= 64 * 1024) {
        const dim3 grid((E + 3) / 4, (T + kTG - 1) / kTG);
        const size_t lds = (size_t)std::min(T, kTG) * d * sizeof(float);
        if (x_dtype == MOE_DT_F32)
            route_logits_rows<float><<<grid, 256, lds, s>>>((const float*)x, T, d, Wr, bias, E, logits);
        else
            route_logits_rows<uint16_t><<<grid, 256, lds, s>>>((const uint16_t*)x, T, d, Wr, bias, E, logits);
    } else {
        dim3 grid((E + RE - 1) / RE, (T + RT - 1) / RT);
        if (x_dtype == MOE_DT_F32)
            route_logits_tiled<float><<<grid, 256, 0, s>>>((const float*)x, T, d, Wr, bias, E, logits);
        else
            route_logits_tiled<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)x, T, d, Wr, bias, E, logits);
    }
    return check_launch();
}

int launch_route_small(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E, int k,
                       int32_t* ids, float* gates, double* logits, bool do_permute, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_idx, int32_t* dest, int32_t* active, hipStream_t s) {
    int rc = launch_logits(x, x_dtype, T, d, Wr, bias, E, logits, s);
    if (rc) return rc;
    route_select_small<<<1, 256, 0, s>>>(logits, T, E, k, ids, gates, do_permute, counts, offsets, sorted_idx,
                                         dest, active);
    return check_launch();
}

int launch_route(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E, int k,
                 int32_t* ids, float* gates, double* logits, hipStream_t s) {
    if (T == 0) return MOE_OK;
    if (route_small_ok(T, d, k))
        return launch_route_small(x, x_dtype, T, d, Wr, bias, E, k, ids, gates, logits, false, nullptr, nullptr,
                                  nullptr, nullptr, nullptr, s);
    int rc = launch_logits(x, x_dtype, T, d, Wr, bias, E, logits, s);
    if (rc) return rc;
    route_topk<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, ids, gates);
    return check_launch();
}

}  // namespace moe

// Router: logits in double (exact products of fp32/bf16 inputs, double sums),
// then one wavefront per token selects the top-k by (logit desc, index asc)
// and forms the softmax over the selected logits.  Selection on logits, not
// probabilities, follows the router description of the Strata pages ("single
// RTX 5090 runs a 125B model": a light gating network picks the top-K
// experts per token; the others do not compute).
//
// Logits by batch size: T <= 8, one wavefront per router row against all
// tokens (route_logits_wave); 8 < T <= 256, 16 x 16 tiles on fp64 MFMA with
// the reduction split over sixteen wavefronts (route_logits_splitk); larger
// T, 64 x 128 tiles on fp64 MFMA (route_logits_mfma); route_logits_rows covers
// widths the split-k kernel is not instantiated for.  For up to 16 tokens and
// 512 slots a single workgroup then selects the top-k of every token and,
// when asked, also groups the routing slots by expert (the moe_permute
// outputs), so decode routing is two launches.  A device-wide last-workgroup
// election would need an agent-scope release per workgroup, which on this
// multi-die part writes back the L2 each time; the kernel boundary is cheaper.
#include <float.h>

#include <algorithm>

#include "common.hpp"
#include "topk.hpp"
#include "wave.hpp"

namespace moe {

template <typename XT>
__device__ __forceinline__ float load_xf(const XT* x, size_t i);
template <>
__device__ __forceinline__ float load_xf<float>(const float* x, size_t i) { return x[i]; }
template <>
__device__ __forceinline__ float load_xf<uint16_t>(const uint16_t* x, size_t i) { return bf16_bits_to_float(x[i]); }

// top-k selection (topk_rank) and its helpers: topk.hpp

template <int NPL>
__global__ __launch_bounds__(256) void route_topk(const double* __restrict__ logits, int T, int E, int k,
                                                  int32_t* __restrict__ ids, float* __restrict__ gates, int planes) {
    __shared__ RankScratch sc[4];
    const int wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    topk_rank<NPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, gates + (size_t)t * k, nullptr, sc[wave],
                   planes, (size_t)T * E);
}

// ------------------------------------------------- block-level permutation ----
// Stable grouping of n <= kSmallSlots slots held in LDS (s_ids) by one
// 256-thread workgroup.  Same outputs as the multi-workgroup path.
constexpr int kSmallSlots = 512;

// Inclusive prefix sum over the 64 lanes (Hillis-Steele with lane shifts).
__device__ __forceinline__ int wave_prefix_incl(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

// The NWR wavefronts of the workgroup each own a contiguous range of the slots
// (a multiple of 64): per-range expert histograms, one scan of the totals over
// the experts, per-range base positions, then every wavefront places its own
// slots in ascending order (ballot ranking within 64-slot chunks), so the
// grouping is stable and the ranges are placed concurrently.
template <int NWR>
__device__ void block_permute(const int32_t* s_ids, int n, int E, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_idx, int32_t* dest, int32_t* active, int32_t (*s_wc)[1024],
                              int32_t* s_part, int32_t* s_flag) {
    constexpr int NTH = 64 * NWR, EPT = 1024 / NTH;  // threads; experts per thread in the scan
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rng = ((n + NTH - 1) / NTH) * 64;  // slots per wavefront range
    const int f_lo = min(n, wave * rng), f_hi = min(n, f_lo + rng);
    for (int i = tid; i < NWR * 1024; i += NTH) (&s_wc[0][0])[i] = 0;
    __syncthreads();
    for (int f = f_lo + lane; f < f_hi; f += 64) {
        const int id = s_ids[f];
        if ((unsigned)id < (unsigned)E) atomicAdd(&s_wc[wave][id], 1);
    }
    __syncthreads();
    // totals of EPT experts per thread, exclusive scan over the experts
    // (wavefront scans, then the totals of the preceding wavefronts)
    int c4[EPT], p = 0, fl = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        int c = 0;
        if (e < E)
#pragma unroll
            for (int w = 0; w < NWR; ++w) c += s_wc[w][e];
        c4[i] = c;
        p += c4[i];
        fl += c4[i] > 0;
    }
    const int pi = wave_prefix_incl(p), fi = wave_prefix_incl(fl);
    if (lane == 63) {
        s_part[wave] = pi;
        s_flag[wave] = fi;
    }
    __syncthreads();
    int run = pi - p, frun = fi - fl;
    for (int w = 0; w < wave; ++w) {
        run += s_part[w];
        frun += s_flag[w];
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        if (e < E) {
            counts[e] = c4[i];
            offsets[e] = run;
            if (c4[i] > 0) active[1 + frun++] = e;
            // base position of expert e in each range: the slots of e in earlier ranges come first
            int b = run;
#pragma unroll
            for (int w = 0; w < NWR; ++w) {
                const int cw = s_wc[w][e];
                s_wc[w][e] = b;
                b += cw;
            }
            run += c4[i];
        }
    }
    if (tid == NTH - 1) {
        offsets[E] = run;
        active[0] = frun;
    }
    __syncthreads();
    // stable scatter: wavefront w places the slots of its range in ascending order
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const unsigned long long lt = (1ull << lane) - 1ull;
    for (int f0 = f_lo; f0 < f_hi; f0 += 64) {
        const int f = f0 + lane;
        const int raw = f < f_hi ? s_ids[f] : -1;
        const bool valid = (unsigned)raw < (unsigned)E;
        const int id = valid ? raw : 0;
        unsigned long long peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const unsigned long long on = __ballot(valid && ((id >> b) & 1));
            peers &= ((id >> b) & 1) ? on : ~on;
        }
        const int rank = __popcll(peers & lt);
        const int cnt = __popcll(peers);
        const int pos = valid ? s_wc[wave][id] + rank : 0;
        __builtin_amdgcn_wave_barrier();
        if (valid && rank == 0) s_wc[wave][id] += cnt;
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            sorted_idx[pos] = f;
            dest[f] = pos;
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

// Stable grouping of n <= 64 slots (ids in LDS) by one 256-thread workgroup:
// wavefront 0 ranks the keys (id << 10 | slot) by counting, which gives
// sorted_idx, dest and the active list; then every thread finds, for its
// experts, the bounds of each expert's key range in the sorted keys (binary
// search): offsets and counts.  Ids outside [0, E) are ignored.  Same outputs
// as block_permute.
__device__ void permute_rank64(const int32_t* s_ids, int n, int E, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_idx, int32_t* dest, int32_t* active, uint32_t* s_keys,
                               uint32_t* s_sorted) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int id = lane < n ? s_ids[lane] : -1;
        const bool valid = (unsigned)id < (unsigned)E;
        const uint32_t key = valid ? ((uint32_t)id << 10) | (uint32_t)lane : 0xFFFFFFFFu;
        s_keys[lane] = key;
        s_sorted[lane] = 0xFFFFFFFFu;
        s_sorted[64 + lane] = 0xFFFFFFFFu;
        wave_lds_sync();
        int pos = 0;  // keys of invalid slots are 0xFFFFFFFF and never count
#pragma unroll
        for (int j = 0; j < 64; j += 4) {
            const uint4 kv = *reinterpret_cast<const uint4*>(&s_keys[j]);
            pos += (kv.x < key) + (kv.y < key) + (kv.z < key) + (kv.w < key);
        }
        if (valid) {
            sorted_idx[pos] = lane;
            dest[lane] = pos;
            s_sorted[pos] = key;
        }
        wave_lds_sync();
        const uint32_t sk = s_sorted[lane];
        const bool kv = sk != 0xFFFFFFFFu;
        const int kid = (int)(sk >> 10);
        const int pid = lane > 0 ? (int)(s_sorted[lane - 1] >> 10) : -1;
        const bool first = kv && (lane == 0 || pid != kid);
        const unsigned long long fb = __ballot(first);
        if (first) active[1 + __popcll(fb & ((1ull << lane) - 1ull))] = kid;
        if (lane == 0) active[0] = __popcll(fb);
    }
    block_lds_sync();
    // lower bound of a key in the sorted keys (padded to 128 with 0xFFFFFFFF)
    auto lower_bound = [&](uint32_t key) {
        int pos = 0;
#pragma unroll
        for (int step = 64; step >= 1; step >>= 1) pos += s_sorted[pos + step - 1] < key ? step : 0;
        return pos;
    };
    for (int e = threadIdx.x; e < E; e += 256) {
        const int below = lower_bound((uint32_t)e << 10);
        const int upto = lower_bound((uint32_t)(e + 1) << 10);
        counts[e] = upto - below;
        offsets[e] = below;
        if (e == E - 1) offsets[E] = upto;
    }
}

// Permutation of up to kBlockPermMax slots by one workgroup (ids staged in
// LDS, then the block-level grouping above): one launch instead of three.
constexpr int kBlockPermMax = 4096;
constexpr int kPermBlockWaves = 8;  // wavefront ranges of perm_block (the in-selection grouping uses 4)
__global__ __launch_bounds__(64 * kPermBlockWaves) void perm_block(const int32_t* __restrict__ ids, int n, int E,
                                                                   int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ sorted_idx,
                                                                   int32_t* __restrict__ dest,
                                                                   int32_t* __restrict__ active) {
    __shared__ int32_t s_ids[kBlockPermMax];
    __shared__ int32_t s_wc[kPermBlockWaves][1024];
    __shared__ int32_t s_part[kPermBlockWaves], s_flag[kPermBlockWaves];
    for (int i = threadIdx.x; i < n; i += 64 * kPermBlockWaves) s_ids[i] = ids[i];
    __syncthreads();
    block_permute<kPermBlockWaves>(s_ids, n, E, counts, offsets, sorted_idx, dest, active, s_wc, s_part, s_flag);
}

int launch_permute_block(const int32_t* ids, int n, int E, int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                         int32_t* dest, int32_t* active, hipStream_t s) {
    if (n > kBlockPermMax) return MOE_ERR_UNSUPPORTED;
    perm_block<<<1, 64 * kPermBlockWaves, 0, s>>>(ids, n, E, counts, offsets, sorted_idx, dest, active);
    return check_launch();
}

// One workgroup: top-k of every token (T <= kSmallSlots / k) and, when asked,
// the grouping of the routing slots by expert.
template <int NPL>
__global__ __launch_bounds__(256) void route_select_small(const double* __restrict__ logits, int T, int E, int k,
                                                          int32_t* __restrict__ ids, float* __restrict__ gates,
                                                          int do_permute, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_idx,
                                                          int32_t* __restrict__ dest, int32_t* __restrict__ active,
                                                          int planes) {
    __shared__ RankScratch sc[4];
    __shared__ int32_t s_ids[kSmallSlots];
    __shared__ int32_t s_wc[4][1024];
    __shared__ int32_t s_part[4], s_flag[4];
    __shared__ __align__(16) uint32_t s_keys[64];
    __shared__ __align__(16) uint32_t s_sorted[128];
    const int wave = threadIdx.x >> 6;
    for (int t = wave; t < T; t += 4)
        topk_rank<NPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, gates + (size_t)t * k, s_ids + t * k,
                       sc[wave], planes, (size_t)T * E);
    block_lds_sync();
    if (do_permute) {
        if (T * k <= 64)
            permute_rank64(s_ids, T * k, E, counts, offsets, sorted_idx, dest, active, s_keys, s_sorted);
        else
            block_permute<4>(s_ids, T * k, E, counts, offsets, sorted_idx, dest, active, s_wc, s_part, s_flag);
    }
}

// ------------------------------------------------ large batches: fp64 MFMA ----
// Workgroup tile: 64 tokens x 128 router rows; wavefront w computes the 32 x 64
// quadrant ((w / 2) * 32, (w % 2) * 64) as 2 x 4 tiles of v_mfma_f64_16x16x4
// (lane l holds A row l % 16 and B column l % 16 at k = l / 16; accumulator
// register r of lane l is row 4 r + l / 16, column l % 16).  k advances in
// chunks of 32: the next chunk is read into registers while the current one is
// multiplied, then stored to LDS as double, k-major with padded rows, so that a
// fragment read is 16 consecutive doubles per k.  Products of fp32/bf16 inputs
// are exact in double; the sums are double.
constexpr int LT = 64, LE = 128, LK = 32, LPT = LT + 16, LPE = LE + 16;
typedef double double4v __attribute__((ext_vector_type(4)));
template <typename XT>
__global__ __launch_bounds__(256) void route_logits_mfma(const XT* __restrict__ x, int T, int d,
                                                         const float* __restrict__ Wr,
                                                         const float* __restrict__ bias, int E,
                                                         double* __restrict__ logits) {
    __shared__ double xs[LK][LPT];
    __shared__ double ws[LK][LPE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.y * LT, e0 = blockIdx.x * LE;
    const int wm = (wave >> 1) * 32, wn = (wave & 1) * 64;
    // staging: token row tid / 4 (8 consecutive k at 8 (tid % 4)); router row
    // tid / 2 (16 consecutive k at 16 (tid % 2)); rows past the end repeat the last
    const int xr = tid >> 2, xk = (tid & 3) * 8;
    const int wrow = tid >> 1, wk = (tid & 1) * 16;
    const XT* xp = x + (size_t)min(t0 + xr, T - 1) * d + xk;
    const float* wp = Wr + (size_t)min(e0 + wrow, E - 1) * d + wk;
    constexpr int XU = sizeof(XT) == 4 ? 2 : 1;
    uint4 xraw[XU];
    float4 wraw[4];
    auto load_chunk = [&](int k0) {
#pragma unroll
        for (int j = 0; j < XU; ++j) xraw[j] = reinterpret_cast<const uint4*>(xp + k0)[j];
#pragma unroll
        for (int j = 0; j < 4; ++j) wraw[j] = reinterpret_cast<const float4*>(wp + k0)[j];
    };
    auto store_chunk = [&]() {
        double xv[8];
        if constexpr (sizeof(XT) == 4) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                xv[4 * j] = __uint_as_float(xraw[j].x);
                xv[4 * j + 1] = __uint_as_float(xraw[j].y);
                xv[4 * j + 2] = __uint_as_float(xraw[j].z);
                xv[4 * j + 3] = __uint_as_float(xraw[j].w);
            }
        } else {
            const uint32_t w[4] = {xraw[0].x, xraw[0].y, xraw[0].z, xraw[0].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xv[2 * q] = __uint_as_float(w[q] << 16);
                xv[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) xs[xk + j][xr] = xv[j];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ws[wk + 4 * j][wrow] = wraw[j].x;
            ws[wk + 4 * j + 1][wrow] = wraw[j].y;
            ws[wk + 4 * j + 2][wrow] = wraw[j].z;
            ws[wk + 4 * j + 3][wrow] = wraw[j].w;
        }
    };
    double4v acc[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = double4v{0.0, 0.0, 0.0, 0.0};
    load_chunk(0);
    for (int k0 = 0; k0 < d; k0 += LK) {
        __syncthreads();  // the previous chunk's fragments have been read
        store_chunk();
        __syncthreads();
        if (k0 + LK < d) load_chunk(k0 + LK);
#pragma unroll
        for (int ks = 0; ks < LK; ks += 4) {
            const int kr = ks + (lane >> 4);
            double a[2], b[4];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) a[mt] = xs[kr][wm + 16 * mt + (lane & 15)];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) b[nt] = ws[kr][wn + 16 * nt + (lane & 15)];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
        }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int e = e0 + wn + 16 * nt + (lane & 15);
        if (e >= E) continue;
        const double be = bias ? (double)bias[e] : 0.0;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + wm + 16 * mt + 4 * r + (lane >> 4);
                if (t < T) logits[(size_t)t * E + e] = acc[mt][nt][r] + be;
            }
    }
}

// ------------------------------------------ moderate batches: split-k fp64 MFMA ----
// Workgroup = 16 tokens x 16 router rows x one of P = gridDim.z planes of k
// (d / P consecutive k each), sixteen wavefronts splitting the plane's k:
// wavefront s, lane group g = l / 16 owns the KPL = d / (64 P) consecutive k at
// plane * d / P + (4 s + g) KPL, so that at MFMA step j every lane multiplies
// its own j-th token value by its own j-th router value (A and B share the k
// assignment; every product appears once).  Operands come straight from
// global memory (no reuse across wavefronts); the sixteen partial tiles meet
// in LDS and are summed in wavefront order.  Plane p writes its partial sums
// to logits + p T E, plane 0 with the bias added; the top-k reads the planes
// back and adds them in plane order.  P > 1 only spreads small tiles grids
// over more compute units.
template <typename XT, int KPL>
__global__ __launch_bounds__(1024) void route_logits_splitk(const XT* __restrict__ x, int T, int d,
                                                            const float* __restrict__ Wr,
                                                            const float* __restrict__ bias, int E,
                                                            double* __restrict__ logits) {
    __shared__ double part[16][4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.y * 16, e0 = blockIdx.x * 16;
    const int t = min(t0 + (lane & 15), T - 1), e = min(e0 + (lane & 15), E - 1);
    const int k0 = blockIdx.z * 64 * KPL + (4 * wave + (lane >> 4)) * KPL;
    float xa[KPL], wb[KPL];
    if constexpr (sizeof(XT) == 4) {
#pragma unroll
        for (int j = 0; j < KPL; j += 4) {
            const float4 v = *reinterpret_cast<const float4*>(x + (size_t)t * d + k0 + j);
            xa[j] = v.x; xa[j + 1] = v.y; xa[j + 2] = v.z; xa[j + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < KPL; j += 4) {
            const uint2 r = *reinterpret_cast<const uint2*>(x + (size_t)t * d + k0 + j);
            xa[j] = __uint_as_float(r.x << 16); xa[j + 1] = __uint_as_float(r.x & 0xFFFF0000u);
            xa[j + 2] = __uint_as_float(r.y << 16); xa[j + 3] = __uint_as_float(r.y & 0xFFFF0000u);
        }
    }
#pragma unroll
    for (int j = 0; j < KPL; j += 4) {
        const float4 v = *reinterpret_cast<const float4*>(Wr + (size_t)e * d + k0 + j);
        wb[j] = v.x; wb[j + 1] = v.y; wb[j + 2] = v.z; wb[j + 3] = v.w;
    }
    double4v acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int j = 0; j < KPL; ++j) acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xa[j], (double)wb[j], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][r][lane] = acc[r];
    __syncthreads();
    if (threadIdx.x < 256) {
        // output (row 4 r + l / 16, column l % 16) of the tile: r = tid / 64, l = tid % 64
        const int r = threadIdx.x >> 6, l = threadIdx.x & 63;
        double sum = 0.0;
#pragma unroll
        for (int q = 0; q < 16; ++q) sum += part[q][r][l];
        const int tt = t0 + 4 * r + (l >> 4), ee = e0 + (l & 15);
        if (tt < T && ee < E)
            logits[(size_t)blockIdx.z * T * E + (size_t)tt * E + ee] =
                sum + (bias && blockIdx.z == 0 ? (double)bias[ee] : 0.0);
    }
}

// k planes of the split-k kernel: enough workgroups for every compute unit,
// at least 4 k per lane; 0 where the kernel does not apply (KPL = d / (64 P)
// must be a power of two from 4 to 64)
static int splitk_planes(int T, int d, int E) {
    const int kpl = d / 64;
    if (d % 64 || kpl < 4 || kpl > 64 || (kpl & (kpl - 1))) return 0;
    const long tiles = (long)((E + 15) / 16) * ((T + 15) / 16);
    int P = 1;
    while (P < kMaxLogitPlanes && tiles * P < 256 && kpl / (2 * P) >= 4) P *= 2;
    return P;
}

template <typename XT>
static bool launch_logits_splitk(const XT* x, int T, int d, const float* Wr, const float* bias, int E,
                                 double* logits, int P, hipStream_t s) {
    const dim3 grid((E + 15) / 16, (T + 15) / 16, P);
    switch (d / (64 * P)) {
    case 4: route_logits_splitk<XT, 4><<<grid, 1024, 0, s>>>(x, T, d, Wr, bias, E, logits); return true;
    case 8: route_logits_splitk<XT, 8><<<grid, 1024, 0, s>>>(x, T, d, Wr, bias, E, logits); return true;
    case 16: route_logits_splitk<XT, 16><<<grid, 1024, 0, s>>>(x, T, d, Wr, bias, E, logits); return true;
    case 32: route_logits_splitk<XT, 32><<<grid, 1024, 0, s>>>(x, T, d, Wr, bias, E, logits); return true;
    case 64: route_logits_splitk<XT, 64><<<grid, 1024, 0, s>>>(x, T, d, Wr, bias, E, logits); return true;
    default: return false;
    }
}

// the single-workgroup selection serialises T / 4 tokens per wavefront: beyond
// 16 tokens the separate top-k (one wavefront per token) and permutation win
bool route_small_ok(int T, int d, int k) { return T <= 16 && (size_t)T * k <= kSmallSlots && (size_t)kTG * d * 4 <= 64 * 1024; }

// ------------------------------------------------ workgroup per row (T <= 8) ----
// Decode batches: grid = E workgroups, each computes one router row against
// all T <= 8 tokens.  The row is split over NW wavefronts (NU float4 per lane
// each); a lane's router values and the matching token values are loaded
// straight from global memory, all before any arithmetic.  Each wavefront
// reduces its share in double; the NW partial sums are added in wavefront
// order (deterministic) after one barrier.
template <typename XT, int TT, int NU, int NW>
__global__ __launch_bounds__(64 * NW) void route_logits_wave(const XT* __restrict__ x, int T, int d,
                                                             const float* __restrict__ Wr,
                                                             const float* __restrict__ bias, int E,
                                                             double* __restrict__ logits) {
    __shared__ double part[NW][TT];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x;
    const int nq = d / 4;
    const int q0 = wave * NU * 64;  // this wavefront's share of the row, in float4
    const float4* w = reinterpret_cast<const float4*>(Wr + (size_t)e * d);
    float4 wv[NU];
    float4 xv[TT][NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {  // each router row is read once: non-temporal
        const float4v v = gload_nt(reinterpret_cast<const float4v*>(w) + min(q0 + u * 64 + lane, nq - 1));
        wv[u] = make_float4(v[0], v[1], v[2], v[3]);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const int tt = min(t, T - 1);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int q = min(q0 + u * 64 + lane, nq - 1);
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
        if (q0 + u * 64 + lane >= nq) continue;
        const double w0 = wv[u].x, w1 = wv[u].y, w2 = wv[u].z, w3 = wv[u].w;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            acc[t] = fma((double)xv[t][u].x, w0, acc[t]);
            acc[t] = fma((double)xv[t][u].y, w1, acc[t]);
            acc[t] = fma((double)xv[t][u].z, w2, acc[t]);
            acc[t] = fma((double)xv[t][u].w, w3, acc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const double sm = wave_sum_xor_d(acc[t]);
        if (lane == 0) part[wave][t] = sm;
    }
    if constexpr (NW > 1) __syncthreads();
    if (threadIdx.x < TT && (int)threadIdx.x < T) {
        const int t = threadIdx.x;
        double sm = part[0][t];
#pragma unroll
        for (int q = 1; q < NW; ++q) sm += part[q][t];  // wavefront order: deterministic
        logits[(size_t)t * E + e] = sm + (bias ? (double)bias[e] : 0.0);
    }
}

template <typename XT, int NU, int NW>
static bool launch_logits_wave(const XT* x, int T, int d, const float* Wr, const float* bias, int E, double* logits,
                               hipStream_t s) {
    if (T <= 1) route_logits_wave<XT, 1, NU, NW><<<E, 64 * NW, 0, s>>>(x, T, d, Wr, bias, E, logits);
    else if (T <= 2) route_logits_wave<XT, 2, NU, NW><<<E, 64 * NW, 0, s>>>(x, T, d, Wr, bias, E, logits);
    else if (T <= 4) route_logits_wave<XT, 4, NU, NW><<<E, 64 * NW, 0, s>>>(x, T, d, Wr, bias, E, logits);
    else if (T <= 8) route_logits_wave<XT, 8, NU, NW><<<E, 64 * NW, 0, s>>>(x, T, d, Wr, bias, E, logits);
    else return false;
    return true;
}

// the logits of T tokens take the split-k kernel
static bool logits_splitk(int T, int d, int E) {
    return T > 0 && !(T <= 8 && d <= 2048) && T <= 256 && splitk_planes(T, d, E) > 0;
}

int logit_planes(int T, int d, int E) { return logits_splitk(T, d, E) ? splitk_planes(T, d, E) : 1; }

static int launch_logits(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E,
                         double* logits, hipStream_t s) {
    if (T <= 8 && d <= 2048) {
        // one workgroup per router row: one wavefront for d <= 512, else four, 2 float4 per lane
        const int nu = (d / 4 + 63) / 64;
        bool ok;
        if (x_dtype == MOE_DT_F32)
            ok = nu <= 2 ? launch_logits_wave<float, 2, 1>((const float*)x, T, d, Wr, bias, E, logits, s)
                         : launch_logits_wave<float, 2, 4>((const float*)x, T, d, Wr, bias, E, logits, s);
        else
            ok = nu <= 2 ? launch_logits_wave<uint16_t, 2, 1>((const uint16_t*)x, T, d, Wr, bias, E, logits, s)
                         : launch_logits_wave<uint16_t, 2, 4>((const uint16_t*)x, T, d, Wr, bias, E, logits, s);
        if (ok) return check_launch();
    }
    if (logits_splitk(T, d, E)) {
        const int P = splitk_planes(T, d, E);
        const bool ok = x_dtype == MOE_DT_F32
                            ? launch_logits_splitk<float>((const float*)x, T, d, Wr, bias, E, logits, P, s)
                            : launch_logits_splitk<uint16_t>((const uint16_t*)x, T, d, Wr, bias, E, logits, P, s);
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
        const dim3 grid((E + LE - 1) / LE, (T + LT - 1) / LT);
        if (x_dtype == MOE_DT_F32)
            route_logits_mfma<float><<<grid, 256, 0, s>>>((const float*)x, T, d, Wr, bias, E, logits);
        else
            route_logits_mfma<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)x, T, d, Wr, bias, E, logits);
    }
    return check_launch();
}

int launch_route_logits(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E,
                        double* logits, hipStream_t s) {
    if (T == 0) return MOE_OK;
    return launch_logits(x, x_dtype, T, d, Wr, bias, E, logits, s);
}

int launch_route_small(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E, int k,
                       int32_t* ids, float* gates, double* logits, bool do_permute, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_idx, int32_t* dest, int32_t* active, hipStream_t s) {
    int rc = launch_logits(x, x_dtype, T, d, Wr, bias, E, logits, s);
    if (rc) return rc;
    const int planes = logit_planes(T, d, E);
#define MOE_SEL(NPL)                                                                                       \
    route_select_small<NPL><<<1, 256, 0, s>>>(logits, T, E, k, ids, gates, do_permute, counts, offsets, sorted_idx, \
                                              dest, active, planes)
    switch (topk_npl(E)) {
    case 1: MOE_SEL(1); break;
    case 2: MOE_SEL(2); break;
    case 4: MOE_SEL(4); break;
    case 8: MOE_SEL(8); break;
    default: MOE_SEL(16); break;
    }
#undef MOE_SEL
    return check_launch();
}

int launch_route(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E, int k,
                 int32_t* ids, float* gates, double* logits, hipStream_t s) {
    if (T == 0) return MOE_OK;
    if (route_small_ok(T, d, k))
        return launch_route_small(x, x_dtype, T, d, Wr, bias, E, k, ids, gates, logits, false, nullptr, nullptr,
                                  nullptr, nullptr, nullptr, s);
    // the workspace layout sizes the logits region for the filter's scratch too
    if (route_filter_ok(T, d, E, k, x_dtype))
        return launch_route_filtered(x, T, d, Wr, bias, E, k, ids, gates, logits, s);
    int rc = launch_logits(x, x_dtype, T, d, Wr, bias, E, logits, s);
    if (rc) return rc;
    const int planes = logit_planes(T, d, E);
    const dim3 grid((T + 3) / 4);
    switch (topk_npl(E)) {
    case 1: route_topk<1><<<grid, 256, 0, s>>>(logits, T, E, k, ids, gates, planes); break;
    case 2: route_topk<2><<<grid, 256, 0, s>>>(logits, T, E, k, ids, gates, planes); break;
    case 4: route_topk<4><<<grid, 256, 0, s>>>(logits, T, E, k, ids, gates, planes); break;
    case 8: route_topk<8><<<grid, 256, 0, s>>>(logits, T, E, k, ids, gates, planes); break;
    default: route_topk<16><<<grid, 256, 0, s>>>(logits, T, E, k, ids, gates, planes); break;
    }
    return check_launch();
}

}  // namespace moe

// Router for large batches (prefill): a certified filter on bf16 matrix cores,
// then exact fp64 logits of the few candidates.  The selected experts and the
// gates are those of the exact router (the top-k of the double logits, ties to
// the lower index, and the softmax over them); only the work differs.
//
//  1. route_filter: zf = x . (w_hi + w_lo) on v_mfma_f32_16x16x32_bf16, where
//     w_hi = bf16(w) and w_lo = bf16(w - w_hi) split each fp32 router weight
//     and the bf16 token values enter exactly, fp32 accumulation.  With
//     |w - w_hi - w_lo| <= 2^-16 |w| and the accumulation error of 2 d exact
//     products bounded by gamma(2 d) times their absolute sum, every entry
//     satisfies |zf - z| <= c ||x_t|| ||w_e|| with
//     c = 2^-16 + 4 * 1.008 * gamma(2 d), gamma(n) = n u / (1 - n u), u = 2^-24
//     (Cauchy-Schwarz bounds the absolute sum by the norms; the factor 4 is a
//     margin over round-to-nearest accumulation, whatever order the matrix
//     cores add in).  The split and ||w_e|| (the root of a double sum of
//     squares) are formed once per call by route_split; the filter stages bf16
//     tiles only.
//  2. route_refine, one wavefront per token: with lo_e = zf_e - delta_e and
//     hi_e = zf_e + delta_e (delta_e the bound above, biases added exactly),
//     L = the k-th largest lo_e is a lower bound on the k-th largest logit, so
//     every expert of the exact top k has hi_e >= L, and every expert with
//     hi_e < L ranks below it.  The candidates (hi_e >= L, usually k to k + 3)
//     get their exact double logits (exact products, double sums), are ranked
//     by (logit desc, index asc), and the softmax over the first k is formed
//     by the same code as the other routers.  A token with more than 64
//     candidates (heavy ties) is appended to an overflow list instead.
//  3. route_overflow: every listed token gets all E exact logits (in LDS) and
//     the ordinary one-wavefront selection.  It exits at once when the list
//     is empty.
#include <float.h>

#include <cmath>

#include "common.hpp"
#include "topk.hpp"
#include "wave.hpp"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int FE = 128, FKC = 64;  // filter tile: router rows x k chunk (tokens: FT, a template argument)
#ifndef MOE_FILTER_TOKENS
#define MOE_FILTER_TOKENS 64
#endif
constexpr int kFilterTokens = MOE_FILTER_TOKENS;  // token tile of the filter (64: two workgroups per CU)
constexpr int kMaxCand = 64;                  // candidates one wavefront refines
constexpr int kMaxExpertsRouter = 1024;       // router rows (the library's limit on E)

// bf16 bits of an fp32 value, rounded to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float v) {
    const uint32_t b = __float_as_uint(v);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Router split, once per call: one wavefront per router row writes
// w_hi = bf16(w) and w_lo = bf16(w - w_hi) (the difference is exact in fp32)
// as bf16 rows [E, d] and ||w_e|| (root of a double sum); the first thread also clears
// the overflow count that the refine and overflow passes read.
__global__ __launch_bounds__(256) void route_split(const float* __restrict__ Wr, int d, int E,
                                                   uint16_t* __restrict__ wh, uint16_t* __restrict__ wl,
                                                   double* __restrict__ wnorm, int32_t* __restrict__ n_overflow) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blockIdx.x == 0 && threadIdx.x == 0) *n_overflow = 0;
    if (e >= E) return;
    const float* w = Wr + (size_t)e * d;
    double s = 0.0;
    for (int k = 8 * lane; k < d; k += 512) {
        const float4 a = *reinterpret_cast<const float4*>(w + k);
        const float4 b = *reinterpret_cast<const float4*>(w + k + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t h[8], l[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            h[q] = bf16_rne(v[q]);
            l[q] = bf16_rne(v[q] - __uint_as_float(h[q] << 16));
            s = fma((double)v[q], (double)v[q], s);
        }
        *reinterpret_cast<uint4*>(wh + (size_t)e * d + k) =
            uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        *reinterpret_cast<uint4*>(wl + (size_t)e * d + k) =
            uint4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
    }
    s = wave_sum_xor_d(s);
    if (lane == 0) wnorm[e] = sqrt(s);  // once per row rather than once per (token, row) in route_refine
}

// LDS tile of FT (or FE) rows x FKC bf16: 16-byte chunk c of row r at c ^ (r & 7)
template <int FT>
struct FilterTiles {
    uint4v x[FT][FKC / 8];
    uint4v wh[FE][FKC / 8];
    uint4v wl[FE][FKC / 8];
};

// Workgroup = FT tokens x FE router rows; wavefront w computes the FT/2 x 64
// quadrant ((w / 2) * FT/2, (w % 2) * 64) as FT/32 x 4 tiles of 16 x 16 (lane l
// holds A row l % 16 / B column l % 16 at k = 8 (l / 16) .. +7 of each 32;
// accumulator register i of lane l is row 4 (l / 16) + i, column l % 16).
// The next k chunk is read into registers while the current one is
// multiplied.  Rows past T or E repeat the last row and are not written.
template <int FT>
__global__ __launch_bounds__(256) void route_filter(const uint16_t* __restrict__ x, int T, int d,
                                                    const uint16_t* __restrict__ wh,
                                                    const uint16_t* __restrict__ wl, int E,
                                                    float* __restrict__ zf) {
    constexpr int MT = FT / 32;   // 16-row tiles per wavefront along the tokens
    constexpr int XJ = FT / 32;   // 16-byte token chunks per thread and k chunk
    __shared__ FilterTiles<FT> S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.y * FT, e0 = blockIdx.x * FE;
    const int wm = (wave >> 1) * (FT / 2), wn = (wave & 1) * 64;
    // staging: chunk j of thread tid is row (tid + 256 j) / 8, 16-byte column
    // tid % 8, for the token tile and for both router tiles
    uint4v xr[XJ], hr[4], lr[4];  // native vectors: arrays of the HIP uint4 struct went to scratch
    const uint16_t* xp[XJ];
    const uint16_t* hp[4];
    const uint16_t* lp[4];
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
        const int r = (tid + 256 * j) >> 3;
        xp[j] = x + (size_t)min(t0 + r, T - 1) * d + (tid & 7) * 8;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const size_t o = (size_t)min(e0 + ((tid + 256 * j) >> 3), E - 1) * d + (tid & 7) * 8;
        hp[j] = wh + o;
        lp[j] = wl + o;
    }
    const int c8 = tid & 7;
    float4v acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < XJ; ++j) xr[j] = gload(reinterpret_cast<const uint4v*>(xp[j]));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        hr[j] = gload(reinterpret_cast<const uint4v*>(hp[j]));
        lr[j] = gload(reinterpret_cast<const uint4v*>(lp[j]));
    }
    for (int k0 = 0; k0 < d; k0 += FKC) {
        __syncthreads();  // the previous chunk's fragments have been read
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int r = (tid + 256 * j) >> 3;
            S.x[r][c8 ^ (r & 7)] = xr[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = (tid + 256 * j) >> 3;
            S.wh[r][c8 ^ (r & 7)] = hr[j];
            S.wl[r][c8 ^ (r & 7)] = lr[j];
        }
        __syncthreads();
        // the next chunk into registers (the last chunk is read again at the end)
        const int kn = min(k0 + FKC, d - FKC);
#pragma unroll
        for (int j = 0; j < XJ; ++j) xr[j] = gload(reinterpret_cast<const uint4v*>(xp[j] + kn));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            hr[j] = gload(reinterpret_cast<const uint4v*>(hp[j] + kn));
            lr[j] = gload(reinterpret_cast<const uint4v*>(lp[j] + kn));
        }
#pragma unroll
        for (int ks = 0; ks < FKC / 32; ++ks) {
            const int c = ks * 4 + (lane >> 4);
            bf16x8 a[MT], bh[4], bl[4];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int r = wm + 16 * mt + (lane & 15);
                a[mt] = __builtin_bit_cast(bf16x8, S.x[r][c ^ (r & 7)]);
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int r = wn + 16 * nt + (lane & 15);
                bh[nt] = __builtin_bit_cast(bf16x8, S.wh[r][c ^ (r & 7)]);
                bl[nt] = __builtin_bit_cast(bf16x8, S.wl[r][c ^ (r & 7)]);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], bh[nt], acc[mt][nt], 0, 0, 0);
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], bl[nt], acc[mt][nt], 0, 0, 0);
                }
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int e = e0 + wn + 16 * nt + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + wm + 16 * mt + 4 * (lane >> 4) + i;
                if (t < T && e < E) zf[(size_t)t * E + e] = acc[mt][nt][i];
            }
        }
}

// the lane's part of router row e (chunk j at k = 8 (lane + 64 j), as for the token)
template <int XPL>
__device__ __forceinline__ void load_row(const float* __restrict__ Wr, int d, int e, float4 (&wv)[XPL][2]) {
    const int lane = threadIdx.x & 63;
    const float* w = Wr + (size_t)e * d;
#pragma unroll
    for (int j = 0; j < XPL; ++j) {
        const int k = 8 * (lane + 64 * j);
        if (k < d) {
            wv[j][0] = *reinterpret_cast<const float4*>(w + k);
            wv[j][1] = *reinterpret_cast<const float4*>(w + k + 4);
        }
    }
}

// exact double logit from a loaded row: exact products, lane sums in k order,
// then the butterfly over the lanes, then the bias
template <int XPL>
__device__ __forceinline__ double row_logit(const double (&xv)[XPL][8], const float4 (&wv)[XPL][2], int d, int e,
                                            const float* __restrict__ bias) {
    const int lane = threadIdx.x & 63;
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < XPL; ++j) {
        if (8 * (lane + 64 * j) >= d) continue;
        const float wq[8] = {wv[j][0].x, wv[j][0].y, wv[j][0].z, wv[j][0].w,
                             wv[j][1].x, wv[j][1].y, wv[j][1].z, wv[j][1].w};
#pragma unroll
        for (int q = 0; q < 8; ++q) s = fma(xv[j][q], (double)wq[q], s);
    }
    s = wave_sum_xor_d(s);
    return s + (bias ? (double)bias[e] : 0.0);
}

// exact double logit of router row e for the token held by the wavefront
// (xv: the lane's XPL chunks of 8 token values, chunk j at k = 8 (lane + 64 j))
template <int XPL>
__device__ __forceinline__ double exact_logit(const double (&xv)[XPL][8], const float* __restrict__ Wr, int d, int e,
                                              const float* __restrict__ bias) {
    float4 wv[XPL][2];
    load_row<XPL>(Wr, d, e, wv);
    return row_logit<XPL>(xv, wv, d, e, bias);
}

// the wavefront's token values as double (bf16 exactly), and ||x||^2
template <int XPL>
__device__ __forceinline__ double load_token(const uint16_t* __restrict__ xt, int d, double (&xv)[XPL][8]) {
    const int lane = threadIdx.x & 63;
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < XPL; ++j) {
        const int k = 8 * (lane + 64 * j);
        uint4 r = {0, 0, 0, 0};
        if (k < d) r = *reinterpret_cast<const uint4*>(xt + k);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            xv[j][2 * q] = __uint_as_float(w[q] << 16);
            xv[j][2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) s = fma(xv[j][q], xv[j][q], s);
    }
    return wave_sum_xor_d(s);
}

// One wavefront per token (four per workgroup).  NPL router rows per lane
// (e = lane + 64 i), XPL token chunks per lane.
template <int NPL, int XPL>
__global__ __launch_bounds__(256) void route_refine(const uint16_t* __restrict__ x, int T, int d,
                                                    const float* __restrict__ Wr, const float* __restrict__ bias,
                                                    int E, int k, double cbound, const float* __restrict__ zf,
                                                    const double* __restrict__ wnorm, int32_t* __restrict__ ids,
                                                    float* __restrict__ gates, int32_t* __restrict__ n_overflow,
                                                    int32_t* __restrict__ overflow) {
    __shared__ RankScratch RS[4];
    __shared__ int32_t s_ce[4][kMaxCand];
    __shared__ double s_cz[4][kMaxCand];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;  // whole wavefronts only: no workgroup barrier below
    RankScratch& S = RS[wave];
    // ||x_t|| first; the token values are loaded again (from cache) for the
    // exact logits, so that they are not held in registers across the selection
    double xn;
    {
        double xv0[XPL][8];
        xn = sqrt(load_token<XPL>(x + (size_t)t * d, d, xv0));
    }
    double lo[NPL], hi[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            const double zb = (double)zf[(size_t)t * E + e] + (bias ? (double)bias[e] : 0.0);
            const double del = cbound * xn * wnorm[e] * (1.0 + 1e-6) + 1e-30;
            lo[i] = zb - del;
            hi[i] = zb + del;
        } else {
            lo[i] = -DBL_MAX;
            hi[i] = -DBL_MAX;
        }
    }
    // L = k-th largest lower bound, counted with multiplicity: the value of
    // rank k - 1 of the top-k selection over the lower bounds
    double L;
    {
        double tmp[NPL];
#pragma unroll
        for (int i = 0; i < NPL; ++i) tmp[i] = lo[i];
        topk_select_regs<NPL>(tmp, E, k, nullptr, S);
        L = S.v[k - 1];
        wave_lds_sync();  // S is written again by the ranking below
    }
    // candidates: hi >= L, compacted in index order
    const unsigned long long lt = (1ull << lane) - 1ull;
    int nc = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        const bool c = e < E && hi[i] >= L;
        const unsigned long long b = __ballot(c);
        const int pos = nc + __popcll(b & lt);
        if (c && pos < kMaxCand) s_ce[wave][pos] = e;
        nc += __popcll(b);
    }
    if (nc > kMaxCand) {  // heavy ties: the exact full row, in the overflow pass
        if (lane == 0) overflow[atomicAdd(n_overflow, 1)] = t;
        return;
    }
    wave_lds_sync();
    double xv[XPL][8];
    (void)load_token<XPL>(x + (size_t)t * d, d, xv);
    // exact logits of the candidates, in candidate order (one router row in
    // flight per wavefront: the pass is bound by cache bandwidth, and more
    // rows in flight cost occupancy)
    for (int c = 0; c < nc; ++c) {
        const double z = exact_logit<XPL>(xv, Wr, d, s_ce[wave][c], bias);
        if (lane == 0) s_cz[wave][c] = z;
    }
    wave_lds_sync();
    // rank among the candidates by (logit desc, index asc); rank r < k -> S
    if (lane < nc) {
        const double zi = s_cz[wave][lane];
        const int ei = s_ce[wave][lane];
        int r = 0;
        for (int j = 0; j < nc; ++j) {
            const double zj = s_cz[wave][j];
            const int ej = s_ce[wave][j];
            r += (zj > zi || (zj == zi && ej < ei)) ? 1 : 0;
        }
        if (r < k) {
            S.v[r] = zi;
            S.i[r] = ei;
        }
    }
    wave_lds_sync();
    topk_gates(S, k, ids + (size_t)t * k, gates + (size_t)t * k);
}

// Tokens on the overflow list: all E exact logits (the four wavefronts split
// the rows), then the one-wavefront selection over them.  Grid-strided over
// the list; nothing to do when it is empty.
template <int NPL, int XPL>
__global__ __launch_bounds__(256) void route_overflow(const uint16_t* __restrict__ x, int d,
                                                      const float* __restrict__ Wr, const float* __restrict__ bias,
                                                      int E, int k, const int32_t* __restrict__ n_overflow,
                                                      const int32_t* __restrict__ overflow, int32_t* __restrict__ ids,
                                                      float* __restrict__ gates) {
    __shared__ double z[kMaxExpertsRouter];
    __shared__ RankScratch S;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = *n_overflow;
    for (int i = blockIdx.x; i < n; i += gridDim.x) {
        const int t = overflow[i];
        double xv[XPL][8];
        (void)load_token<XPL>(x + (size_t)t * d, d, xv);
        for (int e = wave; e < E; e += 4) {
            const double v = exact_logit<XPL>(xv, Wr, d, e, bias);
            if (lane == 0) z[e] = v;
        }
        __syncthreads();
        if (wave == 0) {
            topk_select<NPL>(z, E, k, nullptr, S);
            topk_gates(S, k, ids + (size_t)t * k, gates + (size_t)t * k);
        }
        __syncthreads();  // z and S are reused by the next listed token
    }
}

// scratch in the workspace's logits region: filter logits [T, E] fp32,
// ||w_e|| [E] double, overflow count + list [1 + T] int32, w_hi and w_lo
// [E, d] bf16 each (256-byte aligned pieces)
static size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }
size_t route_filter_bytes(int T, int E, int d) {
    return up256((size_t)T * E * 4) + up256((size_t)E * 8) + up256(4 + (size_t)T * 4) + 2 * up256((size_t)E * d * 2);
}

bool route_filter_ok(int T, int d, int E, int k, int x_dtype) {
    return x_dtype == MOE_DT_BF16 && T > 256 && d % FKC == 0 && d <= 4096 && k <= 32 && E <= kMaxExpertsRouter;
}

int launch_route_filtered(const void* x, int T, int d, const float* Wr, const float* bias, int E, int k,
                          int32_t* ids, float* gates, void* scratch, hipStream_t s) {
    char* base = static_cast<char*>(scratch);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base + off;
        off += up256(bytes);
        return p;
    };
    float* zf = reinterpret_cast<float*>(take((size_t)T * E * 4));
    double* wn = reinterpret_cast<double*>(take((size_t)E * 8));
    int32_t* novf = reinterpret_cast<int32_t*>(take(4 + (size_t)T * 4));
    int32_t* ovf = novf + 1;
    uint16_t* wh = reinterpret_cast<uint16_t*>(take((size_t)E * d * 2));
    uint16_t* wl = reinterpret_cast<uint16_t*>(take((size_t)E * d * 2));
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    // the filter's bound constant for 2 d exact products accumulated in fp32
    const double u = std::ldexp(1.0, -24), n = 2.0 * d;
    const double gamma = n * u / (1.0 - n * u);
    const double cbound = std::ldexp(1.0, -16) + 4.0 * 1.008 * gamma;
    route_split<<<(E + 3) / 4, 256, 0, s>>>(Wr, d, E, wh, wl, wn, novf);
    int rc = check_launch();
    if (rc) return rc;
    route_filter<kFilterTokens><<<dim3((E + FE - 1) / FE, (T + kFilterTokens - 1) / kFilterTokens), 256, 0, s>>>(
        xb, T, d, wh, wl, E, zf);
    rc = check_launch();
    if (rc) return rc;
    const int npl = topk_npl(E);
    const int xpl = (d / 8 + 63) / 64;
#define MOE_RF(NPL, XPL)                                                                                        \
    do {                                                                                                        \
        route_refine<NPL, XPL><<<(T + 3) / 4, 256, 0, s>>>(xb, T, d, Wr, bias, E, k, cbound, zf, wn, ids, gates, \
                                                           novf, ovf);                                          \
        rc = check_launch();                                                                                    \
        if (rc) return rc;                                                                                      \
        route_overflow<NPL, XPL><<<256, 256, 0, s>>>(xb, d, Wr, bias, E, k, novf, ovf, ids, gates);            \
    } while (0)
#define MOE_RF_X(NPL)                  \
    if (xpl <= 4) MOE_RF(NPL, 4);      \
    else MOE_RF(NPL, 8)
    switch (npl) {
    case 1: MOE_RF_X(1); break;
    case 2: MOE_RF_X(2); break;
    case 4: MOE_RF_X(4); break;
    case 8: MOE_RF_X(8); break;
    default: MOE_RF_X(16); break;
    }
#undef MOE_RF_X
#undef MOE_RF
    return check_launch();
}

}  // namespace moe

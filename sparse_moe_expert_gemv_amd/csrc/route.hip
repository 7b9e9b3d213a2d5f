// Router: logits in double (exact products of fp32/bf16 inputs, double sums),
// then one wavefront per token selects the top-k by (logit desc, index asc)
// and forms the softmax over the selected logits.  Selection on logits, not
// probabilities, follows the router description of the Strata pages ("single
// RTX 5090 runs a 125B model": a light gating network picks the top-K
// experts per token; the others do not compute).
#include <float.h>

#include "common.hpp"

namespace moe {

template <typename XT>
__device__ __forceinline__ double load_x(const XT* x, size_t i);
template <>
__device__ __forceinline__ double load_x<float>(const float* x, size_t i) { return (double)x[i]; }
template <>
__device__ __forceinline__ double load_x<uint16_t>(const uint16_t* x, size_t i) {
    return (double)bf16_bits_to_float(x[i]);
}

// Small T: one wavefront per expert row, all T tokens; Wr is read once,
// coalesced (lane l reads features 2l + 128 i).
template <typename XT, int TMAX>
__global__ __launch_bounds__(256) void route_logits_rowdot(const XT* __restrict__ x, int T, int d,
                                                           const float* __restrict__ Wr,
                                                           const float* __restrict__ bias, int E,
                                                           double* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    double acc[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) acc[t] = 0.0;
    const float* w = Wr + (size_t)e * d;
    for (int i = 2 * lane; i < d; i += 128) {
        const float2 wv = *reinterpret_cast<const float2*>(w + i);
        const double w0 = wv.x, w1 = wv.y;
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t < T) {
                acc[t] = fma(load_x(x, (size_t)t * d + i), w0, acc[t]);
                acc[t] = fma(load_x(x, (size_t)t * d + i + 1), w1, acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        double v = acc[t];
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0 && t < T) logits[(size_t)t * E + e] = v + (bias ? (double)bias[e] : 0.0);
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
            xs[kk][r] = t < T ? load_x(x, (size_t)t * d + k0 + kk) : 0.0;
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

// One wavefront per token: iterated wave argmax over the token's E logits
// (lane l holds experts l, l+64, ...), then softmax over the k winners.
constexpr int kMaxPerLane = 16;  // E <= 1024
__global__ __launch_bounds__(256) void route_topk(const double* __restrict__ logits, int T, int E, int k,
                                                  int32_t* __restrict__ ids, float* __restrict__ gates) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const double* z = logits + (size_t)t * E;
    double v[kMaxPerLane];
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? z[e] : -DBL_MAX;
    }
    double zsel_mine = 0.0, z0 = 0.0;
    for (int j = 0; j < k; ++j) {
        // local best: highest value, lowest index on ties (slots scanned in ascending index)
        double bv = -DBL_MAX;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) {
            const int e = lane + 64 * i;
            if (e < E && (v[i] > bv || (v[i] == bv && e < bi))) { bv = v[i]; bi = e; }
        }
        for (int off = 32; off > 0; off >>= 1) {
            const double ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
        }
        if ((bi & 63) == lane) {
#pragma unroll
            for (int i = 0; i < kMaxPerLane; ++i)
                if (lane + 64 * i == bi) v[i] = -DBL_MAX;  // finite logits always beat a taken slot
        }
        if (j == 0) z0 = bv;
        if (lane == j) zsel_mine = bv;
        if (lane == 0) ids[(size_t)t * k + j] = bi;
    }
    // softmax over the selected logits, max-shifted by the first (largest)
    const double p = lane < k ? exp(zsel_mine - z0) : 0.0;
    double s = p;
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane < k) gates[(size_t)t * k + lane] = (float)(p / s);
}

int launch_route(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E, int k,
                 int32_t* ids, float* gates, double* logits, hipStream_t s) {
    if (T == 0) return MOE_OK;
    if (T <= 8) {
        dim3 grid((E + 3) / 4);
        if (x_dtype == MOE_DT_F32)
            route_logits_rowdot<float, 8><<<grid, 256, 0, s>>>((const float*)x, T, d, Wr, bias, E, logits);
        else
            route_logits_rowdot<uint16_t, 8><<<grid, 256, 0, s>>>((const uint16_t*)x, T, d, Wr, bias, E, logits);
    } else {
        dim3 grid((E + RE - 1) / RE, (T + RT - 1) / RT);
        if (x_dtype == MOE_DT_F32)
            route_logits_tiled<float><<<grid, 256, 0, s>>>((const float*)x, T, d, Wr, bias, E, logits);
        else
            route_logits_tiled<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)x, T, d, Wr, bias, E, logits);
    }
    int rc = check_launch();
    if (rc) return rc;
    route_topk<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, ids, gates);
    return check_launch();
}

}  // namespace moe

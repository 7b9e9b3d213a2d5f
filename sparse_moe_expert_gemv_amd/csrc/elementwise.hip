// Activation quantisation (int8 per 32 features), the weighted combine and
// the pre-norm of a stacked layer's input.
#include "common.hpp"
#include "wave.hpp"

namespace moe {

// One thread per (token, 32-feature block).  s = amax / 127 (IEEE fp32
// division), q = clamp(rint(x / s), -127, 127) with ties to even; s = 0 and
// q = 0 for an all-zero block.  Bit-exact by construction: max, division and
// round-to-nearest-even are exact operations on identical inputs.
template <typename XT>
__global__ __launch_bounds__(256) void quant_act(const XT* __restrict__ x, int T, int d, int8_t* __restrict__ xq,
                                                 float* __restrict__ sx) {
    const int nb = d / 32;
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (long)T * nb) return;
    const size_t base = (size_t)gid * 32;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        if constexpr (sizeof(XT) == 4) v[i] = x[base + i];
        else v[i] = bf16_bits_to_float(x[base + i]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float s = amax / 127.0f;
    sx[gid] = s;
    uint32_t packed[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int q = 0;
            if (s != 0.0f) q = (int)fminf(fmaxf(rintf(v[4 * w + j] / s), -127.0f), 127.0f);
            word |= ((uint32_t)q & 0xffu) << (8 * j);
        }
        packed[w] = word;
    }
    uint4* dst = reinterpret_cast<uint4*>(xq + base);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
}

int launch_quant_act(const void* x, int x_dtype, int T, int d, int8_t* xq, float* sx, hipStream_t s) {
    const long n = (long)T * (d / 32);
    if (n == 0) return MOE_OK;
    const int grid = (int)((n + 255) / 256);
    if (x_dtype == MOE_DT_F32) quant_act<float><<<grid, 256, 0, s>>>((const float*)x, T, d, xq, sx);
    else quant_act<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)x, T, d, xq, sx);
    return check_launch();
}

// out[t, o] = residual + y_shared + sum_j gates[t, j] * y_perm[dest[t*k + j], o]; j ascending.
// One thread per (token, 4 consecutive features); the k gathers of a chunk of
// 16 slots are all issued before they are summed, in order.
template <typename YT>
__device__ __forceinline__ float4 load_y4(const YT* y, size_t off) {
    if constexpr (sizeof(YT) == 4) {
        return *reinterpret_cast<const float4*>(y + off);
    } else {
        const uint2 raw = *reinterpret_cast<const uint2*>(y + off);
        const half2v a = __builtin_bit_cast(half2v, raw.x), b = __builtin_bit_cast(half2v, raw.y);
        return make_float4((float)a.x, (float)a.y, (float)b.x, (float)b.y);
    }
}

// fp16 rows: eight outputs per thread (16-byte loads of y_perm)
__device__ __forceinline__ void load_y8(const _Float16* y, size_t off, float4& lo, float4& hi) {
    const uint4 raw = *reinterpret_cast<const uint4*>(y + off);
    const half2v a = __builtin_bit_cast(half2v, raw.x), b = __builtin_bit_cast(half2v, raw.y);
    const half2v c = __builtin_bit_cast(half2v, raw.z), e = __builtin_bit_cast(half2v, raw.w);
    lo = make_float4((float)a.x, (float)a.y, (float)b.x, (float)b.y);
    hi = make_float4((float)c.x, (float)c.y, (float)e.x, (float)e.y);
}

__device__ __forceinline__ void fma4(float g, const float4& v, float4& acc) {
    acc.x = fmaf(g, v.x, acc.x); acc.y = fmaf(g, v.y, acc.y);
    acc.z = fmaf(g, v.z, acc.z); acc.w = fmaf(g, v.w, acc.w);
}

// One workgroup per token (its gates and row indices are uniform, read with
// scalar loads); each thread sums V consecutive outputs (V = 4, or 8 for fp16
// rows: 16-byte loads), looping when d / V exceeds the workgroup.
template <typename YT, int V>
__global__ __launch_bounds__(256) void combine(const YT* __restrict__ y, const int32_t* __restrict__ dest,
                                               const float* __restrict__ gates, const float* __restrict__ ysh,
                                               const float* residual, int T, int k, int d, float* out) {
    constexpr int NQ = V / 4;
    constexpr int U = 16;
    const int t = blockIdx.x;
    for (int o = (int)threadIdx.x * V; o < d; o += 256 * V) {
        float4 acc[NQ];
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (residual) acc[u] = *reinterpret_cast<const float4*>(residual + (size_t)t * d + o + 4 * u);
            if (ysh) {
                const float4 v = *reinterpret_cast<const float4*>(ysh + (size_t)t * d + o + 4 * u);
                acc[u].x += v.x; acc[u].y += v.y; acc[u].z += v.z; acc[u].w += v.w;
            }
        }
        for (int j0 = 0; j0 < k; j0 += U) {
            float g[U];
            float4 v[U][NQ];
#pragma unroll
            for (int j = 0; j < U; ++j) {
                if (j0 + j < k) {
                    g[j] = gates[(size_t)t * k + j0 + j];
                    const size_t off = (size_t)dest[(size_t)t * k + j0 + j] * d + o;
                    if constexpr (V == 4) v[j][0] = load_y4(y, off);
                    else load_y8(reinterpret_cast<const _Float16*>(y), off, v[j][0], v[j][NQ - 1]);
                }
            }
#pragma unroll
            for (int j = 0; j < U; ++j) {
                if (j0 + j < k) {
#pragma unroll
                    for (int u = 0; u < NQ; ++u) fma4(g[j], v[j][u], acc[u]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < NQ; ++u) *reinterpret_cast<float4*>(out + (size_t)t * d + o + 4 * u) = acc[u];
    }
}

// The same sum with every gather of a chunk requested before any is waited
// for: the slots' rows and gates are read for all U positions of the chunk (the
// index clamped to the last slot), and each row piece is a buffer load whose
// offset for a position past k lies outside the resource (it reads nothing
// and returns zero), so that the loads stay straight-line code; with the
// loads under branches the compiler waits for each before the next.  Rows
// must lie in the first 2 GiB of y (the caller checks).  Sum order as combine.
template <typename YT, int V>
__global__ __launch_bounds__(256) void combine_gather(const YT* __restrict__ y, uint32_t y_bytes,
                                                      const int32_t* __restrict__ dest,
                                                      const float* __restrict__ gates,
                                                      const float* __restrict__ ysh, const float* residual, int T,
                                                      int k, int d, float* out) {
    constexpr int NQ = V / 4;
    constexpr int U = 16;
    constexpr int PB = V * (int)sizeof(YT);  // bytes of one thread's piece of a row: 8 or 16
    const int t = blockIdx.x;
    const __amdgpu_buffer_rsrc_t yr = buf_rsrc(y, y_bytes);
    for (int o = (int)threadIdx.x * V; o < d; o += 256 * V) {
        float4 acc[NQ];
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (residual) acc[u] = *reinterpret_cast<const float4*>(residual + (size_t)t * d + o + 4 * u);
            if (ysh) {
                const float4 v = *reinterpret_cast<const float4*>(ysh + (size_t)t * d + o + 4 * u);
                acc[u].x += v.x; acc[u].y += v.y; acc[u].z += v.z; acc[u].w += v.w;
            }
        }
        for (int j0 = 0; j0 < k; j0 += U) {
            float g[U];
            int row[U];
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const int jj = min(j0 + j, k - 1);
                g[j] = gates[(size_t)t * k + jj];
                row[j] = dest[(size_t)t * k + jj];
            }
            float4 v[U][NQ];
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const uint32_t off =
                    j0 + j < k ? ((uint32_t)row[j] * (uint32_t)d + (uint32_t)o) * (uint32_t)sizeof(YT) : 0x80000000u;
                // whole-vector casts only: this compiler narrows a load whose
                // vector elements are bit-cast one by one, reading element 0 for all
                if constexpr (PB == 16) {
                    const auto raw = __builtin_amdgcn_raw_buffer_load_b128(yr, off, 0, 0);
                    if constexpr (sizeof(YT) == 4) {
                        const float4v f = __builtin_bit_cast(float4v, raw);
                        v[j][0] = make_float4(f[0], f[1], f[2], f[3]);
                    } else {
                        const half8 h = __builtin_bit_cast(half8, raw);
                        v[j][0] = make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
                        v[j][NQ - 1] = make_float4((float)h[4], (float)h[5], (float)h[6], (float)h[7]);
                    }
                } else {
                    const half4v h = __builtin_bit_cast(half4v, __builtin_amdgcn_raw_buffer_load_b64(yr, off, 0, 0));
                    v[j][0] = make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
                }
            }
#pragma unroll
            for (int j = 0; j < U; ++j) {
                if (j0 + j < k) {
#pragma unroll
                    for (int u = 0; u < NQ; ++u) fma4(g[j], v[j][u], acc[u]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < NQ; ++u) *reinterpret_cast<float4*>(out + (size_t)t * d + o + 4 * u) = acc[u];
    }
}

// out[t] = x[t] / sqrt(mean(x[t]^2) + eps): one wavefront per row, sums of
// squares and the scale in double, result rounded once to fp32.
__global__ __launch_bounds__(256) void rmsnorm(const float* __restrict__ x, int T, int d, double eps,
                                               float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float4* xr = reinterpret_cast<const float4*>(x + (size_t)t * d);
    float4* orow = reinterpret_cast<float4*>(out + (size_t)t * d);
    double ss = 0.0;
    for (int q = lane; q < d / 4; q += 64) {
        const float4 v = xr[q];
        ss = fma((double)v.x, (double)v.x, ss);
        ss = fma((double)v.y, (double)v.y, ss);
        ss = fma((double)v.z, (double)v.z, ss);
        ss = fma((double)v.w, (double)v.w, ss);
    }
    ss = wave_sum_d(ss);
    const double r = 1.0 / sqrt(ss / (double)d + eps);
    for (int q = lane; q < d / 4; q += 64) {
        const float4 v = xr[q];
        orow[q] = make_float4((float)(v.x * r), (float)(v.y * r), (float)(v.z * r), (float)(v.w * r));
    }
}

int launch_rmsnorm(const float* x, int T, int d, float eps, float* out, hipStream_t s) {
    if (T == 0) return MOE_OK;
    rmsnorm<<<(T + 3) / 4, 256, 0, s>>>(x, T, d, (double)eps, out);
    return check_launch();
}

int launch_combine(const void* y_perm, int y_dtype, const int32_t* dest, const float* gates, const float* y_shared,
                   const float* residual, int T, int k, int d, float* out, hipStream_t s) {
    const int V = (y_dtype == MOE_DT_F16 && d % 8 == 0) ? 8 : 4;
    if (T == 0) return MOE_OK;
    const int grid = T;
    // rows of y_perm addressed by dest are < T k
    const size_t y_bytes = (size_t)T * k * d * (y_dtype == MOE_DT_F32 ? 4 : 2);
    if (y_bytes < ((size_t)1 << 31)) {
        const uint32_t yb = (uint32_t)y_bytes;
        if (y_dtype == MOE_DT_F32)
            combine_gather<float, 4><<<grid, 256, 0, s>>>((const float*)y_perm, yb, dest, gates, y_shared, residual, T,
                                                          k, d, out);
        else if (V == 8)
            combine_gather<_Float16, 8><<<grid, 256, 0, s>>>((const _Float16*)y_perm, yb, dest, gates, y_shared,
                                                             residual, T, k, d, out);
        else
            combine_gather<_Float16, 4><<<grid, 256, 0, s>>>((const _Float16*)y_perm, yb, dest, gates, y_shared,
                                                             residual, T, k, d, out);
        return check_launch();
    }
    if (y_dtype == MOE_DT_F32)
        combine<float, 4><<<grid, 256, 0, s>>>((const float*)y_perm, dest, gates, y_shared, residual, T, k, d, out);
    else if (V == 8)
        combine<_Float16, 8><<<grid, 256, 0, s>>>((const _Float16*)y_perm, dest, gates, y_shared, residual, T, k, d,
                                                   out);
    else
        combine<_Float16, 4><<<grid, 256, 0, s>>>((const _Float16*)y_perm, dest, gates, y_shared, residual, T, k, d,
                                                   out);
    return check_launch();
}

}  // namespace moe

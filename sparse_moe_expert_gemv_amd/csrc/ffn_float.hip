// Grouped SwiGLU expert FFN, float-activation mode (decode / small batches).
//
// Matrix-core formulation of the bandwidth-bound expert GEMV: a wavefront owns
// a strip of 16 weight rows and multiplies it with up to 16 tokens per
// v_mfma_f32_16x16x32_f16 (A = tokens x 32 k, B = 32 k x 16 weight rows, one
// instruction per 32-wide quantisation block).  Weights are dequantised in
// registers to exact fp16 integers (int4: 0x6400|u is 1024+u, minus 1032;
// int8: 0x6400|(q+128) minus 1152), activations are fp16, each block's
// product is exact-integer-weighted and the block's fp16 scale is applied in
// fp32 (acc += s_b * D_b).  This keeps the VALU cost per weight near one
// operation so the kernel stays on the HBM roofline for 1..64 tokens.
//
// Work items are (active expert or shared expert) x (row strip), grid-strided
// over a device-side count, so no host synchronisation is needed.
#include "common.hpp"

namespace moe {

constexpr int kMT = 4;  // m-tiles (16 tokens each) per pass

__device__ __forceinline__ half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }

template <int WFMT>
__device__ __forceinline__ half8 dequant_block(const uint4v& w, int b) {
    half8 r;
    if constexpr (WFMT == MOE_WFMT_I4B32) {
        const uint32_t v = w[b];
        const half2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
        const half2v p0 = as_h2((v & 0x000F000Fu) | 0x64006400u) - off;
        const half2v p1 = as_h2(((v >> 4) & 0x000F000Fu) | 0x64006400u) - off;
        const half2v p2 = as_h2(((v >> 8) & 0x000F000Fu) | 0x64006400u) - off;
        const half2v p3 = as_h2(((v >> 12) & 0x000F000Fu) | 0x64006400u) - off;
        r = half8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    } else {
        const uint32_t v0 = w[2 * b], v1 = w[2 * b + 1];
        const half2v off = {(_Float16)1152.0f, (_Float16)1152.0f};
        const half2v p0 = as_h2((v0 & 0xFFu) | ((v0 << 8) & 0xFF0000u) | 0x64006400u) - off;
        const half2v p1 = as_h2(((v0 >> 16) & 0xFFu) | ((v0 >> 8) & 0xFF0000u) | 0x64006400u) - off;
        const half2v p2 = as_h2((v1 & 0xFFu) | ((v1 << 8) & 0xFF0000u) | 0x64006400u) - off;
        const half2v p3 = as_h2(((v1 >> 16) & 0xFFu) | ((v1 >> 8) & 0xFF0000u) | 0x64006400u) - off;
        r = half8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    }
    return r;
}

template <int WFMT>
__device__ __forceinline__ void load_scales(const uint8_t* p, float* s) {
    constexpr int NB = WFMT == MOE_WFMT_I4B32 ? 4 : 2;
    if constexpr (NB == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        s[0] = (float)as_h2(v.x).x; s[1] = (float)as_h2(v.x).y;
        s[2] = (float)as_h2(v.y).x; s[3] = (float)as_h2(v.y).y;
    } else {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
        s[0] = (float)as_h2(v).x; s[1] = (float)as_h2(v).y;
    }
}

__device__ __forceinline__ half8 load_frag(const _Float16* p) {
    return __builtin_bit_cast(half8, *reinterpret_cast<const uint4v*>(p));
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// x (f32 or bf16) -> fp16 copy used as the A operand.
template <typename XT>
__global__ __launch_bounds__(256) void to_f16(const XT* __restrict__ x, long n, _Float16* __restrict__ out) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    if constexpr (sizeof(XT) == 4) out[i] = (_Float16)x[i];
    else out[i] = (_Float16)bf16_bits_to_float(x[i]);
}

// gate/up + SwiGLU.  One workgroup (4 wavefronts) per item = 16 rows of f;
// the 4 wavefronts split the k tiles and reduce through LDS.
template <int WFMT>
__global__ __launch_bounds__(256) void ffn_float_gateup(const _Float16* __restrict__ x16, int T, int d, int f, int k,
                                                        const void* const* __restrict__ expert_ptrs,
                                                        const uint8_t* __restrict__ shared_blob,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ sorted_idx,
                                                        const int32_t* __restrict__ active, _Float16* __restrict__ h) {
    constexpr int NB = WFMT == MOE_WFMT_I4B32 ? 4 : 2;
    constexpr int STB = NB * 32;  // scale-tile bytes: 16 rows x NB fp16
    __shared__ float red[4][2][kMT][4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_strips = f / 16;
    const int n_active = active[0];
    const int n_items = (n_active + (shared_blob ? 1 : 0)) * n_strips;
    const ExpertLayout L = expert_layout(WFMT, d, f);
    const int nkt = L.g.nkt;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int a = item / n_strips, strip = item % n_strips;
        const uint8_t* blob;
        int c, p0;
        bool routed;
        if (a < n_active) {
            const int e = active[1 + a];
            blob = (const uint8_t*)expert_ptrs[e];
            c = counts[e];
            p0 = offsets[e];
            routed = true;
        } else {
            blob = shared_blob;
            c = T;
            p0 = T * k;
            routed = false;
        }
        const uint4v* gq = reinterpret_cast<const uint4v*>(blob + L.g.qoff + (size_t)strip * nkt * 1024) + lane;
        const uint4v* uq = reinterpret_cast<const uint4v*>(blob + L.u.qoff + (size_t)strip * nkt * 1024) + lane;
        const uint8_t* gs = blob + L.g.soff + (size_t)strip * nkt * STB + (lane & 15) * NB * 2;
        const uint8_t* us = blob + L.u.soff + (size_t)strip * nkt * STB + (lane & 15) * NB * 2;
        for (int m0 = 0; m0 < c; m0 += 16 * kMT) {
            const _Float16* xrow[kMT];
            bool ok[kMT];
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) {
                const int m = m0 + mt * 16 + (lane & 15);
                ok[mt] = m < c;
                const int t = ok[mt] ? (routed ? sorted_idx[p0 + m] / k : m) : 0;
                xrow[mt] = x16 + (size_t)t * d + 8 * (lane >> 4);
            }
            float4v accg[kMT], accu[kMT];
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) { accg[mt] = float4v{0, 0, 0, 0}; accu[mt] = float4v{0, 0, 0, 0}; }
            for (int kt = wave; kt < nkt; kt += 4) {
                const uint4v wg = gq[(size_t)kt * 64];
                const uint4v wu = uq[(size_t)kt * 64];
                float sg[NB], su[NB];
                load_scales<WFMT>(gs + (size_t)kt * STB, sg);
                load_scales<WFMT>(us + (size_t)kt * STB, su);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const half8 Bg = dequant_block<WFMT>(wg, b);
                    const half8 Bu = dequant_block<WFMT>(wu, b);
                    const int kk = (kt * NB + b) * 32;
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt) {
                        if (m0 + mt * 16 >= c) break;
                        const half8 A = ok[mt] ? load_frag(xrow[mt] + kk) : half8{};
                        const float4v dg = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bg, float4v{0, 0, 0, 0}, 0, 0, 0);
                        const float4v du = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bu, float4v{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            accg[mt][r] = fmaf(sg[b], dg[r], accg[mt][r]);
                            accu[mt][r] = fmaf(su[b], du[r], accu[mt][r]);
                        }
                    }
                }
            }
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    red[wave][0][mt][r][lane] = accg[mt][r];
                    red[wave][1][mt][r][lane] = accu[mt][r];
                }
            __syncthreads();
            {
                const int mt = wave;  // wavefront w finalises m-tile w
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + mt * 16 + 4 * (lane >> 4) + r;
                    if (m < c) {
                        const float g = red[0][0][mt][r][lane] + red[1][0][mt][r][lane] + red[2][0][mt][r][lane] +
                                        red[3][0][mt][r][lane];
                        const float u = red[0][1][mt][r][lane] + red[1][1][mt][r][lane] + red[2][1][mt][r][lane] +
                                        red[3][1][mt][r][lane];
                        const int n = strip * 16 + (lane & 15);
                        h[(size_t)(p0 + m) * f + n] = (_Float16)(silu_f(g) * u);
                    }
                }
            }
            __syncthreads();
        }
    }
}

// down projection.  One wavefront per 16 output rows; 4 strips per workgroup.
template <int WFMT, typename YT>
__global__ __launch_bounds__(256) void ffn_float_down(const _Float16* __restrict__ h, int T, int d, int f, int k,
                                                      const void* const* __restrict__ expert_ptrs,
                                                      const uint8_t* __restrict__ shared_blob,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ active, YT* __restrict__ y_perm,
                                                      float* __restrict__ y_shared) {
    constexpr int NB = WFMT == MOE_WFMT_I4B32 ? 4 : 2;
    constexpr int STB = NB * 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_groups = d / 64;
    const int n_active = active[0];
    const int n_items = (n_active + (shared_blob ? 1 : 0)) * n_groups;
    const ExpertLayout L = expert_layout(WFMT, d, f);
    const int nkt = L.dn.nkt;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int a = item / n_groups, strip = (item % n_groups) * 4 + wave;
        const uint8_t* blob;
        int c, p0;
        bool routed;
        if (a < n_active) {
            const int e = active[1 + a];
            blob = (const uint8_t*)expert_ptrs[e];
            c = counts[e];
            p0 = offsets[e];
            routed = true;
        } else {
            blob = shared_blob;
            c = T;
            p0 = T * k;
            routed = false;
        }
        const uint4v* dq = reinterpret_cast<const uint4v*>(blob + L.dn.qoff + (size_t)strip * nkt * 1024) + lane;
        const uint8_t* ds = blob + L.dn.soff + (size_t)strip * nkt * STB + (lane & 15) * NB * 2;
        for (int m0 = 0; m0 < c; m0 += 16 * kMT) {
            const _Float16* hrow[kMT];
            bool ok[kMT];
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) {
                const int m = m0 + mt * 16 + (lane & 15);
                ok[mt] = m < c;
                hrow[mt] = h + (size_t)(p0 + (ok[mt] ? m : 0)) * f + 8 * (lane >> 4);
            }
            float4v acc[kMT];
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) acc[mt] = float4v{0, 0, 0, 0};
            for (int kt = 0; kt < nkt; ++kt) {
                const uint4v wq = dq[(size_t)kt * 64];
                float s[NB];
                load_scales<WFMT>(ds + (size_t)kt * STB, s);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const half8 B = dequant_block<WFMT>(wq, b);
                    const int kk = (kt * NB + b) * 32;
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt) {
                        if (m0 + mt * 16 >= c) break;
                        const half8 A = ok[mt] ? load_frag(hrow[mt] + kk) : half8{};
                        const float4v dv = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, float4v{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[mt][r] = fmaf(s[b], dv[r], acc[mt][r]);
                    }
                }
            }
            const int o = strip * 16 + (lane & 15);
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + mt * 16 + 4 * (lane >> 4) + r;
                    if (m >= c) continue;
                    if (routed) y_perm[(size_t)(p0 + m) * d + o] = (YT)acc[mt][r];
                    else y_shared[(size_t)m * d + o] = acc[mt][r];
                }
        }
    }
}

template <int WFMT>
static int run_float(const moe_ffn_args* a, const Workspace& w, hipStream_t s) {
    const long n = (long)a->T * a->d;
    _Float16* x16 = w.x16;
    const int cgrid = (int)((n + 255) / 256);
    if (a->x_dtype == MOE_DT_F32) to_f16<float><<<cgrid, 256, 0, s>>>((const float*)a->x, n, x16);
    else to_f16<uint16_t><<<cgrid, 256, 0, s>>>((const uint16_t*)a->x, n, x16);
    int rc = check_launch();
    if (rc) return rc;
    const int max_active = a->E < a->T * a->k ? a->E : a->T * a->k;
    const int slots = max_active + (a->shared_blob ? 1 : 0);
    const int g1 = (int)std::min<long>((long)slots * (a->f / 16), 8192);
    _Float16* h = reinterpret_cast<_Float16*>(w.h);
    ffn_float_gateup<WFMT><<<g1, 256, 0, s>>>(x16, a->T, a->d, a->f, a->k, a->expert_ptrs,
                                              (const uint8_t*)a->shared_blob, a->counts, a->offsets, a->sorted_idx,
                                              a->active, h);
    rc = check_launch();
    if (rc) return rc;
    const int g2 = (int)std::min<long>((long)slots * (a->d / 64), 8192);
    if (a->y_dtype == MOE_DT_F32)
        ffn_float_down<WFMT, float><<<g2, 256, 0, s>>>(h, a->T, a->d, a->f, a->k, a->expert_ptrs,
                                                       (const uint8_t*)a->shared_blob, a->counts, a->offsets,
                                                       a->active, (float*)a->y_perm, a->y_shared);
    else
        ffn_float_down<WFMT, _Float16><<<g2, 256, 0, s>>>(h, a->T, a->d, a->f, a->k, a->expert_ptrs,
                                                          (const uint8_t*)a->shared_blob, a->counts, a->offsets,
                                                          a->active, (_Float16*)a->y_perm, a->y_shared);
    return check_launch();
}

int launch_ffn_float(const moe_ffn_args* a, const Workspace& w, hipStream_t s) {
    return a->wfmt == MOE_WFMT_I4B32 ? run_float<MOE_WFMT_I4B32>(a, w, s) : run_float<MOE_WFMT_I8B32>(a, w, s);
}

}  // namespace moe

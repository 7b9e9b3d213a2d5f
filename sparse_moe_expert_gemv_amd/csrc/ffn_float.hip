// Grouped SwiGLU expert FFN, float-activation mode (decode / small batches).
//
// Matrix-core formulation of the bandwidth-bound expert GEMV: a wavefront owns
// a strip of 16 weight rows and multiplies it with up to 16 tokens per
// v_mfma_f32_16x16x32_f16 (A = 16 tokens x 32 k, B = 32 k x 16 weight rows,
// one instruction per 32-wide quantisation block).  Weights become exact fp16
// integers in registers (int4: 0x6400|u is 1024+u; int8: 0x6400|(q+128) is
// 1024+q+128); activations are rounded to fp16 once, when a workgroup stages
// them in LDS.  Three kernel families, chosen per call by run_float:
//
//  * T <= 16, int4 (decode): ffn_gateup_tok16 / ffn_down_tok16.  Every token
//    is a row of A, so a work item (slot, 16-row strip) needs no gather.
//    Gate/up feeds the raw quants to the MFMA and cancels their offsets with
//    a seed MFMA, then scales each exact block sum in fp32; down builds
//    (q - 8) * s in fp16 before its MFMA.
//  * T <= 64 (moderate batches, either weight format): ffn_gateup_tok64 /
//    ffn_down_tok64, the same token-dense idea with four 16-token m-tiles.
//  * otherwise: ffn_float_gateup / ffn_float_down, which gather each slot's
//    rows 16 at a time; the four wavefronts of a gate/up workgroup split the
//    reduction and meet in LDS (fixed order, deterministic); the down kernel
//    keeps a strip's whole reduction in registers.  Both scale each block's
//    exact-integer-weighted product in fp32 (acc += s_b * D_b).
//
// Items are derived from device-side counts and the active-expert list: no
// host synchronisation.
#include "common.hpp"
#include "topk.hpp"

namespace moe {

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

// fp16 scale of block b of a packed tile, from its raw 32-bit words
template <int WFMT>
__device__ __forceinline__ float scale_of(const uint2& raw, int b) {
    if constexpr (WFMT == MOE_WFMT_I4B32) {
        const uint32_t w = b < 2 ? raw.x : raw.y;
        return (float)((b & 1) ? as_h2(w).y : as_h2(w).x);
    } else {
        return (float)((b & 1) ? as_h2(raw.x).y : as_h2(raw.x).x);
    }
}

template <int WFMT>
__device__ __forceinline__ uint2 load_scale_raw(const uint8_t* p) {
    if constexpr (WFMT == MOE_WFMT_I4B32) {
        const uint2v v = gload_nt(reinterpret_cast<const uint2v*>(p));
        return make_uint2(v[0], v[1]);
    } else {
        return make_uint2(gload_nt(reinterpret_cast<const uint32_t*>(p)), 0u);
    }
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

constexpr int kChunkK = 512;       // k held in registers per wavefront and matrix (4 int4 / 8 int8 tiles)

struct SlotInfo {
    const uint8_t* blob;
    int c, p0;
    bool routed;
};

__device__ __forceinline__ SlotInfo slot_info(int a, int n_active, const int32_t* active,
                                              const void* const* expert_ptrs, const uint8_t* shared_blob,
                                              const int32_t* counts, const int32_t* offsets, int T, int k) {
    SlotInfo s;
    if (a < n_active) {
        const int e = active[1 + a];
        s.blob = (const uint8_t*)expert_ptrs[e];
        s.c = counts[e];
        s.p0 = offsets[e];
        s.routed = true;
    } else {
        s.blob = shared_blob;
        s.c = T;
        s.p0 = T * k;
        s.routed = false;
    }
    return s;
}

// 8 consecutive activations as fp16 (x is fp32 or bf16; 16-byte aligned runs)
template <typename XT>
__device__ __forceinline__ half8 load8_h(const XT* p) {
    half8 v;
    if constexpr (sizeof(XT) == 4) {
        const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
        v = half8{(_Float16)a.x, (_Float16)a.y, (_Float16)a.z, (_Float16)a.w,
                  (_Float16)b.x, (_Float16)b.y, (_Float16)b.z, (_Float16)b.w};
    } else {
        const uint4 r = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = (_Float16)__uint_as_float(w[j] << 16);
            v[2 * j + 1] = (_Float16)__uint_as_float(w[j] & 0xFFFF0000u);
        }
    }
    return v;
}

// Registers of one wavefront's weight chunk: NT packed tiles of two matrices.
template <int NT>
struct WChunk {
    uint4v q0[NT], q1[NT];
    uint2 s0[NT], s1[NT];
};

template <int WFMT, int NT>
__device__ __forceinline__ void load_chunk(WChunk<NT>& w, const uint8_t* blob, const MatLayout& M0,
                                           const MatLayout& M1, bool two, size_t tile0, int t_lo, int nt, int lane) {
    constexpr int STB = (WFMT == MOE_WFMT_I4B32 ? 4 : 2) * 32;
    constexpr int NB = STB / 32;
    const uint4v* q0 = reinterpret_cast<const uint4v*>(blob + M0.qoff + tile0 * 1024) + lane;
    const uint4v* q1 = reinterpret_cast<const uint4v*>(blob + M1.qoff + tile0 * 1024) + lane;
    const uint8_t* s0 = blob + M0.soff + tile0 * STB + (lane & 15) * NB * 2;
    const uint8_t* s1 = blob + M1.soff + tile0 * STB + (lane & 15) * NB * 2;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        if (i < nt) {
            w.q0[i] = gload_nt(q0 + (size_t)(t_lo + i) * 64);
            w.s0[i] = load_scale_raw<WFMT>(s0 + (size_t)(t_lo + i) * STB);
            if (two) {
                w.q1[i] = gload_nt(q1 + (size_t)(t_lo + i) * 64);
                w.s1[i] = load_scale_raw<WFMT>(s1 + (size_t)(t_lo + i) * STB);
            }
        }
    }
}

// products of one gate/up weight chunk with the staged 16-token tile
template <int WFMT, int NT>
__device__ __forceinline__ void gu_chunk(const WChunk<NT>& w, int c0, int nt, const uint4* xs4, int XC, bool ok,
                                         int lane, float4v& accg, float4v& accu) {
    constexpr int NB = WFMT == MOE_WFMT_I4B32 ? 4 : 2;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        if (i >= nt) break;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const half8 Bg = dequant_block<WFMT>(w.q0[i], b);
            const half8 Bu = dequant_block<WFMT>(w.q1[i], b);
            const int kk = ((c0 + i) * NB + b) * 32 + 8 * (lane >> 4);
            const int rr = lane & 15;
            const half8 A = ok ? __builtin_bit_cast(half8, xs4[rr * XC + ((kk >> 3) ^ rr)]) : half8{};
            const float4v dg = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bg, float4v{0, 0, 0, 0}, 0, 0, 0);
            const float4v du = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bu, float4v{0, 0, 0, 0}, 0, 0, 0);
            const float sg = scale_of<WFMT>(w.s0[i], b), su = scale_of<WFMT>(w.s1[i], b);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                accg[r] = fmaf(sg, dg[r], accg[r]);
                accu[r] = fmaf(su, du[r], accu[r]);
            }
        }
    }
}

// products of one down weight chunk with the staged 16-row h tile
template <int WFMT, int NT>
__device__ __forceinline__ void dn_chunk(const WChunk<NT>& w, int c0, int nt, const uint4* hs4, int HC, bool ok,
                                         int lane, float4v& acc) {
    constexpr int NB = WFMT == MOE_WFMT_I4B32 ? 4 : 2;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        if (i >= nt) break;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const half8 Bw = dequant_block<WFMT>(w.q0[i], b);
            const int kk = ((c0 + i) * NB + b) * 32 + 8 * (lane >> 4);
            const int rr = lane & 15;
            const half8 A = ok ? __builtin_bit_cast(half8, hs4[rr * HC + ((kk >> 3) ^ rr)]) : half8{};
            const float4v dv = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bw, float4v{0, 0, 0, 0}, 0, 0, 0);
            const float sc = scale_of<WFMT>(w.s0[i], b);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = fmaf(sc, dv[r], acc[r]);
        }
    }
}

// gate/up + SwiGLU.  Workgroup = (slot, 16 rows of f); wavefront w covers the
// w-th quarter of the packed k tiles; activations of the current 16-token
// tile are staged once in LDS as fp16; the four partial sums meet in LDS and
// h = silu(g) * u is written as fp16.
template <int WFMT, typename XT>
__global__ __launch_bounds__(256) void ffn_float_gateup(const XT* __restrict__ x, int T, int d, int f, int k,
                                                        const void* const* __restrict__ expert_ptrs,
                                                        const uint8_t* __restrict__ shared_blob,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ sorted_idx,
                                                        const int32_t* __restrict__ active, _Float16* __restrict__ h) {
    constexpr int KPT = WFMT == MOE_WFMT_I4B32 ? 128 : 64;
    constexpr int kMaxT = kChunkK / KPT;
    // LDS: 16 activation rows of d fp16, 16-byte chunk c of row r stored at
    // chunk (c ^ r) so the 16 rows read by one MFMA operand hit distinct banks;
    // after the products, the same space holds the split-k partial sums.
    extern __shared__ __align__(16) uint4 xs4[];  // [16][d / 8]
    float(*red)[2][4][64] = reinterpret_cast<float(*)[2][4][64]>(xs4);  // [4][2][4][64]
    const int XC = d / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_strips = f / 16;
    const int nkt = d / KPT;
    const int kt_lo = (wave * nkt) / 4, kt_hi = ((wave + 1) * nkt) / 4;
    const int n_active = active[0];
    const int n_items = (n_active + (shared_blob ? 1 : 0)) * n_strips;
    const ExpertLayout L = expert_layout(WFMT, d, f);
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int strip = item % n_strips;
        const SlotInfo S = slot_info(item / n_strips, n_active, active, expert_ptrs, shared_blob, counts, offsets,
                                     T, k);
        if (S.blob == nullptr) continue;  // no weights behind this expert: leave its rows untouched
        const size_t tile0 = (size_t)strip * nkt;
        for (int m0 = 0; m0 < S.c; m0 += 16) {
            const int nrow = min(16, S.c - m0);
            float4v accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
            const bool ok = (lane & 15) < nrow;
            for (int c0 = kt_lo; c0 < kt_hi; c0 += kMaxT) {
                // weight chunk in flight before (on the first chunk) the activations are staged
                const int nt = min(kMaxT, kt_hi - c0);
                WChunk<kMaxT> w;
                load_chunk<WFMT, kMaxT>(w, S.blob, L.g, L.u, true, tile0, c0, nt, lane);
                if (c0 == kt_lo) {
                    __syncthreads();
                    const int per_row = d / 8;
                    for (int idx = threadIdx.x; idx < nrow * per_row; idx += 256) {
                        const int r = idx / per_row, c8 = (idx % per_row) * 8;
                        const int m = m0 + r;
                        const int t = S.routed ? sorted_idx[S.p0 + m] / k : m;
                        xs4[r * XC + ((c8 >> 3) ^ r)] = __builtin_bit_cast(uint4, load8_h(x + (size_t)t * d + c8));
                    }
                    __syncthreads();
                }
                gu_chunk<WFMT, kMaxT>(w, c0, nt, xs4, XC, ok, lane, accg, accu);
            }
            if (kt_lo == kt_hi) {  // no k tiles for this wavefront (small d): join the staging barriers
                __syncthreads();
                __syncthreads();
            }
            __syncthreads();  // all products done before the staging space is reused
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                red[wave][0][r][lane] = accg[r];
                red[wave][1][r][lane] = accu[r];
            }
            __syncthreads();
            // wavefront w finalises accumulator row r = w (tokens 4*(lane/16) + w)
            {
                const int r = wave;
                const int m = m0 + 4 * (lane >> 4) + r;
                if (m < S.c) {
                    const float g = red[0][0][r][lane] + red[1][0][r][lane] + red[2][0][r][lane] + red[3][0][r][lane];
                    const float u = red[0][1][r][lane] + red[1][1][r][lane] + red[2][1][r][lane] + red[3][1][r][lane];
                    h[(size_t)(S.p0 + m) * f + strip * 16 + (lane & 15)] = (_Float16)(silu_f(g) * u);
                }
            }
        }
    }
}

// down projection: workgroup = (slot, 64 output rows), 16 rows per
// wavefront; the reduction over f runs in chunks of kChunkK held in
// registers; h rows of the current 16-token tile are staged in LDS.
template <int WFMT, typename YT>
__global__ __launch_bounds__(256) void ffn_float_down(const _Float16* __restrict__ h, int T, int d, int f, int k,
                                                      const void* const* __restrict__ expert_ptrs,
                                                      const uint8_t* __restrict__ shared_blob,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ active, YT* __restrict__ y_perm,
                                                      float* __restrict__ y_shared) {
    constexpr int KPT = WFMT == MOE_WFMT_I4B32 ? 128 : 64;
    constexpr int kMaxT = kChunkK / KPT;
    extern __shared__ __align__(16) uint4 hs4[];  // [16][f / 8], chunk c of row r at (c ^ r)
    const int HC = f / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_groups = d / 64;
    const int n_active = active[0];
    const int n_items = (n_active + (shared_blob ? 1 : 0)) * n_groups;
    const ExpertLayout L = expert_layout(WFMT, d, f);
    const int nkt = L.dn.nkt;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int grp = item % n_groups;
        const SlotInfo S = slot_info(item / n_groups, n_active, active, expert_ptrs, shared_blob, counts, offsets,
                                     T, k);
        if (S.blob == nullptr) continue;  // no weights behind this expert: leave its rows untouched
        const int strip = grp * 4 + wave;
        const size_t tile0 = (size_t)strip * nkt;
        for (int m0 = 0; m0 < S.c; m0 += 16) {
            const int nrow = min(16, S.c - m0);
            const bool ok = (lane & 15) < nrow;
            float4v acc = {0, 0, 0, 0};
            for (int c0 = 0; c0 < nkt; c0 += kMaxT) {
                const int nt = min(kMaxT, nkt - c0);
                WChunk<kMaxT> w;
                load_chunk<WFMT, kMaxT>(w, S.blob, L.dn, L.dn, false, tile0, c0, nt, lane);
                if (c0 == 0) {
                    __syncthreads();
                    for (int idx = threadIdx.x; idx < nrow * HC; idx += 256) {
                        const int r = idx / HC, c = idx % HC;
                        hs4[r * HC + (c ^ r)] = *reinterpret_cast<const uint4*>(h + (size_t)(S.p0 + m0 + r) * f + 8 * c);
                    }
                    __syncthreads();
                }
                dn_chunk<WFMT, kMaxT>(w, c0, nt, hs4, HC, ok, lane, acc);
            }
            const int o = strip * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 4 * (lane >> 4) + r;
                if (m >= S.c) continue;
                if (S.routed) y_perm[(size_t)(S.p0 + m) * d + o] = (YT)acc[r];
                else y_shared[(size_t)m * d + o] = acc[r];
            }
        }
    }
}

// ---- small batches, int4 weights: token-dense gate/up ------------------------
// For T <= 16 every token is a row of the MFMA A operand (rows >= T repeat the
// last token and are discarded), so a work item needs no gather and the token
// tile is staged once per workgroup.  Work item = (slot, 16-row strip of f);
// S wavefronts (2 or 4) split its reduction (NT tiles each) and
// software-pipeline their quant tiles two ahead, so that loads of later tiles
// overlap the products of earlier ones.  S = 4 when few experts are active,
// so that enough loads are in flight (one item per 256-thread workgroup);
// with S = 2 a 512-thread workgroup takes four items, so the token tile is
// converted and staged once per four items.  The quants enter the MFMA raw (one
// v_and_or_b32 per pair: 1024 + q, or 1024 + 16 q for the high nibbles, whose
// token values are staged divided by 16); a third MFMA of the same A with a
// constant B seeds each block's sum so that the offsets cancel exactly, and
// the exact block sum x . (q - 8) is scaled by the row's block scale in fp32
// (one v_fma_mix per output and block).

// (q - 8) * s for the 8 nibbles of one int4 dword ([k0 k2 k4 k6 k1 k3 k5 k7])
__device__ __forceinline__ half8 dequant4_scaled(uint32_t v, half2v s2, uint32_t mlo, uint32_t mhi,
                                                 uint32_t magic) {
    const half2v m1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2v r16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const half2v m72 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t v8 = v >> 8;
    const half2v p0 = as_h2((v & mlo) | magic) + m1032;                               // k0, k1
    const half2v p1 = __builtin_elementwise_fma(as_h2((v & mhi) | magic), r16, m72);  // k2, k3
    const half2v p2 = as_h2((v8 & mlo) | magic) + m1032;                              // k4, k5
    const half2v p3 = __builtin_elementwise_fma(as_h2((v8 & mhi) | magic), r16, m72); // k6, k7
    const half2v q0 = p0 * s2, q1 = p1 * s2, q2 = p2 * s2, q3 = p3 * s2;
    return half8{q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y};
}

// fp16 scale of block b (of 4) of an int4 tile row, as fp32
__device__ __forceinline__ float scale_f32(const uint2v& raw, int b) {
    const uint32_t w = b < 2 ? raw[0] : raw[1];
    return (float)__builtin_bit_cast(_Float16, (unsigned short)((b & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

// fp16 scale of block b (of 4) of an int4 tile row, broadcast to both halves
__device__ __forceinline__ half2v scale_pair(const uint2v& raw, int b) {
    const uint32_t w = b < 2 ? raw[0] : raw[1];
    const uint32_t hb = (b & 1) ? (w >> 16) : (w & 0xFFFFu);
    return as_h2(hb | (hb << 16));
}

// int4 quants as raw fp16 words, without offset or scale: 1024 + q for the
// low nibbles (k0 k1, k4 k5 of the dword) and 1024 + 16 q for the high ones
// (k2 k3, k6 k7); one v_and_or_b32 per pair
__device__ __forceinline__ half8 raw4(uint32_t v, uint32_t mlo, uint32_t mhi, uint32_t magic) {
    const uint32_t v8 = v >> 8;
    return __builtin_bit_cast(half8, uint4v{(v & mlo) | magic, (v & mhi) | magic, (v8 & mlo) | magic, (v8 & mhi) | magic});
}

// Seed of the raw block products: with the token values at the high-nibble
// positions (k2 k3 k6 k7 of every 8) staged divided by 16, a block's raw MFMA
// sum is sum x (1024 + q) over the low positions plus sum (x / 16)(1024 + 16 q)
// over the high ones; the products of the same A with this constant B,
// -1032 and -1152 per position, remove exactly the offsets (1024 + 8 and
// 16 (64 + 8)), leaving sum x (q - 8).  All values are exact in fp16.
__device__ __forceinline__ half8 offset_seed_b() {
    const _Float16 lo = (_Float16)-1032.0f, hi = (_Float16)-1152.0f;
    return half8{lo, lo, hi, hi, lo, lo, hi, hi};
}

constexpr int kTokMax = 16;   // tokens of the token-dense kernels
constexpr int kDcWaves = 4;     // wavefronts of ffn_down_combine (slots split over them)
constexpr int kDcWavesFew = 8;  // the same for one or two tokens
constexpr int kPipe = 2;      // quant tiles in flight ahead of the products

// Raw 16-byte token chunks, converted to fp16 only when stored to LDS, so that
// the loads can be issued before anything else without waiting on them.
template <typename XT> struct XChunk;
// a token chunk with elements 2, 3, 6, 7 divided by 16 (exact in fp16)
__device__ __forceinline__ half8 pre16(half8 v) {
    const half2v r = {(_Float16)0.0625f, (_Float16)0.0625f};
    const half2v a = half2v{v[2], v[3]} * r, b = half2v{v[6], v[7]} * r;
    return half8{v[0], v[1], a.x, a.y, v[4], v[5], b.x, b.y};
}
template <> struct XChunk<uint16_t> {
    uint4v r;
    __device__ __forceinline__ void load(const uint16_t* p) { r = gload(reinterpret_cast<const uint4v*>(p)); }
    __device__ __forceinline__ half8 cvt() const {
        half8 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = (_Float16)__uint_as_float(r[j] << 16);
            v[2 * j + 1] = (_Float16)__uint_as_float(r[j] & 0xFFFF0000u);
        }
        return v;
    }
    __device__ __forceinline__ half8 cvt_pre16() const { return pre16(cvt()); }
};
template <> struct XChunk<float> {
    uint4v a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = gload(reinterpret_cast<const uint4v*>(p));
        b = gload(reinterpret_cast<const uint4v*>(p) + 1);
    }
    __device__ __forceinline__ half8 cvt() const {
        half8 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = (_Float16)__uint_as_float(a[j]);
            v[4 + j] = (_Float16)__uint_as_float(b[j]);
        }
        return v;
    }
    __device__ __forceinline__ half8 cvt_pre16() const { return pre16(cvt()); }
};

template <> struct XChunk<_Float16> {
    uint4v r;
    __device__ __forceinline__ void load(const _Float16* p) { r = gload(reinterpret_cast<const uint4v*>(p)); }
    __device__ __forceinline__ half8 cvt() const { return __builtin_bit_cast(half8, r); }
    __device__ __forceinline__ half8 cvt_pre16() const { return pre16(cvt()); }
};


// Order of the start: token chunks requested first; slot metadata in two
// dependent rounds (the list entry is read before the list length is known,
// at a clamped index); then the first quant tiles and the slot's token list,
// through buffer resources of size 0 when there is nothing to read, so that
// the code stays straight-line and every wait is exact; only then the tokens
// go to LDS.
// BY_SLOT: no grouping; work slot a < T k is the routed slot a itself (expert
// slot_ids[a], its one row written to h row a), slot T k the shared expert.
// TOPK > 0 (with BY_SLOT): the slot's expert is selected here instead, by the
// router's top-k of token a / k over the logits (TOPK values per lane); the
// first wavefront ranks the token's logits, and one workgroup per token
// writes its ids and gates at the end.
template <int NT, int S, typename XT, int NTH = 256, bool BY_SLOT = false, int TOPK = 0>
__global__ __launch_bounds__(NTH) void ffn_gateup_tok16(const XT* __restrict__ x, int T, int d, int f, int k, int E,
                                                        const void* const* __restrict__ expert_ptrs,
                                                        const uint8_t* __restrict__ shared_blob,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ sorted_idx,
                                                        const int32_t* __restrict__ active, _Float16* __restrict__ h,
                                                        const int32_t* __restrict__ slot_ids,
                                                        const double* __restrict__ logits, int planes,
                                                        int32_t* __restrict__ ids_out, float* __restrict__ gates_out,
                                                        const uint8_t** __restrict__ slot_blob_out) {
    extern __shared__ __align__(16) uint4 xs4[];  // [T][d / 8] fp16, chunk c of row r at (c ^ r); later [4][2][4][64] f32
    __shared__ RankScratch rs;       // TOPK: the selection of this workgroup's token
    __shared__ int32_t s_sel[64];
    const int XC = d / 8;           // a power of two (checked by the launcher)
    const int lxc = __builtin_ctz(XC);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int part = wave % S;
    const int n_strips = f / 16;
    const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * (NTH / 64 / S) + wave / S);
    const int a = item / n_strips, strip = item % n_strips;
    const int nx = T * XC;
    XChunk<XT> xr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // chunks past the end are not requested (no repeated address)
        const int idx = (int)threadIdx.x + j * NTH;
        if (idx < nx) xr[j].load(x + (size_t)idx * 8);
    }
    const uint8_t* blob;
    int e, c, p0, slot_of;
    if constexpr (BY_SLOT) {
        const int n_slots = T * k;
        const bool routed = a < n_slots;
        int e_raw;
        if constexpr (TOPK > 0) {
            const int ts = min(a, n_slots - 1) / k;
            if (wave == 0) topk_select<TOPK>(logits + (size_t)ts * E, E, k, s_sel, rs, planes, (size_t)T * E);
            __syncthreads();
            e_raw = s_sel[min(a, n_slots - 1) - ts * k];
        } else {
            e_raw = slot_ids[min(a, n_slots - 1)];
        }
        const bool valid = (unsigned)e_raw < (unsigned)E;
        const uint8_t* pe = (const uint8_t*)expert_ptrs[valid ? e_raw : 0];
        blob = routed ? (valid ? pe : nullptr) : (a == n_slots ? shared_blob : nullptr);
        e = routed ? e_raw : -1;
        c = routed ? 1 : T;
        p0 = routed ? a : n_slots;
        slot_of = a;  // the slot's single row belongs to token a / k
        // the slot's blob for the down projection, which then needs no lookup of
        // its own (one vector store per slot)
        if (slot_blob_out && routed && strip == 0 && part == 0 && lane == 0) slot_blob_out[a] = blob;
    } else {
        const int n_active = active[0];
        const int e_raw = active[1 + min(a, E - 1)];
        const int e_c = min(max(e_raw, 0), E - 1);
        const uint8_t* pe = (const uint8_t*)expert_ptrs[e_c];
        const int ce = counts[e_c], oe = offsets[e_c];
        const bool routed = a < n_active;
        blob = routed ? pe : (a == n_active ? shared_blob : nullptr);
        e = routed ? e_raw : -1;
        c = routed ? ce : T;
        p0 = routed ? oe : T * k;
        const __amdgpu_buffer_rsrc_t ir = buf_rsrc(sorted_idx, e >= 0 ? (uint32_t)(T * k * 4) : 0u);
        // slot of each of the first 64 rows (row m of the slot belongs to token slot_of / k)
        slot_of = __builtin_amdgcn_raw_buffer_load_b32(ir, (p0 + min(lane, max(c - 1, 0))) * 4, 0, 0);
    }
    const bool work = blob != nullptr;  // no weights behind this expert: leave its rows untouched
    const ExpertLayout L = expert_layout(MOE_WFMT_I4B32, d, f);
    const __amdgpu_buffer_rsrc_t wr = buf_rsrc(blob, work ? (uint32_t)L.total : 0u);
    const uint32_t tile0 = (uint32_t)(strip * (S * NT) + part * NT);
    const uint32_t og = (uint32_t)L.g.qoff + tile0 * 1024 + lane * 16;
    const uint32_t ou = (uint32_t)L.u.qoff + tile0 * 1024 + lane * 16;
    const uint32_t osg = (uint32_t)L.g.soff + tile0 * 128 + (lane & 15) * 8;
    const uint32_t osu = (uint32_t)L.u.soff + tile0 * 128 + (lane & 15) * 8;
    auto ld2 = [&](uint32_t off) { return __builtin_bit_cast(uint2v, __builtin_amdgcn_raw_buffer_load_b64(wr, off, 0, kBufNT)); };
    auto ld4 = [&](uint32_t off) { return __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, kBufNT)); };
    uint4v qg[NT], qu[NT];
    uint2v sg[NT], su[NT];
#pragma unroll
    for (int i = 0; i < kPipe && i < NT; ++i) {
        sg[i] = ld2(osg + i * 128);
        su[i] = ld2(osu + i * 128);
        qg[i] = ld4(og + i * 1024);
        qu[i] = ld4(ou + i * 1024);
    }
    // tokens -> LDS as fp16, the high-nibble positions divided by 16
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int idx = (int)threadIdx.x + j * NTH;
        if (idx < nx) {
            const int r = idx >> lxc, cc = idx & (XC - 1);
            xs4[r * XC + (cc ^ r)] = __builtin_bit_cast(uint4, xr[j].cvt_pre16());
        }
    }
    for (int base = 4 * NTH; base < nx; base += 4 * NTH) {
        XChunk<XT> xq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = base + (int)threadIdx.x + j * NTH;
            if (idx < nx) xq[j].load(x + (size_t)idx * 8);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = base + (int)threadIdx.x + j * NTH;
            if (idx < nx) {
                const int r = idx >> lxc, cc = idx & (XC - 1);
                xs4[r * XC + (cc ^ r)] = __builtin_bit_cast(uint4, xq[j].cvt_pre16());
            }
        }
    }
    __syncthreads();
    float4v accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
    const half8 Bc = offset_seed_b();
    const float4v zero4 = {0, 0, 0, 0};
    {
        const int rr = min(lane & 15, T - 1);
        // bit masks and magic in registers so that each extraction is one v_and_or_b32
        uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, magic = 0x64006400u;
        asm volatile("" : "+s"(mlo), "+s"(mhi), "+v"(magic));
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            if (i + kPipe < NT) {
                const int n = i + kPipe;
                sg[n] = ld2(osg + n * 128);
                su[n] = ld2(osu + n * 128);
                qg[n] = ld4(og + n * 1024);
                qu[n] = ld4(ou + n * 1024);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int kk = ((part * NT + i) * 4 + b) * 32 + 8 * (lane >> 4);
                const half8 A = __builtin_bit_cast(half8, xs4[rr * XC + ((kk >> 3) ^ rr)]);
                // exact block sums x . (q - 8): raw quants seeded with A . Bc,
                // then scaled by the row's block scale in fp32
                const float4v dc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bc, zero4, 0, 0, 0);
                const float4v dg = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, raw4(qg[i][b], mlo, mhi, magic), dc, 0, 0, 0);
                const float4v du = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, raw4(qu[i][b], mlo, mhi, magic), dc, 0, 0, 0);
                const float sgb = scale_f32(sg[i], b), sub = scale_f32(su[i], b);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    accg[r] = fmaf(dg[r], sgb, accg[r]);
                    accu[r] = fmaf(du[r], sub, accu[r]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the parts of the reduction meet in LDS (the token tile is no longer read)
    __syncthreads();
    float(*red)[2][4][64] = reinterpret_cast<float(*)[2][4][64]>(xs4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        red[wave][0][r][lane] = accg[r];
        red[wave][1][r][lane] = accu[r];
    }
    __syncthreads();
    if constexpr (TOPK > 0) {
        // ids and gates of the token (the softmax over the selected logits),
        // written once, by the workgroup of its first slot's first strip, and
        // only after every load of this workgroup: the selection alone gates
        // the weight loads
        const int n_slots = T * k;
        if (wave == 0 && a < n_slots && a % k == 0 && strip == 0)
            topk_gates(rs, k, ids_out + (size_t)(a / k) * k, gates_out + (size_t)(a / k) * k);
    }
    if (!work) return;
    const int w0 = wave - part;
    const int col = strip * 16 + (lane & 15);
    // accumulator row r holds token 4 * (lane / 16) + r; wavefront `part` writes rows r = part, part + S, ..
    // to every position of the slot that token t occupies (a token listed twice gets two rows)
#pragma unroll
    for (int r = part; r < 4; r += S) {
        const int t = 4 * (lane >> 4) + r;
        if (t >= T) continue;
        float g = red[w0][0][r][lane], u = red[w0][1][r][lane];
#pragma unroll
        for (int q = 1; q < S; ++q) {
            g += red[w0 + q][0][r][lane];
            u += red[w0 + q][1][r][lane];
        }
        const _Float16 hv = (_Float16)(silu_f(g) * u);
        if (e < 0) {
            h[(size_t)(p0 + t) * f + col] = hv;
        } else {
            const unsigned lo = (unsigned)(t * k);
            const int cm = min(c, 64);
            for (int m = 0; m < cm; ++m)
                if ((unsigned)__builtin_amdgcn_readlane(slot_of, m) - lo < (unsigned)k) h[(size_t)(p0 + m) * f + col] = hv;
            if constexpr (!BY_SLOT)
                for (int m = 64; m < c; ++m)
                    if (sorted_idx[p0 + m] / k == t) h[(size_t)(p0 + m) * f + col] = hv;
        }
    }
}

template <typename XT, bool BY_SLOT = false, int TOPK = 0>
static bool launch_gateup_tok16(const moe_ffn_args* a, _Float16* h, int slots, hipStream_t s,
                                const int32_t* slot_ids = nullptr, const double* logits = nullptr, int planes = 1,
                                int32_t* ids_out = nullptr, float* gates_out = nullptr,
                                const uint8_t** slot_blob = nullptr) {
    const int nkt = a->d / 128;
    const int items = slots * (a->f / 16);
    // few items (a single token routes to k + 1 slots): four wavefronts per
    // item where an instance exists, else two
    const bool four = items < 1024 && (nkt == 8 || nkt == 16 || nkt == 32);
    const dim3 grid(four ? items : (items + 3) / 4);
    const size_t lds = std::max<size_t>((size_t)a->T * a->d * sizeof(_Float16), 8 * 2 * 4 * 64 * sizeof(float));
#define MOE_GU16(NT, S)                                                                                         \
    ffn_gateup_tok16<NT, S, XT, S == 2 ? 512 : 256, BY_SLOT, TOPK><<<grid, S == 2 ? 512 : 256, lds, s>>>(        \
        (const XT*)a->x, a->T, a->d, a->f, a->k, a->E, a->expert_ptrs, (const uint8_t*)a->shared_blob, a->counts, \
        a->offsets, a->sorted_idx, a->active, h, slot_ids, logits, planes, ids_out, gates_out, slot_blob)
    if (four) {
        switch (nkt) {
        case 8: MOE_GU16(2, 4); return true;
        case 16: MOE_GU16(4, 4); return true;
        case 32: MOE_GU16(8, 4); return true;
        default: return false;
        }
    }
    switch (nkt) {
    case 4: MOE_GU16(2, 2); return true;
    case 8: MOE_GU16(4, 2); return true;
    case 16: MOE_GU16(8, 2); return true;
    case 32: MOE_GU16(16, 2); return true;
    default: return false;
    }
#undef MOE_GU16
}

// Down projection for small batches (int4): work item = (slot, 16 output
// rows), one wavefront per item over the whole reduction, four items of one
// slot per workgroup (eight when few slots are active) sharing the slot's h
// rows staged in LDS (16 rows at a
// time); the first kPipe quant tiles are requested before the h rows, the
// rest pipelined.
template <int NKT, typename YT, int NW>
__global__ __launch_bounds__(64 * NW) void ffn_down_tok16(const _Float16* __restrict__ h, int T, int d, int f, int k,
                                                      const void* const* __restrict__ expert_ptrs,
                                                      const uint8_t* __restrict__ shared_blob,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ active, YT* __restrict__ y_perm,
                                                      float* __restrict__ y_shared) {
    extern __shared__ __align__(16) uint4 hs4[];  // [16][f / 8], chunk c of row r at (c ^ r)
    const int HC = f / 8;
    const int lane = threadIdx.x & 63;
    const int n_strips = d / 16;  // a multiple of NW: the NW items of a workgroup share one slot
    const int item0 = __builtin_amdgcn_readfirstlane(blockIdx.x * NW);
    const int strip = (item0 % n_strips) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int a = item0 / n_strips;
    const int n_active = active[0];
    const uint8_t* blob = nullptr;
    int c = 0, p0 = 0;
    bool routed = false;
    if (a < n_active) {
        const int e = active[1 + a];
        blob = (const uint8_t*)expert_ptrs[e];
        c = counts[e];
        p0 = offsets[e];
        routed = true;
    } else if (a == n_active && shared_blob) {
        blob = shared_blob;
        c = T;
        p0 = T * k;
    }
    if (blob == nullptr || c == 0) return;  // uniform over the workgroup
    const ExpertLayout L = expert_layout(MOE_WFMT_I4B32, d, f);
    const size_t tile0 = (size_t)strip * NKT;
    const uint4v* pq = reinterpret_cast<const uint4v*>(blob + L.dn.qoff + tile0 * 1024) + lane;
    const uint2v* ps = reinterpret_cast<const uint2v*>(blob + L.dn.soff + tile0 * 128 + (lane & 15) * 8);
    uint4v q[NKT];
    uint2v sc[NKT];
#pragma unroll
    for (int i = 0; i < kPipe && i < NKT; ++i) {
        sc[i] = gload_nt(ps + i * 16);
        q[i] = gload_nt(pq + i * 64);
    }
    const int rr0 = lane & 15;
    uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, magic = 0x64006400u;
    asm volatile("" : "+s"(mlo), "+s"(mhi), "+v"(magic));
    const int o = strip * 16 + (lane & 15);
    // rows of the slot in tiles of 16 (more than one tile only when a token lists an expert twice)
    for (int m0 = 0; m0 < c; m0 += 16) {
        const int nr = min(16, c - m0);
        if (m0 > 0) {
            __syncthreads();  // the previous tile's rows are no longer read
#pragma unroll
            for (int i = 0; i < kPipe && i < NKT; ++i) {
                sc[i] = gload_nt(ps + i * 16);
                q[i] = gload_nt(pq + i * 64);
            }
        }
        // the tile's h rows -> LDS, two 16-byte chunks per thread per round
        const int nh = nr * HC;
        for (int base = 0; base < nh; base += 128 * NW) {
            uint4v v[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int idx = min(base + (int)threadIdx.x + j * 64 * NW, nh - 1);
                v[j] = gload(reinterpret_cast<const uint4v*>(h + (size_t)(p0 + m0 + idx / HC) * f) + idx % HC);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int idx = base + (int)threadIdx.x + j * 64 * NW;
                if (idx < nh) {
                    const int r = idx / HC, cc = idx % HC;
                    hs4[r * HC + (cc ^ r)] = __builtin_bit_cast(uint4, v[j]);
                }
            }
        }
        __syncthreads();
        const int rr = min(rr0, nr - 1);
        float4v acc = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < NKT; ++i) {
            if (i + kPipe < NKT) {
                sc[i + kPipe] = gload_nt(ps + (i + kPipe) * 16);
                q[i + kPipe] = gload_nt(pq + (i + kPipe) * 64);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const half8 B = dequant4_scaled(q[i][b], scale_pair(sc[i], b), mlo, mhi, magic);
                const int kk = (i * 4 + b) * 32 + 8 * (lane >> 4);
                const half8 A = __builtin_bit_cast(half8, hs4[rr * HC + ((kk >> 3) ^ rr)]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, acc, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * (lane >> 4) + r;
            if (m >= nr) continue;
            if (routed) y_perm[(size_t)(p0 + m0 + m) * d + o] = (YT)acc[r];
            else y_shared[(size_t)(m0 + m) * d + o] = acc[r];
        }
    }
}

template <typename YT>
static bool launch_down_tok16(const moe_ffn_args* a, const _Float16* h, int slots, hipStream_t s) {
    if (a->d % 64) return false;
    // few slots (a single token): eight items per workgroup share the staged h rows
    const bool wide = a->d % 128 == 0 && (long)slots * (a->d / 64) < 1024;
    const dim3 grid(slots * (a->d / (wide ? 128 : 64)));
    const size_t lds = (size_t)kTokMax * a->f * sizeof(_Float16);
#define MOE_DN16(NKT)                                                                                               \
    if (wide)                                                                                                       \
        ffn_down_tok16<NKT, YT, 8><<<grid, 512, lds, s>>>(h, a->T, a->d, a->f, a->k, a->expert_ptrs,                \
                                                          (const uint8_t*)a->shared_blob, a->counts, a->offsets,    \
                                                          a->active, (YT*)a->y_perm, a->y_shared);                  \
    else                                                                                                            \
        ffn_down_tok16<NKT, YT, 4><<<grid, 256, lds, s>>>(h, a->T, a->d, a->f, a->k, a->expert_ptrs,                \
                                                          (const uint8_t*)a->shared_blob, a->counts, a->offsets,    \
                                                          a->active, (YT*)a->y_perm, a->y_shared)
    switch (a->f / 128) {
    case 2: MOE_DN16(2); return true;
    case 4: MOE_DN16(4); return true;
    case 6: MOE_DN16(6); return true;
    case 8: MOE_DN16(8); return true;
    case 12: MOE_DN16(12); return true;
    case 16: MOE_DN16(16); return true;
    default: return false;
    }
#undef MOE_DN16
}

// ---- few tokens, int4: down projection and weighted combine in one kernel ----
// Workgroup = (token t, 16 output rows); its NW wavefronts split the token's
// k routed slots and the shared expert (slot j goes to wavefront j % NW).
// The slots' expert pointers, gates and h rows are staged once per workgroup
// (h rows in LDS, chunk c of slot j at j * f / 8 + c, the high-nibble
// positions divided by 16 as for the decode gate/up, whose seeded raw-quant
// products and fp32 block scale this kernel uses too).  A wavefront streams
// the 16-row down strip of each of its slots (all f / 128 quant tiles at
// once), issuing the next slot's tiles before the products of the current
// one (a second slot ahead measured slower); the A operand repeats the slot's
// h row in all 16 MFMA rows, so every accumulator row holds the same 16
// outputs.  Each wavefront adds gate * y in
// its slot order; the NW partial vectors meet in LDS and are added in
// wavefront order after the residual (deterministic).  The expert outputs
// stay in fp32: no y_perm rows are written or read back.  dest == nullptr:
// the slots were not grouped and slot j's h row is t k + j.
constexpr int kDcMaxSlots = 65;  // k <= 64 routed slots + the shared expert
constexpr int kDcChunks = 8;     // h chunks staged per thread: nj f / 8 <= kDcChunks * 64 * NW
constexpr int kDcStrips = 1;     // 16-row strips per workgroup (2 measured slower: fewer workgroups)
template <int NKT, int NW, int RS = kDcStrips>
__global__ __launch_bounds__(64 * NW) void ffn_down_combine(const _Float16* __restrict__ h, int T, int d, int f,
                                                            int k, int E, const void* const* __restrict__ expert_ptrs,
                                                            const uint8_t* __restrict__ shared_blob,
                                                            const int32_t* __restrict__ ids,
                                                            const int32_t* __restrict__ dest,
                                                            const float* __restrict__ gates, const float* residual,
                                                            float* out, const uint8_t* const* __restrict__ slot_blob) {
    extern __shared__ __align__(16) uint4 hrow[];  // [nj][f / 8]
    __shared__ const uint8_t* s_blob[kDcMaxSlots];  // nullptr: the slot is ignored
    __shared__ int32_t s_p[kDcMaxSlots];
    __shared__ float s_g[kDcMaxSlots];
    __shared__ float part[NW][16 * RS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_groups = d / (16 * RS);  // RS consecutive 16-row strips per workgroup
    const int t = blockIdx.x / n_groups, strip = (blockIdx.x % n_groups) * RS;
    const int nj = k + (shared_blob ? 1 : 0);
    const int HC = f / 8;
    for (int j = threadIdx.x; j < nj; j += 64 * NW) {
        if (j < k && slot_blob) {  // by slot: the blob the gate/up launch used (nullptr: ignored)
            s_blob[j] = slot_blob[(size_t)t * k + j];
            s_p[j] = t * k + j;
            s_g[j] = gates[(size_t)t * k + j];
        } else if (j < k) {
            const int e = ids[(size_t)t * k + j];
            const bool ok = (unsigned)e < (unsigned)E;  // ids outside [0, E) are ignored, as in the grouping
            s_blob[j] = ok ? (const uint8_t*)expert_ptrs[e] : nullptr;
            s_p[j] = !ok ? 0 : dest ? dest[(size_t)t * k + j] : t * k + j;  // no dest: h row = slot
            s_g[j] = gates[(size_t)t * k + j];
        } else {
            s_blob[j] = shared_blob;
            s_p[j] = T * k + t;
            s_g[j] = 1.f;
        }
    }
    __syncthreads();
    const ExpertLayout L = expert_layout(MOE_WFMT_I4B32, d, f);
    const size_t qoff = L.dn.qoff + (size_t)strip * NKT * 1024 + lane * 16;
    const size_t soff = L.dn.soff + (size_t)strip * NKT * 128 + (lane & 15) * 8;
    constexpr int NQ = RS * NKT;  // the RS strips' tiles are consecutive in the blob
    uint4v q[NQ], qn[NQ];
    uint2v sc[NQ], scn[NQ];
    auto issue = [&](int j, uint4v (&qq)[NQ], uint2v (&ss)[NQ]) {
        const uint8_t* blob = s_blob[j];
        if (blob == nullptr) return;
        const uint4v* pq = reinterpret_cast<const uint4v*>(blob + qoff);
        const uint2v* ps = reinterpret_cast<const uint2v*>(blob + soff);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            ss[i] = gload_nt(ps + i * 16);
            qq[i] = gload_nt(pq + i * 64);
        }
    };
    // the slots' h rows (at most kDcChunks 16-byte chunks per thread) and the
    // first slot's quant tiles are all in flight before any LDS store
    // (straight-line buffer loads: a chunk past the end gets an offset outside
    // the resource, which reads nothing, so no address is requested twice)
    const int nh = nj * HC;
    const __amdgpu_buffer_rsrc_t hres = buf_rsrc(h, (uint32_t)(((size_t)T * k + T) * f * 2));
    uint4v v[kDcChunks];
#pragma unroll
    for (int u = 0; u < kDcChunks; ++u) {
        const int idx = (int)threadIdx.x + u * 64 * NW;
        const int ic = min(idx, nh - 1), j = ic / HC;
        const uint32_t off = idx < nh ? ((uint32_t)s_p[j] * f + (uint32_t)(ic - j * HC) * 8) * 2 : 0x80000000u;
        v[u] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(hres, off, 0, 0));
    }
    if (wave < nj) issue(wave, q, sc);
#pragma unroll
    for (int u = 0; u < kDcChunks; ++u) {
        const int idx = (int)threadIdx.x + u * 64 * NW;
        if (idx < nh) hrow[idx] = __builtin_bit_cast(uint4, pre16(__builtin_bit_cast(half8, v[u])));
    }
    __syncthreads();
    uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, magic = 0x64006400u;
    asm volatile("" : "+s"(mlo), "+s"(mhi), "+v"(magic));
    const half8 Bc = offset_seed_b();
    const float4v zero4 = {0, 0, 0, 0};
    float tot[RS];
#pragma unroll
    for (int r = 0; r < RS; ++r) tot[r] = 0.f;
    for (int j = wave; j < nj; j += NW) {
        if (j + NW < nj) issue(j + NW, qn, scn);
        __builtin_amdgcn_sched_barrier(0);  // the next slot's tiles are in flight before these products
        if (s_blob[j] != nullptr) {
            const uint4* hr = hrow + j * HC + (lane >> 4);
#pragma unroll
            for (int r = 0; r < RS; ++r) {
                float y = 0.f;
#pragma unroll
                for (int i = 0; i < NKT; ++i)
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        // exact block sum h . (q - 8): raw quants seeded with A . Bc,
                        // then the row's block scale in fp32 (row 0 of the tile only)
                        const int n = r * NKT + i;
                        const half8 A = __builtin_bit_cast(half8, hr[(i * 4 + b) * 4]);
                        const float4v dc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bc, zero4, 0, 0, 0);
                        const float4v dq =
                            __builtin_amdgcn_mfma_f32_16x16x32_f16(A, raw4(q[n][b], mlo, mhi, magic), dc, 0, 0, 0);
                        y = fmaf(dq[0], scale_f32(sc[n], b), y);
                    }
                tot[r] = fmaf(s_g[j], y, tot[r]);  // lane l < 16: output row (strip + r) * 16 + l
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            q[i] = qn[i];
            sc[i] = scn[i];
        }
    }
    if (lane < 16)
#pragma unroll
        for (int r = 0; r < RS; ++r) part[wave][16 * r + lane] = tot[r];
    __syncthreads();
    if (threadIdx.x < 16 * RS) {
        const size_t o = (size_t)t * d + strip * 16 + threadIdx.x;
        float sum = residual ? residual[o] : 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += part[w][threadIdx.x];
        out[o] = sum;
    }
}

bool down_combine_ok(const moe_ffn_args* a) {
    const int nkt = a->f / 128;
    const int nj = a->k + (a->shared_blob ? 1 : 0);
    const int nw = a->T <= 2 ? kDcWavesFew : kDcWaves;
    return a->act_mode == MOE_ACT_FLOAT && a->wfmt == MOE_WFMT_I4B32 && a->T <= kDownCombineMax &&
           a->d % (16 * kDcStrips) == 0 &&
           (nkt == 2 || nkt == 4 || nkt == 6 || nkt == 8) && (long)nj * (a->f / 8) <= (long)kDcChunks * 64 * nw;
}

int launch_down_combine(const moe_ffn_args* a, const Workspace& w, const int32_t* ids, const int32_t* dest,
                        const float* gates, const float* residual, float* out, hipStream_t s,
                        const uint8_t* const* slot_blob) {
    if (!down_combine_ok(a)) return MOE_ERR_UNSUPPORTED;
    const _Float16* h = reinterpret_cast<const _Float16*>(w.h);
    const dim3 grid(a->T * (a->d / (16 * kDcStrips)));
    const uint8_t* sb = (const uint8_t*)a->shared_blob;
    const size_t lds = (size_t)(a->k + (sb ? 1 : 0)) * a->f * sizeof(_Float16);
#define MOE_DC(NKT, NW)                                                                                          \
    ffn_down_combine<NKT, NW><<<grid, 64 * NW, lds, s>>>(h, a->T, a->d, a->f, a->k, a->E, a->expert_ptrs, sb, ids, \
                                                        dest, gates, residual, out, slot_blob)
#define MOE_DC_NW(NKT)                          \
    if (a->T <= 2) MOE_DC(NKT, kDcWavesFew);    \
    else MOE_DC(NKT, kDcWaves)
    switch (a->f / 128) {
    case 2: MOE_DC_NW(2); break;
    case 4: MOE_DC_NW(4); break;
    case 6: MOE_DC_NW(6); break;
    default: MOE_DC_NW(8); break;
    }
#undef MOE_DC_NW
#undef MOE_DC
    return check_launch();
}

// the by-slot gate/up launch has an instance (the conditions of
// launch_gateup_tok16 and of the token-dense path in run_float)
static bool gateup_tok16_by_slot_ok(const moe_ffn_args* a) {
    if (a->T > kTokMax || (size_t)a->T * a->d * 2 > 64 * 1024 || (a->d & (a->d - 1)) != 0) return false;
    const int nkt = a->d / 128;
    return nkt == 4 || nkt == 8 || nkt == 16 || nkt == 32;
}

bool ffn_combine_slots_ok(const moe_ffn_args* a) { return down_combine_ok(a) && gateup_tok16_by_slot_ok(a); }

int launch_ffn_combine_slots(const moe_ffn_args* a, const Workspace& w, const int32_t* ids, const float* gates,
                             const float* residual, float* out, hipStream_t s) {
    if (!ffn_combine_slots_ok(a)) return MOE_ERR_UNSUPPORTED;
    const int slots = a->T * a->k + (a->shared_blob ? 1 : 0);
    _Float16* h = reinterpret_cast<_Float16*>(w.h);
    const bool ok =
        a->x_dtype == MOE_DT_F32
            ? launch_gateup_tok16<float, true>(a, h, slots, s, ids, nullptr, 1, nullptr, nullptr, w.slot_blob)
            : launch_gateup_tok16<uint16_t, true>(a, h, slots, s, ids, nullptr, 1, nullptr, nullptr, w.slot_blob);
    if (!ok) return MOE_ERR_UNSUPPORTED;
    const int rc = check_launch();
    if (rc || a->phase == 1) return rc;
    return launch_down_combine(a, w, ids, nullptr, gates, residual, out, s, w.slot_blob);
}

// routing + by-slot FFN + combine for decode batches: the router logits are
// in the workspace (w.logits, `planes` k planes); the gate/up kernel selects
// each slot's expert from them and writes ids and gates for the combine
int launch_ffn_combine_slots_topk(const moe_ffn_args* a, const Workspace& w, int planes, int32_t* ids, float* gates,
                                  const float* residual, float* out, hipStream_t s) {
    if (!ffn_combine_slots_ok(a) || a->E > 1024) return MOE_ERR_UNSUPPORTED;
    const int slots = a->T * a->k + (a->shared_blob ? 1 : 0);
    _Float16* h = reinterpret_cast<_Float16*>(w.h);
    bool ok;
    if (a->E <= 512)
        ok = a->x_dtype == MOE_DT_F32
                 ? launch_gateup_tok16<float, true, 8>(a, h, slots, s, nullptr, w.logits, planes, ids, gates,
                                                       w.slot_blob)
                 : launch_gateup_tok16<uint16_t, true, 8>(a, h, slots, s, nullptr, w.logits, planes, ids, gates,
                                                          w.slot_blob);
    else
        ok = a->x_dtype == MOE_DT_F32
                 ? launch_gateup_tok16<float, true, 16>(a, h, slots, s, nullptr, w.logits, planes, ids, gates,
                                                        w.slot_blob)
                 : launch_gateup_tok16<uint16_t, true, 16>(a, h, slots, s, nullptr, w.logits, planes, ids, gates,
                                                           w.slot_blob);
    if (!ok) return MOE_ERR_UNSUPPORTED;
    const int rc = check_launch();
    if (rc || a->phase == 1) return rc;
    return launch_down_combine(a, w, ids, nullptr, gates, residual, out, s, w.slot_blob);
}

size_t float_h_bytes(int T, int f, int k) { return ((size_t)T * k + T) * (size_t)f * sizeof(_Float16); }

// ---- moderate batches (T <= 64): token-dense gate/up, slot-dense down --------
// Gate/up: every token is a row of the MFMA A operand (four 16-token m-tiles;
// rows >= T repeat the last token and are discarded).  A workgroup takes
// (slot, 16 NW rows of f): wavefront w of NW owns the 16-row strip NW g + w
// and streams its quant tiles through registers kPipe chunks ahead, while all
// NW stage the tokens of the current 128-wide k-chunk in LDS as fp16 (double
// buffered).  NW = 8 on large grids, so each token chunk is converted once per
// 128 rows of f; NW = 4 on small ones.
// Each weight is read once and serves every token; the block-scaled weights
// accumulate in the MFMA as in the small-batch kernel.  The results go to LDS
// as [token][16 features] and are scattered to the slot's rows from there.
// Down: the same streaming over f for (slot, 64 output rows), with the slot's
// h rows (contiguous, at most 64 per pass) as the A operand.
constexpr int kTok64 = 64;
constexpr int kKC = 128;     // k per chunk
constexpr int kPipe64 = 2;   // gate/up chunks in flight ahead of the products (three wavefronts per SIMD fit)

// (q) * s for the 8 int8 weights of one block (two dwords in k order, q stored
// as q + 128): bytes are paired with the 0x64 magic byte by v_perm_b32
// (1024 + q + 128 exactly), the offset is removed and the block scale applied
// with one rounding.
__device__ __forceinline__ half8 dequant8_scaled(uint32_t v0, uint32_t v1, half2v s2, uint32_t magic) {
    const half2v m1152 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const half2v p0 = as_h2(__builtin_amdgcn_perm(magic, v0, 0x04010400u)) + m1152;
    const half2v p1 = as_h2(__builtin_amdgcn_perm(magic, v0, 0x04030402u)) + m1152;
    const half2v p2 = as_h2(__builtin_amdgcn_perm(magic, v1, 0x04010400u)) + m1152;
    const half2v p3 = as_h2(__builtin_amdgcn_perm(magic, v1, 0x04030402u)) + m1152;
    const half2v q0 = p0 * s2, q1 = p1 * s2, q2 = p2 * s2, q3 = p3 * s2;
    return half8{q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y};
}

// Quant tiles of one strip for one 128-k chunk: TPC packed tiles of one matrix.
template <int WFMT>
struct StripChunk {
    static constexpr int TPC = WFMT == MOE_WFMT_I4B32 ? 1 : 2;
    uint4v q[TPC];
    uint2v s[TPC];  // int4: four fp16 block scales; int8: two (.x)
};

template <int WFMT>
__device__ __forceinline__ void load_strip_chunk(StripChunk<WFMT>& w, __amdgpu_buffer_rsrc_t r, uint32_t qoff,
                                                 uint32_t soff, uint32_t tile, int lane) {
    constexpr int TPC = StripChunk<WFMT>::TPC;
#pragma unroll
    for (int j = 0; j < TPC; ++j) {
        w.q[j] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(r, qoff + (tile + j) * 1024 + lane * 16, 0, kBufNT));
        if constexpr (WFMT == MOE_WFMT_I4B32)
            w.s[j] = __builtin_bit_cast(uint2v, __builtin_amdgcn_raw_buffer_load_b64(r, soff + (tile + j) * 128 + (lane & 15) * 8, 0, kBufNT));
        else
            w.s[j] = uint2v{(uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, soff + (tile + j) * 64 + (lane & 15) * 4, 0, kBufNT), 0u};
    }
}

// scaled fp16 weights of block b (0..3) of a 128-k chunk
template <int WFMT>
__device__ __forceinline__ half8 strip_block(const StripChunk<WFMT>& w, int b, uint32_t mlo, uint32_t mhi,
                                             uint32_t magic) {
    if constexpr (WFMT == MOE_WFMT_I4B32) {
        return dequant4_scaled(w.q[0][b], scale_pair(w.s[0], b), mlo, mhi, magic);
    } else {
        const int j = b >> 1, bb = b & 1;
        const uint32_t sw = w.s[j][0];
        const uint32_t hb = bb ? (sw >> 16) : (sw & 0xFFFFu);
        return dequant8_scaled(w.q[j][2 * bb], w.q[j][2 * bb + 1], as_h2(hb | (hb << 16)), 0x64646464u);
    }
}

// token rows of one 128-k chunk -> LDS (fp16; 16-byte piece c of row r at c ^ (r & 15))
template <typename XT, int NTH = 256>
struct RowChunk {
    static constexpr int NP = 1024 / NTH;
    XChunk<XT> v[NP];
    __device__ __forceinline__ void load(const XT* base, int ld, int nrows, int k0) {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int piece = (int)threadIdx.x + NTH * j, row = piece >> 4, ch = piece & 15;
            v[j].load(base + (size_t)min(row, nrows - 1) * ld + k0 + 8 * ch);
        }
    }
    __device__ __forceinline__ void store(uint4 (*dst)[kKC / 8]) const {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int piece = (int)threadIdx.x + NTH * j, row = piece >> 4, ch = piece & 15;
            dst[row][ch ^ (row & 15)] = __builtin_bit_cast(uint4, v[j].cvt());
        }
    }
};

template <int WFMT, typename XT, int NCH, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(3))) void ffn_gateup_tok64(const XT* __restrict__ x, int T, int d, int f, int k, int E,
                                                        const void* const* __restrict__ expert_ptrs,
                                                        const uint8_t* __restrict__ shared_blob,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ sorted_idx,
                                                        const int32_t* __restrict__ active, _Float16* __restrict__ h) {
    constexpr int TPC = StripChunk<WFMT>::TPC;
    __shared__ uint4 xs[2][kTok64][kKC / 8];
    __shared__ _Float16 hv_s[NW][kTok64][16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_groups = f / (16 * NW);
    const int a = blockIdx.x / n_groups, strip = (blockIdx.x % n_groups) * NW + wave;
    RowChunk<XT, 64 * NW> xr;
    xr.load(x, d, T, 0);
    const int n_active = active[0];
    const int e_raw = active[1 + min(a, E - 1)];
    const int e_c = min(max(e_raw, 0), E - 1);
    const uint8_t* pe = (const uint8_t*)expert_ptrs[e_c];
    const int ce = counts[e_c], oe = offsets[e_c];
    const bool routed = a < n_active;
    const uint8_t* blob = routed ? pe : (a == n_active ? shared_blob : nullptr);
    if (blob == nullptr) return;  // past the last slot, or no weights behind this expert (uniform per workgroup)
    const int c = routed ? ce : T, p0 = routed ? oe : T * k;
    const ExpertLayout L = expert_layout(WFMT, d, f);
    const __amdgpu_buffer_rsrc_t wr = buf_rsrc(blob, (uint32_t)L.total);
    const __amdgpu_buffer_rsrc_t ir = buf_rsrc(sorted_idx, routed ? (uint32_t)(T * k * 4) : 0u);
    // token of each of the slot's first 64 rows (routed) or the row itself (shared)
    const int slot_of = __builtin_amdgcn_raw_buffer_load_b32(ir, (p0 + min(lane, max(c - 1, 0))) * 4, 0, 0);
    const uint32_t tile0 = (uint32_t)strip * (uint32_t)(NCH * TPC);
    StripChunk<WFMT> wg[NCH], wu[NCH];
#pragma unroll
    for (int i = 0; i < kPipe64 && i < NCH; ++i) {
        load_strip_chunk<WFMT>(wg[i], wr, (uint32_t)L.g.qoff, (uint32_t)L.g.soff, tile0 + i * TPC, lane);
        load_strip_chunk<WFMT>(wu[i], wr, (uint32_t)L.u.qoff, (uint32_t)L.u.soff, tile0 + i * TPC, lane);
    }
    xr.store(xs[0]);
    __syncthreads();
    uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, magic = 0x64006400u;
    asm volatile("" : "+s"(mlo), "+s"(mhi), "+v"(magic));
    float4v accg[4], accu[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) accg[mt] = accu[mt] = float4v{0, 0, 0, 0};
    const int rsel = lane & 15;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        if (i + 1 < NCH) xr.load(x, d, T, (i + 1) * kKC);
        if (i + kPipe64 < NCH) {
            load_strip_chunk<WFMT>(wg[i + kPipe64], wr, (uint32_t)L.g.qoff, (uint32_t)L.g.soff, tile0 + (i + kPipe64) * TPC, lane);
            load_strip_chunk<WFMT>(wu[i + kPipe64], wr, (uint32_t)L.u.qoff, (uint32_t)L.u.soff, tile0 + (i + kPipe64) * TPC, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const half8 Bg = strip_block<WFMT>(wg[i], b, mlo, mhi, magic);
            const half8 Bu = strip_block<WFMT>(wu[i], b, mlo, mhi, magic);
            const int ch = 4 * b + (lane >> 4);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int row = 16 * mt + rsel;
                const half8 A = __builtin_bit_cast(half8, xs[i & 1][row][ch ^ (row & 15)]);
                accg[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bg, accg[mt], 0, 0, 0);
                accu[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bu, accu[mt], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < NCH) {
            xr.store(xs[(i + 1) & 1]);
            __syncthreads();
        }
    }
    // h = silu(g) * u by token, through LDS, then to every row of the slot
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) hv_s[wave][16 * mt + 4 * (lane >> 4) + r][lane & 15] = (_Float16)(silu_f(accg[mt][r]) * accu[mt][r]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    const int col = strip * 16 + (lane & 15);
    const int tok_lane = routed ? slot_of / k : lane;  // token of row `lane` of the slot
    for (int m0 = 0; m0 < c; m0 += 4) {
        const int m = m0 + (lane >> 4);
        int t;
        if (m < 64) t = __shfl(tok_lane, m);
        else t = routed ? sorted_idx[p0 + min(m, c - 1)] / k : m;
        if (m < c) h[(size_t)(p0 + m) * f + col] = hv_s[wave][t][lane & 15];
    }
}

template <int WFMT, typename YT, int NCH>
__global__ __launch_bounds__(256) void ffn_down_tok64(const _Float16* __restrict__ h, int T, int d, int f, int k,
                                                      int E, const void* const* __restrict__ expert_ptrs,
                                                      const uint8_t* __restrict__ shared_blob,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ active, YT* __restrict__ y_perm,
                                                      float* __restrict__ y_shared) {
    constexpr int TPC = StripChunk<WFMT>::TPC;
    __shared__ uint4 hs[2][kTok64][kKC / 8];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_groups = d / 64;
    const int a = blockIdx.x / n_groups, strip = (blockIdx.x % n_groups) * 4 + wave;
    const int n_active = active[0];
    const int e_raw = active[1 + min(a, E - 1)];
    const int e_c = min(max(e_raw, 0), E - 1);
    const uint8_t* pe = (const uint8_t*)expert_ptrs[e_c];
    const int ce = counts[e_c], oe = offsets[e_c];
    const bool routed = a < n_active;
    const uint8_t* blob = routed ? pe : (a == n_active ? shared_blob : nullptr);
    if (blob == nullptr) return;
    const int c = routed ? ce : T, p0 = routed ? oe : T * k;
    if (c <= 0) return;
    const ExpertLayout L = expert_layout(WFMT, d, f);
    const __amdgpu_buffer_rsrc_t wr = buf_rsrc(blob, (uint32_t)L.total);
    const uint32_t tile0 = (uint32_t)strip * (uint32_t)(NCH * TPC);
    uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, magic = 0x64006400u;
    asm volatile("" : "+s"(mlo), "+s"(mhi), "+v"(magic));
    const int rsel = lane & 15;
    const int col = strip * 16 + (lane & 15);
    // passes of 64 slot rows (more than 64 only when a token lists an expert twice)
    for (int m0 = 0; m0 < c; m0 += kTok64) {
        const int nr = min(kTok64, c - m0);
        const _Float16* hb = h + (size_t)(p0 + m0) * f;
        RowChunk<_Float16> hr;
        hr.load(hb, f, nr, 0);
        StripChunk<WFMT> w[NCH];
#pragma unroll
        for (int i = 0; i < kPipe && i < NCH; ++i)
            load_strip_chunk<WFMT>(w[i], wr, (uint32_t)L.dn.qoff, (uint32_t)L.dn.soff, tile0 + i * TPC, lane);
        if (m0 > 0) __syncthreads();  // the previous pass no longer reads the staging buffers
        hr.store(hs[0]);
        __syncthreads();
        float4v acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = float4v{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            if (i + 1 < NCH) hr.load(hb, f, nr, (i + 1) * kKC);
            if (i + kPipe < NCH)
                load_strip_chunk<WFMT>(w[i + kPipe], wr, (uint32_t)L.dn.qoff, (uint32_t)L.dn.soff, tile0 + (i + kPipe) * TPC, lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const half8 Bw = strip_block<WFMT>(w[i], b, mlo, mhi, magic);
                const int ch = 4 * b + (lane >> 4);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {  // all four m-tiles: rows past the slot repeat its last row
                    const int row = 16 * mt + rsel;
                    const half8 A = __builtin_bit_cast(half8, hs[i & 1][row][ch ^ (row & 15)]);
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bw, acc[mt], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);  // one block's A fragments live at a time
            }
            __builtin_amdgcn_sched_barrier(0);
            if (i + 1 < NCH) {
                hr.store(hs[(i + 1) & 1]);
                __syncthreads();
            }
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * mt + 4 * (lane >> 4) + r;
                if (m >= nr) continue;
                if (routed) y_perm[(size_t)(p0 + m0 + m) * d + col] = (YT)acc[mt][r];
                else y_shared[(size_t)(m0 + m) * d + col] = acc[mt][r];
            }
    }
}

// launchers: grid = (slots) x (row groups); false when the shape has no instance
template <int WFMT, typename XT>
static bool launch_gateup_tok64(const moe_ffn_args* a, _Float16* h, int slots, hipStream_t s) {
    if (a->d % kKC || a->f % 64) return false;
    // eight wavefronts (128 rows of f) per workgroup halve the token conversion
    // work when the grid is large; small grids keep four for parallelism
    const bool wide = a->f % 128 == 0 && (long)slots * (a->f / 64) >= 256;
    const dim3 grid((unsigned)(slots * (a->f / (wide ? 128 : 64))));
#define MOE_GU64(NCH)                                                                                                   \
    if (wide)                                                                                                           \
        ffn_gateup_tok64<WFMT, XT, NCH, 8><<<grid, 512, 0, s>>>((const XT*)a->x, a->T, a->d, a->f, a->k, a->E,          \
                                                                a->expert_ptrs, (const uint8_t*)a->shared_blob,        \
                                                                a->counts, a->offsets, a->sorted_idx, a->active, h);   \
    else                                                                                                                \
        ffn_gateup_tok64<WFMT, XT, NCH, 4><<<grid, 256, 0, s>>>((const XT*)a->x, a->T, a->d, a->f, a->k, a->E,          \
                                                                a->expert_ptrs, (const uint8_t*)a->shared_blob,        \
                                                                a->counts, a->offsets, a->sorted_idx, a->active, h)
    switch (a->d / kKC) {
    case 1: MOE_GU64(1); return true;
    case 2: MOE_GU64(2); return true;
    case 4: MOE_GU64(4); return true;
    case 8: MOE_GU64(8); return true;
    case 16: MOE_GU64(16); return true;
    case 32: MOE_GU64(32); return true;
    default: return false;
    }
#undef MOE_GU64
}

template <int WFMT, typename YT>
static bool launch_down_tok64(const moe_ffn_args* a, const _Float16* h, int slots, hipStream_t s) {
    if (a->f % kKC || a->d % 64) return false;
    const dim3 grid((unsigned)(slots * (a->d / 64)));
#define MOE_DN64(NCH)                                                                                             \
    ffn_down_tok64<WFMT, YT, NCH><<<grid, 256, 0, s>>>(h, a->T, a->d, a->f, a->k, a->E, a->expert_ptrs,         \
                                                       (const uint8_t*)a->shared_blob, a->counts, a->offsets,    \
                                                       a->active, (YT*)a->y_perm, a->y_shared)
    switch (a->f / kKC) {
    case 1: MOE_DN64(1); return true;
    case 2: MOE_DN64(2); return true;
    case 3: MOE_DN64(3); return true;
    case 4: MOE_DN64(4); return true;
    case 6: MOE_DN64(6); return true;
    case 8: MOE_DN64(8); return true;
    case 12: MOE_DN64(12); return true;
    case 16: MOE_DN64(16); return true;
    default: return false;
    }
#undef MOE_DN64
}

template <int WFMT, typename XT>
static int run_float(const moe_ffn_args* a, const Workspace& w, hipStream_t s) {
    const int max_active = a->E < a->T * a->k ? a->E : a->T * a->k;
    const int slots = max_active + (a->shared_blob ? 1 : 0);
    const int rows_lds = std::min(16, a->T);
    _Float16* h = reinterpret_cast<_Float16*>(w.h);
    int dev = 0, n_cu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    const int g1 = (int)std::min<long>((long)slots * (a->f / 16), (long)n_cu * 64);
    const size_t lds1 = std::max<size_t>((size_t)rows_lds * a->d * sizeof(_Float16), 4 * 2 * 4 * 64 * sizeof(float));
    // the general kernels (T > 64) stage 16 rows of d (gate/up) or f (down) fp16 values in LDS
    if (a->T > kTok64 && (size_t)rows_lds * std::max(a->d, a->f) * 2 > 64 * 1024) return MOE_ERR_UNSUPPORTED;
    if (a->phase != 2) {
        // token-dense kernel for small int4 batches; the token tile of d fp16 values per token fits in LDS
        const bool tok16 = WFMT == MOE_WFMT_I4B32 && a->T <= kTokMax && (size_t)a->T * a->d * 2 <= 64 * 1024 &&
                           (a->d & (a->d - 1)) == 0;
        const bool tok64 = !tok16 && a->T <= kTok64;
        if (!(tok16 && launch_gateup_tok16<XT>(a, h, slots, s)) &&
            !(tok64 && launch_gateup_tok64<WFMT, XT>(a, h, slots, s))) {
            // the general kernel stages 16 activation rows of d (fp16) in LDS
            if ((size_t)rows_lds * a->d * 2 > 64 * 1024) return MOE_ERR_UNSUPPORTED;
            ffn_float_gateup<WFMT, XT><<<g1, 256, lds1, s>>>((const XT*)a->x, a->T, a->d, a->f, a->k, a->expert_ptrs,
                                                             (const uint8_t*)a->shared_blob, a->counts, a->offsets,
                                                             a->sorted_idx, a->active, h);
        }
        const int rc = check_launch();
        if (rc || a->phase == 1) return rc;
    }
    const int g2 = (int)std::min<long>((long)slots * (a->d / 64), (long)n_cu * 64);
    const size_t lds2 = (size_t)rows_lds * a->f * sizeof(_Float16);
    // every slot has at most T <= 16 rows: one wavefront per 16 output rows
    const bool tok16 = WFMT == MOE_WFMT_I4B32 && a->T <= kTokMax && (size_t)kTokMax * a->f * 2 <= 64 * 1024;
    const bool tok64 = !tok16 && a->T <= kTok64;
    if (a->y_dtype == MOE_DT_F32) {
        if (!(tok16 && launch_down_tok16<float>(a, h, slots, s)) && !(tok64 && launch_down_tok64<WFMT, float>(a, h, slots, s))) {
            if (lds2 > 64 * 1024) return MOE_ERR_UNSUPPORTED;
            ffn_float_down<WFMT, float><<<g2, 256, lds2, s>>>(h, a->T, a->d, a->f, a->k, a->expert_ptrs,
                                                              (const uint8_t*)a->shared_blob, a->counts, a->offsets,
                                                              a->active, (float*)a->y_perm, a->y_shared);
        }
    } else {
        if (!(tok16 && launch_down_tok16<_Float16>(a, h, slots, s)) &&
            !(tok64 && launch_down_tok64<WFMT, _Float16>(a, h, slots, s))) {
            if (lds2 > 64 * 1024) return MOE_ERR_UNSUPPORTED;
            ffn_float_down<WFMT, _Float16><<<g2, 256, lds2, s>>>(h, a->T, a->d, a->f, a->k, a->expert_ptrs,
                                                                 (const uint8_t*)a->shared_blob, a->counts, a->offsets,
                                                                 a->active, (_Float16*)a->y_perm, a->y_shared);
        }
    }
    return check_launch();
}

int launch_ffn_float(const moe_ffn_args* a, const Workspace& w, hipStream_t s) {
    if (a->f / 8 < 16 || a->d / 8 < 16) return MOE_ERR_UNSUPPORTED;
    if (a->wfmt == MOE_WFMT_I4B32)
        return a->x_dtype == MOE_DT_F32 ? run_float<MOE_WFMT_I4B32, float>(a, w, s)
                                        : run_float<MOE_WFMT_I4B32, uint16_t>(a, w, s);
    return a->x_dtype == MOE_DT_F32 ? run_float<MOE_WFMT_I8B32, float>(a, w, s)
                                    : run_float<MOE_WFMT_I8B32, uint16_t>(a, w, s);
}

}  // namespace moe

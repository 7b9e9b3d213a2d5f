// Grouped SwiGLU expert FFN, int8-activation mode (prefill chunks).
//
// Per expert, the tokens routed to it form a dense M x K tile (about 160 rows
// for an 8,192-token chunk over 512 experts with top-10).  The Strata pages
// report moving expert matmuls to an int8 tensor-core kernel that needs no
// dequantisation ("Strata benchmarks", prefill optimisation table).
//
// Gate/up runs on int8 matrix cores: v_mfma_i32_32x32x32_i8, one instruction
// per 32-wide quantisation block (A = 32 tokens x 32 k, B = 32 k x 32 weight
// rows); the int4 weights become int8 while they are staged in LDS.  Block
// sums are exact integers |P| < 2^22 (the int4 kernel stages the quants as
// 16 q and the scales as s / 16; 16 |P| <= 16 * 32 * 127 * 8 is still below
// 2^22).  The MFMA accumulator is seeded with the bit pattern of 1.5 * 2^23,
// so the int32 result read as fp32 is exactly 1.5 * 2^23 + P.  With the
// weight row's block scale sw constant per lane, t = fma(D, sw,
// -1.5 * 2^23 * sw) = sw * P (one rounding; the constant is exact), then
// acc += sx * t with the token's block scale: two VALU operations per output
// and block.  h = silu(g) * u is then requantised to int8 per 32 features
// (scale amax / 127), as the method defines; exact block sums keep those
// codes equal to the definition's except at rounding ties.
//
// The int8 down projection's result feeds no further quantisation.  With int4
// weights it runs on v_mfma_f32_32x32x16_f16 over fp16 operands holding the
// dequantised values (the requantised h codes times their scale, the int4
// weights times theirs, each rounded once to fp16), with no per-block
// epilogue: on this chip the two-sided block-scale epilogue, not the matrix
// core, bounds an exact int8 product.  With int8 weights both projections use
// the exact int8 form (kernels ffn_q8_gateup / ffn_q8_down below).
#include <type_traits>

#include "common.hpp"
#include "wave.hpp"

namespace moe {

constexpr int kMG = 128;        // tokens per tile (4 m-tiles of 32, one per wavefront)
constexpr int kKC = 256;        // k per LDS chunk (8 blocks)
constexpr int kRows = 128;      // weight rows per workgroup
constexpr int kLdsRow = kKC + 16;  // padded int8 row stride
constexpr uint32_t kMagicBits = 0x4B400000u;  // 1.5 * 2^23
constexpr float kMagic = 12582912.0f;

size_t q8_tile_capacity(int T, int k, int E) {
    return (size_t)E + (size_t)T * k / kMG + (size_t)T / kMG + 4;
}

struct Q8Smem {
    int8_t w[kRows][kLdsRow];          // staged weights, signed int8
    float sw[kKC / 32][kRows];         // weight block scales
    float sa[kKC / 32][kMG];           // activation block scales of the tile's tokens
};

// Plan: tile list of (slot, m0) over the active experts (slot = expert id) and
// the shared expert (slot = E), kMG tokens per tile.  One workgroup.
__global__ __launch_bounds__(1024) void q8_plan(const int32_t* __restrict__ counts,
                                                const int32_t* __restrict__ active, int E, int T, int has_shared,
                                                int2* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
    __shared__ int32_t sc[1024];
    const int a = threadIdx.x;
    const int n_active = active[0];
    int e = -1, c = 0, nt = 0;
    if (a < n_active) {
        e = active[1 + a];
        c = counts[e];
        nt = (c + kMG - 1) / kMG;
    }
    sc[a] = nt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int v = a >= off ? sc[a - off] : 0;
        __syncthreads();
        sc[a] += v;
        __syncthreads();
    }
    const int start = sc[a] - nt;
    for (int i = 0; i < nt; ++i) tiles[start + i] = make_int2(e, i * kMG);
    if (a == 1023) {
        int total = sc[1023];
        if (has_shared) {
            const int ns = (T + kMG - 1) / kMG;
            for (int i = 0; i < ns; ++i) tiles[total + i] = make_int2(E, i * kMG);
            total += ns;
        }
        n_tiles[0] = total;
    }
}

// Stage rows [row0 + 16*s .. +16) for strips s of `mats` (strip list) and k-chunk kc into LDS.
// `ntile` packed tiles (<= kKC / k-per-tile) starting at packed tile kt0.
template <int WFMT>
__device__ __forceinline__ void stage_chunk(Q8Smem& S, const uint8_t* const* qbase, const uint8_t* const* sbase,
                                            const int* strip_ids, int nkt_total, int kt0, int ntile) {
    constexpr int KPT = WFMT == MOE_WFMT_I4B32 ? 128 : 64;  // k per packed tile
    constexpr int NB = KPT / 32;
    constexpr int STB = NB * 32;
    // quants: 8 strips x ntile tiles x 64 lanes, 16 bytes each
    for (int task = threadIdx.x; task < 8 * ntile * 64; task += 256) {
        const int s = task / (ntile * 64), rem = task % (ntile * 64), tl = rem / 64, ll = rem % 64;
        const uint4v w = *reinterpret_cast<const uint4v*>(qbase[s] + ((size_t)strip_ids[s] * nkt_total + kt0 + tl) * 1024 +
                                                          (size_t)ll * 16);
        const int row = s * 16 + (ll & 15);
        const int kq = 8 * (ll >> 4);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            uint32_t w0, w1;
            if constexpr (WFMT == MOE_WFMT_I4B32) {
                const uint32_t v = w[b];
                const uint32_t lo = v & 0x0F0F0F0Fu;         // bytes: k0 k4 k1 k5
                const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;  // bytes: k2 k6 k3 k7
                w0 = (lo & 0xFFu) | ((lo >> 8) & 0xFF00u) | ((hi & 0xFFu) << 16) | ((hi << 8) & 0xFF000000u);
                w1 = ((lo >> 8) & 0xFFu) | ((lo >> 16) & 0xFF00u) | ((hi << 8) & 0xFF0000u) | (hi & 0xFF000000u);
                // offset-binary nibble u -> signed byte u - 8 (no carries: u + 0x78 <= 0x87)
                w0 = (w0 + 0x78787878u) ^ 0x80808080u;
                w1 = (w1 + 0x78787878u) ^ 0x80808080u;
            } else {
                w0 = w[2 * b] ^ 0x80808080u;
                w1 = w[2 * b + 1] ^ 0x80808080u;
            }
            *reinterpret_cast<uint2*>(&S.w[row][(tl * NB + b) * 32 + kq]) = make_uint2(w0, w1);
        }
    }
    // scales: 8 strips x TPC tiles x 16 rows, NB fp16 each
    for (int task = threadIdx.x; task < 8 * ntile * 16; task += 256) {
        const int s = task / (ntile * 16), rem = task % (ntile * 16), tl = rem / 16, rr = rem % 16;
        const _Float16* sp = reinterpret_cast<const _Float16*>(sbase[s] + ((size_t)strip_ids[s] * nkt_total + kt0 + tl) * STB) + rr * NB;
#pragma unroll
        for (int b = 0; b < NB; ++b) S.sw[tl * NB + b][s * 16 + rr] = (float)sp[b];
    }
}

// One k-chunk of MFMA work for one wavefront: 32 tokens x 4 n-tiles of 32 rows.
// arow: this lane's A-operand row (int8 activations, chunk-relative k = 0),
// valid: whether the row exists; sa rows are token rows of the wavefront's m-tile.
__device__ __forceinline__ void mma_chunk(const Q8Smem& S, const int8_t* arow, bool valid, int mtile, int nblk,
                                          float16v (&acc)[4]) {
    const int lane = threadIdx.x & 63;
    const int16v cmagic = {(int)kMagicBits, (int)kMagicBits, (int)kMagicBits, (int)kMagicBits,
                           (int)kMagicBits, (int)kMagicBits, (int)kMagicBits, (int)kMagicBits,
                           (int)kMagicBits, (int)kMagicBits, (int)kMagicBits, (int)kMagicBits,
                           (int)kMagicBits, (int)kMagicBits, (int)kMagicBits, (int)kMagicBits};
    for (int b = 0; b < nblk; ++b) {
        const int kk = b * 32 + 16 * (lane >> 5);
        const int4v A = valid ? *reinterpret_cast<const int4v*>(arow + kk) : int4v{0, 0, 0, 0};
        // activation scales of this lane's 16 token rows: 8*(r/4) + 4*(lane/32) + r%4
        float sa[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(&S.sa[b][mtile * 32 + 8 * q + 4 * (lane >> 5)]);
            sa[4 * q + 0] = v.x; sa[4 * q + 1] = v.y; sa[4 * q + 2] = v.z; sa[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int row = nt * 32 + (lane & 31);
            const int4v B = *reinterpret_cast<const int4v*>(&S.w[row][kk]);
            const int16v D = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, cmagic, 0, 0, 0);
            const float sw = S.sw[b][row];
            const float nc = -kMagic * sw;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float t = fmaf(__int_as_float(D[r]), sw, nc);
                acc[nt][r] = fmaf(t, sa[r], acc[nt][r]);
            }
        }
    }
}

__device__ __forceinline__ float silu_q(float z) { return z / (1.0f + expf(-z)); }

template <int WFMT>
__global__ __launch_bounds__(256) void ffn_q8_gateup(const int8_t* __restrict__ xq, const float* __restrict__ sx,
                                                     int T, int d, int f, int k, int E,
                                                     const void* const* __restrict__ expert_ptrs,
                                                     const uint8_t* __restrict__ shared_blob,
                                                     const int32_t* __restrict__ counts,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ sorted_idx,
                                                     const int2* __restrict__ tiles,
                                                     const int32_t* __restrict__ n_tiles_p, int8_t* __restrict__ hq,
                                                     float* __restrict__ hs) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Q8Smem& S = *reinterpret_cast<Q8Smem*>(smem_raw);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_fg = f / 64;
    const int n_items = n_tiles_p[0] * n_fg;
    const ExpertLayout L = expert_layout(WFMT, d, f);
    const int nkt = L.g.nkt;
    const int nb_d = d / 32;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int2 tl = tiles[item / n_fg];
        const int fg = item % n_fg;
        const bool routed = tl.x < E;
        const uint8_t* blob = routed ? (const uint8_t*)expert_ptrs[tl.x] : shared_blob;
        if (blob == nullptr) continue;  // no weights behind this expert (uniform per workgroup)
        const int c = routed ? counts[tl.x] : T;
        const int p0 = routed ? offsets[tl.x] : T * k;  // first h row of the slot
        const int m0 = tl.y;
        // this lane's A row (token) for the wavefront's m-tile
        const int m = m0 + wave * 32 + (lane & 31);
        const bool valid = m < c;
        const int tok = valid ? (routed ? sorted_idx[p0 + m] / k : m) : 0;
        const int8_t* xrow = xq + (size_t)tok * d;
        // scales of the tile's tokens, per chunk: staged below
        const uint8_t* qb[8];
        const uint8_t* sb[8];
        int sid[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const MatLayout& M = s < 4 ? L.g : L.u;
            qb[s] = blob + M.qoff;
            sb[s] = blob + M.soff;
            sid[s] = fg * 4 + (s & 3);
        }
        float16v acc[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nt][r] = 0.0f;
        constexpr int KPT = WFMT == MOE_WFMT_I4B32 ? 128 : 64;
        const int nkc = (d + kKC - 1) / kKC;
        for (int kc = 0; kc < nkc; ++kc) {
            const int nblk = min(kKC, d - kc * kKC) / 32;
            __syncthreads();
            stage_chunk<WFMT>(S, qb, sb, sid, nkt, kc * (kKC / KPT), nblk * 32 / KPT);
            for (int task = threadIdx.x; task < (kKC / 32) * kMG; task += 256) {
                const int b = task / kMG, mm = task % kMG;
                const int mt = m0 + mm;
                float v = 0.0f;
                if (mt < c && b < nblk) {
                    const int t = routed ? sorted_idx[p0 + mt] / k : mt;
                    v = sx[(size_t)t * nb_d + kc * (kKC / 32) + b];
                }
                S.sa[b][mm] = v;
            }
            __syncthreads();
            if (m0 + wave * 32 < c) mma_chunk(S, xrow + kc * kKC, valid, wave, nblk, acc);
        }
        // SwiGLU + int8 requantisation of h per (token, 32 features)
        if (m0 + wave * 32 < c) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {  // f-blocks fg*2 + half: gate n-tile half, up n-tile 2+half
                const int feat = fg * 64 + half * 32 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float hv = silu_q(acc[half][r]) * acc[2 + half][r];
                    float amax = fabsf(hv);
#pragma unroll
                    for (int off = 16; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
                    const float s = amax / 127.0f;
                    int q = 0;
                    if (s != 0.0f) q = (int)fminf(fmaxf(rintf(hv / s), -127.0f), 127.0f);
                    const int mrow = m0 + wave * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (mrow < c) {
                        const size_t hrow = (size_t)(p0 + mrow);
                        hq[hrow * f + feat] = (int8_t)q;
                        if ((lane & 31) == 0) hs[hrow * (f / 32) + fg * 2 + half] = s;
                    }
                }
            }
        }
    }
}

template <int WFMT, typename YT>
__global__ __launch_bounds__(256) void ffn_q8_down(const int8_t* __restrict__ hq, const float* __restrict__ hs,
                                                   int T, int d, int f, int k, int E,
                                                   const void* const* __restrict__ expert_ptrs,
                                                   const uint8_t* __restrict__ shared_blob,
                                                   const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ offsets,
                                                   const int2* __restrict__ tiles,
                                                   const int32_t* __restrict__ n_tiles_p, YT* __restrict__ y_perm,
                                                   float* __restrict__ y_shared) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Q8Smem& S = *reinterpret_cast<Q8Smem*>(smem_raw);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_og = d / kRows;
    const int n_items = n_tiles_p[0] * n_og;
    const ExpertLayout L = expert_layout(WFMT, d, f);
    const int nkt = L.dn.nkt;
    const int nb_f = f / 32;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int2 tl = tiles[item / n_og];
        const int og = item % n_og;
        const bool routed = tl.x < E;
        const uint8_t* blob = routed ? (const uint8_t*)expert_ptrs[tl.x] : shared_blob;
        if (blob == nullptr) continue;  // no weights behind this expert (uniform per workgroup)
        const int c = routed ? counts[tl.x] : T;
        const int p0 = routed ? offsets[tl.x] : T * k;
        const int m0 = tl.y;
        const int m = m0 + wave * 32 + (lane & 31);
        const bool valid = m < c;
        const int8_t* arow = hq + (size_t)(p0 + (valid ? m : 0)) * f;
        const uint8_t* qb[8];
        const uint8_t* sb[8];
        int sid[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            qb[s] = blob + L.dn.qoff;
            sb[s] = blob + L.dn.soff;
            sid[s] = og * 8 + s;
        }
        float16v acc[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nt][r] = 0.0f;
        const int nkc = (f + kKC - 1) / kKC;
        for (int kc = 0; kc < nkc; ++kc) {
            const int kbase = kc * kKC;
            const int nblk = min(kKC, f - kbase) / 32;
            constexpr int KPT = WFMT == MOE_WFMT_I4B32 ? 128 : 64;
            __syncthreads();
            stage_chunk<WFMT>(S, qb, sb, sid, nkt, kc * (kKC / KPT), nblk * 32 / KPT);
            for (int task = threadIdx.x; task < (kKC / 32) * kMG; task += 256) {
                const int b = task / kMG, mm = task % kMG;
                const int mt = m0 + mm;
                S.sa[b][mm] = (mt < c && b < nblk) ? hs[(size_t)(p0 + mt) * nb_f + kc * (kKC / 32) + b] : 0.0f;
            }
            __syncthreads();
            if (m0 + wave * 32 < c) mma_chunk(S, arow + kbase, valid, wave, nblk, acc);
        }
        if (m0 + wave * 32 < c) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int o = og * kRows + nt * 32 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int mrow = m0 + wave * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (mrow >= c) continue;
                    if (routed) y_perm[(size_t)(p0 + mrow) * d + o] = (YT)acc[nt][r];
                    else y_shared[(size_t)mrow * d + o] = acc[nt][r];
                }
            }
        }
    }
}

// ---- int4 weights: token tiles of up to 192 rows, 512-thread workgroups ------
// A work item is (tile, weight group): gate/up takes 128 features of f (their
// 128 gate rows and 128 up rows), down takes 256 output rows.  Eight
// wavefronts; wavefront w multiplies token tiles 3 (w / 4) .. +2 (32 tokens
// each) by the weight tiles of feature group w % 4, so the two wavefronts a
// SIMD holds (w and w + 4) cover all token tiles of one feature group and the
// SIMDs stay balanced whatever the tile's row count.  Per k-chunk the token
// rows, the weight rows and both sets of block scales are staged in LDS,
// double buffered: chunk c + 1 is read into registers while chunk c is
// multiplied, written to the other buffer afterwards, and one barrier per
// chunk separates the two.  Loads go through buffer resources with per-lane
// offsets computed once per work item.  The work items of one tile share
// blockIdx % 8, i.e. one XCD, whose L2 then serves the tile's token rows to
// all of them.
constexpr int kTM = 6;           // token tiles of 32 per tile (192 rows)
constexpr int kTR = kTM * 32;
constexpr int kPThreads = 512;
constexpr int kGUFeat = 128;     // features of f per gate/up work item (256 weight rows)
constexpr int kDNRows = 256;     // output rows per down work item

// 16-byte chunk c (0..7) of LDS row r is stored at position c ^ ((r >> 1) & 7):
// the sixteen rows read by one quarter-wavefront then hit sixteen distinct
// 16-byte bank groups of the 256 B the LDS serves per cycle.
__device__ __forceinline__ int chunk_swz(int r) { return (r >> 1) & 7; }

// Tiles of <= kTR rows, balanced per expert: tiles[i] = (e, m0, rows, p)
// with e the expert (-1 for the shared expert), m0 the tile's first row
// within the expert's rows and p = the tile's first row in the permuted
// order (offsets[e] + m0, or T k + m0 for the shared expert), and
// tile_blob[i] the expert's weights.  The FFN kernels then need one dependent
// load (the tile's token list) before their data instead of four (tile,
// active entry, expert pointer and offset, token list).  The shared
// expert's tiles (all T tokens, the fullest) come first.
__global__ __launch_bounds__(1024) void q8_tile_plan(const int32_t* __restrict__ counts,
                                                     const int32_t* __restrict__ active,
                                                     const int32_t* __restrict__ offsets,
                                                     const void* const* __restrict__ expert_ptrs,
                                                     const uint8_t* __restrict__ shared_blob, int T, int k,
                                                     int4* __restrict__ tiles, const uint8_t** __restrict__ tile_blob,
                                                     int32_t* __restrict__ n_tiles) {
    __shared__ int32_t sc[1024];
    constexpr int cap = kTR;
    const int a = threadIdx.x;
    const int n_active = active[0];
    const int e = a < n_active ? active[1 + a] : 0;
    const int c = a < n_active ? counts[e] : 0;
    const int nt = (c + cap - 1) / cap;
    sc[a] = nt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int v = a >= off ? sc[a - off] : 0;
        __syncthreads();
        sc[a] += v;
        __syncthreads();
    }
    const int ns = shared_blob ? (T + cap - 1) / cap : 0;
    const int start = ns + sc[a] - nt;
    if (nt > 0) {
        const int per = ((c + nt - 1) / nt + 15) / 16 * 16;
        const int oe = offsets[e];
        const uint8_t* blob = (const uint8_t*)expert_ptrs[e];
        for (int i = 0; i < nt; ++i) {
            tiles[start + i] = make_int4(e, i * per, min(per, c - i * per), oe + i * per);
            tile_blob[start + i] = blob;
        }
    }
    if (ns > 0) {
        const int per = ((T + ns - 1) / ns + 15) / 16 * 16;
        for (int i = a; i < ns; i += 1024) {
            tiles[i] = make_int4(-1, i * per, min(per, T - i * per), T * k + i * per);
            tile_blob[i] = shared_blob;
        }
    }
    if (a == 1023) n_tiles[0] = ns + sc[1023];
}

// One packed int4 word (offset binary u = q + 8, nibbles k0 k2 k4 k6 k1 k3 k5
// k7) -> eight int8 bytes in k order holding 16 q: u ^ 8 is the 4-bit two's
// complement of q, so with it in the high half of a byte the byte read as int8
// is exactly 16 q.  Five operations; the factor 16 is taken out of the weight
// block scale (exact in fp32).
__device__ __forceinline__ void int4_word_to_i8x16(uint32_t v, uint32_t& w0, uint32_t& w1) {
    const uint32_t hi = (v ^ 0x88888888u) & 0xF0F0F0F0u;         // bytes: k2 k6 k3 k7
    const uint32_t lo = ((v << 4) ^ 0x88888888u) & 0xF0F0F0F0u;  // bytes: k0 k4 k1 k5
    w0 = __builtin_amdgcn_perm(hi, lo, 0x06040200u);              // k0 k1 k2 k3
    w1 = __builtin_amdgcn_perm(hi, lo, 0x07050301u);              // k4 k5 k6 k7
}

// One packed int4 word -> four fp16 pairs (k0 k1) (k2 k3) (k4 k5) (k6 k7) of
// q * s: (w >> 4 j) & 0x000F000F puts the nibbles of k 2j and 2j + 1 in the
// two halves, 0x6400 makes each the fp16 1024 + u, subtracting 1032 gives q
// exactly, and the product with the fp16 block scale rounds once.
__device__ __forceinline__ void int4_word_to_f16(uint32_t v, half2v s2, uint32_t (&out)[4]) {
    const half2v off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const uint32_t b = ((v >> (4 * jj)) & 0x000F000Fu) | 0x64006400u;
        const half2v q = __builtin_bit_cast(half2v, b) + off;
        out[jj] = __builtin_bit_cast(uint32_t, q * s2);
    }
}

__device__ __forceinline__ float f16_bits_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(bits16 & 0xFFFFu));
}

struct GUStage {
    uint4 w[2 * kGUFeat][8];  // int8 16 q weight rows (gate 0..127, up 128..255), 128 k
    uint4 a[kTR][8];          // int8 token rows, 128 k
    float sw[4][2 * kGUFeat]; // weight block scales / 16
};
typedef float GUScales[4][kTR];  // token block scales of a stage

// One k-chunk (four 32-wide blocks) of a gate/up wavefront: NM token tiles
// (from mt0) times its gate and up weight tiles.  Within a block the token
// operand and scales of tile m + 1 are requested before the MFMAs and the
// epilogue of tile m; the block loop itself is not unrolled (that would not
// fit in the registers).
template <int NM>
__device__ __forceinline__ void gu_chunk(const GUStage& G, const GUScales& SA, int lane, int rg, int ru, int mt0,
                                         const int16v& cmagic, float16v (&acc)[3][2]) {
#pragma unroll 1
    for (int b = 0; b < 4; ++b) {
        const int kq = 2 * b + (lane >> 5);  // 16-byte chunk holding this lane's 16 k of block b
        int4v A[2];
        float sa[2][16];
        auto fetch = [&](int m) {
            const int row = (mt0 + m) * 32 + (lane & 31);
            A[m & 1] = __builtin_bit_cast(int4v, G.a[row][kq ^ chunk_swz(row)]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = *reinterpret_cast<const float4*>(&SA[b][(mt0 + m) * 32 + 8 * q + 4 * (lane >> 5)]);
                sa[m & 1][4 * q + 0] = v.x; sa[m & 1][4 * q + 1] = v.y;
                sa[m & 1][4 * q + 2] = v.z; sa[m & 1][4 * q + 3] = v.w;
            }
        };
        const int4v Bg = __builtin_bit_cast(int4v, G.w[rg][kq ^ chunk_swz(rg)]);
        const int4v Bu = __builtin_bit_cast(int4v, G.w[ru][kq ^ chunk_swz(ru)]);
        const float swg = G.sw[b][rg], swu = G.sw[b][ru];
        const float ncg = -kMagic * swg, ncu = -kMagic * swu;
        fetch(0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const int16v Dg = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[m & 1], Bg, cmagic, 0, 0, 0);
            const int16v Du = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[m & 1], Bu, cmagic, 0, 0, 0);
            if (m + 1 < NM) fetch(m + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float tg = fmaf(__int_as_float(Dg[r]), swg, ncg);
                const float tu = fmaf(__int_as_float(Du[r]), swu, ncu);
                acc[m][0][r] = fmaf(tg, sa[m & 1][r], acc[m][0][r]);
                acc[m][1][r] = fmaf(tu, sa[m & 1][r], acc[m][1][r]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

struct GURegs {
    uint4v w[2];   // packed int4 weights of two (strip, lane) units
    uint32_t ws;   // two fp16 weight block scales
};

// Gate/up, int8 activations x int4 weights on v_mfma_i32_32x32x32_i8, one
// instruction per 32-wide quantisation block.  The accumulator is seeded with
// the bits of 1.5 * 2^23, so the int32 result read as fp32 is exactly
// 1.5 * 2^23 + P for the block sum P (16 |P| < 2^22); t = fma(D, sw,
// -1.5 * 2^23 * sw) = sw * P with one rounding (the constant is exact: sw has
// an 11-bit significand), then acc = fma(t, sx, acc).  Then h = silu(g) * u is
// requantised per (token, 32 features) to int8 codes q with scale s = amax /
// 127, and the down projection's operand fp16(q * s) is written.
__global__ __launch_bounds__(kPThreads, 1) void ffn_i4_gateup(
    const int8_t* __restrict__ xq, const float* __restrict__ sx, int T, int d, int f, int k,
    const int32_t* __restrict__ sorted_idx, const int4* __restrict__ tiles,
    const uint8_t* const* __restrict__ tile_blob, const int32_t* __restrict__ n_tiles_p,
    _Float16* __restrict__ h_out) {
    // two LDS stages as separate variables: the compiler then knows that the
    // loads filling one do not alias the reads of the other.  The token scales,
    // read 12 times per block and wavefront, are over-aligned so that they are
    // placed first, within the 64 KiB reach of the LDS instructions' immediate
    // offsets (no address arithmetic per read)
    __shared__ GUStage S0, S1;
    __shared__ __align__(1024) GUScales SA0, SA1;
    __shared__ int32_t s_row[kTR];  // token of each tile row
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_groups = f / kGUFeat;
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int ti = (j / n_groups) * 8 + xcd, grp = j % n_groups;
    if (ti >= n_tiles_p[0]) return;
    const int4 tl = tiles[ti];
    const uint8_t* blob = tile_blob[ti];
    if (blob == nullptr) return;  // no weights behind this expert (uniform per workgroup)
    const bool routed = tl.x >= 0;
    const int m0 = tl.y, mc = tl.z, prow0 = tl.w;  // prow0: first row of the tile in the permuted order
    const int nmt = (mc + 31) >> 5;
    for (int i = threadIdx.x; i < kTR; i += kPThreads) {
        const int m = min(i, mc - 1);  // rows past the tile repeat its last row (results discarded)
        s_row[i] = routed ? sorted_idx[prow0 + m] / k : m0 + m;
    }
    const ExpertLayout L = expert_layout(MOE_WFMT_I4B32, d, f);
    const int nkt = d / 128;
    const int nb = d / 32;
    const __amdgpu_buffer_rsrc_t wr = buf_rsrc(blob, (uint32_t)L.total);
    const __amdgpu_buffer_rsrc_t xr = buf_rsrc(xq, (uint32_t)((size_t)T * d));
    const __amdgpu_buffer_rsrc_t sr = buf_rsrc(sx, (uint32_t)((size_t)T * nb * 4));
    __syncthreads();
    // per-lane load offsets (the chunk's offset is the wave-uniform soffset)
    uint32_t wq_off[2], xa_off[3];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = threadIdx.x + q * kPThreads, st = idx >> 6, ll = idx & 63;
        const MatLayout& M = st < 8 ? L.g : L.u;
        wq_off[q] = (uint32_t)(M.qoff + (size_t)(grp * 8 + (st & 7)) * nkt * 1024 + ll * 16);
    }
    uint32_t ws_off;
    {
        const int st = threadIdx.x >> 5;
        const MatLayout& M = st < 8 ? L.g : L.u;
        ws_off = (uint32_t)(M.soff + (size_t)(grp * 8 + (st & 7)) * nkt * 128 + (threadIdx.x & 31) * 4);
    }
    // token rows and their block scales go from global memory straight to LDS:
    // instruction q of wavefront w fills rows 8 (3 w + q) .. +7 (lane l: row
    // + l / 8, position l % 8, which holds chunk (l % 8) ^ swizzle of the row),
    // and wavefronts 0..5 fill the 768 block scales of the chunk ([4][192],
    // 64 per instruction)
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const int row = 8 * (3 * wave + q) + (lane >> 3);
        xa_off[q] = (uint32_t)s_row[row] * (uint32_t)d + (uint32_t)(((lane & 7) ^ chunk_swz(row)) * 16);
    }
    uint32_t sa_off[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = min(wave * 128 + q * 64 + lane, 4 * kTR - 1), bb = idx / kTR, row = idx % kTR;
        sa_off[q] = (uint32_t)s_row[row] * (uint32_t)nb * 4 + bb * 4;
    }
    auto dma_chunk = [&](GUStage& G, GUScales& SA, int c) {
#pragma unroll
        for (int q = 0; q < 3; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)&G.a[8 * (3 * wave + q)][0],
                                                     16, xa_off[q], c * 128, 0, 0);
        if (wave < 6) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    sr, (__attribute__((address_space(3))) void*)(&SA[0][0] + wave * 128 + q * 64), 4, sa_off[q],
                    c * 16, 0, 0);
        }
    };
    auto load_chunk = [&](GURegs& R, int c) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
            R.w[q] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(wr, wq_off[q], c * 1024, kBufNT));
        R.ws = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(wr, ws_off, c * 128, kBufNT);
    };
    auto store_chunk = [&](GUStage& G, const GURegs& R) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = threadIdx.x + q * kPThreads, st = idx >> 6, ll = idx & 63;
            const int row = st * 16 + (ll & 15), jq = ll >> 4;  // bytes 8 jq .. 8 jq + 7 of each block
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                uint32_t w0, w1;
                int4_word_to_i8x16(R.w[q][b], w0, w1);
                const int ch = 2 * b + (jq >> 1);
                reinterpret_cast<uint2*>(&G.w[row][ch ^ chunk_swz(row)])[jq & 1] = make_uint2(w0, w1);
            }
        }
        {
            const int st = threadIdx.x >> 5, wd = threadIdx.x & 31;
            const int row = st * 16 + (wd >> 1), b0 = 2 * (wd & 1);
            G.sw[b0][row] = 0.0625f * f16_bits_to_float(R.ws);
            G.sw[b0 + 1][row] = 0.0625f * f16_bits_to_float(R.ws >> 16);
        }
    };

    const int fg = wave & 3, mt0 = 3 * (wave >> 2);
    const int rg = fg * 32 + (lane & 31), ru = kGUFeat + fg * 32 + (lane & 31);  // this lane's gate / up weight row
    const int nkc = d / 128;
    // The wavefront's loop is instantiated for its number of token tiles (as in
    // the down kernel); every instance stages its share and meets the barriers.
    auto run = [&](auto nm_c) {
        constexpr int NM = decltype(nm_c)::value;
        // the magic accumulator seed is made opaque so that it stays in
        // registers instead of being rebuilt before every MFMA
        int16v cmagic;
#pragma unroll
        for (int r = 0; r < 16; ++r) cmagic[r] = (int)kMagicBits;
        asm volatile("" : "+v"(cmagic));
        float16v acc[3][2];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;
        GURegs R;
        load_chunk(R, 0);
        dma_chunk(S0, SA0, 0);
        store_chunk(S0, R);
        __syncthreads();  // also waits for this wavefront's LDS-bound loads
        // chunk c in S0 (even) or S1 (odd); chunk c + 1 is read into the other
        // stage during the products, which was last read before the previous
        // barrier
        for (int c = 0; c < nkc; c += 2) {
            if (c + 1 < nkc) {
                load_chunk(R, c + 1);
                dma_chunk(S1, SA1, c + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (NM > 0) gu_chunk<NM>(S0, SA0, lane, rg, ru, mt0, cmagic, acc);
            __builtin_amdgcn_sched_barrier(0);
            if (c + 1 < nkc) store_chunk(S1, R);
            __syncthreads();
            if (c + 1 < nkc) {
                if (c + 2 < nkc) {
                    load_chunk(R, c + 2);
                    dma_chunk(S0, SA0, c + 2);
                }
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (NM > 0) gu_chunk<NM>(S1, SA1, lane, rg, ru, mt0, cmagic, acc);
                __builtin_amdgcn_sched_barrier(0);
                if (c + 2 < nkc) store_chunk(S0, R);
                __syncthreads();
            }
        }
        // h = silu(g) * u, requantised per (token, 32 features of this
        // wavefront).  In the MFMA layout the 32 features of a token are the
        // lanes of one half-wavefront, so h first goes through LDS (the stages
        // are free after the last barrier): each wavefront writes its
        // [32 tokens][32 features] fp32 tile (rows padded by 16 bytes) and
        // reads it back as half rows, lane l holding features 16 (l & 1) .. +15
        // of token l / 2.  The block maximum is then 15 local maxima and one
        // with the neighbouring lane, the scale amax / 127 one division per
        // lane, and the 16 codes leave as two 16-byte row stores of fp16(q s).
        constexpr int HRB = 32 * 4 + 16;  // tile row pitch in bytes
        static_assert(kPThreads / 64 * 32 * HRB <= sizeof(GUStage), "h tiles exceed the stage");
        unsigned char* htile = reinterpret_cast<unsigned char*>(&S0) + wave * (32 * HRB);
        const int hrow = lane >> 1, hhalf = lane & 1;
        _Float16* hdst = h_out + (size_t)prow0 * f + grp * kGUFeat + fg * 32 + 16 * hhalf;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float g = acc[m][0][r];
                const float hv = g * acc[m][1][r] * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
                const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                *reinterpret_cast<float*>(htile + row * HRB + (lane & 31) * 4) = hv;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
            float v[16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 t = *reinterpret_cast<const float4*>(htile + hrow * HRB + hhalf * 64 + j * 16);
                v[4 * j + 0] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
            }
            float amax = fabsf(v[0]);
#pragma unroll
            for (int j = 1; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
            amax = fmaxf(amax, __uint_as_float(lane_xor<1>(__float_as_uint(amax))));
            const float sc = amax / 127.0f;
            const float inv = 127.0f * __builtin_amdgcn_rcpf(amax);
            uint32_t pk[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float q0 = 0.0f, q1 = 0.0f;
                if (sc != 0.0f) {
                    q0 = fminf(fmaxf(rintf(v[2 * j] * inv), -127.0f), 127.0f);
                    q1 = fminf(fmaxf(rintf(v[2 * j + 1] * inv), -127.0f), 127.0f);
                }
                const _Float16 h0 = (_Float16)(q0 * sc), h1 = (_Float16)(q1 * sc);
                pk[j] = (uint32_t)__builtin_bit_cast(unsigned short, h0) |
                        ((uint32_t)__builtin_bit_cast(unsigned short, h1) << 16);
            }
            const int trow = (mt0 + m) * 32 + hrow;
            if (trow < mc) {
                uint4* dst = reinterpret_cast<uint4*>(hdst + (size_t)trow * f);
                dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
                dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");  // the next tile reuses the buffer
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        }
    };
    switch (min(max(nmt - mt0, 0), 3)) {  // wave-uniform
        case 3: run(std::integral_constant<int, 3>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 1: run(std::integral_constant<int, 1>{}); break;
        default: run(std::integral_constant<int, 0>{}); break;
    }
}

struct DNStage {
    uint4 w[kDNRows][8];  // fp16 q * s weight rows, 64 k
    uint4 a[kTR][8];      // fp16 h rows, 64 k
};

struct DNRegs {
    uint2v w[2];   // packed int4 words of two (strip, lane) units
    uint32_t s[2]; // their two fp16 block scales
    uint4v a[3];   // three 16-byte pieces of h rows
};

// One k-chunk (four 16-wide MFMA steps) of a down wavefront: NM token tiles
// (from mt0) times its two weight tiles, as 4 NM steps pipelined by one: the
// LDS operands of step i + 1 are requested before the MFMAs of step i.
template <int NM>
__device__ __forceinline__ void dn_chunk(const DNStage& G, int lane, int r0, int r1, int mt0, float16v (&acc)[3][2]) {
    constexpr int NS = 4 * NM;
    half8 A[2], B0[2], B1[2];
    auto fetch_b = [&](int st) {
        const int kq = 2 * st + (lane >> 5);  // 16-byte chunk holding this lane's 8 k of step st
        B0[st & 1] = __builtin_bit_cast(half8, G.w[r0][kq ^ chunk_swz(r0)]);
        B1[st & 1] = __builtin_bit_cast(half8, G.w[r1][kq ^ chunk_swz(r1)]);
    };
    auto fetch_a = [&](int i) {
        const int st = i / NM, m = i % NM;
        const int kq = 2 * st + (lane >> 5);
        const int row = (mt0 + m) * 32 + (lane & 31);
        A[i & 1] = __builtin_bit_cast(half8, G.a[row][kq ^ chunk_swz(row)]);
    };
    fetch_b(0);
    fetch_a(0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int st = i / NM, m = i % NM;
        if (i + 1 < NS) {
            if ((i + 1) % NM == 0) fetch_b(st + 1);
            fetch_a(i + 1);
        }
        __builtin_amdgcn_sched_barrier(0);  // the reads of step i + 1 stay ahead of the MFMAs of step i
        acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i & 1], B0[st & 1], acc[m][0], 0, 0, 0);
        acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i & 1], B1[st & 1], acc[m][1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Bytes of one wavefront's [32][64] output tile of element type YT in LDS
// (rows padded by 16 bytes: the element writes of the two half-wavefronts,
// four rows apart, fall in different banks).
template <typename YT>
constexpr int dn_tile_bytes() { return 32 * (64 * (int)sizeof(YT) + 16); }

// Writes a wavefront's NM output tiles (token rows 32 (mt0 + m) .., the
// wavefront's 64 output columns) to dst[row * d + col] through its LDS tile:
// rows at or past mc are not written.
template <int NM, typename YT>
__device__ __forceinline__ void dn_write_tiles(unsigned char* tile, const float16v (&acc)[3][2], int lane, int mt0,
                                               int mc, YT* dst, int d) {
    constexpr int RB = 64 * (int)sizeof(YT) + 16;  // row pitch in bytes
    constexpr int PER_ROW = 64 * (int)sizeof(YT) / 16;  // 16-byte pieces per row
    constexpr int ROWS_PER = 64 / PER_ROW;              // rows covered by one wavefront read
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                *reinterpret_cast<YT*>(tile + row * RB + (n * 32 + (lane & 31)) * (int)sizeof(YT)) = (YT)acc[m][n][r];
            }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
        for (int i = 0; i < 32 / ROWS_PER; ++i) {
            const int row = i * ROWS_PER + lane / PER_ROW, pc = lane % PER_ROW;
            const uint4 v = *reinterpret_cast<const uint4*>(tile + row * RB + pc * 16);
            const int trow = (mt0 + m) * 32 + row;
            if (trow < mc) *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(dst + (size_t)trow * d) + pc * 16) = v;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");  // the next tile reuses the buffer
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    }
}

// Down projection on v_mfma_f32_32x32x16_f16 over operands that hold the
// dequantised values: fp16(q * s) of the int8 codes of h (written by the
// gate/up kernel) and fp16(q * s) of the int4 weights, built while the weight
// rows are staged in LDS.  Products accumulate in fp32 over all of f; nothing
// downstream is requantised, so the fp16 rounding of the two operands
// (2^-11 relative each) only adds to the output's error.
template <typename YT>
__global__ __launch_bounds__(kPThreads, 1) void ffn_i4_down(
    const _Float16* __restrict__ h, int T, int d, int f, int k, const int4* __restrict__ tiles,
    const uint8_t* const* __restrict__ tile_blob, const int32_t* __restrict__ n_tiles_p, YT* __restrict__ y_perm,
    float* __restrict__ y_shared) {
    __shared__ DNStage S[2];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_groups = (d + kDNRows - 1) / kDNRows;
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int ti = (j / n_groups) * 8 + xcd, grp = j % n_groups;
    if (ti >= n_tiles_p[0]) return;
    const int4 tl = tiles[ti];
    const uint8_t* blob = tile_blob[ti];
    if (blob == nullptr) return;
    const bool routed = tl.x >= 0;
    const int m0 = tl.y, mc = tl.z, prow0 = tl.w;  // prow0: first row of the tile in the permuted order
    const int nmt = (mc + 31) >> 5;
    const ExpertLayout L = expert_layout(MOE_WFMT_I4B32, d, f);
    const int nkt = f / 128;
    const int n_strips = d / 16;
    const __amdgpu_buffer_rsrc_t wr = buf_rsrc(blob, (uint32_t)L.total);
    const __amdgpu_buffer_rsrc_t hr = buf_rsrc(h, (uint32_t)(((size_t)T * k + T) * f * 2));
    uint32_t wq_off[2], ws_off[2], ha_off[3];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = threadIdx.x + q * kPThreads, st = idx >> 6, ll = idx & 63;
        const int strip = min(grp * 16 + st, n_strips - 1);  // strips past d repeat the last one (not written)
        wq_off[q] = (uint32_t)(L.dn.qoff + (size_t)strip * nkt * 1024 + ll * 16);
        ws_off[q] = (uint32_t)(L.dn.soff + (size_t)strip * nkt * 128 + (ll & 15) * 8);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const int idx = threadIdx.x + q * kPThreads, row = idx >> 3;
        ha_off[q] = (uint32_t)(prow0 + min(row, mc - 1)) * (uint32_t)f * 2 + (idx & 7) * 16;
    }
    // chunk c covers k = 64 c .. 64 c + 63: half (c & 1) of packed tile c >> 1
    auto load_chunk = [&](DNRegs& R, int c) {
        const int kt = c >> 1, hh = c & 1;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            R.w[q] = __builtin_bit_cast(uint2v, __builtin_amdgcn_raw_buffer_load_b64(wr, wq_off[q], kt * 1024 + hh * 8, kBufNT));
            R.s[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(wr, ws_off[q], kt * 128 + hh * 4, kBufNT);
        }
#pragma unroll
        for (int q = 0; q < 3; ++q)
            R.a[q] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(hr, ha_off[q], c * 128, 0));
    };
    auto store_chunk = [&](DNStage& G, const DNRegs& R) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = threadIdx.x + q * kPThreads, st = idx >> 6, ll = idx & 63;
            const int row = st * 16 + (ll & 15), jq = ll >> 4;
#pragma unroll
            for (int bl = 0; bl < 2; ++bl) {  // blocks 2 hh + bl: k_local = 32 bl + 8 jq .. +7
                const uint32_t sb = (R.s[q] >> (16 * bl)) & 0xFFFFu;
                const half2v s2 = __builtin_bit_cast(half2v, sb | (sb << 16));
                uint32_t o[4];
                int4_word_to_f16(R.w[q][bl], s2, o);
                const int ch = 4 * bl + jq;
                G.w[row][ch ^ chunk_swz(row)] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            const int idx = threadIdx.x + q * kPThreads, row = idx >> 3, ch = idx & 7;
            G.a[row][ch ^ chunk_swz(row)] = __builtin_bit_cast(uint4, R.a[q]);
        }
    };
    const int og = wave & 3, mt0 = 3 * (wave >> 2);
    const int r0 = og * 64 + (lane & 31), r1 = r0 + 32;  // this lane's two weight rows (output rows)
    const int nkc = f / 64;
    // The wavefront's loop is instantiated for its number of token tiles, so
    // that each instance is straight-line code (and the register allocation of
    // one does not constrain another).  Every instance stages its share of each
    // chunk and meets the same barriers.
    auto run = [&](auto nm_c) {
        constexpr int NM = decltype(nm_c)::value;
        float16v acc[3][2];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;
        // two chunks in flight: while chunk c is multiplied from one LDS
        // buffer, chunk c + 1 waits in registers to be written to the other and
        // chunk c + 2 is being read; one barrier per chunk
        DNRegs R0, R1;
        load_chunk(R0, 0);
        if (nkc > 1) load_chunk(R1, 1);
        store_chunk(S[0], R0);
        __syncthreads();
        if (nkc > 2) load_chunk(R0, 2);
        for (int c = 0; c < nkc; c += 2) {
            if constexpr (NM > 0) dn_chunk<NM>(S[0], lane, r0, r1, mt0, acc);  // chunk c
            if (c + 1 < nkc) store_chunk(S[1], R1);                          // chunk c + 1
            __syncthreads();
            if (c + 3 < nkc) load_chunk(R1, c + 3);
            if (c + 1 < nkc) {
                if constexpr (NM > 0) dn_chunk<NM>(S[1], lane, r0, r1, mt0, acc);  // chunk c + 1
                if (c + 2 < nkc) store_chunk(S[0], R0);                          // chunk c + 2
                __syncthreads();
                if (c + 4 < nkc) load_chunk(R0, c + 4);
            }
        }
        // The expert outputs leave through LDS: the stages are free after the
        // last barrier, and each wavefront owns a [32][64] tile of its own
        // there (its 32 token rows of tile m times its 64 output rows, rows
        // padded by 16 bytes).  Lane l holds rows 8 (r / 4) + 4 (l / 32) + r % 4
        // of columns n 32 + l % 32; written as elements, the tile is read back
        // as 16-byte pieces of rows, so every global store writes whole rows of
        // 64 consecutive outputs (128-bit stores instead of 2-byte ones).
        const int o0 = grp * kDNRows + og * 64;  // first output of this wavefront's columns
        if (o0 < d) {
            if (routed) dn_write_tiles<NM, YT>(reinterpret_cast<unsigned char*>(&S[0]) + wave * dn_tile_bytes<YT>(),
                                               acc, lane, mt0, mc, y_perm + (size_t)prow0 * d + o0, d);
            else dn_write_tiles<NM, float>(reinterpret_cast<unsigned char*>(&S[0]) + wave * dn_tile_bytes<float>(),
                                           acc, lane, mt0, mc, y_shared + (size_t)m0 * d + o0, d);
        }
    };
    switch (min(max(nmt - mt0, 0), 3)) {  // wave-uniform
        case 3: run(std::integral_constant<int, 3>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 1: run(std::integral_constant<int, 1>{}); break;
        default: run(std::integral_constant<int, 0>{}); break;
    }
}

template <int WFMT>
static int run_q8(const moe_ffn_args* a, const Workspace& w, hipStream_t s) {
    int2* tiles = reinterpret_cast<int2*>(w.tiles);
    const size_t cap = q8_tile_capacity(a->T, a->k, a->E);
    int32_t* n_tiles = w.tiles + 4 * cap;  // after the tile list (room for cap int4 or int2 entries)
    int8_t* hq = reinterpret_cast<int8_t*>(w.h);
    int rc;
    if constexpr (WFMT == MOE_WFMT_I4B32) {
        // tiles of <= 192 rows; work items of one tile on one XCD (grid rounded to 8 tiles)
        int4* t4 = reinterpret_cast<int4*>(w.tiles);
        _Float16* h16 = reinterpret_cast<_Float16*>(w.h);
        const long max_tiles = (long)std::min(a->E, a->T * a->k) + (long)a->T * a->k / kTR +
                               (a->shared_blob ? a->T / kTR + 1 : 0);
        const long gt = (max_tiles + 7) / 8 * 8;
        if (a->phase != 2) {
            q8_tile_plan<<<1, 1024, 0, s>>>(a->counts, a->active, a->offsets, a->expert_ptrs,
                                            (const uint8_t*)a->shared_blob, a->T, a->k, t4, w.tile_blob, n_tiles);
            rc = check_launch();
            if (rc) return rc;
            ffn_i4_gateup<<<(unsigned)(gt * (a->f / kGUFeat)), kPThreads, 0, s>>>(
                a->xq, a->sx, a->T, a->d, a->f, a->k, a->sorted_idx, t4, w.tile_blob, n_tiles, h16);
            rc = check_launch();
            if (rc || a->phase == 1) return rc;
        }
        const unsigned g2 = (unsigned)(gt * ((a->d + kDNRows - 1) / kDNRows));
        if (a->y_dtype == MOE_DT_F32)
            ffn_i4_down<float><<<g2, kPThreads, 0, s>>>(h16, a->T, a->d, a->f, a->k, t4, w.tile_blob, n_tiles,
                                                        (float*)a->y_perm, a->y_shared);
        else
            ffn_i4_down<_Float16><<<g2, kPThreads, 0, s>>>(h16, a->T, a->d, a->f, a->k, t4, w.tile_blob, n_tiles,
                                                           (_Float16*)a->y_perm, a->y_shared);
        return check_launch();
    }
    if (a->phase != 2) {
        q8_plan<<<1, 1024, 0, s>>>(a->counts, a->active, a->E, a->T, a->shared_blob ? 1 : 0, tiles, n_tiles);
        rc = check_launch();
        if (rc) return rc;
    }
    const long max_tiles = (long)std::min(a->E, a->T * a->k) + (long)a->T * a->k / kMG + (a->shared_blob ? a->T / kMG + 1 : 0);
    const size_t smem = sizeof(Q8Smem);
    const int g1 = (int)std::min<long>(max_tiles * (a->f / 64), 4096);
    if (a->phase != 2) {
        ffn_q8_gateup<WFMT><<<g1, 256, smem, s>>>(a->xq, a->sx, a->T, a->d, a->f, a->k, a->E, a->expert_ptrs,
                                                  (const uint8_t*)a->shared_blob, a->counts, a->offsets,
                                                  a->sorted_idx, tiles, n_tiles, hq, w.hs);
        rc = check_launch();
        if (rc || a->phase == 1) return rc;
    }
    const int g2 = (int)std::min<long>(max_tiles * (a->d / kRows), 4096);
    if (a->y_dtype == MOE_DT_F32)
        ffn_q8_down<WFMT, float><<<g2, 256, smem, s>>>(hq, w.hs, a->T, a->d, a->f, a->k, a->E, a->expert_ptrs,
                                                       (const uint8_t*)a->shared_blob, a->counts, a->offsets, tiles,
                                                       n_tiles, (float*)a->y_perm, a->y_shared);
    else
        ffn_q8_down<WFMT, _Float16><<<g2, 256, smem, s>>>(hq, w.hs, a->T, a->d, a->f, a->k, a->E, a->expert_ptrs,
                                                          (const uint8_t*)a->shared_blob, a->counts, a->offsets,
                                                          tiles, n_tiles, (_Float16*)a->y_perm, a->y_shared);
    return check_launch();
}

int launch_ffn_q8(const moe_ffn_args* a, const Workspace& w, hipStream_t s) {
    return a->wfmt == MOE_WFMT_I4B32 ? run_q8<MOE_WFMT_I4B32>(a, w, s) : run_q8<MOE_WFMT_I8B32>(a, w, s);
}

}  // namespace moe

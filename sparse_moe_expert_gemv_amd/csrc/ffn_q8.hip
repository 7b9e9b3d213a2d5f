// Grouped SwiGLU expert FFN, int8-activation mode (prefill chunks).
//
// Per expert, the tokens routed to it form a dense M x K tile (about 160 rows
// for an 8,192-token chunk over 512 experts with top-10), so both projections
// run on int8 matrix cores: v_mfma_i32_32x32x32_i8, one instruction per
// 32-wide quantisation block (A = 32 tokens x 32 k, B = 32 k x 32 weight
// rows).  The Strata pages report moving expert matmuls to an int8
// tensor-core kernel that needs no dequantisation ("Strata benchmarks",
// prefill optimisation table); here the int4 weights become int8 while they
// are staged in LDS, once per workgroup and k-chunk.
//
// Block sums are exact integers |P| < 2^22 (the tiled int4 kernels stage the
// quants as 16 q and the scales as s / 16; 16 |P| <= 16 * 32 * 127 * 8 is
// still below 2^22).  The MFMA accumulator is seeded
// with the bit pattern of 1.5 * 2^23, so the int32 result read as fp32 is
// exactly 1.5 * 2^23 + P.  With the weight row's block scale sw constant per
// lane, t = fma(D, sw, -1.5 * 2^23 * sw) = sw * P (one rounding; the constant
// is exact), then acc += sx * t with the token's block scale: two VALU
// operations per output and block.
//
// gate/up: a workgroup owns 64 features of f (gate rows + up rows = 128
// weight rows) for up to 128 tokens of one expert (one 32-token m-tile per
// wavefront), and writes h = silu(g) * u requantised to int8 per 32 features
// (per-token scale amax/127, ties-to-even), the down projection's A operand.
// down: a workgroup owns 128 output rows for the same token tile.
#include "common.hpp"

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

// ---- int4 weights: token tiles of up to 192 rows staged in LDS ---------------
// A work item is (tile, 128 weight rows): gate/up takes 64 features of f (their
// 64 gate rows and 64 up rows), down takes 128 output rows.  Every k-chunk of
// 128 (one packed int4 tile per strip, four 32-blocks) stages the tile's int8
// activation rows, the 128 weight rows (int4 -> int8) and both sets of block
// scales in LDS; wavefront w multiplies m-tiles 3 (w / 2) .. +2 (32 tokens
// each) by n-tiles (w & 1) and 2 + (w & 1) (gate and up rows of the same 32
// features, or two halves of the output rows), so SwiGLU needs no exchange.
// Work items of one tile share blockIdx % 8, i.e. one XCD and its L2, which
// then serves the tile's activation rows to all of them.  The next chunk is
// read into registers while the current one is multiplied.  The per-block
// arithmetic (magic-seeded int32 MFMA, t = sw * P, acc += sa * t, blocks in
// order) is the same as above, so the results are identical.
constexpr int kTM = 6;     // m-tiles of 32 tokens per tile (192 rows)
constexpr int kTKC = 128;  // k per chunk

struct TileSmem {
    uint4 a[kTM * 32][kTKC / 16];   // int8 rows, 16-byte chunk c of row r at (c ^ (r & 7))
    uint4 w[128][kTKC / 16];        // int8 weight rows, same swizzle
    float sa[kTKC / 32][kTM * 32];  // activation block scales
    float sw[kTKC / 32][128];       // weight block scales
};

// Tiles of <= kTM * 32 rows, balanced per expert: (slot, m0, rows, 0) with
// slot = position in the active list, or n_active for the shared expert.
__global__ __launch_bounds__(1024) void q8_tile_plan(const int32_t* __restrict__ counts,
                                                     const int32_t* __restrict__ active, int T, int has_shared,
                                                     int4* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
    __shared__ int32_t sc[1024];
    constexpr int cap = kTM * 32;
    const int a = threadIdx.x;
    const int n_active = active[0];
    const int c = a < n_active ? counts[active[1 + a]] : 0;
    const int nt = (c + cap - 1) / cap;
    sc[a] = nt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int v = a >= off ? sc[a - off] : 0;
        __syncthreads();
        sc[a] += v;
        __syncthreads();
    }
    const int start = sc[a] - nt;
    if (nt > 0) {
        const int per = ((c + nt - 1) / nt + 15) / 16 * 16;
        for (int i = 0; i < nt; ++i) tiles[start + i] = make_int4(a, i * per, min(per, c - i * per), 0);
    }
    if (a == 1023) {
        int total = sc[1023];
        if (has_shared) {  // the shared expert: slot n_active, all T tokens
            const int ns = (T + cap - 1) / cap;
            const int per = ((T + ns - 1) / ns + 15) / 16 * 16;
            for (int i = 0; i < ns; ++i) tiles[total + i] = make_int4(n_active, i * per, min(per, T - i * per), 0);
            total += ns;
        }
        n_tiles[0] = total;
    }
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

// MODE 0: gate/up, A = x (int8 per 32-block), output h requantised; MODE 1: down, A = h, output y
template <int MODE, typename YT>
__global__ __launch_bounds__(256) void ffn_q8_tiled(const int8_t* __restrict__ aq, const float* __restrict__ as_,
                                                    int T, int d, int f, int k,
                                                    const void* const* __restrict__ expert_ptrs,
                                                    const uint8_t* __restrict__ shared_blob,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ sorted_idx,
                                                    const int32_t* __restrict__ active,
                                                    const int4* __restrict__ tiles,
                                                    const int32_t* __restrict__ n_tiles_p, int8_t* __restrict__ hq,
                                                    float* __restrict__ hs, YT* __restrict__ y_perm,
                                                    float* __restrict__ y_shared) {
    __shared__ TileSmem S;
    __shared__ int32_t s_row[kTM * 32];  // source row of each tile row (token for gate/up, h row for down)
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K = MODE == 0 ? d : f;
    const int n_groups = MODE == 0 ? f / 64 : d / 128;
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int ti = (j / n_groups) * 8 + xcd, grp = j % n_groups;
    if (ti >= n_tiles_p[0]) return;
    const int4 tl = tiles[ti];
    const int n_active = active[0];
    const bool routed = tl.x < n_active;
    const int e = routed ? active[1 + tl.x] : -1;
    const uint8_t* blob = routed ? (const uint8_t*)expert_ptrs[e] : shared_blob;
    if (blob == nullptr) return;  // no weights behind this expert (uniform per workgroup)
    const int p0 = routed ? offsets[e] : T * k;
    const int m0 = tl.y, mc = tl.z;
    const int nmt = (mc + 31) >> 5;
    for (int i = threadIdx.x; i < kTM * 32; i += 256) {
        const int m = min(i, mc - 1);  // rows past the tile repeat its last row (results discarded)
        if (MODE == 0) s_row[i] = routed ? sorted_idx[p0 + m0 + m] / k : m0 + m;
        else s_row[i] = p0 + m0 + m;
    }
    const ExpertLayout L = expert_layout(MOE_WFMT_I4B32, d, f);
    const int nkt = K / 128;
    const int nb = K / 32;
    __syncthreads();
    // staging registers: activations 6 x 16 B, weights 2 lane words, weight scales 8 B, activation scales 16 B
    uint4v ra[6];
    uint4v rw[2];
    uint2v rsw = {0u, 0u};
    float4v rsa = {0.f, 0.f, 0.f, 0.f};
    auto load_chunk = [&](int c) {
#pragma unroll
        for (int q = 0; q < 6; ++q) {
            const int idx = threadIdx.x + q * 256, row = idx >> 3, ch = idx & 7;
            ra[q] = gload(reinterpret_cast<const uint4v*>(aq + (size_t)s_row[row] * K + c * kTKC) + ch);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = threadIdx.x + q * 256, st = idx >> 6, ll = idx & 63;
            const MatLayout& M = MODE == 0 ? (st < 4 ? L.g : L.u) : L.dn;
            const int strip = MODE == 0 ? grp * 4 + (st & 3) : grp * 8 + st;
            rw[q] = gload_nt(reinterpret_cast<const uint4v*>(blob + M.qoff + ((size_t)strip * nkt + c) * 1024) + ll);
        }
        if (threadIdx.x < 128) {
            const int st = threadIdx.x >> 4, rr = threadIdx.x & 15;
            const MatLayout& M = MODE == 0 ? (st < 4 ? L.g : L.u) : L.dn;
            const int strip = MODE == 0 ? grp * 4 + (st & 3) : grp * 8 + st;
            rsw = gload_nt(reinterpret_cast<const uint2v*>(blob + M.soff + ((size_t)strip * nkt + c) * 128 + rr * 8));
        }
        if (threadIdx.x < kTM * 32)
            rsa = gload(reinterpret_cast<const float4v*>(as_ + (size_t)s_row[threadIdx.x] * nb + c * 4));
    };
    auto store_chunk = [&]() {
#pragma unroll
        for (int q = 0; q < 6; ++q) {
            const int idx = threadIdx.x + q * 256, row = idx >> 3, ch = idx & 7;
            S.a[row][ch ^ (row & 7)] = __builtin_bit_cast(uint4, ra[q]);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = threadIdx.x + q * 256, st = idx >> 6, ll = idx & 63;
            const int row = st * 16 + (ll & 15), kq = ll >> 4;  // bytes 8 kq .. 8 kq + 7 of each block
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                uint32_t w0, w1;
                int4_word_to_i8x16(rw[q][b], w0, w1);
                const int ch = 2 * b + (kq >> 1);
                uint2* dst = reinterpret_cast<uint2*>(&S.w[row][ch ^ (row & 7)]) + (kq & 1);
                *dst = make_uint2(w0, w1);
            }
        }
        if (threadIdx.x < 128) {
            // fp16 scales by integer extraction (a bit cast of a vector element to a half pair is avoided),
            // divided by 16 for the staged quants 16 q
            const int row = threadIdx.x;
            const uint32_t w01 = rsw[0], w23 = rsw[1];
            S.sw[0][row] = 0.0625f * (float)__builtin_bit_cast(_Float16, (unsigned short)(w01 & 0xFFFFu));
            S.sw[1][row] = 0.0625f * (float)__builtin_bit_cast(_Float16, (unsigned short)(w01 >> 16));
            S.sw[2][row] = 0.0625f * (float)__builtin_bit_cast(_Float16, (unsigned short)(w23 & 0xFFFFu));
            S.sw[3][row] = 0.0625f * (float)__builtin_bit_cast(_Float16, (unsigned short)(w23 >> 16));
        }
        if (threadIdx.x < kTM * 32) {
#pragma unroll
            for (int b = 0; b < 4; ++b) S.sa[b][threadIdx.x] = rsa[b];
        }
    };
    const int mt0 = 3 * (wave >> 1);
    const int nt0 = MODE == 0 ? (wave & 1) : 2 * (wave & 1);
    const int nt1 = MODE == 0 ? 2 + (wave & 1) : 2 * (wave & 1) + 1;
    // the magic accumulator seed is made opaque so that it stays in registers
    // instead of being rebuilt before every MFMA
    int16v cmagic = {(int)kMagicBits, (int)kMagicBits, (int)kMagicBits, (int)kMagicBits,
                     (int)kMagicBits, (int)kMagicBits, (int)kMagicBits, (int)kMagicBits,
                     (int)kMagicBits, (int)kMagicBits, (int)kMagicBits, (int)kMagicBits,
                     (int)kMagicBits, (int)kMagicBits, (int)kMagicBits, (int)kMagicBits};
    asm volatile("" : "+v"(cmagic));
    float16v acc[3][2];
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;
    const int nkc = K / kTKC;
    load_chunk(0);
    for (int c = 0; c < nkc; ++c) {
        if (c > 0) __syncthreads();  // the previous chunk is no longer read
        store_chunk();
        __syncthreads();
        if (c + 1 < nkc) load_chunk(c + 1);  // the next chunk is in flight during the products
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int kq = 2 * b + (lane >> 5);  // 16-byte chunk holding this lane's 16 k of block b
            int4v B[2];
            float sw[2], nc[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int row = (n == 0 ? nt0 : nt1) * 32 + (lane & 31);
                B[n] = __builtin_bit_cast(int4v, S.w[row][kq ^ (row & 7)]);
                sw[n] = S.sw[b][row];
                nc[n] = -kMagic * sw[n];
            }
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                if (mt0 + m >= nmt) continue;
                const int row = (mt0 + m) * 32 + (lane & 31);
                const int4v A = __builtin_bit_cast(int4v, S.a[row][kq ^ (row & 7)]);
                float sa[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = *reinterpret_cast<const float4*>(&S.sa[b][(mt0 + m) * 32 + 8 * q + 4 * (lane >> 5)]);
                    sa[4 * q + 0] = v.x; sa[4 * q + 1] = v.y; sa[4 * q + 2] = v.z; sa[4 * q + 3] = v.w;
                }
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const int16v D = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B[n], cmagic, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float t = fmaf(__int_as_float(D[r]), sw[n], nc[n]);
                        acc[m][n][r] = fmaf(t, sa[r], acc[m][n][r]);
                    }
                }
            }
        }
    }
    if (MODE == 0) {
        // h = silu(g) * u, requantised per (token, 32 features of this wavefront)
        const int feat = grp * 64 + (wave & 1) * 32 + (lane & 31);
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            if (mt0 + m >= nmt) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float hv = silu_q(acc[m][0][r]) * acc[m][1][r];
                float amax = fabsf(hv);
#pragma unroll
                for (int off = 16; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
                const float sc = amax / 127.0f;
                int q = 0;
                if (sc != 0.0f) q = (int)fminf(fmaxf(rintf(hv / sc), -127.0f), 127.0f);
                const int mrow = (mt0 + m) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (mrow < mc) {
                    const size_t hrow = (size_t)(p0 + m0 + mrow);
                    hq[hrow * f + feat] = (int8_t)q;
                    if ((lane & 31) == 0) hs[hrow * (f / 32) + grp * 2 + (wave & 1)] = sc;
                }
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            if (mt0 + m >= nmt) continue;
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int o = grp * 128 + (n == 0 ? nt0 : nt1) * 32 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int mrow = (mt0 + m) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (mrow >= mc) continue;
                    if (routed) y_perm[(size_t)(p0 + m0 + mrow) * d + o] = (YT)acc[m][n][r];
                    else y_shared[(size_t)(m0 + mrow) * d + o] = acc[m][n][r];
                }
            }
        }
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
        const long max_tiles = (long)std::min(a->E, a->T * a->k) + (long)a->T * a->k / (kTM * 32) +
                               (a->shared_blob ? a->T / (kTM * 32) + 1 : 0);
        const long gt = (max_tiles + 7) / 8 * 8;
        if (a->phase != 2) {
            q8_tile_plan<<<1, 1024, 0, s>>>(a->counts, a->active, a->T, a->shared_blob ? 1 : 0, t4, n_tiles);
            rc = check_launch();
            if (rc) return rc;
            ffn_q8_tiled<0, float><<<(unsigned)(gt * (a->f / 64)), 256, 0, s>>>(
                a->xq, a->sx, a->T, a->d, a->f, a->k, a->expert_ptrs, (const uint8_t*)a->shared_blob, a->offsets,
                a->sorted_idx, a->active, t4, n_tiles, hq, w.hs, nullptr, nullptr);
            rc = check_launch();
            if (rc || a->phase == 1) return rc;
        }
        if (a->y_dtype == MOE_DT_F32)
            ffn_q8_tiled<1, float><<<(unsigned)(gt * (a->d / 128)), 256, 0, s>>>(
                hq, w.hs, a->T, a->d, a->f, a->k, a->expert_ptrs, (const uint8_t*)a->shared_blob, a->offsets,
                a->sorted_idx, a->active, t4, n_tiles, nullptr, nullptr, (float*)a->y_perm, a->y_shared);
        else
            ffn_q8_tiled<1, _Float16><<<(unsigned)(gt * (a->d / 128)), 256, 0, s>>>(
                hq, w.hs, a->T, a->d, a->f, a->k, a->expert_ptrs, (const uint8_t*)a->shared_blob, a->offsets,
                a->sorted_idx, a->active, t4, n_tiles, nullptr, nullptr, (_Float16*)a->y_perm, a->y_shared);
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

// Repacking of canonical block-32 expert blobs into the tiled layout read by
// the FFN kernels (layout documented in common.hpp).  One thread per
// (expert, matrix tile, lane): it moves that lane's 16 quant bytes and, for
// lanes 0..15, the row's scales of the tile.  Untimed preparation step.
#include "common.hpp"

namespace moe {

template <bool UNPACK>
__global__ void pack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int wfmt, int d, int f,
                            size_t blob_bytes, int lanes_g, int lanes_total) {
    const int gl = blockIdx.x * blockDim.x + threadIdx.x;
    if (gl >= lanes_total) return;
    const size_t eoff = (size_t)blockIdx.y * blob_bytes;
    const ExpertLayout P = expert_layout(wfmt, d, f);
    const CanonLayout C = canon_layout(wfmt, d, f);
    // which matrix: [0, lanes_g) gate, [lanes_g, 2 lanes_g) up, rest down
    int m, li;
    if (gl < lanes_g) { m = 0; li = gl; }
    else if (gl < 2 * lanes_g) { m = 1; li = gl - lanes_g; }
    else { m = 2; li = gl - 2 * lanes_g; }
    const MatLayout& M = m == 0 ? P.g : (m == 1 ? P.u : P.dn);
    const size_t cq = m == 0 ? C.qg : (m == 1 ? C.qu : C.qd);
    const size_t cs = m == 0 ? C.sg : (m == 1 ? C.su : C.sd);
    const int tile = li >> 6, lane = li & 63;  // tile = rs * nkt + kt
    const int rs = tile / M.nkt, kt = tile % M.nkt;
    const int row = rs * 16 + (lane & 15), kq = lane >> 4;
    const int K = M.K;
    const uint8_t* s = src + eoff;
    uint8_t* o = dst + eoff;
    const size_t pq = M.qoff + (size_t)tile * 1024 + (size_t)lane * 16;  // packed quant bytes of this lane

    if (wfmt == MOE_WFMT_I4B32) {
        for (int i = 0; i < 4; ++i) {
            const int c0 = (4 * kt + i) * 32 + 8 * kq;                  // first column of the 8
            const size_t cb = cq + ((size_t)row * K + c0) / 2;           // 4 canonical bytes
            if (!UNPACK) {
                uint32_t w = 0;
                for (int j = 0; j < 8; ++j) {
                    const uint8_t byte = s[cb + j / 2];
                    const uint32_t u = (j & 1) ? (byte >> 4) : (byte & 15);
                    const int pos = (j & 1) ? 4 + (j >> 1) : (j >> 1);
                    w |= u << (4 * pos);
                }
                for (int b = 0; b < 4; ++b) o[pq + 4 * i + b] = (uint8_t)(w >> (8 * b));
            } else {
                uint32_t w = 0;
                for (int b = 0; b < 4; ++b) w |= (uint32_t)s[pq + 4 * i + b] << (8 * b);
                for (int jb = 0; jb < 4; ++jb) {
                    const int j0 = 2 * jb, j1 = 2 * jb + 1;
                    const uint32_t u0 = (w >> (4 * (j0 >> 1))) & 15;
                    const uint32_t u1 = (w >> (4 * (4 + (j1 >> 1)))) & 15;
                    o[cb + jb] = (uint8_t)(u0 | (u1 << 4));
                }
            }
        }
    } else {
        for (int i = 0; i < 2; ++i) {
            const int c0 = (2 * kt + i) * 32 + 8 * kq;
            const size_t cb = cq + (size_t)row * K + c0;
            for (int j = 0; j < 8; ++j) {
                if (!UNPACK) o[pq + 8 * i + j] = s[cb + j] ^ 0x80;
                else o[cb + j] = s[pq + 8 * i + j] ^ 0x80;
            }
        }
    }
    if (lane < 16) {
        const int bpt = wfmt == MOE_WFMT_I4B32 ? 4 : 2;
        const size_t ps = M.soff + (size_t)tile * scale_tile_bytes(wfmt) + (size_t)lane * bpt * 2;
        const int r = rs * 16 + lane;
        for (int i = 0; i < bpt; ++i) {
            const size_t c = cs + ((size_t)r * (K / 32) + (size_t)(bpt * kt + i)) * 2;
            if (!UNPACK) { o[ps + 2 * i] = s[c]; o[ps + 2 * i + 1] = s[c + 1]; }
            else { o[c] = s[ps + 2 * i]; o[c + 1] = s[ps + 2 * i + 1]; }
        }
    }
}

int launch_pack(const void* src, void* dst, int n, int wfmt, int d, int f, bool unpack, hipStream_t st) {
    if (n == 0) return MOE_OK;
    const ExpertLayout P = expert_layout(wfmt, d, f);
    const int lanes_g = (P.g.R / 16) * P.g.nkt * 64;
    const int lanes_d = (P.dn.R / 16) * P.dn.nkt * 64;
    const int lanes_total = 2 * lanes_g + lanes_d;
    dim3 grid((lanes_total + 255) / 256, n);
    if (unpack)
        pack_kernel<true><<<grid, 256, 0, st>>>((const uint8_t*)src, (uint8_t*)dst, wfmt, d, f, P.total, lanes_g,
                                                lanes_total);
    else
        pack_kernel<false><<<grid, 256, 0, st>>>((const uint8_t*)src, (uint8_t*)dst, wfmt, d, f, P.total, lanes_g,
                                                 lanes_total);
    return check_launch();
}

}  // namespace moe

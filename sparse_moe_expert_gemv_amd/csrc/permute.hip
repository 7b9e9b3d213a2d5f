// Stable grouping of routing slots by expert: per-chunk LDS histograms, one
// workgroup that scans them (per-expert running sums over chunks, then an
// exclusive scan over experts and the compacted list of active experts), and
// a stable scatter in which each wavefront walks its chunk in order and ranks
// equal expert ids inside a 64-slot step with ballots.  Integer work only, so
// the result is bit-exact and independent of scheduling.
#include "common.hpp"

namespace moe {

__global__ __launch_bounds__(256) void perm_hist(const int32_t* __restrict__ ids, int n, int E,
                                                 int32_t* __restrict__ hist) {
    extern __shared__ int32_t cnt[];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int base = blockIdx.x * kPermChunk;
    const int end = min(n, base + kPermChunk);
    for (int f = base + threadIdx.x; f < end; f += blockDim.x) {
        const int id = ids[f];
        if ((unsigned)id < (unsigned)E) atomicAdd(&cnt[id], 1);  // out-of-range ids are ignored
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup of 1024 threads (E <= 1024).  Thread e turns its expert's
// chunk counts into exclusive positions within the expert, reading them 16 at
// a time so that the loads overlap (one dependent round trip per 16 chunks);
// the expert base (offsets[e]) is added by the scatter.
__global__ __launch_bounds__(1024) void perm_scan(int32_t* __restrict__ hist, int nch, int E,
                                                  int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ active) {
    __shared__ int32_t sc[1024];
    __shared__ int32_t sf[1024];
    const int e = threadIdx.x;
    int total = 0;
    if (e < E) {
        constexpr int G = 16;
        for (int c0 = 0; c0 < nch; c0 += G) {
            int v[G];
#pragma unroll
            for (int g = 0; g < G; ++g) v[g] = c0 + g < nch ? hist[(size_t)(c0 + g) * E + e] : 0;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (c0 + g < nch) hist[(size_t)(c0 + g) * E + e] = total;
                total += v[g];
            }
        }
        counts[e] = total;
    }
    sc[e] = e < E ? total : 0;
    sf[e] = (e < E && total > 0) ? 1 : 0;
    __syncthreads();
    // inclusive Hillis-Steele scans of counts and active flags
    for (int off = 1; off < 1024; off <<= 1) {
        const int a = e >= off ? sc[e - off] : 0;
        const int b = e >= off ? sf[e - off] : 0;
        __syncthreads();
        sc[e] += a;
        sf[e] += b;
        __syncthreads();
    }
    const int excl = sc[e] - (e < E ? total : 0);
    if (e < E) {
        offsets[e] = excl;
        if (total > 0) active[1 + sf[e] - 1] = e;
    }
    if (e == E - 1) {
        offsets[E] = sc[e];
        active[0] = sf[e];
    }
}

// One wavefront per chunk, slots visited in ascending order.
__global__ __launch_bounds__(64) void perm_scatter(const int32_t* __restrict__ ids, int n, int E,
                                                   const int32_t* __restrict__ hist,
                                                   const int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ sorted_idx, int32_t* __restrict__ dest) {
    extern __shared__ int32_t pos[];
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += 64) pos[e] = offsets[e] + hist[(size_t)blockIdx.x * E + e];
    __syncthreads();
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const int base = blockIdx.x * kPermChunk;
    const int end = min(n, base + kPermChunk);
    const unsigned long long lt = (1ull << lane) - 1ull;
    for (int f0 = base; f0 < end; f0 += 64) {
        const int f = f0 + lane;
        const int raw = f < end ? ids[f] : -1;
        const bool valid = (unsigned)raw < (unsigned)E;
        const int id = valid ? raw : 0;
        unsigned long long peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const unsigned long long on = __ballot(valid && ((id >> b) & 1));
            peers &= ((id >> b) & 1) ? on : ~on;
        }
        const int rank = __popcll(peers & lt);
        const int cnt = __popcll(peers);
        int p = 0;
        if (valid) p = pos[id] + rank;
        __syncthreads();  // every lane has read pos[] before the group leader advances it
        if (valid && rank == 0) pos[id] += cnt;
        __syncthreads();
        if (valid) {
            sorted_idx[p] = f;
            dest[f] = p;
        }
    }
}

int launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                   int32_t* dest, int32_t* active, int32_t* hist, hipStream_t s) {
    const int n = T * k;
    const int nch = (n + kPermChunk - 1) / kPermChunk;
    if (n == 0) return MOE_OK;  // the API treats T == 0 as a no-op before getting here
    if (n <= 4096) return launch_permute_block(ids, n, E, counts, offsets, sorted_idx, dest, active, s);
    perm_hist<<<nch, 256, E * sizeof(int32_t), s>>>(ids, n, E, hist);
    int rc = check_launch();
    if (rc) return rc;
    perm_scan<<<1, 1024, 0, s>>>(hist, nch, E, counts, offsets, active);
    rc = check_launch();
    if (rc) return rc;
    perm_scatter<<<nch, 64, E * sizeof(int32_t), s>>>(ids, n, E, hist, offsets, sorted_idx, dest);
    return check_launch();
}

}  // namespace moe

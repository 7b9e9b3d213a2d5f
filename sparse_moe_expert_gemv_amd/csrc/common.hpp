// Internal definitions shared by the library's HIP sources (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---- packed expert layout --------------------------------------------------
// Every matrix W [R, K] (R output rows, K reduction, block-32 along K) is stored
// as tiles of 16 rows x 1 KiB of quants, tile (rs, kt) at ((rs * nkt) + kt) KiB:
//   int4: a tile covers 128 k (4 blocks).  Lane l of a wave (row rs*16 + l%16,
//         k sub-range 8*(l/16) .. +7 inside each block) owns 16 bytes: dword i
//         holds block 4*kt+i as 8 offset-binary nibbles in the order
//         [k0 k2 k4 k6 k1 k3 k5 k7] (nibble j at bits 4j), so that
//         (w >> 4s) & 0x000F000F yields the pair (k_2s, k_2s+1) in two 16-bit
//         halves.
//   int8: a tile covers 64 k (2 blocks).  Lane l owns 16 bytes: bytes 0..7 are
//         k = 8*(l/16)+0..7 of block 2*kt, bytes 8..15 the same of block
//         2*kt+1, stored offset-binary (q + 128).
// Scales follow all quants, per matrix, as fp16 tiles [16 rows][blocks/tile]
// in the same (rs, kt) order (128 B per int4 tile, 64 B per int8 tile).
// Blob: [Wg tiles][Wu tiles][Wd tiles][Wg scales][Wu scales][Wd scales].
struct MatLayout {
    size_t qoff, soff;  // byte offsets in the blob
    int R, K;           // rows, reduction length
    int nkt;            // k tiles per 16-row strip
};

struct ExpertLayout {
    MatLayout g, u, dn;
    size_t total;
};

__host__ __device__ inline int k_per_tile(int wfmt) { return wfmt == MOE_WFMT_I4B32 ? 128 : 64; }
__host__ __device__ inline int scale_tile_bytes(int wfmt) { return wfmt == MOE_WFMT_I4B32 ? 128 : 64; }

__host__ __device__ inline ExpertLayout expert_layout(int wfmt, int d, int f) {
    ExpertLayout L;
    const size_t n = (size_t)d * f;
    const size_t qb = wfmt == MOE_WFMT_I4B32 ? n / 2 : n;
    const size_t sb = (n / 32) * 2;
    const int kpt = k_per_tile(wfmt);
    L.g = {0, 3 * qb, f, d, d / kpt};
    L.u = {qb, 3 * qb + sb, f, d, d / kpt};
    L.dn = {2 * qb, 3 * qb + 2 * sb, d, f, f / kpt};
    L.total = 3 * qb + 3 * sb;
    return L;
}

// canonical layout offsets (row-major quants, row-major scales)
struct CanonLayout {
    size_t qg, qu, qd, sg, su, sd, total;
};
__host__ __device__ inline CanonLayout canon_layout(int wfmt, int d, int f) {
    CanonLayout C;
    const size_t n = (size_t)d * f;
    const size_t qb = wfmt == MOE_WFMT_I4B32 ? n / 2 : n;
    const size_t sb = (n / 32) * 2;
    C.qg = 0; C.qu = qb; C.qd = 2 * qb;
    C.sg = 3 * qb; C.su = C.sg + sb; C.sd = C.su + sb;
    C.total = C.sd + sb;
    return C;
}

// ---- vector types -----------------------------------------------------------
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int16v __attribute__((ext_vector_type(16)));
typedef unsigned uint4v __attribute__((ext_vector_type(4)));
typedef unsigned uint2v __attribute__((ext_vector_type(2)));

// Load through a global-address-space pointer.  Pointers read from memory
// (expert blob tables) are generic; without the cast the compiler emits flat
// loads, which also count against the LDS counter and force extra waits.
template <typename V>
__device__ __forceinline__ V gload(const V* p) {
    return *(const __attribute__((address_space(1))) V*)p;
}

// Non-temporal load through a global-address-space pointer, for data read once
// per call (expert weights streamed from HBM): it is not kept in the caches at
// the expense of data that is reused.
template <typename V>
__device__ __forceinline__ V gload_nt(const V* p) {
    return __builtin_nontemporal_load((const __attribute__((address_space(1))) V*)p);
}
constexpr int kBufNT = 2;  // cache-policy operand of a buffer load: non-temporal

// Buffer resource over [base, base + bytes): loads through it are bounds
// checked and return zeros outside the range (bytes = 0: nothing is read).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// ---- error plumbing -----------------------------------------------------------
void set_last_hip_error(hipError_t e);
int check_launch();  // MOE_OK or MOE_ERR_HIP after a kernel launch

inline hipStream_t as_stream(moe_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// ---- workspace carve-up -------------------------------------------------------
// Regions are laid out in this order so that route and permute only need a
// prefix of the workspace.
struct Workspace {
    double* logits;     // [P, T, E] (P k planes)         route
    int32_t* hist;      // [ceil(T*k / kPermChunk), E]    permute
    int32_t* tiles;     // q8 tile list (int2) + count    ffn
    void* h;            // SwiGLU intermediate [T*k + T, f]: fp16 (float mode, q8 with int4 weights) or int8 (q8, int8 weights)
    float* hs;          // q8: [T*k + T, f/32] block scales of h
    const uint8_t** tile_blob;  // q8 mode: expert blob of each tile of the tile list (int4 weights)
    const uint8_t** slot_blob;  // float mode: [T*k] expert blob of each routed slot (by-slot decode;
                                // written by the gate/up launch, read by the down + combine launch)
    size_t route_bytes, permute_bytes, bytes;
};
constexpr int kPermChunk = 1024;
// Fills w (pointers relative to base, which may be null to size only).
void workspace_layout(int T, int d, int f, int E, int k, int act_mode, char* base, Workspace* w);

// ---- launchers (defined in the .hip files) -----------------------------------
int launch_pack(const void* src, void* dst, int n, int wfmt, int d, int f, bool unpack, hipStream_t s);
// number of [T, E] planes of partial router logits the routing writes (k split
// over workgroups for moderate batches; 1 otherwise)
int logit_planes(int T, int d, int E);
constexpr int kMaxLogitPlanes = 4;
int launch_route(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E, int k,
                 int32_t* ids, float* gates, double* logits, hipStream_t s);
bool route_small_ok(int T, int d, int k);
// large bf16 batches: certified bf16 filter + exact refine of the candidates
// (route_filter.hip); its scratch (route_filter_bytes) lives in the logits region
bool route_filter_ok(int T, int d, int E, int k, int x_dtype);
size_t route_filter_bytes(int T, int E, int d);
int launch_route_filtered(const void* x, int T, int d, const float* Wr, const float* bias, int E, int k,
                          int32_t* ids, float* gates, void* scratch, hipStream_t s);
int launch_route_small(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E, int k,
                       int32_t* ids, float* gates, double* logits, bool do_permute, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_idx, int32_t* dest, int32_t* active, hipStream_t s);
size_t float_h_bytes(int T, int f, int k);
int launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                   int32_t* dest, int32_t* active, int32_t* hist, hipStream_t s);
// one-workgroup permutation for at most 4096 slots
int launch_permute_block(const int32_t* ids, int n, int E, int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                         int32_t* dest, int32_t* active, hipStream_t s);
int launch_rmsnorm(const float* x, int T, int d, float eps, float* out, hipStream_t s);
int launch_quant_act(const void* x, int x_dtype, int T, int d, int8_t* xq, float* sx, hipStream_t s);
// down projection + weighted combine in one kernel (float mode, int4, few
// tokens): out = residual + shared + sum_j g_j y_j without y_perm
constexpr int kDownCombineMax = 8;
bool down_combine_ok(const moe_ffn_args* a);
// slot_blob (by-slot batches, dest NULL): the routed slots' expert blobs as the
// gate/up launch wrote them, read instead of expert_ptrs[ids]
int launch_down_combine(const moe_ffn_args* a, const Workspace& w, const int32_t* ids, const int32_t* dest,
                        const float* gates, const float* residual, float* out, hipStream_t s,
                        const uint8_t* const* slot_blob = nullptr);
// decode without the grouping: gate/up per routed slot, then the fused down +
// combine (h row of slot (t, j) = t k + j)
bool ffn_combine_slots_ok(const moe_ffn_args* a);
int launch_ffn_combine_slots(const moe_ffn_args* a, const Workspace& w, const int32_t* ids, const float* gates,
                             const float* residual, float* out, hipStream_t s);
int launch_ffn_combine_slots_topk(const moe_ffn_args* a, const Workspace& w, int planes, int32_t* ids, float* gates,
                                  const float* residual, float* out, hipStream_t s);
// router logits alone (double, into `logits`, logit_planes(T, d, E) k planes)
int launch_route_logits(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E,
                        double* logits, hipStream_t s);
int launch_ffn_float(const moe_ffn_args* a, const Workspace& w, hipStream_t s);
int launch_ffn_q8(const moe_ffn_args* a, const Workspace& w, hipStream_t s);
size_t q8_tile_capacity(int T, int k, int E);  // int2 entries of the q8 tile list
int launch_combine(const void* y_perm, int y_dtype, const int32_t* dest, const float* gates, const float* y_shared,
                   const float* residual, int T, int k, int d, float* out, hipStream_t s);

}  // namespace moe

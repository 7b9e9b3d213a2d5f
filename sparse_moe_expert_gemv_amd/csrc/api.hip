// C ABI entry points: argument validation (before any HIP call), workspace
// carve-up and dispatch to the kernel launchers.
#include <algorithm>
#include <mutex>

#include "common.hpp"

namespace moe {

static thread_local int g_last_hip_error = 0;

void set_last_hip_error(hipError_t e) { g_last_hip_error = (int)e; }

int check_launch() {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_last_hip_error(e);
        return MOE_ERR_HIP;
    }
    return MOE_OK;
}

static size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

void workspace_layout(int T, int d, int f, int E, int k, int act_mode, char* base, Workspace* w) {
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off = align_up(off + bytes);
        return p;
    };
    const size_t rows = (size_t)T * k + (size_t)T;
    const size_t nch = ((size_t)T * k + kPermChunk - 1) / kPermChunk;
    // room for the split-k planes of any batch up to T (a workspace sized for
    // T also serves every smaller batch): P T' <= kMaxLogitPlanes T' with P = 1
    // beyond 256 tokens
    const size_t logit_rows = (size_t)T + (size_t)(kMaxLogitPlanes - 1) * std::min(T, 256);
    // large batches: also room for the filtered router's scratch (route_filter.hip)
    size_t logit_bytes = sizeof(double) * logit_rows * E;
    if (T > 256) logit_bytes = std::max(logit_bytes, route_filter_bytes(T, E, d));
    w->logits = reinterpret_cast<double*>(take(logit_bytes));
    w->route_bytes = off;
    w->hist = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * std::max<size_t>(nch, 1) * E));
    w->permute_bytes = off;
    if (act_mode == MOE_ACT_Q8) {
        w->tiles = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (4 * q8_tile_capacity(T, k, E) + 4)));
        w->tile_blob = reinterpret_cast<const uint8_t**>(take(sizeof(void*) * q8_tile_capacity(T, k, E)));
        w->h = take(rows * (size_t)f * 2);  // int8 codes (int8 weights) or fp16 q * s (int4 weights)
        w->hs = reinterpret_cast<float*>(take(sizeof(float) * rows * (size_t)(f / 32)));
    } else {
        w->tiles = nullptr;
        w->tile_blob = nullptr;
        w->h = take(float_h_bytes(T, f, k));
        w->hs = nullptr;
    }
    w->slot_blob = act_mode == MOE_ACT_Q8 ? nullptr
                                          : reinterpret_cast<const uint8_t**>(take(sizeof(void*) * (size_t)T * k));
    w->bytes = off;
}

static bool shape_ok(int d, int E, int k) { return d > 0 && d % 128 == 0 && k >= 1 && k <= 64 && E >= k && E <= 1024; }

}  // namespace moe

using namespace moe;

extern "C" {

int moe_version(void) { return MOE_VERSION; }

int moe_last_hip_error(void) { return g_last_hip_error; }

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        case MOE_ERR_NO_MEMORY: return "MOE_ERR_NO_MEMORY";
        case MOE_ERR_CACHE_CAPACITY: return "MOE_ERR_CACHE_CAPACITY";
        default: return "MOE_ERR_UNKNOWN";
    }
}

size_t moe_expert_bytes(int wfmt, int d, int f) {
    if ((wfmt != MOE_WFMT_I4B32 && wfmt != MOE_WFMT_I8B32) || d <= 0 || f <= 0 || d % 32 || f % 32) return 0;
    return canon_layout(wfmt, d, f).total;
}

static int pack_common(const void* src, void* dst, int n, int wfmt, int d, int f, bool unpack, moe_stream_t s) {
    if (n < 0 || (wfmt != MOE_WFMT_I4B32 && wfmt != MOE_WFMT_I8B32) || d <= 0 || f <= 0 || d % 128 || f % 128)
        return MOE_ERR_INVALID_ARG;
    if (n == 0) return MOE_OK;
    if (!src || !dst || src == dst || n > 65535) return MOE_ERR_INVALID_ARG;
    return launch_pack(src, dst, n, wfmt, d, f, unpack, as_stream(s));
}

int moe_pack_experts(const void* src, void* dst, int n, int wfmt, int d, int f, moe_stream_t s) {
    return pack_common(src, dst, n, wfmt, d, f, false, s);
}

int moe_unpack_experts(const void* src, void* dst, int n, int wfmt, int d, int f, moe_stream_t s) {
    return pack_common(src, dst, n, wfmt, d, f, true, s);
}

int moe_workspace_size(int T, int d, int f, int E, int k, int act_mode, size_t* bytes) {
    if (!bytes || T < 0 || !shape_ok(d, E, k) || f <= 0 || f % 128 ||
        (act_mode != MOE_ACT_FLOAT && act_mode != MOE_ACT_Q8))
        return MOE_ERR_INVALID_ARG;
    Workspace w;
    workspace_layout(T, d, f, E, k, act_mode, nullptr, &w);
    *bytes = w.bytes;
    return MOE_OK;
}

int moe_route(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E, int k,
              int32_t* ids, float* gates, void* ws, size_t ws_bytes, moe_stream_t s) {
    if (T < 0 || !shape_ok(d, E, k) || (x_dtype != MOE_DT_F32 && x_dtype != MOE_DT_BF16)) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !Wr || !ids || !gates || !ws) return MOE_ERR_INVALID_ARG;
    Workspace w;
    workspace_layout(T, d, 128, E, k, MOE_ACT_FLOAT, (char*)ws, &w);
    if (ws_bytes < w.route_bytes) return MOE_ERR_NO_MEMORY;
    return launch_route(x, x_dtype, T, d, Wr, bias, E, k, ids, gates, w.logits, as_stream(s));
}

int moe_route_permute(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E, int k,
                      int32_t* ids, float* gates, int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                      int32_t* dest, int32_t* active, void* ws, size_t ws_bytes, moe_stream_t s) {
    if (T < 0 || !shape_ok(d, E, k) || (x_dtype != MOE_DT_F32 && x_dtype != MOE_DT_BF16)) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !Wr || !ids || !gates || !counts || !offsets || !sorted_idx || !dest || !active || !ws)
        return MOE_ERR_INVALID_ARG;
    Workspace w;
    workspace_layout(T, d, 128, E, k, MOE_ACT_FLOAT, (char*)ws, &w);
    if (ws_bytes < w.permute_bytes) return MOE_ERR_NO_MEMORY;
    if (route_small_ok(T, d, k))
        return launch_route_small(x, x_dtype, T, d, Wr, bias, E, k, ids, gates, w.logits, true, counts, offsets,
                                  sorted_idx, dest, active, as_stream(s));
    int rc = launch_route(x, x_dtype, T, d, Wr, bias, E, k, ids, gates, w.logits, as_stream(s));
    if (rc) return rc;
    return launch_permute(ids, T, k, E, counts, offsets, sorted_idx, dest, active, w.hist, as_stream(s));
}

int moe_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                int32_t* dest, int32_t* active, void* ws, size_t ws_bytes, moe_stream_t s) {
    if (T < 0 || k < 1 || k > 64 || E < k || E > 1024 || (long)T * k > (1l << 30)) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!ids || !counts || !offsets || !sorted_idx || !dest || !active || !ws) return MOE_ERR_INVALID_ARG;
    Workspace w;
    workspace_layout(T, 128, 128, E, k, MOE_ACT_FLOAT, (char*)ws, &w);
    if (ws_bytes < w.permute_bytes) return MOE_ERR_NO_MEMORY;
    return launch_permute(ids, T, k, E, counts, offsets, sorted_idx, dest, active, w.hist, as_stream(s));
}

int moe_rmsnorm(const float* x, int T, int d, float eps, float* out, moe_stream_t s) {
    if (T < 0 || d <= 0 || d % 4 || !(eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !out) return MOE_ERR_INVALID_ARG;
    return launch_rmsnorm(x, T, d, eps, out, as_stream(s));
}

int moe_quantize_act(const void* x, int x_dtype, int T, int d, int8_t* xq, float* sx, moe_stream_t s) {
    if (T < 0 || d <= 0 || d % 32 || (x_dtype != MOE_DT_F32 && x_dtype != MOE_DT_BF16)) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !xq || !sx) return MOE_ERR_INVALID_ARG;
    return launch_quant_act(x, x_dtype, T, d, xq, sx, as_stream(s));
}

int moe_expert_ffn(const moe_ffn_args* a, moe_stream_t s) {
    if (!a) return MOE_ERR_INVALID_ARG;
    if (a->T < 0 || !shape_ok(a->d, a->E, a->k) || a->f <= 0 || a->f % 128 ||
        (a->wfmt != MOE_WFMT_I4B32 && a->wfmt != MOE_WFMT_I8B32) ||
        (a->act_mode != MOE_ACT_FLOAT && a->act_mode != MOE_ACT_Q8) ||
        (a->y_dtype != MOE_DT_F32 && a->y_dtype != MOE_DT_F16) || a->phase < 0 || a->phase > 2)
        return MOE_ERR_INVALID_ARG;
    if (a->T == 0) return MOE_OK;
    if (!a->expert_ptrs || !a->counts || !a->offsets || !a->sorted_idx || !a->active || !a->y_perm || !a->ws)
        return MOE_ERR_INVALID_ARG;
    if (a->shared_blob && !a->y_shared) return MOE_ERR_INVALID_ARG;
    if (a->act_mode == MOE_ACT_FLOAT) {
        if (!a->x || (a->x_dtype != MOE_DT_F32 && a->x_dtype != MOE_DT_BF16)) return MOE_ERR_INVALID_ARG;
    } else {
        if (!a->xq || !a->sx) return MOE_ERR_INVALID_ARG;
    }
    Workspace w;
    workspace_layout(a->T, a->d, a->f, a->E, a->k, a->act_mode, (char*)a->ws, &w);
    if (a->ws_bytes < w.bytes) return MOE_ERR_NO_MEMORY;
    return a->act_mode == MOE_ACT_FLOAT ? launch_ffn_float(a, w, as_stream(s)) : launch_ffn_q8(a, w, as_stream(s));
}

int moe_expert_ffn_combine(const moe_ffn_args* a, const int32_t* ids, const int32_t* dest, const float* gates,
                           const float* residual, float* out, moe_stream_t s) {
    if (!a || a->phase != 0) return MOE_ERR_INVALID_ARG;
    if (a->T > 0 && (!ids || !dest || !gates || !out)) return MOE_ERR_INVALID_ARG;
    if (!down_combine_ok(a)) {
        const int rc = moe_expert_ffn(a, s);
        if (rc || a->T == 0) return rc;
        return moe_combine(a->y_perm, a->y_dtype, dest, gates, a->shared_blob ? a->y_shared : nullptr, residual,
                           a->T, a->k, a->d, out, s);
    }
    moe_ffn_args g = *a;
    g.phase = 1;  // gate/up + SwiGLU into the workspace; validates every argument
    const int rc = moe_expert_ffn(&g, s);
    if (rc || a->T == 0) return rc;
    Workspace w;
    workspace_layout(a->T, a->d, a->f, a->E, a->k, a->act_mode, (char*)a->ws, &w);
    return launch_down_combine(a, w, ids, dest, gates, residual, out, as_stream(s));
}

int moe_expert_ffn_combine_slots(const moe_ffn_args* a, const int32_t* ids, const float* gates,
                                 const float* residual, float* out, moe_stream_t s) {
    if (!a || (a->phase != 0 && a->phase != 1)) return MOE_ERR_INVALID_ARG;
    if (a->T < 0 || !shape_ok(a->d, a->E, a->k) || a->f <= 0 || a->f % 128 ||
        (a->wfmt != MOE_WFMT_I4B32 && a->wfmt != MOE_WFMT_I8B32) ||
        (a->act_mode != MOE_ACT_FLOAT && a->act_mode != MOE_ACT_Q8) ||
        (a->x_dtype != MOE_DT_F32 && a->x_dtype != MOE_DT_BF16))
        return MOE_ERR_INVALID_ARG;
    if (a->T == 0) return MOE_OK;
    if (!a->x || !a->expert_ptrs || !a->ws || !ids || !gates || !out) return MOE_ERR_INVALID_ARG;
    Workspace w;
    workspace_layout(a->T, a->d, a->f, a->E, a->k, a->act_mode, (char*)a->ws, &w);
    if (a->ws_bytes < w.bytes) return MOE_ERR_NO_MEMORY;
    return launch_ffn_combine_slots(a, w, ids, gates, residual, out, as_stream(s));
}

static int route_ffn_combine_slots_args(const moe_ffn_args* a, const float* Wr, int32_t* ids, float* gates,
                                        float* out, bool need_ws) {
    if (!a || (a->phase != 0 && a->phase != 1)) return MOE_ERR_INVALID_ARG;
    if (a->T < 0 || !shape_ok(a->d, a->E, a->k) || a->f <= 0 || a->f % 128 ||
        (a->wfmt != MOE_WFMT_I4B32 && a->wfmt != MOE_WFMT_I8B32) ||
        (a->act_mode != MOE_ACT_FLOAT && a->act_mode != MOE_ACT_Q8) ||
        (a->x_dtype != MOE_DT_F32 && a->x_dtype != MOE_DT_BF16))
        return MOE_ERR_INVALID_ARG;
    if (a->T == 0) return MOE_OK;
    if (!a->x || !a->expert_ptrs || (need_ws && !a->ws) || !Wr || !ids || !gates || !out) return MOE_ERR_INVALID_ARG;
    return -1;  // arguments valid, work to do
}

static int route_ffn_combine_slots_run(const moe_ffn_args* a, const Workspace& w, const float* Wr, const float* bias,
                                       int32_t* ids, float* gates, const float* residual, float* out,
                                       moe_stream_t s) {
    if (!ffn_combine_slots_ok(a)) return MOE_ERR_UNSUPPORTED;
    if (a->phase == 0) {  // phase 1: the router logits are already in the workspace
        const int rc = launch_route_logits(a->x, a->x_dtype, a->T, a->d, Wr, bias, a->E, w.logits, as_stream(s));
        if (rc) return rc;
    }
    return launch_ffn_combine_slots_topk(a, w, logit_planes(a->T, a->d, a->E), ids, gates, residual, out,
                                         as_stream(s));
}

int moe_route_ffn_combine_slots(const moe_ffn_args* a, const float* Wr, const float* bias, int32_t* ids,
                                float* gates, const float* residual, float* out, moe_stream_t s) {
    const int rc = route_ffn_combine_slots_args(a, Wr, ids, gates, out, true);
    if (rc >= 0) return rc;
    Workspace w;
    workspace_layout(a->T, a->d, a->f, a->E, a->k, a->act_mode, (char*)a->ws, &w);
    if (a->ws_bytes < w.bytes) return MOE_ERR_NO_MEMORY;
    return route_ffn_combine_slots_run(a, w, Wr, bias, ids, gates, residual, out, s);
}

// ---- the same decode layer without a caller workspace ------------------------
// Scratch for callers that cannot allocate: a file-scope device array that
// every GPU the library runs on holds until the process ends.  Host code uses
// only the device address hipGetSymbolAddress returns for the current device
// (the array's name is a host-side stand-in), looked up once per device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

static void* device_scratch(int* rc) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        set_last_hip_error(e != hipSuccess ? e : hipErrorInvalidDevice);
        *rc = MOE_ERR_HIP;
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) {
        set_last_hip_error(g_scratch_err[dev] != hipSuccess ? g_scratch_err[dev] : hipErrorInvalidSymbol);
        *rc = MOE_ERR_HIP;
        return nullptr;
    }
    *rc = MOE_OK;
    return g_scratch_ptr[dev];
}

int moe_route_ffn_combine_slots_noalloc(const moe_ffn_args* a, const float* Wr, const float* bias, int32_t* ids,
                                        float* gates, const float* residual, float* out, moe_stream_t s) {
    int rc = route_ffn_combine_slots_args(a, Wr, ids, gates, out, false);
    if (rc >= 0) return rc;
    if (a->phase != 0) return MOE_ERR_INVALID_ARG;
    Workspace w;
    workspace_layout(a->T, a->d, a->f, a->E, a->k, a->act_mode, nullptr, &w);
    if (w.bytes > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_NO_MEMORY;
    if (!ffn_combine_slots_ok(a)) return MOE_ERR_UNSUPPORTED;
    char* base = static_cast<char*>(device_scratch(&rc));
    if (!base) return rc;
    workspace_layout(a->T, a->d, a->f, a->E, a->k, a->act_mode, base, &w);
    moe_ffn_args b = *a;
    b.ws = base;
    b.ws_bytes = MOE_NOALLOC_SCRATCH_BYTES;
    return route_ffn_combine_slots_run(&b, w, Wr, bias, ids, gates, residual, out, s);
}

int moe_combine(const void* y_perm, int y_dtype, const int32_t* dest, const float* gates, const float* y_shared,
                const float* residual, int T, int k, int d, float* out, moe_stream_t s) {
    if (T < 0 || k < 1 || d <= 0 || d % 4 || (y_dtype != MOE_DT_F32 && y_dtype != MOE_DT_F16))
        return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!y_perm || !dest || !gates || !out) return MOE_ERR_INVALID_ARG;
    return launch_combine(y_perm, y_dtype, dest, gates, y_shared, residual, T, k, d, out, as_stream(s));
}

}  // extern "C"

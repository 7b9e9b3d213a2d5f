// Expert slot cache: host bookkeeping of which global expert occupies which
// slot of a caller-owned HBM pool, and per-layer pointer tables for the
// misses: staged from pinned host memory on a (side) stream, or (decode)
// pointing at the pinned host blobs themselves, read in place by the FFN.
// "How Strata works" (adaptive expert cache section) loads the most-used
// ~4,500 experts by a usage ranking into GPU memory; "Strata benchmarks"
// (prefill optimisation table) streams the next layer's experts over PCIe
// while the current layer computes.
#include <algorithm>
#include <cmath>
#include <numeric>
#include <vector>

#include "common.hpp"

struct moe_cache {
    int n_layers, E, n_slots, n_bufs, staging_slots;
    size_t eb;
    char* pool;
    char* staging;
    std::vector<int32_t> slot_of;        // [n_layers * E] -> slot or -1
    void** tables;                       // pinned host [n_layers][E] pointer tables
    std::vector<hipEvent_t> table_done;  // per layer: last upload of its table
    std::vector<bool> table_pending;
    std::vector<bool> table_written;     // the pinned table of the layer holds a full mapping
    int stage_mode = MOE_STAGE_MEMCPY;   // how moe_cache_stage copies the misses
    int copy_workgroups = 32;            // MOE_STAGE_KERNEL: workgroups of the copy kernel
    uint64_t* copy_list = nullptr;       // pinned host [n_layers][2 * E] (source, destination) device addresses
    moe_stage_fault_fn fault = nullptr;  // test hook consulted before each staging copy
    void* fault_user = nullptr;
};

using namespace moe;

// per-expert selection counter of one layer (wrapping int32)
__global__ __launch_bounds__(256) static void usage_accumulate(int32_t* __restrict__ usage,
                                                              const int32_t* __restrict__ counts, int E) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e < E) usage[e] = (int32_t)((uint32_t)usage[e] + (uint32_t)counts[e]);
}

// Copies the n missed experts of a layer (eb = 16 n16 bytes each) from mapped
// pinned host memory into the staging slots: list holds their (source,
// destination) device addresses and is read once into LDS; every workgroup
// copies its slice of every expert with 16-byte non-temporal loads, four in
// flight per thread.  One launch per layer instead of one copy call per expert.
__global__ __launch_bounds__(256) static void stage_copy(const uint64_t* __restrict__ list, int n, uint32_t n16) {
    __shared__ uint64_t s_list[2 * 1024];
    for (int i = threadIdx.x; i < 2 * n; i += 256) s_list[i] = list[i];
    __syncthreads();
    const uint32_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const uint32_t c0 = blockIdx.x * per, c1 = min(n16, c0 + per);
    for (int i = 0; i < n; ++i) {
        const uint4v* __restrict__ src = reinterpret_cast<const uint4v*>(s_list[2 * i]);
        uint4v* __restrict__ dst = reinterpret_cast<uint4v*>(s_list[2 * i + 1]);
        uint32_t c = c0 + threadIdx.x;
        for (; c + 3 * 256 < c1; c += 4 * 256) {
            const uint4v v0 = __builtin_nontemporal_load(src + c);
            const uint4v v1 = __builtin_nontemporal_load(src + c + 256);
            const uint4v v2 = __builtin_nontemporal_load(src + c + 512);
            const uint4v v3 = __builtin_nontemporal_load(src + c + 768);
            dst[c] = v0;
            dst[c + 256] = v1;
            dst[c + 512] = v2;
            dst[c + 768] = v3;
        }
        for (; c < c1; c += 256) dst[c] = __builtin_nontemporal_load(src + c);
    }
}

static int hip_fail(hipError_t e) {
    set_last_hip_error(e);
    return MOE_ERR_HIP;
}

extern "C" {

int moe_cache_create(moe_cache** cache, int n_layers, int E, int n_slots, size_t expert_bytes, void* dev_pool,
                     void* dev_staging, int n_staging_bufs, int staging_slots) {
    if (!cache || n_layers < 1 || E < 1 || E > 1024 || n_slots < 0 || expert_bytes == 0 || n_staging_bufs < 1 ||
        staging_slots < 0 || (n_slots > 0 && !dev_pool) || (staging_slots > 0 && !dev_staging))
        return MOE_ERR_INVALID_ARG;
    if ((long)n_layers * E > (1l << 30)) return MOE_ERR_INVALID_ARG;
    moe_cache* c = new (std::nothrow) moe_cache();
    if (!c) return MOE_ERR_NO_MEMORY;
    c->n_layers = n_layers; c->E = E; c->n_slots = n_slots; c->n_bufs = n_staging_bufs;
    c->staging_slots = staging_slots; c->eb = expert_bytes;
    c->pool = (char*)dev_pool; c->staging = (char*)dev_staging;
    c->slot_of.assign((size_t)n_layers * E, -1);
    c->tables = nullptr;
    hipError_t e = hipHostMalloc((void**)&c->tables, sizeof(void*) * (size_t)n_layers * E, hipHostMallocDefault);
    if (e != hipSuccess) { delete c; return hip_fail(e); }
    if (staging_slots > 0) {
        e = hipHostMalloc((void**)&c->copy_list, sizeof(uint64_t) * 2 * (size_t)n_layers * E, hipHostMallocDefault);
        if (e != hipSuccess) { (void)hipHostFree(c->tables); delete c; return hip_fail(e); }
    }
    c->table_done.assign(n_layers, nullptr);
    c->table_pending.assign(n_layers, false);
    c->table_written.assign(n_layers, false);
    for (int l = 0; l < n_layers; ++l) {
        e = hipEventCreateWithFlags(&c->table_done[l], hipEventDisableTiming);
        if (e != hipSuccess) { moe_cache_destroy(c); return hip_fail(e); }
    }
    *cache = c;
    return MOE_OK;
}

int moe_cache_destroy(moe_cache* c) {
    if (!c) return MOE_ERR_INVALID_ARG;
    for (hipEvent_t ev : c->table_done)
        if (ev) {
            (void)hipEventSynchronize(ev);
            (void)hipEventDestroy(ev);
        }
    if (c->tables) (void)hipHostFree(c->tables);
    if (c->copy_list) (void)hipHostFree(c->copy_list);
    delete c;
    return MOE_OK;
}

int moe_cache_set_stage_mode(moe_cache* c, int mode, int n_workgroups) {
    if (!c || (mode != MOE_STAGE_MEMCPY && mode != MOE_STAGE_KERNEL)) return MOE_ERR_INVALID_ARG;
    if (mode == MOE_STAGE_KERNEL && (n_workgroups < 1 || n_workgroups > 1024 || c->eb % 16 || c->eb / 16 > 0xFFFFFFFFu))
        return MOE_ERR_INVALID_ARG;
    c->stage_mode = mode;
    if (mode == MOE_STAGE_KERNEL) c->copy_workgroups = n_workgroups;
    return MOE_OK;
}

int moe_cache_set_stage_fault_hook(moe_cache* c, moe_stage_fault_fn hook, void* user) {
    if (!c) return MOE_ERR_INVALID_ARG;
    c->fault = hook;
    c->fault_user = hook ? user : nullptr;
    return MOE_OK;
}

int moe_cache_set_resident(moe_cache* c, const int32_t* ids, int n, const void* const* host_src, moe_stream_t s) {
    if (!c || n < 0 || n > c->n_slots || (n > 0 && (!ids || !host_src))) return MOE_ERR_INVALID_ARG;
    const long total = (long)c->n_layers * c->E;
    std::vector<char> seen(total, 0);
    for (int i = 0; i < n; ++i) {
        if (ids[i] < 0 || ids[i] >= total || seen[ids[i]] || !host_src[i]) return MOE_ERR_INVALID_ARG;
        seen[ids[i]] = 1;
    }
    std::fill(c->slot_of.begin(), c->slot_of.end(), -1);
    for (int i = 0; i < n; ++i) {
        c->slot_of[ids[i]] = i;
        const hipError_t e = hipMemcpyAsync(c->pool + (size_t)i * c->eb, host_src[i], c->eb, hipMemcpyHostToDevice,
                                            as_stream(s));
        if (e != hipSuccess) return hip_fail(e);
    }
    return MOE_OK;
}

int moe_cache_lookup(const moe_cache* c, int layer, int32_t* hit_ids, int* n_hit, int32_t* miss_ids, int* n_miss) {
    if (!c || layer < 0 || layer >= c->n_layers || !miss_ids || !n_miss) return MOE_ERR_INVALID_ARG;
    int h = 0, m = 0;
    for (int e = 0; e < c->E; ++e) {
        if (c->slot_of[(size_t)layer * c->E + e] >= 0) {
            if (hit_ids) hit_ids[h] = e;
            ++h;
        } else {
            miss_ids[m++] = e;
        }
    }
    if (n_hit) *n_hit = h;
    *n_miss = m;
    return MOE_OK;
}

int moe_cache_stage(moe_cache* c, int layer, int buf, const void* const* host_src, void** dev_table, moe_stream_t s,
                    moe_event_t done) {
    if (!c || layer < 0 || layer >= c->n_layers || buf < 0 || buf >= c->n_bufs || !host_src || !dev_table)
        return MOE_ERR_INVALID_ARG;
    int n_miss = 0;
    for (int e = 0; e < c->E; ++e) {
        if (c->slot_of[(size_t)layer * c->E + e] < 0) {
            if (!host_src[e]) return MOE_ERR_INVALID_ARG;
            ++n_miss;
        }
    }
    if (n_miss > c->staging_slots) return MOE_ERR_CACHE_CAPACITY;
    // the pinned table of this layer may still be read by its previous upload
    if (c->table_pending[layer]) {
        const hipError_t e = hipEventSynchronize(c->table_done[layer]);
        if (e != hipSuccess) return hip_fail(e);
        c->table_pending[layer] = false;
    }
    void** table = c->tables + (size_t)layer * c->E;
    char* stage = c->staging + (size_t)buf * c->staging_slots * c->eb;
    const hipStream_t st = as_stream(s);
    const bool kernel = c->stage_mode == MOE_STAGE_KERNEL;
    uint64_t* list = kernel ? c->copy_list + 2 * (size_t)layer * c->E : nullptr;  // guarded by table_done too
    // from here on the pinned table is being rewritten: a failure leaves it
    // holding a partial mapping that moe_cache_replace must not upload
    auto fail = [&](hipError_t e) {
        c->table_written[layer] = false;
        return hip_fail(e);
    };
    int i = 0;
    for (int e = 0; e < c->E; ++e) {
        const int slot = c->slot_of[(size_t)layer * c->E + e];
        if (slot >= 0) {
            table[e] = c->pool + (size_t)slot * c->eb;
        } else {
            char* dst = stage + (size_t)i * c->eb;
            if (c->fault) {
                const int injected = c->fault(c->fault_user, layer, i, e);
                if (injected != 0) return fail(static_cast<hipError_t>(injected));
            }
            if (kernel) {
                void* src = nullptr;
                const hipError_t err = hipHostGetDevicePointer(&src, const_cast<void*>(host_src[e]), 0);
                if (err != hipSuccess) return fail(err);
                list[2 * i] = (uint64_t)(uintptr_t)src;
                list[2 * i + 1] = (uint64_t)(uintptr_t)dst;
            } else {
                const hipError_t err = hipMemcpyAsync(dst, host_src[e], c->eb, hipMemcpyHostToDevice, st);
                if (err != hipSuccess) return fail(err);
            }
            table[e] = dst;
            ++i;
        }
    }
    hipError_t err;
    if (kernel && i > 0) {
        void* dlist = nullptr;
        err = hipHostGetDevicePointer(&dlist, list, 0);
        if (err != hipSuccess) return fail(err);
        stage_copy<<<c->copy_workgroups, 256, 0, st>>>(static_cast<const uint64_t*>(dlist), i, (uint32_t)(c->eb / 16));
        const int rc = check_launch();
        if (rc) {
            c->table_written[layer] = false;
            return rc;
        }
    }
    err = hipMemcpyAsync(dev_table, table, sizeof(void*) * (size_t)c->E, hipMemcpyHostToDevice, st);
    if (err != hipSuccess) return fail(err);
    err = hipEventRecord(c->table_done[layer], st);
    if (err != hipSuccess) return fail(err);
    c->table_pending[layer] = true;
    c->table_written[layer] = true;
    if (done) {
        err = hipEventRecord(reinterpret_cast<hipEvent_t>(done), st);
        if (err != hipSuccess) return hip_fail(err);
    }
    return MOE_OK;
}

int moe_cache_map_host(moe_cache* c, int layer, const void* const* host_src, void** dev_table, moe_stream_t s,
                       moe_event_t done) {
    if (!c || layer < 0 || layer >= c->n_layers || !host_src || !dev_table) return MOE_ERR_INVALID_ARG;
    for (int e = 0; e < c->E; ++e)
        if (c->slot_of[(size_t)layer * c->E + e] < 0 && !host_src[e]) return MOE_ERR_INVALID_ARG;
    if (c->table_pending[layer]) {
        const hipError_t e = hipEventSynchronize(c->table_done[layer]);
        if (e != hipSuccess) return hip_fail(e);
        c->table_pending[layer] = false;
    }
    void** table = c->tables + (size_t)layer * c->E;
    for (int e = 0; e < c->E; ++e) {
        const int slot = c->slot_of[(size_t)layer * c->E + e];
        if (slot >= 0) {
            table[e] = c->pool + (size_t)slot * c->eb;
        } else {
            void* dptr = nullptr;
            const hipError_t err = hipHostGetDevicePointer(&dptr, const_cast<void*>(host_src[e]), 0);
            if (err != hipSuccess) return hip_fail(err);
            table[e] = dptr;
        }
    }
    const hipStream_t st = as_stream(s);
    hipError_t err = hipMemcpyAsync(dev_table, table, sizeof(void*) * (size_t)c->E, hipMemcpyHostToDevice, st);
    if (err != hipSuccess) return hip_fail(err);
    err = hipEventRecord(c->table_done[layer], st);
    if (err != hipSuccess) return hip_fail(err);
    c->table_pending[layer] = true;
    c->table_written[layer] = true;
    if (done) {
        err = hipEventRecord(reinterpret_cast<hipEvent_t>(done), st);
        if (err != hipSuccess) return hip_fail(err);
    }
    return MOE_OK;
}

int moe_usage_accumulate(int32_t* usage, const int32_t* counts, int E, moe_stream_t s) {
    if (!usage || !counts || E < 1) return MOE_ERR_INVALID_ARG;
    usage_accumulate<<<(E + 255) / 256, 256, 0, as_stream(s)>>>(usage, counts, E);
    return check_launch();
}

int moe_cache_replace(moe_cache* c, int n, const int32_t* evict_ids, const int32_t* admit_ids,
                      const void* const* host_src, void** dev_tables, moe_stream_t s) {
    if (!c || n < 0) return MOE_ERR_INVALID_ARG;
    if (n == 0) return MOE_OK;
    if (!evict_ids || !admit_ids || !host_src || !dev_tables) return MOE_ERR_INVALID_ARG;
    const long total = (long)c->n_layers * c->E;
    std::vector<char> seen(total, 0);
    for (int i = 0; i < n; ++i) {
        const int32_t v = evict_ids[i], a = admit_ids[i];
        if (v < 0 || v >= total || a < 0 || a >= total || seen[v] || seen[a] || v == a) return MOE_ERR_INVALID_ARG;
        seen[v] = seen[a] = 1;
        if (c->slot_of[v] < 0 || c->slot_of[a] >= 0 || !host_src[v] || !host_src[a]) return MOE_ERR_INVALID_ARG;
    }
    // device addresses of the evicted experts' host blobs, before anything changes
    std::vector<void*> vdev(n);
    for (int i = 0; i < n; ++i) {
        const hipError_t e = hipHostGetDevicePointer(&vdev[i], const_cast<void*>(host_src[evict_ids[i]]), 0);
        if (e != hipSuccess) return hip_fail(e);
    }
    std::vector<char> touched(c->n_layers, 0);
    for (int i = 0; i < n; ++i) {
        touched[evict_ids[i] / c->E] = 1;
        touched[admit_ids[i] / c->E] = 1;
    }
    for (int l = 0; l < c->n_layers; ++l)
        if (touched[l] && c->table_pending[l]) {
            const hipError_t e = hipEventSynchronize(c->table_done[l]);
            if (e != hipSuccess) return hip_fail(e);
            c->table_pending[l] = false;
        }
    const hipStream_t st = as_stream(s);
    for (int i = 0; i < n; ++i) {
        const int32_t v = evict_ids[i], a = admit_ids[i];
        const int slot = c->slot_of[v];
        char* dst = c->pool + (size_t)slot * c->eb;
        const hipError_t e = hipMemcpyAsync(dst, host_src[a], c->eb, hipMemcpyHostToDevice, st);
        if (e != hipSuccess) return hip_fail(e);
        c->slot_of[v] = -1;
        c->slot_of[a] = slot;
        c->tables[v] = vdev[i];
        c->tables[a] = dst;
    }
    for (int l = 0; l < c->n_layers; ++l) {
        if (!touched[l] || !c->table_written[l]) continue;
        hipError_t e = hipMemcpyAsync(dev_tables + (size_t)l * c->E, c->tables + (size_t)l * c->E,
                                      sizeof(void*) * (size_t)c->E, hipMemcpyHostToDevice, st);
        if (e != hipSuccess) return hip_fail(e);
        e = hipEventRecord(c->table_done[l], st);
        if (e != hipSuccess) return hip_fail(e);
        c->table_pending[l] = true;
    }
    return MOE_OK;
}

}  // extern "C"

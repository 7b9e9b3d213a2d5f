// Expert slot cache: host bookkeeping of which global expert occupies which
// slot of a caller-owned HBM pool, and per-layer pointer tables for the
// misses: staged from pinned host memory on a (side) stream, or (decode)
// pointing at the pinned host blobs themselves, read in place by the FFN.
// "How Strata works" (adaptive expert cache section) loads the most-used
// ~4,500 experts by a usage ranking into GPU memory; "Strata benchmarks"
// (prefill optimisation table) streams the next layer's experts over PCIe
// while the current layer computes.
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
};

using namespace moe;

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
    c->table_done.assign(n_layers, nullptr);
    c->table_pending.assign(n_layers, false);
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
    delete c;
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
    int i = 0;
    for (int e = 0; e < c->E; ++e) {
        const int slot = c->slot_of[(size_t)layer * c->E + e];
        if (slot >= 0) {
            table[e] = c->pool + (size_t)slot * c->eb;
        } else {
            char* dst = stage + (size_t)i * c->eb;
            const hipError_t err = hipMemcpyAsync(dst, host_src[e], c->eb, hipMemcpyHostToDevice, st);
            if (err != hipSuccess) return hip_fail(err);
            table[e] = dst;
            ++i;
        }
    }
    hipError_t err = hipMemcpyAsync(dev_table, table, sizeof(void*) * (size_t)c->E, hipMemcpyHostToDevice, st);
    if (err != hipSuccess) return hip_fail(err);
    err = hipEventRecord(c->table_done[layer], st);
    if (err != hipSuccess) return hip_fail(err);
    c->table_pending[layer] = true;
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
    if (done) {
        err = hipEventRecord(reinterpret_cast<hipEvent_t>(done), st);
        if (err != hipSuccess) return hip_fail(err);
    }
    return MOE_OK;
}

}  // extern "C"

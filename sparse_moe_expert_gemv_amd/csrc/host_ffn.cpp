// Host-core execution of missed experts ("How Strata works", three-tier
// division and adaptive expert cache: experts not held in GPU memory are
// computed by the CPU from system RAM while the GPU computes the cached ones;
// "Strata benchmarks", calibration: the share of misses sent over PCIe and
// the number of CPU expert threads are tuning knobs).
//
// moe_host_expert_ffn adds, for each (token, expert) item, gate * FFN(x_t) to
// the token's output row, reading the expert's CANONICAL blob (row-major
// block-32 quants, fp16 scales) from host memory.  Float arithmetic: each
// block's sum of x * q is formed in fp32 and multiplied by the block's fp16
// scale, accumulated over the row in fp32; SwiGLU in fp32.  Work is split over
// a persistent thread pool by output rows (gate/up rows, then down rows);
// every output is produced by one thread in a fixed order, so the result does
// not depend on the thread count.  Host code only: no HIP call.
#include <immintrin.h>

#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <functional>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "moe.h"

// Per-CPU clones of the row kernels (dispatched through ifunc resolvers).  A
// ThreadSanitizer build has none: its runtime is not initialised yet when the
// resolvers run.
#if defined(__SANITIZE_THREAD__)
#define MOE_HOST_ISA_CLONES
#else
#define MOE_HOST_ISA_CLONES __attribute__((target_clones("avx512f", "avx2", "default")))
#endif

namespace {

// ---- thread pool -------------------------------------------------------------
// Workers spin briefly on a generation counter (a decode layer issues two
// parallel phases every few tens of microseconds), then block on a condition
// variable.  The calling thread takes tasks too.
class Pool {
   public:
    explicit Pool(int n) : n_(n) {
        // every worker starts from generation 0, also one that the OS starts
        // only after the first run (or the destructor) has advanced it
        for (int i = 0; i < n_ - 1; ++i) th_.emplace_back([this] { worker(0); });
    }
    ~Pool() {
        {
            std::lock_guard<std::mutex> g(m_);
            stop_ = true;
            gen_.fetch_add(1);
        }
        cv_.notify_all();
        for (auto& t : th_) t.join();
    }
    // runs fn(i) for i in [0, n_tasks); returns when all have finished and no
    // worker is still inside this run (so the next run cannot hand one of its
    // tasks to a worker holding this run's function)
    void run(int n_tasks, const std::function<void(int)>& fn) {
        if (n_tasks <= 0) return;
        {
            std::lock_guard<std::mutex> g(m_);
            fn_ = &fn;
            n_tasks_ = n_tasks;
            next_.store(0);
            done_.store(0);
            gen_.fetch_add(1);
        }
        cv_.notify_all();
        work(&fn, n_tasks);
        while (done_.load(std::memory_order_acquire) < n_tasks) std::this_thread::yield();
        {
            std::lock_guard<std::mutex> g(m_);
            fn_ = nullptr;  // no worker joins this run any more
        }
        while (active_.load(std::memory_order_acquire) > 0) std::this_thread::yield();
    }

   private:
    void work(const std::function<void(int)>* fn, int n) {
        for (;;) {
            const int i = next_.fetch_add(1);
            if (i >= n) break;
            (*fn)(i);
            done_.fetch_add(1, std::memory_order_release);
        }
    }
    void worker(uint64_t seen) {
        for (;;) {
            int spins = 0;
            while (gen_.load(std::memory_order_acquire) == seen && spins < 20000) {
                ++spins;
                std::this_thread::yield();
            }
            const std::function<void(int)>* fn;
            int n;
            {
                std::unique_lock<std::mutex> lk(m_);
                cv_.wait(lk, [&] { return gen_.load() != seen; });
                seen = gen_.load();
                if (stop_) return;
                fn = fn_;
                n = n_tasks_;
                if (!fn) continue;
                active_.fetch_add(1);
            }
            work(fn, n);
            active_.fetch_sub(1, std::memory_order_release);
        }
    }
    int n_;
    std::vector<std::thread> th_;
    std::mutex m_;
    std::condition_variable cv_;
    std::atomic<uint64_t> gen_{0};
    std::atomic<int> next_{0}, done_{0}, active_{0};
    const std::function<void(int)>* fn_ = nullptr;
    int n_tasks_ = 0;
    bool stop_ = false;
};

// IEEE binary16 -> fp32 (normal, subnormal, zero; scales are finite)
float half_to_float(uint16_t h) {
    const uint32_t s = (uint32_t)(h >> 15) << 31, e = (h >> 10) & 31, m = h & 1023;
    uint32_t bits;
    if (e == 0) {
        if (m == 0) {
            bits = s;
        } else {  // subnormal: m * 2^-24
            float v = (float)m * 5.9604644775390625e-08f;
            std::memcpy(&bits, &v, 4);
            bits |= s;
        }
    } else if (e == 31) {
        bits = s | 0x7F800000u | (m << 13);
    } else {
        bits = s | ((e + 112) << 23) | (m << 13);
    }
    float f;
    std::memcpy(&f, &bits, 4);
    return f;
}

// every binary16 value as fp32, built once (the block scales are looked up)
const float* half_table() {
    static std::vector<float> t;
    static std::once_flag once;
    std::call_once(once, [] {
        t.resize(65536);
        for (uint32_t h = 0; h < 65536; ++h) t[h] = half_to_float((uint16_t)h);
    });
    return t.data();
}

// Dot product of one canonical quantised row [K] with x, scales sc [K / 32]:
// sum_b s_b * (sum_{i in b} x_i * q_i).  int4: q = u - 8 for the nibble u
// (element 2 i low, 2 i + 1 high), with x split into even (xe) and odd (xo)
// elements and xsum the per-block sums of x, so that sum x q = sum x u -
// 8 sum x.  Sixteen (int4) or thirty-two (int8) lane accumulators over the
// row, added in a fixed tree at the end (so the compiler may vectorise the
// lanes without reordering any sum).
MOE_HOST_ISA_CLONES
float row_dot_i4(const uint8_t* __restrict q, const uint16_t* __restrict sc, const float* __restrict xe,
                 const float* __restrict xo, const float* __restrict xsum, const float* __restrict lut, int K) {
    float acc[16] = {};
    float corr = 0.f;
    for (int b = 0; b < K / 32; ++b) {
        const uint8_t* qb = q + b * 16;
        const float* e = xe + b * 16;
        const float* o = xo + b * 16;
        const float s = lut[sc[b]];
        corr += s * xsum[b];
        for (int i = 0; i < 16; ++i) acc[i] += s * (e[i] * (float)(qb[i] & 15) + o[i] * (float)(qb[i] >> 4));
    }
    for (int w = 8; w > 0; w >>= 1)
        for (int i = 0; i < w; ++i) acc[i] += acc[i + w];
    return acc[0] - 8.f * corr;
}

MOE_HOST_ISA_CLONES
float row_dot_i8(const int8_t* __restrict q, const uint16_t* __restrict sc, const float* __restrict x,
                 const float* __restrict lut, int K) {
    float acc[32] = {};
    for (int b = 0; b < K / 32; ++b) {
        const int8_t* qb = q + b * 32;
        const float* xb = x + b * 32;
        const float s = lut[sc[b]];
        for (int i = 0; i < 32; ++i) acc[i] += s * (xb[i] * (float)qb[i]);
    }
    for (int w = 16; w > 0; w >>= 1)
        for (int i = 0; i < w; ++i) acc[i] += acc[i + w];
    return acc[0];
}

// AVX-512 forms of the two row kernels (chosen at run time where the CPU has
// AVX-512F/BW): per 32-block, the 32 quants are widened to int32 and converted
// to fp32 (int4: the low and high nibbles of 16 bytes, against the even and odd
// elements of x), multiplied with x and summed into a 16-lane block sum by one
// multiply and one fused multiply-add, then scaled by the block's fp16 scale
// into a 16-lane accumulator (two accumulators over alternate blocks, added at
// the end); the lanes are then added in the fixed order of the reduction
// instruction sequence.  Deterministic for a given CPU; the order of the sums
// differs from the portable loops above (same tolerance against the oracle).
#define MOE_AVX512 __attribute__((target("avx512f,avx512bw,f16c")))

MOE_AVX512 static inline void i4_block(const uint8_t* __restrict q, const uint16_t* __restrict sc,
                                       const float* __restrict xe, const float* __restrict xo,
                                       const float* __restrict xsum, int b, __m512& acc, float& corr) {
    const __m512i w = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(q + b * 16)));
    const __m512 lo = _mm512_cvtepi32_ps(_mm512_and_si512(w, _mm512_set1_epi32(15)));
    const __m512 hi = _mm512_cvtepi32_ps(_mm512_srli_epi32(w, 4));
    const __m512 t = _mm512_fmadd_ps(_mm512_loadu_ps(xo + b * 16), hi, _mm512_mul_ps(_mm512_loadu_ps(xe + b * 16), lo));
    const float s = _cvtsh_ss(sc[b]);
    acc = _mm512_fmadd_ps(_mm512_set1_ps(s), t, acc);
    corr += s * xsum[b];
}

MOE_AVX512 float row_dot_i4_avx512(const uint8_t* __restrict q, const uint16_t* __restrict sc,
                                   const float* __restrict xe, const float* __restrict xo,
                                   const float* __restrict xsum, int K) {
    __m512 acc0 = _mm512_setzero_ps(), acc1 = _mm512_setzero_ps();
    float corr0 = 0.f, corr1 = 0.f;
    const int nb = K / 32;
    int b = 0;
    for (; b + 1 < nb; b += 2) {
        i4_block(q, sc, xe, xo, xsum, b, acc0, corr0);
        i4_block(q, sc, xe, xo, xsum, b + 1, acc1, corr1);
    }
    if (b < nb) i4_block(q, sc, xe, xo, xsum, b, acc0, corr0);
    return _mm512_reduce_add_ps(_mm512_add_ps(acc0, acc1)) - 8.f * (corr0 + corr1);
}

MOE_AVX512 static inline void i8_block(const int8_t* __restrict q, const uint16_t* __restrict sc,
                                       const float* __restrict x, int b, __m512& acc) {
    const __m512 a = _mm512_cvtepi32_ps(_mm512_cvtepi8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(q + b * 32))));
    const __m512 c = _mm512_cvtepi32_ps(_mm512_cvtepi8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(q + b * 32 + 16))));
    const __m512 t = _mm512_fmadd_ps(_mm512_loadu_ps(x + b * 32 + 16), c, _mm512_mul_ps(_mm512_loadu_ps(x + b * 32), a));
    acc = _mm512_fmadd_ps(_mm512_set1_ps(_cvtsh_ss(sc[b])), t, acc);
}

MOE_AVX512 float row_dot_i8_avx512(const int8_t* __restrict q, const uint16_t* __restrict sc,
                                   const float* __restrict x, int K) {
    __m512 acc0 = _mm512_setzero_ps(), acc1 = _mm512_setzero_ps();
    const int nb = K / 32;
    int b = 0;
    for (; b + 1 < nb; b += 2) {
        i8_block(q, sc, x, b, acc0);
        i8_block(q, sc, x, b + 1, acc1);
    }
    if (b < nb) i8_block(q, sc, x, b, acc0);
    return _mm512_reduce_add_ps(_mm512_add_ps(acc0, acc1));
}

bool have_avx512() {
    static const bool v = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                          __builtin_cpu_supports("f16c");
    return v;
}

struct Canon {
    size_t qg, qu, qd, sg, su, sd;
};

Canon canon_of(int wfmt, int d, int f) {
    const size_t n = (size_t)d * f;
    const size_t qb = wfmt == MOE_WFMT_I4B32 ? n / 2 : n;
    const size_t sb = (n / 32) * 2;
    return Canon{0, qb, 2 * qb, 3 * qb, 3 * qb + sb, 3 * qb + 2 * sb};
}

// the row's operand in the layout row_dot_* wants
struct RowInput {
    std::vector<float> x, xe, xo, xsum;
    void set(const float* v, int K) {
        x.assign(v, v + K);
        xe.resize(K / 2);
        xo.resize(K / 2);
        xsum.resize(K / 32);
        for (int i = 0; i < K / 2; ++i) {
            xe[i] = v[2 * i];
            xo[i] = v[2 * i + 1];
        }
        for (int b = 0; b < K / 32; ++b) {
            float s = 0.f;
            for (int i = 0; i < 32; ++i) s += v[32 * b + i];
            xsum[b] = s;
        }
    }
    float dot(const uint8_t* blob, size_t qoff, size_t soff, int row, int K, int wfmt, const float* lut) const {
        const uint16_t* sc = reinterpret_cast<const uint16_t*>(blob + soff) + (size_t)row * (K / 32);
        if (wfmt == MOE_WFMT_I4B32) {
            const uint8_t* q = blob + qoff + (size_t)row * (K / 2);
            if (have_avx512()) return row_dot_i4_avx512(q, sc, xe.data(), xo.data(), xsum.data(), K);
            return row_dot_i4(q, sc, xe.data(), xo.data(), xsum.data(), lut, K);
        }
        const int8_t* q = reinterpret_cast<const int8_t*>(blob + qoff) + (size_t)row * K;
        if (have_avx512()) return row_dot_i8_avx512(q, sc, x.data(), K);
        return row_dot_i8(q, sc, x.data(), lut, K);
    }
};

}  // namespace

struct moe_host_pool {
    Pool pool;
    explicit moe_host_pool(int n) : pool(n) {}
};

extern "C" {

int moe_host_pool_create(int n_threads, moe_host_pool** out) {
    if (!out || n_threads < 1 || n_threads > 256) return MOE_ERR_INVALID_ARG;
    *out = nullptr;
    try {
        *out = new moe_host_pool(n_threads);
    } catch (...) {
        return MOE_ERR_NO_MEMORY;
    }
    return MOE_OK;
}

int moe_host_pool_destroy(moe_host_pool* p) {
    delete p;
    return MOE_OK;
}

int moe_host_expert_ffn(moe_host_pool* p, int n_items, const int32_t* item_token, const float* item_gate,
                        const void* const* item_blob, int wfmt, int T, int d, int f, const float* x, float* out) {
    if (!p || n_items < 0 || T < 0 || d <= 0 || f <= 0 || d % 32 || f % 32 ||
        (wfmt != MOE_WFMT_I4B32 && wfmt != MOE_WFMT_I8B32))
        return MOE_ERR_INVALID_ARG;
    if (n_items == 0) return MOE_OK;
    if (!item_token || !item_gate || !item_blob || !x || !out) return MOE_ERR_INVALID_ARG;
    for (int i = 0; i < n_items; ++i)
        if (item_token[i] < 0 || item_token[i] >= T || !item_blob[i]) return MOE_ERR_INVALID_ARG;
    const Canon C = canon_of(wfmt, d, f);
    try {
        const float* lut = half_table();
        std::vector<RowInput> xin(n_items), hin(n_items);
        std::vector<float> g((size_t)n_items * f), u((size_t)n_items * f), y((size_t)n_items * d);
        for (int i = 0; i < n_items; ++i) xin[i].set(x + (size_t)item_token[i] * d, d);
        // phase 1: gate and up rows, 64 rows per task
        const int gr = (f + 63) / 64;
        p->pool.run(n_items * gr, [&](int task) {
            const int i = task / gr, r0 = (task % gr) * 64, r1 = std::min(f, r0 + 64);
            const uint8_t* blob = static_cast<const uint8_t*>(item_blob[i]);
            for (int n = r0; n < r1; ++n) {
                g[(size_t)i * f + n] = xin[i].dot(blob, C.qg, C.sg, n, d, wfmt, lut);
                u[(size_t)i * f + n] = xin[i].dot(blob, C.qu, C.su, n, d, wfmt, lut);
            }
        });
        std::vector<float> hrow(f);
        for (int i = 0; i < n_items; ++i) {
            for (int n = 0; n < f; ++n) {
                const float z = g[(size_t)i * f + n];
                hrow[n] = z / (1.f + std::exp(-z)) * u[(size_t)i * f + n];
            }
            hin[i].set(hrow.data(), f);
        }
        // phase 2: down rows, 128 rows per task
        const int dr = (d + 127) / 128;
        p->pool.run(n_items * dr, [&](int task) {
            const int i = task / dr, r0 = (task % dr) * 128, r1 = std::min(d, r0 + 128);
            const uint8_t* blob = static_cast<const uint8_t*>(item_blob[i]);
            for (int o = r0; o < r1; ++o) y[(size_t)i * d + o] = hin[i].dot(blob, C.qd, C.sd, o, f, wfmt, lut);
        });
        // gate-weighted sum into the token rows, items in the given order
        for (int i = 0; i < n_items; ++i) {
            float* orow = out + (size_t)item_token[i] * d;
            const float gi = item_gate[i];
            for (int o = 0; o < d; ++o) orow[o] += gi * y[(size_t)i * d + o];
        }
    } catch (const std::bad_alloc&) {
        return MOE_ERR_NO_MEMORY;
    }
    return MOE_OK;
}

}  // extern "C"

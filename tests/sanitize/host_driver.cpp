// Runs the library's host-only code -- the adaptive cache's replacement plan
// (csrc/cache_plan.cpp) and the host-core expert FFN with its thread pool
// (csrc/host_ffn.cpp) -- on seeded inputs, so that it can be built and run
// under AddressSanitizer + UndefinedBehaviorSanitizer and ThreadSanitizer.
// Test infrastructure only.  Exit status 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "moe.h"

static int fail(const char* what) {
    std::fprintf(stderr, "check failed: %s\n", what);
    return 1;
}

int main(int argc, char** argv) {
    const int reps = argc > 1 ? std::atoi(argv[1]) : 50;
    std::mt19937 rng(12345);
    // ---- replacement plan: the pairs keep the rule's invariants ----
    for (int it = 0; it < 40; ++it) {
        const int n = 1 + (int)(rng() % 3000);
        std::vector<uint8_t> res(n);
        std::vector<float> score(n);
        for (int g = 0; g < n; ++g) {
            res[g] = (uint8_t)(rng() % 3 == 0);
            score[g] = (float)(rng() % 50) * 0.5f;  // many ties
        }
        const int max_swaps = (int)(rng() % 200);
        std::vector<int32_t> ev(max_swaps + 1), ad(max_swaps + 1);
        int ns = -1;
        if (moe_cache_plan(n, res.data(), score.data(), max_swaps, 0.0f, ev.data(), ad.data(), &ns) != MOE_OK)
            return fail("plan status");
        if (ns < 0 || ns > max_swaps) return fail("plan count");
        for (int i = 0; i < ns; ++i) {
            if (!res[ev[i]] || res[ad[i]]) return fail("plan pairs resident/missing");
            if (!(score[ad[i]] > score[ev[i]])) return fail("plan pair scores");
        }
    }
    // ---- host expert FFN: thread-count independence, many back-to-back runs ----
    for (int wfmt : {MOE_WFMT_I4B32, MOE_WFMT_I8B32}) {
        const int d = 256, f = 128, T = 3, E = 5;
        const size_t n = (size_t)d * f, qb = wfmt == MOE_WFMT_I4B32 ? n / 2 : n, eb = 3 * qb + 3 * (n / 32) * 2;
        std::vector<std::vector<uint8_t>> blobs(E, std::vector<uint8_t>(eb));
        for (auto& b : blobs) {
            for (size_t i = 0; i < 3 * qb; ++i) b[i] = (uint8_t)(rng() & 0xFF);
            for (size_t i = 3 * qb; i < eb; i += 2) {  // fp16 scales in [2^-9, 2^-8)
                const uint16_t h = (uint16_t)(0x1800 | (rng() & 0x3FF));
                std::memcpy(&b[i], &h, 2);
            }
        }
        std::vector<float> x((size_t)T * d);
        std::normal_distribution<float> nd(0.f, 1.f);
        for (auto& v : x) v = nd(rng);
        std::vector<float> ref;
        for (int threads : {1, 3, 8}) {
            moe_host_pool* pool = nullptr;
            if (moe_host_pool_create(threads, &pool) != MOE_OK) return fail("pool create");
            for (int r = 0; r < reps; ++r) {
                const int items = 1 + (r % 7);
                std::vector<int32_t> tok(items);
                std::vector<float> gate(items);
                std::vector<const void*> bp(items);
                for (int i = 0; i < items; ++i) {
                    tok[i] = (i * 2 + r) % T;
                    gate[i] = 0.125f * (float)(i + 1);
                    bp[i] = blobs[(i + r) % E].data();
                }
                std::vector<float> out((size_t)T * d, 0.f);
                if (moe_host_expert_ffn(pool, items, tok.data(), gate.data(), bp.data(), wfmt, T, d, f, x.data(),
                                        out.data()) != MOE_OK)
                    return fail("host ffn status");
                if (r == reps - 1) {
                    if (ref.empty()) ref = out;
                    else if (std::memcmp(ref.data(), out.data(), sizeof(float) * out.size()) != 0)
                        return fail("host ffn depends on the pool size");
                }
            }
            moe_host_pool_destroy(pool);
        }
    }
    std::puts("host driver ok");
    return 0;
}

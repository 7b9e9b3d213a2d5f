// Replacement plan of the adaptive expert cache ("How Strata works",
// adaptive expert cache section: the cache keeps learning which experts the
// session uses).  Host code only, no HIP: it pairs the strongest missing
// experts with the weakest resident ones.  Kept apart from the device code so
// that it builds with any host compiler (and its sanitizers).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "moe.h"

extern "C" {

int moe_cache_plan(int n_total, const uint8_t* resident, const float* score, int max_swaps, float margin,
                   int32_t* evict_ids, int32_t* admit_ids, int* n_swaps) {
    if (n_total < 1 || !resident || !score || max_swaps < 0 || !n_swaps || !(margin >= 0.0f) ||
        !std::isfinite(margin) || (max_swaps > 0 && (!evict_ids || !admit_ids)))
        return MOE_ERR_INVALID_ARG;
    std::vector<int32_t> in, out;
    for (int g = 0; g < n_total; ++g) {
        if (resident[g] > 1 || !(score[g] >= 0.0f) || !std::isfinite(score[g])) return MOE_ERR_INVALID_ARG;
        (resident[g] ? in : out).push_back(g);
    }
    const int m = std::min<int>(max_swaps, (int)std::min(in.size(), out.size()));
    // the m weakest residents (score ascending, lower id first) and the m
    // strongest missing ids (score descending, lower id first)
    auto weaker = [&](int32_t a, int32_t b) { return score[a] < score[b] || (score[a] == score[b] && a < b); };
    auto stronger = [&](int32_t a, int32_t b) { return score[a] > score[b] || (score[a] == score[b] && a < b); };
    std::partial_sort(in.begin(), in.begin() + m, in.end(), weaker);
    std::partial_sort(out.begin(), out.begin() + m, out.end(), stronger);
    int n = 0;
    while (n < m && score[out[n]] > (1.0f + margin) * score[in[n]]) {
        evict_ids[n] = in[n];
        admit_ids[n] = out[n];
        ++n;
    }
    *n_swaps = n;
    return MOE_OK;
}

}  // extern "C"

// Adaptive residency policy on the host: the running routing score of each
// expert and the swap plan that moves the experts a layer calls most onto
// the card (bloomery V4.1 README, "Adaptive residency": the engine counts its
// own routing and swaps experts between card and host between steps; a
// prompt call streams its hottest host experts onto the card).  Interface
// and rule: include/qmoe_host.h.
//
// The counts come from the device (moe_route_and_batch / moe_count_routes
// add every routed pair to its expert's counter); this file only turns them
// into decisions.  Integer arithmetic throughout, so a plan is a pure
// function of its inputs.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <numeric>
#include <string>
#include <vector>

#include "qmoe.h"
#include "qmoe_host.h"

namespace qmoe_host {
__attribute__((visibility("hidden"))) int set_error(int status, const char* msg);  // host_leg.cpp
}

namespace {

int fail(int status, const char* fmt, ...) {
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    return qmoe_host::set_error(status, buf);
}

}  // namespace

extern "C" int moe_residency_update_scores(uint64_t* score, const uint32_t* window, int E, int decay_shift) {
    if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARGUMENT, "E = %d outside 1..%d", E, MOE_MAX_EXPERTS);
    if (decay_shift < 0 || decay_shift > 63)
        return fail(MOE_ERR_INVALID_ARGUMENT, "decay_shift = %d outside 0..63", decay_shift);
    if (!score || !window) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL score or window");
    for (int e = 0; e < E; ++e)
        score[e] = score[e] - (score[e] >> decay_shift) + ((uint64_t)window[e] << MOE_RESIDENCY_FRAC_BITS);
    return MOE_OK;
}

extern "C" int moe_residency_plan(const uint64_t* score, int E, const int32_t* slot_of_expert, int max_swaps,
                                  uint64_t margin, int32_t* incoming, int32_t* outgoing, int* n_swaps) {
    if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARGUMENT, "E = %d outside 1..%d", E, MOE_MAX_EXPERTS);
    if (max_swaps < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "max_swaps = %d is negative", max_swaps);
    if (!score || !slot_of_expert || !n_swaps || (max_swaps > 0 && (!incoming || !outgoing)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    // a before b: higher score, then lower id (a strict total order)
    auto before = [score](int a, int b) { return score[a] != score[b] ? score[a] > score[b] : a < b; };
    std::vector<int> host, res;
    host.reserve(E);
    res.reserve(E);
    for (int e = 0; e < E; ++e) (slot_of_expert[e] < 0 ? host : res).push_back(e);
    const size_t n = std::min<size_t>({host.size(), res.size(), (size_t)max_swaps});
    // Only the first n of each side can take part: the n best host experts,
    // the n worst resident ones.
    std::partial_sort(host.begin(), host.begin() + n, host.end(), before);
    std::partial_sort(res.begin(), res.begin() + n, res.end(), [&](int a, int b) { return before(b, a); });
    int m = 0;
    for (size_t i = 0; i < n; ++i) {
        const uint64_t s_in = score[host[i]], s_out = score[res[i]];
        // s_in > s_out + margin, without overflow
        if (s_in <= s_out || s_in - s_out <= margin) break;
        incoming[m] = host[i];
        outgoing[m] = res[i];
        ++m;
    }
    *n_swaps = m;
    return MOE_OK;
}

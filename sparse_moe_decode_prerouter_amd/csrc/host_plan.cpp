// The host-side sticky-slot planner of the staging path (no device code, no
// HIP headers): compiled into the library, and on its own with the address
// and undefined-behaviour sanitizers by the CPU tests.
//
// The plan (Guide, Key terms: staged decode, fixed-slot slab): experts the
// next call routes to that already sit in a slot keep it; each missing one,
// in ascending expert id, takes the next slot, in ascending slot order, that
// holds no wanted expert. Only those copies are made.
#include <algorithm>
#include <vector>

#include "moe_prerouter.h"

extern "C" int moe_plan_slots(int32_t* resident, int n_slots, const int32_t* wanted, int n_wanted, int n_experts,
                              int32_t* copies_slot, int32_t* copies_expert, int* n_copies) {
    if (!resident || n_slots < 0 || n_experts <= 0 || n_wanted < 0 || (n_wanted && !wanted) || !n_copies)
        return MOE_E_INVALID;
    std::vector<int32_t> want(wanted, wanted + n_wanted);
    for (int32_t e : want)
        if (e < 0 || e >= n_experts) return MOE_E_INVALID;
    // a slot table holds an expert at most once (an entry outside [0, E)
    // is an empty slot)
    std::vector<char> present(n_experts, 0);
    for (int s = 0; s < n_slots; ++s) {
        const int32_t e = resident[s];
        if (e < 0 || e >= n_experts) continue;
        if (present[e]) return MOE_E_INVALID;
        present[e] = 1;
    }
    std::sort(want.begin(), want.end());
    want.erase(std::unique(want.begin(), want.end()), want.end());
    if ((int)want.size() > n_slots) return MOE_E_CAPACITY;
    std::vector<char> wanted_flag(n_experts, 0);
    for (int32_t e : want) wanted_flag[e] = 1;
    std::vector<int> free_slots;
    for (int s = 0; s < n_slots; ++s)
        if (!(resident[s] >= 0 && resident[s] < n_experts && wanted_flag[resident[s]])) free_slots.push_back(s);
    // missing experts <= free slots: the slots holding wanted experts hold
    // distinct ones, so n_slots - |free| = |wanted and present|
    int nc = 0;
    size_t fi = 0;
    for (int32_t e : want) {
        if (present[e]) continue;
        const int s = free_slots[fi++];
        resident[s] = e;
        if (copies_slot) copies_slot[nc] = s;
        if (copies_expert) copies_expert[nc] = e;
        ++nc;
    }
    *n_copies = nc;
    return MOE_OK;
}

// Randomised checks of the host sticky-slot planner (moe_plan_slots), built
// with the address and undefined-behaviour sanitizers by
// tests/test_host_sanitizers.py. Each case checks the return code against the
// inputs and, on success, the plan's properties: every wanted expert resident
// exactly once, slots that held a wanted expert unchanged, one copy per missing
// expert (ascending ids into ascending free slots), other slots untouched; on
// an error the table is unchanged.
#include <algorithm>
#include <cstdio>
#include <cstdint>
#include <random>
#include <set>
#include <vector>

#include "moe_prerouter.h"

static int fail(int c, const char* what) {
    std::printf("case %d: %s\n", c, what);
    return 1;
}

int main() {
    std::mt19937 rng(12345);
    auto U = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
    for (int c = 0; c < 20000; ++c) {
        const int E = U(1, 40), S = U(0, 12), W = U(0, 16);
        std::vector<int32_t> res(S), want(W);
        // distinct residents mostly; sometimes a duplicate or an id outside [0, E)
        std::vector<int32_t> perm(E);
        for (int e = 0; e < E; ++e) perm[e] = e;
        std::shuffle(perm.begin(), perm.end(), rng);
        for (int s = 0; s < S; ++s) res[s] = (s < E && U(0, 3)) ? perm[s] : -1;
        const bool dup = S >= 2 && U(0, 9) == 0;
        if (dup) res[U(0, S - 1)] = res[U(0, S - 1)];
        if (S && U(0, 19) == 0) res[U(0, S - 1)] = E + U(0, 3);
        const bool bad_w = W && U(0, 19) == 0;
        for (int w = 0; w < W; ++w) want[w] = U(0, E - 1);
        if (bad_w) want[U(0, W - 1)] = U(0, 1) ? -1 - U(0, 3) : E + U(0, 3);
        // expected code
        std::set<int32_t> held_set;
        bool has_dup = false;
        for (int32_t e : res)
            if (e >= 0 && e < E) has_dup |= !held_set.insert(e).second;
        std::set<int32_t> wset;
        bool out_w = false;
        for (int32_t e : want) {
            if (e < 0 || e >= E) out_w = true;
            else wset.insert(e);
        }
        int exp_rc = MOE_OK;
        if (out_w || has_dup) exp_rc = MOE_E_INVALID;
        else if ((int)wset.size() > S) exp_rc = MOE_E_CAPACITY;
        std::vector<int32_t> before = res, cs(S + 1, -7), ce(S + 1, -7);
        int nc = -1;
        int32_t none = -1;                    // a table of no slots is still a pointer
        const int rc = moe_plan_slots(S ? res.data() : &none, S, want.data(), W, E, cs.data(), ce.data(), &nc);
        if (rc != exp_rc) return fail(c, "return code");
        if (rc != MOE_OK) {
            if (res != before) return fail(c, "table changed on error");
            continue;
        }
        // every wanted expert resident exactly once
        for (int32_t e : wset)
            if (std::count(res.begin(), res.end(), e) != 1) return fail(c, "wanted expert not resident once");
        // sticky: slots holding a wanted expert keep it
        for (int s = 0; s < S; ++s)
            if (wset.count(before[s]) && res[s] != before[s]) return fail(c, "wanted expert moved");
        // copies: the missing experts, ascending, into ascending free slots
        std::vector<int32_t> missing;
        for (int32_t e : wset)
            if (!held_set.count(e)) missing.push_back(e);
        if (nc != (int)missing.size()) return fail(c, "copy count");
        std::vector<int> free_slots;
        for (int s = 0; s < S; ++s)
            if (!wset.count(before[s])) free_slots.push_back(s);
        for (int i = 0; i < nc; ++i)
            if (ce[i] != missing[i] || cs[i] != free_slots[i] || res[cs[i]] != ce[i]) return fail(c, "copy order");
        // every other slot untouched
        for (int s = 0; s < S; ++s) {
            const bool copied = std::find(cs.begin(), cs.begin() + nc, s) != cs.begin() + nc;
            if (!copied && res[s] != before[s]) return fail(c, "untouched slot changed");
        }
        if (cs[nc] != -7 || ce[nc] != -7) return fail(c, "wrote past the copies");
    }
    // null and size errors
    int nc = 0;
    int32_t r[2] = {-1, -1}, w[1] = {0};
    if (moe_plan_slots(nullptr, 2, w, 1, 4, nullptr, nullptr, &nc) != MOE_E_INVALID) return fail(-1, "null table");
    if (moe_plan_slots(r, 2, nullptr, 1, 4, nullptr, nullptr, &nc) != MOE_E_INVALID) return fail(-1, "null wanted");
    if (moe_plan_slots(r, 2, w, 1, 4, nullptr, nullptr, nullptr) != MOE_E_INVALID) return fail(-1, "null count");
    if (moe_plan_slots(r, 2, w, 1, 0, nullptr, nullptr, &nc) != MOE_E_INVALID) return fail(-1, "no experts");
    if (moe_plan_slots(r, 2, w, 0, 4, nullptr, nullptr, &nc) != MOE_OK || nc != 0) return fail(-1, "empty wanted");
    std::printf("plan_fuzz ok\n");
    return 0;
}

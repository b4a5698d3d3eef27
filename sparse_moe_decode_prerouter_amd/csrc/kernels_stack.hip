// One launch per decode step for a stack of identical layers: K_A and K_B of
// every layer run as work items of a single grid, so no layer waits for a
// kernel boundary and every item issues its weight rows (whose addresses the
// routing fixes before the step starts: layer l's routing is head l-1's
// prediction from the previous token) before it waits for its activations.
//
// Work items are numbered layer by layer, K_A items before K_B items: item
// t is layer t / P, and K_A block (t % P) of it or K_B block (t % P - nA),
// with P = nA + nB. The grid is launched cooperatively (all its blocks are
// resident at once) and block b runs items b, b + G, b + 2G, ... in order.
// An item waits only for items with lower numbers (K_A of layer l for every
// K_B item of layer l - 1, K_B of layer l for every K_A item of layer l):
// the smallest unfinished item's block has finished all its earlier items,
// so it is running that item, whose inputs are complete; every wait ends.
//
// Phase completion (a phase is the K_A or the K_B items of one layer) is
// counted in two levels so that no memory word is hit by more than a few
// dozen atomics per phase (same-word device-scope atomics serialise):
// item i adds one to sub-counter i % kSub; the item that completes a
// sub-counter adds one to the phase's top counter; the one that completes
// the top counter writes the launch's epoch into kFlags copies of the
// phase's flag, and a waiting block polls copy (block % kFlags), so at most
// a few blocks poll any one word. Counters, flags and the epoch sit on
// separate 128-byte lines. The patch kernel that runs before each launch
// zeroes the counters and the abort word and advances the epoch (flags are
// never cleared: a flag is current when it holds this launch's epoch).
//
// The per-layer arguments live in a device table: the pointers fixed when
// the stack is created are written once, and the patch kernel writes the
// per-call ones (activations, routing, predictions, trace) before each
// launch.
#include "device_common.h"
#include "moe_internal.h"
#include "dec_common.h"
#include "fuse_sync.h"
#include "dec_a_body.h"
#include "dec_b_body.h"

namespace moe {

static_assert(kStackFlags <= 64 && kStackSub >= 1, "flags are written by one wave");

struct SyncMap {
    uint32_t* base;
    int n_layers;
    __host__ __device__ uint32_t* line(size_t i) const { return base + i * kStackLine; }
    __host__ __device__ uint32_t* epoch() const { return line(0); }
    __host__ __device__ uint32_t* abort() const { return line(0) + 1; }
    __host__ __device__ uint32_t* sub(int p, int j) const { return line(1 + (size_t)p * kStackSub + j); }
    __host__ __device__ uint32_t* top(int p) const { return line(1 + (size_t)2 * n_layers * kStackSub + p); }
    __host__ __device__ uint32_t* flag(int p, int r) const {
        return line(1 + (size_t)2 * n_layers * (kStackSub + 1) + (size_t)p * kStackFlags + r);
    }
};

// every thread of the block, after the item's last store: item i of phase p
// (n_items items) has arrived
__device__ __forceinline__ void stack_arrive(const SyncMap& m, int p, int i, int n_items, uint32_t epoch) {
    fuse_stores_done();
    if (threadIdx.x < 64) {
        int complete = 0;
        if (threadIdx.x == 0) {
            const int j = i % kStackSub;
            const int nsubs = n_items < kStackSub ? n_items : kStackSub;
            const uint32_t cnt = (uint32_t)((n_items - j + kStackSub - 1) / kStackSub);
            const uint32_t old = __hip_atomic_fetch_add(m.sub(p, j), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old + 1 == cnt) {
                const uint32_t o2 = __hip_atomic_fetch_add(m.top(p), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                complete = o2 + 1 == (uint32_t)nsubs;
            }
        }
        complete = __shfl(complete, 0, 64);
        if (complete && (int)threadIdx.x < kStackFlags)
            __hip_atomic_store(m.flag(p, threadIdx.x), epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int D, int F>
__global__ void __launch_bounds__(kThreads, 2) k_dec_stack(StackDecArgs s) {
    const SyncMap m{s.sync, s.n_layers};
    const uint32_t epoch = __builtin_amdgcn_readfirstlane(ld_dev(m.epoch()));
    const int per_layer = s.nA + s.nB;
    const int total = s.n_layers * per_layer;
    const int rf = blockIdx.x % kStackFlags;
    // the per-layer arguments, read as constant memory (the kernel never
    // writes the table): scalar loads, and pointers known to be global, so
    // waiting for one load never waits for the others
    typedef __attribute__((address_space(4))) const StackLayerArgs CLayerArgs;
    const CLayerArgs* tab = (const CLayerArgs*)s.tab;
    for (int t = blockIdx.x; t < total; t += gridDim.x) {
        const int l = t / per_layer, r = t - l * per_layer;
        const bool role_a = r < s.nA;
        if (role_a) {
            const FuseSync fs{l > 0 ? m.flag(2 * (l - 1) + 1, rf) : nullptr, epoch, m.abort(), s.spin_limit};
            dec_a_body<D, false, true, kStackAPass>(tab[l].a, r, fs);
            stack_arrive(m, 2 * l, r, s.nA, epoch);
        } else {
            const FuseSync fs{m.flag(2 * l, rf), epoch, m.abort(), s.spin_limit};
            dec_b_body<F, true, kStackBPass>(tab[l].b, r - s.nA, fs);
            stack_arrive(m, 2 * l + 1, r - s.nA, s.nB, epoch);
        }
    }
}

// per-call fields of every layer's arguments
__global__ void k_stack_patch(StackPatchArgs p) {
    const SyncMap m{p.sync, p.n_layers};
    if (blockIdx.x == 0) {
        // the step kernel's counters (sub and top lines of every phase) and abort word
        const int n_ctr = 2 * p.n_layers * (kStackSub + 1);
        for (int i = threadIdx.x; i < n_ctr; i += blockDim.x) *m.line(1 + (size_t)i) = 0u;
        if (threadIdx.x == 0) {
            *m.abort() = 0u;
            *m.epoch() = *m.epoch() + 1u;
        }
    }
    const int l = blockIdx.x * blockDim.x + threadIdx.x;
    if (l >= p.n_layers) return;
    StackLayerArgs& L = p.tab[l];
    const size_t per = (size_t)p.n_tok * p.k;
    const size_t xs = (size_t)p.n_tok * p.d;
    const bool last = l + 1 == p.n_layers;
    DecAArgs& a = L.a;
    DecBArgs& b = L.b;
    if (l == 0) a.x = p.x_in;                  // later layers read the exchange copies
    a.n_tok = p.n_tok;
    a.nb_h = p.nb_h;
    a.route_idx = l == 0 ? nullptr : p.route_idx + l * per;
    a.route_w = l == 0 ? nullptr : p.route_w + l * per;
    a.user_used_idx = p.used_idx ? p.used_idx + l * per : nullptr;
    a.user_used_w = p.used_w ? p.used_w + l * per : nullptr;
    if (l == 0) b.x = p.x_in;
    b.y = last ? p.x_out : nullptr;
    b.y_copy = (p.trace && !last) ? p.trace + (l + 1) * xs : nullptr;
    b.n_tok = p.n_tok;
    b.route_idx = a.route_idx;
    b.route_w = a.route_w;
    b.pred_idx = last ? nullptr : p.pred_idx + (l + 1) * per;
    b.pred_w = last ? nullptr : p.pred_w + (l + 1) * per;
    b.hist_cur = last ? nullptr : p.route_idx + (l + 1) * per;
    b.hist_prev = (last || !p.hist_prev) ? nullptr : p.hist_prev + (l + 1) * per;
}

int stack_one_hrows(int d) { return kWaves * kStackAPass * (64 / (d / 32)); }
int stack_one_brows(int f) { return kStackBPass * (64 / (f / 8)); }

bool stack_one_fast_ok(int d, int f, int fs, int n_tok, int k) {
    if (!stack_one_launch_shape_ok(d, f) || (fs && fs != f)) return false;
    const int hr = stack_one_hrows(d), rb = stack_one_brows(f);
    return f % hr == 0 && fs % hr == 0 && d % rb == 0 && n_tok >= 1 && n_tok <= kMaxTokB &&
           n_tok * k <= kMaxAssign && n_tok * rb <= kThreads;
}

bool stack_one_launch_shape_ok(int d, int f) {
    return (d == 256 && f == 128) || (d == 512 && f == 256) || (d == 1024 && f == 512) || (d == 2048 && f == 512) ||
           (d == 2048 && f == 256);
}

template <int D, int F>
static int stack_blocks_per_cu() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_dec_stack<D, F>, kThreads, 0) != hipSuccess) return 1;
    return n > 0 ? n : 1;
}

int stack_one_launch_blocks_per_cu(int d, int f) {
    if (d == 256 && f == 128) return stack_blocks_per_cu<256, 128>();
    if (d == 512 && f == 256) return stack_blocks_per_cu<512, 256>();
    if (d == 1024 && f == 512) return stack_blocks_per_cu<1024, 512>();
    if (d == 2048 && f == 512) return stack_blocks_per_cu<2048, 512>();
    if (d == 2048 && f == 256) return stack_blocks_per_cu<2048, 256>();
    return 0;
}

hipError_t launch_stack_one(const StackPatchArgs& p, const StackDecArgs& s, int grid, hipStream_t st,
                            const KTime* tm) {
    hipLaunchKernelGGL(k_stack_patch, dim3((p.n_layers + 255) / 256), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const void* fn = nullptr;
    if (p.d == 256 && p.f == 128) fn = (const void*)k_dec_stack<256, 128>;
    else if (p.d == 512 && p.f == 256) fn = (const void*)k_dec_stack<512, 256>;
    else if (p.d == 1024 && p.f == 512) fn = (const void*)k_dec_stack<1024, 512>;
    else if (p.d == 2048 && p.f == 512) fn = (const void*)k_dec_stack<2048, 512>;
    else if (p.d == 2048 && p.f == 256) fn = (const void*)k_dec_stack<2048, 256>;
    else return hipErrorInvalidValue;
    StackDecArgs sa = s;
    void* args[] = {&sa};
    if (tm && tm->start) {
        e = hipEventRecord(tm->start, st);
        if (e != hipSuccess) return e;
    }
    e = hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, 0, st);
    if (e != hipSuccess) return e;
    if (tm && tm->stop) e = hipEventRecord(tm->stop, st);
    return e;
}

}  // namespace moe

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
// An item waits only for values published by items with lower numbers (K_A
// of layer l for x, from K_B of layer l - 1; K_B of layer l for h, the
// shared gate, LoRA A u and the head logits, from K_A of layer l): the
// smallest unfinished item's block has finished all its earlier items, so
// it is running that item, whose inputs are complete; every wait ends.
//
// The values carry their own readiness (the hand-off is described with
// fuse_poll): the patch kernel that runs before each launch sets every
// exchange word the launch will publish to the empty word and clears the
// abort word; producers store, consumers read until no word is empty. There
// are no arrival counters and no flags.
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
#include "dec_r_body.h"

namespace moe {

template <int D, int F>
__global__ void __launch_bounds__(kThreads, 2) k_dec_stack(StackDecArgs s) {
    uint32_t* abort = s.sync;
    const int per_layer = s.nA + s.nB;
    const int total = s.n_layers * per_layer;
    // the per-layer arguments, read as constant memory (the kernel never
    // writes the table): scalar loads, and pointers known to be global, so
    // waiting for one load never waits for the others
    typedef __attribute__((address_space(4))) const StackLayerArgs CLayerArgs;
    const CLayerArgs* tab = (const CLayerArgs*)s.tab;
    for (int t = blockIdx.x; t < total; t += gridDim.x) {
        const int l = t / per_layer, r = t - l * per_layer;
        if (r < s.nA) {
            // layer 0 reads the caller's x
            const FuseSync fs{l > 0, abort, s.spin_limit};
            dec_a_body<D, false, true, kStackAPass>(tab[l].a, r, fs);
        } else {
            const FuseSync fs{true, abort, s.spin_limit};
            dec_b_body<F, true, kStackBPass>(tab[l].b, r - s.nA, fs);
        }
    }
}

// Before each launch: the per-call fields of every layer's arguments, the
// abort word, and the empty word in every exchange word the launch will
// publish. Block pb of npb takes units pb, pb + npb, ..., unit u being
// (layer u / (C + 1), copy u % (C + 1)) of the exchange (C copies per layer;
// copy C stands for the layer's head logits).
__device__ __forceinline__ void stack_patch_body(const StackPatchArgs& p, int pb, int npb) {
    const u32x4 e4 = {kEmptyWord, kEmptyWord, kEmptyWord, kEmptyWord};
    for (int u = pb; u < p.n_layers * (kXchgCopies + 1); u += npb) {
        const int l = u / (kXchgCopies + 1), c = u % (kXchgCopies + 1);
        if (c < kXchgCopies) {
            float* base = p.xchg + ((size_t)l * kXchgCopies + c) * p.xstride;
            // parts start 64 floats apart at least and are padded to it, so a
            // length rounded up to 4 floats stays inside its part
            for (int i = 0; i < kXchgParts; ++i) {
                const uint32_t len = ((uint32_t)p.n_tok * p.xw[i] + 3u) & ~3u;
                for (uint32_t j = 4u * threadIdx.x; j < len; j += 4u * blockDim.x) st_coh4(base + p.xoff[i], j, e4);
            }
        } else {
            double* lg = p.tab[l].a.logits_h;
            const int n = lg ? p.n_tok * p.tab[l].b.En : 0;
            for (int j = threadIdx.x; j < n; j += blockDim.x)
                __hip_atomic_store(lg + j, __longlong_as_double(-1ll), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (pb == 0 && threadIdx.x == 0) *p.sync = 0u;     // the abort word
    const int l = pb * blockDim.x + threadIdx.x;
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

// The launch before the step kernel: blocks [0, nb_r) route layer 0's rows
// (K_R's body), the others patch the table and mark the exchange empty; the
// two are independent, so the patch's stores overlap the router's latency.
__global__ void __launch_bounds__(kThreads) k_stack_prep(StackPatchArgs p, DecAArgs a, RouteArgs r, int nb_r) {
    extern __shared__ __align__(16) uint8_t lds[];
    if ((int)blockIdx.x < nb_r) dec_r_body(a, r, (int)blockIdx.x, nb_r, (float*)lds);
    else stack_patch_body(p, (int)blockIdx.x - nb_r, (int)gridDim.x - nb_r);
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

hipError_t launch_stack_one(const StackPatchArgs& p, const DecAArgs& a0, const RouteArgs& r0,
                            const StackDecArgs& s, int grid, hipStream_t st, const KTime* tprep, const KTime* tm) {
    if (a0.d > 2048) return hipErrorInvalidValue;
    const int nb_r = dec_r_blocks(r0.E);
    const int pgrid = std::max(p.n_layers * (kXchgCopies + 1), (p.n_layers + kThreads - 1) / kThreads);
    MOE_LAUNCH(k_stack_prep, dim3(nb_r + pgrid), dim3(kThreads), (size_t)a0.d * 4, st, tprep, p, a0, r0, nb_r);
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

// Host runtime of the MoE block library: the C ABI declared in
// include/moe_prerouter.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "moe_internal.h"

using namespace moe;

namespace {

thread_local int g_last_hip = 0;

#define HIPCHK(x)                                              \
    do {                                                       \
        hipError_t e_ = (x);                                   \
        if (e_ != hipSuccess) { g_last_hip = (int)e_; return MOE_E_HIP; } \
    } while (0)

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Carver {
    uint8_t* base;
    size_t off = 0;
    template <class T>
    T* take(size_t count) {
        off = align_up(off, 256);
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
};

int validate_desc(const moe_layer_desc* d) {
    if (!d) return MOE_E_INVALID;
    if (d->d_model <= 0 || d->n_experts <= 0 || d->top_k <= 0 || d->d_ff <= 0 || d->max_tokens <= 0)
        return MOE_E_INVALID;
    if (d->group_size != kGroup) return MOE_E_UNSUPPORTED;
    if (d->d_model % 256 || d->d_model > 8192) return MOE_E_UNSUPPORTED;
    if (d->d_ff % 64 || d->d_ff > 8192) return MOE_E_UNSUPPORTED;
    if (d->d_ff_shared != 0 && d->d_ff_shared != d->d_ff) return MOE_E_UNSUPPORTED;
    if (d->d_ff_shared < 0) return MOE_E_INVALID;
    if (d->top_k > kMaxTopK || d->top_k > d->n_experts || d->n_experts > kMaxExperts) return MOE_E_UNSUPPORTED;
    if (d->lora_rank < 0 || d->lora_rank > 64) return MOE_E_UNSUPPORTED;
    if (d->act_dtype != MOE_ACT_F32 && d->act_dtype != MOE_ACT_BF16) return MOE_E_INVALID;
    if (d->next_n_experts < 0 || d->next_n_experts > kMaxExperts) return MOE_E_UNSUPPORTED;
    if (d->next_n_experts > 0 && (d->next_top_k <= 0 || d->next_top_k > kMaxTopK || d->next_top_k > d->next_n_experts))
        return MOE_E_UNSUPPORTED;
    if (d->max_tokens > 8192) return MOE_E_UNSUPPORTED;
    const bool resident = d->flags & MOE_RESIDENT_STORE;
    if (!resident && (d->slab_slots < 1 || d->slab_slots > 64)) return MOE_E_UNSUPPORTED;
    if (d->flags & ~(MOE_FUSE_NORM_RESIDUAL | MOE_RESIDENT_STORE)) return MOE_E_INVALID;
    return MOE_OK;
}

size_t carve(const moe_layer_desc* d, uint8_t* base, Scratch* s) {
    Carver c{base};
    Scratch tmp;
    Scratch& S = s ? *s : tmp;
    const size_t T = d->max_tokens, D = d->d_model, E = d->n_experts, K = d->top_k;
    const size_t En = d->next_n_experts > 0 ? d->next_n_experts : 1, Kn = d->next_top_k > 0 ? d->next_top_k : 1;
    const bool resident = d->flags & MOE_RESIDENT_STORE;
    const size_t blob = 27ull * D * d->d_ff / 16;
    const size_t slots = resident ? 0 : (size_t)d->slab_slots;
    const bool f32 = d->act_dtype == MOE_ACT_F32;
    const size_t nas = std::min(E, T * K);
    S.err = c.take<int32_t>(64);
    S.counters = c.take<uint32_t>(16);
    S.slot_of = c.take<int32_t>(E);
    S.slot_tag = c.take<int32_t>(slots + 1);
    S.slab = resident ? nullptr : c.take<uint8_t>((slots + (d->d_ff_shared ? 1 : 0)) * blob);
    S.u_pk = c.take<uint32_t>(T * D / 2);
    S.u_pk_lo = f32 ? c.take<uint32_t>(T * D / 2) : nullptr;
    // the routing GEMM's fragment-ordered operands (bf16 activations)
    const size_t T16 = (T + 15) / 16 * 16;
    S.u_frag = f32 ? nullptr : c.take<uint32_t>(T16 * D / 2);
    S.wf_router = f32 ? nullptr : c.take<uint32_t>(frag_rows_words((int)E, (int)D));
    S.wf_head = f32 || d->next_n_experts <= 0 ? nullptr : c.take<uint32_t>(frag_rows_words((int)En, (int)D));
    S.wf_lora = f32 || d->lora_rank <= 0 ? nullptr : c.take<uint32_t>(frag_rows_words(d->lora_rank, (int)D));
    S.wf_sgate = f32 || d->d_ff_shared <= 0 ? nullptr : c.take<uint32_t>(frag_rows_words(1, (int)D));
    S.usum = c.take<float>(T * D / 32);
    S.usum_lo = f32 ? c.take<float>(T * D / 32) : nullptr;
    S.logits_r = c.take<double>(T * E);
    S.logits_h = c.take<double>(T * En);
    S.self_idx = c.take<int32_t>(T * K);
    S.self_w = c.take<float>(T * K);
    S.used_idx = c.take<int32_t>(T * K);
    S.used_w = c.take<float>(T * K);
    S.au = c.take<float>(T * std::max(1, d->lora_rank));
    S.sgate = c.take<float>(std::max<size_t>(T, 64));
    S.sort_meta = c.take<int32_t>(8);
    // the digest arrays are at least one wavefront wide: the decode kernels
    // read 64 entries unconditionally and use the valid ones
    S.active = c.take<int32_t>(std::max<size_t>(nas + 1, 64));
    S.act_off = c.take<int32_t>(std::max<size_t>(nas + 1, 64));
    S.perm = c.take<int32_t>(std::max<size_t>(T * K, 64));
    S.wsort = c.take<float>(std::max<size_t>(T * K, 64));
    S.h = c.take<float>(T * K * d->d_ff);
    S.hs = c.take<float>(T * std::max(1, d->d_ff_shared));
    S.tiles = c.take<int32_t>(4 * (size_t)prefill_max_tiles((int)T, (int)K, (int)E));
    S.tiles64 = c.take<int32_t>(4 * (size_t)prefill_max_tiles((int)T, (int)K, (int)E, 64));
    S.ob = c.take<float>(T * K * D);
    S.obs = c.take<float>(T * D);
    (void)Kn;
    return align_up(c.off, 256);
}

ExpertView view_of(const moe_layer* L) {
    ExpertView ev{};
    ev.E = L->desc.n_experts;
    ev.blob = L->blob;
    ev.shared_blob = L->sblob;
    if (L->resident) {
        ev.base = (const uint8_t*)L->w.expert_store;
        ev.slot_of = nullptr;
        ev.slot_tag = nullptr;
        ev.shared = (const uint8_t*)L->w.shared_blob;
        ev.shared_tag = nullptr;
    } else {
        ev.base = L->s.slab;
        ev.slot_of = L->s.slot_of;
        ev.slot_tag = L->s.slot_tag;
        ev.shared = L->desc.d_ff_shared ? L->s.slab + (size_t)L->slots * L->blob : nullptr;
        ev.shared_tag = L->desc.d_ff_shared ? L->s.slot_tag + L->slots : nullptr;
    }
    return ev;
}

// plan + queue the copies for `wanted` (distinct, validated) on stream `cs`
int stage_set(moe_layer* L, const std::vector<int32_t>& wanted, hipStream_t cs) {
    std::vector<int32_t> res(L->h_slot_expert, L->h_slot_expert + L->slots);
    std::vector<int32_t> cslot(L->slots), cexp(L->slots);
    int ncp = 0;
    int rc = moe_plan_slots(res.data(), L->slots, wanted.data(), (int)wanted.size(), L->desc.n_experts,
                            cslot.data(), cexp.data(), &ncp);
    if (rc != MOE_OK) return rc;
    SlotUpdate up{};
    up.n = ncp;
    up.shared_tag = -1;
    up.shared_slot = L->slots;
    for (int i = 0; i < ncp; ++i) {
        const int s = cslot[i], e = cexp[i];
        up.slot[i] = s;
        up.old_e[i] = L->h_slot_expert[s];
        up.new_e[i] = e;
        HIPCHK(hipMemcpyAsync(L->s.slab + (size_t)s * L->blob,
                              (const uint8_t*)L->w.expert_store + (size_t)e * L->blob, L->blob,
                              hipMemcpyHostToDevice, cs));
        L->staged_bytes += L->blob;
    }
    if (L->desc.d_ff_shared && !L->shared_staged) {
        HIPCHK(hipMemcpyAsync(L->s.slab + (size_t)L->slots * L->blob, L->w.shared_blob, L->sblob,
                              hipMemcpyHostToDevice, cs));
        L->staged_bytes += L->sblob;
        up.shared_tag = L->desc.n_experts;
        L->shared_staged = true;
    }
    if (up.n || up.shared_tag >= 0) HIPCHK(launch_slot_update(L->s.slot_of, L->s.slot_tag, up, cs));
    std::copy(res.begin(), res.end(), L->h_slot_expert);
    std::fill(L->h_last_staged, L->h_last_staged + L->slots, -1);
    std::copy(wanted.begin(), wanted.end(), L->h_last_staged);
    L->n_last_staged = (int)wanted.size();
    return MOE_OK;
}

int check_io(const moe_layer* L, const moe_io* io, int n_tok) {
    if (!L || !io || !io->x_in || !io->y_out) return MOE_E_INVALID;
    if (n_tok < 1 || n_tok > L->desc.max_tokens) return MOE_E_INVALID;
    if ((io->route_idx == nullptr) != (io->route_w == nullptr)) return MOE_E_INVALID;
    if (!io->route_idx && !L->w.router) return MOE_E_INVALID;
    if ((io->pred_idx == nullptr) != (io->pred_w == nullptr)) return MOE_E_INVALID;
    if (io->pred_idx && (!L->w.head || L->desc.next_n_experts <= 0)) return MOE_E_INVALID;
    return MOE_OK;
}

int reactive_stage(moe_layer* L, const int32_t* d_idx, int n_tok, hipStream_t st) {
    // the routing exists only on the device now: read it back and stage it
    const size_t nk = (size_t)n_tok * L->desc.top_k;
    HIPCHK(hipMemcpyAsync(L->h_readback, d_idx, nk * sizeof(int32_t), hipMemcpyDeviceToHost, st));
    HIPCHK(hipStreamSynchronize(st));
    std::vector<int32_t> want;
    for (size_t i = 0; i < nk; ++i)
        if (L->h_readback[i] >= 0 && L->h_readback[i] < L->desc.n_experts) want.push_back(L->h_readback[i]);
    std::sort(want.begin(), want.end());
    want.erase(std::unique(want.begin(), want.end()), want.end());
    return stage_set(L, want, st);
}

// merged routing (given rows + self rows) into `dst`, for the reactive read-back
__global__ void k_merge_route(const int32_t* ridx, const int32_t* sidx, int32_t* dst, int n, int k) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int t = i / k;
    dst[i] = (ridx && ridx[(size_t)t * k] >= 0) ? ridx[i] : sidx[i];
}

// nxt: the next stacked layer's prologue for this call's combine to take
// (*took_nxt tells whether it did); skip_pro: this layer's prologue was taken
// by the previous layer's combine
int run_prefill(moe_layer* L, const moe_io* io, int n_tok, hipStream_t st, bool prefill, int route_shift = 0,
                const PrologueArgs* nxt = nullptr, bool skip_pro = false, bool* took_nxt = nullptr);

// defer_in: a previous layer's head top-k to run inside this layer's K_A.
// defer_out (stack mode): this layer's head top-k is not run here but handed
// back, for the next layer's K_A to run (its prediction is for the next step).
int run_decode(moe_layer* L, const moe_io* io, int n_tok, hipStream_t st, const TopkJob* defer_in = nullptr,
               TopkJob* defer_out = nullptr, const PrologueArgs* nxt = nullptr, bool skip_pro = false,
               bool* took_nxt = nullptr) {
    const moe_layer_desc& D = L->desc;
    if (defer_out) defer_out->pred_idx = nullptr;
    if (took_nxt) *took_nxt = false;
    // shapes outside the fused two-kernel path take the general grouped-GEMM path
    if (!dec_fast_path_ok(D.d_model, D.d_ff, D.d_ff_shared, n_tok, D.top_k)) {
        if (defer_in && defer_in->pred_idx) HIPCHK(launch_topk_job(*defer_in, n_tok, st));
        return run_prefill(L, io, n_tok, st, false, 0, nxt, skip_pro, took_nxt);
    }
    const bool fused = D.flags & MOE_FUSE_NORM_RESIDUAL;
    if (L->staged_pending) HIPCHK(hipStreamWaitEvent(st, L->ev_staged, 0));
    const bool need_router = io->route_idx == nullptr || io->self_rows;
    if (need_router && !L->w.router) return MOE_E_INVALID;

    DecAArgs a{};
    a.x = io->x_in;
    a.x_is_bf16 = (!fused && D.act_dtype == MOE_ACT_BF16) ? 1 : 0;
    a.fused = fused; a.gamma = L->w.norm_gamma; a.eps = D.rms_eps;
    a.act_bf16 = D.act_dtype == MOE_ACT_BF16; a.d = D.d_model; a.n_tok = n_tok;
    a.route_idx = io->route_idx; a.route_w = io->route_w;
    a.self_idx = need_router ? L->s.self_idx : nullptr; a.self_w = need_router ? L->s.self_w : nullptr;
    a.k = D.top_k; a.E = D.n_experts;
    a.ev = view_of(L); a.f = D.d_ff; a.fs = D.d_ff_shared;
    a.head = io->pred_idx ? L->w.head : nullptr; a.En = io->pred_idx ? D.next_n_experts : 0;
    a.lora_a = D.lora_rank ? L->w.lora_a : nullptr; a.r = D.lora_rank;
    a.sgate_w = D.d_ff_shared ? L->w.shared_gate : nullptr;
    a.h = L->s.h; a.hs = L->s.hs; a.logits_h = L->s.logits_h; a.au = L->s.au; a.sgate = L->s.sgate;
    a.meta = L->s.sort_meta; a.active = L->s.active; a.act_off = L->s.act_off; a.perm = L->s.perm;
    a.wsort = L->s.wsort;
    a.used_idx = L->s.used_idx; a.used_w = L->s.used_w; a.user_used_idx = io->used_idx; a.user_used_w = io->used_w;
    a.err = L->s.err;
    dec_a_blocks(D.d_model, D.d_ff, D.d_ff_shared, n_tok, D.top_k, D.n_experts, a.En, D.lora_rank,
                 a.sgate_w != nullptr, &a.nb_h, &a.nb_head, &a.nb_misc);
    if (defer_in && defer_in->pred_idx) a.topk = *defer_in;

    if (need_router) {
        RouteArgs r{};
        r.router = L->w.router; r.router_bias = L->w.router_bias; r.E = D.n_experts; r.k = D.top_k;
        r.route_idx = io->route_idx; r.logits_r = L->s.logits_r;
        r.self_idx = L->s.self_idx; r.self_w = L->s.self_w; r.counters = L->s.counters;
        const KTime tr{L->profiling ? L->ev_t[0] : nullptr, L->profiling ? L->ev_t[1] : nullptr};
        HIPCHK(launch_dec_r(a, r, st, &tr));
        if (L->profiling) L->ev_t_used[0] = true;
    }
    if (!L->resident && (io->route_idx == nullptr || io->reactive)) {
        const int n = n_tok * D.top_k;
        const int32_t* src = L->s.self_idx;
        if (io->route_idx) {
            hipLaunchKernelGGL(k_merge_route, dim3((n + 255) / 256), dim3(256), 0, st, io->route_idx,
                               need_router ? L->s.self_idx : io->route_idx, L->s.used_idx, n, D.top_k);
            HIPCHK(hipGetLastError());
            src = L->s.used_idx;
        }
        int rc = reactive_stage(L, src, n_tok, st);
        if (rc != MOE_OK) return rc;
    }
    const KTime ta{L->profiling ? L->ev_t[2] : nullptr, L->profiling ? L->ev_t[3] : nullptr};
    HIPCHK(launch_dec_a(a, st, &ta));
    if (L->profiling) L->ev_t_used[1] = true;

    DecBArgs b{};
    b.ev = a.ev; b.d = D.d_model; b.f = D.d_ff; b.fs = D.d_ff_shared; b.k = D.top_k; b.n_tok = n_tok;
    b.E = D.n_experts;
    b.route_idx = a.route_idx; b.route_w = a.route_w; b.self_idx = a.self_idx; b.self_w = a.self_w;
    b.sgate = (D.d_ff_shared && L->w.shared_gate) ? L->s.sgate : nullptr;
    b.h = L->s.h; b.hs = L->s.hs;
    b.x = (const float*)io->x_in; b.fused = fused;
    b.au = L->s.au; b.lora_b = D.lora_rank ? L->w.lora_b : nullptr; b.r = D.lora_rank;
    b.lora_scale = D.lora_rank ? D.lora_alpha / (float)D.lora_rank : 0.f;
    b.y = io->y_out;
    b.logits_h = L->s.logits_h; b.En = D.next_n_experts; b.kn = D.next_top_k; b.head_bias = L->w.head_bias;
    b.hist_cur_m = L->w.hist_cur; b.hist_prev_m = L->w.hist_prev; b.hist_cur = io->hist_cur; b.hist_prev = io->hist_prev;
    b.pred_idx = io->pred_idx; b.pred_w = io->pred_w;
    if (defer_out && io->pred_idx && D.next_n_experts <= 64 * kDeferMaxPer) {
        TopkJob& j = *defer_out;
        j.logits = L->s.logits_h; j.En = D.next_n_experts; j.kn = D.next_top_k; j.bias = L->w.head_bias;
        j.mc = L->w.hist_cur; j.hc = io->hist_cur; j.mp = L->w.hist_prev; j.hp = io->hist_prev;
        j.pred_idx = io->pred_idx; j.pred_w = io->pred_w;
        b.pred_idx = nullptr; b.pred_w = nullptr;
    }
    b.err = L->s.err;
    const KTime tb{L->profiling ? L->ev_t[4] : nullptr, L->profiling ? L->ev_t[5] : nullptr};
    HIPCHK(launch_dec_b(b, st, &tb));
    if (L->profiling) L->ev_t_used[2] = true;
    HIPCHK(hipEventRecord(L->ev_done, st));
    L->done_recorded = true;
    return MOE_OK;
}

// route_shift = 1: io->route_idx / route_w hold the previous layer's
// predictions by token; token t takes row t - 1 and token 0 self-routes
PrologueArgs prologue_args(const moe_layer* L, const void* x, int n_tok) {
    const moe_layer_desc& D = L->desc;
    const bool fused = D.flags & MOE_FUSE_NORM_RESIDUAL;
    PrologueArgs pa{};
    pa.x = x;
    pa.x_is_bf16 = (!fused && D.act_dtype == MOE_ACT_BF16) ? 1 : 0;
    pa.fused = fused;
    pa.gamma = L->w.norm_gamma;
    pa.eps = D.rms_eps;
    pa.act_bf16 = D.act_dtype == MOE_ACT_BF16;
    pa.d = D.d_model;
    pa.n_tok = n_tok;
    pa.u_pk = L->s.u_pk; pa.u_pk_lo = L->s.u_pk_lo; pa.usum = L->s.usum; pa.usum_lo = L->s.usum_lo;
    pa.u_frag = L->s.u_frag;
    return pa;
}

int run_prefill(moe_layer* L, const moe_io* io, int n_tok, hipStream_t st, bool prefill, int route_shift,
                const PrologueArgs* nxt, bool skip_pro, bool* took_nxt) {
    const moe_layer_desc& D = L->desc;
    const bool fused = D.flags & MOE_FUSE_NORM_RESIDUAL;
    if (took_nxt) *took_nxt = false;
    if (L->staged_pending) HIPCHK(hipStreamWaitEvent(st, L->ev_staged, 0));

    if (!skip_pro) HIPCHK(launch_prologue(prologue_args(L, io->x_in, n_tok), st));

    RouteMMArgs ra{};
    ra.u_pk = L->s.u_pk; ra.u_pk_lo = L->s.u_pk_lo; ra.d = D.d_model; ra.n_tok = n_tok;
    ra.router = L->w.router; ra.router_bias = L->w.router_bias; ra.E = D.n_experts; ra.k = D.top_k;
    ra.route_idx = io->route_idx; ra.route_shift = route_shift;
    ra.head = io->pred_idx ? L->w.head : nullptr; ra.head_bias = L->w.head_bias;
    ra.En = D.next_n_experts; ra.kn = D.next_top_k;
    ra.hist_cur_m = L->w.hist_cur; ra.hist_prev_m = L->w.hist_prev; ra.hist_cur = io->hist_cur; ra.hist_prev = io->hist_prev;
    ra.lora_a = D.lora_rank ? L->w.lora_a : nullptr; ra.r = D.lora_rank;
    ra.sgate_w = D.d_ff_shared ? L->w.shared_gate : nullptr;
    ra.logits_r = L->s.logits_r; ra.logits_h = L->s.logits_h;
    ra.self_idx = L->s.self_idx; ra.self_w = L->s.self_w;
    ra.pred_idx = io->pred_idx; ra.pred_w = io->pred_w;
    ra.au = L->s.au; ra.sgate = L->s.sgate;
    ra.u_frag = L->s.u_frag;
    ra.wf_router = L->s.wf_router; ra.wf_head = L->s.wf_head; ra.wf_lora = L->s.wf_lora; ra.wf_sgate = L->s.wf_sgate;
    const bool mm = prefill_mm_ok(D.d_model, D.d_ff, D.d_ff_shared);
    const int max_active = std::min(D.n_experts, n_tok * D.top_k);
    const bool big = mm && prefill_big_tiles(D.d_model, D.d_ff, D.d_ff_shared, D.act_dtype != MOE_ACT_BF16, n_tok,
                                             D.top_k, max_active);
    const bool reactive = !L->resident && (io->route_idx == nullptr || io->reactive || prefill);
    // the router's top-k runs here when every row self-routes (or the expert
    // count is large); otherwise the sort takes the few self-routed rows. The
    // head's top-k runs beside the combine on the matrix-core path
    const bool sort_topk = io->route_idx != nullptr && L->w.router != nullptr && D.n_experts <= kSortTopkMaxE;
    // rows before the shift self-route: their top-k rides on the routing GEMM
    ra.pre_rows = sort_topk ? std::min(route_shift, n_tok) : 0;
    ra.counter = L->s.counters + 3;
    int pre_done = 0;
    HIPCHK(launch_route_mm(ra, st, !sort_topk, !mm, &pre_done));

    SortArgs sa{};
    sa.route_idx = io->route_idx; sa.route_w = io->route_w; sa.route_shift = route_shift; sa.pre_rows = pre_done;
    sa.self_idx = L->w.router ? L->s.self_idx : nullptr; sa.self_w = L->s.self_w;
    sa.n_tok = n_tok; sa.k = D.top_k; sa.E = D.n_experts;
    sa.used_idx = L->s.used_idx; sa.used_w = L->s.used_w;
    sa.user_used_idx = io->used_idx; sa.user_used_w = io->used_w;
    sa.meta = L->s.sort_meta; sa.active = L->s.active; sa.act_off = L->s.act_off; sa.perm = L->s.perm;
    sa.err = L->s.err;
    sa.self_topk = sort_topk;
    sa.logits_r = L->s.logits_r; sa.router_bias = L->w.router_bias;
    sa.ev = view_of(L); sa.fs = D.d_ff_shared;
    sa.tiles16 = mm ? L->s.tiles : nullptr;
    sa.tiles64 = big ? L->s.tiles64 : nullptr;
    sa.resolve_blobs = !reactive;
    HIPCHK(launch_sort(sa, st));

    if (reactive) {
        // reactive: the routing exists only now; read it back and stage it
        const size_t nk = (size_t)n_tok * D.top_k;
        HIPCHK(hipMemcpyAsync(L->h_readback, L->s.used_idx, nk * sizeof(int32_t), hipMemcpyDeviceToHost, st));
        HIPCHK(hipStreamSynchronize(st));
        std::vector<int32_t> want;
        for (size_t i = 0; i < nk; ++i)
            if (L->h_readback[i] >= 0) want.push_back(L->h_readback[i]);
        std::sort(want.begin(), want.end());
        want.erase(std::unique(want.begin(), want.end()), want.end());
        int rc = stage_set(L, want, st);
        if (rc != MOE_OK) return rc;
    }

    GemvArgs ga{};
    ga.ev = view_of(L);
    ga.d = D.d_model; ga.f = D.d_ff; ga.fs = D.d_ff_shared; ga.k = D.top_k; ga.n_tok = n_tok;
    ga.meta = L->s.sort_meta; ga.active = L->s.active; ga.act_off = L->s.act_off; ga.perm = L->s.perm;
    ga.used_w = L->s.used_w; ga.sgate = (D.d_ff_shared && L->w.shared_gate) ? L->s.sgate : nullptr;
    ga.u_pk = L->s.u_pk; ga.u_pk_lo = L->s.u_pk_lo; ga.usum = L->s.usum; ga.usum_lo = L->s.usum_lo;
    ga.h = L->s.h; ga.hs = L->s.hs;
    ga.x = (const float*)io->x_in; ga.fused = fused;
    ga.au = L->s.au; ga.lora_b = D.lora_rank ? L->w.lora_b : nullptr; ga.r = D.lora_rank;
    ga.lora_scale = D.lora_rank ? D.lora_alpha / (float)D.lora_rank : 0.f;
    ga.y = io->y_out;
    ga.err = L->s.err;
    ga.max_active = max_active;
    if (mm) {
        // grouped GEMM on the matrix cores (prefill and large decode batches)
        PrefillArgs pf{};
        pf.g = ga;
        pf.tiles = L->s.tiles;
        pf.max_tiles = prefill_max_tiles(n_tok, D.top_k, D.n_experts);
        pf.tiles64 = L->s.tiles64;
        pf.max_tiles64 = prefill_max_tiles(n_tok, D.top_k, D.n_experts, 64);
        pf.meta_w = L->s.sort_meta;
        pf.n_cu = L->n_cu;
        pf.ob = L->s.ob; pf.obs = L->s.obs;
        pf.used_idx = L->s.used_idx; pf.used_w = L->s.used_w;
        if (io->pred_idx && L->w.head)
            pf.head = TopkJob{L->s.logits_h, D.next_n_experts, D.next_top_k, L->w.head_bias, L->w.hist_cur, io->hist_cur,
                              L->w.hist_prev, io->hist_prev, io->pred_idx, io->pred_w};
        if (nxt) {
            pf.nxt = *nxt;
            if (!combine_norm_ok(pf)) pf.nxt = PrologueArgs{};
            else if (took_nxt) *took_nxt = true;
        }
        if (reactive) HIPCHK(launch_tile_blobs(pf, big, st));
        HIPCHK(launch_prefill(pf, st));
    } else {
        HIPCHK(launch_gateup(ga, st));
        HIPCHK(launch_down(ga, st));
    }
    HIPCHK(hipEventRecord(L->ev_done, st));
    L->done_recorded = true;
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_expert_blob_bytes(int d_model, int d_ff, int group_size) {
    if (group_size != kGroup || d_model <= 0 || d_ff <= 0 || d_model % kGroup || d_ff % kGroup) return 0;
    return 27ull * d_model * d_ff / 16;
}

size_t moe_layer_workspace_bytes(const moe_layer_desc* desc) {
    if (validate_desc(desc) != MOE_OK) return 0;
    return carve(desc, nullptr, nullptr);
}

int moe_layer_create(const moe_layer_desc* desc, const moe_layer_weights* w, void* d_workspace, size_t ws_bytes,
                     moe_layer** out) {
    if (!out) return MOE_E_INVALID;
    *out = nullptr;
    int rc = validate_desc(desc);
    if (rc != MOE_OK) return rc;
    if (!w || !d_workspace || ((uintptr_t)d_workspace & 255)) return MOE_E_INVALID;
    const bool fused = desc->flags & MOE_FUSE_NORM_RESIDUAL;
    if (!w->expert_store) return MOE_E_INVALID;
    if ((desc->d_ff_shared != 0) != (w->shared_blob != nullptr)) return MOE_E_INVALID;
    if (fused && !w->norm_gamma) return MOE_E_INVALID;
    if (desc->lora_rank && (!w->lora_a || !w->lora_b)) return MOE_E_INVALID;
    if (desc->next_n_experts > 0 && !w->head) return MOE_E_INVALID;
    if ((w->hist_cur || w->hist_prev) && desc->next_n_experts <= 0) return MOE_E_INVALID;
    const size_t need = carve(desc, nullptr, nullptr);
    if (ws_bytes < need) return MOE_E_CAPACITY;

    moe_layer* L = new (std::nothrow) moe_layer();
    if (!L) return MOE_E_INVALID;
    L->desc = *desc;
    L->w = *w;
    carve(desc, (uint8_t*)d_workspace, &L->s);
    L->L = BlobLayout::make(desc->d_model, desc->d_ff);
    L->Ls = BlobLayout::make(desc->d_model, desc->d_ff_shared ? desc->d_ff_shared : desc->d_ff);
    L->blob = L->L.total;
    L->sblob = desc->d_ff_shared ? L->Ls.total : 0;
    L->resident = desc->flags & MOE_RESIDENT_STORE;
    {
        int dev = 0, ncu = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
            ncu = 256;
        L->n_cu = ncu;
    }
    L->slots = L->resident ? 0 : desc->slab_slots;
    L->h_slot_expert = new int32_t[std::max(1, L->slots)];
    L->h_last_staged = new int32_t[std::max(1, L->slots)];
    std::fill(L->h_slot_expert, L->h_slot_expert + std::max(1, L->slots), -1);
    std::fill(L->h_last_staged, L->h_last_staged + std::max(1, L->slots), -1);
    auto fail = [&](hipError_t e) { g_last_hip = (int)e; moe_layer_destroy(L); return MOE_E_HIP; };
    hipError_t e;
    if ((e = hipGetDevice(&L->dev)) != hipSuccess) return fail(e);
    if ((e = hipEventCreateWithFlags(&L->ev_staged, hipEventDisableTiming)) != hipSuccess) return fail(e);
    if ((e = hipEventCreateWithFlags(&L->ev_done, hipEventDisableTiming)) != hipSuccess) return fail(e);
    if ((e = hipHostMalloc((void**)&L->h_readback, sizeof(int32_t) * desc->max_tokens * desc->top_k, 0)) != hipSuccess)
        return fail(e);
    if ((e = hipMemset(L->s.err, 0, 64 * sizeof(int32_t))) != hipSuccess) return fail(e);
    if ((e = hipMemset(L->s.counters, 0, 16 * sizeof(uint32_t))) != hipSuccess) return fail(e);
    if ((e = hipMemset(L->s.slot_of, 0xFF, sizeof(int32_t) * desc->n_experts)) != hipSuccess) return fail(e);
    if ((e = hipMemset(L->s.slot_tag, 0xFF, sizeof(int32_t) * (L->slots + 1))) != hipSuccess) return fail(e);
    {
        // tile-ordered copies of the routing-side rows for the prefill routing
        // GEMM (contiguous 1 KB loads); a set without its rows is not used
        const int D = desc->d_model;
        auto pack = [&](const uint16_t* w, int n, uint32_t*& out) -> hipError_t {
            if (!out) return hipSuccess;
            if (!w) { out = nullptr; return hipSuccess; }
            return launch_pack_rows(w, n, D, out, nullptr);
        };
        if ((e = pack(w->router, desc->n_experts, L->s.wf_router)) != hipSuccess) return fail(e);
        if ((e = pack(w->head, desc->next_n_experts, L->s.wf_head)) != hipSuccess) return fail(e);
        if ((e = pack(w->lora_a, desc->lora_rank, L->s.wf_lora)) != hipSuccess) return fail(e);
        if ((e = pack(w->shared_gate, 1, L->s.wf_sgate)) != hipSuccess) return fail(e);
    }
    if ((e = hipDeviceSynchronize()) != hipSuccess) return fail(e);
    *out = L;
    return MOE_OK;
}

int moe_stage_experts(moe_layer* L, const int32_t* ids, int n_ids, void* copy_stream) {
    if (!L || n_ids < 0 || (n_ids > 0 && !ids)) return MOE_E_INVALID;
    std::vector<int32_t> want;
    for (int i = 0; i < n_ids; ++i) {
        if (ids[i] < 0 || ids[i] >= L->desc.n_experts) return MOE_E_INVALID;
        want.push_back(ids[i]);
    }
    std::sort(want.begin(), want.end());
    want.erase(std::unique(want.begin(), want.end()), want.end());
    if (L->resident) return MOE_OK;
    if ((int)want.size() > L->slots) return MOE_E_CAPACITY;
    hipStream_t cs = (hipStream_t)copy_stream;
    if (L->done_recorded) HIPCHK(hipStreamWaitEvent(cs, L->ev_done, 0));
    int rc = stage_set(L, want, cs);
    if (rc != MOE_OK) return rc;
    HIPCHK(hipEventRecord(L->ev_staged, cs));
    L->staged_pending = true;
    return MOE_OK;
}

int moe_layer_slots(const moe_layer* L, int32_t* h_slot_expert, int n_slots, uint64_t* staged_bytes) {
    if (!L) return MOE_E_INVALID;
    if (h_slot_expert) {
        for (int i = 0; i < n_slots; ++i) h_slot_expert[i] = i < L->slots ? L->h_slot_expert[i] : -1;
    }
    if (staged_bytes) *staged_bytes = L->staged_bytes;
    return MOE_OK;
}

int moe_decode_step(moe_layer* L, const moe_io* io, int n_tok, void* stream) {
    int rc = check_io(L, io, n_tok);
    if (rc != MOE_OK) return rc;
    if (n_tok * L->desc.top_k > 4096 || n_tok > 256) return MOE_E_UNSUPPORTED;
    return run_decode(L, io, n_tok, (hipStream_t)stream);
}

int moe_prefill(moe_layer* L, const moe_io* io, int n_tok, void* stream) {
    int rc = check_io(L, io, n_tok);
    if (rc != MOE_OK) return rc;
    return run_prefill(L, io, n_tok, (hipStream_t)stream, true);
}

int moe_layer_sync_status(moe_layer* L) {
    if (!L) return MOE_E_INVALID;
    HIPCHK(hipDeviceSynchronize());
    int32_t err = 0;
    HIPCHK(hipMemcpy(&err, L->s.err, sizeof(err), hipMemcpyDeviceToHost));
    HIPCHK(hipMemset(L->s.err, 0, sizeof(err)));
    HIPCHK(hipDeviceSynchronize());
    if (err & ERR_TIMEOUT) return MOE_E_TIMEOUT;
    if (err & ERR_BAD_INDEX) return MOE_E_BAD_INDEX;
    if (err & ERR_NOT_STAGED) return MOE_E_NOT_STAGED;
    return MOE_OK;
}

void moe_layer_destroy(moe_layer* L) {
    if (!L) return;
    for (int i = 0; i < 6; ++i)
        if (L->ev_t[i]) (void)hipEventDestroy(L->ev_t[i]);
    if (L->ev_staged) (void)hipEventDestroy(L->ev_staged);
    if (L->ev_done) (void)hipEventDestroy(L->ev_done);
    if (L->h_readback) (void)hipHostFree(L->h_readback);
    delete[] L->h_slot_expert;
    delete[] L->h_last_staged;
    delete L;
}

int moe_layer_set_profiling(moe_layer* L, int enable) {
    if (!L) return MOE_E_INVALID;
    if (enable && !L->ev_t[0]) {
        for (int i = 0; i < 6; ++i) HIPCHK(hipEventCreate(&L->ev_t[i]));
    }
    L->profiling = enable != 0;
    for (int i = 0; i < 3; ++i) L->ev_t_used[i] = false;
    return MOE_OK;
}

int moe_layer_kernel_ms(moe_layer* L, float* ms_router, float* ms_a, float* ms_b) {
    if (!L) return MOE_E_INVALID;
    float* outs[3] = {ms_router, ms_a, ms_b};
    for (int i = 0; i < 3; ++i) {
        if (!outs[i]) continue;
        *outs[i] = -1.f;
        if (L->ev_t_used[i] && L->ev_t[2 * i]) {
            HIPCHK(hipEventSynchronize(L->ev_t[2 * i + 1]));
            HIPCHK(hipEventElapsedTime(outs[i], L->ev_t[2 * i], L->ev_t[2 * i + 1]));
        }
    }
    return MOE_OK;
}

int moe_stack_create(moe_layer* const* layers, int n, moe_stack** out) {
    if (!out || !layers || n < 1) return MOE_E_INVALID;
    *out = nullptr;
    for (int l = 0; l < n; ++l) {
        const moe_layer* L = layers[l];
        if (!L) return MOE_E_INVALID;
        if (!(L->desc.flags & MOE_FUSE_NORM_RESIDUAL)) return MOE_E_INVALID;
        if (L->desc.d_model != layers[0]->desc.d_model || L->desc.top_k != layers[0]->desc.top_k) return MOE_E_INVALID;
        if (l + 1 < n && (!L->w.head || L->desc.next_n_experts != layers[l + 1]->desc.n_experts ||
                          L->desc.next_top_k != layers[l + 1]->desc.top_k))
            return MOE_E_INVALID;
        if (!L->w.router) return MOE_E_INVALID;
    }
    moe_stack* S = new (std::nothrow) moe_stack();
    if (!S) return MOE_E_INVALID;
    S->layers = new moe_layer*[n];
    for (int l = 0; l < n; ++l) S->layers[l] = layers[l];
    S->n = n;
    // prefill scratch for the predictions passed between layers, sized by the
    // smallest max_tokens
    int T = layers[0]->desc.max_tokens;
    for (int l = 1; l < n; ++l) T = std::min(T, layers[l]->desc.max_tokens);
    const size_t per = (size_t)T * layers[0]->desc.top_k;
    hipError_t e = hipMalloc(&S->d_pred_idx, per * sizeof(int32_t));
    if (e == hipSuccess) e = hipMalloc(&S->d_pred_w, per * sizeof(float));
    if (e != hipSuccess) { g_last_hip = (int)e; moe_stack_destroy(S); return MOE_E_HIP; }
    S->pred_cap = per;
    *out = S;
    return MOE_OK;
}

int moe_stack_decode(moe_stack* S, const float* x_in, float* x_out, int n_tok, const int32_t* route_idx,
                     const float* route_w, int32_t* pred_idx, float* pred_w, int32_t* used_idx, float* used_w,
                     const int32_t* hist_prev, int first_step, void* stream) {
    if (!S || !x_in || !x_out || !pred_idx || !pred_w) return MOE_E_INVALID;
    if (!first_step && (!route_idx || !route_w)) return MOE_E_INVALID;
    const int k = S->layers[0]->desc.top_k;
    const size_t per = (size_t)n_tok * k;
    if (n_tok * k > 4096 || n_tok > 256) return MOE_E_UNSUPPORTED;
    TopkJob pend{};
    bool pro_done = false;                   // this layer's prologue was taken by the previous combine
    for (int l = 0; l < S->n; ++l) {
        moe_layer* L = S->layers[l];
        moe_io io{};
        io.x_in = l == 0 ? x_in : x_out;
        io.y_out = x_out;
        const bool self = first_step || l == 0;
        io.route_idx = self ? nullptr : route_idx + l * per;
        io.route_w = self ? nullptr : route_w + l * per;
        io.used_idx = used_idx ? used_idx + l * per : nullptr;
        io.used_w = used_w ? used_w + l * per : nullptr;
        if (l + 1 < S->n) {
            io.pred_idx = pred_idx + (l + 1) * per;
            io.pred_w = pred_w + (l + 1) * per;
            io.hist_cur = first_step ? nullptr : route_idx + (l + 1) * per;
            io.hist_prev = hist_prev ? hist_prev + (l + 1) * per : nullptr;
        }
        int rc = check_io(L, &io, n_tok);
        if (rc != MOE_OK) return rc;
        TopkJob out{};
        PrologueArgs nxt{};
        if (l + 1 < S->n) nxt = prologue_args(S->layers[l + 1], x_out, n_tok);
        bool took = false;
        rc = run_decode(L, &io, n_tok, (hipStream_t)stream, pend.pred_idx ? &pend : nullptr,
                        l + 1 < S->n ? &out : nullptr, l + 1 < S->n ? &nxt : nullptr, pro_done, &took);
        if (rc != MOE_OK) return rc;
        pend = out;
        pro_done = took;
    }
    if (pend.pred_idx) HIPCHK(launch_topk_job(pend, n_tok, (hipStream_t)stream));
    return MOE_OK;
}

int moe_stack_prefill(moe_stack* S, float* x, int n_tok, int32_t* used_idx, float* used_w, int32_t* pred_idx,
                      float* pred_w, void* stream) {
    if (!S || !x || n_tok < 1) return MOE_E_INVALID;
    const int k = S->layers[0]->desc.top_k;
    const size_t per = (size_t)n_tok * k;
    hipStream_t st = (hipStream_t)stream;
    if (per > S->pred_cap) return MOE_E_INVALID;
    bool pro_done = false;                   // this layer's prologue was taken by the previous combine
    for (int l = 0; l < S->n; ++l) {
        moe_layer* L = S->layers[l];
        moe_io io{};
        io.x_in = x;
        io.y_out = x;
        if (l > 0) {
            // the previous layer's predictions by token, shifted by one token
            // inside the call (token 0 self-routes); they are read before this
            // call's own predictions overwrite the shared buffer
            io.route_idx = pred_idx ? pred_idx + l * per : S->d_pred_idx;
            io.route_w = pred_w ? pred_w + l * per : S->d_pred_w;
        }
        io.used_idx = used_idx ? used_idx + l * per : nullptr;
        io.used_w = used_w ? used_w + l * per : nullptr;
        if (l + 1 < S->n) {
            io.pred_idx = pred_idx ? pred_idx + (l + 1) * per : S->d_pred_idx;
            io.pred_w = pred_w ? pred_w + (l + 1) * per : S->d_pred_w;
        }
        int rc = check_io(L, &io, n_tok);
        if (rc != MOE_OK) return rc;
        PrologueArgs nxt{};
        if (l + 1 < S->n) nxt = prologue_args(S->layers[l + 1], x, n_tok);
        bool took = false;
        rc = run_prefill(L, &io, n_tok, st, true, l > 0 ? 1 : 0, l + 1 < S->n ? &nxt : nullptr, pro_done, &took);
        if (rc != MOE_OK) return rc;
        pro_done = took;
    }
    return MOE_OK;
}

void moe_stack_destroy(moe_stack* S) {
    if (!S) return;
    if (S->d_pred_idx) (void)hipFree(S->d_pred_idx);
    if (S->d_pred_w) (void)hipFree(S->d_pred_w);
    delete[] S->layers;
    delete S;
}

const char* moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_E_INVALID: return "invalid argument";
        case MOE_E_UNSUPPORTED: return "unsupported shape or option";
        case MOE_E_CAPACITY: return "capacity exceeded (workspace or slab slots)";
        case MOE_E_HIP: return "HIP runtime error";
        case MOE_E_NOT_STAGED: return "a routed expert was not staged in the slab";
        case MOE_E_BAD_INDEX: return "routing index out of range";
        case MOE_E_TIMEOUT: return "device-side wait timed out";
        default: return "unknown status";
    }
}

int moe_last_hip_error(void) { return g_last_hip; }

int moe_plan_slots(int32_t* resident, int n_slots, const int32_t* wanted, int n_wanted, int n_experts,
                   int32_t* copies_slot, int32_t* copies_expert, int* n_copies) {
    if (!resident || n_slots < 0 || n_wanted < 0 || (n_wanted && !wanted) || !n_copies) return MOE_E_INVALID;
    std::vector<int32_t> want(wanted, wanted + n_wanted);
    for (int32_t e : want)
        if (e < 0 || e >= n_experts) return MOE_E_INVALID;
    std::sort(want.begin(), want.end());
    want.erase(std::unique(want.begin(), want.end()), want.end());
    if ((int)want.size() > n_slots) return MOE_E_CAPACITY;
    std::vector<char> wanted_flag(n_experts, 0), present(n_experts, 0);
    for (int32_t e : want) wanted_flag[e] = 1;
    for (int s = 0; s < n_slots; ++s)
        if (resident[s] >= 0 && resident[s] < n_experts) present[resident[s]] = 1;
    std::vector<int> free_slots;
    for (int s = 0; s < n_slots; ++s)
        if (!(resident[s] >= 0 && resident[s] < n_experts && wanted_flag[resident[s]])) free_slots.push_back(s);
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

}  // extern "C"

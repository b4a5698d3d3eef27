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
    if ((size_t)d->max_tokens * d->top_k > (1u << 20)) return MOE_E_UNSUPPORTED;
    if (d->max_tokens > 2048) return MOE_E_UNSUPPORTED;
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
    S.u = c.take<float>(T * D);
    S.u_pk = c.take<uint32_t>(T * D / 2);
    S.u_pk_lo = f32 ? c.take<uint32_t>(T * D / 2) : nullptr;
    S.usum = c.take<float>(T * D / 32);
    S.usum_lo = f32 ? c.take<float>(T * D / 32) : nullptr;
    S.logits_r = c.take<double>(T * E);
    S.logits_h = c.take<double>(T * En);
    S.self_idx = c.take<int32_t>(T * K);
    S.self_w = c.take<float>(T * K);
    S.used_idx = c.take<int32_t>(T * K);
    S.used_w = c.take<float>(T * K);
    S.au = c.take<float>(T * std::max(1, d->lora_rank));
    S.sgate = c.take<float>(T);
    S.sort_meta = c.take<int32_t>(4);
    S.active = c.take<int32_t>(nas + 1);
    S.act_off = c.take<int32_t>(nas + 1);
    S.perm = c.take<int32_t>(T * K);
    S.h = c.take<float>(T * K * d->d_ff);
    S.hs = c.take<float>(T * std::max(1, d->d_ff_shared));
    S.hb = c.take<uint16_t>(T * K * d->d_ff);
    S.hb_lo = c.take<uint16_t>(T * K * d->d_ff);
    S.hsb = c.take<uint16_t>(T * std::max(1, d->d_ff_shared));
    S.hsb_lo = c.take<uint16_t>(T * std::max(1, d->d_ff_shared));
    S.rowmap = c.take<int32_t>(T * K);
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

int run_block(moe_layer* L, const moe_io* io, int n_tok, hipStream_t st, bool prefill) {
    const moe_layer_desc& D = L->desc;
    const bool fused = D.flags & MOE_FUSE_NORM_RESIDUAL;
    if (L->staged_pending) HIPCHK(hipStreamWaitEvent(st, L->ev_staged, 0));

    PrologueArgs pa{};
    pa.x = io->x_in;
    pa.x_is_bf16 = (!fused && D.act_dtype == MOE_ACT_BF16) ? 1 : 0;
    pa.fused = fused;
    pa.gamma = L->w.norm_gamma;
    pa.eps = D.rms_eps;
    pa.act_bf16 = D.act_dtype == MOE_ACT_BF16;
    pa.d = D.d_model;
    pa.n_tok = n_tok;
    pa.u = L->s.u; pa.u_pk = L->s.u_pk; pa.u_pk_lo = L->s.u_pk_lo; pa.usum = L->s.usum; pa.usum_lo = L->s.usum_lo;
    HIPCHK(launch_prologue(pa, st));

    RouteArgs ra{};
    ra.u = L->s.u; ra.d = D.d_model; ra.n_tok = n_tok;
    ra.router = L->w.router; ra.router_bias = L->w.router_bias; ra.E = D.n_experts; ra.k = D.top_k;
    ra.route_idx = io->route_idx;
    ra.head = io->pred_idx ? L->w.head : nullptr; ra.head_bias = L->w.head_bias;
    ra.En = D.next_n_experts; ra.kn = D.next_top_k;
    ra.hist_cur_m = L->w.hist_cur; ra.hist_prev_m = L->w.hist_prev; ra.hist_cur = io->hist_cur; ra.hist_prev = io->hist_prev;
    ra.lora_a = D.lora_rank ? L->w.lora_a : nullptr; ra.r = D.lora_rank;
    ra.sgate_w = D.d_ff_shared ? L->w.shared_gate : nullptr;
    ra.logits_r = L->s.logits_r; ra.logits_h = L->s.logits_h;
    ra.self_idx = L->s.self_idx; ra.self_w = L->s.self_w;
    ra.pred_idx = io->pred_idx; ra.pred_w = io->pred_w;
    ra.au = L->s.au; ra.sgate = L->s.sgate;
    ra.counters = L->s.counters;
    HIPCHK(launch_route(ra, st));

    SortArgs sa{};
    sa.route_idx = io->route_idx; sa.route_w = io->route_w;
    sa.self_idx = L->w.router ? L->s.self_idx : nullptr; sa.self_w = L->s.self_w;
    sa.n_tok = n_tok; sa.k = D.top_k; sa.E = D.n_experts;
    sa.used_idx = L->s.used_idx; sa.used_w = L->s.used_w;
    sa.user_used_idx = io->used_idx; sa.user_used_w = io->used_w;
    sa.meta = L->s.sort_meta; sa.active = L->s.active; sa.act_off = L->s.act_off; sa.perm = L->s.perm;
    sa.err = L->s.err;
    HIPCHK(launch_sort(sa, st));

    if (!L->resident && (io->route_idx == nullptr || io->reactive || prefill)) {
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
    ga.max_active = std::min(D.n_experts, n_tok * D.top_k);
    if (prefill) {
        PrefillArgs pf{};
        pf.g = ga;
        pf.u = L->s.u;
        pf.hb = L->s.hb; pf.hb_lo = L->s.hb_lo; pf.hsb = L->s.hsb; pf.hsb_lo = L->s.hsb_lo;
        pf.rowmap = L->s.rowmap;
        HIPCHK(launch_prefill_gateup(pf, st));
        HIPCHK(launch_prefill_down(pf, st));
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
    return run_block(L, io, n_tok, (hipStream_t)stream, false);
}

int moe_prefill(moe_layer* L, const moe_io* io, int n_tok, void* stream) {
    int rc = check_io(L, io, n_tok);
    if (rc != MOE_OK) return rc;
    return run_block(L, io, n_tok, (hipStream_t)stream, true);
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
    if (L->ev_staged) (void)hipEventDestroy(L->ev_staged);
    if (L->ev_done) (void)hipEventDestroy(L->ev_done);
    if (L->h_readback) (void)hipHostFree(L->h_readback);
    delete[] L->h_slot_expert;
    delete[] L->h_last_staged;
    delete L;
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

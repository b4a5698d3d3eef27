// Host runtime of the MoE block library: the C ABI declared in
// include/moe_prerouter.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
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

constexpr int kStageCopyBlocks = 32;     // blocks of a device staging copy (PCIe-bound)
// polls before a device-side wait of the one-launch step gives up (each poll
// is a device-scope load plus a short sleep, about a microsecond: ~0.25 s)
constexpr unsigned kDefaultWaitPolls = 1u << 18;

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
    if (d->head_hidden < 0 || d->head_hidden > kMaxHeadHidden || d->head_hidden % 8) return MOE_E_UNSUPPORTED;
    if (d->head_hidden > 0 && d->next_n_experts <= 0) return MOE_E_INVALID;
    if (d->shared_lora_rank < 0 || d->shared_lora_rank > 64) return MOE_E_UNSUPPORTED;
    if (d->shared_lora_rank > 0 && d->d_ff_shared <= 0) return MOE_E_INVALID;
    const bool resident = d->flags & MOE_RESIDENT_STORE;
    // host staging plans up to 64 slots per call; device staging up to kMaxStageSlots
    const int max_slots = (d->flags & MOE_DEVICE_STAGING) ? kMaxStageSlots : 64;
    if (!resident && (d->slab_slots < 1 || d->slab_slots > max_slots)) return MOE_E_UNSUPPORTED;
    if (d->flags & ~(MOE_FUSE_NORM_RESIDUAL | MOE_RESIDENT_STORE | MOE_DEVICE_STAGING | MOE_DOUBLE_SLAB))
        return MOE_E_INVALID;
    if ((d->flags & (MOE_DEVICE_STAGING | MOE_DOUBLE_SLAB)) && resident) return MOE_E_INVALID;
    if ((d->flags & MOE_DOUBLE_SLAB) && !(d->flags & MOE_DEVICE_STAGING)) return MOE_E_INVALID;
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
    const size_t nbuf = (d->flags & MOE_DOUBLE_SLAB) ? 2 : 1;
    S.err = c.take<int32_t>(64);
    S.counters = c.take<uint32_t>(16);
    S.slot_of = c.take<int32_t>(nbuf * E);
    S.slot_tag = c.take<int32_t>(nbuf * (slots + 1));
    S.slab = resident ? nullptr : c.take<uint8_t>(nbuf * (slots + (d->d_ff_shared ? 1 : 0)) * blob);
    S.stage_plan = c.take<int32_t>(nbuf * stage_plan_ints((int)slots));
    S.stage_bytes = c.take<unsigned long long>(1);
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
    S.sau = d->shared_lora_rank > 0 ? c.take<float>(T * 2 * d->shared_lora_rank) : nullptr;
    S.wf_slora = (d->shared_lora_rank > 0 && !f32) ? c.take<uint32_t>(frag_rows_words(2 * d->shared_lora_rank, (int)D))
                                                   : nullptr;
    S.a1 = d->head_hidden > 0 ? c.take<double>(T * d->head_hidden) : nullptr;
    S.wf_fc1 = (d->head_hidden > 0 && !f32) ? c.take<uint32_t>(frag_rows_words(d->head_hidden, (int)D)) : nullptr;
    (void)Kn;
    return align_up(c.off, 256);
}

// With an adapter on the shared expert, the main kernels run without the
// shared expert (the adapter path adds it); this is the shared width they see.
inline bool has_shared_lora(const moe_layer* L) { return L->desc.shared_lora_rank > 0; }
inline int fs_main(const moe_layer* L) { return has_shared_lora(L) ? 0 : L->desc.d_ff_shared; }

// slab buffer b of a streamed layer: its blobs and its slot tables
inline uint8_t* buf_slab(const moe_layer* L, int b) {
    return L->s.slab + (size_t)b * (L->slots + (L->desc.d_ff_shared ? 1 : 0)) * L->blob;
}
inline int32_t* buf_slot_of(const moe_layer* L, int b) { return L->s.slot_of + (size_t)b * L->desc.n_experts; }
inline int32_t* buf_slot_tag(const moe_layer* L, int b) { return L->s.slot_tag + (size_t)b * (L->slots + 1); }

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
        const int b = L->cur_buf;
        ev.base = buf_slab(L, b);
        ev.slot_of = buf_slot_of(L, b);
        ev.slot_tag = buf_slot_tag(L, b);
        ev.shared = L->desc.d_ff_shared ? buf_slab(L, b) + (size_t)L->slots * L->blob : nullptr;
        ev.shared_tag = L->desc.d_ff_shared ? buf_slot_tag(L, b) + L->slots : nullptr;
    }
    if (has_shared_lora(L)) {
        ev.shared = nullptr;
        ev.shared_tag = nullptr;
        ev.shared_blob = 0;
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

// device-initiated staging of buffer b from routing entries on the device
int stage_device(moe_layer* L, const int32_t* d_ids, int n_ids, int b, hipStream_t st) {
    DevStageArgs a{};
    a.ids = d_ids; a.n_ids = n_ids; a.E = L->desc.n_experts; a.slots = L->slots;
    a.slot_of = buf_slot_of(L, b); a.slot_tag = buf_slot_tag(L, b);
    a.store = L->store_dev; a.shared = L->desc.d_ff_shared ? L->shared_dev : nullptr;
    a.slab = buf_slab(L, b); a.blob = L->blob; a.sblob = L->sblob;
    a.plan = L->s.stage_plan + (size_t)b * stage_plan_ints(L->slots); a.bytes = L->s.stage_bytes; a.err = L->s.err;
    HIPCHK(launch_stage_device(a, kStageCopyBlocks, st));
    return MOE_OK;
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

PrologueArgs prologue_args(const moe_layer* L, const void* x, int n_tok);

// The head's MLP branch: fc1's hidden-state part on the routing GEMM (u from
// the prologue, run here when the call has not), then one-hot columns, bias,
// erf-GELU and fc2 added into the head logits, before any head top-k reads them.
int run_head_mlp(moe_layer* L, const moe_io* io, int n_tok, hipStream_t st, bool run_prologue) {
    const moe_layer_desc& D = L->desc;
    if (run_prologue) HIPCHK(launch_prologue(prologue_args(L, io->x_in, n_tok), st));
    RouteMMArgs ra{};
    ra.u_pk = L->s.u_pk; ra.u_pk_lo = L->s.u_pk_lo; ra.d = D.d_model; ra.n_tok = n_tok;
    ra.head = L->w.head_fc1; ra.En = D.head_hidden; ra.kn = 0;
    ra.logits_h = L->s.a1;
    ra.u_frag = L->s.u_frag; ra.wf_head = L->s.wf_fc1;
    HIPCHK(launch_route_mm(ra, st, false, false, nullptr));
    HeadMlpArgs m{};
    m.a1 = L->s.a1; m.H1 = D.head_hidden;
    m.w1oh = L->w.head_fc1_onehot; m.b1 = L->w.head_fc1_bias; m.w2 = L->w.head_fc2;
    m.hc = io->hist_cur; m.hp = io->hist_prev; m.kn = D.next_top_k; m.En = D.next_n_experts;
    m.logits = L->s.logits_h; m.n_tok = n_tok;
    HIPCHK(launch_head_mlp_out(m, st));
    return MOE_OK;
}

// The shared expert with its adapter. part 1 (needs u only): A_g u, A_u u and
// the shared gate on the routing GEMM, then gate/up + SwiGLU; part 2 (after
// the main path wrote y): down with its adapter, gated, added into y.
SharedLoraArgs shared_lora_args(const moe_layer* L, const moe_io* io, int n_tok) {
    const moe_layer_desc& D = L->desc;
    SharedLoraArgs a{};
    if (L->resident) {
        a.blob = (const uint8_t*)L->w.shared_blob;
    } else {
        a.blob = L->s.slab + (size_t)L->slots * L->blob;
        a.tag = L->s.slot_tag + L->slots;
        a.tag_want = D.n_experts;
    }
    a.d = D.d_model; a.f = D.d_ff_shared; a.rs = D.shared_lora_rank;
    a.scale = D.shared_lora_alpha / (float)D.shared_lora_rank;
    a.u_pk = L->s.u_pk; a.u_pk_lo = L->s.u_pk_lo;
    a.sau = L->s.sau;
    a.b_gu = L->w.shared_lora_b; a.ad = L->w.shared_lora_ad; a.bd = L->w.shared_lora_bd;
    a.sgate = L->w.shared_gate ? L->s.sgate : nullptr;
    a.hs = L->s.hs; a.y = io->y_out; a.n_tok = n_tok; a.err = L->s.err;
    return a;
}

int run_shared_lora_part1(moe_layer* L, const moe_io* io, int n_tok, hipStream_t st) {
    const moe_layer_desc& D = L->desc;
    RouteMMArgs ra{};
    ra.u_pk = L->s.u_pk; ra.u_pk_lo = L->s.u_pk_lo; ra.d = D.d_model; ra.n_tok = n_tok;
    ra.lora_a = L->w.shared_lora_a; ra.r = 2 * D.shared_lora_rank; ra.au = L->s.sau;
    ra.sgate_w = L->w.shared_gate; ra.sgate = L->s.sgate;
    ra.u_frag = L->s.u_frag; ra.wf_lora = L->s.wf_slora; ra.wf_sgate = L->s.wf_sgate;
    HIPCHK(launch_route_mm(ra, st, false, false, nullptr));
    HIPCHK(launch_shared_lora(shared_lora_args(L, io, n_tok), st, true, false));
    return MOE_OK;
}

int run_shared_lora_part2(moe_layer* L, const moe_io* io, int n_tok, hipStream_t st) {
    HIPCHK(launch_shared_lora(shared_lora_args(L, io, n_tok), st, false, true));
    return MOE_OK;
}

// The arguments of the two fast-path launches of one layer's decode call
// (without the deferred head top-k, which the caller adds).
void fill_dec_args(const moe_layer* L, const moe_io* io, int n_tok, bool need_router, DecAArgs& a, DecBArgs& b) {
    const moe_layer_desc& D = L->desc;
    const bool fused = D.flags & MOE_FUSE_NORM_RESIDUAL;
    a = DecAArgs{};
    a.x = io->x_in;
    a.x_is_bf16 = (!fused && D.act_dtype == MOE_ACT_BF16) ? 1 : 0;
    a.fused = fused; a.gamma = L->w.norm_gamma; a.eps = D.rms_eps;
    a.act_bf16 = D.act_dtype == MOE_ACT_BF16; a.d = D.d_model; a.n_tok = n_tok;
    a.route_idx = io->route_idx; a.route_w = io->route_w;
    a.self_idx = need_router ? L->s.self_idx : nullptr; a.self_w = need_router ? L->s.self_w : nullptr;
    a.k = D.top_k; a.E = D.n_experts;
    a.ev = view_of(L); a.f = D.d_ff; a.fs = fs_main(L);
    a.head = io->pred_idx ? L->w.head : nullptr; a.En = io->pred_idx ? D.next_n_experts : 0;
    a.lora_a = D.lora_rank ? L->w.lora_a : nullptr; a.r = D.lora_rank;
    a.sgate_w = fs_main(L) ? L->w.shared_gate : nullptr;
    a.h = L->s.h; a.hs = L->s.hs; a.logits_h = L->s.logits_h; a.au = L->s.au; a.sgate = L->s.sgate;
    a.meta = L->s.sort_meta; a.active = L->s.active; a.act_off = L->s.act_off; a.perm = L->s.perm;
    a.wsort = L->s.wsort;
    a.used_idx = L->s.used_idx; a.used_w = L->s.used_w; a.user_used_idx = io->used_idx; a.user_used_w = io->used_w;
    a.err = L->s.err;
    dec_a_blocks(D.d_model, D.d_ff, fs_main(L), n_tok, D.top_k, D.n_experts, a.En, D.lora_rank,
                 a.sgate_w != nullptr, &a.nb_h, &a.nb_head, &a.nb_misc);
    b = DecBArgs{};
    b.ev = a.ev; b.d = D.d_model; b.f = D.d_ff; b.fs = fs_main(L); b.k = D.top_k; b.n_tok = n_tok;
    b.E = D.n_experts;
    b.route_idx = a.route_idx; b.route_w = a.route_w; b.self_idx = a.self_idx; b.self_w = a.self_w;
    b.sgate = (fs_main(L) && L->w.shared_gate) ? L->s.sgate : nullptr;
    b.h = L->s.h; b.hs = L->s.hs;
    b.x = (const float*)io->x_in; b.fused = fused;
    b.au = L->s.au; b.lora_b = D.lora_rank ? L->w.lora_b : nullptr; b.r = D.lora_rank;
    b.lora_scale = D.lora_rank ? D.lora_alpha / (float)D.lora_rank : 0.f;
    b.y = io->y_out;
    b.logits_h = L->s.logits_h; b.En = D.next_n_experts; b.kn = D.next_top_k; b.head_bias = L->w.head_bias;
    b.hist_cur_m = L->w.hist_cur; b.hist_prev_m = L->w.hist_prev; b.hist_cur = io->hist_cur; b.hist_prev = io->hist_prev;
    b.pred_idx = io->pred_idx; b.pred_w = io->pred_w;
    b.err = L->s.err;
}

// defer_in: a previous layer's head top-k to run inside this layer's K_A.
// defer_out (stack mode): this layer's head top-k is not run here but handed
// back, for the next layer's K_A to run (its prediction is for the next step).
// pred_ready (stack staging): recorded once the prediction of the previous
// layer's head (run inside this call's first launch) is final
int run_decode(moe_layer* L, const moe_io* io, int n_tok, hipStream_t st, const TopkJob* defer_in = nullptr,
               TopkJob* defer_out = nullptr, const PrologueArgs* nxt = nullptr, bool skip_pro = false,
               bool* took_nxt = nullptr, hipEvent_t pred_ready = nullptr) {
    const moe_layer_desc& D = L->desc;
    if (defer_out) defer_out->pred_idx = nullptr;
    if (took_nxt) *took_nxt = false;
    // shapes outside the fused two-kernel path take the general grouped-GEMM path
    if (!dec_fast_path_ok(D.d_model, D.d_ff, fs_main(L), n_tok, D.top_k)) {
        if (defer_in && defer_in->pred_idx) HIPCHK(launch_topk_job(*defer_in, n_tok, st));
        if (pred_ready) HIPCHK(hipEventRecord(pred_ready, st));
        return run_prefill(L, io, n_tok, st, false, 0, nxt, skip_pro, took_nxt);
    }
    if (L->staged_pending_buf[L->cur_buf]) HIPCHK(hipStreamWaitEvent(st, L->ev_staged_buf[L->cur_buf], 0));
    const bool need_router = io->route_idx == nullptr || io->self_rows;
    if (need_router && !L->w.router) return MOE_E_INVALID;

    DecAArgs a{};
    DecBArgs b{};
    fill_dec_args(L, io, n_tok, need_router, a, b);
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
        int rc = L->dev_staging ? stage_device(L, src, n, L->cur_buf, st) : reactive_stage(L, src, n_tok, st);
        if (rc != MOE_OK) return rc;
    }
    const KTime ta{L->profiling ? L->ev_t[2] : nullptr, L->profiling ? L->ev_t[3] : nullptr};
    HIPCHK(launch_dec_a(a, st, &ta));
    if (L->profiling) L->ev_t_used[1] = true;
    if (pred_ready) HIPCHK(hipEventRecord(pred_ready, st));
    // the prologue (u for the routing GEMM) runs before K_B, which may
    // overwrite x in place
    const bool mlp = io->pred_idx && D.head_hidden > 0;
    if (mlp || has_shared_lora(L)) HIPCHK(launch_prologue(prologue_args(L, io->x_in, n_tok), st));
    if (mlp) {
        const int rc = run_head_mlp(L, io, n_tok, st, false);
        if (rc != MOE_OK) return rc;
    }
    if (has_shared_lora(L)) {
        const int rc = run_shared_lora_part1(L, io, n_tok, st);
        if (rc != MOE_OK) return rc;
    }

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
    if (has_shared_lora(L)) {
        const int rc = run_shared_lora_part2(L, io, n_tok, st);
        if (rc != MOE_OK) return rc;
    }
    if (L->ev_done) {
        HIPCHK(hipEventRecord(L->ev_done, st));
        L->done_recorded = true;
    }
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
    if (L->staged_pending_buf[L->cur_buf]) HIPCHK(hipStreamWaitEvent(st, L->ev_staged_buf[L->cur_buf], 0));

    if (!skip_pro) HIPCHK(launch_prologue(prologue_args(L, io->x_in, n_tok), st));

    RouteMMArgs ra{};
    ra.u_pk = L->s.u_pk; ra.u_pk_lo = L->s.u_pk_lo; ra.d = D.d_model; ra.n_tok = n_tok;
    ra.router = L->w.router; ra.router_bias = L->w.router_bias; ra.E = D.n_experts; ra.k = D.top_k;
    ra.route_idx = io->route_idx; ra.route_shift = route_shift;
    ra.head = io->pred_idx ? L->w.head : nullptr; ra.head_bias = L->w.head_bias;
    ra.En = D.next_n_experts; ra.kn = D.next_top_k;
    ra.hist_cur_m = L->w.hist_cur; ra.hist_prev_m = L->w.hist_prev; ra.hist_cur = io->hist_cur; ra.hist_prev = io->hist_prev;
    ra.lora_a = D.lora_rank ? L->w.lora_a : nullptr; ra.r = D.lora_rank;
    ra.sgate_w = fs_main(L) ? L->w.shared_gate : nullptr;
    ra.logits_r = L->s.logits_r; ra.logits_h = L->s.logits_h;
    ra.self_idx = L->s.self_idx; ra.self_w = L->s.self_w;
    ra.pred_idx = io->pred_idx; ra.pred_w = io->pred_w;
    ra.au = L->s.au; ra.sgate = L->s.sgate;
    ra.u_frag = L->s.u_frag;
    ra.wf_router = L->s.wf_router; ra.wf_head = L->s.wf_head; ra.wf_lora = L->s.wf_lora; ra.wf_sgate = L->s.wf_sgate;
    const bool mm = prefill_mm_ok(D.d_model, D.d_ff, fs_main(L));
    const int max_active = std::min(D.n_experts, n_tok * D.top_k);
    const bool big = mm && prefill_big_tiles(D.d_model, D.d_ff, fs_main(L), D.act_dtype != MOE_ACT_BF16, n_tok,
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
    const bool mlp = io->pred_idx && L->w.head && D.head_hidden > 0;
    // Sorted ahead (batched stack decode): no row self-routes, so the sort
    // needs no router rows, and what the routing GEMM writes (head logits,
    // LoRA A u, shared gate) is first read by the combine: it goes with the
    // gate/up launch. (Splitting off only the router rows before the sort
    // of a 512-token stacked prefill measured slower: 6.82 against 6.75 ms.)
    const bool route_later = L->presorted && mm && !big && !mlp && !has_shared_lora(L) && route_fr_ok(ra);
    if (route_later) {
        ra.router = nullptr;
        ra.pre_rows = 0;
    } else {
        HIPCHK(launch_route_mm(ra, st, !sort_topk, !mm && !mlp, &pre_done));
    }
    if (mlp) {
        int rc = run_head_mlp(L, io, n_tok, st, false);
        if (rc != MOE_OK) return rc;
        // off the matrix-core path the head's top-k has its own launch
        if (!mm) HIPCHK(launch_route_topk(ra, st, false, true));
    }
    if (has_shared_lora(L)) {
        int rc = run_shared_lora_part1(L, io, n_tok, st);
        if (rc != MOE_OK) return rc;
    }

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
    sa.ev = view_of(L); sa.fs = fs_main(L);
    sa.tiles16 = mm ? L->s.tiles : nullptr;
    sa.tiles64 = big ? L->s.tiles64 : nullptr;
    sa.resolve_blobs = !reactive;
    if (!L->presorted) HIPCHK(launch_sort(sa, st));

    if (reactive && L->dev_staging) {
        // reactive on the device: the sorted routing drives the staging
        int rc = stage_device(L, L->s.used_idx, n_tok * D.top_k, L->cur_buf, st);
        if (rc != MOE_OK) return rc;
    } else if (reactive) {
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
    ga.d = D.d_model; ga.f = D.d_ff; ga.fs = fs_main(L); ga.k = D.top_k; ga.n_tok = n_tok;
    ga.meta = L->s.sort_meta; ga.active = L->s.active; ga.act_off = L->s.act_off; ga.perm = L->s.perm;
    ga.used_w = L->s.used_w; ga.sgate = (fs_main(L) && L->w.shared_gate) ? L->s.sgate : nullptr;
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
        if (nxt && !has_shared_lora(L)) {
            // (with the shared adapter the layer's output is complete only
            // after its own down kernel, so the next norm runs on its own)
            pf.nxt = *nxt;
            if (!combine_norm_ok(pf)) pf.nxt = PrologueArgs{};
            else if (took_nxt) *took_nxt = true;
        }
        if (reactive) HIPCHK(launch_tile_blobs(pf, big, st));
        HIPCHK(launch_prefill(pf, st, route_later ? &ra : nullptr));
    } else {
        HIPCHK(launch_gateup(ga, st));
        HIPCHK(launch_down(ga, st));
    }
    if (has_shared_lora(L)) {
        int rc = run_shared_lora_part2(L, io, n_tok, st);
        if (rc != MOE_OK) return rc;
    }
    HIPCHK(hipEventRecord(L->ev_done, st));
    L->done_recorded = true;
    return MOE_OK;
}

// ---- scratch of the entry point that allocates nothing ---------------------
// A file-scope device array per GPU (it lives as long as the process). Host
// code never passes its name to a kernel: it looks the array's device
// address up once per device and uses that address.
constexpr size_t kNoallocScratchBytes = 256u << 10;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];
constexpr int kNoallocMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kNoallocMaxDevices] = {};

int noalloc_scratch(uint8_t** out) {
    int dev = 0;
    HIPCHK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kNoallocMaxDevices) return MOE_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) return MOE_E_HIP;
        g_scratch_ptr[dev] = (uint8_t*)p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// the per-call scratch of a fused-path decode call of n_tok tokens
size_t carve_decode(const moe_layer_desc* d, int n_tok, uint8_t* base, Scratch* s) {
    Carver c{base};
    Scratch tmp{};
    Scratch& S = s ? *s : tmp;
    const size_t T = (size_t)n_tok, E = d->n_experts, K = d->top_k;
    const size_t En = d->next_n_experts > 0 ? d->next_n_experts : 1;
    S.err = c.take<int32_t>(64);
    S.counters = c.take<uint32_t>(16);
    S.logits_r = c.take<double>(T * E);
    S.logits_h = c.take<double>(T * En);
    S.self_idx = c.take<int32_t>(T * K);
    S.self_w = c.take<float>(T * K);
    S.used_idx = c.take<int32_t>(T * K);
    S.used_w = c.take<float>(T * K);
    S.au = c.take<float>(T * std::max(1, d->lora_rank));
    S.sgate = c.take<float>(std::max<size_t>(T, 64));
    S.sort_meta = c.take<int32_t>(8);
    S.active = c.take<int32_t>(std::max<size_t>(std::min(E, T * K) + 1, 64));
    S.act_off = c.take<int32_t>(std::max<size_t>(std::min(E, T * K) + 1, 64));
    S.perm = c.take<int32_t>(std::max<size_t>(T * K, 64));
    S.wsort = c.take<float>(std::max<size_t>(T * K, 64));
    S.h = c.take<float>(T * K * d->d_ff);
    S.hs = c.take<float>(T * std::max(1, d->d_ff_shared));
    return align_up(c.off, 256);
}

__global__ void k_noalloc_begin(int32_t* err, uint32_t* counters) {
    const int i = threadIdx.x;
    if (i < 64) err[i] = 0;
    if (i < 16) counters[i] = 0u;
}

__global__ void k_noalloc_status(const int32_t* err, int32_t* status) {
    const int e = err[0];
    status[0] = (e & ERR_TIMEOUT) ? MOE_E_TIMEOUT : (e & ERR_BAD_INDEX) ? MOE_E_BAD_INDEX
                : (e & ERR_NOT_STAGED) ? MOE_E_NOT_STAGED : MOE_OK;
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
    if ((desc->head_hidden > 0) != (w->head_fc1 != nullptr) || (desc->head_hidden > 0) != (w->head_fc1_onehot != nullptr) ||
        (desc->head_hidden > 0) != (w->head_fc2 != nullptr) || (w->head_fc1_bias && desc->head_hidden <= 0))
        return MOE_E_INVALID;
    const bool sl = desc->shared_lora_rank > 0;
    if (sl != (w->shared_lora_a != nullptr) || sl != (w->shared_lora_b != nullptr) ||
        sl != (w->shared_lora_ad != nullptr) || sl != (w->shared_lora_bd != nullptr))
        return MOE_E_INVALID;
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
    L->nbuf = (desc->flags & MOE_DOUBLE_SLAB) ? 2 : 1;
    L->cur_buf = 0;
    L->dev_staging = desc->flags & MOE_DEVICE_STAGING;
    L->h_slot_expert = new int32_t[std::max(1, L->slots)];
    L->h_last_staged = new int32_t[std::max(1, L->slots)];
    std::fill(L->h_slot_expert, L->h_slot_expert + std::max(1, L->slots), -1);
    std::fill(L->h_last_staged, L->h_last_staged + std::max(1, L->slots), -1);
    auto fail = [&](hipError_t e) { g_last_hip = (int)e; moe_layer_destroy(L); return MOE_E_HIP; };
    hipError_t e;
    if ((e = hipGetDevice(&L->dev)) != hipSuccess) return fail(e);
    if ((e = hipEventCreateWithFlags(&L->ev_staged, hipEventDisableTiming)) != hipSuccess) return fail(e);
    if ((e = hipEventCreateWithFlags(&L->ev_done, hipEventDisableTiming)) != hipSuccess) return fail(e);
    L->ev_staged_buf[0] = L->ev_staged;
    if ((e = hipEventCreateWithFlags(&L->ev_staged_buf[1], hipEventDisableTiming)) != hipSuccess) return fail(e);
    if ((e = hipEventCreateWithFlags(&L->ev_pred, hipEventDisableTiming)) != hipSuccess) return fail(e);
    if (L->dev_staging) {
        // the pinned store (and shared blob) as the device sees them
        void* p = nullptr;
        if ((e = hipHostGetDevicePointer(&p, const_cast<void*>(w->expert_store), 0)) != hipSuccess) return fail(e);
        L->store_dev = (const uint8_t*)p;
        if (w->shared_blob) {
            if ((e = hipHostGetDevicePointer(&p, const_cast<void*>(w->shared_blob), 0)) != hipSuccess) return fail(e);
            L->shared_dev = (const uint8_t*)p;
        }
    }
    if ((e = hipHostMalloc((void**)&L->h_readback, sizeof(int32_t) * desc->max_tokens * desc->top_k, 0)) != hipSuccess)
        return fail(e);
    if ((e = hipMemset(L->s.err, 0, 64 * sizeof(int32_t))) != hipSuccess) return fail(e);
    if ((e = hipMemset(L->s.counters, 0, 16 * sizeof(uint32_t))) != hipSuccess) return fail(e);
    if ((e = hipMemset(L->s.slot_of, 0xFF, sizeof(int32_t) * desc->n_experts * L->nbuf)) != hipSuccess) return fail(e);
    if ((e = hipMemset(L->s.slot_tag, 0xFF, sizeof(int32_t) * (L->slots + 1) * L->nbuf)) != hipSuccess) return fail(e);
    if ((e = hipMemset(L->s.stage_bytes, 0, sizeof(unsigned long long))) != hipSuccess) return fail(e);
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
        if ((e = pack(w->head_fc1, desc->head_hidden, L->s.wf_fc1)) != hipSuccess) return fail(e);
        if ((e = pack(w->shared_lora_a, 2 * desc->shared_lora_rank, L->s.wf_slora)) != hipSuccess) return fail(e);
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
    if (L->dev_staging) return MOE_E_UNSUPPORTED;      // one staging mode per layer
    if ((int)want.size() > L->slots) return MOE_E_CAPACITY;
    hipStream_t cs = (hipStream_t)copy_stream;
    if (L->done_recorded) HIPCHK(hipStreamWaitEvent(cs, L->ev_done, 0));
    int rc = stage_set(L, want, cs);
    if (rc != MOE_OK) return rc;
    HIPCHK(hipEventRecord(L->ev_staged, cs));
    L->staged_pending_buf[0] = true;
    return MOE_OK;
}

int moe_stage_experts_device(moe_layer* L, const int32_t* d_ids, int n_ids, int buffer, void* stream) {
    if (!L || n_ids < 0 || (n_ids > 0 && !d_ids) || buffer < 0) return MOE_E_INVALID;
    if (!L->dev_staging || !L->store_dev) return MOE_E_UNSUPPORTED;
    if (buffer >= L->nbuf) return MOE_E_INVALID;
    hipStream_t cs = (hipStream_t)stream;
    if (L->nbuf == 1 && L->done_recorded) HIPCHK(hipStreamWaitEvent(cs, L->ev_done, 0));
    int rc = stage_device(L, d_ids, n_ids, buffer, cs);
    if (rc != MOE_OK) return rc;
    HIPCHK(hipEventRecord(L->ev_staged_buf[buffer], cs));
    L->staged_pending_buf[buffer] = true;
    return MOE_OK;
}

int moe_layer_use_buffer(moe_layer* L, int buffer) {
    if (!L || buffer < 0 || buffer >= std::max(1, L->nbuf)) return MOE_E_INVALID;
    L->cur_buf = buffer;
    return MOE_OK;
}

int moe_layer_slots(const moe_layer* L, int32_t* h_slot_expert, int n_slots, uint64_t* staged_bytes) {
    if (!L) return MOE_E_INVALID;
    if (L->dev_staging) {
        std::vector<int32_t> tags(std::max(1, L->slots), -1);
        unsigned long long dev_bytes = 0;
        HIPCHK(hipDeviceSynchronize());
        HIPCHK(hipMemcpy(tags.data(), buf_slot_tag(L, L->cur_buf), sizeof(int32_t) * L->slots, hipMemcpyDeviceToHost));
        HIPCHK(hipMemcpy(&dev_bytes, L->s.stage_bytes, sizeof(dev_bytes), hipMemcpyDeviceToHost));
        if (h_slot_expert)
            for (int i = 0; i < n_slots; ++i) h_slot_expert[i] = i < L->slots ? tags[i] : -1;
        if (staged_bytes) *staged_bytes = dev_bytes;
        return MOE_OK;
    }
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

int moe_decode_noalloc(const moe_layer_desc* desc, const moe_layer_weights* w, const moe_io* io, int n_tok,
                       int32_t* d_status, void* stream) {
    int rc = validate_desc(desc);
    if (rc != MOE_OK) return rc;
    if (!w || !w->expert_store) return MOE_E_INVALID;
    if (!(desc->flags & MOE_RESIDENT_STORE)) return MOE_E_UNSUPPORTED;
    if ((desc->d_ff_shared != 0) != (w->shared_blob != nullptr)) return MOE_E_INVALID;
    if ((desc->flags & MOE_FUSE_NORM_RESIDUAL) && !w->norm_gamma) return MOE_E_INVALID;
    if (desc->lora_rank && (!w->lora_a || !w->lora_b)) return MOE_E_INVALID;
    if (desc->next_n_experts > 0 && !w->head) return MOE_E_INVALID;
    if ((w->hist_cur || w->hist_prev) && desc->next_n_experts <= 0) return MOE_E_INVALID;
    if (n_tok < 1 || n_tok > desc->max_tokens) return MOE_E_INVALID;
    if (desc->head_hidden > 0 || desc->shared_lora_rank > 0) return MOE_E_UNSUPPORTED;
    if (!dec_fast_path_ok(desc->d_model, desc->d_ff, desc->d_ff_shared, n_tok, desc->top_k))
        return MOE_E_UNSUPPORTED;
    if (carve_decode(desc, n_tok, nullptr, nullptr) > kNoallocScratchBytes) return MOE_E_CAPACITY;
    uint8_t* base = nullptr;
    rc = noalloc_scratch(&base);
    if (rc != MOE_OK) return rc;
    moe_layer L{};
    L.desc = *desc;
    L.w = *w;
    carve_decode(desc, n_tok, base, &L.s);
    L.L = BlobLayout::make(desc->d_model, desc->d_ff);
    L.Ls = BlobLayout::make(desc->d_model, desc->d_ff_shared ? desc->d_ff_shared : desc->d_ff);
    L.blob = L.L.total;
    L.sblob = desc->d_ff_shared ? L.Ls.total : 0;
    L.resident = true;
    rc = check_io(&L, io, n_tok);
    if (rc != MOE_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(k_noalloc_begin, dim3(1), dim3(64), 0, st, L.s.err, L.s.counters);
    HIPCHK(hipGetLastError());
    rc = run_decode(&L, io, n_tok, st);
    if (rc != MOE_OK) return rc;
    if (d_status) {
        hipLaunchKernelGGL(k_noalloc_status, dim3(1), dim3(1), 0, st, (const int32_t*)L.s.err, d_status);
        HIPCHK(hipGetLastError());
    }
    return MOE_OK;
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
    if (L->ev_staged_buf[1]) (void)hipEventDestroy(L->ev_staged_buf[1]);
    if (L->ev_pred) (void)hipEventDestroy(L->ev_pred);
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

static int validate_stack(moe_layer* const* layers, int n) {
    if (!layers || n < 1) return MOE_E_INVALID;
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
    return MOE_OK;
}

// prediction entries per buffer: the smallest max_tokens times k
static size_t stack_pred_entries(moe_layer* const* layers, int n) {
    int T = layers[0]->desc.max_tokens;
    for (int l = 1; l < n; ++l) T = std::min(T, layers[l]->desc.max_tokens);
    return (size_t)T * layers[0]->desc.top_k;
}

// The one-launch step needs layers whose experts are all resident, whose
// shapes take the two-kernel fast path and agree from layer to layer (one
// work-item layout for all), and that run nothing between K_A and K_B (no
// head MLP branch, no adapter on the shared expert).
static bool stack_one_launch_ok(moe_layer* const* layers, int n) {
    const moe_layer_desc& D0 = layers[0]->desc;
    const moe_layer* L0 = layers[0];
    if (!stack_one_fast_ok(D0.d_model, D0.d_ff, fs_main(L0), 1, D0.top_k)) return false;
    for (int l = 0; l < n; ++l) {
        const moe_layer* L = layers[l];
        const moe_layer_desc& D = L->desc;
        if (!L->resident || D.head_hidden > 0 || has_shared_lora(L)) return false;
        if (D.d_model != D0.d_model || D.d_ff != D0.d_ff || fs_main(L) != fs_main(L0) || D.top_k != D0.top_k ||
            D.n_experts != D0.n_experts || D.lora_rank != D0.lora_rank ||
            (L->w.shared_gate != nullptr) != (L0->w.shared_gate != nullptr))
            return false;
        if (D.lora_rank && (D.lora_rank % 8 || D.lora_rank > 16)) return false;
        if (l + 1 < n && (D.next_n_experts > 64 * kStackHeadMaxPer || D.next_n_experts != layers[0]->desc.next_n_experts))
            return false;
    }
    return true;
}

static size_t stack_carve(moe_layer* const* layers, int n, uint8_t* base, moe_stack* S) {
    Carver c{base};
    const size_t per = stack_pred_entries(layers, n);
    for (int b = 0; b < 2; ++b) {
        int32_t* pi = c.take<int32_t>(per);
        float* pw = c.take<float>(per);
        if (S) { S->d_pred_idx[b] = pi; S->d_pred_w[b] = pw; }
    }
    if (S) S->pred_cap = per;
    StackLayerArgs* tab = c.take<StackLayerArgs>((size_t)n);
    uint32_t* sync = c.take<uint32_t>(stack_sync_words(n));
    SortArgs* stab = n > 1 ? c.take<SortArgs>((size_t)n - 1) : nullptr;
    if (S) { S->d_tab = tab; S->d_sync = sync; S->d_sort_tab = stab; }
    if (stack_one_launch_ok(layers, n)) {
        // exchange copies of the one-launch step, sized for the most tokens
        // a step of this stack can take there
        const moe_layer_desc& D = layers[0]->desc;
        int nt = 0;
        for (int t = 1; t <= 64; ++t)
            if (stack_one_fast_ok(D.d_model, D.d_ff, fs_main(layers[0]), t, D.top_k)) nt = t;
        for (int l = 0; l < n; ++l) nt = std::min(nt, layers[l]->desc.max_tokens);
        auto al = [](size_t v) { return (v + 63) / 64 * 64; };
        size_t off[5], o = 0;
        off[0] = o; o += al((size_t)nt * D.d_model);
        off[1] = o; o += al((size_t)nt * D.top_k * D.d_ff);
        off[2] = o; o += al((size_t)nt * std::max(1, fs_main(layers[0])));
        off[3] = o; o += al((size_t)nt * std::max(1, D.lora_rank));
        off[4] = o; o += al((size_t)nt);
        float* xchg = c.take<float>(o * kXchgCopies * n);
        if (S) {
            S->d_xchg = xchg;
            S->xchg_stride = o;
            for (int i = 0; i < 5; ++i) S->xchg_off[i] = off[i];
            S->xchg_tokens = nt;
        }
    }
    return align_up(c.off, 256);
}

// the per-layer table of the one-launch step: the fields fixed at creation
// (the per-call ones are written by the patch kernel before each launch)
static int stack_one_launch_init(moe_stack* S) {
    const int n = S->n;
    std::vector<StackLayerArgs> tab(n);
    int nb_head = 0;
    for (int l = 0; l < n; ++l) {
        moe_layer* L = S->layers[l];
        moe_io io{};
        io.x_in = nullptr;
        io.y_out = nullptr;
        int32_t dummy_pred = 0;
        if (l + 1 < n) { io.pred_idx = &dummy_pred; io.pred_w = (float*)&dummy_pred; }
        fill_dec_args(L, &io, 1, l == 0, tab[l].a, tab[l].b);
        DecAArgs& a = tab[l].a;
        DecBArgs& b = tab[l].b;
        b.pred_idx = nullptr; b.pred_w = nullptr;
        if (l == 0) nb_head = a.nb_head;
        // the values handed from K_A to K_B, and x from layer l-1's K_B, go
        // through kXchgCopies copies (readers spread over them)
        float* reg = S->d_xchg + (size_t)l * kXchgCopies * S->xchg_stride;
        a.h = reg + S->xchg_off[1];
        b.h = a.h;
        a.hs = reg + S->xchg_off[2];
        b.hs = a.hs;
        a.au = reg + S->xchg_off[3];
        b.au = a.au;
        a.sgate = reg + S->xchg_off[4];
        if (b.sgate) b.sgate = a.sgate;
        a.xstride = b.xstride = S->xchg_stride;
        a.xcopies = b.xcopies = kXchgCopies;
        a.x_repl = b.x_repl = l > 0;
        if (l > 0) { a.x = reg + S->xchg_off[0]; b.x = reg + S->xchg_off[0]; }
        b.xnext = l + 1 < n ? S->d_xchg + (size_t)(l + 1) * kXchgCopies * S->xchg_stride + S->xchg_off[0] : nullptr;
    }
    // the last layer has no head: it keeps the others' item count, and its
    // head items find no rows
    tab[n - 1].a.nb_head = nb_head;
    HIPCHK(hipMemcpy(S->d_tab, tab.data(), sizeof(StackLayerArgs) * n, hipMemcpyHostToDevice));
    HIPCHK(hipMemset(S->d_sync, 0, sizeof(uint32_t) * stack_sync_words(n)));
    int dev = 0, ncu = 0;
    HIPCHK(hipGetDevice(&dev));
    HIPCHK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
    const int per_cu = stack_one_launch_blocks_per_cu(S->layers[0]->desc.d_model, S->layers[0]->desc.d_ff);
    S->one_grid = std::max(1, per_cu) * std::max(1, ncu);
    return MOE_OK;
}

static int trace_layer(moe_stack* S, int l, const void* x, int n_tok, hipStream_t st);

// one decode step as a router launch (layer 0 routes itself) + the table
// patch + the step kernel
static int stack_decode_one(moe_stack* S, const float* x_in, float* x_out, int n_tok, const int32_t* route_idx,
                            const float* route_w, int32_t* pred_idx, float* pred_w, int32_t* used_idx,
                            float* used_w, const int32_t* hist_prev, hipStream_t st) {
    moe_layer* L0 = S->layers[0];
    const moe_layer_desc& D = L0->desc;
    moe_io io{};
    io.x_in = x_in;
    io.y_out = x_out;
    io.pred_idx = S->n > 1 ? pred_idx : nullptr;   // (head items counted as for every layer but the last)
    io.pred_w = S->n > 1 ? pred_w : nullptr;
    DecAArgs a{};
    DecBArgs b{};
    fill_dec_args(L0, &io, n_tok, true, a, b);
    int rc = trace_layer(S, 0, x_in, n_tok, st);
    if (rc != MOE_OK) return rc;
    RouteArgs r{};
    r.router = L0->w.router; r.router_bias = L0->w.router_bias; r.E = D.n_experts; r.k = D.top_k;
    r.route_idx = nullptr; r.logits_r = L0->s.logits_r;
    r.self_idx = L0->s.self_idx; r.self_w = L0->s.self_w; r.counters = L0->s.counters;
    const KTime tr{S->profiling ? S->ev_t[0] : nullptr, S->profiling ? S->ev_t[1] : nullptr};
    StackPatchArgs p{};
    p.tab = S->d_tab; p.sync = S->d_sync; p.n_layers = S->n; p.n_tok = n_tok; p.k = D.top_k; p.d = D.d_model; p.f = D.d_ff;
    const int hr = stack_one_hrows(D.d_model);
    const int max_active = std::min(n_tok * D.top_k, D.n_experts);
    p.nb_h = (fs_main(L0) + max_active * D.d_ff + hr - 1) / hr;
    p.x_in = x_in; p.x_out = x_out;
    p.route_idx = route_idx; p.route_w = route_w; p.pred_idx = pred_idx; p.pred_w = pred_w;
    p.used_idx = used_idx; p.used_w = used_w; p.hist_prev = hist_prev;
    p.trace = S->x_trace;
    p.xchg = S->d_xchg;
    p.xstride = S->xchg_stride;
    const uint32_t xw[kXchgParts] = {(uint32_t)D.d_model, (uint32_t)(D.top_k * D.d_ff), (uint32_t)fs_main(L0),
                                     (uint32_t)D.lora_rank, 1u};
    for (int i = 0; i < kXchgParts; ++i) { p.xoff[i] = (uint32_t)S->xchg_off[i]; p.xw[i] = xw[i]; }
    StackDecArgs sd{};
    sd.tab = S->d_tab; sd.n_layers = S->n;
    sd.nA = p.nb_h + a.nb_head + a.nb_misc;
    sd.nB = 1 + D.d_model / stack_one_brows(D.d_ff);
    sd.sync = S->d_sync;
    sd.spin_limit = S->wait_polls;
    const int total = S->n * (sd.nA + sd.nB);
    const KTime tk{S->profiling ? S->ev_t[2] : nullptr, S->profiling ? S->ev_t[3] : nullptr};
    // one block per work item of a layer when they fit on the chip at once
    // (each block then keeps its role from layer to layer), else fewer
    const int per_layer = sd.nA + sd.nB;
    const int grid = per_layer <= S->one_grid ? per_layer : std::min(S->one_grid, total);
    HIPCHK(launch_stack_one(p, a, r, sd, grid, st, &tr, &tk));
    if (S->profiling) S->ev_used[0] = S->ev_used[1] = true;
    return MOE_OK;
}

// Batched decode beyond the fused path: the given routing of layers 1..n-1
// (the previous step's predictions) is known when the step starts, so their
// token->expert sorts run as one launch there instead of one launch on each
// layer's chain. The table holds each layer's fixed sort arguments; no row
// self-routes there (self_idx null: a negative entry is a bad index).
static int stack_sort_init(moe_stack* S) {
    S->sort_ok = false;
    if (S->n < 2 || !S->d_sort_tab) return MOE_OK;
    const moe_layer_desc& D0 = S->layers[0]->desc;
    for (int l = 0; l < S->n; ++l) {
        const moe_layer* L = S->layers[l];
        const moe_layer_desc& D = L->desc;
        if (!L->resident || D.d_model != D0.d_model || D.d_ff != D0.d_ff || fs_main(L) != fs_main(S->layers[0]) ||
            D.n_experts != D0.n_experts || D.top_k != D0.top_k || D.act_dtype != D0.act_dtype)
            return MOE_OK;
    }
    std::vector<SortArgs> tab((size_t)S->n - 1);
    for (int l = 1; l < S->n; ++l) {
        moe_layer* L = S->layers[l];
        const moe_layer_desc& D = L->desc;
        SortArgs& sa = tab[(size_t)l - 1];
        sa = SortArgs{};
        sa.k = D.top_k; sa.E = D.n_experts;
        sa.used_idx = L->s.used_idx; sa.used_w = L->s.used_w;
        sa.meta = L->s.sort_meta; sa.active = L->s.active; sa.act_off = L->s.act_off; sa.perm = L->s.perm;
        sa.err = L->s.err;
        sa.ev = view_of(L); sa.fs = fs_main(L);
        sa.tiles16 = prefill_mm_ok(D.d_model, D.d_ff, fs_main(L)) ? L->s.tiles : nullptr;
        sa.tiles64 = L->s.tiles64;
        sa.resolve_blobs = true;
    }
    HIPCHK(hipMemcpy(S->d_sort_tab, tab.data(), tab.size() * sizeof(SortArgs), hipMemcpyHostToDevice));
    S->sort_ok = true;
    return MOE_OK;
}

// whether this step's sorts of layers 1..n-1 run as one launch (every such
// layer takes the general path at n_tok tokens); big: its 64-row tile lists
static bool stack_sort_hoist(const moe_stack* S, int n_tok, int first_step, bool* big) {
    if (!S->sort_ok || first_step || S->stage_mode != MOE_STAGE_OFF) return false;
    const moe_layer* L = S->layers[1];
    const moe_layer_desc& D = L->desc;
    if (dec_fast_path_ok(D.d_model, D.d_ff, fs_main(L), n_tok, D.top_k)) return false;
    for (int l = 1; l < S->n; ++l)
        if (n_tok > S->layers[l]->desc.max_tokens) return false;
    const bool mm = prefill_mm_ok(D.d_model, D.d_ff, fs_main(L));
    *big = mm && prefill_big_tiles(D.d_model, D.d_ff, fs_main(L), D.act_dtype != MOE_ACT_BF16, n_tok, D.top_k,
                                   std::min(D.n_experts, n_tok * D.top_k));
    return true;
}

size_t moe_stack_workspace_bytes(moe_layer* const* layers, int n) {
    if (validate_stack(layers, n) != MOE_OK) return 0;
    return stack_carve(layers, n, nullptr, nullptr);
}

int moe_stack_create(moe_layer* const* layers, int n, void* d_workspace, size_t ws_bytes, moe_stack** out) {
    if (!out) return MOE_E_INVALID;
    *out = nullptr;
    int rc = validate_stack(layers, n);
    if (rc != MOE_OK) return rc;
    if (!d_workspace || ((uintptr_t)d_workspace & 255)) return MOE_E_INVALID;
    if (ws_bytes < stack_carve(layers, n, nullptr, nullptr)) return MOE_E_CAPACITY;
    moe_stack* S = new (std::nothrow) moe_stack();
    if (!S) return MOE_E_INVALID;
    S->layers = new (std::nothrow) moe_layer*[n];
    if (!S->layers) { delete S; return MOE_E_INVALID; }
    for (int l = 0; l < n; ++l) S->layers[l] = layers[l];
    S->n = n;
    S->wait_polls = kDefaultWaitPolls;
    stack_carve(layers, n, (uint8_t*)d_workspace, S);
    rc = stack_sort_init(S);
    if (rc != MOE_OK) { moe_stack_destroy(S); return rc; }
    S->one_ok = stack_one_launch_ok(layers, n) && S->d_xchg != nullptr && S->xchg_tokens >= 1;
    if (S->one_ok) {
        rc = stack_one_launch_init(S);
        if (rc != MOE_OK) { moe_stack_destroy(S); return rc; }
    }
    *out = S;
    return MOE_OK;
}

int moe_stack_set_one_launch(moe_stack* S, int enable) {
    if (!S) return MOE_E_INVALID;
    if (enable && !S->one_ok) return MOE_E_UNSUPPORTED;
    S->one_launch = enable != 0;
    return MOE_OK;
}

int moe_stack_set_wait_limit(moe_stack* S, unsigned polls) {
    if (!S) return MOE_E_INVALID;
    S->wait_polls = polls ? polls : kDefaultWaitPolls;
    return MOE_OK;
}

int moe_stack_set_profiling(moe_stack* S, int enable) {
    if (!S) return MOE_E_INVALID;
    if (enable && !S->ev_t[0]) {
        for (int i = 0; i < 4; ++i) HIPCHK(hipEventCreate(&S->ev_t[i]));
    }
    S->profiling = enable != 0;
    S->ev_used[0] = S->ev_used[1] = false;
    return MOE_OK;
}

int moe_stack_kernel_ms(moe_stack* S, float* ms_router, float* ms_step) {
    if (!S) return MOE_E_INVALID;
    float* outs[2] = {ms_router, ms_step};
    for (int i = 0; i < 2; ++i) {
        if (!outs[i]) continue;
        *outs[i] = -1.f;
        if (S->ev_used[i] && S->ev_t[2 * i]) {
            HIPCHK(hipEventSynchronize(S->ev_t[2 * i + 1]));
            HIPCHK(hipEventElapsedTime(outs[i], S->ev_t[2 * i], S->ev_t[2 * i + 1]));
        }
    }
    return MOE_OK;
}

int moe_stack_set_staging(moe_stack* S, void* copy_stream, int mode) {
    if (!S || mode < MOE_STAGE_OFF || mode > MOE_STAGE_ON_DEMAND) return MOE_E_INVALID;
    if (mode != MOE_STAGE_OFF)
        for (int l = 0; l < S->n; ++l)
            if (!S->layers[l]->dev_staging) return MOE_E_UNSUPPORTED;
    S->stage_mode = mode;
    S->copy_stream = (hipStream_t)copy_stream;
    return MOE_OK;
}

int moe_stack_set_trace(moe_stack* S, float* d_x_trace, size_t n_floats) {
    if (!S || (n_floats && !d_x_trace)) return MOE_E_INVALID;
    S->x_trace = n_floats ? d_x_trace : nullptr;
    S->trace_cap = n_floats;
    return MOE_OK;
}

// copy layer l's input residual stream into the trace (when one is set)
static int trace_layer(moe_stack* S, int l, const void* x, int n_tok, hipStream_t st) {
    if (!S->x_trace) return MOE_OK;
    const size_t per = (size_t)n_tok * S->layers[0]->desc.d_model;
    HIPCHK(hipMemcpyAsync(S->x_trace + (size_t)l * per, x, per * sizeof(float), hipMemcpyDeviceToDevice, st));
    return MOE_OK;
}

int moe_stack_decode(moe_stack* S, const float* x_in, float* x_out, int n_tok, const int32_t* route_idx,
                     const float* route_w, int32_t* pred_idx, float* pred_w, int32_t* used_idx, float* used_w,
                     const int32_t* hist_prev, int first_step, void* stream) {
    if (!S || !x_in || !x_out || !pred_idx || !pred_w) return MOE_E_INVALID;
    if (!first_step && (!route_idx || !route_w)) return MOE_E_INVALID;
    const int k = S->layers[0]->desc.top_k;
    const size_t per = (size_t)n_tok * k;
    if (n_tok < 1 || n_tok * k > 4096 || n_tok > 256) return MOE_E_UNSUPPORTED;
    if (S->x_trace && (size_t)S->n * n_tok * S->layers[0]->desc.d_model > S->trace_cap) return MOE_E_CAPACITY;
    if (first_step) S->step = 0;
    if (S->one_launch && !first_step && S->stage_mode == MOE_STAGE_OFF && n_tok <= S->xchg_tokens &&
        stack_one_fast_ok(S->layers[0]->desc.d_model, S->layers[0]->desc.d_ff, fs_main(S->layers[0]), n_tok, k)) {
        for (int l = 0; l < S->n; ++l)
            if (n_tok > S->layers[l]->desc.max_tokens) return MOE_E_INVALID;
        const int rc = stack_decode_one(S, x_in, x_out, n_tok, route_idx, route_w, pred_idx, pred_w, used_idx,
                                        used_w, hist_prev, (hipStream_t)stream);
        if (rc == MOE_OK) S->step++;
        return rc;
    }
    const bool on_demand = S->stage_mode == MOE_STAGE_ON_DEMAND;
    const bool prerouted = S->stage_mode == MOE_STAGE_PREROUTED;
    bool big = false;
    const bool presort = stack_sort_hoist(S, n_tok, first_step, &big);
    if (presort) {
        SortCall c{route_idx, route_w, used_idx, used_w, per, n_tok, big ? 1 : 0};
        HIPCHK(launch_sort_layers(S->d_sort_tab, S->n - 1, S->layers[1]->desc.n_experts, c, (hipStream_t)stream));
    }
    TopkJob pend{};
    bool pro_done = false;                   // this layer's prologue was taken by the previous combine
    for (int l = 0; l < S->n; ++l) {
        moe_layer* L = S->layers[l];
        moe_io io{};
        io.x_in = l == 0 ? x_in : x_out;
        io.y_out = x_out;
        const bool self = first_step || l == 0 || on_demand;
        if (S->stage_mode != MOE_STAGE_OFF) L->cur_buf = L->nbuf == 2 ? (int)(S->step & 1) : 0;
        io.route_idx = self ? nullptr : route_idx + l * per;
        io.route_w = self ? nullptr : route_w + l * per;
        io.used_idx = used_idx ? used_idx + l * per : nullptr;
        io.used_w = used_w ? used_w + l * per : nullptr;
        if (l + 1 < S->n) {
            io.pred_idx = pred_idx + (l + 1) * per;
            io.pred_w = pred_w + (l + 1) * per;
            io.hist_cur = (first_step || on_demand) ? nullptr : route_idx + (l + 1) * per;
            io.hist_prev = hist_prev ? hist_prev + (l + 1) * per : nullptr;
        }
        int rc = check_io(L, &io, n_tok);
        if (rc != MOE_OK) return rc;
        rc = trace_layer(S, l, io.x_in, n_tok, (hipStream_t)stream);
        if (rc != MOE_OK) return rc;
        TopkJob out{};
        PrologueArgs nxt{};
        if (l + 1 < S->n) nxt = prologue_args(S->layers[l + 1], x_out, n_tok);
        bool took = false;
        const bool stage_next = prerouted && l >= 1;
        L->presorted = presort && l >= 1;
        rc = run_decode(L, &io, n_tok, (hipStream_t)stream, pend.pred_idx ? &pend : nullptr,
                        l + 1 < S->n ? &out : nullptr, l + 1 < S->n ? &nxt : nullptr, pro_done, &took,
                        stage_next ? L->ev_pred : nullptr);
        L->presorted = false;
        if (rc != MOE_OK) return rc;
        pend = out;
        pro_done = took;
        if (stage_next) {
            // layer l's routing for the next step (head l-1's prediction, final
            // after this call's first launch) goes to the buffer the next step
            // reads; one slab: after this call is done with it
            const int nb = L->nbuf == 2 ? (L->cur_buf ^ 1) : 0;
            HIPCHK(hipStreamWaitEvent(S->copy_stream, L->nbuf == 2 ? L->ev_pred : L->ev_done, 0));
            rc = stage_device(L, pred_idx + l * per, (int)per, nb, S->copy_stream);
            if (rc != MOE_OK) return rc;
            HIPCHK(hipEventRecord(L->ev_staged_buf[nb], S->copy_stream));
            L->staged_pending_buf[nb] = true;
        }
    }
    S->step++;
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
    if (S->x_trace && (size_t)S->n * n_tok * S->layers[0]->desc.d_model > S->trace_cap) return MOE_E_CAPACITY;
    bool pro_done = false;                   // this layer's prologue was taken by the previous combine
    for (int l = 0; l < S->n; ++l) {
        moe_layer* L = S->layers[l];
        moe_io io{};
        io.x_in = x;
        io.y_out = x;
        if (l > 0) {
            // the previous layer's predictions by token, shifted by one token
            // inside the call (token 0 self-routes); without caller buffers
            // they sit in scratch buffer (l - 1) & 1 while this layer writes
            // its own into the other one
            io.route_idx = pred_idx ? pred_idx + l * per : S->d_pred_idx[(l - 1) & 1];
            io.route_w = pred_w ? pred_w + l * per : S->d_pred_w[(l - 1) & 1];
        }
        io.used_idx = used_idx ? used_idx + l * per : nullptr;
        io.used_w = used_w ? used_w + l * per : nullptr;
        if (l + 1 < S->n) {
            io.pred_idx = pred_idx ? pred_idx + (l + 1) * per : S->d_pred_idx[l & 1];
            io.pred_w = pred_w ? pred_w + (l + 1) * per : S->d_pred_w[l & 1];
        }
        int rc = check_io(L, &io, n_tok);
        if (rc != MOE_OK) return rc;
        rc = trace_layer(S, l, x, n_tok, st);
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
    for (int i = 0; i < 4; ++i)
        if (S->ev_t[i]) (void)hipEventDestroy(S->ev_t[i]);
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

// moe_plan_slots: host_plan.cpp (plain C++, also built with the host sanitizers in the CPU tests)

}  // extern "C"

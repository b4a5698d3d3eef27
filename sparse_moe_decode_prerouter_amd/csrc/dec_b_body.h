// K_B's body (int4 down GEMV + routing-weighted combine + sigmoid-gated
// shared expert + LoRA B + residual), shared by the standalone launch and
// by the one-launch-per-layer decode kernel, where it runs in the same grid
// as K_A and waits, inside the launch, for K_A's hidden activations.
//
// Block 0 takes the head's top-k (it is dispatched first, so it overlaps the
// rest); every other block owns RB consecutive output rows.
//
// Lane layout (F = d_ff): a Wd row holds F/2 bytes of packed int4, i.e.
// LPR = F/8 dwords; lane c of a row group owns dword c, so it needs h
// elements [8c, 8c+8) only (no lane loads h it does not use). RPP = 64/LPR
// rows are covered per pass and kPassB passes per block: RB = kPassB * RPP.
// Each wave runs the routed experts s = wave, wave + 4, ... and kPassB/4 of
// the shared expert's passes, so all four waves do the same program: every
// wave reads the routing digest itself (no cross-wave wait) and all loads
// that need no routing are issued before the digest is consumed.
// Partial sums go to LDS indexed by assignment id (t*k + j) or shared
// token, and each (token, row) output sums them in routing order, so the
// result does not depend on how slots are spread over waves.
//
// FUSED (the one-launch stack decode): the values produced in the same
// launch (K_A's h, shared h, shared gate, LoRA A u and head logits; the
// residual rows x, written by the previous layer) are read with device-scope
// loads until every word a wave needs has been published (fuse_poll), and y
// is published with device-scope stores; everything else, weights included,
// is issued before the first poll.
#pragma once
#include "dec_common.h"
#include "fuse_sync.h"
#include "device_common.h"
#include "moe_internal.h"
#include "topk.h"

namespace moe {

constexpr int kPassB = 4;
constexpr int kMaxTokB = 16;

template <int F, int PB = kPassB>
struct BGeo {
    static constexpr int LPR = F / 8;
    static constexpr int RPP = 64 / LPR;
    static constexpr int RB = PB * RPP;
};

// LoRA B row (r bf16) . LoRA A output row (r fp32): the loads are issued
// together up front and the products summed later, in q order.
constexpr int kLoraChunks = 2;                // r <= 16, r % 8 == 0
struct LoraRegs {
    u32x4 b[kLoraChunks];
    float4 u[2 * kLoraChunks];
};
__device__ __forceinline__ void lora_issue_b(LoraRegs& R, const uint16_t* brow, int r) {
#pragma unroll
    for (int c = 0; c < kLoraChunks; ++c) {
        const int cc = 8 * c < r ? c : 0;
        R.b[c] = *(const u32x4*)(brow + 8 * cc);
    }
}
// COH: LoRA A u of this launch (base: the same for the whole wave)
template <bool COH>
__device__ __forceinline__ void lora_issue_u(LoraRegs& R, const float* base, size_t row_off, int r) {
#pragma unroll
    for (int c = 0; c < kLoraChunks; ++c) {
        const int cc = 8 * c < r ? c : 0;
        if constexpr (COH) {
            R.u[2 * c] = u4_as_f4(ld_coh4(base, (uint32_t)(row_off + 8 * cc)));
            R.u[2 * c + 1] = u4_as_f4(ld_coh4(base, (uint32_t)(row_off + 8 * cc + 4)));
        } else {
            const float* urow = base + row_off;
            R.u[2 * c] = *(const float4*)(urow + 8 * cc);
            R.u[2 * c + 1] = *(const float4*)(urow + 8 * cc + 4);
        }
    }
}
__device__ __forceinline__ float lora_dot(const LoraRegs& R, int r) {
    float l = 0.f;
#pragma unroll
    for (int c = 0; c < kLoraChunks; ++c) {
        if (8 * c < r) {
            const uint32_t bw[4] = {R.b[c].x, R.b[c].y, R.b[c].z, R.b[c].w};
            const float uu[8] = {R.u[2 * c].x, R.u[2 * c].y, R.u[2 * c].z, R.u[2 * c].w,
                                 R.u[2 * c + 1].x, R.u[2 * c + 1].y, R.u[2 * c + 1].z, R.u[2 * c + 1].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                l += bf16_to_f32(bw[i] & 0xFFFF) * uu[2 * i];
                l += bf16_to_f32(bw[i] >> 16) * uu[2 * i + 1];
            }
        }
    }
    return l;
}

// One expert's Wd rows for this lane: NP passes of (dword of int4, (s,b)).
template <int NP>
struct DownRegs {
    uint32_t q[NP];
    uint32_t sb[NP];
};

// Rows row_first + i * STEP, i < NP: one base address, compile-time offsets.
template <int F, int NP, int STEP>
__device__ __forceinline__ void down_issue(DownRegs<NP>& R, const uint8_t* blob, const BlobLayout& L, int row_first) {
    using G = BGeo<F>;
    const int lane = threadIdx.x & 63, c = lane % G::LPR;
    const uint32_t* q = (const uint32_t*)(blob + L.down_q) + (size_t)row_first * (F / 8) + c;
    const uint32_t* sb = (const uint32_t*)(blob + L.down_sb) + (size_t)row_first * (F / 64) + c / 8;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        R.q[i] = __builtin_nontemporal_load(q + i * STEP * (F / 8));
        R.sb[i] = __builtin_nontemporal_load(sb + i * STEP * (F / 64));
    }
}

// the lane's 8 elements of h row `row_off` past `base` (COH: published in
// this launch; base the same for the whole wave)
template <bool COH>
__device__ __forceinline__ void h_issue(float4 (&hv)[2], const float* base, size_t row_off, int c) {
    if constexpr (COH) {
        hv[0] = u4_as_f4(ld_coh4(base, (uint32_t)(row_off + 8 * c)));
        hv[1] = u4_as_f4(ld_coh4(base, (uint32_t)(row_off + 8 * c + 4)));
    } else {
        const float* hrow = base + row_off;
        hv[0] = *(const float4*)(hrow + 8 * c);
        hv[1] = *(const float4*)(hrow + 8 * c + 4);
    }
}

// (one-launch step) h_issue<true>, read until its 8 words have been published
__device__ __forceinline__ void h_poll(float4 (&hv)[2], const float* base, size_t row_off, int c, const FuseSync& fs,
                                       int32_t* err) {
    fuse_poll(fs, err, nullptr, [&]() {
        h_issue<true>(hv, base, row_off, c);
        return !(any_empty(hv[0]) | any_empty(hv[1]));
    });
}

// Per-lane partial of each pass: sum_j (s q_j + b) h_j over the lane's 8 elements.
template <int NP>
__device__ __forceinline__ void down_partial(const DownRegs<NP>& R, const float4 (&hv)[2], float (&o)[NP]) {
    const float h[8] = {hv[0].x, hv[0].y, hv[0].z, hv[0].w, hv[1].x, hv[1].y, hv[1].z, hv[1].w};
    float hs = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) hs += h[j];
    // codes split into even and odd nibbles, one per byte (a mask held in a
    // register the compiler cannot see through, so it is not re-materialised
    // per use): each code then converts with one v_cvt_f32_ubyte
    uint32_t m0f = 0x0F0F0F0Fu;
    asm volatile("" : "+v"(m0f));
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const uint32_t ev = R.q[i] & m0f, od = (R.q[i] >> 4) & m0f;
        float acc = 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            acc += (float)((ev >> (8 * b)) & 0xFFu) * h[2 * b];
            acc += (float)((od >> (8 * b)) & 0xFFu) * h[2 * b + 1];
        }
        o[i] = f16_to_f32(R.sb[i] & 0xFFFF) * acc + f16_to_f32(R.sb[i] >> 16) * hs;
    }
}

template <int F, bool FUSED, int PB = kPassB, typename BA = DecBArgs>
__device__ __forceinline__ void dec_b_body(const BA& a, int bid, const FuseSync& fs) {
    using G = BGeo<F, PB>;
    constexpr int NPS = PB / kWaves;               // shared-expert passes per wave
    __shared__ float part[(kMaxAssign + kMaxTokB) * G::RB];
    __shared__ uint32_t sl[kWaves][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (bid == 0) {
        if constexpr (FUSED) {
            // this wave's logit rows (those topk_rows gives it), until published
            if (a.pred_idx)
                for (int t = wave; t < a.n_tok; t += kWaves)
                    fuse_poll(fs, a.err, nullptr, [&]() {
                        bool empty = false;
                        for (int e = lane; e < a.En; e += 64) empty |= empty_word(ld_dev(a.logits_h + (size_t)t * a.En + e));
                        return !empty;
                    });
        }
        // (the one-launch kernel takes heads of up to 256 experts: smaller
        // register arrays, which keep its register budget)
        if (a.pred_idx)
            topk_rows<FUSED ? kStackHeadMaxPer : 16>(FUSED, a.logits_h, a.En, a.kn, a.n_tok, a.head_bias, a.hist_cur_m, a.hist_cur, a.hist_prev_m,
                      a.hist_prev, nullptr, a.kn, a.pred_idx, a.pred_w);
        return;
    }
    const int d = a.d, n_tok = a.n_tok, k = a.k;
    const int n_assign = n_tok * k;
    const int row0 = (bid - 1) * G::RB;
    const bool has_shared = a.fs != 0;
    const BlobLayout L = BlobLayout::make(d, F);
    const int c = lane % G::LPR, rsub = lane / G::LPR;
    // (one-launch step) the exchange-buffer copy this block reads
    const int ncopy = FUSED ? (a.xcopies > 0 ? a.xcopies : 1) : 1;
    const size_t xo = FUSED ? (size_t)((int)blockIdx.x % ncopy) * a.xstride : 0;
    // the epilogue's fields, read here and (one-launch step) held in scalar
    // registers: read after the waits, each would be a dependent scalar load
    // on the critical path
    float* ep_y = a.y;
    float* ep_xn = FUSED ? a.xnext : nullptr;
    float* ep_yc = FUSED ? a.y_copy : nullptr;
    float ep_ls = a.lora_scale;
    size_t ep_xs = FUSED ? a.xstride : 0;
    int ep_k = a.k;
    if constexpr (FUSED) asm volatile("" : "+s"(ep_y), "+s"(ep_xn), "+s"(ep_yc), "+s"(ep_ls), "+s"(ep_xs), "+s"(ep_k));

    // ---- level 0, identical in every wave. The routing entries go first
    // (K_A read them on every XCD, so they are L2 hits); all other loads need
    // no routing and are issued unconditionally (clamped indices, stand-in
    // pointers), so waiting for the routing never waits for them.
    const RouteIn rin = route_load(a.route_idx, a.route_w, a.self_idx, a.self_w, n_assign);
    float v_sg = 0.f;
    if constexpr (!FUSED) v_sg = (a.sgate ? a.sgate : (const float*)a.err)[lane < n_tok ? lane : 0];
    // epilogue operands: thread -> (token, row)
    const int ep_n = n_tok * G::RB;
    const int ep_q = tid < ep_n ? tid : 0;
    const int et = ep_q / G::RB, er = ep_q % G::RB;
    float ep_x = 0.f;
    if constexpr (!FUSED) ep_x = a.fused ? a.x[(size_t)et * d + row0 + er] : 0.f;
    const bool lora_on = a.lora_b && a.r;
    const bool lora_vec = lora_on && (a.r & 7) == 0 && a.r <= 8 * kLoraChunks;
    LoraRegs lr;
    if (lora_vec) {
        lora_issue_b(lr, a.lora_b + (size_t)(row0 + er) * a.r, a.r);
        if constexpr (!FUSED) lora_issue_u<false>(lr, a.au, (size_t)et * a.r, a.r);
    }
    // shared expert: passes [NPS*wave, NPS*wave + NPS), token 0's hidden state
    const uint8_t* sh_blob = has_shared && a.ev.shared ? a.ev.shared : a.ev.base;
    DownRegs<NPS> shr;
    down_issue<F, NPS, G::RPP>(shr, sh_blob, L, row0 + NPS * wave * G::RPP + rsub);
    const int sh_tag = *(a.ev.shared_tag ? a.ev.shared_tag : a.err);
    const bool sh_ok = has_shared && a.ev.shared && (!a.ev.shared_tag || sh_tag == a.ev.E);
    float4 shh[2];
    if constexpr (!FUSED) h_issue<false>(shh, has_shared ? a.hs : a.h, 0, c);
    // zero the partials: entries of invalid assignments are never written
    for (int i = tid; i < (n_assign + n_tok) * G::RB; i += kThreads) part[i] = 0.f;
    lds_barrier();

    // ---- level 1: this wave sorts the routing (registers + its LDS slice),
    // then the routed experts, two slots in flight per wave. The first pair
    // is issued before the shared expert is computed (its loads are the
    // oldest, so waiting for them does not wait for the routed rows).
    int me;
    float mw;
    route_merge(rin, a.route_idx != nullptr, k, n_assign, &me, &mw);
    const WaveDigest W = wave_digest(n_assign, me, a.E, sl[wave]);
    const int n_active = W.n_active, n_valid = W.n_valid;
    auto blob_of = [&](int s) -> const uint8_t* {
        if (s >= n_active) return nullptr;
        const int e = __builtin_amdgcn_readlane((int)(W.sk >> 16), nth_set(W.starts, s));
        if (!a.ev.slot_of) return a.ev.base + (size_t)e * a.ev.blob;
        const int sl = a.ev.slot_of[e];
        if (sl < 0 || (a.ev.slot_tag && a.ev.slot_tag[sl] != e)) return nullptr;
        return a.ev.base + (size_t)sl * a.ev.blob;
    };
    auto slot_compute = [&](const DownRegs<PB>& R, const uint8_t* blob, int s, const float4 (&h0)[2]) {
        const int p0 = nth_set(W.starts, s);
        const int p1 = s + 1 < n_active ? nth_set(W.starts, s + 1) : n_valid;
        for (int p = p0; p < p1; ++p) {
            float4 hv[2];
            if (p == p0) { hv[0] = h0[0]; hv[1] = h0[1]; }
            else if constexpr (FUSED) h_poll(hv, a.h + xo, (size_t)p * F, c, fs, a.err);
            else h_issue<false>(hv, a.h, (size_t)p * F, c);
            float o[PB];
            down_partial<PB>(R, hv, o);
            int pass;
            const float tot = row_reduce<float, PB, G::LPR>(o, &pass);
            const int aid = __builtin_amdgcn_readlane((int)(W.sk & 0xFFFF), p);
            const float wgt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mw), aid < n_assign ? aid : 0));
            if (blob && (c % (G::LPR / PB)) == 0 && aid >= 0 && aid < n_assign)
                part[aid * G::RB + pass * G::RPP + rsub] = wgt * tot;
        }
    };
    auto rows_issue = [&](int s0, DownRegs<PB>& R0, DownRegs<PB>& R1, const uint8_t*& b0, const uint8_t*& b1) {
        const int s1 = s0 + kWaves;
        b0 = blob_of(s0);
        b1 = blob_of(s1);
        // (a slot past the active experts loads the first slot's rows again,
        // which the L2 already holds, instead of rows of some other blob)
        down_issue<F, PB, G::RPP>(R0, b0 ? b0 : a.ev.base, L, row0 + rsub);
        down_issue<F, PB, G::RPP>(R1, b1 ? b1 : (b0 ? b0 : a.ev.base), L, row0 + rsub);
    };
    auto hs_issue = [&](int s0, float4 (&h0)[2], float4 (&h1)[2]) {
        const int s1 = s0 + kWaves;
        const int q0 = s0 < n_active ? nth_set(W.starts, s0) : 0;
        const int q1 = s1 < n_active ? nth_set(W.starts, s1) : 0;
        h_issue<FUSED>(h0, a.h, (size_t)q0 * F, c);
        h_issue<FUSED>(h1, a.h, (size_t)q1 * F, c);
    };
    auto shared_compute = [&]() {
        if (has_shared) {
            for (int t = 0; t < n_tok; ++t) {
                float4 hv[2];
                if (t == 0) { hv[0] = shh[0]; hv[1] = shh[1]; }
                else if constexpr (FUSED) h_poll(hv, a.hs + xo, (size_t)t * F, c, fs, a.err);
                else h_issue<false>(hv, a.hs, (size_t)t * F, c);
                float o[NPS];
                down_partial<NPS>(shr, hv, o);
                int pass;
                const float tot = row_reduce<float, NPS, G::LPR>(o, &pass);
                const float wgt = a.sgate ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v_sg), t)) : 1.f;
                if (sh_ok && (c % (G::LPR / NPS)) == 0)
                    part[(n_assign + t) * G::RB + (NPS * wave + pass) * G::RPP + rsub] = wgt * tot;
            }
        }
    };
    if constexpr (FUSED) {
        // one slot in flight per wave (a batch-1 step has one routed expert
        // per wave); the values of this launch are read after the wait
        auto slot_issue = [&](int s, DownRegs<PB>& R, const uint8_t*& bb) {
            bb = blob_of(s);
            down_issue<F, PB, G::RPP>(R, bb ? bb : a.ev.base, L, row0 + rsub);
        };
        {
            DownRegs<PB> R0;
            float4 h0[2] = {};
            const uint8_t* b0;
            slot_issue(wave, R0, b0);
            // every value of this launch the wave reads before its first
            // slot: the shared gate, the residual rows (published by the
            // previous layer, or the caller's x at layer 0), LoRA A u, the
            // shared expert's h and the first slot's h; the probe is the
            // first slot's h (else the shared h, else nothing)
            const bool h0_on = wave < n_active;
            const int q0 = h0_on ? nth_set(W.starts, wave) : 0;
            const float* probe = h0_on ? a.h + xo + (size_t)q0 * F : (has_shared ? a.hs + xo : nullptr);
            // every load is issued on every poll, absent inputs from a
            // readable stand-in, and only then tested: a load under a branch
            // would be waited for before the next one is issued
            const float* sg_p = a.sgate ? a.sgate + xo + (lane < n_tok ? lane : 0) : (const float*)a.err;
            const float* ex_p = a.fused ? a.x + (size_t)et * d + row0 + er : (const float*)a.err;
            const float* au_p = lora_vec ? a.au + xo : a.h + xo;
            const float* hs_p = has_shared ? a.hs + xo : a.h + xo;
            fuse_poll(fs, a.err, probe, [&]() {
                v_sg = ld_dev(sg_p);
                ep_x = ld_dev(ex_p);
                lora_issue_u<true>(lr, au_p, lora_vec ? (size_t)et * a.r : 0, lora_vec ? a.r : 8);
                h_issue<true>(shh, hs_p, 0, c);
                h_issue<true>(h0, a.h + xo, (size_t)q0 * F, c);
                bool empty = (a.sgate && empty_word(v_sg)) | (a.fused && a.x_repl && empty_word(ep_x));
                bool eu = false;
#pragma unroll
                for (int q = 0; q < 2 * kLoraChunks; ++q) eu |= any_empty(lr.u[q]);
                empty |= lora_vec && eu;
                empty |= has_shared && (any_empty(shh[0]) | any_empty(shh[1]));
                empty |= h0_on && (any_empty(h0[0]) | any_empty(h0[1]));
                return !empty;
            });
            shared_compute();
            if (h0_on) slot_compute(R0, b0, wave, h0);
        }
        for (int s0 = wave + kWaves; s0 < n_active; s0 += kWaves) {
            DownRegs<PB> R0;
            float4 h0[2];
            const uint8_t* b0;
            slot_issue(s0, R0, b0);
            h_poll(h0, a.h + xo, (size_t)nth_set(W.starts, s0) * F, c, fs, a.err);
            slot_compute(R0, b0, s0, h0);
        }
    } else {
        {
            DownRegs<PB> R0, R1;
            float4 h0[2], h1[2];
            const uint8_t *b0, *b1;
            rows_issue(wave, R0, R1, b0, b1);
            hs_issue(wave, h0, h1);
            shared_compute();
            if (wave < n_active) slot_compute(R0, b0, wave, h0);
            if (wave + kWaves < n_active) slot_compute(R1, b1, wave + kWaves, h1);
        }
        for (int s0 = wave + 2 * kWaves; s0 < n_active; s0 += 2 * kWaves) {
            DownRegs<PB> R0, R1;
            float4 h0[2], h1[2];
            const uint8_t *b0, *b1;
            rows_issue(s0, R0, R1, b0, b1);
            hs_issue(s0, h0, h1);
            slot_compute(R0, b0, s0, h0);
            if (s0 + kWaves < n_active) slot_compute(R1, b1, s0 + kWaves, h1);
        }
    }
    lds_barrier();

    // ---- epilogue: shared, then routed in routing order, LoRA B, residual
    if (tid < ep_n) {
        float y = has_shared ? part[(n_assign + et) * G::RB + er] : 0.f;
        for (int j = 0; j < ep_k; ++j) y += part[(et * ep_k + j) * G::RB + er];
        if (lora_on) {
            float l = 0.f;
            if (lora_vec) l = lora_dot(lr, a.r);
            else
                for (int q = 0; q < a.r; ++q)
                    l += bf16_to_f32(a.lora_b[(size_t)(row0 + er) * a.r + q]) *
                         (FUSED ? ld_dev(a.au + xo + (size_t)et * a.r + q) : a.au[(size_t)et * a.r + q]);
            y += ep_ls * l;
        }
        if (a.fused) y += ep_x;
        if constexpr (FUSED) {
            const size_t yi = (size_t)et * d + row0 + er;
            if (ep_y) st_dev(ep_y + yi, y);
            if (ep_xn)
                for (int cc = 0; cc < ncopy; ++cc) st_dev(ep_xn + cc * ep_xs + yi, y);
            if (ep_yc) ep_yc[yi] = y;
        } else {
            ep_y[(size_t)et * d + row0 + er] = y;
        }
    }
}

}  // namespace moe

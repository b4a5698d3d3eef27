// K_A's body: RMSNorm prologue + routing digest + int4 gate/up GEMV with
// SwiGLU (routed experts and the shared expert) + prerouter head logits +
// LoRA A u + shared-expert gate. Shared by the standalone launch and by the
// one-launch-per-step stack decode kernel, where x is produced inside the same
// launch (by the previous layer's K_B blocks): there the block issues every
// load that does not depend on x, then reads x with device-scope loads until
// every word has arrived (fuse_poll), and publishes its outputs with
// device-scope stores.
//
// A block (4 waves) computes the block input u of a token once: thread g
// owns elements [8g, 8g+8), the RMSNorm sum of squares is reduced in fp64
// over the block, and u, rounded once to the activation dtype, goes to LDS
// in the layout the dot products read without bank conflicts. Each wave then
// multiplies its weight rows: a lane owns one 32-element chunk of a row
// (LPR = d/32 lanes per row), i.e. 16 bytes of packed int4 or 64 bytes of a
// bf16 row.
//
// Latency: every load that needs no routing (routing entries, x, gamma, the
// shared expert's rows, the bf16 rows) is issued at kernel start, without
// branches around it, so the compiler's in-order wait counts stay exact; each
// routed wave sorts the routing itself (registers + its own LDS slice) and
// issues its expert's rows before u is computed.
#pragma once
#include "device_common.h"
#include "moe_internal.h"
#include "dec_common.h"
#include "fuse_sync.h"
#include "topk.h"

namespace moe {

constexpr int kAPass = 2;                 // int4 h-row passes per wave
constexpr int kABPass = 1;                // bf16-row passes per wave

template <int D, int AP = kAPass>
struct AGeo {
    static constexpr int LPR = D / 32;    // lanes per weight row
    static constexpr int RPW = 64 / LPR;  // rows per pass
    static constexpr int HROWS = kWaves * AP * RPW;        // h rows per block
    static constexpr int BROWS = kWaves * kABPass * RPW;   // bf16 rows per block
    static constexpr int C = D / 32;      // 32-element chunks
};

// ---- block input u in LDS -------------------------------------------------
// pk: [4 pieces][C chunks][4 dwords] bf16 pairs in GEMV order: dword p of
//     piece i of chunk c is (e_{32c+8i+p}, e_{32c+8i+p+4}); lane c reads
//     piece i of its chunk at step i, consecutive lanes at consecutive 16 B.
// pk_lo: same for the lo part (f32 activations).
// uf: [8 pieces][C chunks][4 floats] activation values.
// usum, usum_lo: [C] chunk sums of the hi / lo parts.
template <int D>
struct ULds {
    uint32_t pk[4 * D / 8];
    uint32_t pk_lo[4 * D / 8];
    float uf[D];
    float usum[D / 32], usum_lo[D / 32];
    double red[kWaves];
};

struct XThread {
    uint32_t w[8];      // 8 fp32 words, or 4 bf16 pairs
    float g[8];
};

// COH: x of this launch, read from copy xo of the exchange buffer
template <bool XB, bool COH = false, typename AA>
__device__ __forceinline__ void x_issue(const AA& a, int t, int e0, uint32_t (&w)[8], size_t xo = 0) {
    if constexpr (COH) {
        static_assert(!XB, "in-launch x is fp32");
        const float* base = (const float*)a.x + xo;
        const uint32_t el = (uint32_t)(t * a.d + e0);
        const u32x4 v0 = ld_coh4(base, el), v1 = ld_coh4(base, el + 4);
        w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
        w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
    } else if (XB) {
        const u32x4 v = *(const u32x4*)((const uint16_t*)a.x + (size_t)t * a.d + e0);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
        const u32x4 v0 = *(const u32x4*)((const float*)a.x + (size_t)t * a.d + e0);
        const u32x4 v1 = *(const u32x4*)((const float*)a.x + (size_t)t * a.d + e0 + 4);
        w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
        w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
    }
}

// (one-launch step) x of token t, read until every word of this lane's
// elements has been published (a plain read when fs is off: layer 0's x is
// the caller's)
template <bool XB, typename AA>
__device__ __forceinline__ void x_poll(const AA& a, int t, int e0, uint32_t (&w)[8], size_t xo, const FuseSync& fs) {
    const float* probe = (const float*)a.x + xo + (size_t)t * a.d + __builtin_amdgcn_readfirstlane(e0);
    fuse_poll(fs, a.err, probe, [&]() {
        x_issue<XB, true>(a, t, e0, w, xo);
        bool empty = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) empty |= w[i] == kEmptyWord;
        return !empty;
    });
}

template <bool XB>
__device__ __forceinline__ float x_elem(const uint32_t (&w)[8], int i) {
    return XB ? bf16_to_f32((w[i >> 1] >> (16 * (i & 1))) & 0xFFFF) : __uint_as_float(w[i]);
}

// All threads of the block: u of one token into LDS (two block barriers).
template <int D, bool XB, typename AA>
__device__ __forceinline__ void u_to_lds(const AA& a, const XThread& X, ULds<D>& S) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool mine = tid * 8 < D;
    double inv = 1.0;
    if (a.fused) {
        double ss = 0.0;
        if (mine) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double xv = x_elem<XB>(X.w, i);
                ss += xv * xv;
            }
        }
        ss = group_sum_dpp<double, 64>(ss);
        if (lane == 0) S.red[wave] = ss;
        lds_barrier();
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tot += S.red[w];
        inv = 1.0 / sqrt(tot / (double)D + (double)a.eps);
    }
    // one branch around each form of the loop, not one per element; with
    // bf16 activations the lo part is zero and is not formed; without the
    // norm, inv and the gains are 1, and (x * 1) * 1 is x exactly
    uint32_t hb[8], lb[8];
    float uf[8];
    const bool act_bf16 = a.act_bf16;
    double gd[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) gd[j] = a.fused ? (double)X.g[j] : 1.0;
    if (act_bf16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            hb[j] = f64_to_bf16((x_elem<XB>(X.w, j) * inv) * gd[j]);
            uf[j] = bf16_to_f32(hb[j]);
            lb[j] = 0u;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uf[j] = (float)((x_elem<XB>(X.w, j) * inv) * gd[j]);
            hb[j] = f32_to_bf16(uf[j]);
            lb[j] = f32_to_bf16(uf[j] - bf16_to_f32(hb[j]));
        }
    }
    float sh = 0.f, sl = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) sh += bf16_to_f32(hb[j]);
    if (!act_bf16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sl += bf16_to_f32(lb[j]);
    }
    const int c = tid >> 2, i = tid & 3;                 // chunk, piece
    if (mine) {
        u32x4 v;
        v.x = hb[0] | (hb[4] << 16); v.y = hb[1] | (hb[5] << 16); v.z = hb[2] | (hb[6] << 16); v.w = hb[3] | (hb[7] << 16);
        *(u32x4*)&S.pk[(i * AGeo<D>::C + c) * 4] = v;
        if (!act_bf16) {
            u32x4 l;
            l.x = lb[0] | (lb[4] << 16); l.y = lb[1] | (lb[5] << 16); l.z = lb[2] | (lb[6] << 16); l.w = lb[3] | (lb[7] << 16);
            *(u32x4*)&S.pk_lo[(i * AGeo<D>::C + c) * 4] = l;
        }
        *(float4*)&S.uf[((2 * i) * AGeo<D>::C + c) * 4] = make_float4(uf[0], uf[1], uf[2], uf[3]);
        *(float4*)&S.uf[((2 * i + 1) * AGeo<D>::C + c) * 4] = make_float4(uf[4], uf[5], uf[6], uf[7]);
    }
    // chunk sums: the 4 threads of a chunk are 4 consecutive lanes
    sh = group_sum_dpp<float, 4>(sh);
    if (!act_bf16) sl = group_sum_dpp<float, 4>(sl);
    if (mine && i == 0) { S.usum[c] = sh; S.usum_lo[c] = sl; }
    lds_barrier();
}

// ---- int4 gate/up rows ----------------------------------------------------
template <int AP>
struct GateUpRegs {
    u32x4 g[AP], u[AP];
    uint32_t sg[AP], su[AP];
};

template <int D, int AP>
__device__ __forceinline__ void gateup_issue(GateUpRegs<AP>& R, const uint8_t* blob, const BlobLayout& L, int row_first) {
    using G = AGeo<D, AP>;
    const int c = (threadIdx.x & 63) % G::LPR;
    const u32x4* gq = (const u32x4*)(blob + L.gate_q) + (size_t)row_first * (D / 32) + c;
    const u32x4* uq = (const u32x4*)(blob + L.up_q) + (size_t)row_first * (D / 32) + c;
    const uint32_t* gs = (const uint32_t*)(blob + L.gate_sb) + (size_t)row_first * (D / 64) + c / 2;
    const uint32_t* us = (const uint32_t*)(blob + L.up_sb) + (size_t)row_first * (D / 64) + c / 2;
#pragma unroll
    for (int i = 0; i < AP; ++i) {
        R.g[i] = __builtin_nontemporal_load(gq + i * G::RPW * (D / 32));
        R.u[i] = __builtin_nontemporal_load(uq + i * G::RPW * (D / 32));
        R.sg[i] = __builtin_nontemporal_load(gs + i * G::RPW * (D / 64));
        R.su[i] = __builtin_nontemporal_load(us + i * G::RPW * (D / 64));
    }
}

// sum over the chunk of (128 + q) * u; nm, nc: the nibble-pair mask and the
// exponent in registers the compiler cannot see through (made once by the
// caller), so that each (128 + q) pair is one v_and_or_b32 (after the shift)
// instead of an AND and an OR with literal operands
__device__ __forceinline__ float chunk_dot(u32x4 w, const u32x4 (&up)[4], float acc, uint32_t nm, uint32_t nc) {
    // opaque copy: keeps the nibble unpacking after u is ready instead of
    // hoisted out of the position loop, where it would wait for the weights
    asm volatile("" : "+v"(w));
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc = dot2_bf16((ws[i] & nm) | nc, up[i].x, acc);
        acc = dot2_bf16(((ws[i] >> 4) & nm) | nc, up[i].y, acc);
        acc = dot2_bf16(((ws[i] >> 8) & nm) | nc, up[i].z, acc);
        acc = dot2_bf16(((ws[i] >> 12) & nm) | nc, up[i].w, acc);
    }
    return acc;
}

// h = silu(gate . u) * (up . u) for the wave's rows; the lanes that hold a
// row's total write h_out[row].
template <int D, bool COH, int AP>
__device__ __forceinline__ void gateup_rows(const GateUpRegs<AP>& R, const ULds<D>& S, bool with_lo, bool ok,
                                            float* h_out, int row_first, size_t xstride = 0, int ncopy = 1) {
    using G = AGeo<D, AP>;
    const int lane = threadIdx.x & 63, c = lane % G::LPR, rsub = lane / G::LPR;
    u32x4 up[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) up[i] = *(const u32x4*)&S.pk[(i * G::C + c) * 4];
    float usm = S.usum[c];
    if (with_lo) {
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = *(const u32x4*)&S.pk_lo[(i * G::C + c) * 4];
        usm += S.usum_lo[c];
    }
    float ga[AP], ua[AP];
    uint32_t nm = 0x000F000Fu, nc = 0x43004300u;
    asm volatile("" : "+v"(nm), "+v"(nc));
#pragma unroll
    for (int i = 0; i < AP; ++i) {
        float accg = chunk_dot(R.g[i], up, 0.f, nm, nc);
        float accu = chunk_dot(R.u[i], up, 0.f, nm, nc);
        if (with_lo) {
            accg = chunk_dot(R.g[i], lo, accg, nm, nc);
            accu = chunk_dot(R.u[i], lo, accu, nm, nc);
        }
        uint32_t sgw = R.sg[i], suw = R.su[i];
        asm volatile("" : "+v"(sgw), "+v"(suw));   // opaque copies, as in chunk_dot
        const float s1 = f16_to_f32(sgw & 0xFFFF), b1 = f16_to_f32(sgw >> 16);
        const float s2 = f16_to_f32(suw & 0xFFFF), b2 = f16_to_f32(suw >> 16);
        ga[i] = s1 * accg + (b1 - 128.f * s1) * usm;
        ua[i] = s2 * accu + (b2 - 128.f * s2) * usm;
    }
    int pg, pu;
    const float g = row_reduce<float, AP, G::LPR>(ga, &pg);
    const float u = row_reduce<float, AP, G::LPR>(ua, &pu);
    if (c % (G::LPR / AP) == 0) {
        const float hv = ok ? silu_f32(g) * u : 0.f;
        if constexpr (COH) {
            for (int cc = 0; cc < ncopy; ++cc) st_dev(h_out + cc * xstride + row_first + pg * G::RPW + rsub, hv);
        } else {
            h_out[row_first + pg * G::RPW + rsub] = hv;
        }
    }
}

// ---- the body -------------------------------------------------------------
// bid: the block's index in K_A's grid. FUSED: x comes from the same launch
// (see the file comment); wait for it with fs. AA: DecAArgs, or the same in
// the constant address space (a table the kernel only reads: its fields load
// as scalar loads, and the pointers in it are known to be global).
template <int D, bool XB, bool FUSED, int AP = kAPass, typename AA = DecAArgs>
__device__ __forceinline__ void dec_a_body(const AA& a, int bid, const FuseSync& fs) {
    using G = AGeo<D, AP>;
    __shared__ __align__(16) ULds<D> S;
    __shared__ uint32_t sl[kWaves][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane % G::LPR, rsub = lane / G::LPR;
    const int n_tok = a.n_tok, k = a.k, n_assign = n_tok * k;
    const bool role_h = bid < a.nb_h;
    const bool with_lo = !a.act_bf16;
    const int e0 = tid * 8 < D ? tid * 8 : 0;       // this thread's elements of x
    // (one-launch step) the exchange-buffer copy this block reads, and how many it writes
    const int ncopy = FUSED ? (a.xcopies > 0 ? a.xcopies : 1) : 1;
    const size_t xo = FUSED ? (size_t)((int)blockIdx.x % ncopy) * a.xstride : 0;
    const size_t xo_x = FUSED && a.x_repl ? xo : 0;

    // ---- level 0 (all threads, no branches around loads): routing entries
    // first, then x and gamma
    const RouteIn rin = route_load(a.route_idx, a.route_w, a.self_idx, a.self_w, n_assign);
    const int sh_tag = *(a.ev.shared_tag ? a.ev.shared_tag : a.meta);
    XThread X;
    if constexpr (!FUSED) x_issue<XB>(a, 0, e0, X.w);
    {
        // unconditional (a stand-in of 8 readable floats when there is no
        // norm): a load under a branch would make its result wait at the join
        const float* gp = a.fused ? a.gamma + e0 : a.wsort;
        const float4 g0 = *(const float4*)gp, g1 = *(const float4*)(gp + 4);
        X.g[0] = g0.x; X.g[1] = g0.y; X.g[2] = g0.z; X.g[3] = g0.w;
        X.g[4] = g1.x; X.g[5] = g1.y; X.g[6] = g1.z; X.g[7] = g1.w;
    }

    if (role_h) {
        const int u0 = bid * G::HROWS;                 // first h row of the block
        const bool shared = u0 < a.fs;
        const int f = shared ? a.fs : a.f;
        const int brow = shared ? u0 : (u0 - a.fs) % a.f;     // block's first row in its expert
        const int slot = shared ? -1 : (u0 - a.fs) / a.f;
        const int row0 = brow + wave * AP * G::RPW;       // wave's first row
        const BlobLayout Lf = BlobLayout::make(D, f);
        GateUpRegs<AP> R;
        const uint8_t* blob = nullptr;
        if (shared) {
            blob = a.ev.shared;
            gateup_issue<D, AP>(R, blob ? blob : a.ev.base, Lf, row0 + rsub);
        }
        int p0 = 0, p1 = n_tok;
        bool ok;
        WaveDigest W{};
        if (!shared) {
            // ---- level 1: routing merged per token row, sorted in registers
            int me;
            float mw;
            route_merge(rin, a.route_idx != nullptr, k, n_assign, &me, &mw);
            W = wave_digest(n_assign, me, a.E, sl[wave]);
            if (bid * G::HROWS == a.fs && wave == 0) {
                // the first routed block publishes the digest and the routing
                // used (read by K_B and the caller)
                const bool in = lane < n_assign;
                const bool bad = in && (me < 0 || me >= a.E);
                if (__ballot(bad) && lane == 0) set_err(a.err, ERR_BAD_INDEX);
                const int ep = (int)(W.sk >> 16);
                const int aid = (int)(W.sk & 0xFFFF);
                const bool valid = lane < W.n_valid;
                const float wsorted = __shfl(mw, valid ? aid : 0, 64);
                if (in) {
                    a.used_idx[lane] = bad ? -1 : me;
                    a.used_w[lane] = mw;
                    if (a.user_used_idx) a.user_used_idx[lane] = bad ? -1 : me;
                    if (a.user_used_w) a.user_used_w[lane] = mw;
                }
                if ((W.starts >> lane) & 1ull) {
                    const int ai = __popcll(W.starts & ((1ull << lane) - 1ull));
                    a.active[ai] = ep;
                    a.act_off[ai] = lane;
                }
                if (valid) { a.perm[lane] = aid; a.wsort[lane] = wsorted; }
                if (lane == 0) { a.meta[0] = W.n_active; a.meta[1] = W.n_valid; a.act_off[W.n_active] = W.n_valid; }
            }
            if (slot >= W.n_active) return;                   // uniform over the block
            p0 = nth_set(W.starts, slot);
            p1 = slot + 1 < W.n_active ? nth_set(W.starts, slot + 1) : W.n_valid;
            const int e = __builtin_amdgcn_readlane((int)(W.sk >> 16), p0);
            if (!a.ev.slot_of) blob = a.ev.base + (size_t)e * a.ev.blob;
            else {
                const int s = a.ev.slot_of[e];
                blob = (s < 0 || (a.ev.slot_tag && a.ev.slot_tag[s] != e)) ? nullptr : a.ev.base + (size_t)s * a.ev.blob;
            }
            gateup_issue<D, AP>(R, blob ? blob : a.ev.base, Lf, row0 + rsub);
            if (!blob && tid == 0) set_err(a.err, ERR_NOT_STAGED);
            ok = blob != nullptr;
        } else {
            ok = blob && !(a.ev.shared_tag && sh_tag != a.ev.E);
            if (!ok && blob && bid == 0 && tid == 0) set_err(a.err, ERR_NOT_STAGED);
        }
        if constexpr (FUSED) {
            const int t0 = shared ? p0 : (int)(__builtin_amdgcn_readlane((int)(W.sk & 0xFFFF), p0)) / k;
            x_poll<XB>(a, t0, e0, X.w, xo_x, fs);
        }
        // ---- level 2: per position, u of its token (whole block), then the rows
        int t_loaded = FUSED ? (shared ? p0 : (int)(__builtin_amdgcn_readlane((int)(W.sk & 0xFFFF), p0)) / k) : 0;
        for (int p = p0; p < p1; ++p) {
            const int t = shared ? p : (int)(__builtin_amdgcn_readlane((int)(W.sk & 0xFFFF), p)) / k;
            if (t != t_loaded) {
                if constexpr (FUSED) x_poll<XB>(a, t, e0, X.w, xo_x, fs);
                else x_issue<XB>(a, t, e0, X.w);
                t_loaded = t;
            }
            u_to_lds<D, XB>(a, X, S);
            float* h_out = shared ? a.hs + (size_t)t * f : a.h + (size_t)p * f;
            gateup_rows<D, FUSED, AP>(R, S, with_lo, ok, h_out, row0, a.xstride, ncopy);
            lds_barrier();                                    // u is rewritten for the next position
        }
        return;
    }

    if (bid >= a.nb_h + a.nb_head + a.nb_misc) {
        // the previous layer's head top-k, deferred to this launch (its logits
        // were written two launches ago; the prediction is for the next step)
        const auto& j = a.topk;
        topk_rows<kDeferMaxPer>(false, j.logits, j.En, j.kn, n_tok, j.bias, j.mc, j.hc, j.mp, j.hp, nullptr, j.kn,
                                j.pred_idx, j.pred_w);
        return;
    }
    // ---- bf16 rows accumulated in fp64: head rows, or LoRA A rows + shared gate
    const bool role_head = bid < a.nb_h + a.nb_head;
    const int row0 = (bid - (role_head ? a.nb_h : a.nb_h + a.nb_head)) * G::BROWS + wave * G::RPW;
    const int nrows = role_head ? a.En : (a.lora_a ? a.r : 0) + (a.sgate_w ? 1 : 0);
    if (nrows <= 0) return;                               // (a layer without a head)
    int row = row0 + rsub;
    const bool rvalid = row < nrows;
    row = rvalid ? row : nrows - 1;
    const uint16_t* wrow = role_head ? a.head + (size_t)row * D
                                     : ((a.lora_a && row < a.r) ? a.lora_a + (size_t)row * D : a.sgate_w);
    u32x4 wb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) wb[q] = __builtin_nontemporal_load((const u32x4*)(wrow + 32 * c) + q);
    if constexpr (FUSED) x_poll<XB>(a, 0, e0, X.w, xo_x, fs);
    for (int t = 0; t < n_tok; ++t) {
        if (t > 0) {
            if constexpr (FUSED) x_poll<XB>(a, t, e0, X.w, xo_x, fs);
            else x_issue<XB>(a, t, e0, X.w);
        }
        u_to_lds<D, XB>(a, X, S);
        double acc = 0.0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // elements 8q..8q+7 of the lane's chunk = uf pieces 2q, 2q+1
            const float4 u0 = *(const float4*)&S.uf[((2 * q) * G::C + c) * 4];
            const float4 u1 = *(const float4*)&S.uf[((2 * q + 1) * G::C + c) * 4];
            const float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
            u32x4 wv = wb[q];
            asm volatile("" : "+v"(wv));   // opaque copy: the widening stays in the token loop
            const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc += (double)bf16_to_f32(ws[j] & 0xFFFF) * (double)uu[2 * j];
                acc += (double)bf16_to_f32(ws[j] >> 16) * (double)uu[2 * j + 1];
            }
        }
        acc = group_sum_dpp<double, G::LPR>(acc);
        if (c == 0 && rvalid) {
            if constexpr (FUSED) {
                if (role_head) st_dev(a.logits_h + (size_t)t * a.En + row, acc);
                else if (a.lora_a && row < a.r) {
                    for (int cc = 0; cc < ncopy; ++cc) st_dev(a.au + cc * a.xstride + (size_t)t * a.r + row, (float)acc);
                } else {
                    const float sg = (float)(1.0 / (1.0 + exp(-acc)));
                    for (int cc = 0; cc < ncopy; ++cc) st_dev(a.sgate + cc * a.xstride + t, sg);
                }
            } else {
                if (role_head) a.logits_h[(size_t)t * a.En + row] = acc;
                else if (a.lora_a && row < a.r) a.au[(size_t)t * a.r + row] = (float)acc;
                else a.sgate[t] = (float)(1.0 / (1.0 + exp(-acc)));
            }
        }
        lds_barrier();
    }
}

}  // namespace moe

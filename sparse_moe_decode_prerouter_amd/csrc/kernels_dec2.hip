// Fused decode kernels: two launches per layer.
//   K_A: RMSNorm prologue + routing digest + int4 gate/up GEMV with SwiGLU
//        (routed experts and the shared expert) + prerouter head logits +
//        LoRA A u + shared-expert gate.
//   K_B: int4 down GEMV + routing-weighted combine + sigmoid-gated shared
//        expert + LoRA B + residual; one extra block takes the head's top-k.
//   K_R: self-routing (router GEMV + top-k) for rows with no prediction.
//
// Latency structure (batch-1 decode is bound by dependent round trips, not
// by bandwidth): every block issues all loads that do not depend on the
// routing at kernel start, resolves the routing with one wave, issues the
// routed expert loads, and only then computes. Block-wide barriers here wait
// for LDS traffic only (lds_barrier), so global loads stay in flight across
// them; HIP's __syncthreads would drain them.
// Decode sizes: n_tok <= 16 and n_tok * k <= 64.
#include "device_common.h"
#include "moe_internal.h"
#include "topk.h"

namespace moe {

constexpr int kMaxAssign = 64;          // n_tok * k on this path
constexpr int kInvalidExpert = 0xFFFF;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): this wave's LDS ops are done
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Token->expert digest built by wave 0: distinct experts ascending, where each
// expert's assignments start, and assignments sorted by (expert, id). Keys
// carry the assignment id, so they are unique and a key's rank is its slot.
struct Digest {
    int n_active, n_valid;
    int active[kMaxAssign + 1];
    int off[kMaxAssign + 1];
    int perm[kMaxAssign];
    int eidx[kMaxAssign];
    float ew[kMaxAssign];
    uint32_t sorted[kMaxAssign];
};

__device__ __forceinline__ bool row_given(const int32_t* route_idx, int t, int k) {
    return route_idx && route_idx[(size_t)t * k] >= 0;
}

// wave 0 only; `e`, `w` are this lane's merged routing entry (lane < n)
__device__ void wave_digest(Digest& D, int n, int e, float w, bool report, int32_t* err, int E) {
    const int lane = threadIdx.x & 63;
    const bool in = lane < n;
    const bool ok = in && e >= 0 && e < E;
    if (in && !ok && report) set_err(err, ERR_BAD_INDEX);
    const uint32_t key = in ? (((uint32_t)(ok ? e : kInvalidExpert) << 16) | (uint32_t)lane) : 0xFFFFFFFFu;
    if (in) { D.eidx[lane] = ok ? e : -1; D.ew[lane] = w; }
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += (uint32_t)__shfl((int)key, j, 64) < key;
    if (in) D.sorted[rank] = key;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const uint32_t sk = in ? D.sorted[lane] : 0xFFFFFFFFu;
    const int ep = (int)(sk >> 16);
    const bool valid = in && ep != kInvalidExpert;
    const int prev = __shfl_up(ep, 1, 64);
    const bool start = valid && (lane == 0 || prev != ep);
    const unsigned long long m = __ballot(start);
    const unsigned long long vm = __ballot(valid);
    if (start) {
        const int ai = __popcll(m & ((1ull << lane) - 1ull));
        D.active[ai] = ep;
        D.off[ai] = lane;
    }
    if (valid) D.perm[lane] = (int)(sk & 0xFFFFu);
    if (lane == 0) {
        const int na = __popcll(m), nv = __popcll(vm);
        D.n_active = na; D.n_valid = nv; D.off[na] = nv;
    }
}

// ---------------------------------------------------------------------------
// Block input u of one token, in parallel: thread g owns elements [8g, 8g+8).
// fp64 RMSNorm (sum of squares, shuffle + LDS reduction in a fixed order),
// one rounding to the activation dtype, then the GEMV-ordered bf16 pairs
// (4 dwords per 8 elements: (e_p, e_{p+4})) and per-32-chunk sums.
// ---------------------------------------------------------------------------
struct URegs {
    float x[8];
    float g[8];
};

__device__ __forceinline__ void u_load(const DecAArgs& a, int t, int grp, URegs& r) {
    const int d = a.d;
    if (grp * 8 >= d) return;
    if (a.x_is_bf16) {
        const u32x4 v = *(const u32x4*)((const uint16_t*)a.x + (size_t)t * d + grp * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { r.x[2 * i] = bf16_to_f32(w[i] & 0xFFFF); r.x[2 * i + 1] = bf16_to_f32(w[i] >> 16); }
    } else {
        const float4 v0 = *(const float4*)((const float*)a.x + (size_t)t * d + grp * 8);
        const float4 v1 = *(const float4*)((const float*)a.x + (size_t)t * d + grp * 8 + 4);
        r.x[0] = v0.x; r.x[1] = v0.y; r.x[2] = v0.z; r.x[3] = v0.w;
        r.x[4] = v1.x; r.x[5] = v1.y; r.x[6] = v1.z; r.x[7] = v1.w;
    }
    if (a.fused) {
        const float4 g0 = *(const float4*)(a.gamma + grp * 8);
        const float4 g1 = *(const float4*)(a.gamma + grp * 8 + 4);
        r.g[0] = g0.x; r.g[1] = g0.y; r.g[2] = g0.z; r.g[3] = g0.w;
        r.g[4] = g1.x; r.g[5] = g1.y; r.g[6] = g1.z; r.g[7] = g1.w;
    }
}

// d <= 8 * kThreads (2048): one group per thread
__device__ void u_finish(const DecAArgs& a, int grp, const URegs& r, float* su, uint32_t* upk, uint32_t* upk_lo,
                         float* usum, float* usum_lo, double* red) {
    const int d = a.d, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool mine = grp * 8 < d;
    double inv = 1.0;
    if (a.fused) {
        double ss = 0.0;
        if (mine) {
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += (double)r.x[i] * (double)r.x[i];
        }
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
        if (lane == 0) red[wave] = ss;
        lds_barrier();
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tot += red[w];
        inv = 1.0 / sqrt(tot / (double)d + (double)a.eps);
    }
    float uf[8];
    uint32_t hb[8];
    if (mine) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double uv = a.fused ? ((double)r.x[i] * inv) * (double)r.g[i] : (double)r.x[i];
            if (a.act_bf16) { hb[i] = f64_to_bf16(uv); uf[i] = bf16_to_f32(hb[i]); }
            else { uf[i] = (float)uv; hb[i] = f32_to_bf16(uf[i]); }
        }
        if (su) {
            *(float4*)(su + grp * 8) = make_float4(uf[0], uf[1], uf[2], uf[3]);
            *(float4*)(su + grp * 8 + 4) = make_float4(uf[4], uf[5], uf[6], uf[7]);
        }
    }
    if (upk) {
        float sh = 0.f, sl = 0.f;
        if (mine) {
            u32x4 pk;
            pk.x = hb[0] | (hb[4] << 16); pk.y = hb[1] | (hb[5] << 16);
            pk.z = hb[2] | (hb[6] << 16); pk.w = hb[3] | (hb[7] << 16);
            *(u32x4*)(upk + grp * 4) = pk;
#pragma unroll
            for (int i = 0; i < 8; ++i) sh += bf16_to_f32(hb[i]);
            if (upk_lo) {
                uint32_t lb[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) { lb[i] = f32_to_bf16(uf[i] - bf16_to_f32(hb[i])); sl += bf16_to_f32(lb[i]); }
                u32x4 pl;
                pl.x = lb[0] | (lb[4] << 16); pl.y = lb[1] | (lb[5] << 16);
                pl.z = lb[2] | (lb[6] << 16); pl.w = lb[3] | (lb[7] << 16);
                *(u32x4*)(upk_lo + grp * 4) = pl;
            }
        }
        // chunk of 32 = 4 consecutive groups = 4 consecutive lanes
        sh += __shfl_xor(sh, 1, 64); sh += __shfl_xor(sh, 2, 64);
        sl += __shfl_xor(sl, 1, 64); sl += __shfl_xor(sl, 2, 64);
        if (mine && (grp & 3) == 0) {
            usum[grp >> 2] = sh;
            if (usum_lo) usum_lo[grp >> 2] = sl;
        }
    }
    lds_barrier();
}

// sum over one 32-element chunk of (128 + q) * u, u in GEMV-ordered pairs
__device__ __forceinline__ float chunk_dot_lds(const u32x4 w, const uint32_t* up, float acc) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4 uv = *(const u32x4*)(up + 4 * i);
        acc = dot2_bf16(nib_pair_bf16(ws[i], 0), uv.x, acc);
        acc = dot2_bf16(nib_pair_bf16(ws[i], 1), uv.y, acc);
        acc = dot2_bf16(nib_pair_bf16(ws[i], 2), uv.z, acc);
        acc = dot2_bf16(nib_pair_bf16(ws[i], 3), uv.w, acc);
    }
    return acc;
}

// bf16 row (d elements) dot fp32 u in LDS, fp64 accumulation; lane covers
// elements lane*8 + 512*m
template <int NLD>
__device__ __forceinline__ double bf16_row_dot(const u32x4 (&wr)[NLD], const float* su, int d, bool valid) {
    const int lane = threadIdx.x & 63;
    double acc = 0.0;
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
        const int j = lane * 8 + 512 * m;
        if (valid && j < d) {
            const float4 u0 = *(const float4*)(su + j);
            const float4 u1 = *(const float4*)(su + j + 4);
            const float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
            const uint32_t ws[4] = {wr[m].x, wr[m].y, wr[m].z, wr[m].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc += (double)bf16_to_f32(ws[q] & 0xFFFF) * (double)uu[2 * q];
                acc += (double)bf16_to_f32(ws[q] >> 16) * (double)uu[2 * q + 1];
            }
        }
    }
    return group_sum(acc, 64);
}

template <int NLD>
__device__ __forceinline__ void bf16_row_load(u32x4 (&wr)[NLD], const uint16_t* w, int d, bool valid) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
        const int j = lane * 8 + 512 * m;
        if (valid && j < d) wr[m] = __builtin_nontemporal_load((const u32x4*)(w + j));
    }
}

constexpr int kHRowsPerBlock = 8;     // h rows (gate row + up row) per K_A block: 2 per wave
constexpr int kHeadRowsPerBlock = 4;  // bf16 rows per K_A block: 1 per wave

// K_A (d <= 2048: one 16-byte chunk per lane and weight row)
__global__ void __launch_bounds__(kThreads) k_dec_a(DecAArgs a) {
    constexpr int kNld = 4;
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ Digest D;
    __shared__ double red[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d = a.d;
    const int n_assign = a.n_tok * a.k;
    const bool role_h = (int)blockIdx.x < a.nb_h;
    const bool role_head = !role_h && (int)blockIdx.x < a.nb_h + a.nb_head;

    // ---- level 0: loads that need no routing. The routing loads go first:
    // the memory counter is in order, so waiting for them must not also wait
    // for the activation and weight loads issued after them.
    int me = -1; float mw = 0.f;
    if (role_h && wave == 0) {
        int vr = -1, vs = -1;
        float vrw = 0.f, vsw = 0.f;
        if (lane < n_assign) {
            if (a.route_idx) { vr = a.route_idx[lane]; vrw = a.route_w[lane]; }
            if (a.self_idx) { vs = a.self_idx[lane]; vsw = a.self_w[lane]; }
        }
        const int first = __shfl(vr, (lane / a.k) * a.k, 64);   // first entry of this lane's row
        const bool given = a.route_idx && first >= 0;
        me = given ? vr : vs;
        mw = given ? vrw : vsw;
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    URegs ur;
    u_load(a, 0, tid, ur);

    if (role_h) {
        const int u0 = blockIdx.x * kHRowsPerBlock;
        const bool shared = u0 < a.fs;
        const int f = shared ? a.fs : a.f;
        const int row0 = shared ? u0 : (u0 - a.fs) % a.f;
        const int slot = shared ? -1 : (u0 - a.fs) / a.f;
        const BlobLayout L = BlobLayout::make(d, f);
        const int LPR = d / 32;                     // lanes per row (<= 64)
        const int RPW = 64 / LPR;                   // rows per wave-load
        const int hw = kHRowsPerBlock / kWaves;     // h rows per wave (2)
        const int rsub = lane / LPR, c0 = lane % LPR;
        u32x4 wg[2], wu[2];
        uint32_t sg[2], su[2];
        bool rv[2];
        int rrow[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int hr = q * RPW + rsub;
            rrow[q] = row0 + wave * hw + hr;
            rv[q] = hr < hw && (q == 0 || RPW < hw) && rrow[q] < f;
        }
        const uint8_t* blob = nullptr;
        auto issue = [&]() {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if (rv[q] && blob) {
                    const size_t row = rrow[q];
                    wg[q] = __builtin_nontemporal_load((const u32x4*)(blob + L.gate_q + row * (d / 2) + c0 * 16));
                    wu[q] = __builtin_nontemporal_load((const u32x4*)(blob + L.up_q + row * (d / 2) + c0 * 16));
                    sg[q] = __builtin_nontemporal_load((const uint32_t*)(blob + L.gate_sb + (row * (d / 64) + c0 / 2) * 4));
                    su[q] = __builtin_nontemporal_load((const uint32_t*)(blob + L.up_sb + (row * (d / 64) + c0 / 2) * 4));
                }
            }
        };
        if (shared) {
            blob = a.ev.shared;
            if (blob && a.ev.shared_tag && *a.ev.shared_tag != a.ev.E) {
                if (tid == 0) set_err(a.err, ERR_NOT_STAGED);
                blob = nullptr;
            }
            issue();
        }
        // ---- level 1: routing digest (wave 0), then the routed expert's rows
        if (wave == 0 && (!shared || blockIdx.x == 0)) wave_digest(D, n_assign, me, mw, blockIdx.x == 0, a.err, a.E);
        lds_barrier();
        int pos0 = 0, pos1 = a.n_tok;
        if (!shared) {
            if (slot >= D.n_active) return;
            const int e = D.active[slot];
            pos0 = D.off[slot]; pos1 = D.off[slot + 1];
            if (!a.ev.slot_of) blob = a.ev.base + (size_t)e * a.ev.blob;
            else {
                const int s = a.ev.slot_of[e];
                if (s < 0 || (a.ev.slot_tag && a.ev.slot_tag[s] != e)) {
                    if (tid == 0) set_err(a.err, ERR_NOT_STAGED);
                    blob = nullptr;
                } else blob = a.ev.base + (size_t)s * a.ev.blob;
            }
            issue();
        }
        if (blockIdx.x == 0) {
            for (int i = tid; i < n_assign; i += kThreads) {
                a.used_idx[i] = D.eidx[i];
                a.used_w[i] = D.ew[i];
                if (a.user_used_idx) a.user_used_idx[i] = D.eidx[i];
                if (a.user_used_w) a.user_used_w[i] = D.ew[i];
            }
            for (int i = tid; i < D.n_active; i += kThreads) { a.active[i] = D.active[i]; a.act_off[i] = D.off[i]; }
            for (int i = tid; i < D.n_valid; i += kThreads) { a.perm[i] = D.perm[i]; a.wsort[i] = D.ew[D.perm[i]]; }
            if (tid == 0) { a.meta[0] = D.n_active; a.meta[1] = D.n_valid; a.act_off[D.n_active] = D.n_valid; }
        }
        // ---- activations and dot products
        uint32_t* upk = (uint32_t*)lds;                                     // [d/2]
        uint32_t* upk_lo = a.act_bf16 ? nullptr : upk + d / 2;              // [d/2]
        float* us = (float*)(lds + (a.act_bf16 ? (size_t)d * 2 : (size_t)d * 4));   // [d/32]
        float* us_lo = a.act_bf16 ? nullptr : us + d / 32;
        int t_loaded = 0;
        for (int pi = pos0; pi < pos1; ++pi) {
            const int t = shared ? pi : D.perm[pi] / a.k;
            if (t != t_loaded) { u_load(a, t, tid, ur); t_loaded = t; }
            u_finish(a, tid, ur, nullptr, upk, upk_lo, us, us_lo, red);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float ga = 0.f, ua = 0.f;
                if (rv[q] && blob) {
                    float accg = chunk_dot_lds(wg[q], upk + c0 * 16, 0.f);
                    float accu = chunk_dot_lds(wu[q], upk + c0 * 16, 0.f);
                    float usm = us[c0];
                    if (upk_lo) {
                        accg = chunk_dot_lds(wg[q], upk_lo + c0 * 16, accg);
                        accu = chunk_dot_lds(wu[q], upk_lo + c0 * 16, accu);
                        usm += us_lo[c0];
                    }
                    const float s1 = f16_to_f32(sg[q] & 0xFFFF), b1 = f16_to_f32(sg[q] >> 16);
                    const float s2 = f16_to_f32(su[q] & 0xFFFF), b2 = f16_to_f32(su[q] >> 16);
                    ga = s1 * accg + (b1 - 128.f * s1) * usm;
                    ua = s2 * accu + (b2 - 128.f * s2) * usm;
                }
                ga = group_sum(ga, LPR);
                ua = group_sum(ua, LPR);
                if (rv[q] && c0 == 0) {
                    const float hv = blob ? silu_f32(ga) * ua : 0.f;
                    if (shared) a.hs[(size_t)t * f + rrow[q]] = hv;
                    else a.h[(size_t)pi * f + rrow[q]] = hv;
                }
            }
            lds_barrier();   // LDS u is rewritten for the next token
        }
        return;
    }

    // ---- bf16 rows accumulated in fp64: head rows, or LoRA A rows + shared gate
    int row0, nrows;
    if (role_head) { row0 = (blockIdx.x - a.nb_h) * kHeadRowsPerBlock; nrows = a.En; }
    else {
        row0 = (blockIdx.x - a.nb_h - a.nb_head) * kHeadRowsPerBlock;
        nrows = (a.lora_a ? a.r : 0) + (a.sgate_w ? 1 : 0);
    }
    const int row = row0 + wave;
    const bool valid = row < nrows;
    const uint16_t* w = nullptr;
    if (valid) {
        if (role_head) w = a.head + (size_t)row * d;
        else w = (a.lora_a && row < a.r) ? a.lora_a + (size_t)row * d : a.sgate_w;
    }
    u32x4 wr[kNld];
    bf16_row_load<kNld>(wr, w, d, valid);
    float* suf = (float*)lds;
    for (int t = 0; t < a.n_tok; ++t) {
        if (t > 0) u_load(a, t, tid, ur);
        u_finish(a, tid, ur, suf, nullptr, nullptr, nullptr, nullptr, red);
        const double acc = bf16_row_dot<kNld>(wr, suf, d, valid);
        if (valid && lane == 0) {
            if (role_head) a.logits_h[(size_t)t * a.En + row] = acc;
            else if (a.lora_a && row < a.r) a.au[(size_t)t * a.r + row] = (float)acc;
            else a.sgate[t] = (float)(1.0 / (1.0 + exp(-acc)));
        }
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// K_R: self-routing for rows with no prediction: RMSNorm prologue + router
// GEMV (bf16 x fp32 products, fp64 accumulation) + top-k in the last block.
// Logits are published with device-scope stores and counted with a relaxed
// atomic, so the last block reads them coherently without cache flushes.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) k_dec_r(DecAArgs a, RouteArgs r) {
    constexpr int kNld = 4;
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ double red[kWaves];
    __shared__ int is_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d = a.d;
    float* suf = (float*)lds;
    const int row = blockIdx.x * kHeadRowsPerBlock + wave;
    const bool valid = row < r.E;
    u32x4 wr[kNld];
    bf16_row_load<kNld>(wr, valid ? r.router + (size_t)row * d : nullptr, d, valid);
    URegs ur;
    for (int t = 0; t < a.n_tok; ++t) {
        if (row_given(r.route_idx, t, r.k)) continue;      // uniform across the block
        u_load(a, t, tid, ur);
        u_finish(a, tid, ur, suf, nullptr, nullptr, nullptr, nullptr, red);
        const double acc = bf16_row_dot<kNld>(wr, suf, d, valid);
        if (valid && lane == 0) st_dev(r.logits_r + (size_t)t * r.E + row, acc);
        lds_barrier();
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const unsigned old = __hip_atomic_fetch_add(r.counters + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = old == gridDim.x - 1;
        if (is_last) __hip_atomic_store(r.counters + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!is_last) return;
    topk_rows(true, r.logits_r, r.E, r.k, a.n_tok, r.router_bias, nullptr, nullptr, nullptr, nullptr,
              r.route_idx, r.k, r.self_idx, r.self_w);
}

hipError_t launch_dec_r(const DecAArgs& a, const RouteArgs& r, hipStream_t s) {
    if (a.d > 2048) return hipErrorInvalidValue;
    const int nb = (r.E + kHeadRowsPerBlock - 1) / kHeadRowsPerBlock;
    hipLaunchKernelGGL(k_dec_r, dim3(nb), dim3(kThreads), (size_t)a.d * 4, s, a, r);
    return hipGetLastError();
}

int dec_a_blocks(int d, int f, int fs, int n_tok, int k, int E, int En, int r, bool sgate, int* nb_h, int* nb_head,
                 int* nb_misc) {
    const int max_active = n_tok * k < E ? n_tok * k : E;
    *nb_h = (fs + max_active * f + kHRowsPerBlock - 1) / kHRowsPerBlock;
    *nb_head = (En + kHeadRowsPerBlock - 1) / kHeadRowsPerBlock;
    *nb_misc = (r + (sgate ? 1 : 0) + kHeadRowsPerBlock - 1) / kHeadRowsPerBlock;
    (void)d;
    return *nb_h + *nb_head + *nb_misc;
}

hipError_t launch_dec_a(const DecAArgs& a, hipStream_t s) {
    if (a.d > 2048 || a.n_tok * a.k > kMaxAssign) return hipErrorInvalidValue;
    const size_t d = a.d;
    const size_t lds_h = (a.act_bf16 ? d * 2 : d * 4) + (a.act_bf16 ? d / 32 * 4 : d / 16 * 4);
    const size_t lds = lds_h > d * 4 ? lds_h : d * 4;
    const int nb = a.nb_h + a.nb_head + a.nb_misc;
    hipLaunchKernelGGL(k_dec_a, dim3(nb), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K_B: each block owns 4 output rows. Slot s (shared expert first, then the
// active experts ascending) is handled by wave s % 4, which computes Wd h for
// the block's 4 rows and every token of the slot into an LDS partial; the
// partials are then summed per (token, row) in slot order (fixed order, so
// results are identical run to run) with LoRA B and the residual.
// ---------------------------------------------------------------------------
constexpr int kRowsB = 4;
constexpr int kMaxSlotsB = kMaxAssign + 1;
constexpr int kMaxTokB = 16;

struct BSlots {
    int n_active, nslots;
    int active[kMaxAssign + 1];
    int off[kMaxAssign + 1];
    int perm[kMaxAssign];
    float w[kMaxAssign];
};

// f <= 2048: one 16-byte chunk per lane and Wd row
__global__ void __launch_bounds__(kThreads) k_dec_b(DecBArgs a) {
    __shared__ BSlots S;
    __shared__ float part[kMaxSlotsB * kMaxTokB * kRowsB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if ((int)blockIdx.x == a.nb_rows) {
        if (a.pred_idx)
            topk_rows(false, a.logits_h, a.En, a.kn, a.n_tok, a.head_bias, a.hist_cur_m, a.hist_cur, a.hist_prev_m,
                      a.hist_prev, nullptr, a.kn, a.pred_idx, a.pred_w);
        return;
    }
    const int d = a.d, f = a.f, n_tok = a.n_tok;
    const int n_assign = n_tok * a.k;
    const int row_base = blockIdx.x * kRowsB;
    const int has_shared = a.fs ? 1 : 0;
    const BlobLayout L = BlobLayout::make(d, f);
    const int LPR = f / 32;                       // lanes per Wd row (<= 64)
    const int g = lane / LPR, c0 = lane % LPR;

    // ---- level 0: routing digest from K_A (no dependent loads), epilogue
    // operands, the shared expert's rows and hidden state
    int v_meta = 0, v_act = 0, v_off = 0, v_perm = 0;
    float v_w = 0.f;
    const int nas = n_assign < a.ev.E ? n_assign : a.ev.E;   // entries of active/act_off in use
    if (wave == 0) {
        v_meta = a.meta[0];
        if (lane <= nas) { v_act = a.active[lane < nas ? lane : 0]; v_off = a.act_off[lane]; }
        if (lane < n_assign) { v_perm = a.perm[lane]; v_w = a.wsort[lane]; }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int et = tid / kRowsB, er = tid % kRowsB, erow = row_base + er;
    const bool ep_on = et < n_tok && erow < d;
    float ep_x = 0.f, ep_l = 0.f;
    if (ep_on) {
        if (a.fused) ep_x = a.x[(size_t)et * d + erow];
        if (a.lora_b && a.r) {
            float l = 0.f;
            for (int q = 0; q < a.r; ++q) l += bf16_to_f32(a.lora_b[(size_t)erow * a.r + q]) * a.au[(size_t)et * a.r + q];
            ep_l = a.lora_scale * l;
        }
    }
    const int grow = row_base + g;                // each LPR-lane group owns one of the 4 rows
    const bool rvalid = g < kRowsB && grow < d;
    const uint8_t* sh_blob = nullptr;
    if (has_shared) {
        sh_blob = a.ev.shared;
        if (sh_blob && a.ev.shared_tag && *a.ev.shared_tag != a.ev.E) sh_blob = nullptr;
    }
    struct SlotPrep {
        int s, p0, p1;
        bool on, sh, hpre;
        const uint8_t* blob;
        u32x4 wd;
        uint32_t sbv;
        float4 hv[8];
    };
    auto load_rows = [&](SlotPrep& P) {
        if (rvalid && P.blob) {
            P.wd = __builtin_nontemporal_load((const u32x4*)(P.blob + L.down_q + (size_t)grow * (f / 2) + c0 * 16));
            P.sbv = __builtin_nontemporal_load((const uint32_t*)(P.blob + L.down_sb + ((size_t)grow * (f / 64) + c0 / 2) * 4));
        }
        P.hpre = P.p1 - P.p0 == 1;
        if (P.hpre && rvalid && P.blob) {
            const float* hrow = P.sh ? a.hs + (size_t)P.p0 * f : a.h + (size_t)P.p0 * f;
#pragma unroll
            for (int i = 0; i < 8; ++i) P.hv[i] = *(const float4*)(hrow + 32 * c0 + 4 * i);
        }
    };
    SlotPrep shp{};
    shp.on = has_shared && wave == 0;
    if (shp.on) {
        shp.s = 0; shp.p0 = 0; shp.p1 = n_tok; shp.sh = true; shp.blob = sh_blob;
        load_rows(shp);
    }
    if (wave == 0) {
        if (lane <= nas) { S.active[lane] = v_act; S.off[lane] = v_off; }
        // entries at or beyond n_valid were not written by K_A (invalid routing
        // indices): keep any index read from them inside [0, n_assign)
        if (lane < n_assign) {
            S.perm[lane] = v_perm < 0 ? 0 : (v_perm >= n_assign ? n_assign - 1 : v_perm);
            S.w[lane] = v_w;
        }
        if (lane == 0) { S.n_active = v_meta; S.nslots = v_meta + has_shared; }
    }
    lds_barrier();
    const int nslots = S.nslots;
    auto resolve = [&](SlotPrep& P, int s) {
        P.s = s;
        P.on = s < nslots;
        P.sh = false;
        if (!P.on) return;
        const int ai = s - has_shared;
        const int e = S.active[ai];
        P.p0 = S.off[ai]; P.p1 = S.off[ai + 1];
        if (!a.ev.slot_of) P.blob = a.ev.base + (size_t)e * a.ev.blob;
        else {
            const int sl = a.ev.slot_of[e];
            P.blob = (sl < 0 || (a.ev.slot_tag && a.ev.slot_tag[sl] != e)) ? nullptr : a.ev.base + (size_t)sl * a.ev.blob;
        }
        load_rows(P);
    };
    auto compute = [&](SlotPrep& P) {
        if (!P.on) return;
        if (lane < n_tok * kRowsB) part[(P.s * kMaxTokB + lane / kRowsB) * kRowsB + lane % kRowsB] = 0.f;
        for (int p = P.p0; p < P.p1; ++p) {
            int t; float wgt;
            if (P.sh) { t = p; wgt = a.sgate ? a.sgate[t] : 1.f; }
            else { t = S.perm[p] / a.k; wgt = S.w[p]; }
            float o = 0.f;
            if (rvalid && P.blob) {
                float4 hv4[8];
                if (P.hpre) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) hv4[i] = P.hv[i];
                } else {
                    const float* hrow = P.sh ? a.hs + (size_t)p * f : a.h + (size_t)p * f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) hv4[i] = *(const float4*)(hrow + 32 * c0 + 4 * i);
                }
                const uint32_t ws[4] = {P.wd.x, P.wd.y, P.wd.z, P.wd.w};
                float accq = 0.f, hsum = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float hv[8] = {hv4[2 * i].x, hv4[2 * i].y, hv4[2 * i].z, hv4[2 * i].w,
                                         hv4[2 * i + 1].x, hv4[2 * i + 1].y, hv4[2 * i + 1].z, hv4[2 * i + 1].w};
#pragma unroll
                    for (int n = 0; n < 8; ++n) {
                        accq += (float)((ws[i] >> (4 * n)) & 0xFu) * hv[n];
                        hsum += hv[n];
                    }
                }
                o = f16_to_f32(P.sbv & 0xFFFF) * accq + f16_to_f32(P.sbv >> 16) * hsum;
            }
            o = group_sum(o, LPR);
            if (g < kRowsB && c0 == 0 && P.blob) part[(P.s * kMaxTokB + t) * kRowsB + g] = wgt * o;
        }
    };
    // ---- level 1: each wave's slots, two at a time with all their loads in flight
    // (slot 0 is the shared expert when present; it was prepared at level 0)
    for (int s0 = wave; s0 < nslots; s0 += 2 * kWaves) {
        SlotPrep A{}, Bp{};
        if (has_shared && s0 == 0) A = shp;
        else resolve(A, s0);
        resolve(Bp, s0 + kWaves);
        compute(A);
        compute(Bp);
    }
    lds_barrier();
    if (ep_on) {
        float y = 0.f;
        for (int s = 0; s < nslots; ++s) y += part[(s * kMaxTokB + et) * kRowsB + er];
        y += ep_l;
        if (a.fused) y = ep_x + y;
        a.y[(size_t)et * d + erow] = y;
    }
}

hipError_t launch_dec_b(const DecBArgs& a, hipStream_t s) {
    if (a.n_tok > kMaxTokB || a.n_tok * a.k > kMaxAssign || a.f > 512) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_dec_b, dim3(a.nb_rows + 1), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe

namespace moe {
int dec_b_row_blocks(int d) { return (d + kRowsB - 1) / kRowsB; }

bool dec_fast_path_ok(int d, int f, int n_tok, int k) {
    const bool dpow = d >= 256 && d <= 2048 && (d & (d - 1)) == 0;
    const bool fpow = f >= 64 && f <= 512 && (f & (f - 1)) == 0;
    return dpow && fpow && n_tok <= kMaxTokB && n_tok * k <= kMaxAssign;
}
}  // namespace moe

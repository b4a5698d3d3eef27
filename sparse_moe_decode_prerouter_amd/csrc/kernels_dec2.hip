// Fused decode kernels, two launches per layer (K_A is in kernels_deca.hip):
//   K_B: int4 down GEMV + routing-weighted combine + sigmoid-gated shared
//        expert + LoRA B + residual; block 0 takes the head's top-k.
//   K_R: self-routing (router GEMV + top-k) for rows with no prediction.
//
// Latency structure (batch-1 decode is bound by dependent round trips, not
// by bandwidth): loads that do not depend on the routing are issued at
// kernel start, the routing digest is read, the routed expert rows are
// issued, and only then is anything computed. Block-wide barriers here wait
// for LDS traffic only (lds_barrier), so global loads stay in flight across
// them; HIP's __syncthreads would drain them.
// Decode sizes: n_tok <= 16 and n_tok * k <= 64.
#include "device_common.h"
#include "moe_internal.h"
#include "topk.h"
#include "dec_common.h"

namespace moe {



__device__ __forceinline__ bool row_given(const int32_t* route_idx, int t, int k) {
    return route_idx && route_idx[(size_t)t * k] >= 0;
}

// ---------------------------------------------------------------------------
// Block input u of one token, in parallel: thread g owns elements [8g, 8g+8).
// fp64 RMSNorm (sum of squares, shuffle + LDS reduction in a fixed order),
// one rounding to the activation dtype, then the GEMV-ordered bf16 pairs
// (4 dwords per 8 elements: (e_p, e_{p+4})) and per-32-chunk sums.
// ---------------------------------------------------------------------------
struct URegs {
    uint32_t x[8];    // raw words: 8 fp32, or 4 bf16 pairs (converted in u_finish)
    float g[8];
};

__device__ __forceinline__ void u_load(const DecAArgs& a, int t, int grp, URegs& r) {
    const int d = a.d;
    if (grp * 8 >= d) return;
    if (a.x_is_bf16) {
        const u32x4 v = *(const u32x4*)((const uint16_t*)a.x + (size_t)t * d + grp * 8);
        r.x[0] = v.x; r.x[1] = v.y; r.x[2] = v.z; r.x[3] = v.w;
    } else {
        const u32x4 v0 = *(const u32x4*)((const float*)a.x + (size_t)t * d + grp * 8);
        const u32x4 v1 = *(const u32x4*)((const float*)a.x + (size_t)t * d + grp * 8 + 4);
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

__device__ __forceinline__ void u_values(const DecAArgs& a, const URegs& r, float (&xv)[8]) {
    if (a.x_is_bf16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { xv[2 * i] = bf16_to_f32(r.x[i] & 0xFFFF); xv[2 * i + 1] = bf16_to_f32(r.x[i] >> 16); }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[i] = __uint_as_float(r.x[i]);
    }
}

// d <= 8 * kThreads (2048): one group per thread
__device__ void u_finish(const DecAArgs& a, int grp, const URegs& r, float* su, uint32_t* upk, uint32_t* upk_lo,
                         float* usum, float* usum_lo, double* red) {
    const int d = a.d, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool mine = grp * 8 < d;
    float xv[8];
    u_values(a, r, xv);
    double inv = 1.0;
    if (a.fused) {
        double ss = 0.0;
        if (mine) {
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += (double)xv[i] * (double)xv[i];
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
            const double uv = a.fused ? ((double)xv[i] * inv) * (double)r.g[i] : (double)xv[i];
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

constexpr int kHeadRowsPerBlock = 4;  // router rows per K_R block: 1 per wave

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

hipError_t launch_dec_r(const DecAArgs& a, const RouteArgs& r, hipStream_t s, const KTime* tm) {
    if (a.d > 2048) return hipErrorInvalidValue;
    const int nb = (r.E + kHeadRowsPerBlock - 1) / kHeadRowsPerBlock;
    MOE_LAUNCH(k_dec_r, dim3(nb), dim3(kThreads), (size_t)a.d * 4, s, tm, a, r);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K_B: int4 down GEMV + combine. Block 0 takes the head's top-k (it is
// dispatched first, so it overlaps the rest); every other block owns RB
// consecutive output rows.
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
// ---------------------------------------------------------------------------
constexpr int kPassB = 4;
constexpr int kMaxTokB = 16;

template <int F>
struct BGeo {
    static constexpr int LPR = F / 8;
    static constexpr int RPP = 64 / LPR;
    static constexpr int RB = kPassB * RPP;
};

// LoRA B row (r bf16) . LoRA A output row (r fp32): the loads are issued
// together up front and the products summed later, in q order.
constexpr int kLoraChunks = 2;                // r <= 16, r % 8 == 0
struct LoraRegs {
    u32x4 b[kLoraChunks];
    float4 u[2 * kLoraChunks];
};
__device__ __forceinline__ void lora_issue(LoraRegs& R, const uint16_t* brow, const float* urow, int r) {
#pragma unroll
    for (int c = 0; c < kLoraChunks; ++c) {
        const int cc = 8 * c < r ? c : 0;
        R.b[c] = *(const u32x4*)(brow + 8 * cc);
        R.u[2 * c] = *(const float4*)(urow + 8 * cc);
        R.u[2 * c + 1] = *(const float4*)(urow + 8 * cc + 4);
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

__device__ __forceinline__ void h_issue(float4 (&hv)[2], const float* hrow, int c) {
    hv[0] = *(const float4*)(hrow + 8 * c);
    hv[1] = *(const float4*)(hrow + 8 * c + 4);
}

// Per-lane partial of each pass: sum_j (s q_j + b) h_j over the lane's 8 elements.
template <int NP>
__device__ __forceinline__ void down_partial(const DownRegs<NP>& R, const float4 (&hv)[2], float (&o)[NP]) {
    const float h[8] = {hv[0].x, hv[0].y, hv[0].z, hv[0].w, hv[1].x, hv[1].y, hv[1].z, hv[1].w};
    float hs = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) hs += h[j];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += (float)((R.q[i] >> (4 * j)) & 0xFu) * h[j];
        o[i] = f16_to_f32(R.sb[i] & 0xFFFF) * acc + f16_to_f32(R.sb[i] >> 16) * hs;
    }
}

template <int F>
__global__ void __launch_bounds__(kThreads, 2) k_dec_b(DecBArgs a) {
    using G = BGeo<F>;
    constexpr int NPS = kPassB / kWaves;           // shared-expert passes per wave
    __shared__ float part[(kMaxAssign + kMaxTokB) * G::RB];
    __shared__ uint32_t sl[kWaves][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (blockIdx.x == 0) {
        if (a.pred_idx)
            topk_rows(false, a.logits_h, a.En, a.kn, a.n_tok, a.head_bias, a.hist_cur_m, a.hist_cur, a.hist_prev_m,
                      a.hist_prev, nullptr, a.kn, a.pred_idx, a.pred_w);
        return;
    }
    const int d = a.d, n_tok = a.n_tok, k = a.k;
    const int n_assign = n_tok * k;
    const int row0 = (blockIdx.x - 1) * G::RB;
    const bool has_shared = a.fs != 0;
    const BlobLayout L = BlobLayout::make(d, F);
    const int c = lane % G::LPR, rsub = lane / G::LPR;

    // ---- level 0, identical in every wave. The routing entries go first
    // (K_A read them on every XCD, so they are L2 hits); all other loads need
    // no routing and are issued unconditionally (clamped indices, stand-in
    // pointers), so waiting for the routing never waits for them.
    const RouteIn rin = route_load(a.route_idx, a.route_w, a.self_idx, a.self_w, n_assign);
    const float v_sg = (a.sgate ? a.sgate : (const float*)a.err)[lane < n_tok ? lane : 0];
    // epilogue operands: thread -> (token, row)
    const int ep_n = n_tok * G::RB;
    const int ep_q = tid < ep_n ? tid : 0;
    const int et = ep_q / G::RB, er = ep_q % G::RB;
    const float ep_x = a.fused ? a.x[(size_t)et * d + row0 + er] : 0.f;
    const bool lora_on = a.lora_b && a.r;
    const bool lora_vec = lora_on && (a.r & 7) == 0 && a.r <= 8 * kLoraChunks;
    LoraRegs lr;
    if (lora_vec) lora_issue(lr, a.lora_b + (size_t)(row0 + er) * a.r, a.au + (size_t)et * a.r, a.r);
    // shared expert: passes [NPS*wave, NPS*wave + NPS), token 0's hidden state
    const uint8_t* sh_blob = has_shared && a.ev.shared ? a.ev.shared : a.ev.base;
    DownRegs<NPS> shr;
    down_issue<F, NPS, G::RPP>(shr, sh_blob, L, row0 + NPS * wave * G::RPP + rsub);
    const int sh_tag = *(a.ev.shared_tag ? a.ev.shared_tag : a.err);
    const bool sh_ok = has_shared && a.ev.shared && (!a.ev.shared_tag || sh_tag == a.ev.E);
    float4 shh[2];
    h_issue(shh, has_shared ? a.hs : a.h, c);
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
    auto slot_compute = [&](const DownRegs<kPassB>& R, const uint8_t* blob, int s, const float4 (&h0)[2]) {
        const int p0 = nth_set(W.starts, s);
        const int p1 = s + 1 < n_active ? nth_set(W.starts, s + 1) : n_valid;
        for (int p = p0; p < p1; ++p) {
            float4 hv[2];
            if (p == p0) { hv[0] = h0[0]; hv[1] = h0[1]; }
            else h_issue(hv, a.h + (size_t)p * F, c);
            float o[kPassB];
            down_partial<kPassB>(R, hv, o);
            int pass;
            const float tot = row_reduce<float, kPassB, G::LPR>(o, &pass);
            const int aid = __builtin_amdgcn_readlane((int)(W.sk & 0xFFFF), p);
            const float wgt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mw), aid < n_assign ? aid : 0));
            if (blob && (c % (G::LPR / kPassB)) == 0 && aid >= 0 && aid < n_assign)
                part[aid * G::RB + pass * G::RPP + rsub] = wgt * tot;
        }
    };
    auto pair_issue = [&](int s0, DownRegs<kPassB>& R0, DownRegs<kPassB>& R1, float4 (&h0)[2], float4 (&h1)[2],
                          const uint8_t*& b0, const uint8_t*& b1) {
        const int s1 = s0 + kWaves;
        b0 = blob_of(s0);
        b1 = blob_of(s1);
        down_issue<F, kPassB, G::RPP>(R0, b0 ? b0 : a.ev.base, L, row0 + rsub);
        down_issue<F, kPassB, G::RPP>(R1, b1 ? b1 : a.ev.base, L, row0 + rsub);
        const int q0 = s0 < n_active ? nth_set(W.starts, s0) : 0;
        const int q1 = s1 < n_active ? nth_set(W.starts, s1) : 0;
        h_issue(h0, a.h + (size_t)q0 * F, c);
        h_issue(h1, a.h + (size_t)q1 * F, c);
    };
    {
        DownRegs<kPassB> R0, R1;
        float4 h0[2], h1[2];
        const uint8_t *b0, *b1;
        pair_issue(wave, R0, R1, h0, h1, b0, b1);
        if (has_shared) {
            for (int t = 0; t < n_tok; ++t) {
                float4 hv[2];
                if (t == 0) { hv[0] = shh[0]; hv[1] = shh[1]; }
                else h_issue(hv, a.hs + (size_t)t * F, c);
                float o[NPS];
                down_partial<NPS>(shr, hv, o);
                int pass;
                const float tot = row_reduce<float, NPS, G::LPR>(o, &pass);
                const float wgt = a.sgate ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v_sg), t)) : 1.f;
                if (sh_ok && (c % (G::LPR / NPS)) == 0)
                    part[(n_assign + t) * G::RB + (NPS * wave + pass) * G::RPP + rsub] = wgt * tot;
            }
        }
        if (wave < n_active) slot_compute(R0, b0, wave, h0);
        if (wave + kWaves < n_active) slot_compute(R1, b1, wave + kWaves, h1);
    }
    for (int s0 = wave + 2 * kWaves; s0 < n_active; s0 += 2 * kWaves) {
        DownRegs<kPassB> R0, R1;
        float4 h0[2], h1[2];
        const uint8_t *b0, *b1;
        pair_issue(s0, R0, R1, h0, h1, b0, b1);
        slot_compute(R0, b0, s0, h0);
        if (s0 + kWaves < n_active) slot_compute(R1, b1, s0 + kWaves, h1);
    }
    lds_barrier();

    // ---- epilogue: shared, then routed in routing order, LoRA B, residual
    if (tid < ep_n) {
        float y = has_shared ? part[(n_assign + et) * G::RB + er] : 0.f;
        for (int j = 0; j < k; ++j) y += part[(et * k + j) * G::RB + er];
        if (lora_on) {
            float l = 0.f;
            if (lora_vec) l = lora_dot(lr, a.r);
            else
                for (int q = 0; q < a.r; ++q)
                    l += bf16_to_f32(a.lora_b[(size_t)(row0 + er) * a.r + q]) * a.au[(size_t)et * a.r + q];
            y += a.lora_scale * l;
        }
        if (a.fused) y += ep_x;
        a.y[(size_t)et * d + row0 + er] = y;
    }
}

__global__ void __launch_bounds__(kThreads) k_topk_job(TopkJob j, int n_tok) {
    topk_rows(false, j.logits, j.En, j.kn, n_tok, j.bias, j.mc, j.hc, j.mp, j.hp, nullptr, j.kn, j.pred_idx, j.pred_w);
}

hipError_t launch_topk_job(const TopkJob& j, int n_tok, hipStream_t s) {
    hipLaunchKernelGGL(k_topk_job, dim3(1), dim3(kThreads), 0, s, j, n_tok);
    return hipGetLastError();
}

int dec_b_rows_per_block(int f) { return kPassB * (64 / (f / 8)); }

hipError_t launch_dec_b(const DecBArgs& a, hipStream_t s, const KTime* tm) {
    if (a.n_tok > kMaxTokB || a.n_tok * a.k > kMaxAssign || (a.fs && a.fs != a.f)) return hipErrorInvalidValue;
    const int rb = dec_b_rows_per_block(a.f);
    if (a.d % rb || a.n_tok * rb > kThreads) return hipErrorInvalidValue;
    const dim3 grid(1 + a.d / rb), block(kThreads);
    switch (a.f) {
        case 64: MOE_LAUNCH(k_dec_b<64>, grid, block, 0, s, tm, a); break;
        case 128: MOE_LAUNCH(k_dec_b<128>, grid, block, 0, s, tm, a); break;
        case 256: MOE_LAUNCH(k_dec_b<256>, grid, block, 0, s, tm, a); break;
        case 512: MOE_LAUNCH(k_dec_b<512>, grid, block, 0, s, tm, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool dec_fast_path_ok(int d, int f, int fs, int n_tok, int k) {
    const bool dpow = d >= 256 && d <= 2048 && (d & (d - 1)) == 0;
    const bool fpow = f >= 64 && f <= 512 && (f & (f - 1)) == 0;
    if (!dpow || !fpow || (fs && fs != f)) return false;
    const int rb = dec_b_rows_per_block(f), ra = dec_a_hrows_per_block(d);
    return d % rb == 0 && f % ra == 0 && fs % ra == 0 && n_tok <= kMaxTokB && n_tok * k <= kMaxAssign &&
           n_tok * rb <= kThreads;
}

}  // namespace moe

// K_R's body (self-routing: RMSNorm prologue + router GEMV in fp64 + the
// top-k in the last block to finish), shared by its standalone launch and by
// the one-launch step's preparation kernel, which runs it for layer 0 beside
// the argument patch.
#pragma once
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
__device__ __forceinline__ void u_finish(const DecAArgs& a, int grp, const URegs& r, float* su, uint32_t* upk, uint32_t* upk_lo,
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
        ss = group_sum_dpp<double, 64>(ss);
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
        sh = group_sum_dpp<float, 4>(sh);
        sl = group_sum_dpp<float, 4>(sl);
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
    return group_sum_dpp<double, 64>(acc);
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

// Router rows of block bid of nblocks (one row per wave); logits are
// published with device-scope stores, then counted after a device-scope
// release fence; the last block to finish acquires and takes the top-k.
// suf: d floats of LDS.
__device__ __forceinline__ void dec_r_body(const DecAArgs& a, const RouteArgs& r, int bid, int nblocks, float* suf) {
    constexpr int kNld = 4;
    __shared__ double red[kWaves];
    __shared__ int is_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d = a.d;
    const int row = bid * kHeadRowsPerBlock + wave;
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
        // release: the block's logit stores (ordered before this thread by
        // the barrier) happen before the count; the last block acquires
        // before it reads the other blocks' logits
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const unsigned old = __hip_atomic_fetch_add(r.counters + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = old == (unsigned)nblocks - 1;
        if (is_last) {
            __hip_atomic_store(r.counters + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
    }
    __syncthreads();
    if (!is_last) return;
    topk_rows(true, r.logits_r, r.E, r.k, a.n_tok, r.router_bias, nullptr, nullptr, nullptr, nullptr,
              r.route_idx, r.k, r.self_idx, r.self_w);
}

inline int dec_r_blocks(int E) { return (E + kHeadRowsPerBlock - 1) / kHeadRowsPerBlock; }

}  // namespace moe

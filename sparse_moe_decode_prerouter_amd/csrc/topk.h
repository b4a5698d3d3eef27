// Top-k with renormalised softmax weights over the selected logits, one wave
// per token row: (logit descending, expert index ascending).
#pragma once
#include "device_common.h"
#include "moe_internal.h"
#include "dec_common.h"

namespace moe {

// (v, i) becomes the best of (v, i) and the pair of lane l - S (mod 16)
// in this lane's row of 16 (a DPP row rotation: no trip through the LDS
// crossbar, which every other lane shuffle takes)
template <int S>
__device__ __forceinline__ void best_row_ror(double& v, int& i) {
    constexpr int kCtrl = 0x120 + S;          // row_ror:S
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)b, kCtrl, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), kCtrl, 0xF, 0xF, false);
    const int oi = __builtin_amdgcn_update_dpp(0, i, kCtrl, 0xF, 0xF, false);
    const double ov = __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
}

// (v, i) becomes the best of (v, i) and the pair of lane l ^ OFF (OFF 16
// or 32): a v_permlane swap of the pair with itself leaves the partner's
// value in one of the two results (which one depends on the lane's half)
template <int OFF>
__device__ __forceinline__ void best_swap(double& v, int& i) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    uint32_t lo0 = (uint32_t)b, lo1 = lo0, hi0 = (uint32_t)(b >> 32), hi1 = hi0, i0 = (uint32_t)i, i1 = i0;
    swap_pair_u32(lo0, lo1, OFF);
    swap_pair_u32(hi0, hi1, OFF);
    swap_pair_u32(i0, i1, OFF);
    const bool upper = (threadIdx.x & OFF) != 0;
    const double ov = __longlong_as_double((long long)(((uint64_t)(upper ? hi0 : hi1) << 32) | (upper ? lo0 : lo1)));
    const int oi = (int)(upper ? i0 : i1);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
}

// every lane ends with the best (v, i) of the wave: rotations by 1, 2, 4
// and 8 cover each row of 16 lanes, two lane swaps join the four rows
__device__ __forceinline__ void wave_best(double& v, int& i) {
    best_row_ror<1>(v, i);
    best_row_ror<2>(v, i);
    best_row_ror<4>(v, i);
    best_row_ror<8>(v, i);
    best_swap<16>(v, i);
    best_swap<32>(v, i);
}

// lane j < k: the j-th selection and its weight (as also written out)
struct TopkSel {
    int idx;
    float w;
};

// PER logits per lane (E <= 64 * PER), held in registers with fixed indices:
// lane l holds experts l + 64 m. topk_load issues the loads (logits and
// bias) and topk_select waits for them, so a caller can issue them early.
template <int PER>
__device__ __forceinline__ void topk_load(bool coherent, const double* logits, int E, int t, const float* bias,
                                          double (&v)[PER], float (&b)[PER]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        const int e = lane + 64 * m;
        const int ec = e < E ? e : 0;
        v[m] = coherent ? ld_dev(logits + (size_t)t * E + ec) : logits[(size_t)t * E + ec];
        b[m] = bias ? bias[ec] : 0.f;
    }
}

template <int PER>
__device__ __forceinline__ TopkSel topk_select(double (&v)[PER], const float (&b)[PER], int E, int k, int t,
                                               const float* bias, const float* mc, const int32_t* hc, const float* mp,
                                               const int32_t* hp, int32_t* out_idx, float* out_w) {
    const int lane = threadIdx.x & 63;
    if (bias) {
#pragma unroll
        for (int m = 0; m < PER; ++m) v[m] += (double)b[m];
    }
    // history terms: each distinct valid expert of the previous routings adds its row
    for (int src = 0; src < 2; ++src) {
        const float* M = src ? mp : mc;
        const int32_t* H = src ? hp : hc;
        if (!M || !H) continue;
        for (int j = 0; j < k; ++j) {
            const int h = H[(size_t)t * k + j];
            bool dup = false;
            for (int jj = 0; jj < j; ++jj) dup |= H[(size_t)t * k + jj] == h;
            if (h < 0 || h >= E || dup) continue;
#pragma unroll
            for (int m = 0; m < PER; ++m) {
                const int e = lane + 64 * m;
                v[m] += (double)M[(size_t)h * E + (e < E ? e : 0)];
            }
        }
    }
#pragma unroll
    for (int m = 0; m < PER; ++m)
        if (lane + 64 * m >= E) v[m] = -INFINITY;
    // lane j keeps the j-th selection (no dynamically indexed arrays)
    double my_v = -INFINITY;
    int my_i = 0;
    for (int j = 0; j < k; ++j) {
        double bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int e = lane + 64 * m;
            if (e < E && better(v[m], e, bv, bi)) { bv = v[m]; bi = e; }
        }
        wave_best(bv, bi);
        if (lane == j) { my_v = bv; my_i = bi; }
#pragma unroll
        for (int m = 0; m < PER; ++m)
            if (lane + 64 * m == bi) v[m] = -INFINITY;
    }
    // softmax over the k selected logits, summed in selection order
    const double top = __shfl(my_v, 0, 64);
    const double ex = lane < k ? exp(my_v - top) : 0.0;
    double ssum = 0.0;
    for (int j = 0; j < k; ++j) ssum += __shfl(ex, j, 64);
    const float wsel = (float)(ex / ssum);
    if (lane < k) {
        out_idx[(size_t)t * k + lane] = my_i;
        out_w[(size_t)t * k + lane] = wsel;
    }
    return TopkSel{my_i, wsel};
}

template <int PER>
__device__ __forceinline__ TopkSel topk_row(bool coherent, const double* logits, int E, int k, int t, const float* bias,
                                const float* mc, const int32_t* hc, const float* mp, const int32_t* hp,
                                int32_t* out_idx, float* out_w) {
    double v[PER];
    float b[PER];
    topk_load<PER>(coherent, logits, E, t, bias, v, b);
    return topk_select<PER>(v, b, E, k, t, bias, mc, hc, mp, hp, out_idx, out_w);
}

// MAXPER bounds the register arrays instantiated (E <= 64 * MAXPER).
template <int MAXPER = 16>
__device__ __forceinline__ void topk_rows(bool coherent, const double* logits, int E, int k, int n_tok, const float* bias,
                                 const float* mc, const int32_t* hc, const float* mp, const int32_t* hp,
                                 const int32_t* route_idx, int kroute, int32_t* out_idx, float* out_w) {
    const int wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    for (int t = wave; t < n_tok; t += nwaves) {
        if (route_idx && route_idx[(size_t)t * kroute] >= 0) continue;   // row has its routing
        if (E <= 64) topk_row<1>(coherent, logits, E, k, t, bias, mc, hc, mp, hp, out_idx, out_w);
        else if (E <= 128 || MAXPER < 4) topk_row<(MAXPER < 2 ? MAXPER : 2)>(coherent, logits, E, k, t, bias, mc, hc, mp, hp, out_idx, out_w);
        else if (E <= 256 || MAXPER < 8) topk_row<(MAXPER < 4 ? MAXPER : 4)>(coherent, logits, E, k, t, bias, mc, hc, mp, hp, out_idx, out_w);
        else if (E <= 512 || MAXPER < 16) topk_row<(MAXPER < 8 ? MAXPER : 8)>(coherent, logits, E, k, t, bias, mc, hc, mp, hp, out_idx, out_w);
        else topk_row<MAXPER>(coherent, logits, E, k, t, bias, mc, hc, mp, hp, out_idx, out_w);
    }
}

}  // namespace moe

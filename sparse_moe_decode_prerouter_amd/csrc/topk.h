// Top-k with renormalised softmax weights over the selected logits, one wave
// per token row: (logit descending, expert index ascending).
#pragma once
#include "device_common.h"
#include "moe_internal.h"

namespace moe {

__device__ inline void topk_rows(bool coherent, const double* logits, int E, int k, int n_tok, const float* bias,
                          const float* mc, const int32_t* hc, const float* mp, const int32_t* hp,
                          const int32_t* route_idx, int kroute, int32_t* out_idx, float* out_w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    for (int t = wave; t < n_tok; t += nwaves) {
        if (route_idx && route_idx[(size_t)t * kroute] >= 0) continue;   // row has its routing
        double v[kMaxExperts / 64];
        const int per = (E + 63) / 64;
        for (int m = 0; m < per; ++m) {
            const int e = lane + 64 * m;
            double z = -INFINITY;
            if (e < E) {
                z = coherent ? ld_dev(logits + (size_t)t * E + e) : logits[(size_t)t * E + e];
                if (bias) z += (double)bias[e];
                if (mc && hc) {
                    for (int j = 0; j < k; ++j) {
                        const int h = hc[(size_t)t * k + j];
                        bool dup = false;
                        for (int jj = 0; jj < j; ++jj) dup |= hc[(size_t)t * k + jj] == h;
                        if (h >= 0 && h < E && !dup) z += (double)mc[(size_t)h * E + e];
                    }
                }
                if (mp && hp) {
                    for (int j = 0; j < k; ++j) {
                        const int h = hp[(size_t)t * k + j];
                        bool dup = false;
                        for (int jj = 0; jj < j; ++jj) dup |= hp[(size_t)t * k + jj] == h;
                        if (h >= 0 && h < E && !dup) z += (double)mp[(size_t)h * E + e];
                    }
                }
            }
            v[m] = z;
        }
        double sel_v[kMaxTopK];
        int sel_i[kMaxTopK];
        for (int j = 0; j < k; ++j) {
            double bv = -INFINITY; int bi = 0x7fffffff;
            for (int m = 0; m < per; ++m) {
                const int e = lane + 64 * m;
                if (e < E && better(v[m], e, bv, bi)) { bv = v[m]; bi = e; }
            }
            for (int o = 32; o > 0; o >>= 1) {
                const double ov = __shfl_xor(bv, o, 64);
                const int oi = __shfl_xor(bi, o, 64);
                if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
            }
            sel_v[j] = bv; sel_i[j] = bi;
            for (int m = 0; m < per; ++m)
                if (lane + 64 * m == bi) v[m] = -INFINITY;
        }
        if (lane == 0) {
            double ssum = 0.0;
            double ex[kMaxTopK];
            for (int j = 0; j < k; ++j) { ex[j] = exp(sel_v[j] - sel_v[0]); ssum += ex[j]; }
            for (int j = 0; j < k; ++j) {
                out_idx[(size_t)t * k + j] = sel_i[j];
                out_w[(size_t)t * k + j] = (float)(ex[j] / ssum);
            }
        }
    }
}

}  // namespace moe

// Shared pieces of the fused decode kernels.
#pragma once
#include "device_common.h"

namespace moe {

constexpr int kMaxAssign = 64;          // n_tok * k on the fused decode path
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Block barrier that waits for LDS traffic only: global loads stay in flight
// across it (HIP's __syncthreads would also wait for them).
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): this wave's LDS ops are done
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wave-local LDS exchange: this wave's LDS writes are visible to its own
// later LDS reads (LDS ops of one wave complete in order).
__device__ __forceinline__ void wave_lds_sync() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Sum NP per-lane values over aligned groups of LPR lanes. Each halving step
// trades half of the values with the partner lane, so after log2(NP) steps
// every lane holds the partial of one of the NP values; plain butterflies
// finish the sum. Returns the lane's total; *which gets its value index.
// Every lane of a group of LPR/NP consecutive lanes ends with the same value.
template <typename T, int NP, int LPR>
__device__ __forceinline__ T row_reduce(const T (&v)[NP], int* which) {
    static_assert(LPR >= NP, "one value per lane at least");
    const int lane = threadIdx.x & 63;
    int lo = 0;
    int off = LPR / 2;
    T cur[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) cur[i] = v[i];
#pragma unroll
    for (int n = NP; n > 1; n >>= 1) {
        const bool upper = (lane & off) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
            const T send = upper ? cur[i] : cur[i + n / 2];
            const T keep = upper ? cur[i + n / 2] : cur[i];
            cur[i] = keep + __shfl_xor(send, off, 64);
        }
        if (upper) lo += n / 2;
        off >>= 1;
    }
    T t = cur[0];
#pragma unroll
    for (int o = LPR / NP / 2; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
    *which = lo;
    return t;
}

}  // namespace moe

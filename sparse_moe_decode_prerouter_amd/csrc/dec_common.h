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

// The routing a decode call uses, one entry per lane (< n_assign): a row's
// given routing, or its self-routing when the row's first given index is
// negative or no routing is given. Loads are unconditional (pointer stand-ins)
// so that waiting for them never waits for later loads.
struct RouteIn {
    int vr, vs;
    float vrw, vsw;
};

__device__ __forceinline__ RouteIn route_load(const int32_t* route_idx, const float* route_w,
                                              const int32_t* self_idx, const float* self_w, int n_assign) {
    const int lane = threadIdx.x & 63;
    const int li = lane < n_assign ? lane : 0;
    const int32_t* ri = route_idx ? route_idx : self_idx;
    const float* rw = route_idx ? route_w : self_w;
    const int32_t* si = self_idx ? self_idx : ri;
    const float* sw = self_idx ? self_w : rw;
    RouteIn r;
    r.vr = ri[li]; r.vs = si[li]; r.vrw = rw[li]; r.vsw = sw[li];
    return r;
}

// merged (expert, weight) of this lane's entry; expert -1 past n_assign
__device__ __forceinline__ void route_merge(const RouteIn& r, bool given_ptr, int k, int n_assign, int* me, float* mw) {
    const int lane = threadIdx.x & 63;
    const int first = __shfl(r.vr, (lane / k) * k, 64);
    const bool given = given_ptr && first >= 0;
    *me = lane < n_assign ? (given ? r.vr : r.vs) : -1;
    *mw = given ? r.vrw : r.vsw;
}

// ---- routing digest of one wave -------------------------------------------
// Entry `lane` (< n) routes to expert e. Sorted by (expert, entry), invalid
// entries last; sorted position p is held by lane p.
struct WaveDigest {
    int n_active, n_valid;
    unsigned long long starts;   // bit p: sorted position p starts an expert
    uint32_t sk;                 // sorted key of position `lane`: expert << 16 | entry
};

__device__ __forceinline__ WaveDigest wave_digest(int n, int e, int E, uint32_t* sl) {
    const int lane = threadIdx.x & 63;
    const bool in = lane < n;
    const bool ok = in && e >= 0 && e < E;
    const uint32_t key = in ? (((uint32_t)(ok ? e : 0xFFFF) << 16) | (uint32_t)lane) : 0xFFFFFFFFu;
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += (uint32_t)__shfl((int)key, j, 64) < key;
    if (in) sl[rank] = key;
    wave_lds_sync();
    WaveDigest W;
    W.sk = in ? sl[lane] : 0xFFFFFFFFu;
    const int ep = (int)(W.sk >> 16);
    const bool valid = in && ep != 0xFFFF;
    const int prev = __shfl_up(ep, 1, 64);
    const bool start = valid && (lane == 0 || prev != ep);
    W.starts = __ballot(start);
    W.n_active = __popcll(W.starts);
    W.n_valid = __popcll(__ballot(valid));
    return W;
}

// position of the s-th set bit of m (s < popcount(m))
__device__ __forceinline__ int nth_set(unsigned long long m, int s) {
    for (int i = 0; i < s; ++i) m &= m - 1;
    return __ffsll((long long)m) - 1;
}

}  // namespace moe

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

// The value of a partner lane in the other half of each aligned block of
// 2*off lanes. Within a row of 16 lanes the partner is taken by a DPP
// permutation (xor 1, xor 2, then the half-row and row mirrors, which pair
// each lane of one half with one of the other), with no trip through the
// LDS crossbar that other lane shuffles take; offsets 16 and 32 shuffle
// (the sums below take those offsets with lane swaps instead).
// Sums over a block come out the same with any such pairing.
__device__ __forceinline__ int partner_i32(int v, int off) {
    switch (off) {
        case 1: return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
        case 2: return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
        case 4: return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);   // row_half_mirror
        case 8: return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);   // row_mirror
        default: return __shfl_xor(v, off, 64);
    }
}
__device__ __forceinline__ float partner(float v, int off) {
    return __int_as_float(partner_i32(__float_as_int(v), off));
}
__device__ __forceinline__ double partner(double v, int off) {
    const long long b = __double_as_longlong(v);
    const int lo = partner_i32((int)(unsigned)b, off), hi = partner_i32((int)(b >> 32), off);
    return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Offsets 16 and 32 without the crossbar: v_permlane16_swap trades the odd
// rows (of 16 lanes) of one register with the even rows of another, and
// v_permlane32_swap the upper half of one with the lower half of another.
// After swap_pair(x, y, off) a lane in the lower half of its 2*off block
// holds its own x and its partner's x, one in the upper half its partner's y
// and its own y: x + y is the halving step of row_reduce in one add.
__device__ __forceinline__ void swap_pair_u32(uint32_t& x, uint32_t& y, int off) {
    if (off == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
        x = r[0]; y = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
        x = r[0]; y = r[1];
    }
}
__device__ __forceinline__ void swap_pair(float& x, float& y, int off) {
    uint32_t a = __float_as_uint(x), b = __float_as_uint(y);
    swap_pair_u32(a, b, off);
    x = __uint_as_float(a); y = __uint_as_float(b);
}
__device__ __forceinline__ void swap_pair(double& x, double& y, int off) {
    const uint64_t a = (uint64_t)__double_as_longlong(x), b = (uint64_t)__double_as_longlong(y);
    uint32_t alo = (uint32_t)a, ahi = (uint32_t)(a >> 32), blo = (uint32_t)b, bhi = (uint32_t)(b >> 32);
    swap_pair_u32(alo, blo, off);
    swap_pair_u32(ahi, bhi, off);
    x = __longlong_as_double((long long)(((uint64_t)ahi << 32) | alo));
    y = __longlong_as_double((long long)(((uint64_t)bhi << 32) | blo));
}
// v + the partner lane's v (a butterfly step; both lanes get the same sum,
// addition being commutative)
template <typename T>
__device__ __forceinline__ T pair_sum(T v, int off) {
    if (off >= 16) {
        T x = v, y = v;
        swap_pair(x, y, off);
        return x + y;
    }
    return v + partner(v, off);
}

// Sum NP per-lane values over aligned groups of LPR lanes. Each halving step
// trades half of the values with a partner lane in the other half of the
// block, so after log2(NP) steps every lane holds the partial of one of the
// NP values; butterflies finish the sum. Returns the lane's total; *which
// gets its value index. Every lane of a group of LPR/NP consecutive lanes
// ends with the same value.
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
        // (opaque: otherwise the compiler merges the lane tests of all the
        // levels into one index and selects each value from the original
        // NP with a chain of compares)
        uint32_t up = (uint32_t)(lane & off);
        asm volatile("" : "+v"(up));
        const bool upper = up != 0;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
            if (off >= 16) {
                T x = cur[i], y = cur[i + n / 2];
                swap_pair(x, y, off);
                cur[i] = x + y;
            } else {
                const T send = upper ? cur[i] : cur[i + n / 2];
                const T keep = upper ? cur[i + n / 2] : cur[i];
                cur[i] = keep + partner(send, off);
            }
        }
        if (upper) lo += n / 2;
        off >>= 1;
    }
    T t = cur[0];
#pragma unroll
    for (int o = LPR / NP / 2; o > 0; o >>= 1) t = pair_sum(t, o);
    *which = lo;
    return t;
}

// sum over aligned groups of `width` lanes (a power of two <= 64), every
// lane of a group ending with the group's sum
template <typename T, int WIDTH>
__device__ __forceinline__ T group_sum_dpp(T v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v = pair_sum(v, o);
    return v;
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

// In-launch hand-off between the phases of the one-launch stack decode.
//
// The handed-off values carry their own readiness. Before each launch every
// exchange word a launch will publish is set to kEmptyWord (all ones: a NaN
// bit pattern that no arithmetic here produces from finite inputs). A
// producer publishes each value with a device-scope store (st_dev: 32 or 64
// bits, single-copy atomic, written through to the device-coherent level)
// and is done: no wait for its stores, no arrival count, no flag. A consumer
// wave reads the values it needs with device-scope loads (ld_dev, ld_coh4:
// served at the device-coherent level, never from a stale line of its own
// XCD's L2) and reads them again until none of its words is empty. Each
// value is written once per launch, so a word that is not empty holds its
// final value. A 64-bit value (a head logit) is tested on its high word: its
// store and load are single 64-bit accesses, so both halves appear together.
//
// A waiting wave first polls one word of its data (one request per wave),
// and polls everything only once that word has arrived, so that the waves
// that wait long do not load their whole data again and again.
//
// The polls are bounded: after `spin_limit` polls the wave sets the abort
// word (every later wait of the launch gives up within a few polls), raises
// ERR_TIMEOUT in the layer's error word and goes on with what it read, so a
// value that never arrives turns into an error status, never a hang.
#pragma once
#include "device_common.h"
#include "dec_common.h"
#include "moe_internal.h"

#ifndef MOE_FUSE_SLEEP
#define MOE_FUSE_SLEEP 2          // s_sleep units (64 clocks each) between polls
#endif

namespace moe {

constexpr uint32_t kEmptyWord = 0xFFFFFFFFu;

struct FuseSync {
    bool on;                    // the inputs are published in this launch: poll them
    uint32_t* abort;            // nonzero once a wait of this launch has timed out
    uint32_t spin_limit;
};

__device__ __forceinline__ bool empty_word(float v) { return __float_as_uint(v) == kEmptyWord; }
__device__ __forceinline__ bool empty_word(double v) {
    return (uint32_t)((uint64_t)__double_as_longlong(v) >> 32) == kEmptyWord;
}
__device__ __forceinline__ bool any_empty(float4 v) {
    return empty_word(v.x) | empty_word(v.y) | empty_word(v.z) | empty_word(v.w);
}

// one more poll of a wave's wait: false while it may go on polling
__device__ __forceinline__ bool poll_tick(const FuseSync& fs, int32_t* err, uint32_t& n) {
    if (++n > fs.spin_limit) {
        if ((threadIdx.x & 63) == 0) {
            __hip_atomic_store(fs.abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            set_err(err, ERR_TIMEOUT);
        }
        return true;
    }
    if ((n & 7) == 0 && ld_dev(fs.abort)) return true;
    __builtin_amdgcn_s_sleep(MOE_FUSE_SLEEP);
    return false;
}

// One wave: `load()` issues this lane's loads into the caller's registers
// and returns true when none of the words it read is empty; it is repeated
// until that holds on every lane (or the wait gives up). probe: one word the
// wave needs, polled alone first (nullptr: none). Wave-uniform control flow.
template <typename Load>
__device__ __forceinline__ void fuse_poll(const FuseSync& fs, int32_t* err, const float* probe, Load&& load) {
    if (!fs.on) {
        (void)load();
        return;
    }
    uint32_t n = 0;
    bool give_up = false;
    if (probe)
        while (empty_word(ld_dev(probe)))
            if (poll_tick(fs, err, n)) { give_up = true; break; }
    while (true) {
        const bool ok = load();
        if (give_up || __ballot(!ok) == 0ull) break;
        if (poll_tick(fs, err, n)) break;
    }
}

// 16 bytes of data published in this launch, at element `elem` past a
// base address that is the same for the whole wave: a buffer load with the
// device-scope cache policy (sc1), which is served at the device-coherent
// level like ld_dev, one 128-bit load instead of four 32-bit ones, and
// (unlike a volatile access) not followed by a wait of its own.
__device__ __forceinline__ u32x4 ld_coh4(const float* base, uint32_t elem) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, 0x7fffffff, 0x00020000);
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)(elem * 4u), 0, 16 /* sc1 */);
}
// the matching store (base the same for the whole wave)
__device__ __forceinline__ void st_coh4(float* base, uint32_t elem, u32x4 v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)(elem * 4u), 0, 16 /* sc1 */);
}
__device__ __forceinline__ float4 u4_as_f4(u32x4 v) {
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

}  // namespace moe

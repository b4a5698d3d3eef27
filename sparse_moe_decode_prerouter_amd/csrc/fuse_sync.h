// In-launch hand-off between the phases of the one-launch stack decode.
//
// A producer block publishes its outputs with device-scope stores (st_dev:
// written through to the device-coherent level) and waits until they are
// complete (s_waitcnt with every counter at zero: on gfx9-class chips the
// vector-memory counter covers stores) before it signals its arrival (the
// arrival protocol itself is the stack kernel's). A consumer block polls a
// flag word with device-scope loads until it holds the expected value, and
// then reads the published values with device-scope loads (ld_dev), which
// are served at the device-coherent level, never from a stale line of its
// own XCD's L2. Because both sides access the handed-off data only through
// device-scope operations, the L2 write-back and invalidate that a
// release/acquire fence would add (which exist for plain accesses) are not
// needed; building with MOE_FUSE_FENCES=1 adds them (release before the
// arrival, acquire after the poll) to measure what they cost.
//
// The poll is bounded: after `spin_limit` polls the block sets the abort word
// (every later wait of the launch gives up at once), raises ERR_TIMEOUT in
// the layer's error word and goes on, so a lost arrival turns into an error
// status, never a hang.
#pragma once
#include "device_common.h"
#include "dec_common.h"
#include "moe_internal.h"

#ifndef MOE_FUSE_FENCES
#define MOE_FUSE_FENCES 0
#endif
#ifndef MOE_FUSE_SLEEP
#define MOE_FUSE_SLEEP 2          // s_sleep units (64 clocks each) between polls
#endif

namespace moe {

struct FuseSync {
    const uint32_t* flag;       // word to wait on (nullptr: no wait)
    uint32_t value;             // until it holds this value
    uint32_t* abort;            // nonzero once a wait of this launch has timed out
    uint32_t spin_limit;
};

// every thread of the block; loads issued before it stay in flight
__device__ __forceinline__ void fuse_wait(const FuseSync& fs, int32_t* err) {
    if (!fs.flag) return;
    if (threadIdx.x == 0) {
        uint32_t n = 0;
        while (ld_dev(fs.flag) != fs.value) {
            if (ld_dev(fs.abort)) break;
            if (++n > fs.spin_limit) {
                __hip_atomic_store(fs.abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                set_err(err, ERR_TIMEOUT);
                break;
            }
            __builtin_amdgcn_s_sleep(MOE_FUSE_SLEEP);
        }
#if MOE_FUSE_FENCES
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#endif
    }
    lds_barrier();
}

// every thread of the block, after its last store of a phase: the block's
// stores are complete when it returns
__device__ __forceinline__ void fuse_stores_done() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);           // this wave's stores are complete
#if MOE_FUSE_FENCES
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
#endif
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
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
__device__ __forceinline__ float4 u4_as_f4(u32x4 v) {
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

}  // namespace moe

// Device-initiated staging: the routing on the device drives the copies
// into the slab, with no host read-back (the guide's Key terms: staged decode
// maps expert ids to fixed slots with a GPU slot table; incr_stack rewrites
// only the slots that changed). The store is pinned host memory mapped into
// the device's address space (it stands in for the SSD tier), so the copies
// are device loads over PCIe.
//   k_stage_plan  one block: the wanted set (bitmap of the routing entries),
//                 the sticky plan of the host planner (resident experts keep
//                 their slot; missing ones, ascending id, take the slots not
//                 holding a wanted expert, ascending), the slot table, the
//                 copy list and the bytes counter; the shared slot on first use
//   k_stage_copy  the copy list's blobs, 16 bytes per load, 8 loads in
//                 flight per thread, spread over the grid
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

__global__ void __launch_bounds__(64) k_stage_plan(DevStageArgs a) {
    __shared__ uint32_t want[kMaxExperts / 32], have[kMaxExperts / 32];
    __shared__ uint8_t keep[kMaxStageSlots];
    const int lane = threadIdx.x;
    const int nw = (a.E + 31) / 32;
    for (int i = lane; i < nw; i += 64) { want[i] = 0u; have[i] = 0u; }
    __syncthreads();
    for (int i = lane; i < a.n_ids; i += 64) {
        const int e = a.ids[i];
        if (e >= 0 && e < a.E) atomicOr(&want[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    // a slot keeps its expert when that expert is wanted
    for (int s = lane; s < a.slots; s += 64) {
        const int tag = a.slot_tag[s];
        const bool k = tag >= 0 && tag < a.E && ((want[tag >> 5] >> (tag & 31)) & 1u);
        keep[s] = k;
        if (k) atomicOr(&have[tag >> 5], 1u << (tag & 31));
    }
    __syncthreads();
    if (lane != 0) return;
    int nwant = 0;
    for (int w = 0; w < nw; ++w) nwant += __popc(want[w]);
    int n = 0;
    if (nwant > a.slots) {
        set_err(a.err, ERR_NOT_STAGED);              // more distinct experts than slots: nothing staged
    } else {
        int s = 0;                                   // next free slot candidate (ascending)
        for (int w = 0; w < nw; ++w) {
            uint32_t m = want[w] & ~have[w];
            while (m) {
                const int e = 32 * w + __ffs(m) - 1;
                m &= m - 1;
                while (keep[s]) ++s;                 // a free slot exists: missing <= slots - kept
                const int old = a.slot_tag[s];
                if (old >= 0 && old < a.E && a.slot_of[old] == s) a.slot_of[old] = -1;
                a.slot_of[e] = s;
                a.slot_tag[s] = e;
                a.plan[1 + 2 * n] = s;
                a.plan[2 + 2 * n] = e;
                ++n;
                ++s;
            }
        }
    }
    int sh = 0;
    if (a.shared && a.slot_tag[a.slots] != a.E) {
        a.slot_tag[a.slots] = a.E;
        sh = 1;
    }
    a.plan[0] = n;
    a.plan[stage_plan_shared(a.slots)] = sh;
    atomicAdd(a.bytes, (unsigned long long)n * a.blob + (sh ? a.sblob : 0ull));
}

__global__ void __launch_bounds__(256) k_stage_copy(DevStageArgs a) {
    const int n = a.plan[0], sh = a.plan[stage_plan_shared(a.slots)];
    const uint32_t per = (uint32_t)(a.blob / 16), per_s = (uint32_t)(a.sblob / 16);
    const uint32_t total = (uint32_t)n * per + (sh ? per_s : 0u);
    const uint32_t stride = gridDim.x * 256u;
    for (uint32_t base = blockIdx.x * 256u + threadIdx.x; base < total; base += 8u * stride) {
        u32x4 v[8];
        u32x4* dst[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t i = base + (uint32_t)j * stride;
            dst[j] = nullptr;
            if (i >= total) continue;
            const u32x4* src;
            if (i < (uint32_t)n * per) {
                const uint32_t c = i / per, off = i - c * per;
                const int s = a.plan[1 + 2 * c], e = a.plan[2 + 2 * c];
                src = (const u32x4*)(a.store + (size_t)e * a.blob) + off;
                dst[j] = (u32x4*)(a.slab + (size_t)s * a.blob) + off;
            } else {
                const uint32_t off = i - (uint32_t)n * per;
                src = (const u32x4*)a.shared + off;
                dst[j] = (u32x4*)(a.slab + (size_t)a.slots * a.blob) + off;
            }
            v[j] = *src;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (dst[j]) *dst[j] = v[j];
    }
}

hipError_t launch_stage_device(const DevStageArgs& a, int blocks, hipStream_t s) {
    if (a.slots < 1 || a.slots > kMaxStageSlots || a.E < 1 || a.E > kMaxExperts || a.blob % 16 || a.sblob % 16 ||
        a.n_ids < 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_stage_plan, dim3(1), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_stage_copy, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe

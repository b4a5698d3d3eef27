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
#include "dec_b_body.h"
#include "dec_r_body.h"

namespace moe {



// ---------------------------------------------------------------------------
// K_R: self-routing for rows with no prediction: RMSNorm prologue + router
// GEMV (bf16 x fp32 products, fp64 accumulation) + top-k in the last block.
// Logits are published with device-scope stores and counted with a relaxed
// atomic, so the last block reads them coherently without cache flushes.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) k_dec_r(DecAArgs a, RouteArgs r) {
    extern __shared__ __align__(16) uint8_t lds[];
    dec_r_body(a, r, (int)blockIdx.x, (int)gridDim.x, (float*)lds);
}

hipError_t launch_dec_r(const DecAArgs& a, const RouteArgs& r, hipStream_t s, const KTime* tm) {
    if (a.d > 2048) return hipErrorInvalidValue;
    MOE_LAUNCH(k_dec_r, dim3(dec_r_blocks(r.E)), dim3(kThreads), (size_t)a.d * 4, s, tm, a, r);
    return hipGetLastError();
}

// K_B: its body is in dec_b_body.h (shared with the one-launch-per-layer
// decode kernel); the standalone launch.
template <int F>
__global__ void __launch_bounds__(kThreads, 2) k_dec_b(DecBArgs a) {
    dec_b_body<F, false>(a, (int)blockIdx.x, FuseSync{});
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

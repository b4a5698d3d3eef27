// K_A of the fused decode path (norm + gate/up GEMV + head + LoRA A +
// shared gate); the body is in dec_a_body.h, shared with the one-launch
// stack decode kernel.
#include "device_common.h"
#include "moe_internal.h"
#include "dec_common.h"
#include "topk.h"
#include "dec_a_body.h"

namespace moe {

int dec_a_hrows_per_block(int d) { return kWaves * kAPass * (64 / (d / 32)); }
int dec_a_brows_per_block(int d) { return kWaves * kABPass * (64 / (d / 32)); }

template <int D, bool XB>
__global__ void __launch_bounds__(kThreads) k_dec_a(DecAArgs a) {
    dec_a_body<D, XB, false>(a, (int)blockIdx.x, FuseSync{});
}

int dec_a_blocks(int d, int f, int fs, int n_tok, int k, int E, int En, int r, bool sgate, int* nb_h, int* nb_head,
                 int* nb_misc) {
    const int hr = dec_a_hrows_per_block(d), br = dec_a_brows_per_block(d);
    const int max_active = n_tok * k < E ? n_tok * k : E;
    *nb_h = (fs + max_active * f + hr - 1) / hr;
    *nb_head = (En + br - 1) / br;
    *nb_misc = (r + (sgate ? 1 : 0) + br - 1) / br;
    return *nb_h + *nb_head + *nb_misc;
}

hipError_t launch_dec_a(const DecAArgs& a, hipStream_t s, const KTime* tm) {
    const int hr = dec_a_hrows_per_block(a.d);
    if (a.n_tok * a.k > kMaxAssign || a.f % hr || a.fs % hr) return hipErrorInvalidValue;
    const dim3 grid(a.nb_h + a.nb_head + a.nb_misc + (a.topk.pred_idx ? 1 : 0)), block(kThreads);
    const bool xb = a.x_is_bf16 != 0;
    switch (a.d) {
        case 256: if (xb) MOE_LAUNCH((k_dec_a<256, true>), grid, block, 0, s, tm, a); else MOE_LAUNCH((k_dec_a<256, false>), grid, block, 0, s, tm, a); break;
        case 512: if (xb) MOE_LAUNCH((k_dec_a<512, true>), grid, block, 0, s, tm, a); else MOE_LAUNCH((k_dec_a<512, false>), grid, block, 0, s, tm, a); break;
        case 1024: if (xb) MOE_LAUNCH((k_dec_a<1024, true>), grid, block, 0, s, tm, a); else MOE_LAUNCH((k_dec_a<1024, false>), grid, block, 0, s, tm, a); break;
        case 2048: if (xb) MOE_LAUNCH((k_dec_a<2048, true>), grid, block, 0, s, tm, a); else MOE_LAUNCH((k_dec_a<2048, false>), grid, block, 0, s, tm, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moe

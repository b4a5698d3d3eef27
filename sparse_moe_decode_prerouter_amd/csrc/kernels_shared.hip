// The shared expert when its projections carry the recovery LoRA: each of
// gate, up and down is W_int4 x + (alpha / r) B A x, kept unmerged (the
// guide's Method section, three-stage training: the adapter sits on the
// shared-expert projections; unmerged adapter execution). The routing GEMM
// has already written A_g u and A_u u (and the shared gate); here:
//   k_sl_gateup  a = Wg u + s Bg (Ag u), c = Wu u + s Bu (Au u), h = silu(a) c
//   k_sl_down    o = Wd h + s Bd (Ad h),  y += sigmoid(g . u) o
// One wave per output row, a block of 16 tokens reusing the row's weights in
// registers; int4 codes and (s, b) read with 128-bit and 32-bit loads.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {

constexpr int kSlTok = 16;          // tokens per block
constexpr int kSlMaxF = 8192;       // f_s held in LDS by the down kernel

// 8 consecutive elements 8p .. 8p + 7 of u from the prologue's pair order:
// dword 4p + i holds elements 8p + i (low half) and 8p + i + 4 (high half)
__device__ __forceinline__ void u_piece(const uint32_t* row, const uint32_t* row_lo, int p, float (&v)[8]) {
    const u32x4 w = *(const u32x4*)(row + 4 * p);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = bf16_to_f32(ws[i] & 0xFFFF);
        v[i + 4] = bf16_to_f32(ws[i] >> 16);
    }
    if (row_lo) {
        const u32x4 l = *(const u32x4*)(row_lo + 4 * p);
        const uint32_t ls[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] += bf16_to_f32(ls[i] & 0xFFFF);
            v[i + 4] += bf16_to_f32(ls[i] >> 16);
        }
    }
}

__global__ void __launch_bounds__(256) k_sl_gateup(SharedLoraArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = a.d, f = a.f, rs = a.rs;
    if (a.tag && *a.tag != a.tag_want) {
        if (threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0) set_err(a.err, ERR_NOT_STAGED);
        return;
    }
    const int n = blockIdx.x * 4 + wave;                 // row of gate and of up
    if (n >= f) return;                                  // whole wave
    const BlobLayout L = BlobLayout::make(d, f);
    const int nch = d / 32;                              // 32-element chunks of a row
    // the adapter's B rows: lane q < rs holds column q
    const float bg = lane < rs ? bf16_to_f32(a.b_gu[(size_t)n * rs + lane]) : 0.f;
    const float bu = lane < rs ? bf16_to_f32(a.b_gu[(size_t)(f + n) * rs + lane]) : 0.f;
    const int t1 = min(a.n_tok, (int)(blockIdx.y + 1) * kSlTok);
    for (int t = blockIdx.y * kSlTok; t < t1; ++t) {
        const uint32_t* urow = a.u_pk + (size_t)t * (d / 2);
        const uint32_t* ulo = a.u_pk_lo ? a.u_pk_lo + (size_t)t * (d / 2) : nullptr;
        float pa = 0.f, pc = 0.f;
        for (int c = lane; c < nch; c += 64) {
            const u32x4 qg = *(const u32x4*)(a.blob + L.gate_q + (size_t)n * (d / 2) + 16 * c);
            const u32x4 qu = *(const u32x4*)(a.blob + L.up_q + (size_t)n * (d / 2) + 16 * c);
            const uint32_t sg = *(const uint32_t*)(a.blob + L.gate_sb + ((size_t)n * (d / 64) + c / 2) * 4);
            const uint32_t su = *(const uint32_t*)(a.blob + L.up_sb + ((size_t)n * (d / 64) + c / 2) * 4);
            const uint32_t gq[4] = {qg.x, qg.y, qg.z, qg.w}, uq[4] = {qu.x, qu.y, qu.z, qu.w};
            float dg = 0.f, du = 0.f, su_ = 0.f;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float v[8];
                u_piece(urow, ulo, 4 * c + p, v);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    // element 8p + j of the chunk is nibble j of dword p
                    dg += (float)((gq[p] >> (4 * j)) & 0xFu) * v[j];
                    du += (float)((uq[p] >> (4 * j)) & 0xFu) * v[j];
                    su_ += v[j];
                }
            }
            pa += f16_to_f32(sg & 0xFFFF) * dg + f16_to_f32(sg >> 16) * su_;
            pc += f16_to_f32(su & 0xFFFF) * du + f16_to_f32(su >> 16) * su_;
        }
        if (lane < rs) {
            pa += a.scale * bg * a.sau[(size_t)t * 2 * rs + lane];
            pc += a.scale * bu * a.sau[(size_t)t * 2 * rs + rs + lane];
        }
        pa = group_sum(pa, 64);
        pc = group_sum(pc, 64);
        if (lane == 0) a.hs[(size_t)t * f + n] = silu_f32(pa) * pc;
    }
}

__global__ void __launch_bounds__(256) k_sl_down(SharedLoraArgs a) {
    __shared__ float hsm[kSlMaxF];
    __shared__ float adh[64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d = a.d, f = a.f, rs = a.rs;
    if (a.tag && *a.tag != a.tag_want) return;       // flagged by the gate/up kernel
    const int i = blockIdx.x * 4 + wave;             // output row
    const bool row_ok = i < d;
    const int ir = row_ok ? i : d - 1;
    const BlobLayout L = BlobLayout::make(d, f);
    const int nch = f / 8;                           // 8-element chunks (one dword of codes)
    const float bd = lane < rs ? bf16_to_f32(a.bd[(size_t)ir * rs + lane]) : 0.f;
    const int t1 = min(a.n_tok, (int)(blockIdx.y + 1) * kSlTok);
    for (int t = blockIdx.y * kSlTok; t < t1; ++t) {
        for (int j = tid; j < f; j += 256) hsm[j] = a.hs[(size_t)t * f + j];
        __syncthreads();
        // A_d h: rows q = wave, wave + 4, ... of A_d, lanes over f
        for (int q = wave; q < rs; q += 4) {
            float s = 0.f;
            for (int j = lane; j < f; j += 64) s += bf16_to_f32(a.ad[(size_t)q * f + j]) * hsm[j];
            s = group_sum(s, 64);
            if (lane == 0) adh[q] = s;
        }
        __syncthreads();
        float po = 0.f;
        for (int c = lane; c < nch; c += 64) {
            const uint32_t q = *(const uint32_t*)(a.blob + L.down_q + (size_t)ir * (f / 2) + 4 * c);
            const uint32_t sb = *(const uint32_t*)(a.blob + L.down_sb + ((size_t)ir * (f / 64) + c / 8) * 4);
            float dq = 0.f, sh = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float h = hsm[8 * c + j];
                dq += (float)((q >> (4 * j)) & 0xFu) * h;
                sh += h;
            }
            po += f16_to_f32(sb & 0xFFFF) * dq + f16_to_f32(sb >> 16) * sh;
        }
        if (lane < rs) po += a.scale * bd * adh[lane];
        po = group_sum(po, 64);
        if (lane == 0 && row_ok) {
            const float gate = a.sgate ? a.sgate[t] : 1.f;
            a.y[(size_t)t * d + i] += gate * po;
        }
        __syncthreads();                             // hsm / adh are rewritten for the next token
    }
}

hipError_t launch_shared_lora(const SharedLoraArgs& a, hipStream_t s, bool gateup, bool down) {
    if (a.d % 256 || a.f % 64 || a.f > kSlMaxF || a.rs < 1 || a.rs > 64 || a.n_tok <= 0) return hipErrorInvalidValue;
    const unsigned ntb = (a.n_tok + kSlTok - 1) / kSlTok;
    if (gateup) {
        hipLaunchKernelGGL(k_sl_gateup, dim3((a.f + 3) / 4, ntb), dim3(256), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (down) {
        hipLaunchKernelGGL(k_sl_down, dim3((a.d + 3) / 4, ntb), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace moe

// Decode-path kernels for gfx950: prologue, bf16 GEMVs with top-k, token to
// expert sort/permute, and the int4 grouped GEMVs (gate/up + SwiGLU, down +
// combine + shared expert + LoRA + residual).
#include "device_common.h"
#include "moe_internal.h"
#include "topk.h"

namespace moe {

// ---------------------------------------------------------------------------
// Prologue: block input u of every token.
// Fused: u = x / sqrt(mean(x^2) + eps) * gamma evaluated in fp64 and rounded
// once to the activation dtype (RMSNorm prologue of the head input: the head
// reads the post-norm hidden state -- reading guide, Method, prerouter head).
// Writes u (fp32, exact act values), the GEMV-ordered bf16 pairs and the
// per-32-chunk sums used by the int4 dot products.
// GEMV order of a 32-element chunk c: dword 4*i + p holds elements
// (32c + 8i + p, 32c + 8i + p + 4), matching the nibble pairs that one
// masked shift of a packed dword yields.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_prologue(PrologueArgs a) {
    extern __shared__ float su[];          // [d]
    __shared__ double red[256];
    const int t = blockIdx.x, d = a.d, tid = threadIdx.x;
    double ss = 0.0;
    for (int j = tid; j < d; j += 256) {
        double xv = a.x_is_bf16 ? (double)bf16_to_f32(((const uint16_t*)a.x)[(size_t)t * d + j])
                                : (double)((const float*)a.x)[(size_t)t * d + j];
        ss += xv * xv;
    }
    red[tid] = ss;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) red[tid] += red[tid + o];
        __syncthreads();
    }
    const double den = sqrt(red[0] / (double)d + (double)a.eps);
    for (int j = tid; j < d; j += 256) {
        double xv = a.x_is_bf16 ? (double)bf16_to_f32(((const uint16_t*)a.x)[(size_t)t * d + j])
                                : (double)((const float*)a.x)[(size_t)t * d + j];
        double uv = a.fused ? (xv / den) * (double)a.gamma[j] : xv;
        float uf = a.act_bf16 ? bf16_to_f32(f64_to_bf16(uv)) : (float)uv;
        su[j] = uf;
        a.u[(size_t)t * d + j] = uf;
    }
    __syncthreads();
    for (int q = tid; q < d / 2; q += 256) {
        const int c = q >> 4, r = q & 15, i = r >> 2, p = r & 3;
        const int e0 = 32 * c + 8 * i + p;
        const float v0 = su[e0], v1 = su[e0 + 4];
        const uint32_t h0 = f32_to_bf16(v0), h1 = f32_to_bf16(v1);
        a.u_pk[(size_t)t * (d / 2) + q] = h0 | (h1 << 16);
        if (a.u_pk_lo) {
            const uint32_t l0 = f32_to_bf16(v0 - bf16_to_f32(h0)), l1 = f32_to_bf16(v1 - bf16_to_f32(h1));
            a.u_pk_lo[(size_t)t * (d / 2) + q] = l0 | (l1 << 16);
        }
    }
    for (int c = tid; c < d / 32; c += 256) {
        float sh = 0.f, sl = 0.f;
        for (int j = 0; j < 32; ++j) {
            const float v = su[32 * c + j];
            const float hv = bf16_to_f32(f32_to_bf16(v));
            sh += hv;
            sl += bf16_to_f32(f32_to_bf16(v - hv));
        }
        a.usum[(size_t)t * (d / 32) + c] = sh;
        if (a.usum_lo) a.usum_lo[(size_t)t * (d / 32) + c] = sl;
    }
}

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_prologue, dim3(a.n_tok), dim3(256), a.d * sizeof(float), s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16-weight GEMVs on u, accumulated in fp64 (bf16 x fp32 products are exact
// in fp64), followed by top-k and renormalised softmax in the last block.
// Virtual row space: [router E | head En | lora_a r | shared gate 1].
// ---------------------------------------------------------------------------
constexpr int kRouteRowsPerBlock = 16;   // 4 waves x 4 rows

__global__ void __launch_bounds__(256) k_route(RouteArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nr_router = a.router ? a.E : 0;
    const int nr_head = a.head ? a.En : 0;
    const int nb_router = (nr_router + kRouteRowsPerBlock - 1) / kRouteRowsPerBlock;
    const int nb_head = (nr_head + kRouteRowsPerBlock - 1) / kRouteRowsPerBlock;
    const int nr_misc = (a.lora_a ? a.r : 0) + (a.sgate_w ? 1 : 0);
    int job, row0, nrows;
    if ((int)blockIdx.x < nb_router) { job = 0; row0 = blockIdx.x * kRouteRowsPerBlock; nrows = nr_router; }
    else if ((int)blockIdx.x < nb_router + nb_head) { job = 1; row0 = (blockIdx.x - nb_router) * kRouteRowsPerBlock; nrows = nr_head; }
    else { job = 2; row0 = (blockIdx.x - nb_router - nb_head) * kRouteRowsPerBlock; nrows = nr_misc; }
    const int d = a.d;
    for (int rr = 0; rr < kRouteRowsPerBlock / 4; ++rr) {
        const int row = row0 + wave * (kRouteRowsPerBlock / 4) + rr;
        if (row >= nrows) break;
        const uint16_t* w;
        if (job == 0) w = a.router + (size_t)row * d;
        else if (job == 1) w = a.head + (size_t)row * d;
        else w = (a.lora_a && row < a.r) ? a.lora_a + (size_t)row * d : a.sgate_w;
        for (int t = 0; t < a.n_tok; ++t) {
            if (job == 0 && a.route_idx && a.route_idx[(size_t)t * a.k] >= 0) continue;
            const float* u = a.u + (size_t)t * d;
            double acc = 0.0;
            for (int j0 = lane * 8; j0 < d; j0 += 512) {
                const u32x4 wv = *(const u32x4*)(w + j0);
                const float4 u0 = *(const float4*)(u + j0);
                const float4 u1 = *(const float4*)(u + j0 + 4);
                acc += (double)bf16_to_f32(wv.x & 0xFFFF) * (double)u0.x;
                acc += (double)bf16_to_f32(wv.x >> 16) * (double)u0.y;
                acc += (double)bf16_to_f32(wv.y & 0xFFFF) * (double)u0.z;
                acc += (double)bf16_to_f32(wv.y >> 16) * (double)u0.w;
                acc += (double)bf16_to_f32(wv.z & 0xFFFF) * (double)u1.x;
                acc += (double)bf16_to_f32(wv.z >> 16) * (double)u1.y;
                acc += (double)bf16_to_f32(wv.w & 0xFFFF) * (double)u1.z;
                acc += (double)bf16_to_f32(wv.w >> 16) * (double)u1.w;
            }
            acc = group_sum(acc, 64);
            if (lane == 0) {
                if (job == 0) st_dev(a.logits_r + (size_t)t * a.E + row, acc);
                else if (job == 1) st_dev(a.logits_h + (size_t)t * a.En + row, acc);
                else if (a.lora_a && row < a.r) a.au[(size_t)t * a.r + row] = (float)acc;
                else a.sgate[t] = (float)(1.0 / (1.0 + exp(-acc)));
            }
        }
    }
    if (job == 2) return;
    // last block of the job computes the top-k for every token
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ int is_last;
    if (threadIdx.x == 0) {
        const unsigned total = job == 0 ? nb_router : nb_head;
        const unsigned old = __hip_atomic_fetch_add(a.counters + job, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = old == total - 1;
        if (is_last) __hip_atomic_store(a.counters + job, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!is_last) return;
    if (job == 0)
        topk_rows(true, a.logits_r, a.E, a.k, a.n_tok, a.router_bias, nullptr, nullptr, nullptr, nullptr,
                  a.route_idx, a.k, a.self_idx, a.self_w);
    else
        topk_rows(true, a.logits_h, a.En, a.kn, a.n_tok, a.head_bias, a.hist_cur_m, a.hist_cur, a.hist_prev_m,
                  a.hist_prev, nullptr, a.kn, a.pred_idx, a.pred_w);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
    const int nb_router = a.router ? (a.E + kRouteRowsPerBlock - 1) / kRouteRowsPerBlock : 0;
    const int nb_head = a.head ? (a.En + kRouteRowsPerBlock - 1) / kRouteRowsPerBlock : 0;
    const int nr_misc = (a.lora_a ? a.r : 0) + (a.sgate_w ? 1 : 0);
    const int nb_misc = (nr_misc + kRouteRowsPerBlock - 1) / kRouteRowsPerBlock;
    const int nb = nb_router + nb_head + nb_misc;
    if (nb == 0) return hipSuccess;
    hipLaunchKernelGGL(k_route, dim3(nb), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Token to expert sort/permute: keys (expert << 20 | assignment) sorted with
// a bitonic network in LDS; segments give the active experts (ascending),
// their offsets, and the assignment permutation.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) k_sort(SortArgs a) {
    extern __shared__ uint32_t keys[];
    __shared__ int wsum[16];
    __shared__ int tot;
    const int n = a.n_tok * a.k;
    int np2 = 1;
    while (np2 < n) np2 <<= 1;
    const int tid = threadIdx.x;
    for (int i = tid; i < np2; i += 1024) {
        uint32_t key = 0xFFFFFFFFu;
        if (i < n) {
            const int t = i / a.k;
            const bool self = !a.route_idx || a.route_idx[(size_t)t * a.k] < 0;
            int e = self ? a.self_idx[i] : a.route_idx[i];
            const float w = self ? a.self_w[i] : a.route_w[i];
            if (e < 0 || e >= a.E) { set_err(a.err, ERR_BAD_INDEX); e = -1; }
            a.used_idx[i] = e; a.used_w[i] = w;
            if (a.user_used_idx) a.user_used_idx[i] = e;
            if (a.user_used_w) a.user_used_w[i] = w;
            if (e >= 0) key = ((uint32_t)e << 20) | (uint32_t)i;
        }
        keys[i] = key;
    }
    __syncthreads();
    for (int size = 2; size <= np2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < np2 / 2; i += 1024) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const uint32_t x = keys[lo], y = keys[hi];
                if ((x > y) == up) { keys[lo] = y; keys[hi] = x; }
            }
            __syncthreads();
        }
    }
    // segment starts -> active list
    const int per = (n + 1023) / 1024;
    const int i0 = tid * per, i1 = min(n, i0 + per);
    int cnt = 0;
    for (int i = i0; i < i1; ++i) {
        const uint32_t key = keys[i];
        if (key == 0xFFFFFFFFu) break;
        a.perm[i] = (int32_t)(key & 0xFFFFFu);
        if (i == 0 || (keys[i - 1] >> 20) != (key >> 20)) ++cnt;
    }
    // block exclusive scan of cnt
    int incl = cnt;
    const int lane = tid & 63, wave = tid >> 6;
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int w = 0; w < 16; ++w) { const int v = wsum[w]; wsum[w] = acc; acc += v; }
        tot = acc;
    }
    __syncthreads();
    int pos = wsum[wave] + incl - cnt;
    int nvalid_local = 0;
    for (int i = i0; i < i1; ++i) {
        const uint32_t key = keys[i];
        if (key == 0xFFFFFFFFu) break;
        ++nvalid_local;
        if (i == 0 || (keys[i - 1] >> 20) != (key >> 20)) {
            a.active[pos] = (int32_t)(key >> 20);
            a.act_off[pos] = i;
            ++pos;
        }
    }
    // number of valid keys: first invalid position
    __shared__ int nvalid;
    if (tid == 0) nvalid = n;
    __syncthreads();
    for (int i = tid; i < n; i += 1024)
        if (keys[i] == 0xFFFFFFFFu && (i == 0 || keys[i - 1] != 0xFFFFFFFFu)) nvalid = i;
    __syncthreads();
    if (tid == 0) {
        a.act_off[tot] = nvalid;
        a.meta[0] = tot;
        a.meta[1] = nvalid;
    }
    (void)nvalid_local;
}

hipError_t launch_sort(const SortArgs& a, hipStream_t s) {
    int n = a.n_tok * a.k, np2 = 1;
    while (np2 < n) np2 <<= 1;
    hipLaunchKernelGGL(k_sort, dim3(1), dim3(1024), np2 * sizeof(uint32_t), s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Expert blob resolution (slot table) with the staging check.
// ---------------------------------------------------------------------------
__device__ __forceinline__ const uint8_t* resolve_expert(const ExpertView& ev, int e, int32_t* err) {
    if (!ev.slot_of) return ev.base + (size_t)e * ev.blob;
    const int s = ev.slot_of[e];
    if (s < 0 || (ev.slot_tag && ev.slot_tag[s] != e)) { set_err(err, ERR_NOT_STAGED); return nullptr; }
    return ev.base + (size_t)s * ev.blob;
}
__device__ __forceinline__ const uint8_t* resolve_shared(const ExpertView& ev, int32_t* err) {
    if (!ev.shared) return nullptr;
    if (ev.shared_tag && *ev.shared_tag != ev.E) { set_err(err, ERR_NOT_STAGED); return nullptr; }
    return ev.shared;
}

// ---------------------------------------------------------------------------
// Gate/up grouped GEMV + SwiGLU. One block = 4 waves; a wave covers RPW rows
// per pass (LPR lanes per row, 32 K-elements = 16 bytes per lane and chunk).
// int4 codes are expanded to bf16 (128 + q) pairs and multiplied with the
// bf16 activations by v_dot2_f32_bf16; the 64-group affine (s, b) is applied
// per lane chunk: sum((s q + b) u) = s * sum((128 + q) u) + (b - 128 s) * sum(u).
// ---------------------------------------------------------------------------
constexpr int kGateupRowsPerBlock = 16;

__device__ __forceinline__ float chunk_dot(const u32x4 w, const uint32_t* up, float acc) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int p = 0; p < 4; ++p) acc = dot2_bf16(nib_pair_bf16(ws[i], p), up[4 * i + p], acc);
    return acc;
}

__global__ void __launch_bounds__(256) k_gateup(GemvArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = a.d;
    const int nchunk = d / 32;
    const int LPR = nchunk < 64 ? nchunk : 64;
    const int RPW = 64 / LPR;
    const int CPL = nchunk / LPR;
    const int f_routed = a.f;
    const int bpe = (f_routed + kGateupRowsPerBlock - 1) / kGateupRowsPerBlock;
    const int n_routed_blocks = a.max_active * bpe;
    int rb, f, pos0, pos1;
    bool shared;
    const uint8_t* blob;
    int e = -1;
    if ((int)blockIdx.x < n_routed_blocks) {
        const int ai = blockIdx.x / bpe;
        rb = blockIdx.x % bpe;
        if (ai >= a.meta[0]) return;
        e = a.active[ai];
        pos0 = a.act_off[ai]; pos1 = a.act_off[ai + 1];
        shared = false; f = a.f;
        blob = resolve_expert(a.ev, e, a.err);
    } else {
        rb = blockIdx.x - n_routed_blocks;
        shared = true; f = a.fs; pos0 = 0; pos1 = a.n_tok;
        blob = resolve_shared(a.ev, a.err);
    }
    const BlobLayout L = BlobLayout::make(d, f);
    const int rows_per_wave = kGateupRowsPerBlock / 4;
    for (int pass = 0; pass < rows_per_wave; pass += RPW) {
        const int row = rb * kGateupRowsPerBlock + wave * rows_per_wave + pass + lane / LPR;
        const bool valid = row < f && (pass + lane / LPR) < rows_per_wave;
        const int c0 = lane % LPR;
        u32x4 wg[8], wu[8];
        uint32_t sbg[8], sbu[8];
        if (valid && blob) {
            for (int m = 0; m < CPL; ++m) {
                const int c = c0 + LPR * m;
                wg[m] = *(const u32x4*)(blob + L.gate_q + (size_t)row * (d / 2) + c * 16);
                wu[m] = *(const u32x4*)(blob + L.up_q + (size_t)row * (d / 2) + c * 16);
                sbg[m] = *(const uint32_t*)(blob + L.gate_sb + ((size_t)row * (d / 64) + c / 2) * 4);
                sbu[m] = *(const uint32_t*)(blob + L.up_sb + ((size_t)row * (d / 64) + c / 2) * 4);
            }
        }
        for (int pos = pos0; pos < pos1; ++pos) {
            const int t = shared ? pos : a.perm[pos] / a.k;
            float ga = 0.f, ua = 0.f;
            if (valid && blob) {
                for (int m = 0; m < CPL; ++m) {
                    const int c = c0 + LPR * m;
                    const uint32_t* up = a.u_pk + (size_t)t * (d / 2) + c * 16;
                    uint32_t uv[16];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const u32x4 v = *(const u32x4*)(up + 4 * q);
                        uv[4 * q] = v.x; uv[4 * q + 1] = v.y; uv[4 * q + 2] = v.z; uv[4 * q + 3] = v.w;
                    }
                    float accg = chunk_dot(wg[m], uv, 0.f);
                    float accu = chunk_dot(wu[m], uv, 0.f);
                    float usum = a.usum[(size_t)t * nchunk + c];
                    if (a.u_pk_lo) {
                        const uint32_t* ul = a.u_pk_lo + (size_t)t * (d / 2) + c * 16;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const u32x4 v = *(const u32x4*)(ul + 4 * q);
                            uv[4 * q] = v.x; uv[4 * q + 1] = v.y; uv[4 * q + 2] = v.z; uv[4 * q + 3] = v.w;
                        }
                        accg = chunk_dot(wg[m], uv, accg);
                        accu = chunk_dot(wu[m], uv, accu);
                        usum += a.usum_lo[(size_t)t * nchunk + c];
                    }
                    const float sg = f16_to_f32(sbg[m] & 0xFFFF), bg = f16_to_f32(sbg[m] >> 16);
                    const float su = f16_to_f32(sbu[m] & 0xFFFF), bu = f16_to_f32(sbu[m] >> 16);
                    ga += sg * accg + (bg - 128.f * sg) * usum;
                    ua += su * accu + (bu - 128.f * su) * usum;
                }
            }
            ga = group_sum(ga, LPR);
            ua = group_sum(ua, LPR);
            if (valid && c0 == 0) {
                const float hv = blob ? silu_f32(ga) * ua : 0.f;
                if (shared) a.hs[(size_t)t * f + row] = hv;
                else a.h[(size_t)pos * f + row] = hv;
            }
        }
    }
}

hipError_t launch_gateup(const GemvArgs& a, hipStream_t s) {
    const int bpe = (a.f + kGateupRowsPerBlock - 1) / kGateupRowsPerBlock;
    const int bsh = a.fs ? (a.fs + kGateupRowsPerBlock - 1) / kGateupRowsPerBlock : 0;
    const int nb = a.max_active * bpe + bsh;
    hipLaunchKernelGGL(k_gateup, dim3(nb), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Down GEMV + routing-weighted combine + sigmoid-gated shared expert + LoRA
// (alpha/r) B (A u) + residual. Each wave owns rows; it walks the active
// experts in ascending id, then the shared expert, so every output element is
// accumulated in one fixed order (run-to-run identical).
// ---------------------------------------------------------------------------
constexpr int kDownRowsPerBlock = 16;

__device__ __forceinline__ void down_chunk(const u32x4 w, const float* hp, float& accq, float& hsum) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 h0 = *(const float4*)(hp + 8 * i);
        const float4 h1 = *(const float4*)(hp + 8 * i + 4);
        const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            accq += (float)((ws[i] >> (4 * n)) & 0xFu) * hv[n];
            hsum += hv[n];
        }
    }
}

__global__ void __launch_bounds__(256) k_down(GemvArgs a) {
    extern __shared__ float yacc[];          // [n_tok][kDownRowsPerBlock]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = a.d;
    const int row_base = blockIdx.x * kDownRowsPerBlock;
    for (int i = threadIdx.x; i < a.n_tok * kDownRowsPerBlock; i += 256) yacc[i] = 0.f;
    __syncthreads();
    const int rows_per_wave = kDownRowsPerBlock / 4;
    const int n_active = a.meta[0];
    for (int ai = 0; ai <= n_active; ++ai) {
        const bool shared = ai == n_active;
        int f, pos0, pos1;
        const uint8_t* blob;
        if (!shared) {
            blob = resolve_expert(a.ev, a.active[ai], a.err);
            f = a.f; pos0 = a.act_off[ai]; pos1 = a.act_off[ai + 1];
        } else {
            if (!a.fs) break;
            blob = resolve_shared(a.ev, a.err);
            f = a.fs; pos0 = 0; pos1 = a.n_tok;
        }
        if (!blob) continue;
        const BlobLayout L = BlobLayout::make(d, f);
        const int nchunk = f / 32;
        const int LPR = nchunk < 64 ? nchunk : 64;
        const int RPW = 64 / LPR;
        const int CPL = nchunk / LPR;
        for (int pass = 0; pass < rows_per_wave; pass += RPW) {
            const int lr = wave * rows_per_wave + pass + lane / LPR;
            const int row = row_base + lr;
            const bool valid = row < d && (pass + lane / LPR) < rows_per_wave;
            const int c0 = lane % LPR;
            u32x4 wd[16];
            uint32_t sb[16];
            if (valid) {
                for (int m = 0; m < CPL; ++m) {
                    const int c = c0 + LPR * m;
                    wd[m] = *(const u32x4*)(blob + L.down_q + (size_t)row * (f / 2) + c * 16);
                    sb[m] = *(const uint32_t*)(blob + L.down_sb + ((size_t)row * (f / 64) + c / 2) * 4);
                }
            }
            for (int pos = pos0; pos < pos1; ++pos) {
                int t; float wgt; const float* hrow;
                if (shared) { t = pos; wgt = a.sgate ? a.sgate[t] : 1.f; hrow = a.hs + (size_t)t * f; }
                else { const int id = a.perm[pos]; t = id / a.k; wgt = a.used_w[id]; hrow = a.h + (size_t)pos * f; }
                float o = 0.f;
                if (valid) {
                    for (int m = 0; m < CPL; ++m) {
                        const int c = c0 + LPR * m;
                        float accq = 0.f, hsum = 0.f;
                        down_chunk(wd[m], hrow + 32 * c, accq, hsum);
                        o += f16_to_f32(sb[m] & 0xFFFF) * accq + f16_to_f32(sb[m] >> 16) * hsum;
                    }
                }
                o = group_sum(o, LPR);
                if (valid && c0 == 0) yacc[t * kDownRowsPerBlock + lr] += wgt * o;
            }
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < a.n_tok * kDownRowsPerBlock; i += 256) {
        const int t = i / kDownRowsPerBlock, lr = i % kDownRowsPerBlock, row = row_base + lr;
        if (row >= d) continue;
        float y = yacc[i];
        if (a.lora_b && a.r) {
            float l = 0.f;
            for (int q = 0; q < a.r; ++q) l += bf16_to_f32(a.lora_b[(size_t)row * a.r + q]) * a.au[(size_t)t * a.r + q];
            y += a.lora_scale * l;
        }
        if (a.fused) y = a.x[(size_t)t * d + row] + y;
        a.y[(size_t)t * d + row] = y;
    }
}

hipError_t launch_down(const GemvArgs& a, hipStream_t s) {
    const int nb = (a.d + kDownRowsPerBlock - 1) / kDownRowsPerBlock;
    hipLaunchKernelGGL(k_down, dim3(nb), dim3(256), a.n_tok * kDownRowsPerBlock * sizeof(float), s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Slot-table update after staging copies (queued on the copy stream).
// ---------------------------------------------------------------------------
__global__ void k_slot_update(int32_t* slot_of, int32_t* slot_tag, SlotUpdate u) {
    if (threadIdx.x != 0) return;
    for (int i = 0; i < u.n; ++i)
        if (u.old_e[i] >= 0 && slot_of[u.old_e[i]] == u.slot[i]) slot_of[u.old_e[i]] = -1;
    for (int i = 0; i < u.n; ++i) {
        slot_of[u.new_e[i]] = u.slot[i];
        slot_tag[u.slot[i]] = u.new_e[i];
    }
    if (u.shared_tag >= 0) slot_tag[u.shared_slot] = u.shared_tag;
}

hipError_t launch_slot_update(int32_t* slot_of, int32_t* slot_tag, const SlotUpdate& u, hipStream_t s) {
    hipLaunchKernelGGL(k_slot_update, dim3(1), dim3(64), 0, s, slot_of, slot_tag, u);
    return hipGetLastError();
}

}  // namespace moe

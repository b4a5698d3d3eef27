// Decode-path kernels for gfx950: prologue, bf16 GEMVs with top-k, token to
// expert sort/permute, and the int4 grouped GEMVs (gate/up + SwiGLU, down +
// combine + shared expert + LoRA + residual).
#include "dec_common.h"
#include "moe_internal.h"
#include "topk.h"

namespace moe {

// ---------------------------------------------------------------------------
// Prologue: block input u of every token.
// Fused: u = x / sqrt(mean(x^2) + eps) * gamma evaluated in fp64 and rounded
// once to the activation dtype (RMSNorm prologue of the head input: the head
// reads the post-norm hidden state -- reading guide, Method, prerouter head).
// Writes the GEMV-ordered bf16 pairs (and the lo parts for fp32 activations)
// and the per-32-chunk sums used by the int4 dot products; with u_frag, the
// same pairs again in MFMA fragment order for the routing GEMM: per 16
// tokens and 32 elements one 1 KB block, whose 16 bytes at 16 l are the
// 8 elements 8 (l / 16) .. of token l mod 16. Blocks are dealt to the 8 XCDs
// round robin, so block b takes token (b mod 8) * per + b / 8 with per a
// multiple of 8: the 8 tokens that share a line of u_frag are written on one
// XCD, and their lines reach memory whole.
// GEMV order of a 32-element chunk c: dword 4*i + p holds elements
// (32c + 8i + p, 32c + 8i + p + 4), matching the nibble pairs that one
// masked shift of a packed dword yields.
// ---------------------------------------------------------------------------
constexpr int kProPieces = 4;                 // 8-element pieces per thread: d <= 8192
__global__ void __launch_bounds__(256) k_prologue(PrologueArgs a) {
    __shared__ double red[4];
    const int per = (((a.n_tok + 7) / 8) + 7) / 8 * 8;
    const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (t >= a.n_tok) return;                 // the grid is 8 per blocks
    const int d = a.d, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // thread tid takes the 8-element pieces tid, tid + 256, ... (at most
    // kProPieces); piece pc is (chunk pc / 4, sub-block pc % 4), whose four
    // pairs are dwords 4 pc .. + 3. x and gamma are loaded once, together.
    float xv[kProPieces][8], gv[kProPieces][8];
#pragma unroll
    for (int j = 0; j < kProPieces; ++j) {
        const int pc = tid + 256 * j;
        if (pc >= d / 8) break;
        if (a.x_is_bf16) {
            const u32x4 w = *(const u32x4*)((const uint16_t*)a.x + (size_t)t * d + 8 * pc);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xv[j][2 * i] = bf16_to_f32(ws[i] & 0xFFFF);
                xv[j][2 * i + 1] = bf16_to_f32(ws[i] >> 16);
            }
        } else {
            const float4 x0 = *(const float4*)((const float*)a.x + (size_t)t * d + 8 * pc);
            const float4 x1 = *(const float4*)((const float*)a.x + (size_t)t * d + 8 * pc + 4);
            xv[j][0] = x0.x; xv[j][1] = x0.y; xv[j][2] = x0.z; xv[j][3] = x0.w;
            xv[j][4] = x1.x; xv[j][5] = x1.y; xv[j][6] = x1.z; xv[j][7] = x1.w;
        }
        if (a.fused) {
            const float4 g0 = *(const float4*)(a.gamma + 8 * pc), g1 = *(const float4*)(a.gamma + 8 * pc + 4);
            gv[j][0] = g0.x; gv[j][1] = g0.y; gv[j][2] = g0.z; gv[j][3] = g0.w;
            gv[j][4] = g1.x; gv[j][5] = g1.y; gv[j][6] = g1.z; gv[j][7] = g1.w;
        }
    }
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < kProPieces; ++j) {
        if (tid + 256 * j >= d / 8) break;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += (double)xv[j][i] * (double)xv[j][i];
    }
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const double den = sqrt((red[0] + red[1] + red[2] + red[3]) / (double)d + (double)a.eps);
#pragma unroll
    for (int j = 0; j < kProPieces; ++j) {
        const int pc = tid + 256 * j;
        if (pc >= d / 8) break;
        uint32_t hi[8], lo[8];
        float sh = 0.f, sl = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double v = (double)xv[j][i];
            const double uv = a.fused ? (v / den) * (double)gv[j][i] : v;
            const float uf = a.act_bf16 ? bf16_to_f32(f64_to_bf16(uv)) : (float)uv;
            hi[i] = f32_to_bf16(uf);
            lo[i] = f32_to_bf16(uf - bf16_to_f32(hi[i]));
            sh += bf16_to_f32(hi[i]);
            sl += bf16_to_f32(lo[i]);
        }
        const u32x4 hv = u32x4{hi[0] | (hi[4] << 16), hi[1] | (hi[5] << 16), hi[2] | (hi[6] << 16), hi[3] | (hi[7] << 16)};
        *(u32x4*)(a.u_pk + (size_t)t * (d / 2) + 4 * pc) = hv;
        if (a.u_pk_lo)
            *(u32x4*)(a.u_pk_lo + (size_t)t * (d / 2) + 4 * pc) =
                u32x4{lo[0] | (lo[4] << 16), lo[1] | (lo[5] << 16), lo[2] | (lo[6] << 16), lo[3] | (lo[7] << 16)};
        if (a.u_frag)
            // block (t / 16, pc / 4), lane 16 (pc mod 4) + t mod 16
            *(u32x4*)(a.u_frag + ((size_t)(t >> 4) * (d / 32) + (pc >> 2)) * 256 + ((pc & 3) * 16 + (t & 15)) * 4) = hv;
        // the chunk's 4 pieces are 4 consecutive lanes
        sh += __shfl_xor(sh, 1, 64);
        sh += __shfl_xor(sh, 2, 64);
        sl += __shfl_xor(sl, 1, 64);
        sl += __shfl_xor(sl, 2, 64);
        if ((pc & 3) == 0) {
            a.usum[(size_t)t * (d / 32) + pc / 4] = sh;
            if (a.usum_lo) a.usum_lo[(size_t)t * (d / 32) + pc / 4] = sl;
        }
    }
}

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s) {
    if (a.d % 64 || a.d > 8 * 256 * kProPieces || a.n_tok <= 0) return hipErrorInvalidValue;
    const int per = ((a.n_tok + 7) / 8 + 7) / 8 * 8;
    hipLaunchKernelGGL(k_prologue, dim3(8 * per), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Token to expert sort/permute: a stable counting sort in one block. Each of
// the 16 waves owns a contiguous chunk of the assignments and walks it 64 at
// a time; lanes holding the same expert find each other with one ballot per
// bit of the expert id, which gives each entry its rank among equal experts
// in the step and the step's count per expert. Pass 1 counts per (wave,
// expert); a scan over waves, then over experts, gives every (wave, expert)
// its first position; pass 2 repeats the walk and places the entries. The
// order is (expert, assignment id), and the active experts come out
// ascending with their offsets.
// ---------------------------------------------------------------------------
constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortPre = 2;                   // assignments per thread whose routing is loaded up front
constexpr int kSortMC = 4;                    // 64-assignment steps per wave whose expert matches pass 2 reuses

constexpr size_t kSortLdsMax = 159 * 1024;
// the assignments' experts stay in LDS between the passes when they fit
__host__ __device__ inline bool sort_cache_e(int n, int E) {
    return ((size_t)(kSortWaves + 1) * E + n) * sizeof(int) <= kSortLdsMax;
}
size_t sort_lds_bytes(int n, int E) {
    return ((size_t)(kSortWaves + 1) * E + (sort_cache_e(n, E) ? n : 0)) * sizeof(int);
}

// lanes (of the valid ones) whose expert equals this lane's; nbits covers E
__device__ __forceinline__ unsigned long long match_expert(int e, bool valid, int nbits) {
    unsigned long long m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const unsigned long long bb = __ballot(valid && bit);
        m &= bit ? bb : ~bb;
    }
    return valid ? m : 0ull;
}

__device__ __forceinline__ void sort_body(const SortArgs& a) {
    extern __shared__ int sm[];
    const int n = a.n_tok * a.k, E = a.E;
    int* wcnt = sm;                          // [kSortWaves][E]: counts, then first positions
    int* cnt = sm + kSortWaves * E;          // [E] bucket sizes
    __shared__ int wsum[kSortWaves], wact[kSortWaves], wt16[kSortWaves], wt64[kSortWaves];
    __shared__ int tot_valid, tot_active, tot16, tot64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // up to 256 experts, four threads per expert (thread 4 e + q takes waves
    // 4 q .. 4 q + 3 of expert e) in the scan below; else one per expert
    const bool quad = 4 * E <= kSortThreads;
    const int my_e = quad ? tid >> 2 : tid;
    // blob of expert my_e for the tile records, loaded early
    int my_blob = -1;
    if ((a.tiles16 || a.tiles64) && a.resolve_blobs && my_e < E) {
        if (!a.ev.slot_of) my_blob = my_e;
        else {
            const int sl = a.ev.slot_of[my_e];
            my_blob = (sl < 0 || (a.ev.slot_tag && a.ev.slot_tag[sl] != my_e)) ? -1 : sl;
        }
    }
    int* se = sm + (kSortWaves + 1) * E;     // [n] experts of the assignments (when cache_e)
    const bool cache_e = sort_cache_e(n, E);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    for (int i = tid; i < kSortWaves * E; i += kSortThreads) wcnt[i] = 0;
    const bool own_topk = a.self_topk && a.route_idx;
    // Loads first, waits later. This thread's first kSortPre assignments: the
    // given routing entry and weight, the row's first entry (negative: the
    // row self-routes), and the self-routing result of an earlier launch.
    int pe[kSortPre], pf[kSortPre], ps[kSortPre];
    float pw[kSortPre], psw[kSortPre];
#pragma unroll
    for (int j = 0; j < kSortPre; ++j) {
        const int i = tid + kSortThreads * j;
        pe[j] = -1; pf[j] = -1; ps[j] = -1; pw[j] = 0.f; psw[j] = 0.f;
        if (i < n) {
            const int t = i / a.k;
            if (a.route_idx && t >= a.route_shift) {
                const size_t gi = (size_t)i - (size_t)a.route_shift * a.k;
                pe[j] = a.route_idx[gi];
                pw[j] = a.route_w[gi];
                pf[j] = a.route_idx[gi - (size_t)(i % a.k)];
            }
            if ((!own_topk || t < a.pre_rows) && a.self_idx) { ps[j] = a.self_idx[i]; psw[j] = a.self_w[i]; }
        }
    }
    // the first 64-row window's row entries for this wave's own top-k
    int wf0 = 0;
    if (own_topk) {
        const int t = wave * 64 + lane;
        if (t >= a.route_shift && t < a.n_tok) wf0 = a.route_idx[(size_t)(t - a.route_shift) * a.k];
    }
    auto place = [&](int i, int e, float w) {
        if (e < 0 || e >= E) { set_err(a.err, ERR_BAD_INDEX); e = -1; }
        a.used_idx[i] = e; a.used_w[i] = w;
        if (a.user_used_idx) a.user_used_idx[i] = e;
        if (a.user_used_w) a.user_used_w[i] = w;
        if (cache_e) se[i] = e;
    };
    if (own_topk) {
        // top-k of the self-routed rows, straight into the used routing (the
        // selection stays in lanes 0 .. k-1)
        auto own_row = [&](int tt) {
            TopkSel sel;
            if (E <= 64) sel = topk_row<1>(false, a.logits_r, E, a.k, tt, a.router_bias, nullptr, nullptr, nullptr, nullptr, a.used_idx, a.used_w);
            else if (E <= 128) sel = topk_row<2>(false, a.logits_r, E, a.k, tt, a.router_bias, nullptr, nullptr, nullptr, nullptr, a.used_idx, a.used_w);
            else sel = topk_row<4>(false, a.logits_r, E, a.k, tt, a.router_bias, nullptr, nullptr, nullptr, nullptr, a.used_idx, a.used_w);
            if (lane < a.k) {
                const int i = tt * a.k + lane;
                if (a.user_used_idx) a.user_used_idx[i] = sel.idx;
                if (a.user_used_w) a.user_used_w[i] = sel.w;
                if (cache_e) se[i] = sel.idx;
            }
        };
        // rows before the shift have no given routing: no read to wait for
        // (the first pre_rows of them came with the routing GEMM)
        const int nsh = min(a.route_shift, a.n_tok);
        for (int tt = a.pre_rows + wave; tt < nsh; tt += kSortWaves) own_row(tt);
        // the others: a wave checks 64 rows at a time and takes each
        // self-routed one in turn
        for (int base = wave * 64; base < a.n_tok; base += kSortThreads) {
            const int t = base + lane;
            int f = wf0;
            if (base != wave * 64) f = t >= a.route_shift && t < a.n_tok ? a.route_idx[(size_t)(t - a.route_shift) * a.k] : 0;
            unsigned long long m = __ballot(t >= a.route_shift && t < a.n_tok && f < 0);
            while (m) {
                const int tt = base + __ffsll((long long)m) - 1;
                m &= m - 1;
                own_row(tt);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kSortPre; ++j) {
        const int i = tid + kSortThreads * j;
        if (i >= n) break;
        const int t = i / a.k;
        const bool self = !a.route_idx || t < a.route_shift || pf[j] < 0;
        if (self && own_topk && t >= a.pre_rows) continue;      // written by the top-k above
        place(i, self ? ps[j] : pe[j], self ? psw[j] : pw[j]);
    }
    for (int i = tid + kSortThreads * kSortPre; i < n; i += kSortThreads) {
        const int t = i / a.k;
        const size_t gi = (size_t)i - (size_t)a.route_shift * a.k;   // the given routing's entry (t >= shift)
        const bool self = !a.route_idx || t < a.route_shift || a.route_idx[gi - (size_t)(i % a.k)] < 0;
        if (self && own_topk && t >= a.pre_rows) continue;      // written by the top-k above
        // (without self-routing results a self-routed row is a bad index)
        if (self) place(i, a.self_idx ? a.self_idx[i] : -1, a.self_idx ? a.self_w[i] : 0.f);
        else place(i, a.route_idx[gi], a.route_w[gi]);
    }
    __threadfence_block();
    __syncthreads();                         // the experts are read below by other threads
    const int chunk = ((n + kSortWaves - 1) / kSortWaves + 63) / 64 * 64;
    const int c0 = wave * chunk, c1 = min(n, c0 + chunk);
    const unsigned long long lt = (1ull << lane) - 1;
    // pass 1: counts per (wave, expert); the first kSortMC steps' matches
    // are kept for pass 2
    unsigned long long mcache[kSortMC];
    int ecache[kSortMC];
    for (int base = c0, it = 0; base < c1; base += 64, ++it) {
        const int i = base + lane;
        const int e = i < c1 ? (cache_e ? se[i] : a.used_idx[i]) : -1;
        const unsigned long long m = match_expert(e, e >= 0, nbits);
#pragma unroll
        for (int j = 0; j < kSortMC; ++j)
            if (it == j) { mcache[j] = m; ecache[j] = e; }
        if (m && (m & lt) == 0) wcnt[wave * E + e] += __popcll(m);
    }
    __syncthreads();
    // scan over waves per expert, then over experts
    static_assert(kSortWaves == 16, "four quarters of four waves");
    const int qq = tid & 3;                   // quad: this thread's quarter of the waves
    int qv[4] = {0, 0, 0, 0}, xs = 0;         // quad: counts of its waves, its quarter's offset in the expert
    const int per = (E + kSortThreads - 1) / kSortThreads;
    const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
    int c = 0, na = 0, n16 = 0, n64 = 0;
    if (quad) {
#pragma unroll
        for (int j = 0; j < 4; ++j) qv[j] = my_e < E ? wcnt[(4 * qq + j) * E + my_e] : 0;
        const int run = qv[0] + qv[1] + qv[2] + qv[3];
        int inc = run;                        // inclusive scan over the quad
        {
            const int t1 = __shfl_up(inc, 1, 4);
            if (qq >= 1) inc += t1;
            const int t2 = __shfl_up(inc, 2, 4);
            if (qq >= 2) inc += t2;
        }
        xs = inc - run;
        const int tot_e = __shfl(inc, (lane & ~3) | 3, 64);
        if (qq == 0) {
            c = tot_e;
            na = tot_e > 0;
            n16 = (tot_e + 15) >> 4;
            n64 = (tot_e + 63) >> 6;
            if (my_e < E) cnt[my_e] = tot_e;
        }
    } else {
        for (int e = e0; e < e1; ++e) {
            int run = 0;
            for (int w = 0; w < kSortWaves; ++w) {
                const int v = wcnt[w * E + e];
                wcnt[w * E + e] = run;
                run += v;
            }
            cnt[e] = run;
            c += run;
            na += run > 0;
            n16 += (run + 15) >> 4;
            n64 += (run + 63) >> 6;
        }
    }
    int ic = c, ia = na, i16 = n16, i64 = n64;
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(ic, o, 64), u = __shfl_up(ia, o, 64);
        const int x16 = __shfl_up(i16, o, 64), x64 = __shfl_up(i64, o, 64);
        if (lane >= o) { ic += v; ia += u; i16 += x16; i64 += x64; }
    }
    if (lane == 63) { wsum[wave] = ic; wact[wave] = ia; wt16[wave] = i16; wt64[wave] = i64; }
    __syncthreads();
    if (tid == 0) {
        int s1 = 0, s2 = 0, s3 = 0, s4 = 0;
        for (int w = 0; w < kSortWaves; ++w) {
            const int v = wsum[w], u = wact[w], x16 = wt16[w], x64 = wt64[w];
            wsum[w] = s1; wact[w] = s2; wt16[w] = s3; wt64[w] = s4;
            s1 += v; s2 += u; s3 += x16; s4 += x64;
        }
        tot_valid = s1; tot_active = s2; tot16 = s3; tot64 = s4;
    }
    __syncthreads();
    int o1 = wsum[wave] + ic - c, o2 = wact[wave] + ia - na;
    int q16 = wt16[wave] + i16 - n16, q64 = wt64[wave] + i64 - n64;
    // the tile records of expert e (my_blob belongs to it), first position o1
    auto expert_records = [&](int e, int ce, int o1e, int o2e, int q16e, int q64e) {
        a.active[o2e] = e;
        a.act_off[o2e] = o1e;
        if (a.tiles16 || a.tiles64) {
            if (my_blob < 0 && a.resolve_blobs) set_err(a.err, ERR_NOT_STAGED);
            if (a.tiles16)
                for (int i = 0; i * 16 < ce; ++i)
                    *(int4*)(a.tiles16 + 4 * (q16e + i)) = make_int4(o2e, o1e + 16 * i, min(16, ce - 16 * i), my_blob);
            if (a.tiles64)
                for (int i = 0; i * 64 < ce; ++i)
                    *(int4*)(a.tiles64 + 4 * (q64e + i)) = make_int4(o2e, o1e + 64 * i, min(64, ce - 64 * i), my_blob);
        }
    };
    if (quad) {
        // the expert's first position comes from its q = 0 thread
        const int base = __shfl(o1, lane & ~3, 64) + xs;
        if (my_e < E) {
            int run = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                wcnt[(4 * qq + j) * E + my_e] = base + run;
                run += qv[j];
            }
            if (qq == 0 && c > 0) expert_records(my_e, c, o1, o2, q16, q64);
        }
    } else {
        for (int e = e0; e < e1; ++e) {
            for (int w = 0; w < kSortWaves; ++w) wcnt[w * E + e] += o1;
            const int ce = cnt[e];
            if (ce > 0) {
                expert_records(e, ce, o1, o2, q16, q64);
                ++o2;
            }
            o1 += ce;
            q16 += (ce + 15) >> 4;
            q64 += (ce + 63) >> 6;
        }
    }
    if (a.tiles16 || a.tiles64) {
        // the shared expert's token tiles follow the routed ones
        int sblob = -1;
        if (a.fs && a.ev.shared && a.resolve_blobs) {
            if (a.ev.shared_tag && *a.ev.shared_tag != a.ev.E) { if (tid == 0) set_err(a.err, ERR_NOT_STAGED); }
            else sblob = -2;
        }
        const int ns16 = a.fs ? (a.n_tok + 15) / 16 : 0, ns64 = a.fs ? (a.n_tok + 63) / 64 : 0;
        if (a.tiles16)
            for (int i = tid; i < ns16; i += kSortThreads)
                *(int4*)(a.tiles16 + 4 * (tot16 + i)) = make_int4(-1, 16 * i, min(16, a.n_tok - 16 * i), sblob);
        if (a.tiles64)
            for (int i = tid; i < ns64; i += kSortThreads)
                *(int4*)(a.tiles64 + 4 * (tot64 + i)) = make_int4(-1, 64 * i, min(64, a.n_tok - 64 * i), sblob);
        if (tid == 0) {
            a.meta[2] = tot16 + ns16; a.meta[3] = tot16;
            a.meta[4] = tot64 + ns64; a.meta[5] = tot64;
        }
    }
    __syncthreads();
    // pass 2: place
    for (int base = c0, it = 0; base < c1; base += 64, ++it) {
        const int i = base + lane;
        int e = -1;
        unsigned long long m = 0;
        bool hit = false;
#pragma unroll
        for (int j = 0; j < kSortMC; ++j)
            if (it == j) { e = ecache[j]; m = mcache[j]; hit = true; }
        if (!hit) {
            e = i < c1 ? (cache_e ? se[i] : a.used_idx[i]) : -1;
            m = match_expert(e, e >= 0, nbits);
        }
        if (m) {
            a.perm[wcnt[wave * E + e] + __popcll(m & lt)] = i;
        }
        // every lane has read its first position; the group's leader advances it
        wave_lds_sync();
        if (m && (m & lt) == 0) wcnt[wave * E + e] += __popcll(m);
        wave_lds_sync();
    }
    if (tid == 0) {
        a.act_off[tot_active] = tot_valid;
        a.meta[0] = tot_active;
        a.meta[1] = tot_valid;
    }
}

__global__ void __launch_bounds__(kSortThreads) k_sort(SortArgs a) { sort_body(a); }

// The sorts of several layers' given routing in one launch: block b takes
// table entry b (a layer's fixed arguments) with the call's routing, used
// routing outputs and token count patched in (entry b's routing starts
// (b + 1) * per entries past the call's base: the stack's layers 1, 2, ...).
// No row may self-route here: a row whose first entry is negative is a bad
// index (the table has no self-routing results).
__global__ void __launch_bounds__(kSortThreads) k_sort_layers(const SortArgs* __restrict__ tab, SortCall c) {
    SortArgs a = tab[blockIdx.x];
    const size_t off = (size_t)(blockIdx.x + 1) * c.per;
    a.route_idx = c.route_idx + off;
    a.route_w = c.route_w + off;
    a.user_used_idx = c.used_idx ? c.used_idx + off : nullptr;
    a.user_used_w = c.used_w ? c.used_w + off : nullptr;
    a.n_tok = c.n_tok;
    if (!c.big) a.tiles64 = nullptr;
    sort_body(a);
}

hipError_t launch_sort_layers(const SortArgs* tab, int n_layers, int E, const SortCall& c, hipStream_t s) {
    const size_t lds = sort_lds_bytes((int)c.per, E);
    if (E > kSortThreads || lds > kSortLdsMax) return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        // above the default dynamic LDS limit: raise it to what this call needs
        static size_t raised = 0;
        if (lds > raised) {
            const hipError_t e =
                hipFuncSetAttribute((const void*)k_sort_layers, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            raised = lds;
        }
    }
    hipLaunchKernelGGL(k_sort_layers, dim3(n_layers), dim3(kSortThreads), lds, s, tab, c);
    return hipGetLastError();
}

hipError_t launch_sort(const SortArgs& a, hipStream_t s) {
    if (a.E > kSortThreads || (a.self_topk && a.E > kSortTopkMaxE)) return hipErrorInvalidValue;
    const size_t lds = sort_lds_bytes(a.n_tok * a.k, a.E);
    if (lds > 64 * 1024) {
        // above the default dynamic LDS limit: raise it to what this call needs
        static size_t raised = 0;
        if (lds > kSortLdsMax) return hipErrorInvalidValue;
        if (lds > raised) {
            const hipError_t e = hipFuncSetAttribute((const void*)k_sort, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            raised = lds;
        }
    }
    hipLaunchKernelGGL(k_sort, dim3(1), dim3(kSortThreads), lds, s, a);
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
// ---------------------------------------------------------------------------
// The head's MLP branch, after fc1's hidden-state part: kMlpTok tokens per
// block. For each token: a = a1 + fc1's one-hot columns of its current and
// previous routing (each distinct valid expert once) + bias, g = erf-GELU(a)
// in fp64 (LDS); then every thread takes logits rows e = tid, tid + 256, ...
// and adds W2[e] . g for the block's tokens (each W2 row is read once for
// all of them). bf16 weights times fp64 activations, fp64 sums.
// ---------------------------------------------------------------------------
constexpr int kMlpTok = 4;

__global__ void __launch_bounds__(256) k_head_mlp_out(HeadMlpArgs a) {
    __shared__ double g[kMlpTok][kMaxHeadHidden];
    __shared__ int ids[kMlpTok][2 * kMaxTopK];
    const int tid = threadIdx.x, t0 = blockIdx.x * kMlpTok;
    const int H1 = a.H1, En = a.En, kn = a.kn;
    const int nt = min(kMlpTok, a.n_tok - t0);
    if (tid < kMlpTok * 2 * kMaxTopK) {
        const int q = tid / (2 * kMaxTopK), i = tid % (2 * kMaxTopK);
        const int src = i / kMaxTopK, j = i % kMaxTopK;      // src 0: current, 1: previous
        const int32_t* H = src ? a.hp : a.hc;
        int e = -1;
        if (q < nt && j < kn && H) e = H[(size_t)(t0 + q) * kn + j];
        ids[q][i] = (e >= 0 && e < En) ? e : -1;
    }
    __syncthreads();
    for (int q = 0; q < nt; ++q) {
        const int t = t0 + q;
        for (int j = tid; j < H1; j += 256) {
            double v = a.a1[(size_t)t * H1 + j] + (a.b1 ? (double)a.b1[j] : 0.0);
            for (int src = 0; src < 2; ++src)
                for (int i = 0; i < kn; ++i) {
                    const int e = ids[q][src * kMaxTopK + i];
                    bool dup = false;
                    for (int i2 = 0; i2 < i; ++i2) dup |= ids[q][src * kMaxTopK + i2] == e;
                    if (e < 0 || dup) continue;
                    v += (double)bf16_to_f32(a.w1oh[(size_t)(src * En + e) * H1 + j]);
                }
            g[q][j] = 0.5 * v * (1.0 + erf(v * M_SQRT1_2));
        }
    }
    __syncthreads();
    for (int e = tid; e < En; e += 256) {
        const uint16_t* w = a.w2 + (size_t)e * H1;
        double acc[kMlpTok] = {};
        for (int j = 0; j < H1; j += 8) {
            const u32x4 wv = *(const u32x4*)(w + j);
            const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const double w0 = (double)bf16_to_f32(ws[i] & 0xFFFF), w1 = (double)bf16_to_f32(ws[i] >> 16);
#pragma unroll
                for (int q = 0; q < kMlpTok; ++q) acc[q] += w0 * g[q][j + 2 * i] + w1 * g[q][j + 2 * i + 1];
            }
        }
        for (int q = 0; q < nt; ++q) a.logits[(size_t)(t0 + q) * En + e] += acc[q];
    }
}

hipError_t launch_head_mlp_out(const HeadMlpArgs& a, hipStream_t s) {
    if (a.H1 <= 0 || a.H1 > kMaxHeadHidden || a.H1 % 8 || a.kn > kMaxTopK || a.n_tok <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_head_mlp_out, dim3((a.n_tok + kMlpTok - 1) / kMlpTok), dim3(256), 0, s, a);
    return hipGetLastError();
}

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

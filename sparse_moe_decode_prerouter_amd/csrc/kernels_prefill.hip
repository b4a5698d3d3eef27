// Prefill path: the token->expert assignments (sorted by expert) run as a
// grouped GEMM on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Work item = (expert, tile of up to 16 consecutive assignments of it), or a
// 16-token tile of the shared expert. In an MFMA the tokens are the M side,
// the weight rows the N side and the hidden dimension K:
//   A (16 tokens x 32 k): lane (m = l%16, piece i = l/16) holds the 8 bf16
//     values of piece i of a 32-element chunk, in the pair order (p, p+4)
//     that the prologue writes (u_pk);
//   B (32 k x 16 rows): lane (n = l%16, i) holds dword i of the chunk's
//     packed int4, expanded to (128 + q) bf16 pairs in the same order;
//   C (16 x 16 fp32): lane holds row n = l%16 for tokens 4*(l/16) + 0..3.
// int4 codes are exact in bf16 and the affine (s, b) of each 64-group is
// applied to a fresh accumulator per group:
//   sum((s q + b) u) = s * sum((128 + q) u) + (b - 128 s) * sum(u),
// with fp32 accumulation. The expert hidden state enters the down projection
// as bf16 hi + lo (two MFMAs), so no operand is rounded beyond the
// activation dtype.
#include "device_common.h"
#include "moe_internal.h"
#include "topk.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTileM = 16;        // assignments (tokens) per tile
constexpr int kMaxGroupsPf = 64;  // d / 64 <= 64

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

// (128 + q) bf16 pairs (p, p + 4), p = 0..3, of one packed int4 dword
__device__ __forceinline__ u32x4 nib4(uint32_t w) {
    u32x4 r;
    r.x = nib_pair_bf16(w, 0);
    r.y = nib_pair_bf16(w, 1);
    r.z = nib_pair_bf16(w, 2);
    r.w = nib_pair_bf16(w, 3);
    return r;
}

int prefill_max_tiles(int T, int K, int E) {
    const int nk = T * K;
    return (nk + kTileM - 1) / kTileM + (nk < E ? nk : E) + (T + kTileM - 1) / kTileM + 1;
}

// ---------------------------------------------------------------------------
// Tile list: entry = (slot + 1) << 16 | first assignment of the tile within
// the slot; slot -1 (code 0) is the shared expert with token tiles. meta[2]
// = number of tiles. One block.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) k_pf_tiles(PrefillArgs a) {
    __shared__ int wsum[16];
    __shared__ int total;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_active = a.g.meta[0];
    int cnt = 0;
    if (tid < n_active) cnt = (a.g.act_off[tid + 1] - a.g.act_off[tid] + kTileM - 1) / kTileM;
    int incl = cnt;
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int w = 0; w < 16; ++w) { const int v = wsum[w]; wsum[w] = acc; acc += v; }
        total = acc;
    }
    __syncthreads();
    const int start = wsum[wave] + incl - cnt;
    for (int i = 0; i < cnt; ++i) a.tiles[start + i] = ((uint32_t)(tid + 1) << 16) | (uint32_t)(i * kTileM);
    const int ns = a.g.fs ? (a.g.n_tok + kTileM - 1) / kTileM : 0;
    for (int i = tid; i < ns; i += 1024) a.tiles[total + i] = (uint32_t)(i * kTileM);
    if (tid == 0) a.meta_w[2] = total + ns;
}

struct PfItem {
    int slot;     // -1: shared expert
    int p0;       // first position (sorted assignment) or first token
    int M;        // rows of the tile (<= 16)
};

__device__ __forceinline__ PfItem pf_item(const PrefillArgs& a, int tile) {
    const uint32_t code = a.tiles[tile];
    PfItem it;
    it.slot = (int)(code >> 16) - 1;
    const int m0 = (int)(code & 0xFFFFu);
    if (it.slot < 0) {
        it.p0 = m0;
        it.M = min(kTileM, a.g.n_tok - m0);
    } else {
        it.p0 = a.g.act_off[it.slot] + m0;
        it.M = min(kTileM, a.g.act_off[it.slot + 1] - it.p0);
    }
    return it;
}

__device__ __forceinline__ const uint8_t* pf_blob(const GemvArgs& g, int slot) {
    const ExpertView& ev = g.ev;
    if (slot < 0) {
        if (!ev.shared) return nullptr;
        if (ev.shared_tag && *ev.shared_tag != ev.E) { set_err(g.err, ERR_NOT_STAGED); return nullptr; }
        return ev.shared;
    }
    const int e = g.active[slot];
    if (!ev.slot_of) return ev.base + (size_t)e * ev.blob;
    const int s = ev.slot_of[e];
    if (s < 0 || (ev.slot_tag && ev.slot_tag[s] != e)) { set_err(g.err, ERR_NOT_STAGED); return nullptr; }
    return ev.base + (size_t)s * ev.blob;
}

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU with LDS staging. Block = 16-token tile x kGuRows rows of
// W_g and of W_u (2 n-tiles per wave). The hidden dimension is walked in
// stages of 4 groups (256 elements): every 128-byte line (one row's int4 for
// the stage) is read by 8 consecutive threads as whole 16-byte pieces, and
// stored to LDS with piece p of line r at slot p ^ (r & 7), so the MFMA reads
// (8 bytes per lane, 16 rows per instruction) hit at most 2 lanes per bank
// group. The next stage is loaded into registers while the current one is
// multiplied.
// k-mapping inside a 64-group (8 pieces of 8 elements): MFMA q (0, 1) takes
// piece 2*pc + q from lane group pc, so every MFMA stays inside one group and
// its scale applies to the whole accumulator.
// ---------------------------------------------------------------------------
constexpr int kGuRows = 64;                   // rows of W_g (and of W_u) per block: one 16-row tile per wave
constexpr int kGuLines = 2 * kGuRows;         // int4 lines per stage
constexpr int kStageK = 256;                  // hidden elements per stage
constexpr int kARow = 512 + 16;               // LDS bytes per token row of a stage (padded)

template <bool LO>
struct GuLds {
    uint8_t b[kGuLines * 128];                // int4 lines, swizzled
    uint32_t sc[kGuLines][4];                 // (s, b) of the stage's 4 groups
    uint8_t a[kTileM * kARow];                // u_pk (hi) of the tile's tokens
    uint8_t al[LO ? kTileM * kARow : 16];     // lo part (f32 activations)
};

template <bool LO>
struct GuRegs {
    u32x4 b[kGuLines * 8 / 256];              // 8 pieces per thread
    u32x4 sc;                                 // one line's scales
    u32x4 a[2], al[2];                        // 2 pieces of the tokens' u
};

template <bool LO>
__device__ __forceinline__ void gu_stage_load(GuRegs<LO>& R, int st, const uint8_t* wb, const BlobLayout& L, int d,
                                              int f, int rb0, const int* tok, const PrefillArgs& a) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kGuLines * 8 / 256; ++i) {
        const int pi = tid + 256 * i, r = pi >> 3, ps = pi & 7, pg = ps ^ (r & 7);
        int row = (r < kGuRows ? r : r - kGuRows) + rb0;
        row = row < f ? row : f - 1;
        const uint8_t* base = wb + (r < kGuRows ? L.gate_q : L.up_q) + (size_t)row * (d / 2);
        R.b[i] = *(const u32x4*)(base + st * (kStageK / 2) + 16 * pg);
    }
    if (tid < kGuLines) {
        const int r = tid;                       // one line's scales per thread
        int row = (r < kGuRows ? r : r - kGuRows) + rb0;
        row = row < f ? row : f - 1;
        const uint8_t* sb = wb + (r < kGuRows ? L.gate_sb : L.up_sb) + (size_t)row * (d / 16);
        R.sc = *(const u32x4*)(sb + st * 16);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int pa = tid + 256 * i, m = pa >> 5, k = pa & 31;
        R.a[i] = *(const u32x4*)(a.g.u_pk + (size_t)tok[m] * (d / 2) + st * (kStageK / 2) + 4 * k);
        if (LO) R.al[i] = *(const u32x4*)(a.g.u_pk_lo + (size_t)tok[m] * (d / 2) + st * (kStageK / 2) + 4 * k);
    }
}

template <bool LO>
__device__ __forceinline__ void gu_stage_store(const GuRegs<LO>& R, GuLds<LO>& S) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kGuLines * 8 / 256; ++i) *(u32x4*)&S.b[(tid + 256 * i) * 16] = R.b[i];
    if (tid < kGuLines) *(u32x4*)&S.sc[tid][0] = R.sc;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int pa = tid + 256 * i, m = pa >> 5, k = pa & 31;
        *(u32x4*)&S.a[m * kARow + 16 * k] = R.a[i];
        if (LO) *(u32x4*)&S.al[m * kARow + 16 * k] = R.al[i];
    }
}

template <bool LO>
__device__ __forceinline__ u32x2 gu_b_read(const GuLds<LO>& S, int r, int q, int pc) {
    const int p = 2 * q + (pc >> 1);
    return *(const u32x2*)&S.b[r * 128 + ((p ^ (r & 7)) << 4) + ((pc & 1) << 3)];
}

template <bool LO>
__global__ void __launch_bounds__(256) k_pf_gateup(PrefillArgs a) {
    const GemvArgs& g = a.g;
    __shared__ __align__(16) GuLds<LO> S[2];
    __shared__ float us64[kTileM][kMaxGroupsPf + 1];
    __shared__ int tok[kTileM];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if ((int)blockIdx.x >= g.meta[2]) return;
    const PfItem it = pf_item(a, blockIdx.x);
    const bool shared = it.slot < 0;
    const int f = shared ? g.fs : g.f;
    const int rb0 = blockIdx.y * kGuRows;
    if (rb0 >= f || it.M <= 0) return;
    const uint8_t* blob = pf_blob(g, it.slot);
    const int d = g.d, G = d / 64, NS = d / kStageK;
    if (tid < kTileM) {
        const int p = it.p0 + (tid < it.M ? tid : it.M - 1);
        tok[tid] = shared ? p : g.perm[p] / g.k;
    }
    __syncthreads();
    const BlobLayout L = BlobLayout::make(d, f);
    const uint8_t* wb = blob ? blob : g.ev.base;
    GuRegs<LO> R;
    gu_stage_load<LO>(R, 0, wb, L, d, f, rb0, tok, a);
    for (int i = tid; i < kTileM * G; i += 256) {
        const int m = i / G, gg = i % G, t = tok[m];
        float s = g.usum[(size_t)t * (d / 32) + 2 * gg] + g.usum[(size_t)t * (d / 32) + 2 * gg + 1];
        if (LO) s += g.usum_lo[(size_t)t * (d / 32) + 2 * gg] + g.usum_lo[(size_t)t * (d / 32) + 2 * gg + 1];
        us64[m][gg] = s;
    }
    gu_stage_store<LO>(R, S[0]);
    __syncthreads();
    const int ml = lane & 15, pc = lane >> 4;
    constexpr int NJ = kGuRows / 64;          // 16-row tiles per wave
    f32x4 accg[NJ], accu[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) { accg[j] = f32x4{0.f, 0.f, 0.f, 0.f}; accu[j] = f32x4{0.f, 0.f, 0.f, 0.f}; }
    for (int st = 0; st < NS; ++st) {
        const GuLds<LO>& C = S[st & 1];
        if (st + 1 < NS) gu_stage_load<LO>(R, st + 1, wb, L, d, f, rb0, tok, a);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int gg = st * 4 + q;
            const u32x4 a0 = *(const u32x4*)&C.a[ml * kARow + q * 128 + pc * 32];
            const u32x4 a1 = *(const u32x4*)&C.a[ml * kARow + q * 128 + pc * 32 + 16];
            u32x4 l0 = {0, 0, 0, 0}, l1 = {0, 0, 0, 0};
            if (LO) {
                l0 = *(const u32x4*)&C.al[ml * kARow + q * 128 + pc * 32];
                l1 = *(const u32x4*)&C.al[ml * kARow + q * 128 + pc * 32 + 16];
            }
            float usm[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) usm[i] = us64[4 * pc + i][gg];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int rg = wave * (16 * NJ) + 16 * j + ml, ru = kGuRows + rg;
                const u32x2 wg = gu_b_read<LO>(C, rg, q, pc), wu = gu_b_read<LO>(C, ru, q, pc);
                const uint32_t sg = C.sc[rg][q], su = C.sc[ru][q];
                const u32x4 bg0 = nib4(wg.x), bg1 = nib4(wg.y), bu0 = nib4(wu.x), bu1 = nib4(wu.y);
                f32x4 pg = {0.f, 0.f, 0.f, 0.f}, pu = {0.f, 0.f, 0.f, 0.f};
                pg = mfma16(a0, bg0, pg);
                pu = mfma16(a0, bu0, pu);
                pg = mfma16(a1, bg1, pg);
                pu = mfma16(a1, bu1, pu);
                if (LO) {
                    pg = mfma16(l0, bg0, pg);
                    pu = mfma16(l0, bu0, pu);
                    pg = mfma16(l1, bg1, pg);
                    pu = mfma16(l1, bu1, pu);
                }
                const float s1 = f16_to_f32(sg & 0xFFFF), c1 = f16_to_f32(sg >> 16) - 128.f * s1;
                const float s2 = f16_to_f32(su & 0xFFFF), c2 = f16_to_f32(su >> 16) - 128.f * s2;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    accg[j][i] += s1 * pg[i] + c1 * usm[i];
                    accu[j][i] += s2 * pu[i] + c2 * usm[i];
                }
            }
        }
        if (st + 1 < NS) gu_stage_store<LO>(R, S[(st + 1) & 1]);
        __syncthreads();
    }
    const bool ok = blob != nullptr;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int n = rb0 + wave * (16 * NJ) + 16 * j + ml;
        if (n >= f) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * pc + i;
            if (m >= it.M) continue;
            const float hv = ok ? silu_f32(accg[j][i]) * accu[j][i] : 0.f;
            if (shared) g.hs[(size_t)(it.p0 + m) * f + n] = hv;
            else g.h[(size_t)(it.p0 + m) * f + n] = hv;
        }
    }
}

// ---------------------------------------------------------------------------
// Down projection with LDS staging (same scheme as gate/up). Block = 16
// positions x kDnRows rows of W_d; K = f walked in stages of 4 groups. A is
// the expert hidden state, staged as fp32 and split into bf16 hi + lo when
// read; its per-group sums (the b-term) come from the same values. Output:
// O[assignment][d] (routed) or O_s[token][d] (shared), unweighted.
// ---------------------------------------------------------------------------
constexpr int kDnRows = 128;
constexpr int kDnSub = 1;                    // 128-row sub-blocks per block (more measured slower)
constexpr int kHRow = kStageK * 4 + 16;      // LDS bytes per position row of a stage (padded)

struct DnLds {
    uint8_t b[kDnRows * 128];
    uint32_t sc[kDnRows][4];
    uint8_t h[kTileM * kHRow];
};

struct DnRegs {
    u32x4 b[kDnRows * 8 / 256];
    u32x4 sc;
    float4 h[kTileM * kStageK / 4 / 256];
};

__device__ __forceinline__ void dn_stage_load(DnRegs& R, int st, const uint8_t* wb, const BlobLayout& L, int d,
                                              int f, int rb0, const int* prow, const float* hbase) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kDnRows * 8 / 256; ++i) {
        const int pi = tid + 256 * i, r = pi >> 3, ps = pi & 7, pg = ps ^ (r & 7);
        int row = rb0 + r;
        row = row < d ? row : d - 1;
        R.b[i] = *(const u32x4*)(wb + L.down_q + (size_t)row * (f / 2) + st * (kStageK / 2) + 16 * pg);
    }
    if (tid < kDnRows) {
        int row = rb0 + tid;
        row = row < d ? row : d - 1;
        R.sc = *(const u32x4*)(wb + L.down_sb + (size_t)row * (f / 16) + st * 16);
    }
#pragma unroll
    for (int i = 0; i < kTileM * kStageK / 4 / 256; ++i) {
        const int pa = tid + 256 * i, m = pa / (kStageK / 4), k = pa % (kStageK / 4);
        R.h[i] = *(const float4*)(hbase + (size_t)prow[m] * f + st * kStageK + 4 * k);
    }
}

__device__ __forceinline__ void dn_stage_store(const DnRegs& R, DnLds& S) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kDnRows * 8 / 256; ++i) *(u32x4*)&S.b[(tid + 256 * i) * 16] = R.b[i];
    if (tid < kDnRows) *(u32x4*)&S.sc[tid][0] = R.sc;
#pragma unroll
    for (int i = 0; i < kTileM * kStageK / 4 / 256; ++i) {
        const int pa = tid + 256 * i, m = pa / (kStageK / 4), k = pa % (kStageK / 4);
        *(float4*)&S.h[m * kHRow + 16 * k] = R.h[i];
    }
}

__global__ void __launch_bounds__(256) k_pf_down(PrefillArgs a) {
    const GemvArgs& g = a.g;
    __shared__ __align__(16) DnLds S[2];
    __shared__ int prow[kTileM];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if ((int)blockIdx.x >= g.meta[2]) return;
    const PfItem it = pf_item(a, blockIdx.x);
    const bool shared = it.slot < 0;
    const int f = shared ? g.fs : g.f;
    const int d = g.d;
    const int rbb = blockIdx.y * kDnRows * kDnSub;           // block's first row
    if (rbb >= d || it.M <= 0) return;
    const uint8_t* blob = pf_blob(g, it.slot);
    const int NS = f / kStageK;
    const int nsub = min(kDnSub, (d - rbb + kDnRows - 1) / kDnRows);
    const int NZ = nsub * NS;                                 // stages over all sub-blocks
    const float* hbase = shared ? g.hs : g.h;
    if (tid < kTileM) prow[tid] = it.p0 + (tid < it.M ? tid : it.M - 1);
    __syncthreads();
    const BlobLayout L = BlobLayout::make(d, f);
    const uint8_t* wb = blob ? blob : g.ev.base;
    DnRegs R;
    dn_stage_load(R, 0, wb, L, d, f, rbb, prow, hbase);
    dn_stage_store(R, S[0]);
    __syncthreads();
    const int ml = lane & 15, pc = lane >> 4;
    constexpr int NJ = kDnRows / 64;
    const bool ok = blob != nullptr;
    f32x4 acc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < NZ; ++z) {
        const DnLds& C = S[z & 1];
        const int st = z % NS, rb0 = rbb + (z / NS) * kDnRows;
        if (z + 1 < NZ) dn_stage_load(R, (z + 1) % NS, wb, L, d, f, rbb + ((z + 1) / NS) * kDnRows, prow, hbase);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // this lane's 16 elements of group q: pieces 2pc, 2pc+1 of position ml
            float e[16];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float4 x = *(const float4*)&C.h[ml * kHRow + q * 256 + pc * 64 + 16 * v];
                e[4 * v] = x.x; e[4 * v + 1] = x.y; e[4 * v + 2] = x.z; e[4 * v + 3] = x.w;
            }
            u32x4 ahi[2], alo[2];
            float hs = 0.f;
#pragma unroll
            for (int pq = 0; pq < 2; ++pq) {
                uint32_t hi[8], lo[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    hi[i] = f32_to_bf16(e[8 * pq + i]);
                    lo[i] = f32_to_bf16(e[8 * pq + i] - bf16_to_f32(hi[i]));
                    hs += bf16_to_f32(hi[i]) + bf16_to_f32(lo[i]);
                }
                ahi[pq].x = hi[0] | (hi[4] << 16); ahi[pq].y = hi[1] | (hi[5] << 16);
                ahi[pq].z = hi[2] | (hi[6] << 16); ahi[pq].w = hi[3] | (hi[7] << 16);
                alo[pq].x = lo[0] | (lo[4] << 16); alo[pq].y = lo[1] | (lo[5] << 16);
                alo[pq].z = lo[2] | (lo[6] << 16); alo[pq].w = lo[3] | (lo[7] << 16);
            }
            // group sum for position ml, then the sums of the C rows 4pc..4pc+3
            hs += __shfl_xor(hs, 16, 64);
            hs += __shfl_xor(hs, 32, 64);
            float hsm[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) hsm[i] = __shfl(hs, 4 * pc + i, 64);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int r = wave * (16 * NJ) + 16 * j + ml;
                const int p = 2 * q + (pc >> 1);
                const u32x2 w = *(const u32x2*)&C.b[r * 128 + ((p ^ (r & 7)) << 4) + ((pc & 1) << 3)];
                const uint32_t sb = C.sc[r][q];
                const u32x4 b0 = nib4(w.x), b1 = nib4(w.y);
                f32x4 pp = {0.f, 0.f, 0.f, 0.f};
                pp = mfma16(ahi[0], b0, pp);
                pp = mfma16(ahi[1], b1, pp);
                pp = mfma16(alo[0], b0, pp);
                pp = mfma16(alo[1], b1, pp);
                const float sv = f16_to_f32(sb & 0xFFFF), cv = f16_to_f32(sb >> 16) - 128.f * sv;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[j][i] += sv * pp[i] + cv * hsm[i];
            }
        }
        if (st == NS - 1) {
            // sub-block done: write its rows, start the next one
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int n = rb0 + wave * (16 * NJ) + 16 * j + ml;
                if (n < d) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = 4 * pc + i;
                        if (m >= it.M) continue;
                        const float o = ok ? acc[j][i] : 0.f;
                        if (shared) a.obs[(size_t)(it.p0 + m) * d + n] = o;
                        else a.ob[(size_t)g.perm[it.p0 + m] * d + n] = o;
                    }
                }
                acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        if (z + 1 < NZ) dn_stage_store(R, S[(z + 1) & 1]);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Combine per (token, row): shared (gated), routed in routing order
// (weighted), LoRA B, residual.
// ---------------------------------------------------------------------------
constexpr int kCombTok = 8;

__global__ void __launch_bounds__(256) k_pf_combine(PrefillArgs a) {
    const GemvArgs& g = a.g;
    const int n = blockIdx.x * 256 + threadIdx.x, d = g.d;
    const int t0 = blockIdx.y * kCombTok;
    if (n >= d) return;
    const bool lora = g.lora_b && g.r;
    const bool lvec = lora && g.r % 8 == 0 && g.r <= 32;
    u32x4 lb[4];
    if (lvec)
#pragma unroll
        for (int c = 0; c < 4; ++c) lb[c] = *(const u32x4*)(g.lora_b + (size_t)n * g.r + 8 * (8 * c < g.r ? c : 0));
    for (int tt = 0; tt < kCombTok; ++tt) {
        const int t = t0 + tt;
        if (t >= g.n_tok) break;
        float y = 0.f;
        if (g.fs && g.ev.shared) y = (g.sgate ? g.sgate[t] : 1.f) * a.obs[(size_t)t * d + n];
        for (int j = 0; j < g.k; ++j) {
            const int aid = t * g.k + j;
            if (a.used_idx[aid] >= 0) y += a.used_w[aid] * a.ob[(size_t)aid * d + n];
        }
        if (lora) {
            float l = 0.f;
            const float* au = g.au + (size_t)t * g.r;
            if (lvec) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (8 * c >= g.r) break;
                    const uint32_t w[4] = {lb[c].x, lb[c].y, lb[c].z, lb[c].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        l += bf16_to_f32(w[i] & 0xFFFF) * au[8 * c + 2 * i];
                        l += bf16_to_f32(w[i] >> 16) * au[8 * c + 2 * i + 1];
                    }
                }
            } else {
                for (int q = 0; q < g.r; ++q) l += bf16_to_f32(g.lora_b[(size_t)n * g.r + q]) * au[q];
            }
            y += g.lora_scale * l;
        }
        if (g.fused) y += g.x[(size_t)t * d + n];
        g.y[(size_t)t * d + n] = y;
    }
}

// ---------------------------------------------------------------------------
// bf16-row GEMM on u for the routing side: rows [router E | head En | LoRA A
// r | shared gate 1] x tokens. bf16 x bf16 products are exact in fp32; each
// 32-wide k-step goes to a fresh fp32 accumulator and the steps are summed in
// fp64, so a logit carries the rounding of at most one 32-term fp32 sum per
// step. Grid: (16-row tiles, 64-token groups); wave w takes token tile w.
// B (weights) pairs are reordered to the (p, p + 4) order of u_pk.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 bf16_pairs_p4(u32x4 v) {
    u32x4 r;
    r.x = (v.x & 0xFFFFu) | (v.z << 16);
    r.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    r.z = (v.y & 0xFFFFu) | (v.w << 16);
    r.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return r;
}

__global__ void __launch_bounds__(256) k_route_mm(RouteMMArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ml = lane & 15, pc = lane >> 4;
    const int d = a.d, T = a.n_tok;
    const int nr_router = a.router ? a.E : 0, nr_head = a.head ? a.En : 0;
    const int nr_lora = a.lora_a ? a.r : 0;
    const int R = nr_router + nr_head + nr_lora + (a.sgate_w ? 1 : 0);
    const int t0 = (blockIdx.y * 4 + wave) * 16;
    if (t0 >= T) return;
    // this lane's weight row (B side) and token (A side)
    int row = blockIdx.x * 16 + ml;
    const bool row_ok = row < R;
    row = row_ok ? row : R - 1;
    const uint16_t* w;
    if (row < nr_router) w = a.router + (size_t)row * d;
    else if (row < nr_router + nr_head) w = a.head + (size_t)(row - nr_router) * d;
    else if (row < nr_router + nr_head + nr_lora) w = a.lora_a + (size_t)(row - nr_router - nr_head) * d;
    else w = a.sgate_w;
    const int tok = t0 + ml < T ? t0 + ml : T - 1;
    const uint32_t* aq = a.u_pk + (size_t)tok * (d / 2) + 4 * pc;
    const uint32_t* aql = a.u_pk_lo ? a.u_pk_lo + (size_t)tok * (d / 2) + 4 * pc : nullptr;
    const u32x4* wq = (const u32x4*)(w + 8 * pc);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    constexpr int kB = 8;                      // k-steps whose loads are issued together
    for (int c0 = 0; c0 < d / 32; c0 += kB) {
        u32x4 av[kB], al[kB], wv[kB];
#pragma unroll
        for (int c = 0; c < kB; ++c) {
            const int cc = c0 + c < d / 32 ? c0 + c : d / 32 - 1;
            av[c] = *(const u32x4*)(aq + 16 * cc);
            wv[c] = wq[4 * cc];
            if (aql) al[c] = *(const u32x4*)(aql + 16 * cc);
        }
#pragma unroll
        for (int c = 0; c < kB; ++c) {
            if (c0 + c >= d / 32) break;
            const u32x4 bv = bf16_pairs_p4(wv[c]);
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
            p = mfma16(av[c], bv, p);
            if (aql) p = mfma16(al[c], bv, p);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += (double)p[i];
        }
    }
    if (!row_ok) return;
    const int r = blockIdx.x * 16 + ml;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * pc + i;
        if (t >= T) continue;
        if (r < nr_router) a.logits_r[(size_t)t * a.E + r] = acc[i];
        else if (r < nr_router + nr_head) a.logits_h[(size_t)t * a.En + (r - nr_router)] = acc[i];
        else if (r < nr_router + nr_head + nr_lora) a.au[(size_t)t * a.r + (r - nr_router - nr_head)] = (float)acc[i];
        else a.sgate[t] = (float)(1.0 / (1.0 + exp(-acc[i])));
    }
}

// top-k per token: blockIdx.y = 0 router (self-routed rows), 1 head
__global__ void __launch_bounds__(256) k_route_topk(RouteMMArgs a) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.n_tok) return;
    if (blockIdx.y == 0) {
        if (!a.router || (a.route_idx && a.route_idx[(size_t)t * a.k] >= 0)) return;
        if (a.E <= 64) topk_row<1>(false, a.logits_r, a.E, a.k, t, a.router_bias, nullptr, nullptr, nullptr, nullptr, a.self_idx, a.self_w);
        else if (a.E <= 128) topk_row<2>(false, a.logits_r, a.E, a.k, t, a.router_bias, nullptr, nullptr, nullptr, nullptr, a.self_idx, a.self_w);
        else if (a.E <= 256) topk_row<4>(false, a.logits_r, a.E, a.k, t, a.router_bias, nullptr, nullptr, nullptr, nullptr, a.self_idx, a.self_w);
        else if (a.E <= 512) topk_row<8>(false, a.logits_r, a.E, a.k, t, a.router_bias, nullptr, nullptr, nullptr, nullptr, a.self_idx, a.self_w);
        else topk_row<16>(false, a.logits_r, a.E, a.k, t, a.router_bias, nullptr, nullptr, nullptr, nullptr, a.self_idx, a.self_w);
    } else {
        if (!a.head || !a.pred_idx) return;
        const int E = a.En;
        if (E <= 64) topk_row<1>(false, a.logits_h, E, a.kn, t, a.head_bias, a.hist_cur_m, a.hist_cur, a.hist_prev_m, a.hist_prev, a.pred_idx, a.pred_w);
        else if (E <= 128) topk_row<2>(false, a.logits_h, E, a.kn, t, a.head_bias, a.hist_cur_m, a.hist_cur, a.hist_prev_m, a.hist_prev, a.pred_idx, a.pred_w);
        else if (E <= 256) topk_row<4>(false, a.logits_h, E, a.kn, t, a.head_bias, a.hist_cur_m, a.hist_cur, a.hist_prev_m, a.hist_prev, a.pred_idx, a.pred_w);
        else if (E <= 512) topk_row<8>(false, a.logits_h, E, a.kn, t, a.head_bias, a.hist_cur_m, a.hist_cur, a.hist_prev_m, a.hist_prev, a.pred_idx, a.pred_w);
        else topk_row<16>(false, a.logits_h, E, a.kn, t, a.head_bias, a.hist_cur_m, a.hist_cur, a.hist_prev_m, a.hist_prev, a.pred_idx, a.pred_w);
    }
}

hipError_t launch_route_mm(const RouteMMArgs& a, hipStream_t s) {
    if (a.d % 32) return hipErrorInvalidValue;
    const int R = (a.router ? a.E : 0) + (a.head ? a.En : 0) + (a.lora_a ? a.r : 0) + (a.sgate_w ? 1 : 0);
    if (R > 0) {
        hipLaunchKernelGGL(k_route_mm, dim3((R + 15) / 16, (a.n_tok + 63) / 64), dim3(256), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.router || (a.head && a.pred_idx)) {
        hipLaunchKernelGGL(k_route_topk, dim3((a.n_tok + 3) / 4, 2), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

bool prefill_mm_ok(int d, int f, int fs) {
    return d % kStageK == 0 && d / 64 <= kMaxGroupsPf && f % kStageK == 0 && (fs == 0 || fs % kStageK == 0);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
    const GemvArgs& g = a.g;
    if (!prefill_mm_ok(g.d, g.f, g.fs)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_pf_tiles, dim3(1), dim3(1024), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int fmax = g.f > g.fs ? g.f : g.fs;
    const dim3 ggrid(a.max_tiles, (fmax + kGuRows - 1) / kGuRows);
    if (g.u_pk_lo) hipLaunchKernelGGL(k_pf_gateup<true>, ggrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_pf_gateup<false>, ggrid, dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_pf_down, dim3(a.max_tiles, (g.d + kDnRows * kDnSub - 1) / (kDnRows * kDnSub)), dim3(256), 0,
                       s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_pf_combine, dim3((g.d + 255) / 256, (g.n_tok + kCombTok - 1) / kCombTok), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe

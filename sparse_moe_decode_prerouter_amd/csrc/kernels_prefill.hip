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
#include "dec_common.h"
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

// nib4 with the mask and the exponent held in registers (m = 0x000F000F,
// c = 0x43004300), so that each pair is one and-or after its shift
__device__ __forceinline__ u32x4 nib4v(uint32_t w, uint32_t m, uint32_t c) {
    u32x4 r;
    r.x = (w & m) | c;
    r.y = ((w >> 4) & m) | c;
    r.z = ((w >> 8) & m) | c;
    r.w = ((w >> 12) & m) | c;
    return r;
}

constexpr int kTileBig = 64;      // assignments (tokens) per tile of the large-tile path

int prefill_max_tiles(int T, int K, int E, int tm) {
    const int nk = T * K;
    return (nk + tm - 1) / tm + (nk < E ? nk : E) + (T + tm - 1) / tm + 1;
}

// ---------------------------------------------------------------------------
// Blob of every tile record, resolved after a reactive staging (the sort
// wrote the records before the routing was known on the host). One block.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) k_tile_blobs(PrefillArgs a, int32_t* tiles, int mi) {
    const GemvArgs& g = a.g;
    const ExpertView& ev = g.ev;
    const int n = a.meta_w[mi], nr = a.meta_w[mi + 1];
    int sblob = -1;
    if (ev.shared) sblob = (ev.shared_tag && *ev.shared_tag != ev.E) ? -1 : -2;
    for (int i = threadIdx.x; i < n; i += 1024) {
        int blob;
        bool missing;
        if (i < nr) {
            const int e = g.active[tiles[4 * i]];
            if (!ev.slot_of) blob = e;
            else {
                const int sl = ev.slot_of[e];
                blob = (sl < 0 || (ev.slot_tag && ev.slot_tag[sl] != e)) ? -1 : sl;
            }
            missing = blob < 0;
        } else {
            blob = sblob;
            missing = ev.shared && blob == -1;           // no shared blob at all is not an error
        }
        if (missing) set_err(g.err, ERR_NOT_STAGED);
        tiles[4 * i + 3] = blob;
    }
}

hipError_t launch_tile_blobs(const PrefillArgs& a, bool big, hipStream_t s) {
    hipLaunchKernelGGL(k_tile_blobs, dim3(1), dim3(1024), 0, s, a, a.tiles, 2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !big) return e;
    hipLaunchKernelGGL(k_tile_blobs, dim3(1), dim3(1024), 0, s, a, a.tiles64, 4);
    return hipGetLastError();
}

struct PfItem {
    int slot;     // -1: shared expert
    int p0;       // first position (sorted assignment) or first token
    int M;        // rows of the tile (<= 16)
    int blob;     // >= 0: blob index, -2: shared blob, -1: none
};

__device__ __forceinline__ PfItem pf_item(const PrefillArgs& a, int tile) {
    const int4 t = *(const int4*)(a.tiles + 4 * tile);
    PfItem it;
    it.slot = t.x; it.p0 = t.y; it.M = t.z; it.blob = t.w;
    return it;
}

__device__ __forceinline__ const uint8_t* pf_blob(const GemvArgs& g, int blob) {
    return blob >= 0 ? g.ev.base + (size_t)blob * g.ev.blob : (blob == -2 ? g.ev.shared : nullptr);
}

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU with LDS staging. Block = 16-token tile x kGuRows rows of
// W_g and of W_u (2 n-tiles per wave). The hidden dimension is walked in
// stages of 4 groups (256 elements): every 128-byte line (one row's int4 for
// the stage) is read by 8 consecutive threads as whole 16-byte pieces, and
// stored to LDS with piece p of line r at slot p ^ (r & 7), so the MFMA reads
// (8 bytes per lane, 16 rows per instruction) hit at most 2 lanes per bank
// group. The next stage is loaded into registers while the current one is
// multiplied, then stored over it once every wave is done with it.
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

// NB LDS stage buffers: one keeps blocks small (three per CU) for calls with
// many tiles; two save a barrier per stage when there are few
template <bool LO, int NB>
__device__ __forceinline__ void gateup_body(const PrefillArgs& a, int bx, int by) {
    const GemvArgs& g = a.g;
    __shared__ __align__(16) GuLds<LO> S[NB];
    __shared__ float us64[kTileM][kMaxGroupsPf + 1];
    __shared__ int tok[kTileM];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (bx >= g.meta[2]) return;
    const PfItem it = pf_item(a, bx);
    const bool shared = it.slot < 0;
    const int f = shared ? g.fs : g.f;
    const int rb0 = by * kGuRows;
    if (rb0 >= f || it.M <= 0) return;
    const uint8_t* blob = pf_blob(g, it.blob);
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
    uint32_t nm = 0x000F000Fu, nc = 0x43004300u;
    asm volatile("" : "+v"(nm), "+v"(nc));
    for (int st = 0; st < NS; ++st) {
        const GuLds<LO>& C = S[st % NB];
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
                const u32x4 bg0 = nib4v(wg.x, nm, nc), bg1 = nib4v(wg.y, nm, nc);
                const u32x4 bu0 = nib4v(wu.x, nm, nc), bu1 = nib4v(wu.y, nm, nc);
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
        if (NB == 1) __syncthreads();            // one buffer: every wave is done with it
        if (st + 1 < NS) gu_stage_store<LO>(R, S[(st + 1) % NB]);
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

template <bool LO, int NB>
__global__ void __launch_bounds__(256) k_pf_gateup(PrefillArgs a) {
    gateup_body<LO, NB>(a, blockIdx.x, blockIdx.y);
}

template <int V>
struct IntC {
    static constexpr int value = V;
};

// ---------------------------------------------------------------------------
// Down projection: a persistent grouped GEMM. A stage is 16 KB of W_d codes,
// R = 32768 / f whole rows (contiguous in the blob), plus their scales; a
// tile's stages walk its d / R row blocks. Block b of the grid takes the
// stages [b Z / nb, (b + 1) Z / nb) of the flat list (routed tiles, then the
// shared expert's), so every block streams the same number of bytes. Stages go
// straight from HBM into a ring of kDnNst LDS buffers (direct-to-LDS loads,
// kDnNst - 1 stages in flight); piece p of row r sits at slot p ^ (r mod n)
// (n = 16-byte pieces per row) so that the MFMA reads of 16 rows spread over
// the banks. A tile's expert hidden state h (16 positions x f, fp32) comes into
// LDS the same way one tile ahead and is split once per tile into bf16 hi + lo
// MFMA operands and per-group sums, held in registers. The block's tile records
// and output rows are read once, at the start, so the loop issues no load that
// it has to wait for. Wave w (of 8) owns rows 16 (w mod 4) + 64 j (+ 0..15) of
// each stage and half of the groups (w / 4); the upper half's partial sums go
// through LDS to the lower half, which adds them one stage later and stores.
// Outputs: O[assignment][d] (routed) or O_s[token][d] (shared), unweighted.
// ---------------------------------------------------------------------------
constexpr int kDnThreads = 512;
constexpr int kDnStage = 16384;              // code bytes per stage
constexpr int kDnNst = 6;                    // ring depth
constexpr int kDnMaxF = 512;                 // largest f (and f_shared); f >= 256
constexpr int kDnTiles = 32;                 // tile records kept in LDS per block
constexpr int kHstRow = kDnMaxF + 4;         // floats per position row of the staged h (padded)

struct DnStage {
    uint8_t b[kDnStage];                     // R rows of f / 2 bytes, pieces swizzled
    uint8_t sc[kDnStage / 8];                // their (s, b) pairs: f / 16 bytes per row
};
struct DnOps {
    float hst[kTileM * kHstRow];             // the next tile's h (fp32), as loaded
    f32x4 part[2][2][4][64];                 // [stage parity][j][row tile][lane]: upper-half partial sums
    int4 tinfo[kDnTiles];                    // the block's tile records
    int prow[kDnTiles][kTileM];              // their output rows
};

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at LDS byte address lds + 16 l (lds wave-uniform). Written as asm so that
// the compiler does not guard every later LDS read of the ring with a wait for
// all of these loads; the ring's own waits (vm_wait) order them instead.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is reserved; the clobber still keeps it live-safe
__device__ __forceinline__ void lds_dma16(const void* gptr, const void* lds) {
    const uint32_t off = (uint32_t)(uintptr_t)lds;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(off), "v"(gptr) : "memory", "m0");
}
// The same with a 64-bit scalar base and a 32-bit per-lane offset.
__device__ __forceinline__ void lds_dma16s(uint32_t voff, uint64_t sbase, const void* lds) {
    const uint32_t off = (uint32_t)(uintptr_t)lds;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(off), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt not waited for)
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// wait until this wave's loads of the stage `ahead` stages before the newest
// issued one have landed, for LN loads per stage per wave (LS for the waves
// that also load the scales); any other load issued after that stage only
// makes the wait longer
template <int LN, int LS>
__device__ __forceinline__ void ring_wait(int ahead, bool sc_wave) {
    if (sc_wave) {
        switch (ahead) {
            case 0: vm_wait<0>(); break;
            case 1: vm_wait<LS>(); break;
            case 2: vm_wait<2 * LS>(); break;
            case 3: vm_wait<3 * LS>(); break;
            default: vm_wait<4 * LS>(); break;
        }
    } else {
        switch (ahead) {
            case 0: vm_wait<0>(); break;
            case 1: vm_wait<LN>(); break;
            case 2: vm_wait<2 * LN>(); break;
            case 3: vm_wait<3 * LN>(); break;
            default: vm_wait<4 * LN>(); break;
        }
    }
}

// wait until this wave's loads of the stage `ahead` stages before the newest
// issued one have landed (2 loads per stage per wave, 3 for waves 0-1; any
// other load issued after that stage only makes the wait longer)
__device__ __forceinline__ void dn_wait(int ahead, bool sc_wave) {
    if (sc_wave) {
        switch (ahead) {
            case 0: vm_wait<0>(); break;
            case 1: vm_wait<3>(); break;
            case 2: vm_wait<6>(); break;
            case 3: vm_wait<9>(); break;
            default: vm_wait<12>(); break;
        }
    } else {
        switch (ahead) {
            case 0: vm_wait<0>(); break;
            case 1: vm_wait<2>(); break;
            case 2: vm_wait<4>(); break;
            case 3: vm_wait<6>(); break;
            default: vm_wait<8>(); break;
        }
    }
}

// stages of one tile of width f: d / R row blocks of R = 32768 / f rows
__device__ __host__ __forceinline__ int dn_tile_stages(int d, int f) { return d * f / (2 * kDnStage); }

__global__ void __launch_bounds__(kDnThreads) k_pf_down(PrefillArgs a) {
    static_assert(kDnNst - 2 <= 4, "dn_wait covers up to 4 stages ahead");
    __shared__ __align__(16) DnStage ring[kDnNst];
    __shared__ __align__(16) DnOps S;
    const GemvArgs& g = a.g;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int d = g.d;
    const int nt = g.meta[2], nrt = g.meta[3];
    const int nsr = dn_tile_stages(d, g.f), nss = g.fs ? dn_tile_stages(d, g.fs) : 1;
    const int zr = nrt * nsr, Z = zr + (nt - nrt) * nss;
    const int z0 = (int)((long long)Z * blockIdx.x / gridDim.x);
    const int z1 = (int)((long long)Z * (blockIdx.x + 1) / gridDim.x);
    if (z0 >= z1) return;
    auto tile_of = [&](int z) { return z < zr ? z / nsr : nrt + (z - zr) / nss; };
    auto sidx_of = [&](int z) { return z < zr ? z % nsr : (z - zr) % nss; };
    const int t0 = tile_of(z0);
    const int ntl = tile_of(z1 - 1) - t0 + 1;

    // ---- the block's tile records and output rows (the launch sizes the grid
    // so that no block spans more than kDnTiles tiles)
    if (ntl > kDnTiles) {
        if (tid == 0) set_err(g.err, ERR_BAD_INDEX);
        return;
    }
    if (tid < ntl) S.tinfo[tid] = *(const int4*)(a.tiles + 4 * (t0 + tid));
    lds_barrier();
    for (int i = tid; i < ntl * kTileM; i += kDnThreads) {
        const int4 ti = S.tinfo[i / kTileM];
        const int m = i % kTileM, p = ti.y + (m < ti.z ? m : ti.z - 1);
        S.prow[i / kTileM][m] = ti.x < 0 ? p : g.perm[p];
    }
    auto tile_rec = [&](int t) -> int4 { return S.tinfo[t - t0]; };

    // ---- h of tile t (16 positions x f fp32, rows past M repeat the last)
    // into S.hst, row m at m * kHstRow (a wave's 64 pieces lie in one row)
    auto issue_h = [&](int t) {
        const int4 ti = tile_rec(t);
        const bool sh = ti.x < 0;
        const int f = sh ? g.fs : g.f;
        const float* hb = sh ? g.hs : g.h;
        const int lpr = f == 512 ? 7 : 6;            // log2 of the 16-byte pieces per row
        for (int j = 0; j < 16 * f / 4 / kDnThreads; ++j) {
            const int pw = wave * 64 + kDnThreads * j, pi = pw + lane;
            const int m = pi >> lpr, c4 = pi & ((1 << lpr) - 1);
            const int mw = pw >> lpr, cw = pw & ((1 << lpr) - 1);
            const float* src = hb + (size_t)(ti.y + (m < ti.z ? m : ti.z - 1)) * f + 4 * c4;
            lds_dma16(src, &S.hst[mw * kHstRow + 4 * cw]);
        }
    };

    // ---- loader: issues the next stage (tile lt, stage ls of it) into ring
    // slot lslot. Per tile: scalar bases of W_d's codes and scales, and the
    // per-thread byte offsets of its pieces within a stage.
    constexpr int kPj = kDnStage / 16 / kDnThreads;            // code pieces per thread per stage
    int lt = t0, ls = sidx_of(z0), lns = 0, lslot = 0;
    uint64_t lq = 0, lsb = 0;
    uint32_t lvq[kPj];
    auto loader_tile = [&](int t) {
        const int4 ti = tile_rec(t);
        const int f = ti.x < 0 ? g.fs : g.f;
        const uint8_t* blob = pf_blob(g, ti.w);
        const uint8_t* wb = blob ? blob : g.ev.base;
        const BlobLayout L = BlobLayout::make(d, f);
        lq = (uint64_t)(uintptr_t)(wb + L.down_q);
        lsb = (uint64_t)(uintptr_t)(wb + L.down_sb);
        lns = dn_tile_stages(d, f);
        const int sh = f == 512 ? 4 : 3;                       // log2 of the pieces per row
#pragma unroll
        for (int j = 0; j < kPj; ++j) {
            const int pi = wave * 64 + kDnThreads * j + lane, r = pi >> sh;
            const int pg = (pi & ((1 << sh) - 1)) ^ (r & ((1 << sh) - 1));
            lvq[j] = (uint32_t)(r * (f / 2) + 16 * pg);
        }
    };
    auto issue = [&]() {
        DnStage& st = ring[lslot];
        const uint64_t bq = lq + (uint64_t)ls * kDnStage;
#pragma unroll
        for (int j = 0; j < kPj; ++j) lds_dma16s(lvq[j], bq, &st.b[(wave * 64 + kDnThreads * j) * 16]);
        if (wave < 2)
            lds_dma16s((uint32_t)(wave * 64 + lane) * 16u, lsb + (uint64_t)ls * (kDnStage / 8), &st.sc[wave * 64 * 16]);
        lslot = lslot + 1 == kDnNst ? 0 : lslot + 1;
        if (++ls == lns) {
            ls = 0;
            if (++lt < t0 + ntl) loader_tile(lt);
        }
    };

    lds_barrier();                                            // tile records visible
    issue_h(t0);
    loader_tile(t0);
    for (int i = 0; i < kDnNst - 1 && z0 + i < z1; ++i) issue();

    // The A operand of this wave's groups (half of them) of the current tile,
    // in registers: lane (ml, pc) holds, for group gq = 4 kh + q, elements
    // 64 gq + 16 pc .. + 15 of position ml as bf16 hi and lo pairs (t = 0, 1:
    // 8 elements each), and the group sums of positions 4 pc .. 4 pc + 3.
    const int rt = wave & 3, kh = wave >> 2;
    u32x4 rah[4][2], ral[4][2];
    float4 rhs[4];
    int ctile = -1, M = 0, cs = sidx_of(z0), cns = 1, cf = 0, cslot = 0;
    int zh = -(1 << 30);                                      // iteration that issued the current h loads
    bool shared = false, ok = false;
    const int ml = lane & 15, pc = lane >> 4;
    uint32_t nm = 0x000F000Fu, nc = 0x43004300u;
    asm volatile("" : "+v"(nm), "+v"(nc));
    // the lower half's pending outputs (stage of the previous iteration)
    f32x4 pend[2];
    bool have_pend = false;
    int p_s = 0, p_tile = 0, p_M = 0, p_par = 0, p_nj = 0, p_R = 0;
    bool p_shared = false, p_ok = false;

    auto flush = [&]() {
        // lower half: add the upper half's partials of the pending stage and store
        const int* orow = S.prow[p_tile - t0];
        float* dst = p_shared ? a.obs : a.ob;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (j >= p_nj) break;
            const f32x4 o = pend[j] + S.part[p_par][j][rt][lane];
            const int n = p_s * p_R + rt * 16 + 64 * j + ml;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * pc + i;
                if (m < p_M) dst[(size_t)orow[m] * d + n] = p_ok ? o[i] : 0.f;
            }
        }
    };

    // one stage of width F: NJ row tiles per wave, 4 of the NG groups
    auto stage_compute = [&](auto FW, const DnStage& st, int par) {
        constexpr int F = decltype(FW)::value;
        constexpr int R = 2 * kDnStage / F, NJ = R / 64, NG = F / 64, NP = F / 32, NQ = NG / 2;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int r = rt * 16 + 64 * j + ml;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int gq = kh * NQ + q, p = 2 * gq + (pc >> 1);
                const u32x2 w = *(const u32x2*)&st.b[r * (F / 2) + ((p ^ (r & (NP - 1))) << 4) + ((pc & 1) << 3)];
                const uint32_t sb = *(const uint32_t*)&st.sc[r * (F / 16) + 4 * gq];
                const u32x4 b0 = nib4v(w.x, nm, nc), b1 = nib4v(w.y, nm, nc);
                f32x4 pp = {0.f, 0.f, 0.f, 0.f};
                pp = mfma16(rah[q][0], b0, pp);
                pp = mfma16(rah[q][1], b1, pp);
                pp = mfma16(ral[q][0], b0, pp);
                pp = mfma16(ral[q][1], b1, pp);
                const float sv = f16_to_f32(sb & 0xFFFF), cv = f16_to_f32(sb >> 16) - 128.f * sv;
                const float4 hsm = rhs[q];
                acc[0] = __builtin_fmaf(sv, pp[0], __builtin_fmaf(cv, hsm.x, acc[0]));
                acc[1] = __builtin_fmaf(sv, pp[1], __builtin_fmaf(cv, hsm.y, acc[1]));
                acc[2] = __builtin_fmaf(sv, pp[2], __builtin_fmaf(cv, hsm.z, acc[2]));
                acc[3] = __builtin_fmaf(sv, pp[3], __builtin_fmaf(cv, hsm.w, acc[3]));
            }
            if (kh) S.part[par][j][rt][lane] = acc;
            else pend[j] = acc;
        }
        p_nj = NJ;
        p_R = R;
    };

    for (int z = z0; z < z1; ++z) {
        const bool new_tile = ctile < 0 || cs == 0;
        // the new tile's h loads are covered by the wait for stage z only if
        // stage z was issued after them (it was issued in iteration z - kDnNst + 1)
        if (new_tile && z - (kDnNst - 1) < zh) vm_wait<0>();
        dn_wait(min(kDnNst - 2, z1 - 1 - z), wave < 2);
        lds_barrier();               // stage z (and h) landed; stage z - 1 consumed, its partials written
        if (have_pend && !kh) flush();
        have_pend = false;
        if (new_tile) {
            // the tile's h becomes the A operand (each wave converts its half)
            ctile = ctile < 0 ? t0 : ctile + 1;
            const int4 ti = tile_rec(ctile);
            shared = ti.x < 0;
            cf = shared ? g.fs : g.f;
            cns = dn_tile_stages(d, cf);
            M = ti.z;
            ok = ti.w != -1;
            const int nq = cf / 128;                          // groups per half
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q >= nq) break;
                const float* src = &S.hst[ml * kHstRow + (kh * nq + q) * 64 + 16 * pc];
                float e[16];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float4 x = *(const float4*)(src + 4 * v);
                    e[4 * v] = x.x; e[4 * v + 1] = x.y; e[4 * v + 2] = x.z; e[4 * v + 3] = x.w;
                }
                float hs = 0.f;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    uint32_t hi[8], lo[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        hi[i] = f32_to_bf16(e[8 * t + i]);
                        lo[i] = f32_to_bf16(e[8 * t + i] - bf16_to_f32(hi[i]));
                        hs += bf16_to_f32(hi[i]) + bf16_to_f32(lo[i]);
                    }
                    rah[q][t] = u32x4{hi[0] | (hi[4] << 16), hi[1] | (hi[5] << 16), hi[2] | (hi[6] << 16),
                                      hi[3] | (hi[7] << 16)};
                    ral[q][t] = u32x4{lo[0] | (lo[4] << 16), lo[1] | (lo[5] << 16), lo[2] | (lo[6] << 16),
                                      lo[3] | (lo[7] << 16)};
                }
                // group sum of position ml, then those of positions 4 pc + i
                hs += __shfl_xor(hs, 16, 64);
                hs += __shfl_xor(hs, 32, 64);
                rhs[q] = make_float4(__shfl(hs, 4 * pc, 64), __shfl(hs, 4 * pc + 1, 64), __shfl(hs, 4 * pc + 2, 64),
                                     __shfl(hs, 4 * pc + 3, 64));
            }
            lds_barrier();                                    // every wave has read S.hst
            if (ctile + 1 < t0 + ntl) {
                issue_h(ctile + 1);
                zh = z;
            }
        }
        const DnStage& st = ring[cslot];
        const int par = (z - z0) & 1;
        if (cf == 512) stage_compute(IntC<512>{}, st, par);
        else stage_compute(IntC<256>{}, st, par);
        // the next stage's loads go out after this wave's compute, so that a
        // full memory queue delays no compute
        if (z + kDnNst - 1 < z1) issue();
        have_pend = true;
        p_s = cs; p_tile = ctile; p_M = M; p_par = par; p_shared = shared; p_ok = ok;
        cslot = cslot + 1 == kDnNst ? 0 : cslot + 1;
        if (++cs == cns) cs = 0;
    }
    lds_barrier();                                            // the last partials are written
    if (have_pend && !kh) flush();
    vm_wait<0>();                                             // no direct-to-LDS load outlives the block
}

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU with 64-token tiles (many tokens per expert, long
// prefills). Block = 64 tokens x 128 rows of W_g and the same rows of W_u;
// wave w owns rows 32 w .. 32 w + 31 (2 row tiles) of both and all 64 tokens
// (4 token tiles), so each unpacked B fragment feeds 4 MFMAs and each A
// fragment 4 weight tiles. k walks in stages of GS groups (64 GS elements)
// through a ring of NST LDS buffers filled NST - 1 stages ahead by
// direct-to-LDS loads. The bias half of
// the affine dequant, sum_g (b - 128 s)_g * sum_{k in g} u_k, is itself a bf16
// MFMA over the group axis (hi/lo of both factors) evaluated before the k loop;
// each group's scale s multiplies that group's fresh MFMA accumulator.
// bf16 activations; d a multiple of 128 up to 2048 (at most 32 groups, one
// MFMA k-step); f a multiple of 128.
// ---------------------------------------------------------------------------
constexpr int kBgWaves = 8;                   // waves per block
constexpr int kBgRt = 1;                      // 16-row tiles of W_g (and of W_u) per wave
constexpr int kBgRows = 16 * kBgRt * kBgWaves;   // rows of W_g (and of W_u) per block
constexpr int kBgGs = 2;                      // groups per stage
constexpr int kBgNst = 2;                     // ring depth (two blocks per CU fit the LDS)

// one stage of GS groups: PA = 8 GS 16-byte pieces of u per token row, PB =
// 2 GS pieces of int4 per weight row
template <int GS, int TM, int NR>
struct BgStage {
    static constexpr int PA = 8 * GS, PB = 2 * GS;
    uint8_t a[TM * PA * 16];                  // piece c of token row m at slot c ^ (m mod PA)
    uint8_t b[2 * NR * PB * 16];              // 2 NR rows (gate, then up); piece p of row r at slot p ^ bsw(r)
    uint32_t sc[2 * NR][GS];                  // (s, b) of the stage's groups per row
    // slot swizzle of the weight rows: the 16 rows of one MFMA read spread
    // over all bank groups
    static __device__ __forceinline__ int bsw(int r) { return PB == 4 ? (r >> 2) & 3 : (r >> 3) & 1; }
};

// 4 bytes per lane from global memory straight into LDS (lane l at lds + 4 l)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma4(const void* gptr, const void* lds) {
    const uint32_t off = (uint32_t)(uintptr_t)lds;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" : : "s"(off), "v"(gptr) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int GS, int NST, int TM, int RT, int NW>
__global__ void __launch_bounds__(64 * NW) k_pf_gateup_big(PrefillArgs a) {
    constexpr int NT = 64 * NW;               // threads
    constexpr int NR = 16 * RT * NW;          // rows of W_g (and of W_u) per block
    using Stage = BgStage<GS, TM, NR>;
    constexpr int PA = Stage::PA, PB = Stage::PB, KS = 64 * GS, MT = TM / 16;
    // direct-to-LDS loads per stage per wave: LA of u, LB of codes, LS of
    // scales (fewer than one per thread: only the first SW waves load them)
    constexpr int LA = TM * PA / NT, LB = 2 * NR * PB / NT;
    constexpr int LS = 2 * NR * GS >= NT ? 2 * NR * GS / NT : 1, SW = 2 * NR * GS >= NT ? NW : 2 * NR * GS / 64;
    constexpr int LN = LA + LB;
    static_assert(TM * PA >= NT && 2 * NR * PB >= NT && 2 * NR * GS >= 64, "one piece per thread at least");
    const GemvArgs& g = a.g;
    __shared__ __align__(16) Stage S[NST];
    __shared__ __align__(16) uint16_t ush[TM][32], usl[TM][32];   // group sums of u, bf16 hi / lo
    __shared__ int tok[TM];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if ((int)blockIdx.x >= g.meta[TM == kTileBig ? 4 : 2]) return;
    const int4 ti = *(const int4*)((TM == kTileBig ? a.tiles64 : a.tiles) + 4 * blockIdx.x);
    const bool shared = ti.x < 0;
    const int f = shared ? g.fs : g.f;
    const int rb0 = blockIdx.y * NR;
    const int p0 = ti.y, M = ti.z;
    if (rb0 >= f || M <= 0) return;
    const uint8_t* blob = pf_blob(g, ti.w);
    const uint8_t* wb = blob ? blob : g.ev.base;
    const int d = g.d, G = d / 64, NS = d / KS;
    const BlobLayout L = BlobLayout::make(d, f);
    if (tid < TM) {
        const int p = p0 + (tid < M ? tid : M - 1);
        tok[tid] = shared ? p : g.perm[p] / g.k;
    }
    __syncthreads();
    // per-thread sources of a stage (direct-to-LDS, contiguous per wave instruction)
    const uint32_t* asrc[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int pa = wave * 64 + NT * i + lane, m = pa / PA, c = (pa % PA) ^ (m % PA);
        asrc[i] = g.u_pk + (size_t)tok[m] * (d / 2) + 4 * c;
    }
    const uint8_t* bsrc[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int pi = wave * 64 + NT * i + lane, r = pi / PB, pg = (pi % PB) ^ Stage::bsw(r);
        bsrc[i] = wb + (r < NR ? L.gate_q : L.up_q) + (size_t)(rb0 + (r & (NR - 1))) * (d / 2) + 16 * pg;
    }
    const uint8_t* ssrc[LS];
#pragma unroll
    for (int j = 0; j < LS; ++j) {
        const int di = wave * 64 + NT * j + lane, r = di / GS;
        ssrc[j] = wb + (r < NR ? L.gate_sb : L.up_sb) + (size_t)(rb0 + (r & (NR - 1))) * (d / 16) + 4 * (di % GS);
    }
    auto stage_issue = [&](int kc, Stage& st) {
#pragma unroll
        for (int i = 0; i < LA; ++i) lds_dma16(asrc[i] + kc * (KS / 2), &st.a[(wave * 64 + NT * i) * 16]);
#pragma unroll
        for (int i = 0; i < LB; ++i) lds_dma16(bsrc[i] + kc * (KS / 2), &st.b[(wave * 64 + NT * i) * 16]);
#pragma unroll
        for (int j = 0; j < LS; ++j)
            if (wave < SW) lds_dma4(ssrc[j] + kc * 4 * GS, (const uint8_t*)&st.sc[0][0] + (wave * 64 + NT * j) * 4);
    };
    for (int i = 0; i < NST - 1 && i < NS; ++i) stage_issue(i, S[i]);

    // ---- bias term, as one MFMA k-step over the groups: A = group sums of u
    // (tokens x groups), B = (b - 128 s) (groups x rows), both bf16 hi + lo
    for (int i = tid; i < TM * 32; i += NT) {
        const int m = i >> 5, gg = i & 31;
        float us = 0.f;
        if (gg < G) us = g.usum[(size_t)tok[m] * (d / 32) + 2 * gg] + g.usum[(size_t)tok[m] * (d / 32) + 2 * gg + 1];
        const uint32_t hi = f32_to_bf16(us);
        ush[m][gg] = (uint16_t)hi;
        usl[m][gg] = (uint16_t)f32_to_bf16(us - bf16_to_f32(hi));
    }
    const int ml = lane & 15, pc = lane >> 4;
    f32x4 acc[MT][RT][2];                      // [token tile][row tile][gate / up]
    {
        u32x4 chi[RT][2], clo[RT][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int gu = 0; gu < 2; ++gu) {
                const int n = rb0 + 16 * RT * wave + 16 * rt + ml;
                const uint32_t* sbp = (const uint32_t*)(wb + (gu ? L.up_sb : L.gate_sb) + (size_t)n * (d / 16));
                uint32_t h8[8], l8[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int gg = 8 * pc + j;
                    float c = 0.f;
                    if (gg < G) {
                        const uint32_t sb = sbp[gg];
                        c = f16_to_f32(sb >> 16) - 128.f * f16_to_f32(sb & 0xFFFF);
                    }
                    h8[j] = f32_to_bf16(c);
                    l8[j] = f32_to_bf16(c - bf16_to_f32(h8[j]));
                }
                chi[rt][gu] = u32x4{h8[0] | (h8[1] << 16), h8[2] | (h8[3] << 16), h8[4] | (h8[5] << 16),
                                    h8[6] | (h8[7] << 16)};
                clo[rt][gu] = u32x4{l8[0] | (l8[1] << 16), l8[2] | (l8[3] << 16), l8[4] | (l8[5] << 16),
                                    l8[6] | (l8[7] << 16)};
            }
        lds_barrier();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const u32x4 uh = *(const u32x4*)&ush[16 * mt + ml][8 * pc];
            const u32x4 ul = *(const u32x4*)&usl[16 * mt + ml][8 * pc];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int gu = 0; gu < 2; ++gu) {
                    f32x4 c = {0.f, 0.f, 0.f, 0.f};
                    c = mfma16(uh, chi[rt][gu], c);
                    c = mfma16(uh, clo[rt][gu], c);
                    c = mfma16(ul, chi[rt][gu], c);
                    acc[mt][rt][gu] = c;
                }
        }
    }

    // ---- k loop: stages kc + 1 .. kc + NST - 1 load while stage kc is multiplied
    uint32_t nm = 0x000F000Fu, nc = 0x43004300u;
    asm volatile("" : "+v"(nm), "+v"(nc));
    for (int kc = 0; kc < NS; ++kc) {
        ring_wait<LN, LN + LS>(min(NST - 2, NS - 1 - kc), wave < SW);
        lds_barrier();                                  // stage kc landed everywhere; stage kc - 1 consumed
        const Stage& st = S[kc % NST];
        if (kc + NST - 1 < NS) stage_issue(kc + NST - 1, S[(kc + NST - 1) % NST]);
#pragma unroll
        for (int q = 0; q < GS; ++q) {
            const int p = 2 * q + (pc >> 1);
            u32x4 b0[RT][2], b1[RT][2];
            float sv[RT][2];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int gu = 0; gu < 2; ++gu) {
                    const int r = gu * NR + 16 * RT * wave + 16 * rt + ml;
                    const u32x2 w = *(const u32x2*)&st.b[r * (PB * 16) + ((p ^ Stage::bsw(r)) << 4) + ((pc & 1) << 3)];
                    b0[rt][gu] = nib4v(w.x, nm, nc);
                    b1[rt][gu] = nib4v(w.y, nm, nc);
                    sv[rt][gu] = f16_to_f32(st.sc[r][q] & 0xFFFF);
                }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = 16 * mt + ml, gp = 8 * q + 2 * pc;        // pieces gp, gp + 1 of row m
                const u32x4 a0 = *(const u32x4*)&st.a[m * (PA * 16) + ((gp ^ (m % PA)) << 4)];
                const u32x4 a1 = *(const u32x4*)&st.a[m * (PA * 16) + (((gp + 1) ^ (m % PA)) << 4)];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int gu = 0; gu < 2; ++gu) {
                        f32x4 pp = {0.f, 0.f, 0.f, 0.f};
                        pp = mfma16(a0, b0[rt][gu], pp);
                        pp = mfma16(a1, b1[rt][gu], pp);
                        const float s1 = sv[rt][gu];
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[mt][rt][gu][i] = __builtin_fmaf(s1, pp[i], acc[mt][rt][gu][i]);
                    }
            }
        }
    }
    const bool ok = blob != nullptr;
    float* hb = shared ? g.hs : g.h;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int n = rb0 + 16 * RT * wave + 16 * rt + ml;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * mt + 4 * pc + i;
                if (m < M && n < f) hb[(size_t)(p0 + m) * f + n] = ok ? silu_f32(acc[mt][rt][0][i]) * acc[mt][rt][1][i] : 0.f;
            }
        }
}

// ---------------------------------------------------------------------------
// Combine per (token, row): shared (gated), routed in routing order
// (weighted), LoRA B, residual. A thread takes 4 consecutive rows of
// kCombTok tokens; every load of a term is issued for all its tokens before
// any is used.
// ---------------------------------------------------------------------------
constexpr int kCombTok = 4;

// the head's top-k of token t (one wave)
__device__ __forceinline__ void head_topk_wave(const PrefillArgs& a, int t) {
    const TopkJob& j = a.head;
    if (j.En <= 64) topk_row<1>(false, j.logits, j.En, j.kn, t, j.bias, j.mc, j.hc, j.mp, j.hp, j.pred_idx, j.pred_w);
    else if (j.En <= 128) topk_row<2>(false, j.logits, j.En, j.kn, t, j.bias, j.mc, j.hc, j.mp, j.hp, j.pred_idx, j.pred_w);
    else if (j.En <= 256) topk_row<4>(false, j.logits, j.En, j.kn, t, j.bias, j.mc, j.hc, j.mp, j.hp, j.pred_idx, j.pred_w);
    else if (j.En <= 512) topk_row<8>(false, j.logits, j.En, j.kn, t, j.bias, j.mc, j.hc, j.mp, j.hp, j.pred_idx, j.pred_w);
    else topk_row<16>(false, j.logits, j.En, j.kn, t, j.bias, j.mc, j.hc, j.mp, j.hp, j.pred_idx, j.pred_w);
}

// y of tokens t0 .. t0 + nt - 1 at columns n .. n + 3: gated shared expert, the
// routed outputs in routing order, LoRA B, residual
template <int NT>
__device__ __forceinline__ void combine_cols(const PrefillArgs& a, int t0, int nt, int n, float4 (&y)[NT]) {
    const GemvArgs& g = a.g;
    const int d = g.d;
    const bool sh = g.fs && g.ev.shared;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        const int t = t0 + (tt < nt ? tt : 0);
        y[tt] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (sh) {
            const float sg = g.sgate ? g.sgate[t] : 1.f;
            const float4 o = *(const float4*)(a.obs + (size_t)t * d + n);
            y[tt] = make_float4(sg * o.x, sg * o.y, sg * o.z, sg * o.w);
        }
    }
    for (int j = 0; j < g.k; ++j) {
        float4 o[NT];
        float w[NT];
        bool v[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int aid = (t0 + (tt < nt ? tt : 0)) * g.k + j;
            v[tt] = a.used_idx[aid] >= 0;            // an invalid entry's row was never written
            w[tt] = a.used_w[aid];
            o[tt] = *(const float4*)(a.ob + (size_t)aid * d + n);
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            if (!v[tt]) continue;
            y[tt].x += w[tt] * o[tt].x; y[tt].y += w[tt] * o[tt].y;
            y[tt].z += w[tt] * o[tt].z; y[tt].w += w[tt] * o[tt].w;
        }
    }
    if (g.lora_b && g.r) {
        const int r = g.r;
        float l[NT][4];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) l[tt][i] = 0.f;
        if (r % 8 == 0 && r <= 32) {
            u32x4 lb[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    lb[i][c] = *(const u32x4*)(g.lora_b + (size_t)(n + i) * r + 8 * (8 * c < r ? c : 0));
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (8 * c >= r) break;
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const float* au = g.au + (size_t)(t0 + (tt < nt ? tt : 0)) * r + 8 * c;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t wv[4] = {lb[i][c].x, lb[i][c].y, lb[i][c].z, lb[i][c].w};
#pragma unroll
                        for (int h = 0; h < 4; ++h) {
                            l[tt][i] += bf16_to_f32(wv[h] & 0xFFFF) * au[2 * h];
                            l[tt][i] += bf16_to_f32(wv[h] >> 16) * au[2 * h + 1];
                        }
                    }
                }
            }
        } else {
            for (int q = 0; q < r; ++q) {
                float wq[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) wq[i] = bf16_to_f32(g.lora_b[(size_t)(n + i) * r + q]);
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const float u = g.au[(size_t)(t0 + (tt < nt ? tt : 0)) * r + q];
#pragma unroll
                    for (int i = 0; i < 4; ++i) l[tt][i] += wq[i] * u;
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            y[tt].x += g.lora_scale * l[tt][0]; y[tt].y += g.lora_scale * l[tt][1];
            y[tt].z += g.lora_scale * l[tt][2]; y[tt].w += g.lora_scale * l[tt][3];
        }
    }
    if (g.fused) {
        float4 x[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) x[tt] = *(const float4*)(g.x + (size_t)(t0 + (tt < nt ? tt : 0)) * d + n);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            y[tt].x += x[tt].x; y[tt].y += x[tt].y; y[tt].z += x[tt].z; y[tt].w += x[tt].w;
        }
    }
}

__global__ void __launch_bounds__(256) k_pf_combine(PrefillArgs a) {
    const GemvArgs& g = a.g;
    const int gy = (g.n_tok + kCombTok - 1) / kCombTok;
    if ((int)blockIdx.y >= gy) {
        // the head's top-k for the next layer: one token per wave
        const int t = (((int)blockIdx.y - gy) * (int)gridDim.x + (int)blockIdx.x) * 4 + (int)(threadIdx.x >> 6);
        if (t >= g.n_tok) return;
        head_topk_wave(a, t);
        return;
    }
    const int d = g.d, n = (blockIdx.x * 256 + threadIdx.x) * 4;
    const int t0 = blockIdx.y * kCombTok;
    if (n >= d) return;
    const int nt = min(kCombTok, g.n_tok - t0);
    float4 y[kCombTok];
    combine_cols<kCombTok>(a, t0, nt, n, y);
#pragma unroll
    for (int tt = 0; tt < kCombTok; ++tt)
        if (tt < nt) *(float4*)(g.y + (size_t)(t0 + tt) * d + n) = y[tt];
}

// ---------------------------------------------------------------------------
// The combine with the next stacked layer's prologue: a block holds whole rows
// (d <= 4 kCnThreads) of kCnTok tokens, so once it has x + y it also takes
// that layer's RMSNorm (fp64 sum of squares over the block, u rounded once)
// and writes its u in the prologue's three forms (GEMV-order pairs with their
// lo parts, fragment order, 32-chunk sums, each piece summed in element
// order), and the next layer launches no prologue. Head top-k blocks (one
// token per wave) come before the combine blocks.
// ---------------------------------------------------------------------------
constexpr int kCnThreads = 512;
constexpr int kCnTok = 1;                     // tokens per block
constexpr int kCnMaxTok = 128;                // calls of at most this many tokens take the fused form

__global__ void __launch_bounds__(kCnThreads) k_pf_combine_norm(PrefillArgs a) {
    const GemvArgs& g = a.g;
    const PrologueArgs& p = a.nxt;
    __shared__ double red[kCnTok][kCnThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // head top-k blocks first (they run longest), then the combine blocks
    const int gt = a.head.pred_idx ? (g.n_tok + kCnThreads / 64 - 1) / (kCnThreads / 64) : 0;
    if ((int)blockIdx.x < gt) {
        const int t = (int)blockIdx.x * (kCnThreads / 64) + wave;
        if (t < g.n_tok) head_topk_wave(a, t);
        return;
    }
    const int d = g.d, n = tid * 4;
    const int t0 = ((int)blockIdx.x - gt) * kCnTok;
    const int nt = min(kCnTok, g.n_tok - t0);
    const bool act = n < d;                   // threads past d only take part in the reductions
    float4 y[kCnTok];
#pragma unroll
    for (int tt = 0; tt < kCnTok; ++tt) y[tt] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (act) {
        combine_cols<kCnTok>(a, t0, nt, n, y);
#pragma unroll
        for (int tt = 0; tt < kCnTok; ++tt)
            if (tt < nt) *(float4*)(g.y + (size_t)(t0 + tt) * d + n) = y[tt];
    }
    float4 gm = make_float4(0.f, 0.f, 0.f, 0.f);
    if (act) gm = *(const float4*)(p.gamma + n);
#pragma unroll
    for (int tt = 0; tt < kCnTok; ++tt) {
        double ss = (double)y[tt].x * y[tt].x;
        ss += (double)y[tt].y * y[tt].y;
        ss += (double)y[tt].z * y[tt].z;
        ss += (double)y[tt].w * y[tt].w;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
        if (lane == 0) red[tt][wave] = ss;
    }
    __syncthreads();
    const int pc = n >> 3;                    // 8-element piece; even threads hold its first half
#pragma unroll
    for (int tt = 0; tt < kCnTok; ++tt) {
        if (tt >= nt) break;                  // block-uniform
        const int t = t0 + tt;
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < kCnThreads / 64; ++w) tot += red[tt][w];
        const double den = sqrt(tot / (double)d + (double)p.eps);
        const float xv[4] = {y[tt].x, y[tt].y, y[tt].z, y[tt].w};
        const float gv[4] = {gm.x, gm.y, gm.z, gm.w};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double uv = ((double)xv[i] / den) * (double)gv[i];
            const float uf = p.act_bf16 ? bf16_to_f32(f64_to_bf16(uv)) : (float)uv;
            hi[i] = f32_to_bf16(uf);
            lo[i] = f32_to_bf16(uf - bf16_to_f32(hi[i]));
        }
        uint32_t ho[4], lw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ho[i] = (uint32_t)__shfl_xor((int)hi[i], 1, 64);
            lw[i] = (uint32_t)__shfl_xor((int)lo[i], 1, 64);
        }
        // the piece's sums in element order, then over the chunk's 4 pieces
        float sh = 0.f, sl = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) { sh += bf16_to_f32(hi[i]); sl += bf16_to_f32(lo[i]); }
#pragma unroll
        for (int i = 0; i < 4; ++i) { sh += bf16_to_f32(ho[i]); sl += bf16_to_f32(lw[i]); }
        sh += __shfl_xor(sh, 2, 64);
        sh += __shfl_xor(sh, 4, 64);
        sl += __shfl_xor(sl, 2, 64);
        sl += __shfl_xor(sl, 4, 64);
        if (act && (tid & 1) == 0) {
            const u32x4 hv = u32x4{hi[0] | (ho[0] << 16), hi[1] | (ho[1] << 16), hi[2] | (ho[2] << 16), hi[3] | (ho[3] << 16)};
            *(u32x4*)(p.u_pk + (size_t)t * (d / 2) + 4 * pc) = hv;
            if (p.u_pk_lo)
                *(u32x4*)(p.u_pk_lo + (size_t)t * (d / 2) + 4 * pc) =
                    u32x4{lo[0] | (lw[0] << 16), lo[1] | (lw[1] << 16), lo[2] | (lw[2] << 16), lo[3] | (lw[3] << 16)};
            if (p.u_frag)
                *(u32x4*)(p.u_frag + ((size_t)(t >> 4) * (d / 32) + (pc >> 2)) * 256 + ((pc & 3) * 16 + (t & 15)) * 4) = hv;
            if ((n & 31) == 0) {
                p.usum[(size_t)t * (d / 32) + (n >> 5)] = sh;
                if (p.usum_lo) p.usum_lo[(size_t)t * (d / 32) + (n >> 5)] = sl;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16-row GEMM on u for the routing side: rows [router E | head En | LoRA A
// r | shared gate 1] x tokens. bf16 x bf16 products are exact in fp32; each
// 32-wide k-step goes to a fresh fp32 accumulator and the steps are summed in
// fp64, so a logit carries the rounding of at most one 32-term fp32 sum per
// step. Grid: (blocks of 16 RT rows, blocks of 16 TT tokens); the NW waves
// of a block take consecutive slices of the k-steps, summed in slice order.
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

// whether any of the tokens t0 .. t0 + n - 1 takes the layer's own router
// (block-uniform; every thread of the block calls it)
__device__ __forceinline__ bool route_tile_needed(const RouteMMArgs& a, int t0, int n) {
    if (!a.route_idx) return true;
    const int t = t0 + (int)threadIdx.x;
    const int self = (int)threadIdx.x < n && t < a.n_tok &&
                     (t < a.route_shift || a.route_idx[(size_t)(t - a.route_shift) * a.k] < 0);
    return __syncthreads_or(self) != 0;
}

// RT x TT 16 x 16 tiles (rows x tokens) per block; NW waves split the d / 32
// k-steps into NW consecutive slices (a wave's loads issued kMaxSteps k-steps
// at a time); LO: activations carry a bf16 lo part (two MFMAs per product)
template <int RT, int TT, int NW, bool LO>
__global__ void __launch_bounds__(64 * NW) k_route_mm(RouteMMArgs a) {
    __shared__ double red[NW - 1][RT * TT * 4][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ml = lane & 15, pc = lane >> 4;
    const int d = a.d, T = a.n_tok;
    const int nr_router = a.router ? a.E : 0, nr_head = a.head ? a.En : 0;
    const int nr_lora = a.lora_a ? a.r : 0;
    const int R = nr_router + nr_head + nr_lora + (a.sgate_w ? 1 : 0);
    const int r0 = blockIdx.x * 16 * RT, t0 = blockIdx.y * 16 * TT;
    // router rows are needed only for self-routed tokens
    if (r0 + 16 * RT <= nr_router && !route_tile_needed(a, t0, 16 * TT)) return;
    // this lane's weight rows (B side) and tokens (A side), clamped into range
    const u32x4* wq[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        int row = r0 + 16 * i + ml;
        row = row < R ? row : R - 1;
        const uint16_t* w;
        if (row < nr_router) w = a.router + (size_t)row * d;
        else if (row < nr_router + nr_head) w = a.head + (size_t)(row - nr_router) * d;
        else if (row < nr_router + nr_head + nr_lora) w = a.lora_a + (size_t)(row - nr_router - nr_head) * d;
        else w = a.sgate_w;
        wq[i] = (const u32x4*)(w + 8 * pc);
    }
    const uint32_t* aq[TT];
    const uint32_t* aql[TT];
    constexpr bool lo = LO;
#pragma unroll
    for (int j = 0; j < TT; ++j) {
        const int tok = t0 + 16 * j + ml < T ? t0 + 16 * j + ml : T - 1;
        aq[j] = a.u_pk + (size_t)tok * (d / 2) + 4 * pc;
        aql[j] = lo ? a.u_pk_lo + (size_t)tok * (d / 2) + 4 * pc : aq[j];
    }
    // wave w takes k-steps [w * ns, (w + 1) * ns)
    const int ns = d / (32 * NW), c0 = wave * ns;
    constexpr int kMaxSteps = RT * TT > 1 ? (LO ? 4 : 8) : (LO ? 8 : 16);   // k-steps whose loads are issued together
    double acc[RT][TT][4];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < TT; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0;
    for (int b0 = 0; b0 < ns; b0 += kMaxSteps) {
        const int nb = min(kMaxSteps, ns - b0);
        u32x4 wv[kMaxSteps][RT], av[kMaxSteps][TT], al[kMaxSteps][LO ? TT : 1];
        // unconditional loads (indices clamped into the slice), so that the
        // arrays stay in registers
#pragma unroll
        for (int c = 0; c < kMaxSteps; ++c) {
            const int cc = c0 + b0 + (c < nb ? c : nb - 1);
#pragma unroll
            for (int i = 0; i < RT; ++i) wv[c][i] = wq[i][4 * cc];
#pragma unroll
            for (int j = 0; j < TT; ++j) {
                av[c][j] = *(const u32x4*)(aq[j] + 16 * cc);
                if constexpr (LO) al[c][j] = *(const u32x4*)(aql[j] + 16 * cc);
            }
        }
#pragma unroll
        for (int c = 0; c < kMaxSteps; ++c) {
            if (c >= nb) continue;
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                const u32x4 bv = bf16_pairs_p4(wv[c][i]);
#pragma unroll
                for (int j = 0; j < TT; ++j) {
                    f32x4 p = {0.f, 0.f, 0.f, 0.f};
                    p = mfma16(av[c][j], bv, p);
                    if constexpr (LO) p = mfma16(al[c][j], bv, p);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[i][j][v] += (double)p[v];
                }
            }
        }
    }
    // the k-slices are summed in slice order
    if (wave > 0)
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int j = 0; j < TT; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) red[wave - 1][(i * TT + j) * 4 + v][lane] = acc[i][j][v];
    __syncthreads();
    if (wave > 0) return;
#pragma unroll 1
    for (int w = 0; w < NW - 1; ++w)
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int j = 0; j < TT; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[i][j][v] += red[w][(i * TT + j) * 4 + v][lane];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int r = r0 + 16 * i + ml;
        if (r >= R) continue;
#pragma unroll
        for (int j = 0; j < TT; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + 16 * j + 4 * pc + v;
                if (t >= T) continue;
                const double z = acc[i][j][v];
                if (r < nr_router) a.logits_r[(size_t)t * a.E + r] = z;
                else if (r < nr_router + nr_head) a.logits_h[(size_t)t * a.En + (r - nr_router)] = z;
                else if (r < nr_router + nr_head + nr_lora) a.au[(size_t)t * a.r + (r - nr_router - nr_head)] = (float)z;
                else a.sgate[t] = (float)(1.0 / (1.0 + exp(-z)));
            }
    }
}

// The same products on operands stored in MFMA fragment order: for 16 rows
// (or tokens) and 32 hidden elements, one 1 KB block whose 16 bytes at 16 l
// are the 8 elements 8 (l / 16) .. of row l mod 16, so every load
// instruction reads 1 KB of contiguous memory (the row-major form makes each
// instruction touch 16 rows 4 KB apart, and the loads run at about half the
// rate). u comes so from the prologue; router, head, LoRA A and shared-gate
// rows are packed at layer creation, each set in tiles of its own 16 rows,
// pairs already in u's (p, p + 4) order. Block = one row tile x 16 tokens;
// the 4 waves take consecutive quarters of the k-steps, summed in order.
constexpr int kFrWaves = 4;

__global__ void __launch_bounds__(256) k_pack_rows(const uint16_t* w, int n, int d, uint32_t* out) {
    const int S = d / 32;
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;        // one 16-byte piece
    const long long total = (long long)((n + 15) / 16) * S * 64;
    if (i >= total) return;
    const int l = (int)(i & 63);
    const long long blk = i >> 6;
    const int c = (int)(blk % S), rt = (int)(blk / S);
    const int row = rt * 16 + (l & 15);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < n) v = bf16_pairs_p4(*(const u32x4*)(w + (size_t)row * d + 32 * c + 8 * (l >> 4)));
    *(u32x4*)(out + 4 * i) = v;
}

hipError_t launch_pack_rows(const uint16_t* w, int n, int d, uint32_t* out, hipStream_t s) {
    if (n <= 0 || d % 32) return hipErrorInvalidValue;
    const long long total = (long long)((n + 15) / 16) * (d / 32) * 64;
    hipLaunchKernelGGL(k_pack_rows, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, w, n, d, out);
    return hipGetLastError();
}

// row tiles of the four sets, in order: router, head, LoRA A, shared gate
struct FrSets {
    int n0, n1, n2, n3;
    __device__ __host__ int rows(int i) const { return i == 0 ? n0 : i == 1 ? n1 : i == 2 ? n2 : n3; }
    __device__ __host__ int tiles(int i) const { return (rows(i) + 15) / 16; }
    __device__ __host__ int total() const { return tiles(0) + tiles(1) + tiles(2) + tiles(3); }
};
__device__ __host__ __forceinline__ FrSets fr_sets(const RouteMMArgs& a) {
    return FrSets{a.router ? a.E : 0, a.head ? a.En : 0, a.lora_a ? a.r : 0, a.sgate_w ? 1 : 0};
}

__device__ __forceinline__ void route_mm_fr_body(const RouteMMArgs& a, int bx, int by) {
    __shared__ double red[kFrWaves - 1][4][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pc = lane >> 4, ml = lane & 15;
    const int d = a.d, T = a.n_tok, S = d / 32;
    const FrSets fs = fr_sets(a);
    int rt = bx, set = 0;
    while (set < 3 && rt >= fs.tiles(set)) { rt -= fs.tiles(set); ++set; }
    const int t0 = by * 16;
    // router rows are needed only for self-routed tokens
    if (set == 0 && !route_tile_needed(a, t0, 16)) return;
    const uint32_t* wf = set == 0 ? a.wf_router : set == 1 ? a.wf_head : set == 2 ? a.wf_lora : a.wf_sgate;
    const u32x4* wq = (const u32x4*)wf + (size_t)rt * S * 64 + lane;
    const u32x4* aq = (const u32x4*)a.u_frag + (size_t)by * S * 64 + lane;
    // wave w takes k-steps [w * ns, (w + 1) * ns), loads issued 16 steps at a time
    const int ns = S / kFrWaves, c0 = wave * ns;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int b0 = 0; b0 < ns; b0 += 16) {
        const int nb = min(16, ns - b0);
        u32x4 wv[16], av[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int cc = c0 + b0 + (c < nb ? c : nb - 1);
            wv[c] = wq[64 * cc];
            av[c] = aq[64 * cc];
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            if (c >= nb) continue;
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
            p = mfma16(av[c], wv[c], p);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] += (double)p[v];
        }
    }
    if (wave > 0)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave - 1][v][lane] = acc[v];
    __syncthreads();
    // router rows of the first token tile when it holds rows before the shift
    const bool pre = set == 0 && by == 0 && a.pre_rows > 0;
    const int r = 16 * rt + ml;                          // row within its set
    if (wave == 0 && r < fs.rows(set)) {
#pragma unroll 1
        for (int w = 0; w < kFrWaves - 1; ++w)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] += red[w][v][lane];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int t = t0 + 4 * pc + v;
            if (t >= T) continue;
            const double z = acc[v];
            if (set == 0) {
                if (pre) st_dev(a.logits_r + (size_t)t * a.E + r, z);   // read by another block below
                else a.logits_r[(size_t)t * a.E + r] = z;
            } else if (set == 1) a.logits_h[(size_t)t * a.En + r] = z;
            else if (set == 2) a.au[(size_t)t * a.r + r] = (float)z;
            else a.sgate[t] = (float)(1.0 / (1.0 + exp(-z)));
        }
    }
    if (!pre) return;
    // the last of these blocks to finish takes the top-k of rows 0 .. pre_rows-1
    // (device-scope stores, a barrier, a device-scope release fence, then the
    // count; the last block acquires and reads every block's logits with
    // coherent loads)
    __shared__ int is_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const unsigned old = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = old == (unsigned)fs.tiles(0) - 1;
        if (is_last) {
            __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
    }
    __syncthreads();
    if (!is_last) return;
    for (int t = wave; t < a.pre_rows; t += kFrWaves) {
        if (a.E <= 64) topk_row<1>(true, a.logits_r, a.E, a.k, t, a.router_bias, nullptr, nullptr, nullptr, nullptr, a.self_idx, a.self_w);
        else if (a.E <= 128) topk_row<2>(true, a.logits_r, a.E, a.k, t, a.router_bias, nullptr, nullptr, nullptr, nullptr, a.self_idx, a.self_w);
        else topk_row<4>(true, a.logits_r, a.E, a.k, t, a.router_bias, nullptr, nullptr, nullptr, nullptr, a.self_idx, a.self_w);
    }
}

__global__ void __launch_bounds__(64 * kFrWaves) k_route_mm_fr(RouteMMArgs a) {
    route_mm_fr_body(a, blockIdx.x, blockIdx.y);
}

// Gate/up and the routing-side GEMM of the same layer in one launch, for
// calls whose routing is given and already sorted (batched stack decode):
// nothing the routing GEMM writes (head logits, LoRA A u, shared gate) is
// read before the combine, so its blocks run beside the gate/up blocks
// instead of in a launch of their own ahead of them. Blocks [0, gx gy) are
// gate/up tiles (x fastest, as in k_pf_gateup's grid), the rest routing tiles.
static_assert(64 * kFrWaves == 256, "one block size for both bodies");
template <int NB>
__global__ void __launch_bounds__(256) k_pf_gateup_route(PrefillArgs a, RouteMMArgs r, int gx, int gy) {
    const int b = blockIdx.x, ng = gx * gy;
    if (b < ng) {
        gateup_body<false, NB>(a, b % gx, b / gx);
        return;
    }
    const int rx = fr_sets(r).total();
    route_mm_fr_body(r, (b - ng) % rx, (b - ng) / rx);
}

// The same products for many tokens: block = 64 tokens x 64 rows staged
// through LDS 64 elements of k at a time (the next stage's loads in flight
// while the current one is multiplied); wave (wm, wn) computes tokens
// 32 wm .. + 31 x rows 32 wn .. + 31. Same per-step fp32 / fp64 split.
constexpr int kRmTile = 64;                  // tokens and rows per block
constexpr int kRmK = 64;                     // hidden elements per stage (2 k-steps)

__global__ void __launch_bounds__(256) k_route_mm_tiled(RouteMMArgs a) {
    // [token or row][piece of 8 elements], padded by one piece against bank conflicts
    __shared__ __align__(16) u32x4 sa[2][kRmTile][kRmK / 8 + 1], sl[2][kRmTile][kRmK / 8 + 1], sw[2][kRmTile][kRmK / 8 + 1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ml = lane & 15, pc = lane >> 4;
    const int d = a.d, T = a.n_tok;
    const int nr_router = a.router ? a.E : 0, nr_head = a.head ? a.En : 0;
    const int nr_lora = a.lora_a ? a.r : 0;
    const int R = nr_router + nr_head + nr_lora + (a.sgate_w ? 1 : 0);
    const int t0 = blockIdx.y * kRmTile, r0 = blockIdx.x * kRmTile;
    if (r0 + kRmTile <= nr_router && !route_tile_needed(a, t0, kRmTile)) return;
    const bool lo = a.u_pk_lo != nullptr;
    // this thread's two load pieces of each stage: row/token q >> 3, piece q & 7
    const uint32_t* ap[2];
    const uint32_t* alp[2];
    const uint16_t* wp[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = tid + 256 * j, rr = q >> 3, pcs = q & 7;
        const int tok = t0 + rr < T ? t0 + rr : T - 1;
        ap[j] = a.u_pk + (size_t)tok * (d / 2) + 4 * pcs;
        alp[j] = lo ? a.u_pk_lo + (size_t)tok * (d / 2) + 4 * pcs : ap[j];
        int row = r0 + rr < R ? r0 + rr : R - 1;
        const uint16_t* w;
        if (row < nr_router) w = a.router + (size_t)row * d;
        else if (row < nr_router + nr_head) w = a.head + (size_t)(row - nr_router) * d;
        else if (row < nr_router + nr_head + nr_lora) w = a.lora_a + (size_t)(row - nr_router - nr_head) * d;
        else w = a.sgate_w;
        wp[j] = w + 8 * pcs;
    }
    u32x4 ra[2], rl[2], rw[2];
    auto load = [&](int st) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            ra[j] = *(const u32x4*)(ap[j] + st * (kRmK / 2));
            rw[j] = *(const u32x4*)(wp[j] + st * kRmK);
            rl[j] = lo ? *(const u32x4*)(alp[j] + st * (kRmK / 2)) : u32x4{0, 0, 0, 0};
        }
    };
    auto store = [&](int b) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int q = tid + 256 * j, rr = q >> 3, pcs = q & 7;
            sa[b][rr][pcs] = ra[j];
            sw[b][rr][pcs] = bf16_pairs_p4(rw[j]);
            if (lo) sl[b][rr][pcs] = rl[j];
        }
    };
    // wave (wm, wn): tokens 32 wm + 16 i, rows 32 wn + 16 j
    const int wm = wave & 1, wn = wave >> 1;
    double acc[2][2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0;
    const int NS = d / kRmK;
    load(0);
    store(0);
    __syncthreads();
    for (int st = 0; st < NS; ++st) {
        const int b = st & 1;
        if (st + 1 < NS) load(st + 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            u32x4 av[2], alv[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                av[i] = sa[b][32 * wm + 16 * i + ml][4 * ks + pc];
                alv[i] = lo ? sl[b][32 * wm + 16 * i + ml][4 * ks + pc] : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) bv[j] = sw[b][32 * wn + 16 * j + ml][4 * ks + pc];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    f32x4 p = {0.f, 0.f, 0.f, 0.f};
                    p = mfma16(av[i], bv[j], p);
                    if (lo) p = mfma16(alv[i], bv[j], p);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[i][j][v] += (double)p[v];
                }
        }
        if (st + 1 < NS) store((st + 1) & 1);
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = r0 + 32 * wn + 16 * j + ml;
        if (r >= R) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + 32 * wm + 16 * i + 4 * pc + v;
                if (t >= T) continue;
                const double z = acc[i][j][v];
                if (r < nr_router) a.logits_r[(size_t)t * a.E + r] = z;
                else if (r < nr_router + nr_head) a.logits_h[(size_t)t * a.En + (r - nr_router)] = z;
                else if (r < nr_router + nr_head + nr_lora) a.au[(size_t)t * a.r + (r - nr_router - nr_head)] = (float)z;
                else a.sgate[t] = (float)(1.0 / (1.0 + exp(-z)));
            }
    }
}

// top-k per token: job (blockIdx.y + job0) 0 router (self-routed rows), 1 head
__global__ void __launch_bounds__(256) k_route_topk(RouteMMArgs a, int job0) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.n_tok) return;
    if ((int)blockIdx.y + job0 == 0) {
        if (!a.router || (a.route_idx && t >= a.route_shift && a.route_idx[(size_t)(t - a.route_shift) * a.k] >= 0))
            return;
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

// whether launch_route_mm would take k_route_mm_fr for these arguments
bool route_fr_ok(const RouteMMArgs& a) {
    const int R = (a.router ? a.E : 0) + (a.head ? a.En : 0) + (a.lora_a ? a.r : 0) + (a.sgate_w ? 1 : 0);
    const long long big_blocks = (long long)((R + kRmTile - 1) / kRmTile) * ((a.n_tok + kRmTile - 1) / kRmTile);
    return R > 0 && a.d % 128 == 0 && big_blocks < 512 && a.u_frag && !a.u_pk_lo && a.d % (32 * kFrWaves) == 0 &&
           (!a.router || a.wf_router) && (!a.head || a.wf_head) && (!a.lora_a || a.wf_lora) && (!a.sgate_w || a.wf_sgate);
}

hipError_t launch_route_mm(const RouteMMArgs& a_in, hipStream_t s, bool router_topk, bool head_topk, int* pre_done) {
    RouteMMArgs a = a_in;
    if (pre_done) *pre_done = 0;
    if (a.d % 128) return hipErrorInvalidValue;
    const int R = (a.router ? a.E : 0) + (a.head ? a.En : 0) + (a.lora_a ? a.r : 0) + (a.sgate_w ? 1 : 0);
    if (R > 0) {
        // 64 x 64 LDS tiles once they alone fill the chip twice over
        const long long big_blocks = (long long)((R + kRmTile - 1) / kRmTile) * ((a.n_tok + kRmTile - 1) / kRmTile);
        if (big_blocks >= 512)
            hipLaunchKernelGGL(k_route_mm_tiled, dim3((R + kRmTile - 1) / kRmTile, (a.n_tok + kRmTile - 1) / kRmTile),
                               dim3(256), 0, s, a);
        else if (a.u_frag && !a.u_pk_lo && a.d % (32 * kFrWaves) == 0 && (!a.router || a.wf_router) &&
                 (!a.head || a.wf_head) && (!a.lora_a || a.wf_lora) && (!a.sgate_w || a.wf_sgate)) {
            // the top-k of the rows before the shift, when asked for and possible
            if (!(a.pre_rows > 0 && a.pre_rows <= 16 && a.router && a.E <= 256 && a.counter && a.self_idx)) a.pre_rows = 0;
            if (a.pre_rows > a.n_tok) a.pre_rows = a.n_tok;
            hipLaunchKernelGGL(k_route_mm_fr, dim3(fr_sets(a).total(), (a.n_tok + 15) / 16), dim3(64 * kFrWaves), 0, s, a);
            if (pre_done) *pre_done = a.pre_rows;
        } else {
            a.pre_rows = 0;
            const dim3 grid((R + 15) / 16, (a.n_tok + 15) / 16);
            if (a.u_pk_lo) hipLaunchKernelGGL((k_route_mm<1, 1, 4, true>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((k_route_mm<1, 1, 4, false>), grid, dim3(256), 0, s, a);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_route_topk(a, s, router_topk, head_topk);
}

hipError_t launch_route_topk(const RouteMMArgs& a, hipStream_t s, bool router_topk, bool head_topk) {
    router_topk = router_topk && a.router;
    head_topk = head_topk && a.head && a.pred_idx;
    if (router_topk || head_topk) {
        hipLaunchKernelGGL(k_route_topk, dim3((a.n_tok + 3) / 4, (router_topk ? 1 : 0) + (head_topk ? 1 : 0)), dim3(256), 0, s,
                           a, router_topk ? 0 : 1);
        return hipGetLastError();
    }
    return hipSuccess;
}

bool prefill_mm_ok(int d, int f, int fs) {
    auto fok = [](int x) { return x == 256 || x == 512; };    // the down projection's stage widths
    return d % kStageK == 0 && d % 128 == 0 && d / 64 <= kMaxGroupsPf && fok(f) && (fs == 0 || fok(fs));
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s, const RouteMMArgs* route) {
    const GemvArgs& g = a.g;
    if (!prefill_mm_ok(g.d, g.f, g.fs)) return hipErrorInvalidValue;
    hipError_t e;
    const int fmax = g.f > g.fs ? g.f : g.fs;
    const bool big = prefill_big_tiles(g.d, g.f, g.fs, g.u_pk_lo != nullptr, g.n_tok, g.k, g.max_active);
    // routing GEMM handed over (its results are read from the combine on):
    // in the gate/up launch when both take their 16-token forms, else ahead
    if (route && (big || g.u_pk_lo || route->pre_rows > 0 || !route_fr_ok(*route))) {
        if ((e = launch_route_mm(*route, s, false, false, nullptr)) != hipSuccess) return e;
        route = nullptr;
    }
    // the tile lists were written by the sort (64-row ones when big)
    if (route) {
        const int gx = a.max_tiles, gy = (fmax + kGuRows - 1) / kGuRows;
        const int nr = fr_sets(*route).total() * ((route->n_tok + 15) / 16);
        const dim3 grid((unsigned)(gx * gy + nr));
        if ((long long)g.n_tok * g.k >= 4LL * g.max_active)
            hipLaunchKernelGGL(k_pf_gateup_route<1>, grid, dim3(256), 0, s, a, *route, gx, gy);
        else
            hipLaunchKernelGGL(k_pf_gateup_route<2>, grid, dim3(256), 0, s, a, *route, gx, gy);
    } else if (big) {
        hipLaunchKernelGGL((k_pf_gateup_big<kBgGs, kBgNst, kTileBig, kBgRt, kBgWaves>), dim3(a.max_tiles64, (fmax + kBgRows - 1) / kBgRows),
                           dim3(64 * kBgWaves), 0, s, a);
    } else {
        const dim3 ggrid(a.max_tiles, (fmax + kGuRows - 1) / kGuRows);
        // one stage buffer once the experts average 4 or more tokens
        const bool many = (long long)g.n_tok * g.k >= 4LL * g.max_active;
        if (g.u_pk_lo) {
            if (many) hipLaunchKernelGGL((k_pf_gateup<true, 1>), ggrid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((k_pf_gateup<true, 2>), ggrid, dim3(256), 0, s, a);
        } else {
            if (many) hipLaunchKernelGGL((k_pf_gateup<false, 1>), ggrid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((k_pf_gateup<false, 2>), ggrid, dim3(256), 0, s, a);
        }
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        // enough blocks that none spans more than kDnTiles tiles: a block
        // takes at most ceil(Z / nb) stages and a tile has at least ns_min
        const long long nsr = dn_tile_stages(g.d, g.f), nss = g.fs ? dn_tile_stages(g.d, g.fs) : nsr;
        const long long z_max = (long long)a.max_tiles * (nsr > nss ? nsr : nss);
        const long long per = (long long)(kDnTiles - 2) * (nsr < nss ? nsr : nss) + 1;
        long long nb = a.n_cu > 0 ? a.n_cu : 1;
        if (nb * per < z_max) nb = (z_max + per - 1) / per;
        hipLaunchKernelGGL(k_pf_down, dim3((unsigned)nb), dim3(kDnThreads), 0, s, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        // combine blocks, then the head top-k blocks (one token per wave)
        if (combine_norm_ok(a)) {
            const int gy = (g.n_tok + kCnTok - 1) / kCnTok;
            const int gt = a.head.pred_idx ? (g.n_tok + kCnThreads / 64 - 1) / (kCnThreads / 64) : 0;
            hipLaunchKernelGGL(k_pf_combine_norm, dim3(gy + gt), dim3(kCnThreads), 0, s, a);
        } else {
            const int gy = (g.n_tok + kCombTok - 1) / kCombTok;
            const int gx = (g.d + 1023) / 1024;
            const int gt = a.head.pred_idx ? ((g.n_tok + 3) / 4 + gx - 1) / gx : 0;
            hipLaunchKernelGGL(k_pf_combine, dim3(gx, gy + gt), dim3(256), 0, s, a);
        }
    }
    return hipGetLastError();
}

bool combine_norm_ok(const PrefillArgs& a) {
    const PrologueArgs& p = a.nxt;
    // measured: one launch instead of two pays for 32 tokens (batched decode
    // 2.36 against 2.48 ms per 40-layer step); at 512 tokens the two forms tie
    return p.u_pk && p.usum && p.gamma && p.fused && a.g.fused && p.d == a.g.d && p.n_tok == a.g.n_tok &&
           a.g.d % 32 == 0 && a.g.d <= 4 * kCnThreads && a.g.n_tok <= kCnMaxTok;
}

bool prefill_big_tiles(int d, int f, int fs, bool act_lo, int n_tok, int k, int max_active) {
    // many tokens per expert (on average 48 or more): 64-token tiles for gate/up
    return !act_lo && d <= 2048 && d % 128 == 0 && f % kBgRows == 0 && (fs == 0 || fs % kBgRows == 0) &&
           (long long)n_tok * k >= 48LL * max_active;
}

}  // namespace moe

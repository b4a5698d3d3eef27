// Internal structures of the MoE block library (host + device).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_prerouter.h"
#include <hip/hip_ext.h>

namespace moe {

// Optional kernel timestamps: when set, the launch records the kernel's own
// start and end (the dispatch's begin/end timestamps), not the stream gaps.
struct KTime {
    hipEvent_t start = nullptr, stop = nullptr;
};
#define MOE_LAUNCH(kern, grid, block, shm, stream, tm, ...)                                                  \
    do {                                                                                                     \
        if ((tm) && (tm)->start)                                                                             \
            hipExtLaunchKernelGGL(kern, grid, block, shm, stream, (tm)->start, (tm)->stop, 0, __VA_ARGS__);  \
        else                                                                                                 \
            hipLaunchKernelGGL(kern, grid, block, shm, stream, __VA_ARGS__);                                 \
    } while (0)

constexpr int kGroup = 64;
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 1024;

// device error flag bits (sticky until read by the host)
enum : int { ERR_NOT_STAGED = 1, ERR_BAD_INDEX = 2, ERR_TIMEOUT = 4 };

// Where a layer's expert weights are found on the device.
struct ExpertView {
    const uint8_t* base;          // slab (streamed) or store (resident)
    const int32_t* slot_of;       // [E] slot per expert, -1 absent (streamed); nullptr: slot = expert
    const int32_t* slot_tag;      // [slots] expert held per slot (streamed); nullptr: no check
    const uint8_t* shared;        // shared blob (device) or nullptr
    const int32_t* shared_tag;    // streamed: tag of the shared slot (== E when staged); nullptr: no check
    size_t blob;                  // bytes per routed blob
    size_t shared_blob;           // bytes of the shared blob
    int E;
};

// Byte offsets inside a blob (see the format in moe_prerouter.h).
struct BlobLayout {
    size_t gate_q, up_q, down_q, gate_sb, up_sb, down_sb, total;
    __host__ __device__ static BlobLayout make(int d, int f) {
        BlobLayout L;
        const size_t q = (size_t)d * f / 2, sb = (size_t)d * f / kGroup * 4;
        L.gate_q = 0; L.up_q = q; L.down_q = 2 * q;
        L.gate_sb = 3 * q; L.up_sb = 3 * q + sb; L.down_sb = 3 * q + 2 * sb;
        L.total = 3 * q + 3 * sb;
        return L;
    }
};

// Device scratch of one layer (carved from the caller's workspace).
struct Scratch {
    int32_t* err;            // [1] sticky error flag
    uint32_t* counters;      // [16] last-block counters (self-resetting)
    int32_t* slot_of;        // [nbuf][E]
    int32_t* slot_tag;       // [nbuf][slots + 1]; entry `slots` is the shared slot
    uint8_t* slab;           // [nbuf][(slots + 1) * blob] (streamed); shared slot last
    int32_t* stage_plan;     // [nbuf][stage_plan_ints(slots)]: device staging scratch
    unsigned long long* stage_bytes;   // [1]: bytes staged by device staging
    uint32_t* u_pk;          // [T][d/2] bf16 pairs, GEMV order (hi part)
    uint32_t* u_pk_lo;       // [T][d/2] lo part (f32 act) or nullptr
    uint32_t* u_frag;        // [T/16][d/32][64 lanes][4]: u_pk in MFMA fragment order (bf16 act), or nullptr
    uint32_t* wf_router;     // routing-side bf16 rows in MFMA fragment order (packed at create):
    uint32_t* wf_head;       //   [rows/16][d/32][64 lanes][4], rows padded to 16 with zeros
    uint32_t* wf_lora;
    uint32_t* wf_sgate;
    float* usum;             // [T][d/32] sums of hi part per 32-chunk
    float* usum_lo;          // [T][d/32] or nullptr
    double* logits_r;        // [T][E] router logits
    double* logits_h;        // [T][E_next] head logits
    int32_t* self_idx;       // [T][k]
    float* self_w;           // [T][k]
    int32_t* used_idx;       // [T][k]
    float* used_w;           // [T][k]
    float* au;               // [T][r]  A u
    float* sgate;            // [T]     sigmoid(g . u)
    int32_t* sort_meta;      // [4]: n_active, n_assign, ...
    int32_t* active;         // [min(E, T*k)] active experts ascending
    int32_t* act_off;        // [.. + 1] start of each active expert's assignments
    int32_t* perm;           // [T*k] assignment ids (t*k + j) sorted by (expert, id)
    float* wsort;            // [T*k] routing weight of each sorted assignment
    float* h;                // [T*k][f] routed expert hidden (sorted order)
    float* hs;               // [T][fs] shared expert hidden
    int32_t* tiles;          // prefill: grouped-GEMM work list, 4 ints per tile (16-row tiles)
    int32_t* tiles64;        // the same with 64-row tiles (many tokens per expert)
    float* ob;               // prefill: [T*k][d] routed expert outputs by assignment
    float* obs;              // prefill: [T][d] shared expert outputs
    float* sau;              // shared-expert LoRA: [T][2 rs] A_g u, A_u u
    uint32_t* wf_slora;      // shared-expert LoRA: A rows in MFMA fragment order (bf16 act)
    double* a1;              // head MLP: [T][H1] fc1 hidden-state part
    uint32_t* wf_fc1;        // head MLP: fc1 hidden-state rows in MFMA fragment order (bf16 act)
};

}  // namespace moe

struct moe_layer {
    moe_layer_desc desc;
    moe_layer_weights w;
    moe::Scratch s;
    moe::BlobLayout L, Ls;
    size_t blob, sblob;
    int slots;                 // routed slots (streamed)
    bool resident;
    int n_cu;                  // compute units of the device (persistent kernels)
    int dev;
    // host mirror of the slab
    int32_t* h_slot_expert;    // [slots]
    int32_t* h_last_staged;    // [slots] last wanted set (sorted, -1 padded)
    int n_last_staged;
    bool shared_staged;
    uint64_t staged_bytes;
    hipEvent_t ev_staged, ev_done;
    bool done_recorded;
    // slab buffers (2 with MOE_DOUBLE_SLAB), the one calls read, device staging
    int nbuf, cur_buf;
    hipEvent_t ev_staged_buf[2];
    bool staged_pending_buf[2];
    bool dev_staging;          // MOE_DEVICE_STAGING: reactive staging runs on the device
    const uint8_t* store_dev;  // device address of the pinned store (streamed), or nullptr
    const uint8_t* shared_dev;
    hipEvent_t ev_pred;        // recorded once this call's predictions are final (stack staging)
    int32_t* h_readback;       // pinned [max_tokens * k]
    // kernel timing (profiling mode)
    bool profiling;
    hipEvent_t ev_t[6];        // router start/end, A start/end, B start/end
    bool ev_t_used[3];
    bool presorted;            // set by the stack around a call whose sort already ran
};

namespace moe {
struct StackLayerArgs;
struct SortArgs;
}
struct moe_stack {
    moe_layer** layers;
    int n;
    // device staging driven by the stack (moe_stack_set_staging)
    int stage_mode;          // 0 off, MOE_STAGE_PREROUTED, MOE_STAGE_ON_DEMAND
    hipStream_t copy_stream;
    long long step;
    // prefill scratch (caller's workspace): two prediction buffers, layer l
    // writing buffer l & 1 while it reads layer l-1's from the other one
    int32_t* d_pred_idx[2];
    float* d_pred_w[2];
    size_t pred_cap;         // entries per buffer
    // optional trace of every layer's input residual stream (device fp32)
    float* x_trace;
    size_t trace_cap;        // floats
    // one launch per decode step (moe_stack_set_one_launch)
    moe::StackLayerArgs* d_tab;   // [n] per-layer arguments (caller's workspace)
    float* d_xchg;           // per layer: copies of the activations handed between phases
    size_t xchg_stride;      // floats per copy
    size_t xchg_off[5];      // offsets in a copy: x, h, hs, au, sgate
    int xchg_tokens;         // tokens a copy holds
    uint32_t* d_sync;        // stack_sync_words(n) counters, zero between launches
    bool one_ok;             // the layers qualify (resident, identical fast-path shapes)
    bool one_launch;         // enabled
    int one_grid;            // blocks resident on the chip at once
    uint32_t wait_polls;     // bound of each device-side wait (polls)
    // batched decode beyond the fused path: layers 1..n-1 sort their given
    // routing in one launch at the start of the step
    moe::SortArgs* d_sort_tab;    // [n - 1] fixed sort arguments of layers 1..n-1 (caller's workspace)
    bool sort_ok;            // every layer resident with the same shape
    // kernel timestamps (moe_stack_set_profiling): layer 0's router, the step kernel
    bool profiling;
    bool ev_used[2];
    hipEvent_t ev_t[4];
};

// ---- kernel launchers (kernels_*.hip) -------------------------------------
namespace moe {

struct PrologueArgs {
    const void* x; int x_is_bf16; int fused; const float* gamma; float eps;
    int act_bf16; int d; int n_tok;
    uint32_t* u_pk; uint32_t* u_pk_lo; float* usum; float* usum_lo;
    uint32_t* u_frag;                   // or nullptr
};
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s);

struct RouteArgs {
    // router (self-routing rows) and head (prediction) logits + top-k, plus
    // LoRA A u and the shared gate, all from bf16 weights on the block input
    int d; int n_tok;
    const uint16_t* router; const float* router_bias; int E; int k;
    const int32_t* route_idx;           // rows to self-route: idx[t*k] < 0 or route_idx == nullptr
    int route_shift;                    // 1: token t takes row t - 1 of route_idx, token 0 self-routes
    const uint16_t* head; const float* head_bias; int En; int kn;
    const float* hist_cur_m; const float* hist_prev_m; const int32_t* hist_cur; const int32_t* hist_prev;
    const uint16_t* lora_a; int r;
    const uint16_t* sgate_w;
    double* logits_r; double* logits_h;
    int32_t* self_idx; float* self_w; int32_t* pred_idx; float* pred_w;
    float* au; float* sgate;
    uint32_t* counters;
};

// routing-side GEMM for many tokens (prefill, large decode batches)
struct RouteMMArgs {
    const uint32_t* u_pk; const uint32_t* u_pk_lo; int d; int n_tok;
    const uint16_t* router; const float* router_bias; int E; int k;
    const int32_t* route_idx;           // rows to self-route: idx[t*k] < 0 or route_idx == nullptr
    int route_shift;                    // 1: token t takes row t - 1 of route_idx, token 0 self-routes
    const uint16_t* head; const float* head_bias; int En; int kn;
    const float* hist_cur_m; const float* hist_prev_m; const int32_t* hist_cur; const int32_t* hist_prev;
    const uint16_t* lora_a; int r;
    const uint16_t* sgate_w;
    double* logits_r; double* logits_h;
    int32_t* self_idx; float* self_w; int32_t* pred_idx; float* pred_w;
    float* au; float* sgate;
    // fragment-ordered operands (both or neither; bf16 activations): u, and
    // the packed rows of router / head / LoRA A / shared gate (non-null where
    // the plain pointer above is)
    const uint32_t* u_frag;
    const uint32_t* wf_router; const uint32_t* wf_head; const uint32_t* wf_lora; const uint32_t* wf_sgate;
    // rows 0 .. pre_rows-1 (before the routing shift; at most 16, E <= 256):
    // the last router block of the first token tile takes their top-k into
    // self_idx / self_w (fragment-order kernel only); counter: zero between calls
    int pre_rows; uint32_t* counter;
};
// pack n bf16 rows of length d into MFMA fragment order (rows padded to 16)
hipError_t launch_pack_rows(const uint16_t* w, int n, int d, uint32_t* out, hipStream_t s);
inline size_t frag_rows_words(int n, int d) { return (size_t)((n + 15) / 16) * 16 * d / 2; }
// router_topk: top-k of the self-routed rows here (else the sort does it);
// head_topk: the head's top-k here (else the combine launch does it)
// *pre_done: how many of the requested a.pre_rows rows got their top-k here
hipError_t launch_route_mm(const RouteMMArgs& a, hipStream_t s, bool router_topk, bool head_topk, int* pre_done);

// The head's MLP branch after fc1's hidden-state part (a1, from the routing
// GEMM): per token, add fc1's one-hot columns and bias, erf-GELU, then fc2
// into the head logits (which then hold l(x) + fc2(gelu(fc1(x)))).
constexpr int kMaxHeadHidden = 1024;
struct HeadMlpArgs {
    const double* a1; int H1;
    const uint16_t* w1oh; const float* b1; const uint16_t* w2;
    const int32_t* hc; const int32_t* hp; int kn; int En;
    double* logits; int n_tok;
};
hipError_t launch_head_mlp_out(const HeadMlpArgs& a, hipStream_t s);
// The shared expert with the recovery LoRA on its projections.
struct SharedLoraArgs {
    const uint8_t* blob;                 // shared expert blob (device)
    const int32_t* tag; int tag_want;    // streamed: the shared slot's tag must equal tag_want; nullptr: no check
    int d; int f; int rs; float scale;
    const uint32_t* u_pk; const uint32_t* u_pk_lo;   // the prologue's u (pair order), lo part or nullptr
    const float* sau;                    // [T][2 rs]: A_g u, then A_u u
    const uint16_t* b_gu;                // [2 f][rs]: B of gate, then B of up
    const uint16_t* ad;                  // [rs][f]
    const uint16_t* bd;                  // [d][rs]
    const float* sgate;                  // [T] or nullptr (gate 1)
    float* hs;                           // [T][f]
    float* y;                            // [T][d], added to
    int n_tok;
    int32_t* err;
};
hipError_t launch_shared_lora(const SharedLoraArgs& a, hipStream_t s, bool gateup, bool down);

// the routing GEMM's per-token top-k launch alone (router and / or head)
hipError_t launch_route_topk(const RouteMMArgs& a, hipStream_t s, bool router_topk, bool head_topk);

// A head top-k run by a later launch than the one that wrote its logits
// (only for E_next <= 64 * kDeferMaxPer; larger heads keep their own launch).
constexpr int kDeferMaxPer = 4;
struct TopkJob {
    const double* logits; int En; int kn; const float* bias;
    const float* mc; const int32_t* hc; const float* mp; const int32_t* hp;
    int32_t* pred_idx; float* pred_w;
};

constexpr int kSortTopkMaxE = 256;
struct SortArgs {
    const int32_t* route_idx; const float* route_w; int32_t* self_idx; float* self_w;
    int route_shift;                    // 1: token t takes row t - 1 of the given routing, token 0 self-routes
    int pre_rows;                       // rows whose top-k an earlier launch wrote to self_idx / self_w
    int n_tok; int k; int E;
    int32_t* used_idx; float* used_w; int32_t* user_used_idx; float* user_used_w;
    int32_t* meta; int32_t* active; int32_t* act_off; int32_t* perm;
    int32_t* err;
    // when set: the top-k of the self-routed rows (route_idx[t*k] < 0) from
    // the router logits, written to self_idx / self_w before the sort reads them
    bool self_topk; const double* logits_r; const float* router_bias;   // self_topk: E <= kSortTopkMaxE
    // when set: the grouped GEMM's tile lists (16-row, and 64-row if tiles64),
    // records {active slot or -1 (shared), first position, rows, blob}, with
    // meta[2] = tiles, meta[3] = routed tiles (meta[4], meta[5]: 64-row)
    ExpertView ev; int fs; int32_t* tiles16; int32_t* tiles64;
    bool resolve_blobs;                 // false: blob fields left -1, resolved after staging (launch_tile_blobs)
};
hipError_t launch_sort(const SortArgs& a, hipStream_t s);
// one call's part of several layers' sorts (k_sort_layers): routing
// [layer][n_tok][k] from route_idx / route_w (per = n_tok * k entries per
// layer), optional used-routing outputs of the same shape
struct SortCall {
    const int32_t* route_idx; const float* route_w; int32_t* used_idx; float* used_w;
    size_t per; int n_tok; int big;
};
hipError_t launch_sort_layers(const SortArgs* tab, int n_layers, int E, const SortCall& c, hipStream_t s);

struct GemvArgs {
    ExpertView ev; int d; int f; int fs; int k; int n_tok;
    const int32_t* meta; const int32_t* active; const int32_t* act_off; const int32_t* perm;
    const float* used_w; const float* sgate;
    const uint32_t* u_pk; const uint32_t* u_pk_lo; const float* usum; const float* usum_lo;
    float* h; float* hs;
    // down / epilogue
    const float* x; int fused; const float* au; const uint16_t* lora_b; int r; float lora_scale;
    float* y;
    int32_t* err;
    int max_active;
};
hipError_t launch_gateup(const GemvArgs& a, hipStream_t s);
hipError_t launch_down(const GemvArgs& a, hipStream_t s);

struct PrefillArgs {
    GemvArgs g;
    // work list of the grouped GEMM, one tile = {slot (-1: shared expert),
    // first position, rows (<= 16), blob (>= 0: index in the store or slab,
    // -2: shared blob, -1: not staged)}
    int32_t* tiles; int max_tiles;
    int32_t* tiles64; int max_tiles64;   // 64-row tiles (large-tile gate/up)
    const int32_t* meta_w;               // meta[2] = tiles, meta[3] = routed tiles (meta[4], [5]: 64-row), from the sort
    int n_cu;                            // blocks of the persistent down projection
    float* ob; float* obs;               // down outputs: [T*k][d] by assignment, [T][d] shared
    const int32_t* used_idx; const float* used_w;
    TopkJob head;                        // the head's top-k, run beside the combine (pred_idx null: none)
    PrologueArgs nxt;                    // the next stacked layer's prologue, taken by the combine (u_pk null: none)
};
// whether the combine takes a.nxt (the next layer then launches no prologue)
bool combine_norm_ok(const PrefillArgs& a);
int prefill_max_tiles(int T, int K, int E, int tm = 16);
bool prefill_mm_ok(int d, int f, int fs);
// whether the gate/up projection takes 64-token tiles (many tokens per expert)
bool prefill_big_tiles(int d, int f, int fs, bool act_lo, int n_tok, int k, int max_active);
// route (optional): the layer's routing-side GEMM, whose outputs nothing
// before the combine reads; it runs in the gate/up launch when it can, else
// just before it. Its top-k steps are the caller's (none may be pending).
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s, const RouteMMArgs* route = nullptr);
bool route_fr_ok(const RouteMMArgs& a);
// resolve the blob field of the tile records once the experts are staged
hipError_t launch_tile_blobs(const PrefillArgs& a, bool big, hipStream_t s);


struct DecAArgs {
    const void* x; int x_is_bf16; int fused; const float* gamma; float eps; int act_bf16; int d; int n_tok;
    const int32_t* route_idx; const float* route_w;   // given routing (rows with idx < 0: self) or nullptr
    const int32_t* self_idx; const float* self_w;     // router result for self rows, or nullptr
    int k; int E;
    ExpertView ev; int f; int fs;
    const uint16_t* head; int En;
    const uint16_t* lora_a; int r; const uint16_t* sgate_w;
    float* h; float* hs; double* logits_h; float* au; float* sgate;
    int32_t* meta; int32_t* active; int32_t* act_off; int32_t* perm; float* wsort;
    int32_t* used_idx; float* used_w; int32_t* user_used_idx; float* user_used_w;
    int32_t* err;
    int nb_h, nb_head, nb_misc;
    TopkJob topk;          // pred_idx == nullptr: none
    // one-launch stack decode: h, hs, au and sgate are written to xcopies
    // copies xstride floats apart, and x is read from one of them (0: unused)
    size_t xstride; int xcopies;
    int x_repl;            // x is read from the exchange copies too (else from a.x itself)
};
hipError_t launch_dec_a(const DecAArgs& a, hipStream_t s, const KTime* tm = nullptr);
bool dec_fast_path_ok(int d, int f, int fs, int n_tok, int k);
int dec_a_hrows_per_block(int d);
int dec_b_rows_per_block(int f);
hipError_t launch_dec_r(const DecAArgs& a, const RouteArgs& r, hipStream_t s, const KTime* tm = nullptr);
int dec_a_blocks(int d, int f, int fs, int n_tok, int k, int E, int En, int r, bool sgate, int* nb_h, int* nb_head,
                 int* nb_misc);

struct DecBArgs {
    ExpertView ev; int d; int f; int fs; int k; int n_tok; int E;
    const int32_t* route_idx; const float* route_w; const int32_t* self_idx; const float* self_w;
    const float* sgate; const float* h; const float* hs;
    const float* x; int fused; const float* au; const uint16_t* lora_b; int r; float lora_scale;
    float* y;
    float* y_copy;         // one-launch stack decode: a second copy of y (the layer trace), or nullptr
    float* xnext;          // one-launch stack decode: the next layer's x exchange copies (or nullptr)
    size_t xstride; int xcopies;
    int x_repl;            // x is the previous layer's exchange copy (else the caller's x)
    // head top-k (extra block)
    const double* logits_h; int En; int kn; const float* head_bias; const float* hist_cur_m; const float* hist_prev_m;
    const int32_t* hist_cur; const int32_t* hist_prev; int32_t* pred_idx; float* pred_w;
    int32_t* err;
};
hipError_t launch_dec_b(const DecBArgs& a, hipStream_t s, const KTime* tm = nullptr);

// One launch per decode step for a stack of identical layers (kernels_stack.hip)
struct StackLayerArgs {
    DecAArgs a;
    DecBArgs b;
};
constexpr int kStackLine = 32;                 // words per 128-byte line
#ifndef MOE_XCHG_COPIES
#define MOE_XCHG_COPIES 4
#endif
constexpr int kXchgCopies = MOE_XCHG_COPIES;   // copies of the activations handed between phases
constexpr int kStackAPass = 4;                 // the step kernel's gate/up passes per wave (16 h rows a block)
constexpr int kStackBPass = 8;                 // the step kernel's down passes per block
constexpr int kXchgParts = 5;                  // x, h, shared h, LoRA A u, shared gate
// one line: the abort word of the step kernel's waits
inline size_t stack_sync_words(int) { return kStackLine; }
struct StackDecArgs {
    const StackLayerArgs* tab; int n_layers; int nA; int nB;
    uint32_t* sync;               // stack_sync_words(n_layers): the abort word
    uint32_t spin_limit;
};
struct StackPatchArgs {
    StackLayerArgs* tab; uint32_t* sync; int n_layers; int n_tok; int k; int d; int f; int nb_h;
    const float* x_in; float* x_out;
    const int32_t* route_idx; const float* route_w;          // [layer][n_tok * k] (layer 0 unused)
    int32_t* pred_idx; float* pred_w;
    int32_t* used_idx; float* used_w;
    const int32_t* hist_prev;
    float* trace;                 // [layer][n_tok * d] or nullptr (layer 0 copied by the host)
    // the exchange words the step kernel publishes, set to the empty word
    // before it runs: per layer kXchgCopies copies xstride floats apart, part
    // i at xoff[i] with xw[i] floats per token; and each layer's head logits
    float* xchg; size_t xstride; uint32_t xoff[kXchgParts]; uint32_t xw[kXchgParts];
};
constexpr int kStackHeadMaxPer = 4;         // the step kernel's head top-k: E <= 64 * 4
bool stack_one_launch_shape_ok(int d, int f);
int stack_one_hrows(int d);                      // h rows per K_A item of the step kernel
int stack_one_brows(int f);                      // output rows per K_B item of the step kernel
bool stack_one_fast_ok(int d, int f, int fs, int n_tok, int k);
int stack_one_launch_blocks_per_cu(int d, int f);
// layer 0's router and the table patch (one launch), then the step kernel
hipError_t launch_stack_one(const StackPatchArgs& p, const DecAArgs& a0, const RouteArgs& r0,
                            const StackDecArgs& s, int grid, hipStream_t st, const KTime* tprep = nullptr,
                            const KTime* tm = nullptr);
hipError_t launch_topk_job(const TopkJob& j, int n_tok, hipStream_t s);

struct SlotUpdate {
    int n;
    int slot[64];
    int old_e[64];
    int new_e[64];
    int shared_tag;   // >= 0: write into slot_tag[shared_slot]
    int shared_slot;
};
hipError_t launch_slot_update(int32_t* slot_of, int32_t* slot_tag, const SlotUpdate& u, hipStream_t s);

// Device-initiated staging of one slab buffer (kernels_stage.hip).
constexpr int kMaxStageSlots = 1024;            // slab slots a device-staged layer may have
// plan: [0] copies, then (slot, expert) pairs, then the shared flag
__host__ __device__ inline int stage_plan_shared(int slots) { return 1 + 2 * slots; }
__host__ __device__ inline int stage_plan_ints(int slots) { return 2 + 2 * slots; }
struct DevStageArgs {
    const int32_t* ids; int n_ids;               // routing entries on the device (any order, duplicates, < 0 absent)
    int E; int slots;
    int32_t* slot_of; int32_t* slot_tag;         // this buffer's tables: [E], [slots + 1] (entry `slots`: shared)
    const uint8_t* store; const uint8_t* shared; // device addresses of the mapped pinned store / shared blob
    uint8_t* slab; size_t blob; size_t sblob;    // this buffer's slab: slots blobs, then the shared slot
    int32_t* plan;                               // [stage_plan_ints(slots)] scratch
    unsigned long long* bytes;                   // staged-bytes counter
    int32_t* err;
};
hipError_t launch_stage_device(const DevStageArgs& a, int blocks, hipStream_t s);

}  // namespace moe

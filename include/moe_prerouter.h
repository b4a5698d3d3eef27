/*
 * moe_prerouter.h -- C ABI of the MI355X (gfx950) per-layer MoE block library.
 *
 * The block (per layer, per token):
 *   u      = RMSNorm(x) rounded to the activation dtype     (when the norm is fused)
 *   routing: the top-k experts predicted for this layer one token earlier by
 *            the previous layer's prerouter head, used as the routing itself
 *            ("prediction-as-routing": xyznot.com reading guide of "The Other
 *            Half of the Memory Wall", Key ideas and Key terms); rows with no
 *            prediction self-route with this layer's own router (the reactive
 *            on-demand mode of the guide's Results section)
 *   y      = sum_j w_j FFN_{e_j}(u) + sigmoid(g_s . u) FFN_shared(u)
 *            + (alpha/r) B A u                     (guide, Method: unmerged adapter execution)
 *   FFN(u) = Wd (silu(Wg u) * (Wu u)), W = s*q + b, int4 affine groups of 64
 *            (ai.info news article on Edge0, section on the 35B version)
 *   pred   = top-k of this layer's head on u: the routing of the next layer
 *            at the next token (guide, Method: prerouter head architecture;
 *            Q&A: why one token ahead)
 *   x_out  = x + y                                    (when the residual is fused)
 *
 * Conventions
 *   - Every function returns MOE_OK (0) or a negative MOE_E_* code; no C++
 *     exception crosses the ABI. MOE_E_HIP keeps the failing hipError_t,
 *     readable with moe_last_hip_error().
 *   - "device" pointers are HIP device memory of the current device; "host
 *     pinned" pointers come from hipHostMalloc (or torch pin_memory). Streams
 *     are hipStream_t passed as void* (NULL = the default stream).
 *   - The caller owns every buffer it passes and keeps it alive until
 *     moe_layer_destroy. The library keeps pointers; it allocates only its
 *     host handle, HIP events and a small pinned host buffer for read-backs.
 *     One copy is made: with bf16 activations, moe_layer_create writes the
 *     bf16 router, head, LoRA A and shared-gate rows into the workspace in
 *     matrix-core fragment order (the prefill routing GEMM reads them there),
 *     so those four arrays must not change after create; the expert store
 *     and the other weights are read in place.
 *   - A layer handle is not thread-safe. Calls on one handle must not overlap
 *     on different streams; separate handles are independent.
 *   - Routing indices are int32, routing weights fp32, logits fp64 inside.
 *     Top-k order is (logit descending, expert index ascending); weights are
 *     the softmax over the selected logits (equal to the full softmax
 *     renormalised over the top-k).
 *
 * Byte formats
 *   expert blob (d = model dim, f = expert intermediate, 64-groups along K):
 *     gate q [f][d/2] | up q [f][d/2] | down q [d][f/2] (uint8, element k of a
 *     row in byte k/2, low nibble for even k) | gate (s,b) fp16 [f][d/64][2] |
 *     up (s,b) fp16 [f][d/64][2] | down (s,b) fp16 [d][f/64][2];
 *     27*d*f/16 bytes; weight = s*q + b.
 *   bf16 matrices are row-major [rows][d].
 */
#ifndef MOE_PREROUTER_H
#define MOE_PREROUTER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define MOE_OK               0
#define MOE_E_INVALID       -1  /* bad argument: null pointer, size, index   */
#define MOE_E_UNSUPPORTED   -2  /* shape or option this build does not serve */
#define MOE_E_CAPACITY      -3  /* workspace or slab too small               */
#define MOE_E_HIP           -4  /* a HIP runtime call failed                 */
#define MOE_E_NOT_STAGED    -5  /* device flag: a routed expert was not in the slab */
#define MOE_E_BAD_INDEX     -6  /* device flag: routing index outside [0, E)  */
#define MOE_E_TIMEOUT       -7  /* device flag: a bounded device-side wait expired */

/* ---- activation dtype of the block input -------------------------------- */
#define MOE_ACT_F32   0
#define MOE_ACT_BF16  1

/* ---- layer flags -------------------------------------------------------- */
/* x_in is the fp32 residual stream: the call applies RMSNorm (gamma, eps),
 * rounds u to the activation dtype and writes x_in + y to y_out.           */
#define MOE_FUSE_NORM_RESIDUAL  0x1u
/* expert_store / shared_blob are device memory holding every expert: no
 * slab, no copies; moe_stage_experts only validates ids.                   */
#define MOE_RESIDENT_STORE      0x2u
/* streamed mode: staging runs on the device. The pinned store is mapped into
 * the device's address space; the routing on the device drives a plan kernel
 * (the sticky-slot plan of moe_plan_slots on the GPU slot table) and a copy
 * kernel, with no host read-back (moe_stage_experts_device; calls that route
 * themselves stage this way inside the call).                              */
#define MOE_DEVICE_STAGING      0x4u
/* with MOE_DEVICE_STAGING: two slab buffers (the guide's Key terms describe
 * staged decode with fixed slots in two alternating buffers): calls read the
 * buffer chosen by moe_layer_use_buffer while the other one is staged for
 * the next step.                                                          */
#define MOE_DOUBLE_SLAB         0x8u

/* staging modes of a stack (moe_stack_set_staging) */
#define MOE_STAGE_OFF           0
#define MOE_STAGE_PREROUTED     1   /* one token ahead: layer l's experts for step t+1 are copied on the
                                       copy stream as soon as head l-1's prediction at step t is final */
#define MOE_STAGE_ON_DEMAND     2   /* reactive: every layer routes itself and stages before it computes */

typedef struct moe_layer_desc {
    int   d_model;        /* d: multiple of 256, <= 8192                          */
    int   n_experts;      /* E: routed experts, 1..1024                           */
    int   top_k;          /* k: 1..8, <= E                                        */
    int   d_ff;           /* f: routed expert intermediate, multiple of 64        */
    int   d_ff_shared;    /* f_s: shared expert intermediate (0 = none; else == f) */
    int   group_size;     /* must be 64                                           */
    int   lora_rank;      /* r: 0..64 (0 = no LoRA branch)                        */
    float lora_alpha;     /* alpha; the branch is scaled by alpha / r             */
    float rms_eps;        /* epsilon of RMSNorm (fused norm only)                 */
    int   act_dtype;      /* MOE_ACT_F32 or MOE_ACT_BF16                          */
    int   max_tokens;     /* largest n_tok of any decode/prefill call: <= 8192  */
    int   slab_slots;     /* streamed mode: routed-expert slots (>= distinct experts per call) */
    int   next_n_experts; /* experts of the layer the head predicts (0 = no head) */
    int   next_top_k;     /* k of the layer the head predicts                     */
    unsigned flags;       /* MOE_FUSE_NORM_RESIDUAL | MOE_RESIDENT_STORE          */
    /* H1: hidden width of the head's MLP branch (guide, Method: prerouter head
     * architecture: head(x) = fc2(erf-GELU(fc1(x))) + l(x) on x = [u, top-k
     * one-hot of the current token, of the previous token]); 0 = the linear
     * path l(x) alone. 0..1024, a multiple of 8; needs a head.              */
    int   head_hidden;
    /* recovery LoRA on the shared expert's gate, up and down projections
     * (guide, Method: three-stage training, the adapter on the shared-expert
     * projections; unmerged adapter execution): rank r_s (0 = none; 1..64,
     * needs a shared expert) and alpha_s (scale alpha_s / r_s).          */
    int   shared_lora_rank;
    float shared_lora_alpha;
} moe_layer_desc;

typedef struct moe_layer_weights {
    /* E blobs back to back (E * blob bytes). Pinned host memory in streamed
     * mode (it stands in for the SSD tier), device memory with RESIDENT.   */
    const void*     expert_store;
    /* one blob of the shared expert (f = d_ff_shared); same memory kind as
     * expert_store; NULL iff d_ff_shared == 0.                             */
    const void*     shared_blob;
    const uint16_t* shared_gate;  /* device bf16 [d]; NULL: gate fixed at 1  */
    const uint16_t* router;       /* device bf16 [E][d]: self-routing; may be NULL if never used */
    const float*    router_bias;  /* device fp32 [E] or NULL                 */
    const uint16_t* head;         /* device bf16 [E_next][d] or NULL (no prediction) */
    const float*    head_bias;    /* device fp32 [E_next] or NULL            */
    /* history one-hot terms of the head input (guide, Method: the head reads
     * top-k one-hots of the predicted layer's routing at the current and the
     * previous token): row j is added to the logits when expert j is in that
     * one-hot set. device fp32 [E_next][E_next] or NULL.                   */
    const float*    hist_cur;
    const float*    hist_prev;
    const uint16_t* lora_a;       /* device bf16 [r][d]                      */
    const uint16_t* lora_b;       /* device bf16 [d][r]                      */
    const float*    norm_gamma;   /* device fp32 [d]; needed with FUSE_NORM_RESIDUAL */
    /* the head's MLP branch (head_hidden = H1 > 0; all NULL otherwise):
     * fc1 = [head_fc1 | head_fc1_onehot^T] acting on [u, one-hot] plus
     * head_fc1_bias; fc2 = head_fc2. Its output adds to l(x) (whose bias
     * head_bias also serves as fc2's). The one-hot inputs are the history
     * routings of moe_io (hist_cur, hist_prev), each distinct valid expert
     * once.                                                                */
    const uint16_t* head_fc1;         /* device bf16 [H1][d]                 */
    const uint16_t* head_fc1_onehot;  /* device bf16 [2 E_next][H1]: row j is fc1's column
                                         for expert j in the current token's routing, row
                                         E_next + j for expert j in the previous token's */
    const float*    head_fc1_bias;    /* device fp32 [H1] or NULL            */
    const uint16_t* head_fc2;         /* device bf16 [E_next][H1]            */
    /* the shared expert's adapter (shared_lora_rank = r_s > 0; else NULL):
     * gate = Wg u + s Bg Ag u, up = Wu u + s Bu Au u, down = Wd h + s Bd Ad h */
    const uint16_t* shared_lora_a;    /* device bf16 [2 r_s][d]: Ag, then Au   */
    const uint16_t* shared_lora_b;    /* device bf16 [2 f_s][r_s]: Bg, then Bu */
    const uint16_t* shared_lora_ad;   /* device bf16 [r_s][f_s]                */
    const uint16_t* shared_lora_bd;   /* device bf16 [d][r_s]                  */
} moe_layer_weights;

/* Per-call inputs and outputs (all device memory). */
typedef struct moe_io {
    /* [n_tok][d]: fp32 residual stream with FUSE_NORM_RESIDUAL, else the
     * block input u in the activation dtype.                               */
    const void*    x_in;
    /* fp32 [n_tok][d]: x_in + y (fused) or y; may alias x_in when fused.   */
    float*         y_out;
    /* int32 / fp32 [n_tok][k]: routing of this layer for each row, or NULL
     * (every row self-routes). A row whose first index is negative
     * self-routes with the layer's router.                                 */
    const int32_t* route_idx;
    const float*   route_w;
    /* optional outputs [n_tok][k]: the routing this call used.              */
    int32_t*       used_idx;
    float*         used_w;
    /* optional outputs [n_tok][k_next]: the head's prediction for the next
     * layer (at the next token). NULL skips the head.                       */
    int32_t*       pred_idx;
    float*         pred_w;
    /* optional inputs [n_tok][k_next] for the history terms (negative
     * entries are absent): routing of the predicted layer at this token and
     * at the previous token.                                               */
    const int32_t* hist_cur;
    const int32_t* hist_prev;
    /* streamed mode only: nonzero forces the reactive path (route on the
     * device, read the routing back, stage the missing experts, continue);
     * implied when route_idx is NULL. Blocks the host until the read-back.  */
    int            reactive;
    /* decode only: nonzero when some rows of a non-NULL route_idx may start
     * with a negative index (those rows self-route, which adds a router
     * launch); zero promises every row is given. Prefill always checks.     */
    int            self_rows;
} moe_io;

typedef struct moe_layer moe_layer;

/* Bytes of one expert blob: 27*d*f/16 for group 64; 0 if unsupported. */
size_t moe_expert_blob_bytes(int d_model, int d_ff, int group_size);

/* Device workspace bytes a layer needs (slab in streamed mode, slot table,
 * activations, routing and sort scratch for max_tokens, the fragment-ordered
 * routing rows); 0 on invalid desc. */
size_t moe_layer_workspace_bytes(const moe_layer_desc* desc);

/* Create a layer on the current device (one layer of the per-layer MoE block:
 * 256 routed experts plus one shared expert, int4 affine group-64 weights --
 * ai.info news article, section on the 35B version; the unmerged adapter of
 * the guide's Method section, unmerged adapter execution; the prerouter head
 * of the guide's Method section, prerouter head architecture). d_workspace: device memory of at
 * least moe_layer_workspace_bytes(desc), 256-byte aligned, owned by the
 * caller. The struct contents are copied; the pointers inside are kept.
 * Errors: MOE_E_INVALID (null/size), MOE_E_UNSUPPORTED (shape),
 * MOE_E_CAPACITY (workspace too small), MOE_E_HIP.                         */
int moe_layer_create(const moe_layer_desc* desc, const moe_layer_weights* w,
                     void* d_workspace, size_t ws_bytes, moe_layer** out);

/* Stage the experts the next call on this layer will use ("staged decode":
 * fixed slots mapped by a device slot table; "incr_stack": only changed
 * slots are rewritten -- guide, Key terms). h_expert_ids: host int32 ids
 * (duplicates allowed), read before return. Experts already resident keep
 * their slot; missing ones (ascending id) take the slots not holding a
 * wanted expert (ascending slot). The copies (pinned host -> HBM slab) and
 * the slot-table update are queued on copy_stream after the layer's last
 * call finished (event); the next call on the layer waits for them. The
 * shared expert is staged once, on the first call, into its own slot.
 * Resident mode: ids are validated and nothing is copied.
 * Errors: MOE_E_INVALID (id outside [0, E)), MOE_E_CAPACITY (more distinct
 * ids than slab_slots), MOE_E_HIP.                                          */
int moe_stage_experts(moe_layer* layer, const int32_t* h_expert_ids, int n_ids,
                      void* copy_stream);

/* Device-initiated staging (layers created with MOE_DEVICE_STAGING): the
 * n_ids routing entries at d_ids (device int32, duplicates allowed, negative
 * entries absent) name the experts slab buffer `buffer` must hold. A plan
 * kernel applies the sticky-slot plan to that buffer's GPU slot table and a
 * copy kernel copies the changed blobs from the mapped pinned store, both on
 * `stream`, with no host synchronisation ("staged decode" and "incr_stack",
 * guide, Key terms); the next call reading `buffer` waits for them. Single
 * slab: the copies wait for the layer's last call. Double slab: the caller
 * orders `stream` after the last call that read `buffer`. More distinct
 * experts than slots sets the NOT_STAGED flag and stages nothing.
 * Errors: MOE_E_INVALID (null, buffer out of range), MOE_E_UNSUPPORTED
 * (layer without device staging), MOE_E_HIP.                               */
int moe_stage_experts_device(moe_layer* layer, const int32_t* d_ids, int n_ids, int buffer, void* stream);

/* The slab buffer later calls read (0, or 0/1 with MOE_DOUBLE_SLAB).        */
int moe_layer_use_buffer(moe_layer* layer, int buffer);

/* Host copy of the current slot table (expert id per routed slot, -1 empty;
 * n_slots entries) and the number of bytes copied by staging so far. Layers
 * with device staging: the table of the current buffer, read from the device
 * after a device synchronisation.                                           */
int moe_layer_slots(const moe_layer* layer, int32_t* h_slot_expert, int n_slots,
                    uint64_t* staged_bytes);

/* Decode call for n_tok (1..max_tokens) independent tokens: grouped GEMV
 * path. The routing used is the prediction passed in (prediction-as-routing:
 * guide, Key ideas and Key terms); the head's output is the next layer's
 * routing at the next token (guide, Q&A: why one token ahead). Asynchronous on `stream` except the reactive read-back.
 * Errors (returned): MOE_E_INVALID, MOE_E_UNSUPPORTED, MOE_E_HIP. Device
 * errors (NOT_STAGED, BAD_INDEX) set a sticky flag read by
 * moe_layer_sync_status; the affected expert's contribution is dropped.    */
int moe_decode_step(moe_layer* layer, const moe_io* io, int n_tok, void* stream);

/* moe_decode_noalloc: the decode call for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). No layer handle and no workspace: desc and w as for
 * moe_layer_create (MOE_RESIDENT_STORE required: the store is device
 * memory and is read in place), io as for moe_decode_step. The per-call
 * scratch (logits, routing digest, hidden activations, flags) lives in a
 * 256 KiB array of device memory that the library holds per GPU for the
 * life of the process; the call allocates nothing. Every call on one GPU
 * shares that array and the last call's contents stay in it, so calls that
 * overlap on one GPU race (issue them on one stream or order them). Only
 * the fused two-kernel decode path is served: 1..16 tokens, n_tok * k <= 64,
 * d and f powers of two (d in 256..2048, f in 64..512, f_s 0 or f).
 * The head's MLP branch (head_hidden > 0) and the shared expert's adapter
 * (shared_lora_rank > 0) are not served here.
 * d_status (optional, device int32): receives this call's device flag as a
 * status code (MOE_OK, MOE_E_BAD_INDEX, MOE_E_NOT_STAGED). Asynchronous on
 * `stream`. Errors (returned): MOE_E_INVALID, MOE_E_UNSUPPORTED (shape or
 * path not served, streamed store), MOE_E_CAPACITY (the call's scratch
 * exceeds 256 KiB, e.g. 16 tokens over 1024 experts), MOE_E_HIP.            */
int moe_decode_noalloc(const moe_layer_desc* desc, const moe_layer_weights* w, const moe_io* io, int n_tok,
                       int32_t* d_status, void* stream);

/* Prefill call for n_tok tokens of one sequence (or any rows): token-to-
 * expert sort/permute and int4->bf16 MFMA grouped GEMM (the prefill of the
 * ai.info news article's 35B section; the routing and head as in decode). Same io contract;
 * pred row i is the head on token i, i.e. the routing of the next layer for
 * token i+1 (the caller shifts it down by one row).                         */
int moe_prefill(moe_layer* layer, const moe_io* io, int n_tok, void* stream);

/* Wait for the device, return and clear the sticky device error flag
 * (MOE_OK, MOE_E_NOT_STAGED, MOE_E_BAD_INDEX or MOE_E_TIMEOUT).             */
int moe_layer_sync_status(moe_layer* layer);

/* Release the handle, its events and its pinned read-back buffer (not the
 * caller's memory). Safe on NULL.                                           */
void moe_layer_destroy(moe_layer* layer);

/* ---- stack of layers ------------------------------------------------------
 * A stack of n_layers layers (each with MOE_FUSE_NORM_RESIDUAL, the same d
 * and top_k, a router, and a head on every layer but the last) driven with
 * the one-token-ahead dataflow (guide, Q&A: why one token ahead): head l at
 * token t predicts the routing of layer l+1 at token t+1, and that
 * prediction is the routing. Launches only (no host synchronisation, no
 * allocation; in streamed mode the reactive layer-0 staging reads back), so
 * resident-mode calls can be captured into a HIP graph.
 *
 * moe_stack_workspace_bytes: device scratch the stack needs (two prediction
 *   buffers of min(max_tokens) * k entries for stack prefill calls without
 *   caller prediction buffers, the one-launch step's per-layer argument
 *   table and its counters); 0 if the layers do not form a valid stack.
 * moe_stack_create: d_workspace is caller-owned device memory of at least
 *   that size, 256-byte aligned, kept until destroy. The library allocates
 *   only the host handle. Errors: MOE_E_INVALID (null, misaligned, layers
 *   not chainable), MOE_E_CAPACITY (workspace too small).
 * moe_stack_decode: one decode step for n_tok independent sequences.
 *   x_in       device fp32 [n_tok][d]: step input (may equal x_out)
 *   x_out      device fp32 [n_tok][d]: residual stream after the last layer
 *   route_*    device [n_layers][n_tok][k]: this step's routing (entry l = 0
 *              and every entry on the first step are ignored: those layers
 *              self-route with their router). Entries of layers l >= 1 must
 *              be expert indices (the previous step's predictions are): a
 *              negative entry is MOE_E_BAD_INDEX in that layer's status on the
 *              general path (batches beyond the fused one), where the sorts of
 *              layers 1..n-1 run as one launch at the start of the step; it
 *              must not alias pred_* (the step's heads overwrite pred_*).
 *   pred_*     device [n_layers][n_tok][k] out: pred[l] for l >= 1 (pred[0]
 *              is left untouched); the next step's route
 *   used_*     optional out [n_layers][n_tok][k]: routing each layer used
 *   hist_prev  optional in [n_layers][n_tok][k]: routing each layer used at
 *              the previous step (history one-hot of the previous token);
 *              the current-token history of head l is route[l+1].
 * moe_stack_prefill: n_tok tokens of one sequence. Token i >= 1 at layer
 *   l >= 1 uses head l-1's prediction on token i-1 (shifted on the device);
 *   token 0 and layer 0 self-route. x is updated in place; used_* as above;
 *   pred_* (optional) receive each head's unshifted predictions; without
 *   them the predictions pass through the stack's workspace.
 * moe_stack_set_staging: for stacks of streamed layers with device staging:
 *   mode MOE_STAGE_PREROUTED stages, during decode step t, each layer l >= 1's
 *   routing for step t+1 on copy_stream into the buffer step t+1 reads (with
 *   double slabs the other one, so the copies overlap the rest of step t;
 *   with one slab after layer l's call finished), and layer l at step t+1
 *   waits for it; layer 0 and every layer of the first step route themselves
 *   and stage inside the call. MOE_STAGE_ON_DEMAND: every layer routes itself
 *   at every step and stages before it computes (the route_* inputs are
 *   ignored). MOE_STAGE_OFF: the caller stages (moe_stage_experts).
 * moe_stack_set_trace: with d_x_trace non-NULL (device fp32, n_floats), every
 *   later stack call first copies layer l's input residual stream [n_tok][d]
 *   to d_x_trace + l * n_tok * d (a device-to-device copy per layer, for
 *   checking each layer on the input it saw); calls whose trace would not
 *   fit return MOE_E_CAPACITY. NULL / 0 turns the trace off.
 * moe_stack_set_one_launch: enable != 0 runs each later decode step that
 *   qualifies as two launches (layer 0's router together with a patch of
 *   the per-layer argument table that also marks every exchange word the
 *   step will publish as empty, then one step kernel in which every layer's K_A
 *   and K_B run as work items, each issuing its weight rows before it
 *   reads, until they have been published, the activations it needs; the
 *   addresses are known before the step starts because each layer's routing
 *   is the previous token's prediction: guide, Q&A on why one token ahead).
 *   A step qualifies when it is not the first step, staging is
 *   MOE_STAGE_OFF and n_tok takes the fast path; other steps run per layer
 *   as before. The stack qualifies (else MOE_E_UNSUPPORTED) when every layer
 *   is resident, the layers share d, d_ff, the shared width, k, E, the LoRA
 *   rank (0, 8 or 16) and the presence of the shared gate, heads have at
 *   most 256 outputs, and no layer has the head's MLP branch or the shared
 *   expert's adapter. The activations must be finite (a value whose bits
 *   are all ones reads as not yet published). The waits are bounded: a
 *   value that never arrives sets MOE_E_TIMEOUT in the layer's status
 *   (moe_layer_sync_status) instead of hanging. Calls on one stack must not
 *   overlap (the table and exchange buffers are per stack). Default: off.
 * moe_stack_set_wait_limit: the bound of each of those waits, in polls of
 *   about a microsecond each (0: the default, 2^18). A wait that runs out
 *   sets MOE_E_TIMEOUT and lets every later wait of the launch give up at
 *   once, so the launch ends (with wrong outputs) instead of hanging.
 * moe_stack_set_profiling / moe_stack_kernel_ms: kernel-timestamp events on
 *   the one-launch step's router launch and step kernel (as
 *   moe_layer_set_profiling); -1 where not launched.                      */
typedef struct moe_stack moe_stack;
size_t moe_stack_workspace_bytes(moe_layer* const* layers, int n_layers);
int moe_stack_create(moe_layer* const* layers, int n_layers, void* d_workspace, size_t ws_bytes, moe_stack** out);
int moe_stack_decode(moe_stack* st, const float* x_in, float* x_out, int n_tok,
                     const int32_t* route_idx, const float* route_w, int32_t* pred_idx, float* pred_w,
                     int32_t* used_idx, float* used_w, const int32_t* hist_prev, int first_step, void* stream);
int moe_stack_prefill(moe_stack* st, float* x, int n_tok, int32_t* used_idx, float* used_w,
                      int32_t* pred_idx, float* pred_w, void* stream);
int moe_stack_set_trace(moe_stack* st, float* d_x_trace, size_t n_floats);
int moe_stack_set_staging(moe_stack* st, void* copy_stream, int mode);
int moe_stack_set_one_launch(moe_stack* st, int enable);
int moe_stack_set_wait_limit(moe_stack* st, unsigned polls);
int moe_stack_set_profiling(moe_stack* st, int enable);
int moe_stack_kernel_ms(moe_stack* st, float* ms_router, float* ms_step);
void moe_stack_destroy(moe_stack* st);

/* ---- measurement --------------------------------------------------------
 * With profiling on, each decode kernel of this layer is launched with HIP
 * kernel-timestamp events (the dispatch's own begin and end, as a kernel
 * trace reports them, not the gaps between launches); moe_layer_kernel_ms
 * returns the durations of the most recent launches of the router
 * (self-routing), K_A (norm + gate/up + head) and K_B (down + combine +
 * epilogue) kernels, -1 where not launched. Not for use under graph capture. */
int moe_layer_set_profiling(moe_layer* layer, int enable);
int moe_layer_kernel_ms(moe_layer* layer, float* ms_router, float* ms_a, float* ms_b);

const char* moe_status_str(int status);
int moe_last_hip_error(void);

/* ---- pure host helper (no device use) ------------------------------------
 * The sticky-slot plan moe_stage_experts applies. resident[n_slots]: expert
 * per slot (-1 empty), updated in place; an expert may sit in one slot only
 * (in two: MOE_E_INVALID). wanted[n_wanted] (duplicates ok).
 * copies_slot/copies_expert receive up to n_slots entries; *n_copies is set.
 * Returns MOE_OK, MOE_E_INVALID or MOE_E_CAPACITY (resident unchanged).     */
int moe_plan_slots(int32_t* resident, int n_slots, const int32_t* wanted, int n_wanted,
                   int n_experts, int32_t* copies_slot, int32_t* copies_expert, int* n_copies);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PREROUTER_H */

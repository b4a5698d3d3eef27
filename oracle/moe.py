"""fp64 NumPy oracle of the per-layer MoE block and of its stack dataflow.

TEST INFRASTRUCTURE (see oracle/__init__.py): imported only by tests, the
smoke check and the bench's CPU-baseline leg.

Every function takes plain NumPy arrays; bf16/fp16 tensors arrive as raw
uint16 bit patterns and are decoded here. All arithmetic is float64.

Pins (tests/test_oracle_pins.py, marked "not gpu"):
  dequant_matrix   hand-built groups with closed-form values, nibble order,
                   s = 0 groups, quantiser round-trip bound
  rmsnorm          constant rows (closed form), scale invariance
  round_bf16       exhaustive neighbours of bf16 values, ties to even
  topk / weights   brute force over all k-subsets, exact ties, k = E,
                   shift invariance, sum to one
  head_mlp         erf-GELU at textbook normal-CDF values (and against the
                   tanh form), one-hot wiring of fc1 (current block vs
                   previous block), fc2 orientation, W2 = 0 gives the linear
                   head, l + MLP composed in predict_next
  expert_ffn       permutation-structured experts with closed-form outputs
  moe_block        identical experts, k = 1, sigmoid(0) gate and
                   sigmoid(ln 3) = 3/4 on the normalised input, LoRA rank 1
                   and rank 4 (alpha / r) closed forms, residual x + y,
                   expert relabelling invariance
  shared_ffn       the shared expert's adapter on gate, up and down in
                   closed form (each projection's A and B picking known
                   entries), B = 0 reduces to the plain shared expert
  stack dataflow   prefill == sequential per-token decode with the same
                   shifted routing; batch rows == separate batch-1 runs;
                   history one-hots of head l = layer l+1's routing at this
                   step and the previous one (hand-derived 3-layer run)
  plan_slots       brute-force minimal-copy / sticky-slot properties
Parity unpinned: the prediction *quality* of heads (no trained heads exist)
and the pages' absolute throughputs; neither is computed here. The MLP
branch's fc1 width is not on the pages: it is a parameter.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

GROUP = 64


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_to_f64(bits) -> np.ndarray:
    """fp16 bit patterns (uint16) -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits. With x = m * 2**e, 0.5 <= |m| < 1, the
    nearest representable value is rint(m * 2**8) * 2**(e - 8) (rint rounds
    half to even). Values below the bf16 normal range are not expected in
    this workload and are rounded the same way (no subnormal handling).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def bf16_bits_of(x) -> np.ndarray:
    """Bit patterns of values that are exactly representable in bf16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# O1: int4 affine group-64 dequantisation
# [News] "La versione da 35B usa 256 esperti ...": int4 affine quantisation
# with groups of 64. Byte format: element k of a row in byte k/2, low nibble
# for even k; (scale, bias) fp16 per 64 consecutive elements of a row.
# ----------------------------------------------------------------------------
def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """uint8 [N, K/2] -> integer codes float64 [N, K]."""
    packed = np.asarray(packed, dtype=np.uint8)
    N, half = packed.shape
    q = np.empty((N, 2 * half), dtype=np.float64)
    q[:, 0::2] = packed & 0x0F
    q[:, 1::2] = packed >> 4
    return q


def dequant_matrix(packed: np.ndarray, sb_bits: np.ndarray) -> np.ndarray:
    """W[n, k] = s[n, k // 64] * q[n, k] + b[n, k // 64]   (float64 [N, K])."""
    q = unpack_nibbles(packed)
    N, K = q.shape
    sb = np.asarray(sb_bits, dtype=np.uint16).reshape(N, K // GROUP, 2)
    s = f16_to_f64(sb[..., 0])
    b = f16_to_f64(sb[..., 1])
    W = np.empty((N, K), dtype=np.float64)
    for g in range(K // GROUP):
        cols = slice(g * GROUP, (g + 1) * GROUP)
        W[:, cols] = s[:, g:g + 1] * q[:, cols] + b[:, g:g + 1]
    return W


def blob_bytes(d: int, f: int) -> int:
    """Bytes of one expert: 3 matrices of d*f int4 codes (d*f/2 bytes each)
    plus, per 64 codes, an fp16 scale and an fp16 bias (4 bytes)."""
    return 3 * (d * f // 2) + 3 * (d * f // GROUP) * 4


def unpack_blob(blob: np.ndarray, d: int, f: int):
    """One expert blob (uint8) -> (Wg [f, d], Wu [f, d], Wd [d, f]) float64."""
    blob = np.asarray(blob, dtype=np.uint8).reshape(-1)
    assert blob.size == blob_bytes(d, f), (blob.size, d, f)
    qsz = d * f // 2
    ssz = (d * f // GROUP) * 4
    o = 0
    gq = blob[o:o + qsz].reshape(f, d // 2); o += qsz
    uq = blob[o:o + qsz].reshape(f, d // 2); o += qsz
    dq = blob[o:o + qsz].reshape(d, f // 2); o += qsz
    gs = blob[o:o + ssz].view(np.uint16).reshape(f, d // GROUP, 2); o += ssz
    us = blob[o:o + ssz].view(np.uint16).reshape(f, d // GROUP, 2); o += ssz
    ds = blob[o:o + ssz].view(np.uint16).reshape(d, f // GROUP, 2); o += ssz
    return dequant_matrix(gq, gs), dequant_matrix(uq, us), dequant_matrix(dq, ds)


# ----------------------------------------------------------------------------
# O2: RMSNorm prologue (the head reads the post-norm hidden state:
# [Guide] Method, prerouter head architecture)
# ----------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


# ----------------------------------------------------------------------------
# O3-O5: head logits, top-k, renormalised softmax weights
# [Guide] Method, prerouter head architecture: the head reads the hidden state
# plus top-k one-hot routing vectors of the current and previous token;
# head(x) = fc2(gelu(fc1(x))) + l(x), and head_logits is the linear path l(x)
# (the MLP branch is head_mlp below). [Guide] Key terms, prediction-as-routing:
# the predicted set is the routing itself.
# ----------------------------------------------------------------------------
def head_logits(H_bits: np.ndarray, u: np.ndarray, bias: Optional[np.ndarray] = None,
                hist_cur_mat: Optional[np.ndarray] = None, hist_cur: Optional[Sequence[int]] = None,
                hist_prev_mat: Optional[np.ndarray] = None, hist_prev: Optional[Sequence[int]] = None):
    """z = H u + bias + sum_{j in cur} Mc[j, :] + sum_{j in prev} Mp[j, :].

    H: bf16 bits [E, d]; u: [d] float64; Mc/Mp: float [E, E] whose row j is
    the contribution of expert j being present in that one-hot vector
    (equivalently z += Mc^T onehot(cur)); indices < 0 are absent.
    """
    H = bf16_to_f64(H_bits)
    z = H @ np.asarray(u, dtype=np.float64)
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)
    E = z.shape[0]
    for mat, ids in ((hist_cur_mat, hist_cur), (hist_prev_mat, hist_prev)):
        if mat is None or ids is None:
            continue
        onehot = np.zeros(E, dtype=np.float64)
        for j in ids:
            if j >= 0:
                onehot[int(j)] = 1.0
        z = z + np.asarray(mat, dtype=np.float64).T @ onehot
    return z


def topk(z: np.ndarray, k: int) -> np.ndarray:
    """First k experts in the order (logit descending, index ascending)."""
    z = np.asarray(z, dtype=np.float64)
    order = sorted(range(z.shape[0]), key=lambda e: (-z[e], e))
    return np.array(order[:k], dtype=np.int64)


def route_weights(z: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over all E logits (max subtracted), then renormalised over idx."""
    z = np.asarray(z, dtype=np.float64)
    p = np.exp(z - z.max())
    p = p / p.sum()
    sel = p[np.asarray(idx)]
    return sel / sel.sum()


def route(z: np.ndarray, k: int):
    idx = topk(z, k)
    return idx, route_weights(z, idx)


# ----------------------------------------------------------------------------
# O3b: the head's MLP branch. [Guide] Method, prerouter head architecture: the
# head computes fc2(erf-GELU(fc1(x))) + l(x) on x = [hidden state, top-k
# one-hot of the current token's routing, top-k one-hot of the previous
# token's], of width d + 2E. l(x) is head_logits above (H u + bias + the
# one-hot rows). fc1 is stored as its hidden-state columns W1u [H1, d] and
# its one-hot columns W1oh [2E, H1] (row j < E: column d + j, the current
# token's expert j; row E + j: column d + E + j, the previous token's).
# ----------------------------------------------------------------------------
def gelu_erf(a):
    """GELU with the exact normal CDF: a * Phi(a) = a / 2 * (1 + erf(a / sqrt 2))."""
    a = np.asarray(a, dtype=np.float64)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * a * (1.0 + erf(a / math.sqrt(2.0)))


def onehot_input(E: int, cur: Optional[Sequence[int]], prev: Optional[Sequence[int]]) -> np.ndarray:
    """The 2E one-hot part of the head input: 1 at j for expert j in cur, at
    E + j for expert j in prev (indices < 0 are absent)."""
    v = np.zeros(2 * E, dtype=np.float64)
    for j in (cur if cur is not None else []):
        if j >= 0:
            v[int(j)] = 1.0
    for j in (prev if prev is not None else []):
        if j >= 0:
            v[E + int(j)] = 1.0
    return v


def head_mlp(W1u_bits, W1oh_bits, b1, W2_bits, u, E: int, cur=None, prev=None) -> np.ndarray:
    """fc2(gelu(fc1(x))): fc1(x) = [W1u | W1oh^T] x + b1 with x = [u, onehot];
    fc2 is W2 [E, H1] (its bias is the head bias, added with l(x))."""
    W1u = bf16_to_f64(W1u_bits)
    W1oh = bf16_to_f64(W1oh_bits)
    x_oh = onehot_input(E, cur, prev)
    a1 = W1u @ np.asarray(u, dtype=np.float64) + W1oh.T @ x_oh
    if b1 is not None:
        a1 = a1 + np.asarray(b1, dtype=np.float64)
    return bf16_to_f64(W2_bits) @ gelu_erf(a1)


# ----------------------------------------------------------------------------
# O6-O9: expert FFN, combine, sigmoid-gated shared expert, unmerged LoRA
# [Guide] Method, unmerged adapter execution: y = W_int4(x) + (alpha/r) B A x.
# [News] 35B model section: 256 experts per layer plus one shared expert,
# four experts per token.
# ----------------------------------------------------------------------------
def silu(a):
    a = np.asarray(a, dtype=np.float64)
    return a / (1.0 + np.exp(-a))


def sigmoid(a):
    return 1.0 / (1.0 + math.exp(-float(a)))


def expert_ffn(W, u: np.ndarray) -> np.ndarray:
    """o = Wd (silu(Wg u) * (Wu u)) for W = (Wg, Wu, Wd) float64."""
    Wg, Wu, Wd = W
    u = np.asarray(u, dtype=np.float64)
    h = silu(Wg @ u) * (Wu @ u)
    return Wd @ h


@dataclass
class LayerWeights:
    """One layer's tensors in oracle form (float64 or raw bits)."""
    d: int
    E: int
    k: int
    f: int
    fs: int
    r: int
    alpha: float
    eps: float
    act: str                         # "f32" or "bf16": precision of u
    store: np.ndarray                # uint8 [E, blob]
    shared: Optional[np.ndarray]     # uint8 [blob_s] or None
    shared_gate: Optional[np.ndarray]  # bf16 bits [d] or None (gate = 1)
    lora_a: Optional[np.ndarray]     # bf16 bits [r, d]
    lora_b: Optional[np.ndarray]     # bf16 bits [d, r]
    gamma: Optional[np.ndarray]      # float [d]
    head: Optional[np.ndarray]       # bf16 bits [E, d]  (predicts the next layer)
    router: Optional[np.ndarray]     # bf16 bits [E, d]  (self-routing)
    head_bias: Optional[np.ndarray] = None
    router_bias: Optional[np.ndarray] = None
    hist_cur: Optional[np.ndarray] = None    # float [E, E]
    hist_prev: Optional[np.ndarray] = None   # float [E, E]
    head_fc1: Optional[np.ndarray] = None      # bf16 bits [H1, d]: fc1's hidden-state columns
    head_fc1_oh: Optional[np.ndarray] = None   # bf16 bits [2E, H1]: fc1's one-hot columns
    head_fc1_bias: Optional[np.ndarray] = None  # float [H1]
    head_fc2: Optional[np.ndarray] = None      # bf16 bits [E, H1]
    # recovery LoRA on the shared expert's projections (rank rs, alpha as):
    shared_lora_rank: int = 0
    shared_lora_alpha: float = 0.0
    shared_lora_a: Optional[np.ndarray] = None    # bf16 bits [2 rs, d]: A of gate, then A of up
    shared_lora_b: Optional[np.ndarray] = None    # bf16 bits [2 fs, rs]: B of gate, then B of up
    shared_lora_ad: Optional[np.ndarray] = None   # bf16 bits [rs, fs]: A of down
    shared_lora_bd: Optional[np.ndarray] = None   # bf16 bits [d, rs]: B of down
    max_cache: int = 8                       # dequantised experts kept (memory bound)
    _cache: dict = field(default_factory=dict, repr=False)

    def expert(self, e: int):
        if e not in self._cache:
            if len(self._cache) >= self.max_cache:
                drop = next(k for k in self._cache if k != "shared")
                del self._cache[drop]
            self._cache[e] = unpack_blob(self.store[e], self.d, self.f)
        return self._cache[e]

    def shared_expert(self):
        if "shared" not in self._cache:
            self._cache["shared"] = unpack_blob(self.shared, self.d, self.fs)
        return self._cache["shared"]


def shared_ffn(lw: LayerWeights, u: np.ndarray) -> np.ndarray:
    """The shared expert, with the recovery LoRA on its gate, up and down
    projections when the layer has one ([Guide] Method, three-stage training:
    the adapter sits on the attention, linear-attention and shared-expert
    projections, not on the streamed experts; unmerged adapter execution:
    each projection is W_int4 x + (alpha / r) B A x):
        a = Wg u + s Bg Ag u,  c = Wu u + s Bu Au u,  h = silu(a) * c,
        o = Wd h + s Bd Ad h,  s = alpha / r."""
    Wg, Wu, Wd = lw.shared_expert()
    u = np.asarray(u, dtype=np.float64)
    a = Wg @ u
    c = Wu @ u
    rs = lw.shared_lora_rank
    if rs:
        sc = lw.shared_lora_alpha / rs
        A = bf16_to_f64(lw.shared_lora_a)
        B = bf16_to_f64(lw.shared_lora_b)
        fs = Wg.shape[0]
        a = a + sc * (B[:fs] @ (A[:rs] @ u))
        c = c + sc * (B[fs:] @ (A[rs:] @ u))
    h = silu(a) * c
    o = Wd @ h
    if rs:
        o = o + sc * (bf16_to_f64(lw.shared_lora_bd) @ (bf16_to_f64(lw.shared_lora_ad) @ h))
    return o


def lora_delta(lw: LayerWeights, u: np.ndarray) -> np.ndarray:
    if not lw.r or lw.lora_a is None:
        return np.zeros(lw.d)
    A = bf16_to_f64(lw.lora_a)
    B = bf16_to_f64(lw.lora_b)
    return (lw.alpha / lw.r) * (B @ (A @ np.asarray(u, dtype=np.float64)))


def shared_gate_value(lw: LayerWeights, u: np.ndarray) -> float:
    if lw.shared_gate is None:
        return 1.0
    return sigmoid(bf16_to_f64(lw.shared_gate) @ np.asarray(u, dtype=np.float64))


def moe_block(lw: LayerWeights, u: np.ndarray, idx: Sequence[int], w: Sequence[float]) -> np.ndarray:
    """Block output y (pre-residual) for one token:
    y = sum_j w_j FFN_{idx_j}(u) + sigmoid(g_s . u) FFN_shared(u) + (alpha/r) B A u."""
    u = np.asarray(u, dtype=np.float64)
    y = np.zeros(lw.d, dtype=np.float64)
    for e, wj in zip(idx, w):
        y += float(wj) * expert_ffn(lw.expert(int(e)), u)
    if lw.fs and lw.shared is not None:
        y += shared_gate_value(lw, u) * shared_ffn(lw, u)
    y += lora_delta(lw, u)
    return y


def block_input(lw: LayerWeights, x: np.ndarray, fused_norm: bool) -> np.ndarray:
    """u as the block sees it: RMSNorm(x) when the norm is fused, else x; then
    rounded (to nearest even) to the block's activation dtype, bf16 or fp32."""
    u = rmsnorm(x, lw.gamma, lw.eps) if fused_norm else np.asarray(x, dtype=np.float64)
    if lw.act == "bf16":
        u = round_bf16(u)
    else:
        u = u.astype(np.float32).astype(np.float64)   # fp32 activations
    return u


def self_route(lw: LayerWeights, u: np.ndarray):
    z = head_logits(lw.router, u, lw.router_bias)
    return route(z, lw.k)


def predict_next(lw: LayerWeights, u: np.ndarray, k_next: int, cur=None, prev=None):
    """head(x) = l(x) + fc2(gelu(fc1(x))) (the MLP branch when the layer has one),
    then top-k and the renormalised weights."""
    z = head_logits(lw.head, u, lw.head_bias, lw.hist_cur, cur, lw.hist_prev, prev)
    if lw.head_fc1 is not None:
        E = z.shape[0]
        z = z + head_mlp(lw.head_fc1, lw.head_fc1_oh, lw.head_fc1_bias, lw.head_fc2, u, E, cur, prev)
    idx, w = route(z, k_next)
    return idx, w, z


# ----------------------------------------------------------------------------
# O10-O11: one layer call and the stack dataflow
# [Guide] Q&A "why one token ahead": head N at token t predicts layer N+1 at
# token t+1, so every staged layer of the next step is known after this step.
# [Guide] Results: one-token-ahead prefetch vs reactive on-demand streaming;
# the reactive mode routes a layer only once its own input exists (used here
# for layer 0 and for the first step, where no prediction exists).
# ----------------------------------------------------------------------------
@dataclass
class StepRecord:
    routes: list        # per layer: (idx [B, k], w [B, k]) used at this step
    preds: list         # per layer l: (idx, w) predicted for layer l+1 at t+1 (None for last)
    logits: list        # per layer l: head logits [B, E] (None for last)
    u: list             # per layer: block input u [B, d]
    y: list             # per layer: block output [B, d]
    x_out: np.ndarray   # residual stream after the last layer [B, d]
    self_routed: list   # per layer: bool


def decode_layer(lw: LayerWeights, x: np.ndarray, route_in, next_k: Optional[int],
                 cur=None, prev=None, fused_norm=True):
    """One layer for B tokens. route_in: None (self-route every row) or
    (idx [B,k], w [B,k]) where a row with idx[b,0] < 0 self-routes.
    Returns (x_out, y, u, (idx, w), pred or None, logits or None)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    B = x.shape[0]
    idx = np.zeros((B, lw.k), dtype=np.int64)
    w = np.zeros((B, lw.k), dtype=np.float64)
    us, ys = [], []
    pidx = np.zeros((B, next_k), dtype=np.int64) if next_k else None
    pw = np.zeros((B, next_k), dtype=np.float64) if next_k else None
    zs = [] if next_k else None
    for b in range(B):
        u = block_input(lw, x[b], fused_norm)
        if route_in is None or route_in[0][b][0] < 0:
            ib, wb = self_route(lw, u)
        else:
            ib, wb = np.asarray(route_in[0][b]), np.asarray(route_in[1][b], dtype=np.float64)
        idx[b], w[b] = ib, wb
        ys.append(moe_block(lw, u, ib, wb))
        us.append(u)
        if next_k:
            c = None if cur is None else cur[b]
            p = None if prev is None else prev[b]
            pi, pwb, z = predict_next(lw, u, next_k, c, p)
            pidx[b], pw[b] = pi, pwb
            zs.append(z)
    y = np.stack(ys)
    x_out = x + y if fused_norm else None
    pred = (pidx, pw) if next_k else None
    return x_out, y, np.stack(us), (idx, w), pred, (np.stack(zs) if next_k else None)


def stack_decode_step(layers: List[LayerWeights], x: np.ndarray, pred_in: list,
                      used_prev: list, forced: Optional[list] = None) -> StepRecord:
    """One decode step through the stack for B independent sequences.

    pred_in[l]: routing for layer l predicted at the previous step by head
    l-1, or None (self-route). used_prev[l]: routing layer l used at the
    previous step (history "previous token"), or None.
    forced[l] (optional): routing to use at layer l in place of pred_in.
    """
    L = len(layers)
    # routing each layer will use at this step, where known before the step
    route_for = [forced[l] if forced is not None and forced[l] is not None else pred_in[l]
                 for l in range(L)]
    routes, preds, logits, us, ys, selfr = [], [], [], [], [], []
    for l, lw in enumerate(layers):
        ri = route_for[l]
        selfr.append(ri is None)
        nk = layers[l + 1].k if l + 1 < L else None
        # history one-hots of the predicted layer l+1: its routing at this
        # token (known when it was predicted) and at the previous token
        cur = route_for[l + 1][0] if (nk and route_for[l + 1] is not None) else None
        prev = used_prev[l + 1][0] if (nk and used_prev[l + 1] is not None) else None
        x, y, u, used, pred, z = decode_layer(lw, x, ri, nk, cur, prev, fused_norm=True)
        routes.append(used)
        preds.append(pred)
        logits.append(z)
        us.append(u)
        ys.append(y)
    return StepRecord(routes, preds, logits, us, ys, x, selfr)


def stack_decode(layers: List[LayerWeights], xs: np.ndarray, steps: int):
    """Free-running decode for `steps` steps; xs [steps, B, d] are the
    per-step inputs. Returns the list of StepRecords."""
    L = len(layers)
    pred_in = [None] * L
    used_prev = [None] * L
    recs = []
    for t in range(steps):
        rec = stack_decode_step(layers, xs[t], pred_in, used_prev)
        recs.append(rec)
        pred_in = [None] + [rec.preds[l - 1] for l in range(1, L)]
        used_prev = rec.routes
    return recs


def shift_prefill_routing(pred):
    """Head l on token i predicts layer l+1 for token i+1: shift rows down by
    one; row 0 has no prediction and self-routes (idx -1)."""
    idx, w = pred
    T, k = idx.shape
    si = np.full((T, k), -1, dtype=np.int64)
    sw = np.zeros((T, k), dtype=np.float64)
    si[1:] = idx[:-1]
    sw[1:] = w[:-1]
    return si, sw


def stack_prefill(layers: List[LayerWeights], x: np.ndarray, forced: Optional[list] = None):
    """Prefill T tokens through the stack. Token i at layer l >= 1 is routed
    by head l-1 on token i-1; token 0 and layer 0 self-route.
    Returns (x_out, per-layer (routes used, preds, y))."""
    L = len(layers)
    route_in = None
    recs = []
    for l, lw in enumerate(layers):
        ri = forced[l] if forced is not None and forced[l] is not None else route_in
        nk = layers[l + 1].k if l + 1 < L else None
        x, y, u, used, pred, z = decode_layer(lw, x, ri, nk, fused_norm=True)
        recs.append(dict(route=used, pred=pred, y=y, u=u, logits=z))
        route_in = shift_prefill_routing(pred) if pred is not None else None
    return x, recs


# ----------------------------------------------------------------------------
# O12: staging into a fixed-slot slab
# [Guide] Key terms: staged decode (fixed slots, expert ids mapped to slots by
# a slot table) and incr_stack (persistent stacked expert tensors updated in
# place, only the slots that changed). [Guide] Abstract: the staged set equals
# the routed set.
# ----------------------------------------------------------------------------
def plan_slots(resident: Sequence[int], wanted: Sequence[int]):
    """Sticky-slot plan. resident[s] = expert in slot s (-1 empty).
    Experts already resident keep their slot; missing experts (ascending id)
    take the slots not holding a wanted expert (ascending slot index).
    Returns (new_resident, copies [(slot, expert)]); raises ValueError when
    the distinct wanted experts exceed the slots or an expert sits in two
    slots."""
    want = sorted(set(int(e) for e in wanted))
    res = list(int(e) for e in resident)
    held = [e for e in res if e >= 0]
    if len(held) != len(set(held)):
        raise ValueError("an expert in two slots")   # a slot table holds each expert once
    if len(want) > len(res):
        raise ValueError("capacity")
    have = set(res)
    missing = [e for e in want if e not in have]
    free = [s for s, e in enumerate(res) if e not in want]
    copies = []
    for e, s in zip(missing, free):
        res[s] = e
        copies.append((s, e))
    return res, copies

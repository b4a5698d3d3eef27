"""Test-side glue: builds the same seeded layer for the oracle (NumPy) and for
the HIP library (device tensors), and the comparison metrics."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


def layer_tensors(shape: synth.Shape, layer: int = 0, tag: str = "t", device="cpu") -> dict:
    return synth.layer_weights(shape, layer, device=device, tag=tag)


def oracle_layer(shape: synth.Shape, w: dict, act=None) -> oracle.LayerWeights:
    b = synth.bf16_bits
    return oracle.LayerWeights(
        d=shape.d, E=shape.E, k=shape.k, f=shape.f, fs=shape.fs, r=shape.r, alpha=shape.alpha, eps=shape.eps,
        act=act or shape.act,
        store=synth.to_numpy_bytes(w["store"]),
        shared=synth.to_numpy_bytes(w["shared"]) if w["shared"] is not None else None,
        shared_gate=b(w["shared_gate"]) if w["shared_gate"] is not None else None,
        lora_a=b(w["lora_a"]) if w["lora_a"] is not None else None,
        lora_b=b(w["lora_b"]) if w["lora_b"] is not None else None,
        gamma=w["gamma"].double().numpy(),
        head=b(w["head"]) if w["head"] is not None else None,
        router=b(w["router"]) if w["router"] is not None else None,
        head_bias=w["head_bias"].double().numpy() if w.get("head_bias") is not None else None,
        hist_cur=w["hist_cur"].double().numpy() if w.get("hist_cur") is not None else None,
        hist_prev=w["hist_prev"].double().numpy() if w.get("hist_prev") is not None else None,
        head_fc1=b(w["head_fc1"]) if w.get("head_fc1") is not None else None,
        head_fc1_oh=b(w["head_fc1_onehot"]) if w.get("head_fc1_onehot") is not None else None,
        head_fc1_bias=w["head_fc1_bias"].double().cpu().numpy() if w.get("head_fc1_bias") is not None else None,
        head_fc2=b(w["head_fc2"]) if w.get("head_fc2") is not None else None,
        shared_lora_rank=int(w["shared_lora_a"].shape[0]) // 2 if w.get("shared_lora_a") is not None else 0,
        shared_lora_alpha=float(w.get("shared_lora_alpha", 0.0)),
        shared_lora_a=b(w["shared_lora_a"]) if w.get("shared_lora_a") is not None else None,
        shared_lora_b=b(w["shared_lora_b"]) if w.get("shared_lora_b") is not None else None,
        shared_lora_ad=b(w["shared_lora_ad"]) if w.get("shared_lora_ad") is not None else None,
        shared_lora_bd=b(w["shared_lora_bd"]) if w.get("shared_lora_bd") is not None else None,
    )


def gpu_layer(shape: synth.Shape, w: dict, *, fused: bool, resident: bool = True, slab_slots: int = 0,
              max_tokens: int = 8, head: bool = True, act=None, keep_host: bool = False, device_staging=False,
              double_slab=False, pinned=None):
    import sparse_moe_decode_prerouter_amd as moe
    dev = "cuda"

    def dv(t):
        return None if t is None else t.to(dev).contiguous()

    if resident:
        store, shared = dv(w["store"]), dv(w["shared"])
    elif pinned is not None:
        store, shared = pinned
    else:
        store = w["store"].contiguous().pin_memory()
        shared = w["shared"].contiguous().pin_memory() if w["shared"] is not None else None
    act = act or shape.act
    return moe.MoeLayer(
        d_model=shape.d, n_experts=shape.E, top_k=shape.k, d_ff=shape.f, d_ff_shared=shape.fs,
        lora_rank=shape.r, lora_alpha=shape.alpha,
        act_dtype=moe.MOE_ACT_BF16 if act == "bf16" else moe.MOE_ACT_F32, max_tokens=max_tokens,
        expert_store=store, shared_blob=shared, shared_gate=dv(w["shared_gate"]), router=dv(w["router"]),
        head=dv(w["head"]) if head else None, head_bias=dv(w.get("head_bias")) if head else None,
        next_n_experts=shape.E if head else 0, next_top_k=shape.k if head else 0,
        hist_cur=dv(w.get("hist_cur")) if head else None, hist_prev=dv(w.get("hist_prev")) if head else None,
        lora_a=dv(w["lora_a"]), lora_b=dv(w["lora_b"]), norm_gamma=dv(w["gamma"]), rms_eps=shape.eps,
        fuse_norm_residual=fused, resident=resident, slab_slots=slab_slots,
        head_fc1=dv(w.get("head_fc1")) if head else None, head_fc1_onehot=dv(w.get("head_fc1_onehot")) if head else None,
        head_fc1_bias=dv(w.get("head_fc1_bias")) if head else None, head_fc2=dv(w.get("head_fc2")) if head else None,
        shared_lora_a=dv(w.get("shared_lora_a")), shared_lora_b=dv(w.get("shared_lora_b")),
        shared_lora_ad=dv(w.get("shared_lora_ad")), shared_lora_bd=dv(w.get("shared_lora_bd")),
        shared_lora_alpha=w.get("shared_lora_alpha", 0.0), device_staging=device_staging, double_slab=double_slab)


def rel_l2_rows(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.atleast_2d(np.asarray(got, dtype=np.float64))
    ref = np.atleast_2d(np.asarray(ref, dtype=np.float64))
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    return float(np.max(num / den))


# ----------------------------------------------------------------------------
# Routing comparison (bit-exact indices; the only exception is a certified near
# tie, whose window comes from an error bound on each side's logits)
# ----------------------------------------------------------------------------
U53 = 2.0 ** -53


def gamma_n(n: int, u: float) -> float:
    """Higham's gamma_n = n u / (1 - n u): bound on the relative error of an
    n-term sum (any order) with unit roundoff u, relative to sum |terms|."""
    return n * u / (1.0 - n * u)


# How each routing site evaluates its logits, as the bound's factor on
# sum_j |H_ej u_j| (the oracle's own fp64 evaluation is added separately):
#   "f64"        decode kernels: bf16 x (bf16 or fp32) products, exact in fp64,
#                accumulated in fp64
#   "mfma"       routing GEMM of prefill / batched decode: bf16 products in
#                32-term fp32 matrix-core partials (u = 2^-23 covers a
#                hardware sum that does not round to nearest), the partials
#                summed in fp64
#   "mfma_split" the same with fp32 activations entering as bf16 hi + lo:
#                64-term partials and |u - hi - lo| <= 2^-16 |u|
#   "exact"      inputs built so that every product and partial sum is exact
#                on both sides (the exact-tie tests): no window at all
def gpu_error_factor(mode: str, d: int) -> float:
    if mode == "exact":
        return 0.0
    if mode == "f64":
        return gamma_n(d, U53)
    if mode == "mfma":
        return gamma_n(32, 2.0 ** -23) + gamma_n(d // 32 + 8, U53)
    if mode == "mfma_split":
        return 2.0 ** -16 + gamma_n(64, 2.0 ** -23) + gamma_n(d // 32 + 8, U53)
    raise ValueError(mode)


def routing_mode(shape, n_tok: int, prefill: bool) -> str:
    """The logit evaluation a call takes: the decode kernels for up to 16
    tokens and 64 assignments (d a power of two in [256, 2048], f one in
    [64, 512]), else the routing GEMM."""
    pow2 = lambda v: v & (v - 1) == 0
    gemv = (not prefill and n_tok <= 16 and n_tok * shape.k <= 64 and 256 <= shape.d <= 2048 and pow2(shape.d)
            and 64 <= shape.f <= 512 and pow2(shape.f))
    if gemv:
        return "f64"
    return "mfma_split" if shape.act == "f32" else "mfma"


def c3_delta(H_bits, u, mode: str, extra_abs=None) -> np.ndarray:
    """Per-expert bound on |z_gpu - z_oracle| when both evaluate the same rows
    on the same u: the GPU's accumulation bound plus the oracle's fp64 one,
    plus fp64 rounding of the added bias / history terms (extra_abs: their
    absolute values)."""
    H = np.abs(oracle.bf16_to_f64(H_bits))
    u = np.abs(np.asarray(u, dtype=np.float64))
    absdot = H @ u
    d = u.shape[-1]
    if mode == "exact":
        return np.zeros_like(absdot)
    delta = (gpu_error_factor(mode, d) + gamma_n(d, U53)) * absdot
    if extra_abs is not None:
        delta = delta + 8 * U53 * (absdot + np.abs(extra_abs))
    return delta


def routing_check(z, got, ref, delta):
    """'exact' when the ordered top-k lists agree; 'certified' when they differ
    but the GPU's list is the top-k order of some logits within delta of the
    oracle's (pairwise interval conditions, which suffice for intervals);
    None otherwise."""
    got = [int(g) for g in got]
    ref = [int(r) for r in ref]
    if got == ref:
        return "exact"
    z = np.asarray(z, dtype=np.float64)
    delta = np.broadcast_to(np.asarray(delta, dtype=np.float64), z.shape)
    E, k = z.shape[0], len(got)
    if len(set(got)) != k or any(g < 0 or g >= E for g in got):
        return None
    hi, lo = z + delta, z - delta

    def may_precede(a, b):
        return hi[a] > lo[b] or (hi[a] == lo[b] and a < b)

    for i in range(k):
        for j in range(i + 1, k):
            if not may_precede(got[i], got[j]):
                return None
    sel = set(got)
    others = np.array([e for e in range(E) if e not in sel], dtype=np.int64)
    for g in got:
        bad = ~((hi[g] > lo[others]) | ((hi[g] == lo[others]) & (g < others)))
        if np.any(bad):
            return None
    return "certified"


def check_routing(z, got, ref, delta, what) -> int:
    """Assert the routing agrees (exact or certified); return 1 for a certified
    near tie, 0 for an exact match."""
    r = routing_check(z, got, ref, delta)
    assert r is not None, (what, list(got), list(ref))
    return 1 if r == "certified" else 0


def batched_logits(H_bits, u, mode, bias=None):
    """Logits H u (+ bias) of many rows u [n, d] and their C3 bounds [n, E]."""
    H = oracle.bf16_to_f64(H_bits)
    z = u @ H.T
    absdot = np.abs(u) @ np.abs(H).T
    d = u.shape[-1]
    delta = (gpu_error_factor(mode, d) + gamma_n(d, U53)) * absdot
    if mode == "exact":
        delta = np.zeros_like(absdot)
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)
        if mode != "exact":
            delta = delta + 8 * U53 * (absdot + np.abs(bias))
    return z, delta


GELU_SLOPE = 1.13     # max |d/da a Phi(a)| = Phi(sqrt 2) + sqrt 2 phi(sqrt 2) = 1.1289


def mlp_logits_and_delta(lw, u, cur, prev, mode):
    """The head's MLP branch on u (oracle) and a bound on the GPU's deviation
    from it: fc1's hidden part through the routing GEMM (mode), its one-hot
    columns and bias added in fp64, erf-GELU in fp64 (|GELU'| <= 1.13, erf
    within a few ulps), fc2 in fp64."""
    E = lw.head.shape[0]
    W1u = oracle.bf16_to_f64(lw.head_fc1)
    W1oh = oracle.bf16_to_f64(lw.head_fc1_oh)
    W2 = oracle.bf16_to_f64(lw.head_fc2)
    x_oh = oracle.onehot_input(E, cur, prev)
    b1 = np.zeros(W1u.shape[0]) if lw.head_fc1_bias is None else np.asarray(lw.head_fc1_bias, np.float64)
    a1 = W1u @ u + W1oh.T @ x_oh + b1
    d = u.shape[-1]
    da1 = (gpu_error_factor(mode, d) + gamma_n(d, U53)) * (np.abs(W1u) @ np.abs(u)) \
        + 8 * U53 * (np.abs(a1) + np.abs(W1oh).T @ x_oh + np.abs(b1))
    g = oracle.gelu_erf(a1)
    dg = GELU_SLOPE * da1 + 8 * U53 * (np.abs(g) + np.abs(a1))
    z = W2 @ g
    dz = np.abs(W2) @ dg + 2 * gamma_n(W2.shape[1], U53) * (np.abs(W2) @ np.abs(g))
    return z, dz


def layer_same_input_check(lw, x, mode, *, got_used, got_used_w, route_in, got_y=None, got_pred=None,
                           got_pred_w=None, cur=None, prev=None, tol=2e-3, rows=None, what=""):
    """Check one layer call on the input the GPU saw (x: fp64 [n, d], the fp32
    residual stream; the norm is fused). route_in: (idx, w) given per row
    (rows starting with -1 self-route) or None. rows: the rows whose block
    output is computed (all when None); routing is checked on every row.
    Returns (certified near ties, max block rel-L2 over the computed rows)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    n = x.shape[0]
    u = np.stack([oracle.block_input(lw, x[t], True) for t in range(n)])
    flips = 0
    self_rows = [t for t in range(n) if route_in is None or route_in[0][t][0] < 0]
    if self_rows:
        zr, dr = batched_logits(lw.router, u[self_rows], mode, lw.router_bias)
        for i, t in enumerate(self_rows):
            ref_i, ref_w = oracle.route(zr[i], lw.k)
            c = check_routing(zr[i], got_used[t], ref_i, dr[i], f"{what} self-routed row {t}")
            flips += c
            if not c:
                assert np.allclose(got_used_w[t], ref_w, rtol=1e-5, atol=1e-7), (what, t)
    sr = set(self_rows)
    for t in range(n):
        if t in sr:
            continue
        assert np.array_equal(got_used[t], route_in[0][t]), (what, t)
        assert np.array_equal(np.asarray(got_used_w[t], np.float32), np.asarray(route_in[1][t], np.float32)), (what, t)
    if got_pred is not None:
        zh, dh = batched_logits(lw.head, u, mode, lw.head_bias)
        for t in range(n):
            z, dz = zh[t], dh[t]
            ct = None if cur is None else cur[t]
            pt = None if prev is None else prev[t]
            if (lw.hist_cur is not None and ct is not None) or (lw.hist_prev is not None and pt is not None):
                hist = oracle.head_logits(np.zeros_like(lw.head), u[t], None, lw.hist_cur, ct, lw.hist_prev, pt)
                z = z + hist
                if mode != "exact":
                    dz = dz + 8 * U53 * (np.abs(z) + np.abs(hist))
            if lw.head_fc1 is not None:
                # the MLP branch's fc1 always takes the routing GEMM
                zm, dm = mlp_logits_and_delta(lw, u[t], ct, pt, "mfma_split" if lw.act == "f32" else "mfma")
                z = z + zm
                dz = dz + dm + 8 * U53 * np.abs(z)
            ref_i, ref_w = oracle.route(z, len(got_pred[t]))
            c = check_routing(z, got_pred[t], ref_i, dz, f"{what} prediction row {t}")
            flips += c
            if not c:
                assert np.allclose(got_pred_w[t], ref_w, rtol=1e-5, atol=1e-7), (what, t)
    err = 0.0
    if got_y is not None:
        for t in (range(n) if rows is None else rows):
            y_ref = oracle.moe_block(lw, u[t], got_used[t], np.asarray(got_used_w[t], dtype=np.float64))
            e = rel_l2_rows(np.asarray(got_y[t], dtype=np.float64), y_ref)
            assert e <= tol, (what, t, e)
            err = max(err, e)
    return flips, err

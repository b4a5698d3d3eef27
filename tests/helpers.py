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
    )


def gpu_layer(shape: synth.Shape, w: dict, *, fused: bool, resident: bool = True, slab_slots: int = 0,
              max_tokens: int = 8, head: bool = True, act=None, keep_host: bool = False):
    import sparse_moe_decode_prerouter_amd as moe
    dev = "cuda"

    def dv(t):
        return None if t is None else t.to(dev).contiguous()

    if resident:
        store, shared = dv(w["store"]), dv(w["shared"])
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
        fuse_norm_residual=fused, resident=resident, slab_slots=slab_slots)


def rel_l2_rows(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.atleast_2d(np.asarray(got, dtype=np.float64))
    ref = np.atleast_2d(np.asarray(ref, dtype=np.float64))
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    return float(np.max(num / den))


def logit_gap_ok(z: np.ndarray, k: int, got_idx, ref_idx, delta: float) -> bool:
    """Certified near tie: the two top-k selections differ only among experts
    whose logits lie within 2*delta of the k-th / (k+1)-th boundary."""
    z = np.asarray(z, dtype=np.float64)
    order = oracle.topk(z, len(z))
    kth, k1 = z[order[k - 1]], z[order[k]] if k < len(z) else -np.inf
    lo, hi = k1 - 2 * delta, kth + 2 * delta
    diff = set(int(i) for i in got_idx) ^ set(int(i) for i in ref_idx)
    return all(lo <= z[e] <= hi for e in diff)

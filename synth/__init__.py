"""Seeded synthetic inputs for the per-layer MoE block (prerouter -> staged int4
experts -> SwiGLU/combine -> unmerged LoRA).

This module is shared by the oracle-side tests, the GPU tests and the bench.
It holds random draws, the shapes of the workloads, and the affine int4
group-64 *quantiser* that turns Gaussian weights into a packed checkpoint
(the paper's base weights are int4 affine with groups of 64: "The Other Half of
the Memory Wall", ai.info news page, section on the 35B model). It holds none
of the block's forward arithmetic: no dequantisation, norm, routing, expert
FFN, combine or LoRA lives here.

Byte formats written here (the interface both sides read independently):

expert blob (one expert, model dim d, intermediate f, group G = 64), bytes:
    [0,            f*d/2)   gate  q : uint8 [f][d/2]
    [f*d/2,        f*d)     up    q : uint8 [f][d/2]
    [f*d,          3fd/2)   down  q : uint8 [d][f/2]
    then gate (s,b): fp16 [f][d/64][2], up (s,b): fp16 [f][d/64][2],
         down (s,b): fp16 [d][f/64][2]
    total 27*d*f/16 bytes.
    Element k of a row sits in byte k/2 of that row, low nibble when k is even.
    Weight = s * q + b with (s, b) of the 64-group along the row (K axis).

bf16 tensors are torch.bfloat16; fp16/fp32 as usual.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import torch

GROUP = 64


# ----------------------------------------------------------------------------
# workload shapes
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    d: int            # hidden size
    E: int            # routed experts per layer
    k: int            # experts per token
    f: int            # routed expert intermediate size
    fs: int           # shared expert intermediate size (0: none)
    r: int            # LoRA rank (0: none)
    alpha: float      # LoRA alpha
    act: str          # "f32" or "bf16": dtype of the block input u
    layers: int = 1
    eps: float = 1e-6
    std: float = 0.02  # weight std before quantisation / bf16 rounding

    @property
    def blob_bytes(self) -> int:
        return 27 * self.d * self.f // 16

    @property
    def shared_blob_bytes(self) -> int:
        return 27 * self.d * self.fs // 16


# single layer, one decode token, toy sizes
TINY = Shape("tiny_d256_e16_k2", d=256, E=16, k=2, f=128, fs=128, r=8, alpha=16.0, act="f32")
# one layer at the 35B tier shape (decode B in {1, 4})
LAYER35B = Shape("layer_d2048_e256_k4", d=2048, E=256, k=4, f=512, fs=512, r=16, alpha=16.0, act="bf16")
# 40-layer MoE-only stack at the 35B tier shape
STACK35B = dataclasses.replace(LAYER35B, name="stack40_d2048_e256_k4", layers=40)


def scaled_stack(layers: int, name: Optional[str] = None) -> Shape:
    return dataclasses.replace(STACK35B, layers=layers, name=name or f"stack{layers}_d2048_e256_k4")


# ----------------------------------------------------------------------------
# seeded draws
# ----------------------------------------------------------------------------
def seed_of(*key) -> int:
    h = hashlib.sha256(repr(tuple(key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def generator(key, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*key) if isinstance(key, tuple) else seed_of(key))
    return g


def gaussian(shape, std, key, device="cpu") -> torch.Tensor:
    g = generator(key, device)
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * std


def uniform_int(shape, lo, hi, key, device="cpu") -> torch.Tensor:
    g = generator(key, device)
    return torch.randint(lo, hi, tuple(shape), generator=g, device=device, dtype=torch.int64)


# ----------------------------------------------------------------------------
# affine int4 group-64 quantiser (data generation only)
# ----------------------------------------------------------------------------
def quantize_g64(w: torch.Tensor):
    """w [..., N, K] float32 -> (packed uint8 [..., N, K/2], sb fp16 [..., N, K/64, 2]).

    Per 64-group along K: s = fp16((max-min)/15), b = fp16(min),
    q = clip(round_half_even((w - b)/s), 0, 15); s = 0 gives q = 0.
    """
    *lead, N, K = w.shape
    assert K % GROUP == 0
    g = w.reshape(*lead, N, K // GROUP, GROUP).float()
    lo = g.amin(-1)
    hi = g.amax(-1)
    s = ((hi - lo) / 15.0).half()
    b = lo.half()
    sf = s.float().unsqueeze(-1)
    bf = b.float().unsqueeze(-1)
    safe = torch.where(sf > 0, sf, torch.ones_like(sf))
    q = torch.where(sf > 0, torch.round((g - bf) / safe), torch.zeros_like(g))
    q = q.clamp_(0, 15).to(torch.uint8).reshape(*lead, N, K)
    packed = q[..., 0::2] | (q[..., 1::2] << 4)
    sb = torch.stack([s, b], dim=-1)
    return packed.contiguous(), sb.contiguous()


def pack_blob(gate_q, gate_sb, up_q, up_sb, down_q, down_sb) -> torch.Tensor:
    """Concatenate one or many experts' parts into blobs (uint8 [..., 27df/16])."""
    lead = gate_q.shape[:-2]
    parts = [gate_q, up_q, down_q, gate_sb, up_sb, down_sb]
    flat = [p.contiguous().view(torch.uint8).reshape(*lead, -1) for p in parts]
    return torch.cat(flat, dim=-1).contiguous()


def expert_blobs(d, f, n, key, std=0.02, device="cpu", chunk=16) -> torch.Tensor:
    """n experts' blobs, uint8 [n, 27df/16]; weights ~ N(0, std) then quantised."""
    out = torch.empty((n, 27 * d * f // 16), dtype=torch.uint8, device=device)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        m = c1 - c0
        kk = tuple(key) + (c0,)
        wg = gaussian((m, f, d), std, kk + ("gate",), device)
        wu = gaussian((m, f, d), std, kk + ("up",), device)
        wd = gaussian((m, d, f), std, kk + ("down",), device)
        gq, gs = quantize_g64(wg)
        uq, us = quantize_g64(wu)
        dq, ds = quantize_g64(wd)
        out[c0:c1] = pack_blob(gq, gs, uq, us, dq, ds)
        del wg, wu, wd
    return out


# ----------------------------------------------------------------------------
# per-layer weights
# ----------------------------------------------------------------------------
def layer_weights(shape: Shape, layer: int, device="cpu", with_head=True, with_router=True,
                  tag: str = "w") -> dict:
    """All tensors of one MoE layer (seeded by shape name, layer index and tensor name)."""
    d, E, r = shape.d, shape.E, shape.r
    key = (tag, shape.name, layer)
    sd = shape.std
    w = {}
    w["head"] = gaussian((E, d), sd, key + ("head",), device).bfloat16() if with_head else None
    w["router"] = gaussian((E, d), sd, key + ("router",), device).bfloat16() if with_router else None
    w["shared_gate"] = gaussian((d,), sd, key + ("sgate",), device).bfloat16() if shape.fs else None
    if r:
        w["lora_a"] = gaussian((r, d), sd, key + ("lora_a",), device).bfloat16()
        w["lora_b"] = gaussian((d, r), sd, key + ("lora_b",), device).bfloat16()
    else:
        w["lora_a"] = w["lora_b"] = None
    w["gamma"] = 1.0 + gaussian((d,), sd, key + ("gamma",), device)
    w["store"] = expert_blobs(d, shape.f, E, key + ("experts",), sd, device)
    w["shared"] = expert_blobs(d, shape.fs, 1, key + ("shared",), sd, device)[0] if shape.fs else None
    w["head_bias"] = None
    w["hist_cur"] = None
    w["hist_prev"] = None
    return w


def head_mlp_weights(shape: Shape, layer: int, hidden: int, device="cpu", tag: str = "w") -> dict:
    """The head's MLP branch of one layer, every entry ~ N(0, std) (the
    matrices rounded to bf16): fc1's hidden-state columns [H1, d], its
    one-hot columns [2E, H1] (current token's experts, then the previous
    token's), fc1's bias fp32 [H1], fc2 [E, H1]."""
    d, E = shape.d, shape.E
    key = (tag, shape.name, layer, "mlp", hidden)
    sd = shape.std
    return {
        "head_fc1": gaussian((hidden, d), sd, key + ("fc1",), device).bfloat16(),
        "head_fc1_onehot": gaussian((2 * E, hidden), sd * 10, key + ("fc1oh",), device).bfloat16(),
        "head_fc1_bias": gaussian((hidden,), sd * 10, key + ("b1",), device),
        "head_fc2": gaussian((E, hidden), sd * 5, key + ("fc2",), device).bfloat16(),
    }


def shared_adapter(shape: Shape, layer: int, rank: int, delta_rms: float = 1e-3, device="cpu", tag: str = "w") -> dict:
    """A and B of a recovery adapter on the shared expert's gate, up and down
    projections, bf16, entries ~ N(0, sigma) with sigma^2 = delta_rms / sqrt(r):
    with alpha = r (scale 1) each projection's delta B A then has an RMS of
    about delta_rms (the pages put the adapter's delta near 1e-3, below the
    int4 step)."""
    d, fs = shape.d, shape.fs
    sig = math.sqrt(delta_rms / math.sqrt(rank))
    key = (tag, shape.name, layer, "sadapter", rank)
    return {
        "shared_lora_a": gaussian((2 * rank, d), sig, key + ("a",), device).bfloat16(),
        "shared_lora_b": gaussian((2 * fs, rank), sig, key + ("b",), device).bfloat16(),
        "shared_lora_ad": gaussian((rank, fs), sig, key + ("ad",), device).bfloat16(),
        "shared_lora_bd": gaussian((d, rank), sig, key + ("bd",), device).bfloat16(),
        "shared_lora_alpha": float(rank),
    }


def activations(shape: Shape, n_tok: int, key, device="cpu", dtype=None) -> torch.Tensor:
    """x ~ N(0, 1), [n_tok, d]; dtype defaults to the shape's act dtype."""
    x = gaussian((n_tok, shape.d), 1.0, ("act", shape.name) + tuple(key), device)
    dt = dtype or (torch.bfloat16 if shape.act == "bf16" else torch.float32)
    return x.to(dt)


def random_routing(n_tok: int, E: int, k: int, key, device="cpu"):
    """Distinct expert ids per row plus positive weights that sum to one (for
    exercising the block with routing supplied from outside)."""
    g = generator(("route",) + tuple(key), "cpu")
    idx = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(n_tok)]).to(torch.int32)
    w = torch.rand(n_tok, k, generator=g, dtype=torch.float64) + 0.1
    w = (w / w.sum(-1, keepdim=True)).float()
    return idx.to(device), w.to(device)


# ----------------------------------------------------------------------------
# Zipf popularity bias (batched decode workload)
# ----------------------------------------------------------------------------
def zipf_bias(E: int, s: float, tau: float, key, device="cpu") -> torch.Tensor:
    """b_e = tau * log p_{pi(e)}, p_r proportional to r^-s, pi a seeded permutation."""
    g = generator(("zipf",) + tuple(key), "cpu")
    perm = torch.randperm(E, generator=g)
    ranks = torch.arange(1, E + 1, dtype=torch.float64)
    logp = -s * torch.log(ranks)
    logp = logp - torch.logsumexp(logp, 0)
    b = torch.empty(E, dtype=torch.float64)
    b[perm] = logp
    return (tau * b).float().to(device)


def sticky_history(E: int, beta: float, device="cpu") -> torch.Tensor:
    """History matrix adding beta to an expert's logit when it is in the
    current routing of the predicted layer: beta * I (fp32 [E, E])."""
    return (beta * torch.eye(E, dtype=torch.float32)).to(device)


def bf16_bits(t: torch.Tensor):
    """Raw bf16 bit patterns (numpy uint16) of a bf16 tensor."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def f16_bits(t: torch.Tensor):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def to_numpy_bytes(t: torch.Tensor):
    return t.detach().cpu().contiguous().numpy()

#!/usr/bin/env python3
"""Benchmark of the MoE block stack on one MI355X.

Headline: batch-1 decode through a 40-layer MoE-only stack (RMSNorm -> MoE
block -> residual per layer; hidden 2048, 256 experts, top-4 + 1 shared
expert, intermediate 512, int4 affine group-64 experts, bf16 activations,
LoRA rank 16, prerouter heads routing layer l+1 one token ahead), experts
resident in HBM, K steps replayed from a HIP graph. Also reported: prefill
of 512 tokens through the same stack, the HBM roofline of the decode path
and of its dominant kernel, and the fp64 oracle timed on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD public figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def step_bytes(shape, L, k, with_router_l0=True):
    """Algorithmic HBM bytes of one batch-1 decode step through L layers:
    per layer k routed + 1 shared expert blobs, LoRA A and B, shared gate,
    RMSNorm gamma; heads on layers 0..L-2; layer 0's router."""
    d, E, r = shape.d, shape.E, shape.r
    per_layer = (k + 1) * shape.blob_bytes + 2 * (2 * r * d) + 2 * d + 4 * d
    heads = (L - 1) * 2 * E * d
    router = 2 * E * d if with_router_l0 else 0
    return L * per_layer + heads + router


def kernel_a_bytes(shape, k):
    """Algorithmic bytes of one K_A launch at batch 1 (a layer with a head):
    gate+up of k routed + shared experts, head, LoRA A, shared gate, x, gamma."""
    d, f, E, r = shape.d, shape.f, shape.E, shape.r
    gate_up = 2 * (d * f // 2 + d * f // 64 * 4)
    return (k + 1) * gate_up + 2 * E * d + 2 * r * d + 2 * d + 4 * d + 4 * d


def kernel_b_bytes(shape, k):
    d, f, r = shape.d, shape.f, shape.r
    down = d * f // 2 + d * f // 64 * 4
    return (k + 1) * down + 2 * r * d + (k + 1) * f * 4 + 2 * 4 * d


KA_SOURCES = ("sparse_moe_decode_prerouter_amd/csrc/kernels_deca.hip",
              "sparse_moe_decode_prerouter_amd/csrc/dec_common.h",
              "sparse_moe_decode_prerouter_amd/csrc/device_common.h",
              "sparse_moe_decode_prerouter_amd/csrc/moe_internal.h",
              "sparse_moe_decode_prerouter_amd/csrc/topk.h")
KA_TRAFFIC = "profiles/k_dec_a_hbm_traffic_40layer_decode_bs1.txt"


def source_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per K_A launch from the committed counter summary, if it was
    taken on the kernel source as it is now (else None)."""
    path = os.path.join(ROOT, KA_TRAFFIC)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest(KA_SOURCES):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class LazyStore:
    """Host view of a device expert store for the oracle: blob e is copied on
    first use (the oracle touches only the experts a step routes to)."""

    def __init__(self, dev_store):
        self.dev = dev_store
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = self.dev[e].cpu().numpy()
        return self.cache[e]


def make_layer(moe, shape, w, l, L, *, max_tokens, resident=True, store=None, shared=None, slab_slots=0,
               head_bias=None, hist_cur=None):
    return moe.MoeLayer(
        d_model=shape.d, n_experts=shape.E, top_k=shape.k, d_ff=shape.f, d_ff_shared=shape.fs,
        lora_rank=shape.r, lora_alpha=shape.alpha, act_dtype=moe.MOE_ACT_BF16, max_tokens=max_tokens,
        expert_store=w["store"] if store is None else store, shared_blob=w["shared"] if shared is None else shared,
        shared_gate=w["shared_gate"], router=w["router"], head=w["head"] if l + 1 < L else None,
        head_bias=head_bias if l + 1 < L else None, hist_cur=hist_cur if l + 1 < L else None,
        next_n_experts=shape.E if l + 1 < L else 0, next_top_k=shape.k if l + 1 < L else 0,
        lora_a=w["lora_a"], lora_b=w["lora_b"], norm_gamma=w["gamma"], rms_eps=shape.eps,
        fuse_norm_residual=True, resident=resident, slab_slots=slab_slots)


def time_stack_steps(torch, stack, L, B, k, d, steps, warm, key, synth, shape, used=None):
    """Graph-replayed decode steps of a stack (eager first step); returns
    (ms per step, the last routing buffer)."""
    dev = "cuda"
    xbank = torch.stack([synth.activations(shape, B, (key, t), device=dev, dtype=torch.float32)
                         for t in range(warm + steps)])
    xout = torch.empty((B, d), dtype=torch.float32, device=dev)
    pidx = [torch.full((L, B, k), -1, dtype=torch.int32, device=dev) for _ in range(2)]
    pw = [torch.zeros((L, B, k), dtype=torch.float32, device=dev) for _ in range(2)]

    def step(t):
        stack.decode(xbank[t], pidx[t % 2], pw[t % 2], pidx[(t + 1) % 2], pw[(t + 1) % 2], x_out=xout,
                     first_step=(t == 0), used_idx=used)

    step(0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g_warm, g_timed = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_warm, stream=s):
        for t in range(1, warm):
            step(t)
    with torch.cuda.graph(g_timed, stream=s):
        for t in range(warm, warm + steps):
            step(t)
    g_warm.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g_timed.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, pidx[(warm + steps) % 2]


def extra_measurements(args, torch, np, moe, synth, shape, ws, layers):
    """The other workloads of the method, each timed on this GPU: batched
    decode with Zipf-popular, sticky routing; streamed decode (experts staged
    per step from pinned host memory) against on-demand staging; one layer per
    call at batch 1 and 4; a long prefill for the matrix-core rate."""
    out = {}
    L, k, d, E, blob = len(layers), shape.k, shape.d, shape.E, shape.blob_bytes

    # ---- batched decode, B = 32, Zipf(1.1) popularity + stickiness (calibrated)
    with open(os.path.join(ROOT, "tests", "golden", "zipf_calibration.json")) as fh:
        cal = json.load(fh)
    B = 32
    hist = synth.sticky_history(E, cal["beta"], device="cuda")
    zl = [make_layer(moe, shape, w, l, L, max_tokens=B,
                     head_bias=synth.zipf_bias(E, cal["zipf_s"], cal["tau"], ("bench", l), device="cuda"),
                     hist_cur=hist) for l, w in enumerate(ws)]
    zs = moe.MoeStack(zl)
    used = torch.full((L, B, k), -1, dtype=torch.int32, device="cuda")
    ms, _ = time_stack_steps(torch, zs, L, B, k, d, 32, 5, "bench_zipf", synth, shape, used=used)
    assert all(Lr.status() == 0 for Lr in zl)
    u = used.cpu().numpy()
    U = [len(set(u[l].ravel().tolist()) - {-1}) for l in range(L)]
    bb = sum((x + 1) * blob for x in U) + (L - 1) * 2 * E * d + L * (4 * shape.r * d + 6 * d)
    out["batched_decode_b32"] = {"tok_s": round(B / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
                                 "distinct_experts_per_layer": round(float(np.mean(U)), 1),
                                 "algorithmic_GBs": round(bb / (ms * 1e-3) / 1e9, 1),
                                 "hbm_frac": round(bb / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4)}
    log(f"batched decode B={B} (Zipf + sticky): {ms * 1e3:.0f} us/step, {B / (ms / 1e3):.0f} tok/s, "
        f"U={np.mean(U):.1f} experts/layer, {bb / (ms * 1e-3) / 1e9:.0f} GB/s algorithmic")
    zs.close()
    for Lr in zl:
        Lr.close()
    del zl, zs

    # ---- streamed decode, B = 1: every layer's routed experts staged per step
    # from pinned host memory into a 5-slot HBM slab on a side stream (one pinned
    # copy of a layer's experts serves all layers: the bytes moved are the same)
    pstore = ws[0]["store"].cpu().pin_memory()
    pshared = ws[0]["shared"].cpu().pin_memory()
    sl = [make_layer(moe, shape, w, l, L, max_tokens=1, resident=False, store=pstore, shared=pshared,
                     slab_slots=k + 1) for l, w in enumerate(ws)]
    ss = moe.MoeStack(sl)
    cs = torch.cuda.Stream()
    xs = [synth.activations(shape, 1, ("bench_str", t), device="cuda", dtype=torch.float32) for t in range(24)]
    xo = torch.empty((1, d), dtype=torch.float32, device="cuda")
    pidx = [torch.full((L, 1, k), -1, dtype=torch.int32, device="cuda") for _ in range(2)]
    pw = [torch.zeros((L, 1, k), dtype=torch.float32, device="cuda") for _ in range(2)]

    def streamed_step(t, reactive):
        if reactive or t == 0:
            # on demand: every layer routes itself and stages inside the call
            ss.decode(xs[t], pidx[t % 2], pw[t % 2], pidx[(t + 1) % 2], pw[(t + 1) % 2], x_out=xo, first_step=True)
            return
        pred = pidx[t % 2].cpu().numpy()            # the previous step's predictions
        for l in range(1, L):
            sl[l].stage(sorted(set(int(e) for e in pred[l, 0] if e >= 0)), stream=cs)
        ss.decode(xs[t], pidx[t % 2], pw[t % 2], pidx[(t + 1) % 2], pw[(t + 1) % 2], x_out=xo, first_step=False)

    res = {}
    for mode, reactive in (("prerouted", False), ("on_demand", True)):
        for t in range(4):
            streamed_step(t, reactive)
        torch.cuda.synchronize()
        b0 = sum(Lr.slots()[1] for Lr in sl)
        n = 16
        c0 = time.time()
        for t in range(4, 4 + n):
            streamed_step(t, reactive)
        torch.cuda.synchronize()
        el = time.time() - c0
        moved = sum(Lr.slots()[1] for Lr in sl) - b0
        assert all(Lr.status() == 0 for Lr in sl), [Lr.status() for Lr in sl]
        res[mode] = {"tok_s": round(n / el, 1), "ms_per_step": round(el / n * 1e3, 3),
                     "staged_MB_per_step": round(moved / n / 1e6, 1),
                     "staging_GBs": round(moved / el / 1e9, 2)}
        log(f"streamed decode ({mode}): {el / n * 1e3:.2f} ms/step, {n / el:.1f} tok/s, "
            f"{moved / n / 1e6:.0f} MB staged/step, {moved / el / 1e9:.1f} GB/s host->HBM")
    out["streamed_decode_b1"] = res
    ss.close()
    for Lr in sl:
        Lr.close()
    del sl, ss, pstore, pshared

    # ---- one layer per call, batch 1 and 4 (given routing; graph of 64 calls)
    lay = make_layer(moe, shape, ws[1], 1, L, max_tokens=4)
    for B in (1, 4):
        x = synth.activations(shape, B, ("bench_one", B), device="cuda", dtype=torch.float32)
        ridx, rw = synth.random_routing(B, E, k, ("bench_one", B))
        ridx, rw = ridx.cuda(), rw.cuda()
        y = torch.empty_like(x)
        lay.decode(x, ridx, rw, y=y)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(64):
                lay.decode(x, ridx, rw, y=y)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(4):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 256
        Ub = len(set(ridx.cpu().numpy().ravel().tolist()))
        lb = (Ub + 1) * blob + 2 * E * d + 4 * shape.r * d + 6 * d
        out[f"layer_decode_b{B}"] = {"us_per_call": round(us, 2), "algorithmic_GBs": round(lb / (us * 1e-6) / 1e9, 1)}
        log(f"one layer, B={B}: {us:.2f} us/call, {lb / (us * 1e-6) / 1e9:.0f} GB/s algorithmic")
    lay.close()

    # ---- long prefill (T = 8192 tokens through one layer): the matrix-core rate
    T = 8192
    lay = make_layer(moe, shape, ws[1], 1, L, max_tokens=T)
    x = synth.activations(shape, T, ("bench_long",), device="cuda", dtype=torch.float32)
    y = torch.empty_like(x)
    lay.prefill(x, y=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        lay.prefill(x, y=y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    assert lay.status() == 0
    flops = T * (6 * d * shape.f * (k + 1) + 2 * d * E * 2 + 4 * shape.r * d)
    out["prefill_t8192_one_layer"] = {"ms": round(ms, 3), "tok_s": round(T / (ms / 1e3), 1),
                                      "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
                                      "mfma_frac_bf16": round(flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4)}
    log(f"prefill T={T}, one layer: {ms:.3f} ms, {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s "
        f"({flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12):.3f} of bf16 MFMA peak)")
    lay.close()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=40)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--prefill-tokens", type=int, default=512)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=8)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads (batched, streamed, ...)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (scale for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the MoE block path here runs on a single MI355X "
              f"(--gpus {args.gpus} is not supported; how it would shard is described in DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe:
        # a plain copy kernel of known size: the reference the HBM byte counters
        # of the profiled kernels are scaled by
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 3}), flush=True)
        return

    import synth
    import sparse_moe_decode_prerouter_amd as moe

    assert torch.cuda.is_available()
    dev = "cuda"
    L, B, K, W = args.layers, args.batch, args.steps, args.warmup
    shape = synth.scaled_stack(L) if L != 40 else synth.STACK35B
    k = shape.k
    T = args.prefill_tokens
    t0 = time.time()
    layers, ws = [], []
    for l in range(L):
        w = synth.layer_weights(shape, l, device=dev, tag="bench")
        ws.append(w)
        layers.append(moe.MoeLayer(
            d_model=shape.d, n_experts=shape.E, top_k=k, d_ff=shape.f, d_ff_shared=shape.fs, lora_rank=shape.r,
            lora_alpha=shape.alpha, act_dtype=moe.MOE_ACT_BF16, max_tokens=max(B, 1 if args.no_prefill else T),
            expert_store=w["store"], shared_blob=w["shared"], shared_gate=w["shared_gate"], router=w["router"],
            head=w["head"] if l + 1 < L else None, next_n_experts=shape.E if l + 1 < L else 0,
            next_top_k=k if l + 1 < L else 0, lora_a=w["lora_a"], lora_b=w["lora_b"], norm_gamma=w["gamma"],
            rms_eps=shape.eps, fuse_norm_residual=True, resident=True))
    torch.cuda.synchronize()
    log(f"built {L} layers ({L * shape.E * shape.blob_bytes / 2**30:.1f} GiB experts) in {time.time() - t0:.1f}s")
    stack = moe.MoeStack(layers)

    # ---- decode: step inputs and rotating routing buffers
    xbank = torch.stack([synth.activations(shape, B, ("bench", t), device=dev, dtype=torch.float32)
                         for t in range(W + K)])
    xout = torch.empty((B, shape.d), dtype=torch.float32, device=dev)
    pidx = [torch.full((L, B, k), -1, dtype=torch.int32, device=dev) for _ in range(2)]
    pw = [torch.zeros((L, B, k), dtype=torch.float32, device=dev) for _ in range(2)]

    def step(t):
        stack.decode(xbank[t], pidx[t % 2], pw[t % 2], pidx[(t + 1) % 2], pw[(t + 1) % 2], x_out=xout,
                     first_step=(t == 0))

    # eager first step (all layers self-route), then graphs for warmup and timed steps
    step(0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g_warm, g_timed = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_warm, stream=s):
        for t in range(1, W):
            step(t)
    with torch.cuda.graph(g_timed, stream=s):
        for t in range(W, W + K):
            step(t)
    torch.cuda.synchronize()
    log("graphs captured")
    g_warm.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g_timed.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    st = [Lr.status() for Lr in layers]
    assert all(v == 0 for v in st), st
    ms_step = ms / K
    tok_s = B * K / (ms / 1e3)
    sb = step_bytes(shape, L, k)
    roof_tok_s = HBM_PEAK_GBS * 1e9 / sb * B
    log(f"decode: {ms_step * 1e3:.1f} us/step, {tok_s:.0f} tok/s, {sb / ms_step / 1e6:.0f} GB/s algorithmic, "
        f"{tok_s / roof_tok_s:.3f} of the HBM roofline ({roof_tok_s:.0f} tok/s)")

    # ---- kernel-level timing: eager replays of the timed steps with kernel-timestamp
    # events (each launch's own begin/end, as a kernel trace reports them)
    for Lr in layers:
        Lr.set_profiling(True)
    a_ms, b_ms, r_ms = [], [], []
    with torch.cuda.stream(s):
        for t in range(W, W + min(K, 16)):
            step(t)
            torch.cuda.current_stream().synchronize()
            for l, Lr in enumerate(layers):
                rr, aa, bb = Lr.kernel_ms()
                if l + 1 < L:
                    a_ms.append(aa)
                b_ms.append(bb)
                if rr >= 0:
                    r_ms.append(rr)
    for Lr in layers:
        Lr.set_profiling(False)
    a_avg = float(np.mean(a_ms))
    b_avg = float(np.mean(b_ms))
    ab = kernel_a_bytes(shape, k)
    bb_ = kernel_b_bytes(shape, k)
    log(f"K_A avg {a_avg * 1e3:.2f} us ({ab / (a_avg * 1e-3) / 1e9:.0f} GB/s), K_B avg {b_avg * 1e3:.2f} us "
        f"({bb_ / (b_avg * 1e-3) / 1e9:.0f} GB/s), router avg {np.mean(r_ms) * 1e3 if r_ms else -1:.2f} us")

    # ---- prefill
    prefill = None
    if not args.no_prefill:
        xp = synth.activations(shape, T, ("bench_prefill",), device=dev, dtype=torch.float32)
        xw = xp.clone()
        stack.prefill(xw)
        torch.cuda.synchronize()
        reps = 3
        times = []
        for _ in range(reps):
            xw.copy_(xp)
            torch.cuda.synchronize()
            e0.record()
            stack.prefill(xw)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        pms = float(np.median(times))
        assert all(Lr.status() == 0 for Lr in layers)
        # algorithmic bytes: every expert of every layer (all are touched at 512 tokens w.h.p.),
        # shared, heads, routers (token 0 self-routes everywhere), LoRA
        pb = L * ((shape.E + 1) * shape.blob_bytes + 2 * shape.E * shape.d + 4 * shape.r * shape.d) \
            + (L - 1) * 2 * shape.E * shape.d
        flops = L * T * (6 * shape.d * shape.f * (k + 1) + 2 * shape.d * shape.E * 2 + 4 * shape.r * shape.d)
        prefill = {"value": round(T / (pms / 1e3), 1), "unit": "tok/s", "tokens": T, "ms": round(pms, 3),
                   "hbm_frac": round(pb / (pms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                   "mfma_frac_bf16": round(flops / (pms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 5)}
        log(f"prefill {T} tokens: {pms:.2f} ms, {prefill['value']:.0f} tok/s, hbm frac {prefill['hbm_frac']:.3f}")

    extra = None if args.no_extra else extra_measurements(args, torch, np, moe, synth, shape, ws, layers)

    # ---- CPU baseline: the fp64 oracle on a bounded sample (1 decode step of the stack)
    cpu = None
    if not args.no_cpu:
        import oracle
        cores = os.cpu_count()
        try:
            from threadpoolctl import threadpool_info
            thr = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:
            thr = cores
        ora = []
        for l, w in enumerate(ws):
            ora.append(oracle.LayerWeights(
                d=shape.d, E=shape.E, k=k, f=shape.f, fs=shape.fs, r=shape.r, alpha=shape.alpha, eps=shape.eps,
                act="bf16", store=LazyStore(w["store"]), shared=w["shared"].cpu().numpy(),
                shared_gate=synth.bf16_bits(w["shared_gate"]), lora_a=synth.bf16_bits(w["lora_a"]),
                lora_b=synth.bf16_bits(w["lora_b"]), gamma=w["gamma"].double().cpu().numpy(),
                head=synth.bf16_bits(w["head"]) if l + 1 < L else None, router=synth.bf16_bits(w["router"])))
        xs = xbank[:args.cpu_steps].double().cpu().numpy()
        # step 0 self-routes every layer; report steady-state-like cost per step incl. that
        c0 = time.time()
        oracle.stack_decode(ora, xs, args.cpu_steps)
        cs = time.time() - c0
        cpu = {"value": round(B * args.cpu_steps / cs, 4), "unit": "tok/s", "cores": int(thr), "kind": "oracle",
               "sample": f"{args.cpu_steps} decode step(s) of the {L}-layer stack at batch {B}, fp64 NumPy "
                         f"(first step: every layer self-routes), {cs:.1f} s"}
        log(f"oracle: {cs:.1f} s for {args.cpu_steps} step(s)")

    out = {
        "metric": "decode tok/s (40-layer MoE stack, bs=1) + % of HBM roofline; prefill tok/s",
        "value": round(tok_s, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,0.02) weights quantised to int4 g64, N(0,1) step inputs",
        "config": {"workload": f"{L}-layer MoE-only stack, batch-{B} decode", "layers": L, "batch": B,
                   "hidden": shape.d, "experts": shape.E, "top_k": k, "expert_intermediate": shape.f,
                   "shared_intermediate": shape.fs, "lora_rank": shape.r, "experts_resident": True},
        "hbm_roofline_frac": round(tok_s / roof_tok_s, 4),
        "hbm_roofline_tok_s": round(roof_tok_s, 1),
        "bytes_per_step": sb,
        "roofline": {"bound": "hbm", "kernel": "k_dec_a (norm + routed/shared gate-up GEMV + head)",
                     "achieved": round(ab / (a_avg * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ab / (a_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "bytes_per_launch": ab, "avg_launch_us": round(a_avg * 1e3, 3)},
        "kernel_b": {"kernel": "k_dec_b", "avg_launch_us": round(b_avg * 1e3, 3), "bytes_per_launch": bb_,
                     "achieved_GBs": round(bb_ / (b_avg * 1e-3) / 1e9, 1)},
        "prefill": prefill,
        "other_workloads": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

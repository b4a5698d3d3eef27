"""GPU parity at full sizes: the 512-token prefill (and a long 8192-token one)
and a 32-token decode batch
of one 35B-shape layer (the grouped-GEMM path), the batched decode stack
with the Zipf popularity + stickiness routing workload, and the 40-layer
batch-1 decode stack.

At these sizes the oracle computes sampled rows one by one (the block is
per-token), while the routing of every row is compared: indices bit-exact
except certified near ties (oracle logit gap < 1e-3, counted), block outputs
within rel-L2 2e-3 per row.
"""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (gpu_layer, layer_same_input_check, layer_tensors, oracle_layer, rel_l2_rows, routing_mode,
                     say)

pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

TOL = 2e-3
STACK_TOL = 1e-2
HERE = os.path.dirname(os.path.abspath(__file__))


def sampled_layer_check(n_tok, prefill, seed, sample, shape=synth.LAYER35B, same_experts=None):
    """One layer call at full size. Every row's routing decisions (the
    self-routed row 0 and every row's head prediction) are checked against
    the oracle's logits on the same input; block outputs of the sampled rows
    within rel-L2 2e-3."""
    say(f"{shape.name} n_tok={n_tok} prefill={prefill} sampled rows={len(sample)} same_experts={same_experts}")
    w = layer_tensors(shape, layer=seed, tag="large")
    lw = oracle_layer(shape, w)
    x = synth.activations(shape, n_tok, ("large", seed, n_tok), dtype=torch.float32)
    ridx, rw = synth.random_routing(n_tok, shape.E, shape.k, ("large", seed, n_tok))
    if same_experts is not None:
        # every row routes to the same experts (in a row-dependent order)
        base = torch.tensor(same_experts, dtype=torch.int32)
        ridx = torch.stack([torch.roll(base, t % shape.k) for t in range(n_tok)])
    ridx[0] = -1                     # row 0 self-routes (as the first prefill row does)
    L = gpu_layer(shape, w, fused=True, max_tokens=n_tok)
    call = L.prefill if prefill else L.decode
    out = call(x.cuda(), ridx.cuda(), rw.cuda())
    torch.cuda.synchronize()
    assert L.status() == 0
    mode = routing_mode(shape, n_tok, prefill)
    y = out["y"].double().cpu().numpy() - x.double().numpy()
    flips, err = layer_same_input_check(
        lw, x.double().numpy(), mode, got_used=out["used_idx"].cpu().numpy(), got_used_w=out["used_w"].cpu().numpy(),
        route_in=(ridx.numpy().astype(np.int64), rw.numpy()), got_y=y, got_pred=out["pred_idx"].cpu().numpy(),
        got_pred_w=out["pred_w"].cpu().numpy(), rows=sample, what=f"{n_tok} tokens")
    say(f"  routing of all {n_tok} rows checked ({mode} bound), certified near ties {flips}; "
        f"sampled outputs max rel-L2 {err:.2e}")


def test_prefill_512_sampled():
    sample = [0, 1, 2, 77, 128, 255, 256, 300, 383, 449, 500, 511]
    sampled_layer_check(512, True, 21, sample)


@pytest.mark.timeout(600)
def test_prefill_8192_sampled():
    """A long prefill: 32768 assignments through the token->expert sort, about
    128 tokens per expert (several tiles each)."""
    sample = [0, 1, 1000, 2047, 2048, 4095, 4096, 5555, 8000, 8191]
    sampled_layer_check(8192, True, 23, sample)


def test_prefill_ragged_long_sampled():
    """A long prefill whose token count is not a multiple of 64: the 64 x 64
    routing tiles and the 64-token gate/up tiles both end in a partial tile."""
    sample = [0, 63, 64, 2500, 4095, 4096, 4132]
    sampled_layer_check(4133, True, 24, sample)


def test_prefill_f32_activations_sampled():
    """fp32 block input on the matrix-core path: u enters every MFMA as a bf16
    hi + lo pair (two products), both gate/up buffering modes."""
    shape = dataclasses.replace(synth.LAYER35B, name="layer_d2048_e256_k4_f32", act="f32")
    sampled_layer_check(300, True, 25, [0, 1, 150, 299], shape=shape)
    sampled_layer_check(37, True, 26, [0, 5, 36], shape=shape)


def test_prefill_one_hot_experts_sampled():
    """Degenerate routing: all 511 given rows use the same 4 experts (511
    assignments each: 32 tiles per expert, a down
    projection block spanning one expert's tiles), plus a single-token
    prefill."""
    sampled_layer_check(512, True, 27, [0, 1, 63, 64, 255, 511], same_experts=[3, 200, 77, 255])
    sampled_layer_check(1, True, 28, [0])


def test_decode_batch32_sampled():
    sample = [0, 1, 5, 13, 16, 22, 30, 31]
    sampled_layer_check(32, False, 22, sample)


def zipf_layers(shape, L_, tag, device="cpu"):
    with open(os.path.join(HERE, "golden", "zipf_calibration.json")) as fh:
        cal = json.load(fh)
    ws = []
    for l in range(L_):
        w = synth.layer_weights(shape, l, device=device, tag=tag)
        w["head_bias"] = synth.zipf_bias(shape.E, cal["zipf_s"], cal["tau"], (tag, l), device=device)
        w["hist_cur"] = synth.sticky_history(shape.E, cal["beta"], device=device)
        ws.append(w)
    return cal, ws


def test_batched_sticky_stack():
    """B = 32 sequences through a 2-layer stack whose heads carry the calibrated
    Zipf popularity bias and stickiness, every layer checked on its input."""
    shape = synth.LAYER35B
    L_, B, steps = 2, 32, 3
    cal, ws = zipf_layers(shape, L_, "zipfstack")
    say(f"batched sticky stack L={L_} B={B} steps={steps} tau={cal['tau']} beta={cal['beta']}")
    ora = [oracle_layer(shape, w) for w in ws]
    gpus = [gpu_layer(shape, w, fused=True, max_tokens=B, head=(l + 1 < L_)) for l, w in enumerate(ws)]
    import sparse_moe_decode_prerouter_amd as moe
    stack = moe.MoeStack(gpus)
    xs = np.stack([synth.activations(shape, B, ("zst", t), dtype=torch.float32).double().numpy() for t in range(steps)])
    from test_gpu_stack import check_steps, run_gpu
    g = run_gpu(stack, L_, xs, shape.k)
    for Lr in gpus:
        assert Lr.status() == 0
    flips, worst, e2e = check_steps(ora, g, routing_mode(shape, B, False), what="zipf B=32")
    reuse = [len(set(g[t]["pred"][1][b].tolist()) & set(g[t]["used"][1][b].tolist())) / shape.k
             for t in range(1, steps) for b in range(B)]
    say(f"  per-layer max rel-L2 {worst:.2e}, stack {e2e:.2e}, certified near ties {flips}; "
        f"mean next-token reuse of the predictions {np.mean(reuse):.3f}")


def test_batched_stack_presorted_bad_route_flagged():
    """At B = 32 (the general path) the given routing of layers >= 1 is sorted
    in one launch at the start of the step; a negative entry there is not
    self-routed but flagged on that layer (MOE_E_BAD_INDEX), the other layers
    stay clean. The routing comes from a host-side edit, so every kernel runs
    to its end."""
    import sparse_moe_decode_prerouter_amd as moe
    shape = synth.LAYER35B
    L_, B = 2, 32
    ws = [synth.layer_weights(shape, l, tag="badroute") for l in range(L_)]
    gpus = [gpu_layer(shape, w, fused=True, max_tokens=B, head=(l + 1 < L_)) for l, w in enumerate(ws)]
    stack = moe.MoeStack(gpus)
    say(f"presorted batched stack L={L_} B={B}: a negative routing entry of layer 1")
    x = synth.activations(shape, B, ("badroute",), dtype=torch.float32).cuda()
    xo = torch.empty_like(x)
    pidx = [torch.full((L_, B, shape.k), -1, dtype=torch.int32, device="cuda") for _ in range(2)]
    pw = [torch.zeros((L_, B, shape.k), dtype=torch.float32, device="cuda") for _ in range(2)]
    stack.decode(x, pidx[0], pw[0], pidx[1], pw[1], x_out=xo, first_step=True)
    torch.cuda.synchronize()
    assert [Lr.status() for Lr in gpus] == [0, 0]
    assert bool((pidx[1][1] >= 0).all())
    pidx[1][1, 5, 0] = -1
    stack.decode(x, pidx[1], pw[1], pidx[0], pw[0], x_out=xo, first_step=False)
    torch.cuda.synchronize()
    assert [Lr.status() for Lr in gpus] == [0, moe.MOE_E_BAD_INDEX]


class _BlobsOnDemand:
    """Host view of a device (or pinned) expert store for the oracle: blob e
    is copied on first use (a decode step touches only the experts it routes
    to)."""

    def __init__(self, store):
        self.dev = store
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = self.dev[e].cpu().numpy()
        return self.cache[e]


def _oracle_layer_dev(shape, w, has_head, store=None):
    """Oracle weights of a layer whose tensors live on the GPU (expert blobs
    copied on demand)."""
    st = w["store"] if store is None else store
    return oracle.LayerWeights(
        d=shape.d, E=shape.E, k=shape.k, f=shape.f, fs=shape.fs, r=shape.r, alpha=shape.alpha, eps=shape.eps,
        act=shape.act, store=_BlobsOnDemand(st.view(shape.E, shape.blob_bytes)),
        shared=w["shared"].cpu().numpy(), shared_gate=synth.bf16_bits(w["shared_gate"].cpu()),
        lora_a=synth.bf16_bits(w["lora_a"].cpu()), lora_b=synth.bf16_bits(w["lora_b"].cpu()),
        gamma=w["gamma"].double().cpu().numpy(),
        head=synth.bf16_bits(w["head"].cpu()) if has_head else None, router=synth.bf16_bits(w["router"].cpu()),
        head_bias=w["head_bias"].double().cpu().numpy() if (has_head and w.get("head_bias") is not None) else None,
        hist_cur=w["hist_cur"].double().cpu().numpy() if (has_head and w.get("hist_cur") is not None) else None)


def check_decode_stack(ora, g, mode, out_steps, rows=None, what=""):
    """Every routing decision of every step on its own input; block outputs
    and the stack output on out_steps (rows: sequences whose outputs are
    computed)."""
    from test_gpu_stack import check_steps
    return check_steps(ora, g, mode, steps_out=set(out_steps), rows=rows, what=what)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("one,steps", [(True, 128), (False, 16)], ids=["one_launch", "per_layer"])
def test_decode_stack_40_layers(one, steps):
    """The benchmarked configuration at full size: 40 layers of the 35B shape
    (16.9 GiB of int4 experts resident), batch 1, the stack decode the bench
    replays (one launch per step), for 128 steps; the per-layer launches for
    16. Every step's 40 routing decisions (layer 0's self-routing, 39 head
    predictions with their history) are checked on the input each layer saw;
    the block outputs of every layer and the output after 40 layers on a
    subset of steps."""
    import sparse_moe_decode_prerouter_amd as moe
    from test_gpu_stack import run_gpu
    shape = synth.LAYER35B
    L_, B = 40, 1
    say(f"40-layer decode stack B={B} steps={steps} one_launch={one}")
    ws = [synth.layer_weights(shape, l, device="cuda", tag="full40") for l in range(L_)]
    gpus = [gpu_layer(shape, w, fused=True, max_tokens=B, head=(l + 1 < L_)) for l, w in enumerate(ws)]
    ora = [_oracle_layer_dev(shape, w, l + 1 < L_) for l, w in enumerate(ws)]
    stack = moe.MoeStack(gpus)
    if one:
        stack.set_one_launch(True)
    xs = np.stack([synth.activations(shape, B, ("full40", t), dtype=torch.float32).double().numpy()
                   for t in range(steps)])
    g = run_gpu(stack, L_, xs, shape.k)
    for Lr in gpus:
        assert Lr.status() == 0
    say("  GPU steps done; checking")
    out_steps = [0, 1, 2, 63, 127] if steps == 128 else [0, 1, steps - 1]
    flips, worst, e2e = check_decode_stack(ora, g, "f64", out_steps=out_steps, what="40-layer")
    say(f"  {steps * L_} routing decisions checked, certified near ties {flips}; per-layer max rel-L2 {worst:.2e}; "
        f"after {L_} layers {e2e:.2e}")
    stack.close()
    for Lr in gpus:
        Lr.close()


@pytest.mark.timeout(600)
def test_streamed_stack_40_layers():
    """The configuration as the pages run it: 40 layers whose experts live in
    pinned host memory and are staged per step into a slab of 4 routed slots
    + the shared slot per layer, on a side stream, from the predictions of
    the step before (layer 0, and every layer at step 0, route themselves and
    stage inside the call). The staged set equals the routed set at every
    (layer, step); no call finds an expert missing; every routing decision
    and block output is checked on its input, and the output after 40
    layers. One pinned store of experts serves all 40 layers (each layer has
    its own router, head, adapter, norm and slab)."""
    import sparse_moe_decode_prerouter_amd as moe
    from test_gpu_stack import run_gpu
    shape = synth.LAYER35B
    L_, B, steps, k = 40, 1, 6, shape.k
    say(f"streamed 40-layer decode stack, slab of {k} + 1 slots, steps={steps}")
    ws = [synth.layer_weights(shape, l, device="cuda", tag="str40") for l in range(L_)]
    pstore = ws[0]["store"].cpu().pin_memory()
    pshared = ws[0]["shared"].cpu().pin_memory()
    gpus = []
    for l, w in enumerate(ws):
        w["store"] = pstore
        w["shared"] = pshared
        gpus.append(moe.MoeLayer(
            d_model=shape.d, n_experts=shape.E, top_k=k, d_ff=shape.f, d_ff_shared=shape.fs, lora_rank=shape.r,
            lora_alpha=shape.alpha, act_dtype=moe.MOE_ACT_BF16, max_tokens=B, expert_store=pstore,
            shared_blob=pshared, shared_gate=w["shared_gate"], router=w["router"],
            head=w["head"] if l + 1 < L_ else None, next_n_experts=shape.E if l + 1 < L_ else 0,
            next_top_k=k if l + 1 < L_ else 0, lora_a=w["lora_a"], lora_b=w["lora_b"], norm_gamma=w["gamma"],
            rms_eps=shape.eps, fuse_norm_residual=True, resident=False, slab_slots=k))
    ora = [_oracle_layer_dev(shape, w, l + 1 < L_, store=pstore) for l, w in enumerate(ws)]
    stack = moe.MoeStack(gpus)
    cs = torch.cuda.Stream()
    dev = "cuda"
    pidx = [torch.full((L_, B, k), -1, dtype=torch.int32, device=dev) for _ in range(2)]
    pw = [torch.zeros((L_, B, k), dtype=torch.float32, device=dev) for _ in range(2)]
    used_i = torch.empty((L_, B, k), dtype=torch.int32, device=dev)
    used_w = torch.empty((L_, B, k), dtype=torch.float32, device=dev)
    tr = torch.zeros((L_, B, shape.d), dtype=torch.float32, device=dev)
    xo = torch.empty((B, shape.d), dtype=torch.float32, device=dev)
    stack.set_trace(tr)
    g = []
    for t in range(steps):
        x = synth.activations(shape, B, ("str40", t), device=dev, dtype=torch.float32)
        ci, cw = pidx[t % 2].cpu().numpy().copy(), pw[t % 2].cpu().numpy().copy()
        if t > 0:
            for l in range(1, L_):
                gpus[l].stage(sorted(set(int(e) for e in ci[l, 0])), stream=cs)
                # staged set == routed set (k distinct experts into k slots)
                assert set(gpus[l].slots()[0]) == set(int(e) for e in ci[l, 0]), (t, l)
        stack.decode(x, pidx[t % 2], pw[t % 2], pidx[(t + 1) % 2], pw[(t + 1) % 2], x_out=xo, used_idx=used_i,
                     used_w=used_w, first_step=(t == 0))
        torch.cuda.synchronize()
        for l, Lr in enumerate(gpus):
            assert Lr.status() == 0, (t, l)
        u = used_i.cpu().numpy().copy()
        # layer 0 (and every layer at step 0) staged its own routing inside the call
        for l in ([0] if t > 0 else range(L_)):
            assert set(gpus[l].slots()[0]) == set(int(e) for e in u[l, 0]), (t, l)
        given = [None] + [None if t == 0 else (ci[l].astype(np.int64), cw[l]) for l in range(1, L_)]
        g.append(dict(x=x.double().cpu().numpy(), trace=tr.double().cpu().numpy(), x_out=xo.double().cpu().numpy(),
                      used=u, used_w=used_w.cpu().numpy().copy(), given=given, pred=pidx[(t + 1) % 2].cpu().numpy(),
                      pred_w=pw[(t + 1) % 2].cpu().numpy(), cur=None, prev=None))
    stack.set_trace(None)
    say("  GPU steps done; checking")
    # the history one-hots: the stack was given none (no hist_prev; cur = the routing passed in)
    for t in range(steps):
        g[t]["cur"] = [None if (t == 0 or l + 1 >= L_) else g[t]["given"][l + 1][0] for l in range(L_)]
    flips, worst, e2e = check_decode_stack(ora, g, "f64", out_steps=[0, 1, steps - 1], what="streamed")
    staged = sum(Lr.slots()[1] for Lr in gpus)
    say(f"  staged {staged / 1e6:.0f} MB over {steps} steps; certified near ties {flips}; per-layer max rel-L2 "
        f"{worst:.2e}; after {L_} layers {e2e:.2e}")
    stack.close()
    for Lr in gpus:
        Lr.close()


@pytest.mark.timeout(600)
def test_batched_stack_40_layers_b32():
    """Batched decode at full size: 32 independent sequences through the
    40-layer stack whose heads carry the Zipf popularity bias and stickiness.
    Every routing decision of all 32 sequences is checked on its input; the
    block outputs and the output after 40 layers for three sampled
    sequences."""
    import sparse_moe_decode_prerouter_amd as moe
    from test_gpu_stack import run_gpu
    shape = synth.LAYER35B
    L_, B, steps = 40, 32, 3
    cal, ws = zipf_layers(shape, L_, "zipf40", device="cuda")
    say(f"40-layer batched decode B={B} steps={steps}")
    gpus = [gpu_layer(shape, w, fused=True, max_tokens=B, head=(l + 1 < L_)) for l, w in enumerate(ws)]
    ora = [_oracle_layer_dev(shape, w, l + 1 < L_) for l, w in enumerate(ws)]
    stack = moe.MoeStack(gpus)
    xs = np.stack([synth.activations(shape, B, ("zipf40", t), dtype=torch.float32).double().numpy()
                   for t in range(steps)])
    g = run_gpu(stack, L_, xs, shape.k)
    for Lr in gpus:
        assert Lr.status() == 0
    say("  GPU steps done; checking")
    flips, worst, e2e = check_decode_stack(ora, g, routing_mode(shape, B, False), out_steps=[1, 2],
                                           rows=[0, 13, 31], what="batched 40-layer")
    say(f"  {steps * L_ * B} routing decisions checked, certified near ties {flips}; per-layer max rel-L2 "
        f"{worst:.2e}; after {L_} layers {e2e:.2e}")
    stack.close()
    for Lr in gpus:
        Lr.close()


@pytest.mark.timeout(600)
def test_stack_prefill_40_layers_sampled():
    """The benchmarked prefill at full size: 512 tokens through the 40-layer
    stack (layer l >= 1 routes token i by head l-1 on token i-1, token 0
    self-routes; layer 0 self-routes every token). Every routing decision of
    all 512 tokens at every layer is checked on the layer's input; the block
    outputs of sampled tokens at every layer and their outputs after 40
    layers."""
    import sparse_moe_decode_prerouter_amd as moe
    from stack_check import check_stack_layers, stack_output_check
    from test_gpu_stack import prefill_given
    shape = synth.LAYER35B
    L_, T, k = 40, 512, synth.LAYER35B.k
    sample = [0, 1, 77, 255, 256, 511]
    say(f"40-layer stack prefill T={T} sampled tokens {sample}")
    ws = [synth.layer_weights(shape, l, device="cuda", tag="pf40") for l in range(L_)]
    gpus = [gpu_layer(shape, w, fused=True, max_tokens=T, head=(l + 1 < L_)) for l, w in enumerate(ws)]
    stack = moe.MoeStack(gpus)
    x0 = synth.activations(shape, T, ("pf40",), dtype=torch.float32)
    xg = x0.cuda().contiguous()
    used_i = torch.empty((L_, T, k), dtype=torch.int32, device="cuda")
    used_w = torch.empty((L_, T, k), dtype=torch.float32, device="cuda")
    pred_i = torch.full((L_, T, k), -7, dtype=torch.int32, device="cuda")
    pred_w = torch.zeros((L_, T, k), dtype=torch.float32, device="cuda")
    tr = torch.zeros((L_, T, shape.d), dtype=torch.float32, device="cuda")
    stack.set_trace(tr)
    stack.prefill(xg, used_idx=used_i, used_w=used_w, pred_idx=pred_i, pred_w=pred_w)
    torch.cuda.synchronize()
    for Lr in gpus:
        assert Lr.status() == 0
    ui, uw = used_i.cpu().numpy(), used_w.cpu().numpy()
    pi, pw = pred_i.cpu().numpy(), pred_w.cpu().numpy()
    for l in range(1, L_):
        assert np.array_equal(ui[l][1:], pi[l][:-1]), l
        assert np.array_equal(uw[l][1:], pw[l][:-1]), l
    ora = [_oracle_layer_dev(shape, w, l + 1 < L_) for l, w in enumerate(ws)]
    say("  GPU done; checking")
    flips, worst = check_stack_layers(ora, tr.double().cpu().numpy(), xg.double().cpu().numpy(), ui, uw,
                                      prefill_given(ui, uw, L_), pi, pw, "mfma", rows=sample, what="prefill 40")
    e2e = stack_output_check(ora, x0.double().numpy(), xg.double().cpu().numpy(), ui, uw, STACK_TOL, rows=sample)
    say(f"  {L_ * T} rows' routing checked, certified near ties {flips}; sampled per-layer max rel-L2 {worst:.2e}; "
        f"after {L_} layers {e2e:.2e}")
    stack.close()
    for Lr in gpus:
        Lr.close()

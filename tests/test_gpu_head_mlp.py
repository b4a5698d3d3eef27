"""The pages' full prerouter head on the GPU: head(x) = l(x) + fc2(erf-GELU(
fc1(x))) on x = [u, top-k one-hot of the current token's routing, of the
previous token's] (l: the linear path with its bias and one-hot rows).
Every prediction is checked against the oracle's head on the same input,
bit-exact or a certified near tie within the computed bound (fc1 through
the routing GEMM, GELU's slope, fc2 in fp64). Paths: the fused decode
(B = 1, 4), the batched decode's general path (B = 32), prefill on the
matrix cores, the toy shape's general path, and the decode and prefill
stacks (whose heads take their history one-hots)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import gpu_layer, layer_same_input_check, layer_tensors, oracle_layer, routing_mode, say
from stack_check import check_stack_layers

pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

H1 = 256


def mlp_layer(shape, layer, tag, hidden=H1, history=False):
    w = layer_tensors(shape, layer=layer, tag=tag)
    w.update(synth.head_mlp_weights(shape, layer, hidden, tag=tag))
    if history:
        w["hist_cur"] = synth.sticky_history(shape.E, 0.3)
        w["hist_prev"] = synth.sticky_history(shape.E, 0.1)
    return w


def check_call(shape, n_tok, prefill, given, tag, hidden=H1):
    say(f"MLP head {shape.name} H1={hidden} n_tok={n_tok} prefill={prefill} given={given}")
    w = mlp_layer(shape, 2, tag, hidden, history=True)
    lw = oracle_layer(shape, w)
    x = synth.activations(shape, n_tok, (tag, n_tok), dtype=torch.float32)
    route = None
    if given:
        ri, rw = synth.random_routing(n_tok, shape.E, shape.k, (tag, "r", n_tok))
        ri[0] = -1
        route = (ri, rw)
    hc, _ = synth.random_routing(n_tok, shape.E, shape.k, (tag, "hc", n_tok))
    hp, _ = synth.random_routing(n_tok, shape.E, shape.k, (tag, "hp", n_tok))
    hp[0, 1] = hp[0, 0]               # a duplicate inside one history list
    hp[min(1, n_tok - 1), 0] = -1     # and an absent entry
    L = gpu_layer(shape, w, fused=True, max_tokens=n_tok)
    call = L.prefill if prefill else L.decode
    out = call(x.cuda(), None if route is None else route[0].cuda(), None if route is None else route[1].cuda(),
               hist_cur=hc.cuda(), hist_prev=hp.cuda())
    torch.cuda.synchronize()
    assert L.status() == 0
    mode = routing_mode(shape, n_tok, prefill)
    y = out["y"].double().cpu().numpy() - x.double().numpy()
    flips, err = layer_same_input_check(
        lw, x.double().numpy(), mode, got_used=out["used_idx"].cpu().numpy(), got_used_w=out["used_w"].cpu().numpy(),
        route_in=None if route is None else (route[0].numpy().astype(np.int64), route[1].numpy()), got_y=y,
        got_pred=out["pred_idx"].cpu().numpy(), got_pred_w=out["pred_w"].cpu().numpy(), cur=hc.numpy(),
        prev=hp.numpy(), rows=[0, n_tok - 1], what=f"mlp {n_tok}")
    # the branch matters: the linear path alone would pick other experts on most rows
    changed = 0
    for t in range(n_tok):
        u = oracle.block_input(lw, x.double().numpy()[t], True)
        zl = oracle.head_logits(lw.head, u, lw.head_bias, lw.hist_cur, hc.numpy()[t], lw.hist_prev, hp.numpy()[t])
        changed += list(oracle.topk(zl, shape.k)) != list(out["pred_idx"].cpu().numpy()[t])
    say(f"  predictions checked, certified near ties {flips}; rows whose top-k the MLP branch changes: "
        f"{changed}/{n_tok}; block rel-L2 {err:.1e}")
    assert changed > 0


@pytest.mark.parametrize("n_tok", [1, 4])
def test_mlp_head_fused_decode(n_tok):
    check_call(synth.LAYER35B, n_tok, False, given=False, tag="mlpd")


def test_mlp_head_batched_decode():
    check_call(synth.LAYER35B, 32, False, given=True, tag="mlpb")


@pytest.mark.parametrize("n_tok", [37, 300])
def test_mlp_head_prefill(n_tok):
    check_call(synth.LAYER35B, n_tok, True, given=True, tag="mlpp")


@pytest.mark.parametrize("prefill", [False, True])
def test_mlp_head_tiny(prefill):
    """The toy shape: fp32 activations (fc1 through the hi + lo GEMM), the
    general path's own head top-k launch after the branch."""
    check_call(synth.TINY, 6, prefill, given=False, tag="mlpt", hidden=32)


def test_mlp_head_stack_decode():
    """Decode stack with MLP heads and history rows: the deferred head top-k
    reads logits that already hold the branch; the one-hots are the next
    layer's routing at this step and the previous one."""
    import sparse_moe_decode_prerouter_amd as moe
    from test_gpu_stack import check_steps, run_gpu
    shape = synth.LAYER35B
    L_, B, steps = 3, 2, 4
    say(f"MLP-head decode stack L={L_} B={B} steps={steps}")
    ws = [mlp_layer(shape, l, "mlps", history=True) for l in range(L_)]
    ora = [oracle_layer(shape, w) for w in ws]
    for l in range(L_ - 1):
        assert ora[l].head_fc1 is not None
    gpus = [gpu_layer(shape, w, fused=True, max_tokens=B, head=(l + 1 < L_)) for l, w in enumerate(ws)]
    for l in range(L_):
        if l + 1 >= L_:
            ora[l].head = None
            ora[l].head_fc1 = None
    stack = moe.MoeStack(gpus)
    xs = np.stack([synth.activations(shape, B, ("mlps", t), dtype=torch.float32).double().numpy()
                   for t in range(steps)])
    g = run_gpu(stack, L_, xs, shape.k)
    for Lr in gpus:
        assert Lr.status() == 0
    flips, worst, e2e = check_steps(ora, g, "f64", what="mlp stack")
    say(f"  per-layer max rel-L2 {worst:.2e}, stack {e2e:.2e}, certified near ties {flips}")


def test_mlp_head_stack_prefill():
    import sparse_moe_decode_prerouter_amd as moe
    from test_gpu_stack import prefill_given
    shape = synth.LAYER35B
    L_, T = 3, 37
    say(f"MLP-head stack prefill L={L_} T={T}")
    ws = [mlp_layer(shape, l, "mlpsp") for l in range(L_)]
    ora = [oracle_layer(shape, w) for w in ws]
    ora[-1].head_fc1 = None
    gpus = [gpu_layer(shape, w, fused=True, max_tokens=T, head=(l + 1 < L_)) for l, w in enumerate(ws)]
    stack = moe.MoeStack(gpus)
    x0 = synth.activations(shape, T, ("mlpsp",), dtype=torch.float32)
    xg = x0.cuda().contiguous()
    k = shape.k
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
    ui, uw, pi, pw = (a.cpu().numpy() for a in (used_i, used_w, pred_i, pred_w))
    for l in range(1, L_):
        assert np.array_equal(ui[l][1:], pi[l][:-1]), l
    flips, worst = check_stack_layers(ora, tr.double().cpu().numpy(), xg.double().cpu().numpy(), ui, uw,
                                      prefill_given(ui, uw, L_), pi, pw, "mfma", what="mlp prefill stack")
    say(f"  per-layer max rel-L2 {worst:.2e}, certified near ties {flips}")

"""Exact logit ties through every top-k site of the library, with the ties
broken by the lowest expert index.

The router and head rows come in groups of identical rows (expert e copies
the row of group e mod G), with entries j / 128 for integers |j| <= 15, and
the block inputs stay away from zero (|x| >= 1/4, RMSNorm gain 1, so that
|u| >= 2^-3 or so). Every product and every partial sum is then exact in
fp32 and fp64, on the GPU and in the oracle, so the logits agree bit for
bit and tied groups tie exactly: the comparison allows no window, and the
only correct order is (logit descending, index ascending). The experts are
zero (W = 0 exactly), so the residual stream does not change along a stack
and every layer sees the same exact inputs.

Sites driven: the decode router (K_R) and the head's top-k in the decode
down-projection launch; in a stack, the deferred head top-k in the next
layer's gate/up launch and the final top-k launch; prefill's routing top-k
launch, the sort's own top-k of a self-routed row, the routing GEMM's
last-block top-k of the rows before the routing shift, the head top-k beside
the combine (and beside the combine that takes the next layer's norm); the
LDS-tiled routing GEMM of long prompts; the batched decode's general path;
the toy shape with fp32 activations.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import gpu_layer, layer_same_input_check, say
from stack_check import check_stack_layers

pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

TIE35 = dataclasses.replace(synth.LAYER35B, name="ties_d2048_e256_k4", fs=0, r=0)
TIETINY = dataclasses.replace(synth.TINY, name="ties_d256_e16_k2", fs=0, r=0)


def grouped_rows(E, d, group, key):
    """bf16 [E, d]: expert e copies base row e mod G (G = ceil(E / group)),
    entries j / 128 with j uniform in [-15, 15]."""
    G = -(-E // group)
    base = synth.uniform_int((G, d), -15, 16, ("ties", key) + (E, d, group)).float() / 128.0
    rows = base[torch.arange(E) % G]
    return rows.bfloat16()


def tie_weights(shape, group, key):
    d, E = shape.d, shape.E
    w = {
        "store": torch.zeros((E, shape.blob_bytes), dtype=torch.uint8),
        "shared": None, "shared_gate": None, "lora_a": None, "lora_b": None,
        "gamma": torch.ones(d),
        "router": grouped_rows(E, d, group, key + ("router",)),
        "head": grouped_rows(E, d, group, key + ("head",)),
        "head_bias": None, "hist_cur": None, "hist_prev": None,
    }
    return w


def tie_inputs(shape, n, key):
    """x with |x| in [1/4, 4]: u = x / rms stays away from zero."""
    x = synth.gaussian((n, shape.d), 1.0, ("tiex",) + key)
    x = torch.sign(x) * x.abs().clamp(0.25, 4.0)
    x[x == 0] = 0.25
    return x


def oracle_tie_layer(shape, w, with_head=True):
    b = synth.bf16_bits
    return oracle.LayerWeights(
        d=shape.d, E=shape.E, k=shape.k, f=shape.f, fs=0, r=0, alpha=shape.alpha, eps=shape.eps, act=shape.act,
        store=w["store"].numpy(), shared=None, shared_gate=None, lora_a=None, lora_b=None,
        gamma=w["gamma"].double().numpy(), head=b(w["head"]) if with_head else None, router=b(w["router"]))


def assert_ties_exercised(lw, x, fused, k):
    """At least one row ties inside its top-k and one ties across its k-th /
    (k+1)-th boundary (so the test really decides ties)."""
    inside = across = 0
    for t in range(min(x.shape[0], 64)):
        u = oracle.block_input(lw, x[t], fused)
        for H in (lw.router, lw.head):
            if H is None:
                continue
            z = oracle.head_logits(H, u)
            order = oracle.topk(z, k + 1)
            inside += any(z[order[i]] == z[order[i + 1]] for i in range(k - 1))
            across += z[order[k - 1]] == z[order[k]]
    assert inside > 0 and across > 0, (inside, across)


def layer_call(shape, group, n_tok, *, prefill, given, fused=True, key=("L",)):
    say(f"ties {shape.name} group={group} n_tok={n_tok} prefill={prefill} given={given} fused={fused}")
    w = tie_weights(shape, group, key)
    lw = oracle_tie_layer(shape, w)
    x = tie_inputs(shape, n_tok, key + (n_tok,))
    if not fused:
        x = x.bfloat16().float()           # u given directly: bf16-valued fp32 activations
    assert_ties_exercised(lw, x.double().numpy(), fused, shape.k)
    L = gpu_layer(shape, w, fused=fused, max_tokens=n_tok)
    route = None
    if given:
        ridx, rw = synth.random_routing(n_tok, shape.E, shape.k, ("ties",) + key)
        ridx[0] = -1
        route = (ridx, rw)
    call = L.prefill if prefill else L.decode
    out = call(x.cuda(), None if route is None else route[0].cuda(), None if route is None else route[1].cuda())
    torch.cuda.synchronize()
    assert L.status() == 0
    flips, _ = layer_same_input_check_unfused(lw, x.double().numpy(), fused, out, route)
    assert flips == 0
    L.close()


def layer_same_input_check_unfused(lw, x, fused, out, route):
    route_in = None if route is None else (route[0].numpy().astype(np.int64), route[1].numpy())
    if fused:
        return layer_same_input_check(lw, x, "exact", got_used=out["used_idx"].cpu().numpy(),
                                      got_used_w=out["used_w"].cpu().numpy(), route_in=route_in,
                                      got_pred=out["pred_idx"].cpu().numpy(), got_pred_w=out["pred_w"].cpu().numpy(),
                                      what="ties")
    # unfused: u = x; compare every self-routed row and every prediction directly
    used, pred = out["used_idx"].cpu().numpy(), out["pred_idx"].cpu().numpy()
    for t in range(x.shape[0]):
        u = oracle.block_input(lw, x[t], False)
        if route_in is None or route_in[0][t][0] < 0:
            assert list(used[t]) == list(oracle.topk(oracle.head_logits(lw.router, u), lw.k)), t
        assert list(pred[t]) == list(oracle.topk(oracle.head_logits(lw.head, u), lw.k)), t
    return 0, 0.0


@pytest.mark.parametrize("group", [3, 5])
@pytest.mark.parametrize("n_tok", [1, 4])
def test_ties_decode(group, n_tok):
    """Decode router (K_R) and the head top-k of the down-projection launch."""
    layer_call(TIE35, group, n_tok, prefill=False, given=False, key=("dec", group))


def test_ties_decode_batch32():
    """Batched decode on the general path: routing GEMM + routing top-k
    launch for the self-routed rows, head top-k beside the combine."""
    layer_call(TIE35, 3, 32, prefill=False, given=False, key=("b32",))


@pytest.mark.parametrize("given", [False, True])
def test_ties_prefill_512(given):
    """Every row self-routed (routing top-k launch), or only row 0 (the
    sort's own top-k); the head's top-k beside the combine."""
    layer_call(TIE35, 3, 512, prefill=True, given=given, key=("pf", given))


def test_ties_prefill_long():
    """A long prompt: the LDS-tiled routing GEMM."""
    layer_call(TIE35, 5, 4096, prefill=True, given=False, key=("long",))


@pytest.mark.parametrize("prefill", [False, True])
def test_ties_tiny_fp32(prefill):
    """The toy shape (E = 16, top-2) with fp32 activations given directly."""
    layer_call(TIETINY, 3, 6, prefill=prefill, given=False, fused=False, key=("tiny", prefill))


def tie_stack(shape, L_, group, max_tokens, key):
    import sparse_moe_decode_prerouter_amd as moe
    ws = [tie_weights(shape, group, key + (l,)) for l in range(L_)]
    ora = [oracle_tie_layer(shape, w, with_head=l + 1 < L_) for l, w in enumerate(ws)]
    gpus = [gpu_layer(shape, w, fused=True, max_tokens=max_tokens, head=(l + 1 < L_)) for l, w in enumerate(ws)]
    return ora, gpus, moe.MoeStack(gpus)


@pytest.mark.parametrize("one", [False, True], ids=["per_layer", "one_launch"])
@pytest.mark.parametrize("B", [1, 3])
def test_ties_stack_decode(B, one):
    """Stack decode: layer 0's router every step, the deferred head top-k in
    the next layer's gate/up launch, the final top-k launch; or, as one launch
    per step, the router beside the argument patch and every head's top-k in
    its layer's top-k work item of the step kernel."""
    from test_gpu_stack import run_gpu, one_launch_ran
    shape = TIE35
    L_, steps = 4, 3
    say(f"ties stack decode L={L_} B={B} steps={steps} one_launch={one}")
    ora, gpus, stack = tie_stack(shape, L_, 3, B, ("sd", B))
    if one:
        stack.set_one_launch(True)
    xs = np.stack([tie_inputs(shape, B, ("sd", B, t)).double().numpy() for t in range(steps)])
    assert_ties_exercised(ora[0], xs[0], True, shape.k)
    g = run_gpu(stack, L_, xs, shape.k)
    for Lr in gpus:
        assert Lr.status() == 0
    for t, s in enumerate(g):
        f, _ = check_stack_layers(ora, s["trace"], s["x_out"], s["used"], s["used_w"], s["given"], s["pred"],
                                  s["pred_w"], "exact", outputs=False, what=f"ties step {t}")
        assert f == 0
    if one:
        assert one_launch_ran(stack, L_, B, shape)


@pytest.mark.parametrize("T", [37, 150])
def test_ties_stack_prefill(T):
    """Stack prefill: layer 0's routing top-k launch; row 0 of later layers
    in the routing GEMM's last block; the head top-k beside the combine that
    takes the next norm (37 tokens) or the plain combine (150)."""
    shape = TIE35
    L_ = 3
    say(f"ties stack prefill L={L_} T={T}")
    ora, gpus, stack = tie_stack(shape, L_, 3, T, ("sp", T))
    x0 = tie_inputs(shape, T, ("sp", T))
    assert_ties_exercised(ora[0], x0.double().numpy(), True, shape.k)
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
    from test_gpu_stack import prefill_given
    ui, uw, pi, pw = (a.cpu().numpy() for a in (used_i, used_w, pred_i, pred_w))
    for l in range(1, L_):
        assert np.array_equal(ui[l][1:], pi[l][:-1]), l
    f, _ = check_stack_layers(ora, tr.double().cpu().numpy(), xg.double().cpu().numpy(), ui, uw,
                              prefill_given(ui, uw, L_), pi, pw, "exact", outputs=False, what=f"ties prefill {T}")
    assert f == 0

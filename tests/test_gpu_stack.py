"""GPU parity of the stacked calls (moe_stack_decode, moe_stack_prefill)
against the fp64 oracle's one-token-ahead dataflow: layer 0 self-routes,
head l at step t routes layer l+1 at step t+1, RMSNorm -> MoE block ->
residual per layer.

The stack records each layer's input residual stream (its trace), so every
layer is checked on the input it saw: each routing decision (self-routed
rows, head predictions with their history one-hots) bit-exact against the
oracle's logits on that input, or a certified near tie within the computed
error bound; each block output within rel-L2 2e-3. The stack output is
compared with the oracle's stack on the same routing within rel-L2 1e-2.
Two ways of driving it:
  forced - the oracle's free run gives the routing both sides take;
  free   - the GPU follows its own predictions (the realistic dataflow).
Each runs per layer (two launches a layer) and as one launch per step
(moe_stack_set_one_launch), whose steps after the first run every layer's
K_A and K_B as work items of a single kernel.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import gpu_layer, layer_tensors, oracle_layer, rel_l2_rows, say
from stack_check import check_stack_layers, stack_output_check

pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

STACK_TOL = 1e-2


def build(shape, L, tag, max_tokens=8, one=False):
    ws = [layer_tensors(shape, layer=l, tag=tag) for l in range(L)]
    ora = [oracle_layer(shape, w) for w in ws]
    gpus = [gpu_layer(shape, w, fused=True, max_tokens=max_tokens, head=(l + 1 < L)) for l, w in enumerate(ws)]
    import sparse_moe_decode_prerouter_amd as moe
    stack = moe.MoeStack(gpus)
    if one:
        stack.set_one_launch(True)
    return ora, gpus, stack


def run_gpu(stack, L, xs, k, forced_routes=None, trace=True):
    """xs: [steps, B, d] fp32. forced_routes[t][l] = (idx [B,k], w [B,k]) or
    None. Returns per step: x (input), trace [L, B, d], x_out, used, used_w,
    given (per layer: routing handed to it or None), pred, pred_w, cur, prev
    (history one-hots of each head)."""
    steps, B, d = xs.shape
    dev = "cuda"
    pidx = [torch.full((L, B, k), -1, dtype=torch.int32, device=dev) for _ in range(2)]
    pw = [torch.zeros((L, B, k), dtype=torch.float32, device=dev) for _ in range(2)]
    used_i = torch.empty((L, B, k), dtype=torch.int32, device=dev)
    used_w = torch.empty((L, B, k), dtype=torch.float32, device=dev)
    prev_used = torch.full((L, B, k), -1, dtype=torch.int32, device=dev)
    tr = torch.zeros((L, B, d), dtype=torch.float32, device=dev) if trace else None
    stack.set_trace(tr)
    xo = torch.empty((B, d), dtype=torch.float32, device=dev)
    out = []
    for t in range(steps):
        x = torch.from_numpy(xs[t]).float().to(dev).contiguous()
        cur_i, cur_w = pidx[t % 2], pw[t % 2]
        nxt_i, nxt_w = pidx[(t + 1) % 2], pw[(t + 1) % 2]
        if forced_routes is not None and t > 0:
            for l in range(1, L):
                fi, fw = forced_routes[t][l]
                cur_i[l] = torch.from_numpy(fi.astype(np.int32)).to(dev)
                cur_w[l] = torch.from_numpy(fw.astype(np.float32)).to(dev)
        ci, cw = cur_i.cpu().numpy().copy(), cur_w.cpu().numpy().copy()
        pu = prev_used.cpu().numpy().copy()
        stack.decode(x, cur_i, cur_w, nxt_i, nxt_w, x_out=xo, used_idx=used_i, used_w=used_w,
                     hist_prev=prev_used if t > 0 else None, first_step=(t == 0))
        torch.cuda.synchronize()
        given = [None] + [None if t == 0 else (ci[l].astype(np.int64), cw[l]) for l in range(1, L)]
        cur = [None if (t == 0 or l + 1 >= L) else ci[l + 1] for l in range(L)]
        prev = [None if (t == 0 or l + 1 >= L) else pu[l + 1] for l in range(L)]
        out.append(dict(x=x.double().cpu().numpy(), trace=None if tr is None else tr.double().cpu().numpy(),
                        x_out=xo.double().cpu().numpy(), used=used_i.cpu().numpy().copy(),
                        used_w=used_w.cpu().numpy().copy(), given=given, pred=nxt_i.cpu().numpy().copy(),
                        pred_w=nxt_w.cpu().numpy().copy(), cur=cur, prev=prev))
        prev_used.copy_(used_i)
    stack.set_trace(None)
    return out


def check_steps(ora, g, mode, steps_out=None, rows=None, what=""):
    """Per-layer checks of every step; outputs on steps_out (all when None)."""
    flips, worst, e2e = 0, 0.0, 0.0
    for t, s in enumerate(g):
        if t % 16 == 15:
            say(f"  {what}: checked {t} steps")
        outputs = steps_out is None or t in steps_out
        assert np.array_equal(s["trace"][0], s["x"]), t          # the trace starts at the step input
        f, e = check_stack_layers(ora, s["trace"], s["x_out"], s["used"], s["used_w"], s["given"], s["pred"],
                                  s["pred_w"], mode, cur=s["cur"], prev=s["prev"], rows=rows, outputs=outputs,
                                  what=f"{what} step {t}")
        flips += f
        worst = max(worst, e)
        if outputs:
            e2e = max(e2e, stack_output_check(ora, s["x"], s["x_out"], s["used"], s["used_w"], STACK_TOL, rows))
    return flips, worst, e2e


@pytest.mark.parametrize("one", [False, True], ids=["per_layer", "one_launch"])
@pytest.mark.parametrize("B", [1, 3])
def test_stack_forced_routing(B, one):
    shape = synth.LAYER35B
    L, steps = 4, 4
    say(f"stack forced L={L} B={B} steps={steps} one_launch={one}")
    ora, gpus, stack = build(shape, L, f"stackF{B}", one=one)
    xs = np.stack([synth.activations(shape, B, ("stk", B, t), dtype=torch.float32).double().numpy()
                   for t in range(steps)])
    recs = oracle.stack_decode(ora, xs, steps)
    forced = [None] + [[None] + [recs[t - 1].preds[l - 1] for l in range(1, L)] for t in range(1, steps)]
    g = run_gpu(stack, L, xs, shape.k, forced_routes=forced)
    for L_ in gpus:
        assert L_.status() == 0
    flips, worst, e2e = check_steps(ora, g, "f64", what=f"forced B={B}")
    # the oracle's free run took the same routing: its outputs agree too
    for t in range(steps):
        if all(np.array_equal(g[t]["used"][l], recs[t].routes[l][0]) for l in range(L)):
            assert rel_l2_rows(g[t]["x_out"], recs[t].x_out) <= STACK_TOL
    say(f"  per-layer max rel-L2 {worst:.2e}, stack {e2e:.2e}, certified near ties {flips}")


@pytest.mark.parametrize("one", [False, True], ids=["per_layer", "one_launch"])
def test_stack_free_running(one):
    shape = synth.LAYER35B
    L, steps, B = 4, 6, 2
    say(f"stack free-running L={L} B={B} steps={steps} one_launch={one}")
    ora, gpus, stack = build(shape, L, "stackR", one=one)
    xs = np.stack([synth.activations(shape, B, ("stkR", t), dtype=torch.float32).double().numpy()
                   for t in range(steps)])
    g = run_gpu(stack, L, xs, shape.k)
    for L_ in gpus:
        assert L_.status() == 0
    flips, worst, e2e = check_steps(ora, g, "f64", what="free")
    # the prediction of step t is the routing of step t + 1
    for t in range(1, steps):
        for l in range(1, L):
            assert np.array_equal(g[t]["used"][l], g[t - 1]["pred"][l])
    say(f"  per-layer max rel-L2 {worst:.2e}, stack {e2e:.2e}, certified near ties {flips}")


@pytest.mark.parametrize("one", [False, True], ids=["per_layer", "one_launch"])
def test_stack_tiny_shape_free_running(one):
    """The fp32-activation toy shape through a 3-layer stack."""
    shape = synth.TINY
    L, steps, B = 3, 4, 2
    say(f"tiny stack free-running L={L} B={B} steps={steps} one_launch={one}")
    ora, gpus, stack = build(shape, L, "stackT", one=one)
    xs = np.stack([synth.activations(shape, B, ("stkT", t), dtype=torch.float32).double().numpy()
                   for t in range(steps)])
    g = run_gpu(stack, L, xs, shape.k)
    for L_ in gpus:
        assert L_.status() == 0
    flips, worst, e2e = check_steps(ora, g, "f64", what="tiny")
    say(f"  per-layer max rel-L2 {worst:.2e}, stack {e2e:.2e}, certified near ties {flips}")


@pytest.mark.parametrize("B", [8, 16])
def test_stack_one_launch_largest_batches(B):
    """The one-launch step at the largest batches it takes (n_tok * k up to 64
    assignments at k = 4), free-running, every layer checked on its input."""
    shape = synth.LAYER35B
    L, steps = 3, 3
    say(f"stack one-launch L={L} B={B} steps={steps}")
    ora, gpus, stack = build(shape, L, f"stackOB{B}", max_tokens=B, one=True)
    xs = np.stack([synth.activations(shape, B, ("stkOB", B, t), dtype=torch.float32).double().numpy()
                   for t in range(steps)])
    g = run_gpu(stack, L, xs, shape.k)
    for L_ in gpus:
        assert L_.status() == 0
    flips, worst, e2e = check_steps(ora, g, "f64", what=f"one-launch B={B}")
    say(f"  per-layer max rel-L2 {worst:.2e}, stack {e2e:.2e}, certified near ties {flips}")
    assert one_launch_ran(stack, L, B, shape), "the step did not take the one-launch path"


def one_launch_ran(stack, L, B, shape):
    """Two more steps with kernel timestamps on: the second (not a first step)
    must have launched the step kernel."""
    dev = "cuda"
    k = shape.k
    pidx = [torch.full((L, B, k), -1, dtype=torch.int32, device=dev) for _ in range(2)]
    pw = [torch.zeros((L, B, k), dtype=torch.float32, device=dev) for _ in range(2)]
    x = synth.activations(shape, B, ("stkOBx",), dtype=torch.float32).to(dev).contiguous()
    xo = torch.empty_like(x)
    stack.set_profiling(True)
    stack.decode(x, pidx[0], pw[0], pidx[1], pw[1], x_out=xo, first_step=True)
    stack.decode(x, pidx[1], pw[1], pidx[0], pw[0], x_out=xo)
    torch.cuda.synchronize()
    _, ms = stack.kernel_ms()
    stack.set_profiling(False)
    return ms > 0


def test_one_launch_wait_timeout_reported():
    """The one-launch step's bounded waits, forced to run out from the host
    (a bound of one poll): the launch still ends, a layer reports
    MOE_E_TIMEOUT, and with the default bound the next steps are correct
    again (the counters were reset by the launch that timed out)."""
    import sparse_moe_decode_prerouter_amd as moe
    shape = synth.TINY
    L, B = 3, 2
    ora, gpus, stack = build(shape, L, "stackTO", one=True)
    xs = np.stack([synth.activations(shape, B, ("stkTO", t), dtype=torch.float32).double().numpy()
                   for t in range(4)])
    timeouts = 0
    for attempt in range(3):
        stack.set_wait_limit(1)
        run_gpu(stack, L, xs[:2], shape.k, trace=False)
        st = [Lr.status() for Lr in gpus]
        assert all(c in (moe.MOE_OK, moe.MOE_E_TIMEOUT) for c in st), st
        timeouts += sum(c == moe.MOE_E_TIMEOUT for c in st)
        if timeouts:
            break
    say(f"  layers reporting a timeout: {timeouts}")
    assert timeouts > 0
    stack.set_wait_limit(0)
    g = run_gpu(stack, L, xs, shape.k)
    for Lr in gpus:
        assert Lr.status() == 0
    flips, worst, e2e = check_steps(ora, g, "f64", what="after timeout")
    say(f"  per-layer max rel-L2 {worst:.2e}, stack {e2e:.2e}, certified near ties {flips}")


def run_stack_prefill(shape, L_, T, tag, pred_buffers=True):
    ws = [layer_tensors(shape, layer=l, tag=tag) for l in range(L_)]
    ora = [oracle_layer(shape, w) for w in ws]
    gpus = [gpu_layer(shape, w, fused=True, max_tokens=T, head=(l + 1 < L_)) for l, w in enumerate(ws)]
    import sparse_moe_decode_prerouter_amd as moe
    stack = moe.MoeStack(gpus)
    x0 = synth.activations(shape, T, (tag,), dtype=torch.float32)
    xg = x0.cuda().contiguous()
    k = shape.k
    used_i = torch.empty((L_, T, k), dtype=torch.int32, device="cuda")
    used_w = torch.empty((L_, T, k), dtype=torch.float32, device="cuda")
    pred_i = torch.full((L_, T, k), -7, dtype=torch.int32, device="cuda") if pred_buffers else None
    pred_w = torch.zeros((L_, T, k), dtype=torch.float32, device="cuda") if pred_buffers else None
    tr = torch.zeros((L_, T, shape.d), dtype=torch.float32, device="cuda")
    stack.set_trace(tr)
    stack.prefill(xg, used_idx=used_i, used_w=used_w, pred_idx=pred_i, pred_w=pred_w)
    torch.cuda.synchronize()
    for Lr in gpus:
        assert Lr.status() == 0
    res = dict(ora=ora, x=x0.double().numpy(), x_out=xg.double().cpu().numpy(), trace=tr.double().cpu().numpy(),
               used=used_i.cpu().numpy(), used_w=used_w.cpu().numpy(),
               pred=None if pred_i is None else pred_i.cpu().numpy(),
               pred_w=None if pred_w is None else pred_w.cpu().numpy())
    stack.close()
    for Lr in gpus:
        Lr.close()
    return res


def prefill_given(used, used_w, L_):
    """Routing each layer of a stack prefill was handed: layer 0 none (every
    row self-routes); layer l >= 1 the used routing with row 0 marked
    self-routed (the shifted predictions are checked separately)."""
    given = [None]
    for l in range(1, L_):
        gi = used[l].astype(np.int64).copy()
        gi[0] = -1
        given.append((gi, used_w[l]))
    return given


@pytest.mark.parametrize("T", [37, 150])
def test_stack_prefill(T):
    """moe_stack_prefill through 3 layers (the grouped-GEMM path): layer 0
    self-routes every token; layer l >= 1 routes token i by head l-1 on token
    i-1 (shifted inside the call) and token 0 self-routes. At 37 tokens each
    combine also takes the next layer's RMSNorm prologue; at 150 the layers
    run their own."""
    shape = synth.LAYER35B
    L_ = 3
    say(f"stack prefill L={L_} T={T}")
    r = run_stack_prefill(shape, L_, T, f"spf{T}")
    for l in range(1, L_):
        # token i of layer l took head l-1's prediction on token i-1
        assert np.array_equal(r["used"][l][1:], r["pred"][l][:-1]), l
        assert np.array_equal(r["used_w"][l][1:], r["pred_w"][l][:-1]), l
    given = prefill_given(r["used"], r["used_w"], L_)
    flips, worst = check_stack_layers(r["ora"], r["trace"], r["x_out"], r["used"], r["used_w"], given, r["pred"],
                                      r["pred_w"], "mfma", what=f"prefill T={T}")
    e2e = stack_output_check(r["ora"], r["x"], r["x_out"], r["used"], r["used_w"], STACK_TOL)
    say(f"  per-layer max rel-L2 {worst:.2e}, stack {e2e:.2e}, certified near ties {flips}")


@pytest.mark.parametrize("tiny", [False, True])
def test_stack_prefill_without_prediction_buffers(tiny):
    """Without caller prediction buffers the predictions pass through the
    stack's two scratch buffers (layer l writes one while it reads layer
    l-1's from the other). The result must equal the run with caller
    buffers, on the matrix-core path and on the general path of the toy
    shape (whose routing launch also takes the head's top-k)."""
    shape = synth.TINY if tiny else synth.LAYER35B
    L_, T = 3, 40
    say(f"stack prefill without prediction buffers, {shape.name}, T={T}")
    a = run_stack_prefill(shape, L_, T, "spfnb", pred_buffers=True)
    b = run_stack_prefill(shape, L_, T, "spfnb", pred_buffers=False)
    assert np.array_equal(a["used"], b["used"])
    assert np.array_equal(a["used_w"], b["used_w"])
    assert np.array_equal(a["x_out"], b["x_out"])
    for l in range(1, L_):
        assert np.array_equal(a["used"][l][1:], a["pred"][l][:-1]), l

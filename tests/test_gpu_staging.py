"""Device-initiated staging: the routing on the device drives a plan kernel
(the sticky-slot plan on the GPU slot table) and a copy kernel that pulls
the changed blobs from the mapped pinned store, with no host read-back.

Checked: the slot table after each staging equals the oracle's sticky plan
(staged set == routed set, resident experts keep their slots, only missing
experts are copied, counted in bytes); a call that routes itself stages on
the device inside the call; the two slab buffers of a double-slab layer are
independent; more experts than slots raises NOT_STAGED; the decode and
prefill outputs through staged slabs match the oracle; the stack's
one-token-ahead staging (prerouted: layer l's experts for step t+1 copied
on a side stream during step t) and its on-demand mode at full size."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import gpu_layer, layer_same_input_check, layer_tensors, oracle_layer, routing_mode, say

pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def staged_layer(shape, tag, slots, double=False, max_tokens=4, layer=1):
    w = layer_tensors(shape, layer=layer, tag=tag)
    pinned = (w["store"].contiguous().pin_memory(), w["shared"].contiguous().pin_memory())
    L = gpu_layer(shape, w, fused=True, resident=False, slab_slots=slots, max_tokens=max_tokens, device_staging=True,
                  double_slab=double, pinned=pinned)
    return w, L


def test_device_plan_matches_sticky_plan():
    """Five stagings of one single-slab layer (6 slots) with overlapping
    wanted sets: after each, the slot table equals oracle.plan_slots applied
    to the previous one, and the bytes counter grew by the copies' blobs
    (plus the shared blob once)."""
    shape = synth.LAYER35B
    say("device staging plan vs the sticky-slot plan")
    w, L = staged_layer(shape, "plan", slots=6)
    resident = [-1] * 6
    total = 0
    sets = [[5, 9, 3, 3], [9, 11, 5], [200, 3, 9, 17, 11, 5], [], [1, 2, 3, 4, 5, 6]]
    for i, want in enumerate(sets):
        ids = torch.tensor(want if want else [-1], dtype=torch.int32, device="cuda")
        L.stage_device(ids)
        torch.cuda.synchronize()
        new, copies = oracle.plan_slots(resident, want)
        slots, nbytes = L.slots()
        assert slots == new, (i, slots, new)
        total += len(copies) * shape.blob_bytes + (shape.shared_blob_bytes if i == 0 else 0)
        assert nbytes == total, (i, nbytes, total)
        resident = new
    assert L.status() == 0
    # more distinct experts than slots: nothing staged, the flag is raised
    L.stage_device(torch.arange(7, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    import sparse_moe_decode_prerouter_amd as moe
    assert L.status() == moe.MOE_E_NOT_STAGED
    assert L.slots()[0] == resident


@pytest.mark.parametrize("n_tok", [1, 4])
def test_device_staged_decode(n_tok):
    """Given routing staged on the device, then a self-routing call that
    stages inside itself (no host read-back); both against the oracle."""
    shape = synth.LAYER35B
    say(f"device-staged decode n_tok={n_tok}")
    w, L = staged_layer(shape, "sdec", slots=4 * n_tok, max_tokens=n_tok)
    lw = oracle_layer(shape, w)
    x = synth.activations(shape, n_tok, ("sdec", n_tok), dtype=torch.float32)
    ri, rw = synth.random_routing(n_tok, shape.E, shape.k, ("sdec", n_tok))
    L.stage_device(ri.flatten().cuda())
    out = L.decode(x.cuda(), ri.cuda(), rw.cuda())
    torch.cuda.synchronize()
    assert L.status() == 0
    assert set(L.slots()[0]) - {-1} == set(ri.flatten().tolist())
    y = out["y"].double().cpu().numpy() - x.double().numpy()
    mode = routing_mode(shape, n_tok, False)
    layer_same_input_check(lw, x.double().numpy(), mode, got_used=out["used_idx"].cpu().numpy(),
                           got_used_w=out["used_w"].cpu().numpy(), route_in=(ri.numpy().astype(np.int64), rw.numpy()),
                           got_y=y, got_pred=out["pred_idx"].cpu().numpy(), got_pred_w=out["pred_w"].cpu().numpy(),
                           what="given")
    out = L.decode(x.cuda())                       # routes itself, stages on the device
    torch.cuda.synchronize()
    assert L.status() == 0
    used = out["used_idx"].cpu().numpy()
    assert set(L.slots()[0]) - {-1} == set(used.flatten().tolist())
    y = out["y"].double().cpu().numpy() - x.double().numpy()
    layer_same_input_check(lw, x.double().numpy(), mode, got_used=used, got_used_w=out["used_w"].cpu().numpy(),
                           route_in=None, got_y=y, got_pred=out["pred_idx"].cpu().numpy(),
                           got_pred_w=out["pred_w"].cpu().numpy(), what="self")


def test_double_slab_buffers_independent():
    """Buffer 1 staged while calls read buffer 0: each call sees its own
    buffer's experts."""
    shape = synth.LAYER35B
    say("double slab: two independent buffers")
    w, L = staged_layer(shape, "dbl", slots=4, double=True, max_tokens=1)
    lw = oracle_layer(shape, w)
    x = synth.activations(shape, 1, ("dbl",), dtype=torch.float32)
    r0 = (torch.tensor([[1, 7, 33, 250]], dtype=torch.int32), torch.full((1, 4), 0.25))
    r1 = (torch.tensor([[2, 7, 90, 128]], dtype=torch.int32), torch.tensor([[0.4, 0.3, 0.2, 0.1]]))
    L.stage_device(r0[0].flatten().cuda(), buffer=0)
    L.stage_device(r1[0].flatten().cuda(), buffer=1)
    for b, r in ((0, r0), (1, r1), (0, r0)):
        L.use_buffer(b)
        out = L.decode(x.cuda(), r[0].cuda(), r[1].cuda())
        torch.cuda.synchronize()
        assert L.status() == 0
        assert set(L.slots()[0]) == set(r[0].flatten().tolist())
        y = out["y"].double().cpu().numpy() - x.double().numpy()
        layer_same_input_check(lw, x.double().numpy(), "f64", got_used=out["used_idx"].cpu().numpy(),
                               got_used_w=out["used_w"].cpu().numpy(),
                               route_in=(r[0].numpy().astype(np.int64), r[1].numpy()), got_y=y, what=f"buffer {b}")
    # routing to an expert the current buffer does not hold: flagged
    L.use_buffer(1)
    L.decode(x.cuda(), r0[0].cuda(), r0[1].cuda())
    import sparse_moe_decode_prerouter_amd as moe
    assert L.status() == moe.MOE_E_NOT_STAGED


def test_device_staged_cold_prefill():
    """A cold prefill: the layer's slab (all 256 experts + shared) starts
    empty and the call stages every expert its 200 tokens route to, on the
    device, between the sort and the grouped GEMMs."""
    shape = synth.LAYER35B
    T = 200
    say(f"cold prefill with device staging, T={T}")
    w, L = staged_layer(shape, "cold", slots=shape.E, max_tokens=T)
    lw = oracle_layer(shape, w)
    x = synth.activations(shape, T, ("cold",), dtype=torch.float32)
    ri, rw = synth.random_routing(T, shape.E, shape.k, ("cold",))
    ri[0] = -1
    out = L.prefill(x.cuda(), ri.cuda(), rw.cuda())
    torch.cuda.synchronize()
    assert L.status() == 0
    used = out["used_idx"].cpu().numpy()
    slots, nbytes = L.slots()
    assert set(slots) - {-1} == set(used.flatten().tolist())
    assert nbytes == len(set(used.flatten().tolist())) * shape.blob_bytes + shape.shared_blob_bytes
    y = out["y"].double().cpu().numpy() - x.double().numpy()
    layer_same_input_check(lw, x.double().numpy(), "mfma", got_used=used, got_used_w=out["used_w"].cpu().numpy(),
                           route_in=(ri.numpy().astype(np.int64), rw.numpy()), got_y=y,
                           got_pred=out["pred_idx"].cpu().numpy(), got_pred_w=out["pred_w"].cpu().numpy(),
                           rows=[0, 1, 99, 199], what="cold prefill")


def run_staged_stack(shape, L_, B, steps, mode, double, tag, check_every=True):
    """A stack of device-staged streamed layers driven by moe_stack_decode
    with the stack's staging; every layer checked on its input; after each
    step, every slab buffer of every layer equals the oracle's sticky plan
    replayed over the stagings it received (the routing a self-routed call
    used; the next step's predicted routing, prerouted), so each holds the
    routed set (exactly, when the distinct experts fill the slots)."""
    import sparse_moe_decode_prerouter_amd as moe
    from test_gpu_stack import check_steps
    say(f"staged stack {shape.name} L={L_} B={B} steps={steps} mode={mode} double={double}")
    ws = [synth.layer_weights(shape, l, device="cuda", tag=tag) for l in range(L_)]
    pstore = ws[0]["store"].cpu().pin_memory()
    pshared = ws[0]["shared"].cpu().pin_memory()
    for w in ws:
        w["store"], w["shared"] = pstore, pshared
    k = shape.k
    gpus = [gpu_layer(shape, w, fused=True, resident=False, slab_slots=k * B, max_tokens=B, head=(l + 1 < L_),
                      device_staging=True, double_slab=double, pinned=(pstore, pshared)) for l, w in enumerate(ws)]
    from test_gpu_large import _oracle_layer_dev
    ora = [_oracle_layer_dev(shape, w, l + 1 < L_, store=pstore) for l, w in enumerate(ws)]
    stack = moe.MoeStack(gpus)
    cs = torch.cuda.Stream()
    stack.set_staging(mode, cs)
    dev = "cuda"
    pidx = [torch.full((L_, B, k), -1, dtype=torch.int32, device=dev) for _ in range(2)]
    pw = [torch.zeros((L_, B, k), dtype=torch.float32, device=dev) for _ in range(2)]
    used_i = torch.empty((L_, B, k), dtype=torch.int32, device=dev)
    used_w = torch.empty((L_, B, k), dtype=torch.float32, device=dev)
    tr = torch.zeros((L_, B, shape.d), dtype=torch.float32, device=dev)
    xo = torch.empty((B, shape.d), dtype=torch.float32, device=dev)
    stack.set_trace(tr)
    g = []
    nbuf = 2 if double else 1
    sim = [[[-1] * (k * B) for _ in range(nbuf)] for _ in range(L_)]    # the oracle's plan per buffer
    for t in range(steps):
        x = synth.activations(shape, B, (tag, t), device=dev, dtype=torch.float32)
        ci, cw = pidx[t % 2].cpu().numpy().copy(), pw[t % 2].cpu().numpy().copy()
        stack.decode(x, pidx[t % 2], pw[t % 2], pidx[(t + 1) % 2], pw[(t + 1) % 2], x_out=xo, used_idx=used_i,
                     used_w=used_w, first_step=(t == 0))
        torch.cuda.synchronize()
        cs.synchronize()
        for l, Lr in enumerate(gpus):
            assert Lr.status() == 0, (t, l)
        u = used_i.cpu().numpy().copy()
        nxt = pidx[(t + 1) % 2].cpu().numpy()
        cur = t % 2 if double else 0
        nb = (t + 1) % 2 if double else 0
        on_demand_ = mode == moe.MOE_STAGE_ON_DEMAND
        for l, Lr in enumerate(gpus):
            # layers that routed themselves staged their used experts inside the call
            if on_demand_ or l == 0 or t == 0:
                sim[l][cur] = oracle.plan_slots(sim[l][cur], u[l].flatten().tolist())[0]
            # prerouted layers then staged the next step's routing into the next buffer
            if mode == moe.MOE_STAGE_PREROUTED and l >= 1:
                sim[l][nb] = oracle.plan_slots(sim[l][nb], nxt[l].flatten().tolist())[0]
                assert set(nxt[l].flatten().tolist()) <= set(sim[l][nb])
            for b in range(nbuf):
                Lr.use_buffer(b)
                assert Lr.slots()[0] == sim[l][b], (t, l, b, Lr.slots()[0], sim[l][b])
        on_demand = mode == moe.MOE_STAGE_ON_DEMAND
        given = [None] + [None if (t == 0 or on_demand) else (ci[l].astype(np.int64), cw[l]) for l in range(1, L_)]
        g.append(dict(x=x.double().cpu().numpy(), trace=tr.double().cpu().numpy(), x_out=xo.double().cpu().numpy(),
                      used=u, used_w=used_w.cpu().numpy().copy(), given=given, pred=nxt.copy(),
                      pred_w=pw[(t + 1) % 2].cpu().numpy().copy(),
                      cur=[None if (t == 0 or on_demand or l + 1 >= L_) else ci[l + 1] for l in range(L_)],
                      prev=None))
    stack.set_trace(None)
    staged = sum(Lr.slots()[1] for Lr in gpus)
    flips, worst, e2e = check_steps(ora, g, routing_mode(shape, B, False),
                                    steps_out=None if check_every else {0, steps - 1}, what=f"staged {mode}")
    say(f"  staged {staged / 1e6:.0f} MB; per-layer max rel-L2 {worst:.2e}, stack {e2e:.2e}, certified near ties {flips}")
    stack.close()
    for Lr in gpus:
        Lr.close()


@pytest.mark.parametrize("double", [True, False])
def test_staged_stack_prerouted(double):
    import sparse_moe_decode_prerouter_amd as moe
    run_staged_stack(synth.LAYER35B, 4, 2, 5, moe.MOE_STAGE_PREROUTED, double, f"stgP{int(double)}")


def test_staged_stack_on_demand():
    import sparse_moe_decode_prerouter_amd as moe
    run_staged_stack(synth.LAYER35B, 4, 2, 4, moe.MOE_STAGE_ON_DEMAND, True, "stgD")


@pytest.mark.timeout(600)
def test_staged_stack_40_layers():
    """The pages' streamed configuration with device-initiated staging: 40
    layers, batch 1, 4 + 1 slots in each of two slab buffers, layer l's
    experts for step t+1 copied on a side stream during step t."""
    import sparse_moe_decode_prerouter_amd as moe
    run_staged_stack(synth.LAYER35B, 40, 1, 6, moe.MOE_STAGE_PREROUTED, True, "stg40", check_every=False)

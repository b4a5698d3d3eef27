"""GPU parity of one MoE layer call through the C ABI against the fp64 oracle.

Shapes: the single-layer toy workload (d=256, E=16, top-2, fp32 activations)
and the 35B-tier layer (d=2048, E=256, top-4, bf16 activations), decode at
batch 1 and 4, resident and streamed (pinned host store -> HBM slab), plus a
ragged prefill. Routing indices must match exactly (ties: lowest index);
block outputs within max rel-L2 2e-3 per token.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import gpu_layer, layer_tensors, oracle_layer, rel_l2_rows, say

pytestmark = pytest.mark.gpu
TOL = 2e-3

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def run_oracle(lw, x, route, fused, pred=True):
    return oracle.decode_layer(lw, x, route, lw.k if pred else None, fused_norm=fused)


def check_layer(shape, n_tok, *, fused, given_route, resident=True, seed=0, prefill=False, gate_fixed=False):
    say(f"{shape.name} n_tok={n_tok} fused={fused} given_route={given_route} resident={resident} prefill={prefill}"
        f" gate_fixed={gate_fixed}")
    w = layer_tensors(shape, layer=seed)
    if gate_fixed:
        w["shared_gate"] = None      # the shared expert's gate is fixed at 1
    lw = oracle_layer(shape, w)
    x = synth.activations(shape, n_tok, ("layer", seed, n_tok), dtype=torch.float32 if fused else None)
    route = None
    ridx = rw = None
    if given_route:
        ridx, rw = synth.random_routing(n_tok, shape.E, shape.k, ("L", seed, n_tok))
        if prefill:
            ridx[0] = -1  # row 0 self-routes
        route = (ridx.numpy().astype(np.int64), rw.double().numpy())
    xo, y_ref, u_ref, used_ref, pred_ref, z_ref = run_oracle(lw, x.double().numpy() if x.dtype == torch.float32
                                                             else x.float().double().numpy(), route, fused)
    slots = 0
    if not resident:
        slots = shape.k * n_tok
    L = gpu_layer(shape, w, fused=fused, resident=resident, slab_slots=slots, max_tokens=max(8, n_tok))
    xd = x.cuda()
    if not resident and given_route:
        L.stage(sorted(set(int(e) for e in ridx.flatten().tolist() if e >= 0)))
    call = L.prefill if prefill else L.decode
    out = call(xd, ridx.cuda() if given_route else None, rw.cuda() if given_route else None)
    torch.cuda.synchronize()
    assert L.status() == 0
    used = out["used_idx"].cpu().numpy()
    assert np.array_equal(used, used_ref[0]), (used, used_ref[0])
    assert np.allclose(out["used_w"].cpu().numpy(), used_ref[1], rtol=1e-6, atol=1e-7)
    assert np.array_equal(out["pred_idx"].cpu().numpy(), pred_ref[0])
    assert np.allclose(out["pred_w"].cpu().numpy(), pred_ref[1], rtol=1e-6, atol=1e-7)
    y = out["y"].double().cpu().numpy()
    if fused:
        y = y - x.double().numpy()
    err = rel_l2_rows(y, y_ref)
    say(f"  rel-L2 {err:.3e}")
    assert err <= TOL, err
    return L


@pytest.mark.parametrize("given_route", [False, True])
def test_tiny_decode(given_route):
    check_layer(synth.TINY, 1, fused=False, given_route=given_route)


def test_tiny_decode_fused_batch():
    check_layer(synth.TINY, 3, fused=True, given_route=False)


@pytest.mark.parametrize("n_tok", [1, 4])
@pytest.mark.parametrize("given_route", [False, True])
def test_layer35b_decode(n_tok, given_route):
    check_layer(synth.LAYER35B, n_tok, fused=False, given_route=given_route)


def test_layer35b_fused_norm():
    check_layer(synth.LAYER35B, 2, fused=True, given_route=True, seed=3)


@pytest.mark.parametrize("given_route", [True, False])
def test_layer35b_streamed(given_route):
    L = check_layer(synth.LAYER35B, 1, fused=False, given_route=given_route, resident=False, seed=5)
    slots, nbytes = L.slots()
    staged = set(e for e in slots if e >= 0)
    assert len(staged) == synth.LAYER35B.k          # staged set == routed set at B=1
    assert nbytes == 4 * synth.LAYER35B.blob_bytes + synth.LAYER35B.shared_blob_bytes


def test_streamed_not_staged_flag():
    shape = synth.LAYER35B
    say("streamed routing to an unstaged expert raises NOT_STAGED")
    w = layer_tensors(shape, layer=7)
    L = gpu_layer(shape, w, fused=False, resident=False, slab_slots=4, max_tokens=4)
    ridx = torch.tensor([[1, 2, 3, 4]], dtype=torch.int32)
    rw = torch.full((1, 4), 0.25)
    L.stage([1, 2, 3, 5])
    x = synth.activations(shape, 1, ("ns",)).cuda()
    L.decode(x, ridx.cuda(), rw.cuda())
    import sparse_moe_decode_prerouter_amd as moe
    assert L.status() == moe.MOE_E_NOT_STAGED
    # sticky slots: staging the routed set copies only the missing expert
    before = L.slots()[1]
    L.stage([1, 2, 3, 4])
    assert L.slots()[1] - before == shape.blob_bytes
    L.decode(x, ridx.cuda(), rw.cuda())
    assert L.status() == 0


def test_bad_index_flag():
    shape = synth.TINY
    say("routing index out of range raises BAD_INDEX")
    w = layer_tensors(shape, layer=8)
    L = gpu_layer(shape, w, fused=False, max_tokens=2)
    ridx = torch.tensor([[0, shape.E + 3]], dtype=torch.int32)
    rw = torch.full((1, 2), 0.5)
    x = synth.activations(shape, 1, ("bi",)).cuda()
    L.decode(x, ridx.cuda(), rw.cuda())
    import sparse_moe_decode_prerouter_amd as moe
    assert L.status() == moe.MOE_E_BAD_INDEX


@pytest.mark.parametrize("n_tok", [5, 37])
def test_prefill_small(n_tok):
    check_layer(synth.LAYER35B, n_tok, fused=True, given_route=True, prefill=True, seed=11)


@pytest.mark.parametrize("given_route", [True, False])
def test_prefill_streamed(given_route):
    """Streamed store on the matrix-core path: the routing is read back and
    staged inside the call, then the tile records get their slab slots."""
    check_layer(synth.LAYER35B, 13, fused=True, given_route=given_route, prefill=True, resident=False, seed=13)


def test_tiny_prefill():
    check_layer(synth.TINY, 9, fused=True, given_route=True, prefill=True, seed=12)


@pytest.mark.parametrize("prefill", [True, False])
@pytest.mark.parametrize("variant", ["no_lora", "no_shared", "gate_fixed"])
def test_layer_without_branch(variant, prefill):
    """A layer without LoRA, without a shared expert, or with the shared
    gate fixed at 1: prefill (the routing GEMM packs each row set in tiles of
    its own 16 rows, one of them now empty) and a 4-token decode."""
    shape = synth.LAYER35B
    if variant == "no_lora":
        shape = dataclasses.replace(shape, name="layer_d2048_e256_k4_nolora", r=0)
    elif variant == "no_shared":
        shape = dataclasses.replace(shape, name="layer_d2048_e256_k4_noshared", fs=0)
    check_layer(shape, 21 if prefill else 4, fused=True, given_route=True, prefill=prefill, seed=14,
                gate_fixed=variant == "gate_fixed")

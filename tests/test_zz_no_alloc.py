"""moe_decode_noalloc, the decode call that allocates nothing (its scratch is
a device array the library holds per GPU), against moe_decode_step on the
same layer through the C ABI: two calls in a row, the second with fewer
tokens, must give bit-identical outputs (the same kernels run on the same
inputs); its status output reports a bad routing index; a call whose
scratch would exceed the array is rejected."""
import numpy as np
import pytest
import torch

import synth
from helpers import gpu_layer, layer_tensors, say

pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def noalloc_call(moe, L, x, route=None, status=None):
    n = x.shape[0]
    y = torch.full((n, L.d_model), float("nan"), dtype=torch.float32, device=x.device)
    io, out = L._io(x, y, None if route is None else route[0], None if route is None else route[1], True, True,
                    None, None, False)
    moe.moe_decode_noalloc(L.desc, L.weights, io, n, None if status is None else status.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    return out


@pytest.mark.parametrize("shape,fused", [(synth.LAYER35B, True), (synth.LAYER35B, False), (synth.TINY, True)])
def test_noalloc_matches_decode_step(shape, fused):
    import sparse_moe_decode_prerouter_amd as moe
    say(f"no-alloc decode vs decode step, {shape.name}, fused={fused}")
    w = layer_tensors(shape, layer=3, tag="noalloc")
    L = gpu_layer(shape, w, fused=fused, max_tokens=16)
    status = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    for i, n in enumerate([min(16, 64 // shape.k), 3]):
        for given in (False, True):
            x = synth.activations(shape, n, ("noalloc", i, given), dtype=torch.float32 if fused else None).cuda()
            route = None
            if given:
                ri, rw = synth.random_routing(n, shape.E, shape.k, ("noalloc", i))
                route = (ri.cuda(), rw.cuda())
            ref = L.decode(x, None if route is None else route[0], None if route is None else route[1])
            torch.cuda.synchronize()
            out = noalloc_call(moe, L, x, route, status)
            torch.cuda.synchronize()
            assert status.item() == moe.MOE_OK
            for key in ("y", "used_idx", "used_w", "pred_idx", "pred_w"):
                assert torch.equal(out[key], ref[key]), (n, given, key)
    assert L.status() == 0


def test_noalloc_status_bad_index():
    import sparse_moe_decode_prerouter_amd as moe
    shape = synth.TINY
    say("no-alloc decode reports a bad routing index, then a clean call reports ok")
    w = layer_tensors(shape, layer=4, tag="noalloc")
    L = gpu_layer(shape, w, fused=False, max_tokens=4)
    status = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    x = synth.activations(shape, 1, ("noalloc_bad",)).cuda()
    bad = (torch.tensor([[0, shape.E + 3]], dtype=torch.int32, device="cuda"),
           torch.full((1, 2), 0.5, device="cuda"))
    noalloc_call(moe, L, x, bad, status)
    torch.cuda.synchronize()
    assert status.item() == moe.MOE_E_BAD_INDEX
    noalloc_call(moe, L, x, None, status)
    torch.cuda.synchronize()
    assert status.item() == moe.MOE_OK


def test_noalloc_rejects_beyond_maximum():
    import sparse_moe_decode_prerouter_amd as moe
    say("no-alloc decode rejects a call whose scratch exceeds the array, and a streamed store")
    d, E, k, f = 256, 1024, 4, 128
    dev = "cuda"
    store = torch.zeros((E, 27 * d * f // 16), dtype=torch.uint8, device=dev)
    router = torch.zeros((E, d), dtype=torch.bfloat16, device=dev)
    head = torch.zeros((E, d), dtype=torch.bfloat16, device=dev)
    # 16 tokens: router and head logits alone take 2 * 16 * 1024 * 8 bytes = 256 KiB
    L = moe.MoeLayer(d_model=d, n_experts=E, top_k=k, d_ff=f, d_ff_shared=0, lora_rank=0, lora_alpha=16.0,
                     act_dtype=moe.MOE_ACT_F32, max_tokens=16, expert_store=store, router=router, head=head,
                     next_n_experts=E, next_top_k=k, resident=True)
    x = torch.zeros((16, d), dtype=torch.float32, device=dev)
    with pytest.raises(moe.MoeError) as ei:
        noalloc_call(moe, L, x)
    assert ei.value.code == moe.MOE_E_CAPACITY
    # a smaller call of the same layer fits
    out = noalloc_call(moe, L, x[:4])
    torch.cuda.synchronize()
    assert out["used_idx"].shape == (4, k)
    # a streamed (host) store is not served
    desc = moe.moe_layer_desc(*[getattr(L.desc, n) for n, _ in moe.moe_layer_desc._fields_])
    desc.flags = 0
    desc.slab_slots = 8
    io, _ = L._io(x[:1], torch.empty((1, d), device=dev), None, None, True, False, None, None, False)
    rc = moe._lib.moe_decode_noalloc(moe.ctypes.byref(desc), moe.ctypes.byref(L.weights), moe.ctypes.byref(io), 1,
                                     None, None)
    assert rc == moe.MOE_E_UNSUPPORTED

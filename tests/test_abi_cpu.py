"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every function the header declares, and its pure-host logic (slot planner,
size queries, descriptor validation) behaves as specified."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_prerouter.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    import sparse_moe_decode_prerouter_amd as moe
    lib = ctypes.CDLL(moe.LIB_PATH)
    names = header_functions()
    assert "moe_layer_create" in names and "moe_decode_step" in names and "moe_prefill" in names
    assert "moe_stage_experts" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.EXPORTED)


def test_blob_bytes():
    import sparse_moe_decode_prerouter_amd as moe
    assert moe.moe_expert_blob_bytes(2048, 512) == oracle.blob_bytes(2048, 512) == 1769472
    assert moe.moe_expert_blob_bytes(256, 128) == oracle.blob_bytes(256, 128) == 55296
    assert moe.moe_expert_blob_bytes(2048, 512, 32) == 0
    assert moe.moe_expert_blob_bytes(100, 512) == 0


def desc(**kw):
    import sparse_moe_decode_prerouter_amd as moe
    base = dict(d_model=2048, n_experts=256, top_k=4, d_ff=512, d_ff_shared=512, group_size=64, lora_rank=16,
                lora_alpha=16.0, rms_eps=1e-6, act_dtype=moe.MOE_ACT_BF16, max_tokens=4, slab_slots=5,
                next_n_experts=256, next_top_k=4, flags=moe.MOE_FUSE_NORM_RESIDUAL, head_hidden=0,
                shared_lora_rank=0, shared_lora_alpha=0.0)
    base.update(kw)
    return moe.moe_layer_desc(*[base[f] for f, _ in moe.moe_layer_desc._fields_])


def test_workspace_bytes_and_validation():
    import sparse_moe_decode_prerouter_amd as moe
    ok = moe.moe_layer_workspace_bytes(desc())
    # streamed mode holds the slab: (5 routed + 1 shared) blobs
    assert ok >= 6 * 1769472
    res = moe.moe_layer_workspace_bytes(desc(flags=moe.MOE_RESIDENT_STORE))
    assert 0 < res < ok - 6 * 1769472 + 4096
    for bad in (dict(group_size=32), dict(d_model=100), dict(top_k=9), dict(top_k=0), dict(d_ff_shared=256),
                dict(n_experts=2000), dict(act_dtype=7), dict(slab_slots=0), dict(next_top_k=0),
                dict(flags=0x80), dict(max_tokens=0), dict(head_hidden=12), dict(head_hidden=2048),
                dict(head_hidden=256, next_n_experts=0, next_top_k=0), dict(shared_lora_rank=65),
                dict(shared_lora_rank=8, d_ff_shared=0)):
        assert moe.moe_layer_workspace_bytes(desc(**bad)) == 0, bad


@pytest.mark.parametrize("seed", range(40))
def test_plan_slots_matches_oracle(seed):
    import sparse_moe_decode_prerouter_amd as moe
    rng = np.random.default_rng(1000 + seed)
    C = int(rng.integers(1, 9))
    E = 16
    resident = [int(e) for e in rng.permutation(E)[:C]]
    for s in range(C):
        if rng.random() < 0.3:
            resident[s] = -1
    wanted = [int(x) for x in rng.integers(0, E, int(rng.integers(0, C + 1)))]
    exp = oracle.plan_slots(resident, wanted)
    got = moe.moe_plan_slots(resident, wanted, E)
    assert got[0] == exp[0] and got[1] == exp[1]


def test_plan_slots_errors():
    import sparse_moe_decode_prerouter_amd as moe
    with pytest.raises(moe.MoeError) as e:
        moe.moe_plan_slots([-1, -1], [1, 2, 3], 8)
    assert e.value.code == moe.MOE_E_CAPACITY
    with pytest.raises(moe.MoeError) as e:
        moe.moe_plan_slots([-1, -1], [9], 8)
    assert e.value.code == moe.MOE_E_INVALID
    # an expert in two slots: not a slot table (both planners refuse it)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_plan_slots([5, 5, -1], [5, 7], 8)
    assert e.value.code == moe.MOE_E_INVALID
    with pytest.raises(ValueError):
        oracle.plan_slots([5, 5, -1], [5, 7])


def test_status_strings():
    import sparse_moe_decode_prerouter_amd as moe
    for c in range(0, -8, -1):
        assert moe.moe_status_str(c) != "unknown status"

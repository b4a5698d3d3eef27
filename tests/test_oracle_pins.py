"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics
(closed forms, brute force, invariants). CPU only.

Each test is chosen so that a plausible slip in the oracle (a swapped nibble,
a transposed matrix, a dropped term, a wrong sign, a wrong tie-break) fails.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16bits(v):
    return np.array(v, dtype=np.float16).view(np.uint16)


def pack_codes(q):
    """Test-side packing of integer codes [N, K] into the byte format:
    byte j holds codes 2j (low nibble) and 2j+1 (high nibble)."""
    q = np.asarray(q, dtype=np.uint8)
    out = np.zeros((q.shape[0], q.shape[1] // 2), dtype=np.uint8)
    for j in range(q.shape[1] // 2):
        out[:, j] = q[:, 2 * j] | (q[:, 2 * j + 1] << 4)
    return out


def sb_array(s, b, N, G):
    sb = np.zeros((N, G, 2), dtype=np.uint16)
    sb[..., 0] = f16bits(s)
    sb[..., 1] = f16bits(b)
    return sb


# ----------------------------------------------------------------------------
# O1 dequant
# ----------------------------------------------------------------------------
def test_dequant_closed_form_group():
    # codes 0..15 repeated, s = 1/8, b = -1  ->  W = q/8 - 1 exactly
    q = np.tile(np.arange(16), 4)[None, :]
    W = oracle.dequant_matrix(pack_codes(q), sb_array(0.125, -1.0, 1, 1))
    expect = np.tile(np.arange(16), 4) / 8.0 - 1.0
    assert np.array_equal(W[0], expect)


@pytest.mark.parametrize("pos", [0, 1, 2, 31, 62, 63])
def test_dequant_single_nibble_order(pos):
    q = np.zeros((1, 64), dtype=np.uint8)
    q[0, pos] = 9
    W = oracle.dequant_matrix(pack_codes(q), sb_array(0.5, 0.25, 1, 1))
    expect = np.full(64, 0.25)
    expect[pos] = 0.25 + 4.5
    assert np.array_equal(W[0], expect)


def test_dequant_single_nibble_raw_byte():
    # byte 3 = 0x70: code 7 at element 7 (high nibble), code 0 at element 6
    packed = np.zeros((1, 32), dtype=np.uint8)
    packed[0, 3] = 0x70
    W = oracle.dequant_matrix(packed, sb_array(1.0, 0.0, 1, 1))
    assert W[0, 7] == 7.0 and W[0, 6] == 0.0 and W[0].sum() == 7.0


def test_dequant_groups_and_zero_scale():
    N, K = 2, 192
    q = np.full((N, K), 3)
    sb = np.zeros((N, 3, 2), dtype=np.uint16)
    for g, (s, b) in enumerate([(1.0, 0.0), (2.0, 10.0), (0.0, -7.5)]):
        sb[:, g, 0] = f16bits(s)
        sb[:, g, 1] = f16bits(b)
    W = oracle.dequant_matrix(pack_codes(q), sb)
    assert np.all(W[:, :64] == 3.0)
    assert np.all(W[:, 64:128] == 16.0)
    assert np.all(W[:, 128:] == -7.5)      # s = 0 gives the bias alone


def test_quantiser_roundtrip_bound():
    w = synth.gaussian((8, 256), 0.02, ("pin", "roundtrip"))
    packed, sb = synth.quantize_g64(w)
    W = oracle.dequant_matrix(packed.numpy(), sb.view(torch.int16).numpy().view(np.uint16))
    s = oracle.f16_to_f64(sb[..., 0].view(torch.int16).numpy().view(np.uint16))
    b = oracle.f16_to_f64(sb[..., 1].view(torch.int16).numpy().view(np.uint16))
    wn = w.double().numpy().reshape(8, 4, 64)
    err = np.abs(wn - W.reshape(8, 4, 64))
    lo = b[..., None]
    hi = b[..., None] + 15 * s[..., None]
    inside = (wn >= lo) & (wn <= hi)
    # codes within range: error at most half a step (plus fp32 division slack)
    assert np.all(err[inside] <= (s[..., None] / 2 * (1 + 1e-3) + 1e-9).repeat(64, -1)[inside])
    # clipped codes: error bounded by the fp16 rounding of the range ends
    assert np.all(err <= s[..., None] * 0.5 + 2e-4)


def test_blob_regions_and_orientation():
    d, f = 128, 64
    # gate codes 1, up codes 2, down codes 3 with s = 1, b = 0; plus one marker
    gq = np.full((f, d), 1, dtype=np.uint8)
    uq = np.full((f, d), 2, dtype=np.uint8)
    dq = np.full((d, f), 3, dtype=np.uint8)
    gq[5, 70] = 15   # gate row 5, column 70
    dq[100, 9] = 14  # down row 100, column 9
    parts = [pack_codes(gq), pack_codes(uq), pack_codes(dq),
             sb_array(1.0, 0.0, f, d // 64), sb_array(1.0, 0.0, f, d // 64), sb_array(1.0, 0.0, d, f // 64)]
    blob = np.concatenate([p.reshape(-1).view(np.uint8) for p in parts])
    assert blob.size == oracle.blob_bytes(d, f) == 27 * d * f // 16
    Wg, Wu, Wd = oracle.unpack_blob(blob, d, f)
    assert Wg.shape == (f, d) and Wu.shape == (f, d) and Wd.shape == (d, f)
    assert Wg[5, 70] == 15 and Wg.sum() == f * d + 14
    assert np.all(Wu == 2)
    assert Wd[100, 9] == 14 and Wd.sum() == 3 * d * f + 11


def test_blob_size_matches_pages_checkpoint():
    """4.5 bits per weight (int4 + fp16 scale + fp16 bias per 64) puts a 35B
    model at 35e9*4.5/8 = 19.7 GB, the pages' 19.5 GB at 4-bit; an fp32-scale
    format (5 bits, 21.9 GB) or a bias-free one (4.25 bits, 18.6 GB) would not."""
    g = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    d, f = 2048, 512
    bits = oracle.blob_bytes(d, f) * 8 / (3 * d * f)
    assert bits == 4.5
    gb = g["checkpoint_35b_gb"]["params"] * bits / 8 / 1e9
    assert abs(gb - g["checkpoint_35b_gb"]["value"]) / g["checkpoint_35b_gb"]["value"] < 0.02
    assert oracle.blob_bytes(d, f) == 1769472


# ----------------------------------------------------------------------------
# O2 RMSNorm and bf16 rounding
# ----------------------------------------------------------------------------
def test_rmsnorm_constant_row():
    d, c, eps = 64, 0.7, 1e-6
    gamma = np.linspace(0.5, 1.5, d)
    u = oracle.rmsnorm(np.full(d, c), gamma, eps)
    assert np.allclose(u, gamma * c / math.sqrt(c * c + eps), rtol=0, atol=1e-15)


def test_rmsnorm_unit_rms_and_scale():
    x = np.random.default_rng(1).standard_normal(256) * 3.0
    u = oracle.rmsnorm(x, np.ones(256), 0.0)
    assert abs(np.sqrt(np.mean(u * u)) - 1.0) < 1e-14
    u2 = oracle.rmsnorm(5.0 * x, np.ones(256), 0.0)
    assert np.allclose(u, u2, atol=1e-14)


def test_round_bf16_ties_and_neighbours():
    rng = np.random.default_rng(3)
    # random positive/negative normal bf16 values
    exps = rng.integers(-60, 60, 500)
    mant = rng.integers(128, 256, 500)
    sign = rng.choice([-1.0, 1.0], 500)
    v = sign * np.ldexp(mant.astype(np.float64), exps - 8)   # exactly 8 significant bits
    assert np.array_equal(oracle.round_bf16(v), v)
    ulp = np.ldexp(1.0, exps - 8)
    mid = v + sign * ulp / 2            # halfway to the next value away from zero
    r = oracle.round_bf16(mid)
    even_is_v = (mant % 2 == 0)
    expect = np.where(even_is_v, v, v + sign * ulp)
    assert np.array_equal(r, expect)
    tiny = ulp * 2.0 ** -20
    assert np.array_equal(oracle.round_bf16(mid - sign * tiny), v)
    assert np.array_equal(oracle.round_bf16(mid + sign * tiny), v + sign * ulp)


def test_bf16_decode_known_patterns():
    assert oracle.bf16_to_f64(np.uint16(0x3F80)) == 1.0
    assert oracle.bf16_to_f64(np.uint16(0xC000)) == -2.0
    assert oracle.bf16_to_f64(np.uint16(0x4300)) == 128.0
    assert oracle.bf16_to_f64(np.uint16(0x3E80)) == 0.25


# ----------------------------------------------------------------------------
# O3-O5 routing
# ----------------------------------------------------------------------------
def precedes(z, a, b):
    return z[a] > z[b] or (z[a] == z[b] and a < b)


@pytest.mark.parametrize("seed", range(20))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 9))
    k = int(rng.integers(1, E + 1))
    z = rng.integers(-3, 4, E).astype(np.float64)  # many exact ties
    idx = list(oracle.topk(z, k))
    # brute force: the unique k-subset whose members precede every non-member
    ok = [S for S in itertools.combinations(range(E), k)
          if all(precedes(z, a, b) for a in S for b in range(E) if b not in S)]
    assert len(ok) == 1 and sorted(idx) == list(ok[0])
    assert all(precedes(z, idx[i], idx[i + 1]) for i in range(k - 1))


def test_topk_exact_ties_lowest_index():
    z = np.array([1.0, 3.0, 3.0, 2.0, 3.0])
    assert list(oracle.topk(z, 2)) == [1, 2]
    assert list(oracle.topk(z, 3)) == [1, 2, 4]
    assert list(oracle.topk(z, 5)) == [1, 2, 4, 3, 0]


def test_route_weights_closed_form():
    z = np.array([0.0, math.log(2.0), math.log(3.0), -5.0])
    idx, w = oracle.route(z, 2)
    assert list(idx) == [2, 1]
    assert np.allclose(w, [3 / 5, 2 / 5], rtol=0, atol=1e-15)


@pytest.mark.parametrize("seed", range(5))
def test_route_weights_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    z = rng.standard_normal(256)
    idx, w = oracle.route(z, 4)
    assert abs(w.sum() - 1.0) < 1e-12 and np.all(w > 0)
    assert np.all(np.diff(w) <= 0)   # descending logits give descending weights
    idx2, w2 = oracle.route(z + 37.25, 4)
    assert np.array_equal(idx, idx2) and np.allclose(w, w2, atol=1e-14)


def test_head_logits_bias_and_history():
    E, d = 6, 64
    H = np.zeros((E, d), dtype=np.uint16)   # +0.0 everywhere
    u = np.ones(d)
    bias = np.arange(E, dtype=np.float64)
    Mc = 10.0 * np.eye(E)
    Mp = np.zeros((E, E)); Mp[2, 0] = 100.0   # prev contains 2 -> boosts expert 0
    z = oracle.head_logits(H, u, bias, Mc, [1, 3], Mp, [2, -1])
    assert np.array_equal(z, [100.0, 11.0, 2.0, 13.0, 4.0, 5.0])
    # H contribution: single nonzero row entry, bf16 0x3F80 = 1.0 at (4, 7)
    H2 = np.zeros((E, d), dtype=np.uint16); H2[4, 7] = 0x3F80
    u2 = np.zeros(d); u2[7] = 2.5
    assert np.array_equal(oracle.head_logits(H2, u2), [0, 0, 0, 0, 2.5, 0])


# ----------------------------------------------------------------------------
# O6 expert FFN with permutation structure (closed form)
# ----------------------------------------------------------------------------
def perm_expert(d, f, pg, pu, pd, sg, su, sd):
    """Blob whose matrices are scaled permutation-selectors: Wg[n, pg[n]] = 15*sg, etc."""
    gq = np.zeros((f, d), np.uint8); uq = np.zeros((f, d), np.uint8); dq = np.zeros((d, f), np.uint8)
    gq[np.arange(f), pg] = 15
    uq[np.arange(f), pu] = 15
    dq[np.arange(d), pd] = 15
    parts = [pack_codes(gq), pack_codes(uq), pack_codes(dq),
             sb_array(sg, 0.0, f, d // 64), sb_array(su, 0.0, f, d // 64), sb_array(sd, 0.0, d, f // 64)]
    return np.concatenate([p.reshape(-1).view(np.uint8) for p in parts])


def silu_scalar(a):
    return a / (1.0 + math.exp(-a))


def test_expert_ffn_closed_form():
    d, f = 128, 64
    rng = np.random.default_rng(7)
    pg = rng.permutation(d)[:f]
    pu = rng.permutation(d)[:f]
    pd = rng.integers(0, f, d)
    blob = perm_expert(d, f, pg, pu, pd, 0.0625, 0.125, 0.25)
    u = rng.standard_normal(d)
    o = oracle.expert_ffn(oracle.unpack_blob(blob, d, f), u)
    a = [15 * 0.0625 * u[pg[n]] for n in range(f)]
    c = [15 * 0.125 * u[pu[n]] for n in range(f)]
    h = [silu_scalar(a[n]) * c[n] for n in range(f)]
    expect = np.array([15 * 0.25 * h[pd[i]] for i in range(d)])
    assert np.allclose(o, expect, rtol=1e-14, atol=1e-15)


def test_silu_values():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12
    assert abs(oracle.silu(-40.0)) < 1e-15
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


# ----------------------------------------------------------------------------
# O7-O9 block
# ----------------------------------------------------------------------------
def tiny_layer(E=8, k=2, d=128, f=64, fs=64, r=4, seed=0, identical=False, shared_gate=True):
    sh = synth.Shape("pin_tiny", d=d, E=E, k=k, f=f, fs=fs, r=r, alpha=8.0, act="f32")
    w = synth.layer_weights(sh, seed, tag="pin")
    store = synth.to_numpy_bytes(w["store"])
    if identical:
        store = np.repeat(store[:1], E, axis=0)
    lw = oracle.LayerWeights(
        d=d, E=E, k=k, f=f, fs=fs, r=r, alpha=8.0, eps=1e-6, act="f32", store=store,
        shared=synth.to_numpy_bytes(w["shared"]) if fs else None,
        shared_gate=synth.bf16_bits(w["shared_gate"]) if (fs and shared_gate) else None,
        lora_a=synth.bf16_bits(w["lora_a"]) if r else None, lora_b=synth.bf16_bits(w["lora_b"]) if r else None,
        gamma=w["gamma"].double().numpy(), head=synth.bf16_bits(w["head"]), router=synth.bf16_bits(w["router"]))
    return lw


def test_block_identical_experts_combine():
    lw = tiny_layer(identical=True, fs=0, r=0)
    u = np.random.default_rng(0).standard_normal(lw.d)
    single = oracle.expert_ffn(lw.expert(0), u)
    y = oracle.moe_block(lw, u, [3, 5], [0.3, 0.7])
    assert np.allclose(y, single, rtol=1e-13, atol=1e-15)


def test_block_k1_and_linearity_in_weights():
    lw = tiny_layer(fs=0, r=0)
    u = np.random.default_rng(1).standard_normal(lw.d)
    o2 = oracle.expert_ffn(lw.expert(2), u)
    o6 = oracle.expert_ffn(lw.expert(6), u)
    assert np.array_equal(oracle.moe_block(lw, u, [2], [1.0]), o2)
    y = oracle.moe_block(lw, u, [6, 2], [0.25, 0.75])
    assert np.allclose(y, 0.25 * o6 + 0.75 * o2, rtol=1e-14, atol=1e-15)


def test_shared_gate_half_at_zero():
    lw = tiny_layer(r=0)
    lw.shared_gate = np.zeros(lw.d, dtype=np.uint16)
    u = np.random.default_rng(2).standard_normal(lw.d)
    y = oracle.moe_block(lw, u, [1], [1.0])
    expect = oracle.expert_ffn(lw.expert(1), u) + 0.5 * oracle.expert_ffn(lw.shared_expert(), u)
    assert np.allclose(y, expect, rtol=1e-14, atol=1e-15)


def test_lora_rank1_closed_form_and_noop():
    lw = tiny_layer(fs=0, r=1)
    d = lw.d
    a = np.zeros(d); a[3] = 2.0; a[10] = -0.5
    bvec = np.zeros(d); bvec[7] = 0.25
    lw.lora_a = oracle.bf16_bits_of(a)[None, :]
    lw.lora_b = oracle.bf16_bits_of(bvec)[:, None]
    u = np.random.default_rng(3).standard_normal(d)
    base = oracle.expert_ffn(lw.expert(0), u)
    y = oracle.moe_block(lw, u, [0], [1.0])
    delta = np.zeros(d); delta[7] = lw.alpha * 0.25 * (2.0 * u[3] - 0.5 * u[10])
    assert np.allclose(y - base, delta, rtol=1e-13, atol=1e-14)
    lw.lora_b = np.zeros((d, 1), dtype=np.uint16)
    assert np.array_equal(oracle.moe_block(lw, u, [0], [1.0]), base)


def test_relabel_experts_invariance():
    lw = tiny_layer()
    u = np.random.default_rng(4).standard_normal(lw.d)
    y = oracle.moe_block(lw, u, [1, 4], [0.6, 0.4])
    perm = np.random.default_rng(5).permutation(lw.E)     # new slot of old expert e = perm[e]
    store2 = np.empty_like(lw.store)
    store2[perm] = lw.store
    lw2 = tiny_layer()
    lw2.store = store2
    y2 = oracle.moe_block(lw2, u, [perm[1], perm[4]], [0.6, 0.4])
    assert np.array_equal(y, y2)


# ----------------------------------------------------------------------------
# O11 dataflow
# ----------------------------------------------------------------------------
def small_stack(L=4, seed=0, act="bf16"):
    layers = []
    for l in range(L):
        lw = tiny_layer(seed=100 * seed + l)
        lw.act = act
        layers.append(lw)
    return layers


def test_prefill_equals_sequential_decode():
    """Head l on token i routes layer l+1 on token i+1 in prefill, exactly as
    head l at step t routes layer l+1 at step t+1 in decode: prefill rows must
    equal a B=1 decode run whose step inputs are the prefill tokens."""
    layers = small_stack()
    T = 6
    xs = np.random.default_rng(9).standard_normal((T, 1, layers[0].d))
    xp, recs = oracle.stack_prefill(layers, xs[:, 0, :])
    steps = oracle.stack_decode(layers, xs, T)
    for t in range(T):
        assert np.array_equal(steps[t].x_out[0], xp[t])
        for l in range(len(layers)):
            assert np.array_equal(steps[t].routes[l][0][0], recs[l]["route"][0][t])
    # the routing really is the shifted prediction (layer >= 1, token >= 1)
    for l in range(1, len(layers)):
        assert np.array_equal(recs[l]["route"][0][1:], recs[l - 1]["pred"][0][:-1])


def test_batch_rows_equal_single_rows():
    layers = small_stack(L=2)
    lw = layers[0]
    x = np.random.default_rng(11).standard_normal((3, lw.d))
    xo, y, u, used, pred, z = oracle.decode_layer(lw, x, None, lw.k)
    for b in range(3):
        xo1, y1, *_ = oracle.decode_layer(lw, x[b:b + 1], None, lw.k)
        assert np.array_equal(y[b], y1[0]) and np.array_equal(xo[b], xo1[0])


def test_decode_step0_self_routes_then_predicted():
    layers = small_stack(L=3)
    xs = np.random.default_rng(12).standard_normal((3, 2, layers[0].d))
    recs = oracle.stack_decode(layers, xs, 3)
    assert all(recs[0].self_routed)
    assert recs[1].self_routed == [True, False, False]
    for l in (1, 2):
        assert np.array_equal(recs[2].routes[l][0], recs[1].preds[l - 1][0])


# ----------------------------------------------------------------------------
# O12 staging plan
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(30))
def test_plan_slots_properties(seed):
    rng = np.random.default_rng(seed)
    C = int(rng.integers(1, 7))
    E = 12
    resident = [int(e) for e in rng.permutation(E)[:C]]
    for s in range(C):
        if rng.random() < 0.3:
            resident[s] = -1
    n = int(rng.integers(0, C + 1))
    wanted = list(rng.choice(E, n, replace=True))
    new, copies = oracle.plan_slots(resident, wanted)
    want = set(int(e) for e in wanted)
    assert want <= set(new)                                     # staged set covers routed set
    assert len(copies) == len(want - set(resident))             # minimal copies
    for s in range(C):                                          # sticky
        if resident[s] in want:
            assert new[s] == resident[s]
    for s, e in copies:
        assert resident[s] not in want and new[s] == e
    # deterministic order: missing ids ascending fill free slots ascending
    assert [e for _, e in copies] == sorted(e for _, e in copies)
    assert [s for s, _ in copies] == sorted(s for s, _ in copies)


def test_plan_slots_capacity():
    with pytest.raises(ValueError):
        oracle.plan_slots([-1, -1], [1, 2, 3])


def test_head_input_width_from_pages():
    g = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))["head_input_width_35b"]
    assert g["d_model"] + 2 * g["experts"] == g["value"]


# ----------------------------------------------------------------------------
# Pins of the shared gate's sign and input, the LoRA scale at r > 1, the
# residual, and the stack's history wiring. Each is a closed form or a
# hand-derived trajectory that a plausible slip changes.
# ----------------------------------------------------------------------------
def zero_blob(d, f):
    """An expert whose three matrices are exactly zero (codes 0, s = b = 0)."""
    return np.zeros(oracle.blob_bytes(d, f), dtype=np.uint8)


def test_shared_gate_three_quarters_on_normalised_input():
    """sigma(g . u) with g . u = ln 3 is 3/4 exactly (1 / (1 + 1/3)). Here the
    input x is all ones, the norm has eps = 0, so u = gamma (in fp32) and
    g = e_0 picks u_0 = fp32(ln 3). A gate with the opposite sign gives 1/4;
    a gate taken on x instead of u gives sigma(1) = 0.731."""
    lw = tiny_layer(r=0)
    d = lw.d
    lw.eps = 0.0
    lw.gamma = np.ones(d)
    lw.gamma[0] = math.log(3.0)
    g = np.zeros(d); g[0] = 1.0
    lw.shared_gate = oracle.bf16_bits_of(g)
    x = np.ones((1, d))
    route = (np.array([[2, 5]]), np.array([[0.5, 0.5]]))
    xo, y, u, used, pred, z = oracle.decode_layer(lw, x, route, None, fused_norm=True)
    u0 = u[0]
    assert u0[0] == float(np.float32(math.log(3.0))) and np.all(u0[1:] == 1.0)
    routed = 0.5 * oracle.expert_ffn(lw.expert(2), u0) + 0.5 * oracle.expert_ffn(lw.expert(5), u0)
    shared = oracle.expert_ffn(lw.shared_expert(), u0)
    ratio = (y[0] - routed) / shared
    assert np.allclose(ratio, 0.75, rtol=0, atol=1e-7)


def test_lora_scale_alpha_over_r_at_rank4():
    """Rank 4, alpha 8: the branch is scaled by alpha / r = 2 (a scale of alpha
    would give 8, alpha / sqrt(r) would give 4). A = the first four unit rows
    and B[7, i] = (i + 1) / 4 make (B A u)_7 = sum_i (i + 1) u_i / 4, with every
    other output zero; the experts are zero so y is the branch alone."""
    d, r = 128, 4
    lw = tiny_layer(fs=0, r=r)
    assert lw.alpha == 8.0 and lw.r == 4
    lw.store = np.stack([zero_blob(d, lw.f)] * lw.E)
    A = np.zeros((r, d)); A[np.arange(r), np.arange(r)] = 1.0
    Bm = np.zeros((d, r)); Bm[7, :] = (np.arange(r) + 1) / 4.0
    lw.lora_a = oracle.bf16_bits_of(A)
    lw.lora_b = oracle.bf16_bits_of(Bm)
    u = np.random.default_rng(21).standard_normal(d)
    y = oracle.moe_block(lw, u, [0, 1], [0.5, 0.5])
    expect = np.zeros(d)
    expect[7] = 2.0 * (1 * u[0] + 2 * u[1] + 3 * u[2] + 4 * u[3]) / 4.0
    assert np.allclose(y, expect, rtol=1e-14, atol=1e-15)


def test_residual_adds_block_output_to_x():
    """x_out = x + y. With zero experts, no shared expert and a rank-1 branch
    of closed form, y = 8 * b (a . u) at one coordinate, so x_out - x is that
    value there and exactly zero elsewhere. A residual taken from u (the
    normalised input) or a dropped residual fails."""
    d = 128
    lw = tiny_layer(fs=0, r=1)
    lw.store = np.stack([zero_blob(d, lw.f)] * lw.E)
    a = np.zeros(d); a[5] = 1.0
    bvec = np.zeros(d); bvec[9] = 0.5
    lw.lora_a = oracle.bf16_bits_of(a)[None, :]
    lw.lora_b = oracle.bf16_bits_of(bvec)[:, None]
    x = np.random.default_rng(22).standard_normal((2, d)) * 3.0
    route = (np.array([[0, 1], [3, 2]]), np.array([[0.5, 0.5], [0.9, 0.1]]))
    xo, y, u, used, pred, z = oracle.decode_layer(lw, x, route, None, fused_norm=True)
    for b in range(2):
        un = float(np.float32(x[b, 5] / math.sqrt(np.mean(x[b] ** 2) + lw.eps) * lw.gamma[5]))
        delta = np.zeros(d); delta[9] = lw.alpha * 0.5 * un
        assert np.allclose(xo[b] - x[b], delta, rtol=1e-13, atol=1e-14)
        assert np.array_equal(xo[b][np.arange(d) != 9], x[b][np.arange(d) != 9])


# The history wiring of the stack. Head l predicts layer l+1 at the next step;
# its one-hot inputs are layer l+1's routing at this step (cur) and at the
# previous step (prev). In the hand-built stack below every expert is zero, so
# x never changes, every head and router matrix is zero, and the logits are
# bias + history only:
#   routers (self-routing, layer 0 every step and all layers at step 0):
#     layer 0 -> {0, 1}, layer 1 -> {2, 3}, layer 2 -> {4, 5}
#   head 0 bias (.2 on 6, .1 on 7); head 1 bias (.2 on 0, .1 on 1)
#   Mc = 10 I (an expert in cur gains 10)
#   Mp[j, (j + 1) mod 8] = 10 (an expert j in prev lifts expert j + 1 by 10)
# Step 0: no history; head 0 predicts layer 1 = [6, 7], head 1 predicts
#   layer 2 = [0, 1].
# Step 1: layer 1 uses [6, 7], layer 2 uses [0, 1].
#   head 0: cur = {6, 7}, prev = layer 1 at step 0 = {2, 3} lifts {3, 4};
#     z6 = 10.2, z7 = 10.1, z3 = z4 = 10 -> [6, 7]
#   head 1: cur = {0, 1}, prev = layer 2 at step 0 = {4, 5} lifts {5, 6};
#     z0 = 10.2, z1 = 10.1, z5 = z6 = 10 -> [0, 1]
# Step 2: layer 1 uses [6, 7], layer 2 uses [0, 1].
#   head 0: cur = {6, 7}, prev = {6, 7} lifts {7, 0}; z7 = 20.1, z6 = 10.2,
#     z0 = 10 -> [7, 6]
#   head 1: cur = {0, 1}, prev = {0, 1} lifts {1, 2}; z1 = 20.1, z0 = 10.2,
#     z2 = 10 -> [1, 0]
# Taking cur or prev from layer l, or cur from step t-1, or prev from step t,
# changes at least one of these predictions (checked below; e.g. cur from
# step t-1 gives head 0 at step 1 cur = {2, 3}, so z3 = 20 and [3, 2]).
HIST_EXPECT = {            # step -> (head 0 prediction, head 1 prediction)
    0: ([6, 7], [0, 1]),
    1: ([6, 7], [0, 1]),
    2: ([7, 6], [1, 0]),
}


def history_stack():
    E, k, d, f = 8, 2, 64, 64
    layers = []
    router_bias = [np.array([2, 1, 0, 0, 0, 0, 0, 0.]), np.array([0, 0, 2, 1, 0, 0, 0, 0.]),
                   np.array([0, 0, 0, 0, 2, 1, 0, 0.])]
    head_bias = [np.array([0, 0, 0, 0, 0, 0, .2, .1]), np.array([.2, .1, 0, 0, 0, 0, 0, 0])]
    Mp = np.zeros((E, E))
    for j in range(E):
        Mp[j, (j + 1) % E] = 10.0
    for l in range(3):
        lw = oracle.LayerWeights(
            d=d, E=E, k=k, f=f, fs=0, r=0, alpha=0.0, eps=1e-6, act="bf16",
            store=np.stack([zero_blob(d, f)] * E), shared=None, shared_gate=None, lora_a=None, lora_b=None,
            gamma=np.ones(d), head=np.zeros((E, d), np.uint16) if l < 2 else None,
            router=np.zeros((E, d), np.uint16), router_bias=router_bias[l],
            head_bias=head_bias[l] if l < 2 else None,
            hist_cur=10.0 * np.eye(E) if l < 2 else None, hist_prev=Mp if l < 2 else None)
        layers.append(lw)
    return layers


def simulate_routing(wiring):
    """Routing-only replay of the hand-built stack under a given reading of
    which routing feeds the history one-hots (the test's own derivation; the
    correct reading must reproduce HIST_EXPECT)."""
    E = 8
    b0 = [np.array([0, 0, 0, 0, 0, 0, .2, .1]), np.array([.2, .1, 0, 0, 0, 0, 0, 0])]
    selfr = {0: [0, 1], 1: [2, 3], 2: [4, 5]}
    used = {}          # (layer, step) -> list
    preds = {}
    for t in range(3):
        for l in range(3):
            used[(l, t)] = selfr[l] if (t == 0 or l == 0) else preds[(l - 1, t - 1)]
        for l in range(2):
            cur, prev = wiring(used, l, t)
            z = b0[l].copy()
            for e in (cur or []):
                z[e] += 10.0
            for e in (prev or []):
                z[(e + 1) % E] += 10.0
            order = sorted(range(E), key=lambda e: (-z[e], e))
            preds[(l, t)] = order[:2]
    return {t: (preds[(0, t)], preds[(1, t)]) for t in range(3)}


def _w_correct(used, l, t):
    return (used[(l + 1, t)] if t > 0 else None), (used[(l + 1, t - 1)] if t > 0 else None)


def test_stack_history_wiring_hand_derived():
    layers = history_stack()
    xs = np.random.default_rng(23).standard_normal((3, 1, layers[0].d))
    recs = oracle.stack_decode(layers, xs, 3)
    for t, (p0, p1) in HIST_EXPECT.items():
        assert list(recs[t].preds[0][0][0]) == p0, (t, recs[t].preds[0][0][0])
        assert list(recs[t].preds[1][0][0]) == p1, (t, recs[t].preds[1][0][0])
        if t >= 1:
            # the routing really is the prediction of the step before
            assert list(recs[t].routes[1][0][0]) == HIST_EXPECT[t - 1][0]
            assert list(recs[t].routes[2][0][0]) == HIST_EXPECT[t - 1][1]
    assert simulate_routing(_w_correct) == HIST_EXPECT
    mutations = {
        "cur from layer l": lambda u, l, t: ((u[(l, t)] if t > 0 else None), _w_correct(u, l, t)[1]),
        "prev from layer l": lambda u, l, t: (_w_correct(u, l, t)[0], (u[(l, t - 1)] if t > 0 else None)),
        "cur from step t-1": lambda u, l, t: ((u[(l + 1, t - 1)] if t > 0 else None), _w_correct(u, l, t)[1]),
        "prev from step t": lambda u, l, t: (_w_correct(u, l, t)[0], (u[(l + 1, t)] if t > 0 else None)),
    }
    for name, wiring in mutations.items():
        assert simulate_routing(wiring) != HIST_EXPECT, name


# ----------------------------------------------------------------------------
# O3b the head's MLP branch: fc2(erf-GELU(fc1([u, onehot cur, onehot prev])))
# ----------------------------------------------------------------------------
PHI_1 = 0.8413447460685429      # standard normal CDF at 1 (textbook table value)
PHI_2 = 0.9772498680518208      # at 2


def test_gelu_erf_normal_cdf_values():
    """erf-GELU(a) = a Phi(a): Phi(1), Phi(2) and Phi(0) = 1/2 from the normal
    table; GELU(a) - GELU(-a) = a; the tanh approximation of GELU differs at
    1 by 1.5e-4, so a tanh form would fail."""
    g = oracle.gelu_erf(np.array([1.0, -1.0, 2.0, 0.0, 0.5]))
    assert abs(g[0] - PHI_1) < 1e-15
    assert abs(g[1] - (-(1.0 - PHI_1))) < 1e-15
    assert abs(g[2] - 2.0 * PHI_2) < 1e-15
    assert g[3] == 0.0
    a = np.linspace(-4, 4, 17)
    assert np.allclose(oracle.gelu_erf(a) - oracle.gelu_erf(-a), a, atol=1e-15)
    tanh_form = 0.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * (1 + 0.044715)))
    assert abs(g[0] - tanh_form) > 1e-4


def mlp_case():
    """E = 6 experts, H1 = 3 hidden units, d = 64. W1u = 0. The one-hot
    columns: current expert j adds v_j to unit 0; previous expert j adds
    -2 v_j to unit 1 (v = 1/2, 1/4, 3/4, 1/8, 3/8, 5/8, exact in bf16); unit
    2 sees only its bias. W2 [6, 3]: rows 0, 1, 2 pick units 0, 1, 2; rows
    3..5 are zero."""
    E, H1, d = 6, 3, 64
    W1u = np.zeros((H1, d), np.uint16)
    vals = [0.5, 0.25, 0.75, 0.125, 0.375, 0.625]
    W1oh = np.zeros((2 * E, H1))
    for j in range(E):
        W1oh[j, 0] = vals[j]
        W1oh[E + j, 1] = -2.0 * vals[j]
    W2 = np.zeros((E, H1))
    W2[0, 0] = W2[1, 1] = W2[2, 2] = 1.0
    return E, H1, d, W1u, oracle.bf16_bits_of(W1oh), oracle.bf16_bits_of(W2)


def test_head_mlp_onehot_wiring_closed_form():
    """cur = {1, 2} gives unit 0 the value 1/4 + 3/4 = 1; prev = {0} gives
    unit 1 -2 (1/2) = -1; unit 2 has bias 2. The logits are then the table
    values [Phi(1), -(1 - Phi(1)), 2 Phi(2), 0, 0, 0]. Swapping cur and prev
    (unit 0 = 1/2, unit 1 = -2), reading prev at column j instead of E + j
    (unit 1 = 0), or a transposed W2 gives other values."""
    E, H1, d, W1u, W1oh, W2 = mlp_case()
    u = np.random.default_rng(31).standard_normal(d)
    b1 = np.array([0.0, 0.0, 2.0])
    z = oracle.head_mlp(W1u, W1oh, b1, W2, u, E, cur=[1, 2, -1], prev=[0])
    assert np.allclose(z, [PHI_1, -(1.0 - PHI_1), 2.0 * PHI_2, 0, 0, 0], rtol=0, atol=1e-15)
    # duplicates in a routing list set the one-hot once
    z2 = oracle.head_mlp(W1u, W1oh, b1, W2, u, E, cur=[1, 2, 2], prev=[0, 0])
    assert np.array_equal(z, z2)


def test_head_mlp_hidden_columns_and_zero_fc2():
    """The hidden-state columns: W1u row 0 picks 2 u_5, so unit 0 = 2 u_5; with
    u_5 = 1/2 that is GELU(1) = Phi(1). W2 = 0 leaves the linear head alone in
    predict_next, and a nonzero W2 adds exactly head_mlp to it."""
    E, H1, d, W1u, W1oh, W2 = mlp_case()
    W1u = np.zeros((H1, d)); W1u[0, 5] = 2.0
    W1u = oracle.bf16_bits_of(W1u)
    u = np.zeros(d); u[5] = 0.5
    z = oracle.head_mlp(W1u, W1oh, None, W2, u, E)
    assert abs(z[0] - PHI_1) < 1e-15 and np.all(z[1:] == 0.0)
    lw = tiny_layer(E=E, k=2, d=d, f=64, fs=0, r=0)
    H = np.zeros((E, d)); H[4, 5] = 1.0                      # l(x)_4 = u_5
    lw.head = oracle.bf16_bits_of(H)
    lw.head_fc1, lw.head_fc1_oh, lw.head_fc1_bias = W1u, W1oh, None
    lw.head_fc2 = np.zeros((E, H1), np.uint16)
    idx0, w0, z0 = oracle.predict_next(lw, u, 2)
    assert np.array_equal(z0, oracle.head_logits(lw.head, u))
    lw.head_fc2 = W2
    idx1, w1, z1 = oracle.predict_next(lw, u, 2)
    assert abs(z1[0] - PHI_1) < 1e-15 and z1[4] == 0.5 and list(idx1) == [0, 4]


# ----------------------------------------------------------------------------
# O8b the recovery LoRA on the shared expert's projections
# ----------------------------------------------------------------------------
def shared_lora_case():
    """A layer whose shared expert is zero (W = 0 exactly), with a rank-2
    adapter of alpha 4 (scale 2) on its projections: A of gate picks u_0,
    u_1; B of gate sends the first to unit 3 with weight 1/2; A of up picks
    u_2, u_3, B of up sends the second to unit 3 with weight 1/4; A of down
    reads unit 3 of h, B of down writes it to output 7."""
    d, f, rs = 64, 64, 2
    lw = tiny_layer(d=d, f=f, fs=f, r=0, shared_gate=False)
    lw.shared = zero_blob(d, f)
    lw._cache.clear()
    A = np.zeros((2 * rs, d)); A[0, 0] = A[1, 1] = 1.0; A[2, 2] = A[3, 3] = 1.0
    B = np.zeros((2 * f, rs)); B[3, 0] = 0.5; B[f + 3, 1] = 0.25
    Ad = np.zeros((rs, f)); Ad[0, 3] = 1.0
    Bd = np.zeros((d, rs)); Bd[7, 0] = 1.0
    lw.shared_lora_rank, lw.shared_lora_alpha = rs, 4.0
    lw.shared_lora_a, lw.shared_lora_b = oracle.bf16_bits_of(A), oracle.bf16_bits_of(B)
    lw.shared_lora_ad, lw.shared_lora_bd = oracle.bf16_bits_of(Ad), oracle.bf16_bits_of(Bd)
    return lw


def test_shared_lora_closed_form():
    """a_3 = 2 (1/2) u_0 = u_0, c_3 = 2 (1/4) u_3 = u_3 / 2, h_3 = silu(u_0) u_3 / 2
    and o_7 = 2 h_3 = silu(u_0) u_3; with u_0 = 40 (silu(40) = 40 to 1e-16)
    the shared output is 40 u_3 at 7 and zero elsewhere. A scale of alpha
    (4x), swapped gate / up adapters, or a down adapter reading u instead of
    h all give other values."""
    lw = shared_lora_case()
    u = np.random.default_rng(41).standard_normal(lw.d)
    u[0] = 40.0
    o = oracle.shared_ffn(lw, u)
    expect = np.zeros(lw.d); expect[7] = 40.0 * u[3]
    assert np.allclose(o, expect, rtol=1e-14, atol=1e-14)
    # inside the block, with the gate fixed at 1 and zero routed experts
    lw.store = np.stack([zero_blob(lw.d, lw.f)] * lw.E)
    lw._cache.clear()
    y = oracle.moe_block(lw, u, [0, 1], [0.5, 0.5])
    assert np.allclose(y, expect, rtol=1e-14, atol=1e-14)


def test_shared_lora_zero_b_is_plain_shared():
    lw = tiny_layer(r=0)
    u = np.random.default_rng(42).standard_normal(lw.d)
    plain = oracle.expert_ffn(lw.shared_expert(), u)
    rs = 4
    lw.shared_lora_rank, lw.shared_lora_alpha = rs, 8.0
    lw.shared_lora_a = oracle.bf16_bits_of(np.random.default_rng(43).standard_normal((2 * rs, lw.d)))
    lw.shared_lora_b = np.zeros((2 * lw.fs, rs), np.uint16)
    lw.shared_lora_ad = oracle.bf16_bits_of(np.random.default_rng(44).standard_normal((rs, lw.fs)))
    lw.shared_lora_bd = np.zeros((lw.d, rs), np.uint16)
    assert np.array_equal(oracle.shared_ffn(lw, u), plain)

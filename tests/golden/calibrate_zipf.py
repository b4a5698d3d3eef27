"""Calibrates the batched-decode routing workload and writes zipf_calibration.json.

The workload is a 35B-shape layer whose prerouter head gets two extra terms:
  - a Zipf popularity bias b_e = tau * log p_{pi(e)}, with p_r proportional
    to r^-1.1;
  - a stickiness term beta * 1[e in the current routing of the predicted layer].
tau is chosen so that expert usage falls off with rank with a fitted log-log
slope near -1.1. beta is chosen so that the mean next-token reuse
|R(t) ∩ R(t+1)| / k is 0.444. That reuse figure is the next-token expert-reuse
probability from the routing-trace section of the cache article
("MoE μοντέλα στην άκρη: γιατί η cache δεν λύνει μόνη της το bandwidth
bottleneck").

Only oracle/ does the arithmetic; synth/ supplies the seeded draws. Run:
    python tests/golden/calibrate_zipf.py
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

TARGET_REUSE = 0.444
TARGET_SLOPE = -1.1
STEPS = 1500


def chain(hu: np.ndarray, bias: np.ndarray, beta: float, k: int):
    """Routing chain R(t+1) = topk(H u_t + bias + beta * 1[R(t)]); returns the
    mean reuse and the usage counts per expert."""
    E = hu.shape[1]
    cur = None
    reuse, counts = [], np.zeros(E)
    mat = beta * np.eye(E) if beta else None
    for t in range(hu.shape[0]):
        z = hu[t] + bias
        if mat is not None and cur is not None:
            # the oracle's history term, fed precomputed H u (see head_logits)
            onehot = np.zeros(E)
            onehot[cur] = 1.0
            z = z + mat.T @ onehot
        nxt = oracle.topk(z, k)
        if cur is not None:
            reuse.append(len(set(nxt.tolist()) & set(cur.tolist())) / k)
        counts[nxt] += 1
        cur = nxt
    return float(np.mean(reuse)), counts


def usage_slope(counts: np.ndarray) -> float:
    c = np.sort(counts)[::-1]
    c = c[c > 0]
    n = max(8, min(len(c), 64))
    r = np.arange(1, n + 1)
    return float(np.polyfit(np.log(r), np.log(c[:n]), 1)[0])


def main():
    shape = synth.LAYER35B
    w = synth.layer_weights(shape, 0, device="cpu", tag="zipfcal")
    H = synth.bf16_bits(w["head"])
    gamma = w["gamma"].double().numpy()
    xs = synth.activations(shape, STEPS, ("zipfcal",), dtype=torch_float32()).double().numpy()
    # block inputs as the stack computes them (RMSNorm, one rounding to bf16),
    # then the head term through the oracle
    us = np.stack([oracle.round_bf16(oracle.rmsnorm(x[None, :], gamma, shape.eps)[0]) for x in xs])
    hu = np.stack([oracle.head_logits(H, u) for u in us])
    logp = synth.zipf_bias(shape.E, 1.1, 1.0, ("zipfcal",)).double().numpy()   # tau = 1: log p_{pi(e)}
    # tau: usage slope closest to -1.1 at beta = 0 (grid, then refine)
    best = None
    for tau in np.linspace(0.1, 3.0, 30):
        _, cnt = chain(hu, tau * logp, 0.0, shape.k)
        s = usage_slope(cnt)
        if best is None or abs(s - TARGET_SLOPE) < abs(best[1] - TARGET_SLOPE):
            best = (float(tau), s)
    tau = best[0]
    # beta: bisection on reuse (monotone in beta)
    lo, hi = 0.0, 10.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        r, _ = chain(hu, tau * logp, mid, shape.k)
        if r < TARGET_REUSE:
            lo = mid
        else:
            hi = mid
    beta = 0.5 * (lo + hi)
    reuse, cnt = chain(hu, tau * logp, beta, shape.k)
    reuse0, _ = chain(hu, tau * logp, 0.0, shape.k)
    out = {
        "workload": "layer d2048 E256 k4, head N(0,0.02) bf16, x ~ N(0,1) per step, Zipf 1.1 bias + stickiness",
        "zipf_s": 1.1, "tau": round(tau, 4), "beta": round(beta, 4),
        "fitted_usage_slope": round(best[1], 3), "reuse_at_beta": round(reuse, 4),
        "reuse_at_beta0": round(reuse0, 4), "target_reuse": TARGET_REUSE, "steps": STEPS,
        "target_source": "cache article, routing-trace section: next-token expert reuse probability 0.444",
        "written_by": "tests/golden/calibrate_zipf.py (oracle head logits and top-k only)",
    }
    with open(os.path.join(HERE, "zipf_calibration.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def torch_float32():
    import torch
    return torch.float32


if __name__ == "__main__":
    main()

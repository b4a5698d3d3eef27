"""Checks of a stacked call layer by layer, on the inputs the GPU saw.

The stack writes each layer's input residual stream into a trace (the
stack's set_trace). Layer l is then checked on exactly that input: its
routing decisions against the oracle's logits on the same u (bit-exact, or a
certified near tie within the computed bound), and its block output
y_l = x_{l+1} - x_l against the oracle's block on the routing the GPU used.
"""
from __future__ import annotations

import numpy as np

import oracle
from helpers import layer_same_input_check, rel_l2_rows


def check_stack_layers(ora, trace, x_out, used, used_w, given, pred, pred_w, mode, *, cur=None, prev=None,
                       rows=None, outputs=True, tol=2e-3, what=""):
    """ora: oracle layers; trace [L, n, d] inputs; x_out [n, d]; used/used_w
    [L, n, k]; given[l]: (idx, w) [n, k] routing handed to layer l (rows with
    -1 self-route) or None (every row self-routes); pred/pred_w [L, n, k]
    with pred[l+1] the prediction of head l (None: not checked); cur[l] /
    prev[l]: history one-hots of head l ([n, k] or None). rows: rows whose
    block outputs are computed (all when None). Returns (certified near ties,
    max per-layer rel-L2)."""
    L = len(ora)
    flips, worst = 0, 0.0
    for l in range(L):
        x_l = np.asarray(trace[l], dtype=np.float64)
        x_n = np.asarray(trace[l + 1] if l + 1 < L else x_out, dtype=np.float64)
        has_head = pred is not None and l + 1 < L
        f, e = layer_same_input_check(
            ora[l], x_l, mode, got_used=used[l], got_used_w=used_w[l], route_in=given[l],
            got_y=(x_n - x_l) if outputs else None,
            got_pred=pred[l + 1] if has_head else None, got_pred_w=pred_w[l + 1] if has_head else None,
            cur=None if cur is None else cur[l], prev=None if prev is None else prev[l], tol=tol, rows=rows,
            what=f"{what} layer {l}")
        flips += f
        worst = max(worst, e)
    return flips, worst


def oracle_stack_on_routing(ora, x, used, used_w, rows=None):
    """The oracle's stack output from x with every layer forced to the given
    routing (the routing the GPU used, each decision of which is checked
    separately)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    sel = list(range(x.shape[0])) if rows is None else list(rows)
    x = x[sel]
    for l, lw in enumerate(ora):
        route = (np.asarray(used[l])[sel].astype(np.int64), np.asarray(used_w[l])[sel].astype(np.float64))
        x, *_ = oracle.decode_layer(lw, x, route, None, fused_norm=True)
    return x


def stack_output_check(ora, x_in, x_out_gpu, used, used_w, tol=1e-2, rows=None):
    ref = oracle_stack_on_routing(ora, x_in, used, used_w, rows)
    got = np.atleast_2d(np.asarray(x_out_gpu, dtype=np.float64))
    if rows is not None:
        got = got[list(rows)]
    err = rel_l2_rows(got, ref)
    assert err <= tol, err
    return err

"""Conditioned layer inputs for parity checks -- TEST INFRASTRUCTURE.

Draws a workload's inputs with the seeded generator and then applies the
gap rule: any token whose 4th/5th (k-th/(k+1)-th) router-logit gap, computed
in float64 by the oracle from the bf16 inputs, is at most ``GAP`` gets its
activation row redrawn from the next counter block, until every row clears
it.  Exact top-k parity is only meaningful on such inputs.
"""
from __future__ import annotations

import numpy as np

from moe_inputs import synth
from moe_inputs.workloads import ZIPF_BETA, Workload

from .moe_oracle import route, topk_gap

GAP = 1e-3


def router_for(wl: Workload, layer: int = 0):
    seed = wl.seed + layer
    wr, br = synth.gen_router(seed, wl.E, wl.d)
    if wl.routing == "zipf":
        br = synth.zipf_router_bias(seed, wl.E, ZIPF_BETA)
    return wr, br


def make_inputs(wl: Workload, layer: int = 0, condition: bool = True, T: int | None = None,
                experts: bool = True):
    """Returns dict(x, router_w, router_b, [expert arrays], redraw)."""
    seed = wl.seed + layer
    T = wl.T if T is None else T
    wr, br = router_for(wl, layer)
    redraw: dict[int, int] = {}
    x = synth.gen_x(seed, T, wl.d)
    if condition and wl.k < wl.E:
        for _ in range(64):
            logits, _, _ = route(x, wr, br, wl.k)
            bad = np.nonzero(topk_gap(logits, wl.k) <= GAP)[0]
            if bad.size == 0:
                break
            for r in bad.tolist():
                redraw[r] = redraw.get(r, 0) + 1
            x = synth.gen_x(seed, T, wl.d, redraw)
        else:  # pragma: no cover
            raise RuntimeError("gap rule did not converge")
    out = dict(x=x, router_w=wr, router_b=br, redraw=redraw)
    if experts:
        out.update(synth.gen_experts(seed, wl.E, wl.d, wl.I))
    return out

"""Calibrates the Zipf router-bias strength of the 120b prefill workload.

Run as ``python -m oracle.zipf_beta``.  The router bias is
b(e) = -beta * ln(rank(e)); this script bisects beta until the
least-squares slope of log(load) against log(rank) over all experts is
-1.2 (Zipf exponent s = 1.2), using the oracle's own router and top-k on the
workload's seeded activations and router weight.  It prints the constant
that the workload table stores.
"""
from __future__ import annotations

import numpy as np

from moe_inputs import synth
from moe_inputs.workloads import WORKLOADS

from .moe_oracle import route


def load_slope(beta: float, wl, x, wr) -> tuple[float, np.ndarray, np.ndarray]:
    br = synth.zipf_router_bias(wl.seed, wl.E, beta)
    _, ids, _ = route(x, wr, br, wl.k)
    load = np.bincount(ids.reshape(-1), minlength=wl.E).astype(np.float64)
    rank = np.rint(np.exp(-br.astype(np.float64) / beta)) if beta > 0 else np.arange(1, wl.E + 1)
    lr, ll = np.log(rank), np.log(np.maximum(load, 0.5))
    slope = np.polyfit(lr, ll, 1)[0]
    return slope, load, rank


def main(target: float = -1.2) -> float:
    wl = WORKLOADS["120b_prefill_zipf"]
    x = synth.gen_x(wl.seed, wl.T, wl.d)
    wr, _ = synth.gen_router(wl.seed, wl.E, wl.d)
    lo, hi = 0.05, 8.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        s, load, _ = load_slope(mid, wl, x, wr)
        if s > target:
            lo = mid
        else:
            hi = mid
    beta = 0.5 * (lo + hi)
    s, load, rank = load_slope(beta, wl, x, wr)
    order = np.argsort(rank)
    print(f"beta={beta:.6f} slope={s:.4f} max_load={load.max():.0f} min_load={load.min():.0f}")
    print("loads by rank:", load[order][:16].astype(int).tolist(), "...", load[order][-8:].astype(int).tolist())
    return beta


if __name__ == "__main__":
    main()

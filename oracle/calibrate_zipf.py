"""Calibrate the decode workload's Zipf-skewed router bias with the CPU oracle's router.

The workload asks for a router bias "drawn so expert popularity is Zipf(s = 1.1)".  Reading:
a seeded permutation gives expert i a popularity rank r_i and b_i = -beta * ln(r_i) (shifted
to zero mean); beta is chosen by bisection so that the least-squares slope of
log(load) against log(rank), over 8 calibration batches of 256 tokens (seeded batches
disjoint from the run's), is -1.1.  Writes sparse_moe_layer_sigmoid_amd/zipf_bias.json.

    python -m oracle.calibrate_zipf
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import moe_oracle as O  # noqa: E402
from sparse_moe_layer_sigmoid_amd import inputs as I  # noqa: E402

TARGET = -1.1
CAL_STEPS = range(1000, 1008)


def slope(beta, cfg, xs, wr):
    b = I.zipf_bias(cfg, beta).numpy()
    load = np.zeros(cfg.n_experts)
    for x in xs:
        r = O.route(x, wr, b, cfg.top_k)
        load += O.expert_counts(r["idx"], cfg.n_experts)
    rank = np.argsort(np.argsort(-load, kind="stable"), kind="stable") + 1
    ok = load > 0
    A = np.vstack([np.log(rank[ok]), np.ones(ok.sum())]).T
    return float(np.linalg.lstsq(A, np.log(load[ok]), rcond=None)[0][0]), load


def main():
    cfg = I.V3_DECODE
    wr = I.gen_router(cfg).double().numpy()
    xs = [I.gen_x(cfg, step=s).double().numpy() for s in CAL_STEPS]
    lo, hi = 0.0, 1.0
    s_hi, _ = slope(hi, cfg, xs, wr)
    while s_hi > TARGET:
        hi *= 2
        s_hi, _ = slope(hi, cfg, xs, wr)
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        s, _ = slope(mid, cfg, xs, wr)
        if s > TARGET:
            lo = mid
        else:
            hi = mid
    beta = 0.5 * (lo + hi)
    s, load = slope(beta, cfg, xs, wr)
    rec = {"beta": beta, "fitted_slope": s, "target_slope": TARGET,
           "calibration": f"{len(CAL_STEPS)} batches of T={cfg.T} (x steps {CAL_STEPS.start}..{CAL_STEPS.stop - 1}), "
                          "oracle router, zero-mean b_i = -beta ln(rank_i)",
           "max_over_mean_load": float(load.max() / load.mean()),
           "active_experts_mean_per_batch": float((load > 0).sum())}
    out = os.path.join(ROOT, "sparse_moe_layer_sigmoid_amd", "zipf_bias.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()

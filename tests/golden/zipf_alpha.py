"""Calibrate the Zipf log-bias factor alpha of the skewed-routing workloads.

For each workload with a Zipf expert bias, find by bisection an alpha for which the
hottest expert's routed load is 3.8x-4.2x the mean load T*k/E on the fixed seeds.
Routing uses the CPU oracle only.  Prints the values stored in workloads/__init__.py.

    python tests/golden/zipf_alpha.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def load_ratio(w, alpha):
    ids, _ = oracle.route(workloads.router_logits(w, alpha=alpha), w.k)
    counts = np.bincount(ids.ravel(), minlength=w.E)
    return counts.max() / (w.T * w.k / w.E)


def calibrate(w, lo=0.0, hi=1.0, target=4.0, iters=40):
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if load_ratio(w, mid) < target:
            lo = mid
        else:
            hi = mid
    return round(0.5 * (lo + hi), 4)


if __name__ == "__main__":
    for w in (workloads.AGGREGATED, workloads.FP8_DSV3):
        a = calibrate(w)
        print(f"{w.name}: alpha={a} max/mean={load_ratio(w, a):.3f}")

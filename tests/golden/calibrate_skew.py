"""Calibrates the temperature of the skewed (Zipf) router bias.

The skewed fp8 workload asks for a hottest expert with about 10x the mean
load and at least 4 experts with no token.  This script bisects the
temperature tau of the bias b_e = tau * log p_rank(e) until the oracle's
top-k routing gives max/mean = 10, and prints the value that the input
generator uses (SKEW_TAU).  It calls only the oracle and the input generator.

    python tests/golden/calibrate_skew.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

from combine_top_route_amd import synthetic as S  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402


def load_stats(tau: float, seed: int = 0):
    wl = S.WORKLOADS["fp8_skew"]
    seq = S._streams(seed)["bias"]
    b = S.zipf_bias(wl.E, seq, tau)
    lg = S.make_logits(wl, seed=seed, bias=b).double().numpy()
    ids = O.topk_select(lg, wl.k)
    c, _ = O.expert_counts_fast(ids, wl.E)
    return c.max() / c.mean(), int((c == 0).sum()), int(c[c > 0].min())


def main():
    lo, hi = 0.1, 1.0
    for _ in range(12):
        mid = 0.5 * (lo + hi)
        r, _, _ = load_stats(mid)
        if r < 10.0:
            lo = mid
        else:
            hi = mid
    tau = round(0.5 * (lo + hi), 2)
    for seed in (0, 1, 2):
        print("seed", seed, "tau", tau, "max/mean, empty, min nonempty:", load_stats(tau, seed))


if __name__ == "__main__":
    main()

"""Calibrate the draft-noise std-dev of a recipe to a target acceptance rate.

alpha = sum_x min(p(x), q(x)) is the probability that the accept rule accepts a
draft token drawn from q (the exactness rule of the EAGLE lesson accepts x with
probability min(1, p(x)/q(x))).  The distributions come from the oracle's
softmax; the rows are drawn exactly as the generators draw them (bf16 rounded).
Prints the bisection result; the generators hold the chosen constants.

  python -m workloads.tune_sigma
"""

import numpy as np

import workloads
from oracle.accept import softmax_T


def mean_alpha(sigma, V, std, T, rows, seed):
    rng = np.random.default_rng(seed)
    a = []
    for _ in range(rows):
        zt = workloads.round_bf16(rng.normal(0, std, V).astype(np.float32))
        zd = workloads.round_bf16(workloads.draft_from_target(rng, zt, sigma))
        a.append(np.minimum(softmax_T(zt, T), softmax_T(zd, T)).sum())
    return float(np.mean(a))


def tune(target, V, std, T, rows=64, seed=0):
    lo, hi = 0.0, 4.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if mean_alpha(mid, V, std, T, rows, seed) > target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


if __name__ == "__main__":
    for name, target, V, T in [("chain", 0.80, 32000, 1.0), ("eagle", 0.80, 128256, 0.7),
                               ("ptd", 0.75, 128256, 1.0)]:
        s = tune(target, V, 3.0, T)
        print(f"{name}: sigma = {s:.4f}  (alpha at that sigma on fresh rows: "
              f"{mean_alpha(s, V, 3.0, T, 64, 1):.4f})")

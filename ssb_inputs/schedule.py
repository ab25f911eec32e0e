"""Target lengths and planted-draft accept lengths.

Lengths: lognormal with sigma 0.8 and mu = ln(mean) - sigma^2/2, so the mean
equals the pages' per-type mean output length (text 73, table 872 in
Table 4; the formula mean of 200 is this workload's own choice), rounded and
clamped to [1, cap].

Planted accept lengths: per round G ~ Geometric(p) on {0, 1, ...} (mean
(1-p)/p = 19 at p = 1/20, matching the blog's figure of about 19 consecutive
matches per round), A* = min(G, B); with probability ``full_accept_p`` a round
is forced to A* = B.  Only the draws live here; how a draft is built from
them is the decoding harness's business.
"""

import numpy as np

SIGMA = 0.8


def region_kinds(wl):
    kinds = []
    for kind, count, _mean, _cap in wl.length_mix:
        kinds += [kind] * count
    return kinds


def target_lengths(wl):
    out = []
    idx = 0
    for _kind, count, mean, cap in wl.length_mix:
        mu = np.log(mean) - SIGMA ** 2 / 2.0
        for _ in range(count):
            rng = np.random.default_rng([wl.wid, 2, idx])
            x = rng.lognormal(mean=mu, sigma=SIGMA)
            out.append(int(min(max(int(round(x)), 1), cap)))
            idx += 1
    return out


def plant_accept_lengths(wid, index, n_rounds, B, p, full_accept_p=0.0):
    """A* for each of ``n_rounds`` rounds of region ``index``."""
    rng = np.random.default_rng([wid, 3, index])
    g = rng.geometric(p, size=n_rounds) - 1        # numpy's geometric starts at 1
    a = np.minimum(g, B)
    if full_accept_p > 0.0:
        frng = np.random.default_rng([wid, 4, index])
        force = frng.random(n_rounds) < full_accept_p
        a = np.where(force, B, a)
    return a.astype(np.int64)

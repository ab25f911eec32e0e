"""A GPU round against the oracle's round from the same state (shared by the GPU tests).

The round (GravityOCR review, section 3.2 and Appendix B.2): a draft forward over [x0, M x B],
a causal verify forward over [a0, d_1..d_B], A = longest prefix with d_j = a_j, commit a0,
d_1..d_A, a_{A+1}.  Planted drafts replace d before verification on both sides.

What is compared:
  * draft logits, every row, within ``tol``;
  * verify row k sees a0, d_1..d_k, so its logits are comparable while both sides fed the same
    tokens; an unplanted draft token may differ only at an oracle near-tie, and then every later
    verify row differs too;
  * every argmax decision whose oracle top-2 margin exceeds twice the logit error measured on
    the rows compared (a flip needs a smaller margin);
  * A, the committed tokens and the new state exactly, unless a decision on the accepted path is
    that close.
"""

import numpy as np

from oracle import spec_round
from oracle.model import argmax_excluding


def _am(logits, mask_id):
    return argmax_excluding(np.asarray(logits, dtype=np.float64), mask_id)


def check_round(cfg, orc, st, B, plant, committed, A, dl, vl, tol, budget=None):
    """``st`` is the oracle state before the round (advanced in place); ``dl``/``vl`` the GPU's
    draft and verify logits as numpy arrays.  Returns a dict of what was compared."""
    r = spec_round(orc, st, B, planted=plant, budget=budget, keep_logits=True)
    derr = float(np.abs(dl - r.draft_logits).max())
    assert derr < tol, (derr, tol)
    g_in = [_am(dl[0], cfg.mask_id)[0]] + [plant[j - 1] if plant[j - 1] >= 0 else _am(dl[j], cfg.mask_id)[0]
                                           for j in range(1, B + 1)]
    o_in = [r.a0] + list(r.d)
    same = 0
    while same < B + 1 and g_in[same] == o_in[same]:
        same += 1
    for j in range(same, min(same + 1, B + 1)):
        _, t1, t2 = _am(r.draft_logits[j], cfg.mask_id)
        assert t1 - t2 <= 2 * derr, f"draft row {j} differs away from a near-tie"
    verr = float(np.abs(vl[:same] - r.verify_logits[:same]).max()) if same else 0.0
    assert verr < tol, (verr, tol)
    close = 2 * max(derr, verr)
    tie = False
    for j in range(B + 1):
        t, t1, t2 = _am(r.draft_logits[j], cfg.mask_id)
        if t1 - t2 > close:
            assert _am(dl[j], cfg.mask_id)[0] == t, f"draft row {j}"
        elif j == 0:
            tie = True
    for j in range(B + 1):
        if j >= same:
            tie = tie or j <= r.A
            break
        t, t1, t2 = _am(r.verify_logits[j], cfg.mask_id)
        if t1 - t2 > close:
            assert _am(vl[j], cfg.mask_id)[0] == t, f"verify row {j}"
        elif j <= r.A:
            tie = True
    if not tie:
        assert A == r.A, (A, r.A)
        assert committed == r.committed, (committed, r.committed)
    return dict(oracle=r, derr=derr, verr=verr, same_rows=same, tie=tie)

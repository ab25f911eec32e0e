"""Shared checks of stochastic-round GPU tests (not a test module).

A GPU stochastic round is replayed in float64 from the GPU's own logits and
the uniforms it was given: every draw must be a valid inverse-CDF draw and
every acceptance decision must follow the rule, except where the float64
replay puts the uniform within ``tol`` (relative) of a decision boundary,
where either outcome is accepted.
"""

import numpy as np

from oracle.stochastic import probs, residual, sample_index


def draw_ok(w, u, v, tol):
    """v is the inverse-CDF draw of weights w at u, up to tol of the total at a boundary."""
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    tot = c[-1]
    if not (0 <= v < len(w)) or w[v] <= 0:
        return False
    lo = c[v - 1] if v else 0.0
    x = u * tot
    return lo - tol * tot <= x < c[v] + tol * tot


def draw_safe(w, u, tol):
    """The draw at u is unambiguous: u * total is farther than tol from every boundary."""
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    x = u * c[-1]
    return np.abs(c - x).min() > tol * c[-1]


def replay_round(dl, vl, u, B, T, mask_id, eos_id, committed, A, tol=1e-4):
    """Checks one GPU stochastic round; returns the number of decisions found ambiguous."""
    u = np.asarray(u, dtype=np.float64)
    u_a0, u_d, u_acc, u_t = u[0], u[1: B + 1], u[B + 1: 2 * B + 1], u[2 * B + 1]
    q = [probs(dl[j], mask_id, T) for j in range(B + 1)]
    p = [probs(vl[j], mask_id, T) for j in range(B + 1)]
    amb = 0
    assert draw_ok(q[0], u_a0, committed[0], tol)
    full = [committed[0]]
    for j in range(1, B + 1):
        if j <= A and j < len(committed):
            d = committed[j]
            assert draw_ok(q[j], u_d[j - 1], d, tol), f"d_{j}"
            lhs, rhs = u_acc[j - 1] * q[j][d], p[j - 1][d]
            if abs(lhs - rhs) > tol * max(lhs, rhs, 1e-300):
                assert lhs < rhs, f"d_{j} accepted against the rule"
            else:
                amb += 1
    if A < B:
        # the rejected draft d_{A+1}, drawn again in float64
        j = A + 1
        if draw_safe(q[j], u_d[j - 1], tol):
            d = sample_index(q[j], u_d[j - 1])
            lhs, rhs = u_acc[j - 1] * q[j][d], p[j - 1][d]
            if abs(lhs - rhs) > tol * max(lhs, rhs, 1e-300):
                assert not lhs < rhs, f"d_{j} rejected against the rule"
            else:
                amb += 1
        else:
            amb += 1
        w = residual(p[A], q[A + 1])
        if w.sum() <= 0:
            w = p[A]
    else:
        w = p[B]
    if len(committed) == A + 2:
        assert draw_ok(w, u_t, committed[A + 1], tol), "next token"
    return amb

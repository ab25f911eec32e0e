"""Stochastic self-speculative decoding (test infrastructure only).

The sampling variant of the round: drafts are sampled from the diffusion
path's distributions and verified with the standard speculative
acceptance-rejection rule, which leaves the output distributed exactly as
sampling from the AR path (GravityOCR review, section 2 "Speculative
Decoding"; Trillion Labs blog, the passage on the speculative rejection rule
preserving the distribution when sampling).  The pages name the rule and its
property only; its steps below are the published standard rule (Leviathan
et al. 2023, "Fast Inference from Transformers via Speculative Decoding";
Chen et al. 2023, "Accelerating Large Language Model Decoding with
Speculative Sampling").

Round over state (p, x0), block B, temperature T, uniforms u in [0, 1):
* draft forward [x0, [M] x B] as in the greedy round; every row's
  distribution is softmax(logits / T) over the vocabulary without [M].
  Row 0 is causal, so it is the AR distribution of position p+1:
  a0 ~ row 0.  d_j ~ q_j = row j, each drawn independently;
* verify forward [a0, d_1..d_B] as in the greedy round; verify row j-1 is
  the AR distribution p_j of d_j's position, row B that of the bonus;
* d_j is accepted while u_acc[j] * q_j(d_j) < p_j(d_j) (probability
  min(1, p_j(d_j) / q_j(d_j))); A = number accepted before the first
  rejection;
* if A < B, the next token t is drawn from the residual distribution
  proportional to max(0, p_{A+1} - q_{A+1}); if A = B, from p_{B+1};
* commit a0, d_1..d_A, t (A + 2 tokens), cut after EOS and at the budget;
  t becomes the next boundary; the rest is rolled back as in the greedy
  round.

Sampling from a distribution w with a uniform u is the inverse CDF over the
vocabulary in id order: the smallest id v with w_0 + ... + w_v > u * sum(w).

Uniform numbers are inputs (one round uses 2B + 2: u_a0, u_d[1..B],
u_acc[1..B], u_t), so the oracle and the GPU draw the same sample.

Readings (also in the design notes): the temperature divides the logits of
both paths alike; [M] has probability zero in every distribution; a0 is
drawn from the draft's causal row (the same distribution the verifier would
use for that position, so it needs no test).
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .decode import commit_tokens, draft_visibility, verify_visibility


def probs(logits, mask_id, temperature):
    """softmax(logits / T) over the vocabulary with [M] removed (probability 0)."""
    if not temperature > 0:
        raise ValueError("temperature must be > 0")
    z = np.array(logits, dtype=np.float64, copy=True) / temperature
    z[mask_id] = -np.inf
    e = np.exp(z - z.max())
    return e / e.sum()


def sample_index(w, u):
    """Inverse-CDF draw: the smallest v with w[0] + ... + w[v] > u * sum(w)."""
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    v = int(np.searchsorted(c, u * c[-1], side="right"))
    # rounding can leave u * total at the last partial sum: take the last positive weight
    return min(v, int(np.flatnonzero(w > 0)[-1]))


def residual(p, q):
    """max(0, p - q); all zeros only when p == q."""
    return np.maximum(np.asarray(p, dtype=np.float64) - np.asarray(q, dtype=np.float64), 0.0)


def accept_draft(p_d, q_d, u):
    """Standard test: accept with probability min(1, p/q), written u * q < p."""
    return u * q_d < p_d


def split_uniforms(u, B):
    u = np.asarray(u, dtype=np.float64)
    if u.shape != (2 * B + 2,):
        raise ValueError("a round needs 2B + 2 uniforms")
    return u[0], u[1: B + 1], u[B + 1: 2 * B + 1], u[2 * B + 1]


@dataclass
class SampleRoundResult:
    committed: List[int]
    A: int
    a0: int
    d: List[int]
    t: int
    draft_logits: Optional[np.ndarray] = None
    verify_logits: Optional[np.ndarray] = None


def spec_round_sample(model, state, B, u, temperature=1.0, budget=None, keep_logits=False):
    cfg = model.cfg
    u_a0, u_d, u_acc, u_t = split_uniforms(u, B)
    p, x0, cache = state.n, state.x0, state.cache

    h = model.embed_tokens([x0] + [cfg.mask_id] * B)
    dl = model.forward(cache, h, p + np.arange(B + 1), draft_visibility(p, B))
    q = [probs(dl[j], cfg.mask_id, temperature) for j in range(B + 1)]
    a0 = sample_index(q[0], u_a0)
    d = [sample_index(q[j], u_d[j - 1]) for j in range(1, B + 1)]

    h = model.embed_tokens([a0] + d)
    vl = model.forward(cache, h, p + 1 + np.arange(B + 1), verify_visibility(p, B))
    pv = [probs(vl[j], cfg.mask_id, temperature) for j in range(B + 1)]

    A = 0
    while A < B and accept_draft(pv[A][d[A]], q[A + 1][d[A]], u_acc[A]):
        A += 1
    if A < B:
        r = residual(pv[A], q[A + 1])
        t = sample_index(r if r.sum() > 0 else pv[A], u_t)
    else:
        t = sample_index(pv[B], u_t)

    a = list(d[:A]) + [t]
    committed = commit_tokens(a0, a, A, cfg.eos_id, B + 2 if budget is None else budget)
    state.n = p + A + 2
    state.x0 = t
    cache.release_from(state.n)
    res = SampleRoundResult(committed=committed, A=A, a0=a0, d=d, t=t)
    if keep_logits:
        res.draft_logits, res.verify_logits = dl, vl
    return res


def ar_step_sample(model, state, u, temperature=1.0):
    """One AR sampling step: feed x0 causally, draw the next token with u."""
    from .decode import causal_visibility
    p = state.n
    logits = model.forward(state.cache, model.embed_tokens([state.x0]), [p], causal_visibility([p], p + 1))
    y = sample_index(probs(logits[0], model.cfg.mask_id, temperature), u)
    state.n = p + 1
    state.x0 = y
    return y


def prefill_sample(model, prefix_emb, max_positions, u, temperature=1.0):
    """Prefill, with y1 drawn from the last row's distribution."""
    from .decode import DecodeState, causal_visibility
    P = prefix_emb.shape[0]
    cache = model.new_cache(max_positions)
    pos = np.arange(P)
    logits = model.forward(cache, prefix_emb, pos, causal_visibility(pos, P))
    y1 = sample_index(probs(logits[P - 1], model.cfg.mask_id, temperature), u)
    return DecodeState(cache=cache, n=P, x0=y1), y1


def spec_decode_sample(model, prefix_emb, B, max_len, uniforms, temperature=1.0, max_positions=None,
                       rounds_out=None):
    """Stochastic self-speculative decoding until EOS or ``max_len`` tokens.

    ``uniforms``: [n_rounds + 1, 2B + 2]; row 0's first entry draws y1,
    row k (k >= 1) drives round k.
    """
    cfg = model.cfg
    if max_len <= 0:
        return []
    P = prefix_emb.shape[0]
    state, y1 = prefill_sample(model, prefix_emb, max_positions or P + max_len + B + 3, uniforms[0][0],
                               temperature)
    out = [y1]
    k = 1
    while out[-1] != cfg.eos_id and len(out) < max_len:
        r = spec_round_sample(model, state, B, uniforms[k], temperature, budget=max_len - len(out))
        if rounds_out is not None:
            rounds_out.append(r)
        out += r.committed
        k += 1
    return out

"""Prefill, AR greedy decoding and the self-speculative round (test infrastructure only).

Round semantics follow the GravityOCR review, section 3.2 "Self-Speculative
Decoding" and Appendix B.2 "Self-Speculative Decoding and KV-Cache Update",
and the velog review's step-by-step round description ("inference: one
draft forward + one verify forward"):

* state: the cache holds the causal state of every committed token except
  the last one, the boundary x0, which has not been fed yet;
* draft: [x0, M x B] in one forward; the boundary row is causal and
  predicts a0, the mask rows see the cache and the whole window and
  propose d1..dB in one shot;
* verify: [a0, d1..dB] causally, giving a1..a(B+1); it reuses the mask
  slots and overwrites their state with causal state;
* accept: A = longest prefix with d_j = a_j; commit a0, d1..dA, a(A+1);
  release the rejected suffix; a(A+1) becomes the next boundary.

Readings where the pages are silent (each also listed in the design notes):
shift-by-one prediction (row at position i predicts position i+1, review
section 3.1 states this convention for both paths); masks sit at positions
p+1..p+B; the boundary row does not see the masks; greedy ties go to the
lowest id; [M] is never an output; the first EOS is committed and ends the
output; ``max_len`` caps the total output length.
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .model import argmax_excluding


@dataclass
class DecodeState:
    cache: object
    n: int          # committed tokens whose KV is in the cache = position of x0
    x0: int         # boundary token: committed, not yet in the cache


@dataclass
class RoundResult:
    committed: List[int]
    A: int
    a0: int
    d: List[int]            # d_1..d_B (after planting)
    a: List[int]            # a_1..a_{B+1}
    draft_logits: Optional[np.ndarray] = None
    verify_logits: Optional[np.ndarray] = None
    margins: List[float] = field(default_factory=list)


def causal_visibility(positions, n_keys):
    """AR / prefill rule: a row at position t sees keys 0..t."""
    pos = np.asarray(positions)[:, None]
    return np.arange(n_keys)[None, :] <= pos


def draft_visibility(p, B):
    """Draft forward over [x0 at p, masks at p+1..p+B] (review section 3.2).

    The boundary row keeps causal attention: keys 0..p.  Every mask row
    attends causally to the cache and bidirectionally inside the window:
    keys 0..p+B.
    """
    n_keys = p + B + 1
    vis = np.zeros((B + 1, n_keys), dtype=bool)
    vis[0, : p + 1] = True
    vis[1:, : p + B + 1] = True
    return vis


def verify_visibility(p, B):
    """Verify forward over [a0, d1..dB] at positions p+1..p+B+1, causal."""
    return causal_visibility(p + 1 + np.arange(B + 1), p + B + 2)


def accept_length(d, a):
    """A = max{j <= B : d_i = a_i for all i <= j} (review section 3.2).

    ``d`` holds d_1..d_B and ``a`` holds a_1..a_B (a_{B+1} unused here).
    """
    A = 0
    while A < len(d) and d[A] == a[A]:
        A += 1
    return A


def commit_tokens(a0, a, A, eos_id, budget):
    """Committed list a0, a_1..a_{A+1}, cut after the first EOS and at ``budget``.

    Since d_j = a_j for j <= A, this is a0, d_1..d_A, a_{A+1}.  A stop
    condition commits up to that point only (review Appendix B.2); EOS
    itself is committed (Appendix F colours EOS with its round).
    """
    out = [a0] + list(a[: A + 1])
    if eos_id in out:
        out = out[: out.index(eos_id) + 1]
    return out[: max(budget, 0)]


def _am(model, logits):
    return argmax_excluding(logits, model.cfg.mask_id)


def prefill(model, prefix_emb, max_positions):
    """Causal forward over the P prefix rows; y1 = argmax of row P-1."""
    P = prefix_emb.shape[0]
    cache = model.new_cache(max_positions)
    pos = np.arange(P)
    logits = model.forward(cache, prefix_emb, pos, causal_visibility(pos, P))
    y1, t1, t2 = _am(model, logits[P - 1])
    return DecodeState(cache=cache, n=P, x0=y1), y1, t1 - t2


def ar_step(model, state):
    """Feed x0 at position n causally; the argmax is the next token."""
    p = state.n
    h = model.embed_tokens([state.x0])
    logits = model.forward(state.cache, h, [p], causal_visibility([p], p + 1))
    y, t1, t2 = _am(model, logits[0])
    state.n = p + 1
    state.x0 = y
    return y, t1 - t2


def ar_decode(model, prefix_emb, max_len, max_positions=None):
    """Plain greedy AR decoding (review section 2, task formulation)."""
    cfg = model.cfg
    if max_len <= 0:
        return []
    P = prefix_emb.shape[0]
    state, y1, _ = prefill(model, prefix_emb, max_positions or P + max_len + 2)
    out = [y1]
    while out[-1] != cfg.eos_id and len(out) < max_len:
        y, _ = ar_step(model, state)
        out.append(y)
    return out


def spec_round(model, state, B, planted=None, budget=None, keep_logits=False):
    """One draft -> verify -> accept -> rollback round.

    ``planted`` (optional, length B, -1 = keep) replaces draft tokens before
    verification; it is a test hook that does not change the rule.
    """
    cfg = model.cfg
    p, x0 = state.n, state.x0
    cache = state.cache

    # (1) draft forward over [x0, [M] x B] at positions p..p+B
    h = model.embed_tokens([x0] + [cfg.mask_id] * B)
    dl = model.forward(cache, h, p + np.arange(B + 1), draft_visibility(p, B))
    a0 = _am(model, dl[0])[0]
    d = [_am(model, dl[j])[0] for j in range(1, B + 1)]
    if planted is not None:
        d = [int(t) if int(t) >= 0 else dj for t, dj in zip(planted, d)]

    # (2) verify forward over [a0, d_1..d_B] at positions p+1..p+B+1, causal;
    #     overwrites slots p+1..p+B and writes slot p+B+1
    h = model.embed_tokens([a0] + d)
    vl = model.forward(cache, h, p + 1 + np.arange(B + 1), verify_visibility(p, B))
    am = [_am(model, vl[j]) for j in range(B + 1)]
    a = [t for t, _, _ in am]                   # a_1..a_{B+1}

    # (3) accept
    A = accept_length(d, a[:B])
    committed = commit_tokens(a0, a, A, cfg.eos_id, B + 2 if budget is None else budget)

    # (4) commit + rollback: x0, a0, d_1..d_A are now causal state in slots
    #     p..p+A+1; a_{A+1} is the next boundary; the rest is released
    state.n = p + A + 2
    state.x0 = a[A]
    cache.release_from(state.n)

    r = RoundResult(committed=committed, A=A, a0=a0, d=d, a=a,
                    margins=[t1 - t2 for _, t1, t2 in am])
    if keep_logits:
        r.draft_logits, r.verify_logits = dl, vl
    return r


def build_plant(cont, c, A_star, B, vocab, mask_id):
    """Planted draft for a round starting after output token y_c (1-based).

    cont = [y_1, y_2, ...] is the AR greedy output of the same implementation.
    d_j = y_{c+1+j} for j <= A_star; if A_star < B, d_{A_star+1} is a token
    different from y_{c+A_star+2} and from [M]; the rest stays -1 (keep the
    draft's own proposal).  Entries past the end of ``cont`` stay -1.
    """
    plant = [-1] * B
    for j in range(1, B + 1):
        idx = c + j          # 0-based index of y_{c+1+j}
        if idx >= len(cont):
            break
        if j <= A_star:
            plant[j - 1] = int(cont[idx])
        elif j == A_star + 1:
            plant[j - 1] = int((cont[idx] + 1) % (vocab - 1))
            break
    return plant


def spec_decode(model, prefix_emb, B, max_len, plant_fn=None, max_positions=None,
                rounds_out=None):
    """Greedy self-speculative decoding until EOS or ``max_len`` tokens.

    ``plant_fn(round_index, c)`` may return a planted draft (see build_plant).
    ``rounds_out``, if a list, receives one RoundResult per round.
    """
    cfg = model.cfg
    if max_len <= 0:
        return []
    P = prefix_emb.shape[0]
    state, y1, _ = prefill(model, prefix_emb, max_positions or P + max_len + B + 3)
    out = [y1]
    k = 0
    while out[-1] != cfg.eos_id and len(out) < max_len:
        planted = plant_fn(k, len(out)) if plant_fn is not None else None
        r = spec_round(model, state, B, planted=planted, budget=max_len - len(out))
        if rounds_out is not None:
            rounds_out.append(r)
        out += r.committed
        k += 1
    return out


def tpf(rounds):
    """Tokens per forward (review section 4.1, eq. 5 as described in prose).

    Committed output tokens over draft + verify forwards; prefill and its
    token y1 are excluded.  Also returns the mean accepted draft tokens A
    (boundary prediction and the verifier's extra token not counted).
    """
    if not rounds:
        return 0.0, 0.0
    committed = sum(len(r.committed) for r in rounds)
    return committed / (2.0 * len(rounds)), float(np.mean([r.A for r in rounds]))


def teacher_forced_argmax(model, prefix_emb, tokens):
    """Causal forward over prefix + E[tokens[:-1]]; per-position argmax and margin.

    Entry t is the greedy prediction for tokens[t] given prefix and
    tokens[:t]; used to judge a decoded sequence position by position.
    """
    P = prefix_emb.shape[0]
    n = len(tokens)
    h = np.concatenate([np.asarray(prefix_emb, dtype=model.dtype),
                        model.embed_tokens(tokens[:-1]) if n > 1 else
                        np.zeros((0, model.cfg.hidden), model.dtype)], axis=0)
    cache = model.new_cache(P + n)
    pos = np.arange(P + n - 1)
    logits = model.forward(cache, h, pos, causal_visibility(pos, P + n - 1))
    res = [_am(model, logits[P - 1 + t]) for t in range(n)]
    return [r[0] for r in res], [r[1] - r[2] for r in res]

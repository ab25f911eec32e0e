"""Direct block-diffusion decoding (test infrastructure only).

The decoding mode the pages compare self-speculation against: the block is
filled by the diffusion path alone, several positions per forward, with no
AR verification (GravityOCR review, section 2 "Block Diffusion" and
Appendix B.1 "Direct Block-Diffusion Decoding"; Trillion Labs blog, the
"confidence threshold" glossary entry and Figure 2).

* The current block starts as all [M].  Each denoising step is one forward
  over [x0, s_1..s_B] in draft mode (the boundary row causal, the block rows
  see the cache and the whole window); s_j is the committed token of
  position j or [M].
* Every still-masked position whose confidence reaches the threshold tau_c
  is committed; if none reaches it, only the single most confident one is.
  Committed positions keep their token; the rest are predicted again.
* A completed block needs a separate cache-write forward (it verifies or
  replaces nothing); the finished block's last token becomes the next
  boundary.
* A completed block that holds EOS ends the output at its first EOS.
* Forward accounting (review, Appendix C): only the forwards that commit
  tokens count toward tokens per forward; prefill and the cache-write
  forwards do not.

Readings where the pages are silent (each also listed in the design notes):
* shift-by-one prediction as in the self-speculative draft: the token of
  block position j (absolute position p + j) is read from window row j - 1,
  so a block holds B tokens and row B's prediction is unused;
* confidence = softmax probability of the greedy token, over the vocabulary
  without [M] (the [M] row is input-only, so it is not in the output
  distribution);
* "reaches the threshold" is >= (Figure 2 of the blog shows a token of
  confidence .70 committed at tau_c = 0.7);
* the most confident fallback breaks ties by the lowest position;
* the cache-write forward is causal over s_1..s_{B-1} at positions
  p+1..p+B-1: with x0 already causal in the cache after the steps, that
  leaves every committed token but the new boundary s_B in the cache, the
  same state invariant as the self-speculative round (Appendix B.2);
* ``max_len`` caps the total output length, as for the other decoders.

The multi-step draft schedule of the self-speculative round (blog, the
draft-schedule passage; review, Appendix D) uses the same denoising steps
as its drafter.  Readings: a schedule of S steps runs at most S draft
forwards, the last one committing every slot still open (S = 1 is the
one-shot draft); slot i holds the prediction of row i - 1 (a0 for i = 1);
d_B, which has no slot, is row B's prediction in the last draft forward.
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .decode import (accept_length, causal_visibility, commit_tokens, draft_visibility, prefill,
                     verify_visibility)
from .model import argmax_excluding


def confidence(logits, mask_id):
    """Greedy token and its softmax probability, [M] excluded.

    Returns (token, p) with p = exp(z_tok) / sum_{v != [M]} exp(z_v); the
    token is the lowest id among the maxima.
    """
    z = np.array(logits, dtype=np.float64, copy=True)
    z[mask_id] = -np.inf
    tok = int(np.argmax(z))
    e = np.exp(z - z[tok])
    return tok, float(1.0 / e.sum())


def select_positions(undecided, conf, tau):
    """Positions a denoising step commits (blog, "confidence threshold").

    Every undecided position with conf >= tau; if there is none, the single
    undecided position of largest conf (lowest position on ties).
    """
    cand = [j for j, u in enumerate(undecided) if u]
    if not cand:
        return []
    hit = [j for j in cand if conf[j] >= tau]
    if hit:
        return hit
    best = cand[0]
    for j in cand[1:]:
        if conf[j] > conf[best]:
            best = j
    return [best]


@dataclass
class BlockResult:
    tokens: List[int]                   # s_1..s_B
    steps: int                          # committing forwards of the block
    step_of: List[int]                  # step (0-based) at which each position was committed
    step_logits: List[np.ndarray] = field(default_factory=list)   # [B+1, vocab] per step
    step_conf: List[List[float]] = field(default_factory=list)    # conf of rows 0..B-1 per step
    step_tok: List[List[int]] = field(default_factory=list)       # greedy token of rows 0..B-1


def dd_fill(model, state, B, tau, keep_logits=False):
    """Denoising steps of one block of B positions after the boundary.

    The state's cache holds the window's draft-mode KV afterwards; the
    caller either writes the block's causal state (``dd_cache_write``) or
    ends the output (``dd_release``).
    """
    cfg = model.cfg
    if B < 1:
        raise ValueError("a direct-diffusion block needs B >= 1")
    p, x0, cache = state.n, state.x0, state.cache
    s = [cfg.mask_id] * B
    step_of = [-1] * B
    res = BlockResult(tokens=s, steps=0, step_of=step_of)
    while cfg.mask_id in s:
        h = model.embed_tokens([x0] + s)
        logits = model.forward(cache, h, p + np.arange(B + 1), draft_visibility(p, B))
        tc = [confidence(logits[j], cfg.mask_id) for j in range(B)]   # row j -> position j + 1
        conf = [c for _, c in tc]
        for j in select_positions([t == cfg.mask_id for t in s], conf, tau):
            s[j] = tc[j][0]
            step_of[j] = res.steps
        if keep_logits:
            res.step_logits.append(logits)
        res.step_conf.append(conf)
        res.step_tok.append([t for t, _ in tc])
        res.steps += 1
    return res


def dd_cache_write(model, state, tokens):
    """Cache-write forward of a completed block (review, Appendix B.1).

    Causal over s_1..s_{B-1} at positions p+1..p+B-1 (x0 at p is already
    causal state), then the state advances to (p + B, s_B).
    """
    B = len(tokens)
    p = state.n
    if B > 1:
        pos = p + 1 + np.arange(B - 1)
        model.forward(state.cache, model.embed_tokens(tokens[: B - 1]), pos, causal_visibility(pos, p + B))
    state.n = p + B
    state.x0 = tokens[B - 1]
    state.cache.release_from(state.n)


def dd_release(state):
    """End of output: the window's draft-mode slots are dropped, the state
    stays at the block's start."""
    state.cache.release_from(state.n)


@dataclass
class MultiStepRoundResult:
    committed: List[int]
    A: int
    draft: List[int]                    # a0, d_1..d_B as verified
    draft_forwards: int
    step_of: List[int]                  # step at which each window slot was committed
    verify_logits: Optional[np.ndarray] = None


def spec_round_multistep(model, state, B, steps, tau_d, budget=None, keep_logits=False):
    """Self-speculative round with a multi-step draft schedule (Trillion Labs
    blog, the draft-schedule passage; review, Appendix D "Draft Schedule").

    The draft is refined by denoising steps before verification: window slot
    i (position p + i, i = 1..B) holds a0 (i = 1) or d_{i-1}, predicted by
    window row i - 1.  Each step commits slots by the draft-side threshold
    tau_d with the most-confident fallback; the last of at most ``steps``
    forwards commits every slot still open.  d_B (position p + B + 1, which
    has no slot) is window row B's prediction in the last draft forward.
    Verification, acceptance and rollback are those of the greedy round.
    With ``steps`` = 1 this is the one-shot round.
    """
    cfg = model.cfg
    if steps < 1:
        raise ValueError("a draft schedule needs at least one forward")
    p, x0, cache = state.n, state.x0, state.cache
    s = [cfg.mask_id] * B
    step_of = [-1] * B
    k = 0
    last = None
    while True:
        h = model.embed_tokens([x0] + s)
        logits = model.forward(cache, h, p + np.arange(B + 1), draft_visibility(p, B))
        last = logits
        tc = [confidence(logits[j], cfg.mask_id) for j in range(B)]
        und = [t == cfg.mask_id for t in s]
        if k == steps - 1:
            chosen = [j for j in range(B) if und[j]]
        else:
            chosen = select_positions(und, [c for _, c in tc], tau_d)
        for j in chosen:
            s[j] = tc[j][0]
            step_of[j] = k
        k += 1
        if cfg.mask_id not in s:
            break
    # slots s_1..s_B hold a0, d_1..d_{B-1}; d_B is row B's prediction (B = 0: a0 is row 0's)
    draft = list(s) + [argmax_excluding(last[B], cfg.mask_id)[0]]
    a0, d = draft[0], draft[1:]
    h = model.embed_tokens([a0] + d)
    vl = model.forward(cache, h, p + 1 + np.arange(B + 1), verify_visibility(p, B))
    a = [argmax_excluding(vl[j], cfg.mask_id)[0] for j in range(B + 1)]
    A = accept_length(d, a[:B])
    committed = commit_tokens(a0, a, A, cfg.eos_id, B + 2 if budget is None else budget)
    state.n = p + A + 2
    state.x0 = a[A]
    cache.release_from(state.n)
    return MultiStepRoundResult(committed=committed, A=A, draft=draft, draft_forwards=k, step_of=step_of,
                                verify_logits=vl if keep_logits else None)


def spec_decode_multistep(model, prefix_emb, B, steps, tau_d, max_len, max_positions=None, rounds_out=None):
    """Greedy self-speculative decoding with a multi-step draft schedule."""
    cfg = model.cfg
    if max_len <= 0:
        return []
    P = prefix_emb.shape[0]
    state, y1, _ = prefill(model, prefix_emb, max_positions or P + max_len + B + 3)
    out = [y1]
    while out[-1] != cfg.eos_id and len(out) < max_len:
        r = spec_round_multistep(model, state, B, steps, tau_d, budget=max_len - len(out))
        if rounds_out is not None:
            rounds_out.append(r)
        out += r.committed
    return out


@dataclass
class DDStats:
    blocks: int = 0
    steps: int = 0               # committing forwards
    cache_writes: int = 0        # cache-write forwards
    tokens: int = 0              # output tokens, y1 included


def dd_tpf(stats):
    """Tokens per forward in the pages' direct-diffusion accounting (review,
    Appendix C): decoded tokens (y1 from prefill excluded) over committing
    forwards; prefill and cache-write forwards are not counted."""
    return (stats.tokens - 1) / stats.steps if stats.steps else 0.0


def dd_decode(model, prefix_emb, B, tau, max_len, max_positions=None, blocks_out=None):
    """Direct block-diffusion decoding until EOS or ``max_len`` tokens.

    Returns (tokens, DDStats).  A block that holds EOS, or that reaches
    ``max_len``, ends the output without a cache-write forward.
    ``blocks_out``, if a list, receives one BlockResult per block.
    """
    cfg = model.cfg
    st = DDStats()
    if max_len <= 0:
        return [], st
    P = prefix_emb.shape[0]
    state, y1, _ = prefill(model, prefix_emb, max_positions or P + max_len + B + 2)
    out = [y1]
    while out[-1] != cfg.eos_id and len(out) < max_len:
        r = dd_fill(model, state, B, tau)
        if blocks_out is not None:
            blocks_out.append(r)
        st.blocks += 1
        st.steps += r.steps
        toks = list(r.tokens)
        eos = cfg.eos_id in toks
        if eos:
            toks = toks[: toks.index(cfg.eos_id) + 1]
        out += toks[: max_len - len(out)]
        if eos or len(out) >= max_len:
            dd_release(state)
            break
        dd_cache_write(model, state, r.tokens)
        st.cache_writes += 1 if B > 1 else 0
    st.tokens = len(out)
    return out, st

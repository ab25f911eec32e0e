"""Pins of the oracle's stochastic self-speculative round.

* Distribution preservation, the property the pages state for sampling
  (GravityOCR review, section 2; Trillion Labs blog): the first output tokens
  of stochastic self-speculative decoding follow the AR sampling
  distribution of the same model.  Checked by a chi-square test against the
  exact AR distribution, enumerated by teacher-forced forwards on a micro
  model (vocab 6).  The same test rejects the unverified draft (committing
  the sampled drafts without the acceptance test), so it has the power to
  catch a broken rule.
* Greedy limit: at a vanishing temperature every distribution is one-hot and
  the stochastic round commits exactly what the greedy round commits.
* Inverse-CDF sampling: closed forms (one-hot weights, u = 0, u -> 1) and the
  frequency property over a uniform grid of u.
* probs = scipy's softmax of logits / T with [M] removed.
"""

import itertools

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import chisquare

from ssb_inputs import ModelConfig, generate_weights, prefix_embeddings, workload
from oracle import Decoder, DecodeState, prefill, spec_round
from oracle.decode import causal_visibility
from oracle.stochastic import (accept_draft, prefill_sample, probs, residual, sample_index,
                               spec_round_sample)


def _micro(seed=77):
    cfg = ModelConfig(name="micro", n_layers=2, hidden=16, n_heads=2, n_kv_heads=2, head_dim=8, ffn=32,
                      vocab=6, mask_id=5, eos_id=4, dtype="f32", weight_seed_id=seed, weight_std=0.35)
    return Decoder(cfg, generate_weights(cfg))


def test_sample_index_closed_forms_and_frequencies():
    assert sample_index([0, 0, 3.0, 0], 0.0) == 2
    assert sample_index([0, 0, 3.0, 0], 0.999999) == 2
    assert sample_index([0.5, 0, 1.0, 0.5], 0.0) == 0
    assert sample_index([0.5, 0, 1.0, 0.5], 1 - 1e-12) == 3
    assert sample_index([0.5, 0, 1.0, 0.5], 0.25) == 2      # boundary: sum(w[:1]) = 0.5 = u * 2 -> next
    rng = np.random.default_rng([5, 5])
    for _ in range(5):
        w = rng.random(7) * (rng.random(7) > 0.3)
        if w.sum() == 0:
            continue
        N = 20000
        draws = np.array([sample_index(w, (i + 0.5) / N) for i in range(N)])
        freq = np.bincount(draws, minlength=7) / N
        assert np.abs(freq - w / w.sum()).max() <= 1.0 / N + 1e-12
        assert all(freq[w == 0] == 0)


def test_probs_is_softmax_without_mask():
    rng = np.random.default_rng([5, 6])
    for T in (0.3, 1.0, 2.5):
        z = rng.standard_normal(11) * 3
        p = probs(z, 4, T)
        ref = softmax(np.delete(z, 4) / T)
        assert p[4] == 0 and np.abs(np.delete(p, 4) - ref).max() < 1e-15
    with pytest.raises(ValueError):
        probs(z, 4, 0.0)


def test_residual_and_accept_rule_forms():
    p = np.array([0.5, 0.3, 0.2])
    q = np.array([0.2, 0.5, 0.3])
    assert np.allclose(residual(p, q), [0.3, 0, 0])
    assert accept_draft(0.5, 0.2, 0.999)          # p >= q: always accepted
    assert accept_draft(0.3, 0.5, 0.59) and not accept_draft(0.3, 0.5, 0.6)   # accepted iff u < p/q


def _ar_exact(m, pre, K):
    """Exact AR sampling distribution of y_1..y_K (T = 1) by teacher-forced forwards."""
    cfg = m.cfg
    P = pre.shape[0]
    live = [v for v in range(cfg.vocab) if v != cfg.mask_id]
    dist = {}

    def rec(prefix_toks, prob):
        k = len(prefix_toks)
        if k == K or (k and prefix_toks[-1] == cfg.eos_id):
            dist[tuple(prefix_toks)] = dist.get(tuple(prefix_toks), 0.0) + prob
            return
        h = np.concatenate([pre, m.embed_tokens(prefix_toks)], axis=0) if k else pre
        pos = np.arange(P + k)
        lg = m.forward(m.new_cache(P + k), h, pos, causal_visibility(pos, P + k))
        w = probs(lg[-1], cfg.mask_id, 1.0)
        for v in live:
            if w[v] > 0:
                rec(prefix_toks + [v], prob * w[v])

    rec([], 1.0)
    return dist


def _chi2(counts, dist, N):
    keys = sorted(dist)
    exp = np.array([dist[k] * N for k in keys])
    obs = np.array([counts.get(k, 0) for k in keys], dtype=np.float64)
    assert sum(counts.get(k, 0) for k in counts if k not in dist) == 0
    small = exp < 5
    e2 = np.append(exp[~small], exp[small].sum())
    o2 = np.append(obs[~small], obs[small].sum())
    if e2[-1] == 0:
        e2, o2 = e2[:-1], o2[:-1]
    return chisquare(o2, e2 * o2.sum() / e2.sum()).pvalue


def test_stochastic_round_preserves_ar_distribution():
    m = _micro()
    cfg = m.cfg
    B, K, N = 2, 4, 6000
    pre = np.random.default_rng([77, 3]).standard_normal((3, cfg.hidden))
    dist = _ar_exact(m, pre, K)
    assert abs(sum(dist.values()) - 1) < 1e-12
    base, _, _ = prefill(m, pre, 16)
    p1 = probs(m.forward(base.cache.copy(), pre, np.arange(3), causal_visibility(np.arange(3), 3))[2],
               cfg.mask_id, 1.0)
    rng = np.random.default_rng([77, 4])
    spec, draft_only = {}, {}
    for _ in range(N):
        out = [sample_index(p1, rng.random())]
        st = DecodeState(cache=base.cache.copy(), n=base.n, x0=out[0])
        first = None
        while len(out) < K and out[-1] != cfg.eos_id:
            r = spec_round_sample(m, st, B, rng.random(2 * B + 2), budget=K - len(out))
            if first is None:
                first = [r.a0] + r.d
            out += r.committed
        spec[tuple(out)] = spec.get(tuple(out), 0) + 1
        # the unverified draft: y1 then a0, d_1, d_2 of the first round
        dr = [out[0]] + (first or [])
        if cfg.eos_id in dr:
            dr = dr[: dr.index(cfg.eos_id) + 1]
        dr = tuple(dr[:K])
        draft_only[dr] = draft_only.get(dr, 0) + 1
    assert _chi2(spec, dist, N) > 1e-3
    # power: drafts committed without the acceptance test are not AR-distributed
    bad = {k: v for k, v in draft_only.items() if k in dist}
    assert sum(v for k, v in draft_only.items() if k not in dist) == 0
    assert _chi2(bad, dist, N) < 1e-6


def test_vanishing_temperature_is_the_greedy_round():
    wl = workload(1)
    m = Decoder(wl.model, generate_weights(wl.model))
    B = wl.block
    rng = np.random.default_rng([1, 9])
    for s in range(5):
        pre = prefix_embeddings(wl.wid, s, wl.prefix_len, m.cfg.hidden)
        g, _, _ = prefill(m, pre, wl.prefix_len + 3 * B + 8)
        st = DecodeState(cache=g.cache.copy(), n=g.n, x0=g.x0)
        for k in range(3):
            rg = spec_round(m, g, B)
            rs = spec_round_sample(m, st, B, rng.random(2 * B + 2), temperature=1e-6)
            assert rs.committed == rg.committed and rs.A == rg.A
            assert (st.n, st.x0) == (g.n, g.x0)

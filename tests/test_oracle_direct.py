"""Pins of the oracle's direct block-diffusion decoder against what the pages
and the mathematics fix.

* The commit rule at the threshold, from the blog's Figure 2 failure example
  (three tokens of confidence .70/.79/.79 committed together at tau_c = 0.7,
  so the comparison is inclusive), and its fallback to the single most
  confident position (blog glossary; review, Appendix B.1).
* The confidence is a softmax probability: checked against scipy's softmax
  and against two closed forms (uniform logits, two live tokens).
* Block size 1 reduces direct diffusion to greedy AR decoding for every
  threshold: the window [x0, M] has one causal row, which is the AR step.
* tau_c = 0 commits a whole block in one forward, which is the one-shot
  draft of the self-speculative round (a0, d_1..d_{B-1}).
* tau_c > 1 commits exactly one position per forward, the most confident.
* After the cache-write forward the cache equals a causal prefill of the
  committed tokens (review, Appendix B.1/B.2: only causal state survives).
* EOS truncation and the output budget.
* Multi-step draft schedule: one step is the one-shot round exactly; any
  schedule leaves the output and the cache AR-identical (the verifier
  decides every committed token); the causal boundary row makes a0 the AR
  token whatever the schedule.
"""

import dataclasses
import os

import numpy as np
import pytest
from scipy.special import softmax

from ssb_inputs import generate_weights, prefix_embeddings, workload
from oracle import (Decoder, DecodeState, ar_decode, causal_visibility, confidence, dd_cache_write,
                    dd_decode, dd_fill, dd_tpf, prefill, select_positions, spec_round)
from oracle import ar_step as ar_step_o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def tiny():
    wl = workload(1)
    return wl, Decoder(wl.model, generate_weights(wl.model))


def _copy(st):
    return DecodeState(cache=st.cache.copy(), n=st.n, x0=st.x0)


def _mid_tau(m, pre, B):
    """A threshold inside the tiny model's confidence range (its logits are
    small, so every confidence sits near 1/(vocab-1)): about half of the
    first step's positions reach it."""
    st, _, _ = prefill(m, pre, pre.shape[0] + B + 4)
    r = dd_fill(m, st, B, 2.0)
    return float(np.median(r.step_conf[0]))


def test_select_rule_figure2_golden():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "dd_select_fig2.txt")) if l.strip() and l[0] != "#"]
    tau = float(rows[0][1])
    conf = [float(r[0]) for r in rows[1:]]
    want = [j for j, r in enumerate(rows[1:]) if r[1] == "1"]
    assert select_positions([True] * len(conf), conf, tau) == want
    # the same step above every confidence: only the most confident, lowest position on ties
    assert select_positions([True] * len(conf), conf, 0.8) == [1]
    # committed positions are never committed again
    assert select_positions([False, True, True], conf, tau) == [1, 2]
    assert select_positions([False, False, False], conf, tau) == []
    assert select_positions([True, False, False], conf, 0.99) == [0]


def test_confidence_is_softmax_probability():
    rng = np.random.default_rng([9, 1])
    for _ in range(20):
        V = int(rng.integers(3, 40))
        mask = int(rng.integers(0, V))
        z = rng.standard_normal(V) * rng.uniform(0.1, 8.0)
        tok, c = confidence(z, mask)
        live = np.delete(np.arange(V), mask)
        p = softmax(z[live])
        assert tok == live[int(np.argmax(p))]
        assert abs(c - p.max()) < 1e-14
    # closed forms: uniform logits over V-1 live tokens; two live tokens -> logistic
    assert abs(confidence(np.zeros(9), 4)[1] - 1 / 8) < 1e-15
    d = 1.3
    tok, c = confidence(np.array([0.2, 0.2 + d, 50.0]), 2)
    assert tok == 1 and abs(c - 1 / (1 + np.exp(-d))) < 1e-15


def test_block_size_one_is_ar_decoding(tiny):
    wl, m = tiny
    for s in range(6):
        pre = prefix_embeddings(wl.wid, s, wl.prefix_len, m.cfg.hidden)
        ar = ar_decode(m, pre, 24)
        for tau in (0.0, 0.5, 1.5):
            out, st = dd_decode(m, pre, 1, tau, 24)
            assert out == ar, (s, tau)
            assert st.steps == len(out) - 1 and st.cache_writes == 0


def test_tau_zero_block_is_one_shot_draft(tiny):
    wl, m = tiny
    B = wl.block
    for s in range(4):
        pre = prefix_embeddings(wl.wid, s, wl.prefix_len, m.cfg.hidden)
        st, _, _ = prefill(m, pre, wl.prefix_len + 2 * B + 4)
        sp = _copy(st)
        r = dd_fill(m, st, B, 0.0)
        rr = spec_round(m, sp, B)
        assert r.steps == 1 and r.step_of == [0] * B
        assert r.tokens == [rr.a0] + rr.d[: B - 1]


def test_tau_above_one_commits_most_confident_each_step(tiny):
    wl, m = tiny
    B = wl.block
    pre = prefix_embeddings(wl.wid, 2, wl.prefix_len, m.cfg.hidden)
    st, _, _ = prefill(m, pre, wl.prefix_len + 2 * B + 4)
    r = dd_fill(m, st, B, 1.01)
    assert r.steps == B and sorted(r.step_of) == list(range(B))
    for k in range(B):
        j = r.step_of.index(k)
        undecided = [r.step_of[i] >= k for i in range(B)]
        best = max((r.step_conf[k][i], -i) for i in range(B) if undecided[i])
        assert j == -best[1]
        assert r.tokens[j] == r.step_tok[k][j]


def test_mixed_threshold_steps_are_consistent(tiny):
    wl, m = tiny
    B = wl.block
    pre = prefix_embeddings(wl.wid, 4, wl.prefix_len, m.cfg.hidden)
    tau = _mid_tau(m, pre, B)
    st, _, _ = prefill(m, pre, wl.prefix_len + 2 * B + 4)
    r = dd_fill(m, st, B, tau)
    assert 1 <= r.steps <= B and min(r.step_of) == 0 and max(r.step_of) == r.steps - 1
    for k in range(r.steps):
        got = [j for j in range(B) if r.step_of[j] == k]
        und = [r.step_of[j] >= k for j in range(B)]
        assert got == select_positions(und, r.step_conf[k], tau)
        for j in got:
            assert r.tokens[j] == r.step_tok[k][j]
    assert any(len([j for j in range(B) if r.step_of[j] == k]) > 1 for k in range(r.steps))


def test_cache_after_cache_write_is_causal_prefill(tiny):
    wl, m = tiny
    B = wl.block
    P = wl.prefix_len
    pre = prefix_embeddings(wl.wid, 6, P, m.cfg.hidden)
    tau = _mid_tau(m, pre, B)
    st, y1, _ = prefill(m, pre, P + 3 * B + 4)
    toks = [y1]
    for _ in range(2):
        r = dd_fill(m, st, B, tau)
        dd_cache_write(m, st, r.tokens)
        toks += r.tokens
        assert st.n == P + len(toks) - 1 and st.x0 == toks[-1]
        # causal forward over prefix + every committed token but the boundary
        h = np.concatenate([pre, m.embed_tokens(toks[:-1])], axis=0)
        ref = m.new_cache(st.n)
        pos = np.arange(st.n)
        m.forward(ref, h, pos, causal_visibility(pos, st.n))
        n = st.n
        np.testing.assert_allclose(st.cache.K[:, :n], ref.K[:, :n], rtol=0, atol=1e-12)
        np.testing.assert_allclose(st.cache.V[:, :n], ref.V[:, :n], rtol=0, atol=1e-12)
        assert np.isnan(st.cache.K[:, n:]).all()


def test_eos_budget_and_tpf(tiny):
    wl, m = tiny
    B = 4
    # a prefix whose third block holds a token not seen before (the tiny model repeats itself)
    for s in range(8, 60):
        pre = prefix_embeddings(wl.wid, s, wl.prefix_len, m.cfg.hidden)
        tau = _mid_tau(m, pre, B)
        full, st = dd_decode(m, pre, B, tau, 30)
        ks = [i for i in range(9, 13) if full[i] not in full[:i]]
        if ks:
            break
    else:
        pytest.fail("no prefix with a fresh token in the third block")
    assert len(full) == 30 and st.blocks == 8
    assert abs(dd_tpf(st) - 29 / st.steps) < 1e-15 and 1.0 <= dd_tpf(st) <= B
    assert st.cache_writes == st.blocks - 1
    for max_len in (1, 2, 5, 6, 13):
        assert dd_decode(m, pre, B, tau, max_len)[0] == full[:max_len]
    # EOS inside the third block: the block completes, the output ends at the first EOS
    k = ks[0]
    m2 = Decoder.__new__(Decoder)
    m2.__dict__.update(m.__dict__)
    m2.cfg = dataclasses.replace(m.cfg, eos_id=full[k])
    out, st2 = dd_decode(m2, pre, B, tau, 30)
    assert out == full[: k + 1]
    assert st2.blocks == 3 and st2.cache_writes == 2
    # tau = 0: one forward per block, B tokens per forward
    out0, st0 = dd_decode(m, pre, B, 0.0, 1 + 5 * B)
    assert st0.steps == st0.blocks == 5 and dd_tpf(st0) == B


# ---- multi-step draft schedule (blog, draft-schedule passage; review, Appendix D) ----

def test_multistep_one_step_is_the_one_shot_round(tiny):
    from oracle import spec_round_multistep
    wl, m = tiny
    B = wl.block
    for s in range(4):
        pre = prefix_embeddings(wl.wid, s, wl.prefix_len, m.cfg.hidden)
        st, _, _ = prefill(m, pre, wl.prefix_len + 4 * B + 8)
        sp = _copy(st)
        for k in range(3):
            r = spec_round_multistep(m, st, B, 1, 0.5)
            rr = spec_round(m, sp, B)
            assert r.committed == rr.committed and r.A == rr.A and r.draft_forwards == 1
            assert r.draft == [rr.a0] + rr.d
            assert (st.n, st.x0) == (sp.n, sp.x0)


def test_multistep_decoding_is_ar_decoding(tiny):
    """The verifier makes the output AR-identical whatever the draft schedule."""
    from oracle import spec_decode_multistep, spec_round_multistep
    wl, m = tiny
    B = wl.block
    for s in range(3):
        pre = prefix_embeddings(wl.wid, s, wl.prefix_len, m.cfg.hidden)
        ar = ar_decode(m, pre, 40)
        tau = _mid_tau(m, pre, B)
        for steps, td in ((2, tau), (4, tau), (B, 2.0), (3, 0.0)):
            rounds = []
            out = spec_decode_multistep(m, pre, B, steps, td, 40, rounds_out=rounds)
            assert out == ar, (s, steps, td)
            for r in rounds:
                assert 1 <= r.draft_forwards <= steps
                assert max(r.step_of) == r.draft_forwards - 1 and min(r.step_of) >= 0
                if td == 0.0:
                    assert r.draft_forwards == 1
            # the boundary row is causal: a0 is always the AR token
            c = 1
            for r in rounds:
                if c < len(ar):
                    assert r.draft[0] == ar[c]
                c += len(r.committed)


def test_multistep_cache_is_ar_cache(tiny):
    from oracle import spec_round_multistep
    wl, m = tiny
    B = wl.block
    pre = prefix_embeddings(wl.wid, 5, wl.prefix_len, m.cfg.hidden)
    tau = _mid_tau(m, pre, B)
    cap = wl.prefix_len + 80
    ar_state, _, _ = prefill(m, pre, cap)
    for _ in range(60):
        ar_step_o(m, ar_state)
    st, _, _ = prefill(m, pre, cap)
    for k in range(4):
        spec_round_multistep(m, st, B, 3, tau)
        n = st.n
        np.testing.assert_allclose(st.cache.K[:, :n], ar_state.cache.K[:, :n], rtol=0, atol=1e-12)
        np.testing.assert_allclose(st.cache.V[:, :n], ar_state.cache.V[:, :n], rtol=0, atol=1e-12)
        assert np.isnan(st.cache.K[:, n:]).all()

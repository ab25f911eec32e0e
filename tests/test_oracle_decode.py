"""Pins of the oracle's decoding round against what the pages fix.

* Self-speculative greedy output equals AR greedy output of the same model
  in exact arithmetic, by induction over rounds (GravityOCR review,
  Appendix B.3; velog review, round description).
* A non-truncated round commits between 2 and B+2 tokens (review 3.2).
* Full acceptance (A = B) commits the bonus token (Appendix B.2).
* Only causal state survives a round (Appendix B.2): after each round the
  cache equals the AR cache for the same committed prefix.
* Visibility of draft and verify rows (review 3.2): hand-written fixture
  plus perturbation.
* TPF accounting (review 4.1) against the pages' printed tables.
"""

import dataclasses
import itertools
import os

import numpy as np
import pytest

from ssb_inputs import ModelConfig, generate_weights, prefix_embeddings, workload
from oracle import (Decoder, DecodeState, RoundResult, accept_length, ar_decode, ar_step,
                    build_plant, commit_tokens, draft_visibility, prefill, spec_decode,
                    spec_round, tpf, verify_visibility, teacher_forced_argmax)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def tiny():
    wl = workload(1)
    return wl, Decoder(wl.model, generate_weights(wl.model))


def _micro_cfg(eos=4, seed=77, std=0.5, layers=2):
    return ModelConfig(name="micro", n_layers=layers, hidden=16, n_heads=2, n_kv_heads=2,
                       head_dim=8, ffn=32, vocab=6, mask_id=5, eos_id=eos, dtype="f32",
                       weight_seed_id=seed, weight_std=std)


def test_spec_decode_equals_ar_decode_all_seeds(tiny):
    wl, m = tiny
    n_tokens = 0
    for s in range(wl.n_regions):
        pre = prefix_embeddings(wl.wid, s, wl.prefix_len, m.cfg.hidden)
        ar = ar_decode(m, pre, wl.max_len)
        rounds = []
        sp = spec_decode(m, pre, wl.block, wl.max_len, rounds_out=rounds)
        assert sp == ar, f"seed {s}"
        for r in rounds[:-1]:
            assert 2 <= len(r.committed) <= wl.block + 2
        n_tokens += len(sp)
    assert n_tokens > wl.n_regions * 2


def test_planted_drafts_realize_every_accept_length(tiny):
    wl, m = tiny
    B = wl.block
    seen = set()
    for s in range(12):
        pre = prefix_embeddings(wl.wid, s, wl.prefix_len, m.cfg.hidden)
        ar = ar_decode(m, pre, wl.max_len)
        targets = [(s + k) % (B + 1) for k in range(64)]
        rounds = []
        plant = lambda k, c: build_plant(ar, c, targets[k], B, m.cfg.vocab, m.cfg.mask_id)
        sp = spec_decode(m, pre, B, wl.max_len, plant_fn=plant, rounds_out=rounds)
        assert sp == ar
        c = 1
        for k, r in enumerate(rounds):
            # the planted accept length is realized whenever the AR output covers it
            if c + targets[k] + 1 < len(ar):
                assert r.A == targets[k], (s, k)
                seen.add(r.A)
            c += len(r.committed)
    assert seen == set(range(B + 1))


def test_full_accept_commits_bonus_token(tiny):
    wl, m = tiny
    B = wl.block
    pre = prefix_embeddings(wl.wid, 3, wl.prefix_len, m.cfg.hidden)
    ar = ar_decode(m, pre, 40)
    state, y1, _ = prefill(m, pre, wl.prefix_len + 64)
    assert y1 == ar[0]
    r = spec_round(m, state, B, planted=ar[2:2 + B])
    assert r.A == B
    assert len(r.committed) == B + 2
    assert r.committed == ar[1:B + 3]          # last one is the bonus a_{B+1}
    assert state.x0 == ar[B + 2]


def test_block_zero_round_is_two_ar_steps(tiny):
    wl, m = tiny
    pre = prefix_embeddings(wl.wid, 5, wl.prefix_len, m.cfg.hidden)
    s1, y1, _ = prefill(m, pre, wl.prefix_len + 8)
    s2, _, _ = prefill(m, pre, wl.prefix_len + 8)
    r = spec_round(m, s1, 0)
    t1, _ = ar_step(m, s2)
    t2, _ = ar_step(m, s2)
    assert r.committed == [t1, t2] and r.A == 0
    assert s1.n == s2.n and s1.x0 == s2.x0


def test_cache_after_each_round_equals_ar_cache(tiny):
    wl, m = tiny
    B = wl.block
    for s in (0, 7):
        pre = prefix_embeddings(wl.wid, s, wl.prefix_len, m.cfg.hidden)
        cap = wl.prefix_len + 80
        ar_state, _, _ = prefill(m, pre, cap)
        ar_out = []
        for _ in range(60):
            ar_out.append(ar_step(m, ar_state)[0])
        sp_state, y1, _ = prefill(m, pre, cap)
        cont = [y1] + ar_out
        for k in range(6):
            plant = build_plant(cont, sp_state.n - wl.prefix_len + 1, (3 * k + s) % (B + 1), B,
                                m.cfg.vocab, m.cfg.mask_id)
            spec_round(m, sp_state, B, planted=plant)
            n = sp_state.n
            np.testing.assert_allclose(sp_state.cache.K[:, :n], ar_state.cache.K[:, :n],
                                       rtol=0, atol=1e-12)
            np.testing.assert_allclose(sp_state.cache.V[:, :n], ar_state.cache.V[:, :n],
                                       rtol=0, atol=1e-12)
            assert np.isnan(sp_state.cache.K[:, n:]).all()    # released suffix


def test_brute_force_all_drafts_micro_model():
    """Every one of the V^B draft vectors leaves output and cache AR-identical."""
    B = 3
    cfg = _micro_cfg()
    m = Decoder(cfg, generate_weights(cfg))
    for seed in range(50):
        pre = np.random.default_rng([77, seed]).standard_normal((4, cfg.hidden))
        st, y1, _ = prefill(m, pre, 16)
        ar_st = DecodeState(cache=st.cache.copy(), n=st.n, x0=st.x0)
        ar = [ar_step(m, ar_st)[0] for _ in range(B + 2)]
        if cfg.eos_id not in ar:
            break
    else:
        pytest.fail("no prefix without early EOS")
    for d in itertools.product(range(cfg.vocab), repeat=B):
        s = DecodeState(cache=st.cache.copy(), n=st.n, x0=st.x0)
        r = spec_round(m, s, B, planted=list(d))
        assert r.committed == ar[:len(r.committed)]
        assert len(r.committed) == r.A + 2
        expect_A = 0
        while expect_A < B and d[expect_A] == ar[1 + expect_A]:
            expect_A += 1
        assert r.A == expect_A
        n = s.n
        np.testing.assert_allclose(s.cache.K[:, :n], ar_st.cache.K[:, :n], rtol=0, atol=1e-12)
        np.testing.assert_allclose(s.cache.V[:, :n], ar_st.cache.V[:, :n], rtol=0, atol=1e-12)


def test_accept_rule_enumeration():
    for B in range(0, 5):
        for d in itertools.product(range(3), repeat=B):
            for a in itertools.product(range(3), repeat=B + 1):
                A = accept_length(list(d), list(a[:B]))
                eq = np.array(d) == np.array(a[:B])
                ref = int(np.cumprod(eq).sum()) if B else 0
                assert A == ref
                c = commit_tokens(9, list(a), A, eos_id=99, budget=B + 2)
                assert c[0] == 9 and c[1:] == list(a[:A + 1])
                assert all(d[j] == c[j + 1] for j in range(A))


def test_commit_truncation_eos_and_budget():
    a = [1, 2, 7, 3, 4]
    assert commit_tokens(0, a, 4, eos_id=7, budget=6) == [0, 1, 2, 7]
    assert commit_tokens(7, a, 4, eos_id=7, budget=6) == [7]
    assert commit_tokens(0, a, 4, eos_id=99, budget=3) == [0, 1, 2]
    assert commit_tokens(0, a, 1, eos_id=99, budget=6) == [0, 1, 2]


def test_eos_and_max_len_truncation_end_to_end(tiny):
    wl, m = tiny
    pre = prefix_embeddings(wl.wid, 11, wl.prefix_len, m.cfg.hidden)
    ar_full = ar_decode(m, pre, 40)
    # make the 10th output token the EOS of a copy of the model
    eos = ar_full[9]
    cfg2 = dataclasses.replace(m.cfg, eos_id=eos)
    m2 = Decoder.__new__(Decoder)
    m2.__dict__.update(m.__dict__)
    m2.cfg = cfg2
    ar = ar_decode(m2, pre, 40)
    assert ar[-1] == eos and ar == ar_full[: ar_full.index(eos) + 1]
    for B in (1, 4, 8):
        assert spec_decode(m2, pre, B, 40) == ar
    for max_len in (0, 1, 2, 3, 7, 11, 23):
        assert spec_decode(m, pre, wl.block, max_len) == ar_full[:max_len]
        assert ar_decode(m, pre, max_len) == ar_full[:max_len]


def _read_golden_vis():
    mats, cur = {}, None
    for line in open(os.path.join(GOLDEN, "visibility_p2_B3.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            cur = line.strip("[]")
            mats[cur] = []
        else:
            mats[cur].append([int(t) for t in line.split()])
    return {k: np.array(v, dtype=bool) for k, v in mats.items()}


def test_visibility_matches_hand_written_fixture():
    g = _read_golden_vis()
    np.testing.assert_array_equal(draft_visibility(2, 3), g["draft"])
    np.testing.assert_array_equal(verify_visibility(2, 3), g["verify"])


def test_window_rows_influence_exactly_the_rows_that_see_them():
    """Perturb one window row's input: rows that do not see its key are unchanged."""
    cfg = _micro_cfg(seed=78)
    m = Decoder(cfg, generate_weights(cfg))
    for p, B in itertools.product(range(1, 5), range(1, 4)):
        pre = np.random.default_rng([78, p, B]).standard_normal((p + 1, cfg.hidden))
        for mode in ("draft", "verify"):
            vis = draft_visibility(p, B) if mode == "draft" else verify_visibility(p, B)
            pos = (p if mode == "draft" else p + 1) + np.arange(B + 1)
            # draft: cache holds 0..p-1; verify: the boundary slot p is filled too
            st, _, _ = prefill(m, pre[: p if mode == "draft" else p + 1], p + B + 3)
            h = np.random.default_rng([79, p, B]).standard_normal((B + 1, cfg.hidden))
            base = m.forward(st.cache.copy(), h, pos, vis)
            for k in range(B + 1):
                h2 = h.copy()
                h2[k] += 0.3
                out = m.forward(st.cache.copy(), h2, pos, vis)
                for r in range(B + 1):
                    changed = not np.array_equal(out[r], base[r])
                    assert changed == (r == k or bool(vis[r, pos[k]])), (mode, p, B, k, r)


def test_tpf_accounting_against_printed_tables():
    for line in open(os.path.join(GOLDEN, "tpf_tables.txt")):
        if line.startswith("#") or not line.strip():
            continue
        parts = line.split()
        A_mean, printed = float(parts[1]), float(parts[2])
        n = 10
        total = int(round(A_mean * n))
        As = [total // n + (1 if i < total % n else 0) for i in range(n)]
        rounds = [RoundResult(committed=[0] * (a + 2), A=a, a0=0, d=[], a=[]) for a in As]
        t, mean_A = tpf(rounds)
        assert abs(mean_A - A_mean) < 1e-9
        assert abs(t - (A_mean + 2) / 2) < 1e-9
        assert abs(t - printed) <= 0.05 + 1e-9, parts[0]


def test_round_commit_bounds_fixture(tiny):
    rows = [l.split() for l in open(os.path.join(GOLDEN, "round_bounds.txt"))
            if l.strip() and not l.startswith("#")]
    B, lo, hi = (int(x) for x in rows[0])
    for tokens, rounds in ((int(a), int(b)) for a, b in rows[1:]):
        assert lo * rounds <= tokens <= hi * rounds + 1
    # the oracle realizes both bounds at B = 32
    wl, m = tiny
    pre = prefix_embeddings(wl.wid, 2, wl.prefix_len, m.cfg.hidden)
    ar = ar_decode(m, pre, 60)
    st, _, _ = prefill(m, pre, wl.prefix_len + 80)
    r = spec_round(m, st, B, planted=ar[2:2 + B])
    assert len(r.committed) == hi
    st, _, _ = prefill(m, pre, wl.prefix_len + 80)
    r = spec_round(m, st, B, planted=build_plant(ar, 1, 0, B, m.cfg.vocab, m.cfg.mask_id))
    assert len(r.committed) == lo


def test_teacher_forced_argmax_reproduces_ar(tiny):
    wl, m = tiny
    pre = prefix_embeddings(wl.wid, 4, wl.prefix_len, m.cfg.hidden)
    ar = ar_decode(m, pre, 30)
    pred, margins = teacher_forced_argmax(m, pre, ar)
    assert pred == ar
    assert all(x >= 0 for x in margins)

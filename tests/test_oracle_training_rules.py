"""Brute-force checks of the training-time rules (rule checks only).

Complementary masks and the three-stream attention predicate: GravityOCR
review section 3.1 "Joint AR-Diffusion Training"; velog review "training:
three streams in one forward"; blog description of the attention figure.
"""

import numpy as np

from oracle import complementary_masks, draft_visibility, training_visibility


def test_complementary_masks_enumerated():
    for B in range(1, 13):
        t = 0.5
        for bits in range(2 ** B):
            want = np.array([(bits >> i) & 1 for i in range(B)], dtype=bool)
            u = np.where(want, 0.25, 0.75)
            m1, m2 = complementary_masks(t, u)
            np.testing.assert_array_equal(m1, want)
            assert not np.any(m1 & m2)                 # disjoint
            assert np.all(m1 | m2)                     # union covers the block
            assert np.all(m1.astype(int) + m2.astype(int) == 1)   # supervised once


def test_complementary_mask_fractions():
    rng = np.random.default_rng(0)
    for t in (0.1, 0.35, 0.8):
        u = rng.random(200_000)
        m1, m2 = complementary_masks(t, u)
        assert abs(m1.mean() - t) < 0.005
        assert abs(m2.mean() - (1 - t)) < 0.005


def test_training_visibility_rules():
    P, nb, B = 3, 3, 4
    vis, kinds = training_visibility(P, nb, B)
    for qi, (qs, qb, qx) in enumerate(kinds):
        for ki, (ks, kb, kx) in enumerate(kinds):
            v = vis[qi, ki]
            if qs == "clean" and ks in ("c1", "c2"):
                assert not v                             # clean never sees corrupted
            if qs in ("c1", "c2") and ks == "clean":
                assert v == (kb < qb)                    # only earlier clean blocks
            if qs in ("c1", "c2") and ks in ("c1", "c2"):
                assert v == (ks == qs and kb == qb)      # own block only, bidirectional
            if qs != "prefix" and ks == "prefix":
                assert v
    # no corrupted token can see its own or a later ground-truth token
    for qi, (qs, qb, qx) in enumerate(kinds):
        if qs in ("c1", "c2"):
            for ki, (ks, kb, kx) in enumerate(kinds):
                if ks == "clean" and kx >= qb * B:
                    assert not vis[qi, ki]


def test_inference_draft_window_is_the_training_corrupted_block():
    """At a block-aligned boundary, the draft window's visibility equals the
    training predicate restricted to (last clean token, corrupted block)."""
    P, nb, B = 3, 3, 4
    vis, kinds = training_visibility(P, nb, B)
    idx = {k: i for i, k in enumerate(kinds)}
    for b in range(1, nb):
        p = P + b * B - 1                       # boundary x0 = last clean token before block b
        rows = [idx[("clean", b - 1, b * B - 1)]] + [idx[("c1", b, b * B + j)] for j in range(B)]
        keys = [idx[("prefix", -1, i)] for i in range(P)] + \
               [idx[("clean", t // B, t)] for t in range(b * B)] + \
               [idx[("c1", b, b * B + j)] for j in range(B)]
        sub = vis[np.ix_(rows, keys)]
        np.testing.assert_array_equal(sub, draft_visibility(p, B))

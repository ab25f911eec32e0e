"""Seeded input generators: bf16 rounding, determinism, shapes and length mix."""

import numpy as np
import torch

from ssb_inputs import (MODELS, WORKLOADS, bf16_round, generate_weights, plant_accept_lengths,
                        prefix_embeddings, target_lengths, weight_names)


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([(rng.standard_normal(100_000) * 10.0 ** rng.integers(-5, 5, size=100_000)).astype(np.float32),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 65504.0, 0.0, -0.0],
                                 dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(bf16_round(x), ref)
    assert bf16_round(np.float32([1 + 2 ** -8]))[0] == 1.0               # tie to even
    assert bf16_round(np.float32([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6


def test_tiny_weights_deterministic_and_bf16_exact():
    cfg = MODELS["tiny_fp32"]
    a = generate_weights(cfg)
    b = generate_weights(cfg)
    assert list(a) == list(b)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
        assert a[k].dtype == np.float32
        assert np.all((a[k].view(np.uint32) & 0xFFFF) == 0)
    assert a["embed"].shape == (cfg.vocab, cfg.hidden)
    assert a["layers.0.wk"].shape == (cfg.kv_dim, cfg.hidden)
    assert a["layers.1.wd"].shape == (cfg.hidden, cfg.ffn)
    assert abs(a["lm_head"].std() - cfg.weight_std) < 0.002
    assert weight_names(cfg)[0] == "embed" and weight_names(cfg)[-1] == "lm_head"


def test_prefix_embeddings():
    e = prefix_embeddings(3, 5, 16, 1024)
    np.testing.assert_array_equal(e, prefix_embeddings(3, 5, 16, 1024))
    assert not np.array_equal(e, prefix_embeddings(3, 6, 16, 1024))
    assert np.all((e.view(np.uint32) & 0xFFFF) == 0)
    assert abs(e.std() - 1.0) < 0.02


def test_length_mix_and_plant_draws():
    wl = WORKLOADS[3]
    L = target_lengths(wl)
    assert len(L) == 256 and min(L) >= 1 and max(L) <= 512
    assert 55 < np.mean(L) < 90
    wl5 = WORKLOADS[5]
    assert len(target_lengths(wl5)) == 16
    a = plant_accept_lengths(2, 0, 20000, 32, 1 / 20)
    assert a.min() == 0 and a.max() == 32
    # E[min(G, 32)] with G ~ Geometric(1/20) on {0,1,...} is sum_{k=1..32} 0.95^k = 15.32
    assert abs(a.mean() - sum(0.95 ** k for k in range(1, 33))) < 0.3
    f = plant_accept_lengths(4, 0, 20000, 32, 1 / 20, full_accept_p=0.05)
    assert (f == 32).mean() > (a == 32).mean() + 0.03

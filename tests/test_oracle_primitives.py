"""Pins of the oracle's building blocks against closed forms and library routines.

Each check is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign or index, a transposed operand, the wrong GQA head mapping)
fails at least one of them.
"""

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from ssb_inputs import ModelConfig, generate_weights
from oracle import Decoder, rms_norm, rope, silu, attend, argmax_excluding
from oracle.decode import causal_visibility


def test_rms_norm_closed_form():
    x = np.array([[3.0, 4.0]])
    y = rms_norm(x, np.ones(2), 0.0)
    np.testing.assert_allclose(y, x / np.sqrt(12.5), rtol=0, atol=1e-15)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64)) * 3.0
    y = rms_norm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-12)
    g = rng.standard_normal(64)
    np.testing.assert_allclose(rms_norm(x, g, 0.0), y * g, atol=1e-12)
    # scale invariance (eps = 0) and eps entering under the square root
    np.testing.assert_allclose(rms_norm(7.0 * x, np.ones(64), 0.0), y, atol=1e-12)
    z = rms_norm(np.array([[1.0, 1.0]]), np.ones(2), 3.0)
    np.testing.assert_allclose(z, [[0.5, 0.5]], atol=1e-15)


def test_silu_closed_form():
    x = np.linspace(-20, 20, 101)
    np.testing.assert_allclose(silu(x), x * scipy.special.expit(x), rtol=1e-12, atol=1e-300)
    assert silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(silu(np.array([50.0])), [50.0], rtol=1e-15)


def _rope_complex(x, positions, theta):
    """Independent formulation: pair (x_i, x_{i+d/2}) is the complex number
    x_i + 1j*x_{i+d/2}, multiplied by exp(1j * pos * theta^(-2i/d))."""
    d = x.shape[-1]
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    freqs = np.array([theta ** (-2.0 * i / d) for i in range(half)])
    rot = np.exp(1j * np.outer(positions, freqs))[:, None, :]
    w = z * rot
    return np.concatenate([w.real, w.imag], axis=-1)


def test_rope_identity_norm_and_complex_form():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 3, 32))
    np.testing.assert_array_equal(rope(x[:1], [0], 1e4), x[:1])
    pos = np.array([0, 1, 5, 77, 1000, 5183])
    y = rope(x, pos, 1e4)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    np.testing.assert_allclose(y, _rope_complex(x, pos, 1e4), atol=1e-12)


def test_rope_relative_position():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    def dot(pq, pk):
        return float(np.sum(rope(q, [pq], 1e4) * rope(k, [pk], 1e4)))
    base = dot(10, 3)
    for c in (1, 17, 400, 4000):
        assert abs(dot(10 + c, 3 + c) - base) < 1e-9
    assert abs(dot(10, 3) - dot(3, 10)) > 1e-6   # direction matters


def test_attend_single_key_and_uniform():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((5, 2, 8))
    V = rng.standard_normal((5, 2, 8))
    q = rng.standard_normal((1, 4, 8))
    vis = np.zeros((1, 5), dtype=bool)
    vis[0, 3] = True
    o = attend(q, K, V, vis, n_rep=2)
    for h in range(4):
        np.testing.assert_allclose(o[0, h], V[3, h // 2], atol=1e-15)
    vis = np.array([[True, False, True, True, False]])
    o = attend(np.zeros((1, 4, 8)), K, V, vis, n_rep=2)
    for h in range(4):
        np.testing.assert_allclose(o[0, h], V[[0, 2, 3], h // 2].mean(axis=0), atol=1e-14)


def test_attend_matches_dense_softmax_and_invisible_keys_are_ignored():
    rng = np.random.default_rng(4)
    M, n, Hq, Hkv, d = 7, 11, 4, 2, 16
    q = rng.standard_normal((M, Hq, d))
    K = rng.standard_normal((n, Hkv, d))
    V = rng.standard_normal((n, Hkv, d))
    vis = rng.random((M, n)) < 0.6
    vis[:, 0] = True
    o = attend(q, K, V, vis, n_rep=Hq // Hkv)
    for r in range(M):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            s = K[:, g] @ q[r, h] / np.sqrt(d)
            s[~vis[r]] = -np.inf
            ref = scipy.special.softmax(s) @ V[:, g]
            np.testing.assert_allclose(o[r, h], ref, atol=1e-13)
    # perturbing a key's K and V changes row r's output iff that key is visible
    for j in range(n):
        K2, V2 = K.copy(), V.copy()
        K2[j] += 0.5
        V2[j] -= 0.25
        o2 = attend(q, K2, V2, vis, n_rep=Hq // Hkv)
        for r in range(M):
            changed = not np.array_equal(o2[r], o[r])
            assert changed == bool(vis[r, j]), (r, j)


def test_gqa_equals_mha_with_duplicated_kv():
    rng = np.random.default_rng(5)
    M, n, Hq, Hkv, d = 3, 9, 8, 2, 8
    q = rng.standard_normal((M, Hq, d))
    K = rng.standard_normal((n, Hkv, d))
    V = rng.standard_normal((n, Hkv, d))
    vis = np.tril(np.ones((M, n), dtype=bool), k=n - M)
    n_rep = Hq // Hkv
    o_gqa = attend(q, K, V, vis, n_rep=n_rep)
    K_mha = np.repeat(K, n_rep, axis=1)          # q head h -> kv head h // n_rep
    V_mha = np.repeat(V, n_rep, axis=1)
    o_mha = attend(q, K_mha, V_mha, vis, n_rep=1)
    np.testing.assert_allclose(o_gqa, o_mha, atol=1e-15)


def test_argmax_excluding_mask_and_ties():
    z = np.array([0.1, 0.7, 0.7, 0.2, 0.9])
    tok, t1, t2 = argmax_excluding(z, mask_id=4)
    assert (tok, t1, t2) == (1, 0.7, 0.7)
    tok, t1, t2 = argmax_excluding(z, mask_id=0)
    assert (tok, t1, t2) == (4, 0.9, 0.7)
    rng = np.random.default_rng(6)
    for _ in range(200):
        z = rng.standard_normal(50)
        m = int(rng.integers(50))
        ref = int(np.argmax(np.delete(z, m)))
        ref = ref + (ref >= m)
        assert argmax_excluding(z, m)[0] == ref


def _torch_reference_logits(cfg, w, h0, positions):
    """Causal forward written with torch library routines (float64, CPU)."""
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
    h = t(h0)
    M = h.shape[0]
    pos = torch.tensor(np.asarray(positions, dtype=np.float64))
    d = cfg.head_dim
    freqs = cfg.rope_theta ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    rot = torch.polar(torch.ones(M, d // 2, dtype=torch.float64), pos[:, None] * freqs[None, :])

    def rotary(x):  # x [M, H, d]
        z = torch.complex(x[..., : d // 2], x[..., d // 2:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    mask = torch.tensor(causal_visibility(np.asarray(positions), int(max(positions)) + 1))
    n_rep = cfg.n_heads // cfg.n_kv_heads
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        x = F.rms_norm(h, (cfg.hidden,), weight=t(w[p + "attn_norm"]), eps=cfg.rms_eps)
        q = F.linear(x, t(w[p + "wq"])).view(M, cfg.n_heads, d)
        k = F.linear(x, t(w[p + "wk"])).view(M, cfg.n_kv_heads, d)
        v = F.linear(x, t(w[p + "wv"])).view(M, cfg.n_kv_heads, d)
        q, k = rotary(q), rotary(k)
        k = k.repeat_interleave(n_rep, dim=1)
        v = v.repeat_interleave(n_rep, dim=1)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                           attn_mask=mask)
        h = h + F.linear(o.transpose(0, 1).reshape(M, cfg.q_dim), t(w[p + "wo"]))
        x = F.rms_norm(h, (cfg.hidden,), weight=t(w[p + "mlp_norm"]), eps=cfg.rms_eps)
        h = h + F.linear(F.silu(F.linear(x, t(w[p + "wg"]))) * F.linear(x, t(w[p + "wu"])),
                         t(w[p + "wd"]))
    x = F.rms_norm(h, (cfg.hidden,), weight=t(w["final_norm"]), eps=cfg.rms_eps)
    return F.linear(x, t(w["lm_head"])).numpy()


@pytest.mark.parametrize("n_kv", [4, 2])
def test_decoder_forward_matches_torch_library_composition(n_kv):
    cfg = ModelConfig(name="t", n_layers=2, hidden=64, n_heads=4, n_kv_heads=n_kv, head_dim=16,
                      ffn=96, vocab=40, mask_id=39, eos_id=38, dtype="f32", weight_seed_id=900 + n_kv,
                      weight_std=0.2)
    w = generate_weights(cfg)
    # non-unit norm gains so a dropped gain is caught
    rng = np.random.default_rng(7)
    for key in list(w):
        if key.endswith("norm"):
            w[key] = (1.0 + 0.3 * rng.standard_normal(cfg.hidden)).astype(np.float32)
    model = Decoder(cfg, w)
    M = 9
    h0 = rng.standard_normal((M, cfg.hidden))
    pos = np.arange(M)
    cache = model.new_cache(M)
    got = model.forward(cache, h0, pos, causal_visibility(pos, M))
    ref = _torch_reference_logits(cfg, w, h0, pos)
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=1e-10)
    # every written cache slot holds finite state
    assert np.isfinite(cache.K).all() and np.isfinite(cache.V).all()

"""Decoder forward pass of the oracle (test infrastructure only).

One decoder serves both decoding modes: the pages' recognizer shares its
language decoder and LM head between the AR path and the block-diffusion
path, and the only added parameter is the [M] embedding row (GravityOCR
review, section 3.1 "AR-to-Diffusion Conversion"; velog review, "method").
The modes differ only in which keys each query row may attend to, so the
forward below takes an explicit visibility matrix ``vis[row, key]``.

The architecture is not described on the pages; this oracle uses a pre-norm
Llama-style block (RMSNorm, rotary position embedding with rotate-half
pairing, grouped-query attention, SwiGLU MLP, no biases, untied LM head).
"""

import numpy as np


def rms_norm(x, g, eps):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def silu(x):
    """SiLU (swish): x * sigmoid(x)."""
    return x / (1.0 + np.exp(-x))


def rope(x, positions, theta):
    """Rotary embedding, rotate-half pairing: dims (i, i + d/2) form the pair.

    x: [M, heads, d]; positions: [M] absolute positions.  Pair i rotates by
    angle positions * theta^(-2i/d).
    """
    d = x.shape[-1]
    half = d // 2
    inv_freq = theta ** (-(np.arange(half, dtype=np.float64) * 2.0) / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang).astype(x.dtype)[:, None, :]
    sin = np.sin(ang).astype(x.dtype)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def attend(q, K, V, vis, n_rep):
    """Masked softmax attention with grouped KV heads.

    q: [M, Hq, d]; K, V: [n_keys, Hkv, d]; vis: bool [M, n_keys].
    Query head h reads KV head h // n_rep.  For every row r and head h:
    o[r, h] = sum_{j : vis[r, j]} softmax_j(q[r,h] . K[j,g] / sqrt(d)) V[j, g].
    Invisible keys get probability exactly zero.
    """
    M, Hq, d = q.shape
    out = np.empty_like(q)
    scale = 1.0 / np.sqrt(d)
    for h in range(Hq):
        g = h // n_rep
        s = (q[:, h, :] @ K[:, g, :].T) * scale           # [M, n_keys]
        s = np.where(vis, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.where(vis, np.exp(s), 0.0)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, g, :]
    return out


def argmax_excluding(logits, mask_id):
    """Greedy top-1 over the vocabulary without [M]; lowest id wins ties.

    Returns (token, top1 value, top2 value).  Greedy top-1 verification is
    the decision rule of the round (GravityOCR review, section 2
    "Speculative Decoding"; Appendix B.3 runs greedy).  [M] is an input-only
    embedding row, so it is never a candidate output.
    """
    z = np.array(logits, dtype=np.float64, copy=True)
    z[mask_id] = -np.inf
    tok = int(np.argmax(z))                 # first maximum = lowest id
    top1 = z[tok]
    z[tok] = -np.inf
    top2 = z.max()
    return tok, float(top1), float(top2)


class KVCache:
    """Per-layer K and V for every absolute position; unwritten slots hold NaN.

    NaN makes any read of a slot that no forward has written (or that a
    rollback has released) visible in the output.
    """

    def __init__(self, cfg, max_positions, dtype=np.float64):
        shape = (cfg.n_layers, max_positions, cfg.n_kv_heads, cfg.head_dim)
        self.K = np.full(shape, np.nan, dtype=dtype)
        self.V = np.full(shape, np.nan, dtype=dtype)

    def release_from(self, n):
        """Drop every slot at position >= n (rollback of a rejected suffix)."""
        self.K[:, n:] = np.nan
        self.V[:, n:] = np.nan

    def copy(self):
        c = KVCache.__new__(KVCache)
        c.K = self.K.copy()
        c.V = self.V.copy()
        return c


class Decoder:
    """The shared AR / block-diffusion decoder, in float64 (or float32)."""

    def __init__(self, cfg, weights, dtype=np.float64):
        self.cfg = cfg
        self.dtype = dtype
        c = lambda a: np.asarray(a, dtype=dtype)
        self.embed = c(weights["embed"])
        self.lm_head = c(weights["lm_head"])
        self.final_norm = c(weights["final_norm"])
        self.layers = []
        for l in range(cfg.n_layers):
            p = f"layers.{l}."
            self.layers.append({k: c(weights[p + k]) for k in
                                ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wg", "wu", "wd")})

    def new_cache(self, max_positions):
        return KVCache(self.cfg, max_positions, self.dtype)

    def embed_tokens(self, tokens):
        return self.embed[np.asarray(tokens, dtype=np.int64)]

    def forward(self, cache, h, positions, vis):
        """Run all layers over rows ``h`` at absolute ``positions``.

        Each layer first writes the K and V of every row into
        ``cache[positions]`` (overwriting what was there), then lets every
        row attend to the keys ``vis`` allows.  Returns the logits
        [M, vocab].  vis has one column per key position 0..n_keys-1.
        """
        cfg = self.cfg
        M = h.shape[0]
        positions = np.asarray(positions, dtype=np.int64)
        n_keys = vis.shape[1]
        n_rep = cfg.n_heads // cfg.n_kv_heads
        h = np.array(h, dtype=self.dtype, copy=True)
        for l, L in enumerate(self.layers):
            x = rms_norm(h, L["attn_norm"], cfg.rms_eps)
            q = (x @ L["wq"].T).reshape(M, cfg.n_heads, cfg.head_dim)
            k = (x @ L["wk"].T).reshape(M, cfg.n_kv_heads, cfg.head_dim)
            v = (x @ L["wv"].T).reshape(M, cfg.n_kv_heads, cfg.head_dim)
            q = rope(q, positions, cfg.rope_theta)
            k = rope(k, positions, cfg.rope_theta)
            cache.K[l, positions] = k
            cache.V[l, positions] = v
            o = attend(q, cache.K[l, :n_keys], cache.V[l, :n_keys], vis, n_rep)
            h = h + o.reshape(M, cfg.q_dim) @ L["wo"].T
            x = rms_norm(h, L["mlp_norm"], cfg.rms_eps)
            h = h + (silu(x @ L["wg"].T) * (x @ L["wu"].T)) @ L["wd"].T
        return rms_norm(h, self.final_norm, cfg.rms_eps) @ self.lm_head.T

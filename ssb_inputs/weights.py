"""Seeded random decoder weights.

Every matrix is drawn as float32 N(0, std^2) in a fixed tensor order from one
generator, then rounded to the nearest bfloat16 (ties to even) and kept as
float32.  The values are therefore exactly representable in bf16: the GPU
engine stores them as bf16 without further rounding, and the oracle upcasts
the very same values to float64.  RMSNorm gains are 1.

Matrices use the [out_features][in_features] convention, so a linear map is
``y = W @ x``.
"""

import numpy as np


def bf16_round(a):
    """Round float32 values to the nearest bfloat16 (ties to even), as float32.

    Works on the bit pattern: add 0x7FFF plus the lowest kept bit, then clear
    the low 16 bits (no overflow for finite inputs).
    """
    a = np.array(a, dtype=np.float32, copy=True, order="C")
    u = a.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return a


def weight_names(cfg):
    """Tensor names in draw order (norm gains are not drawn)."""
    names = ["embed"]
    for l in range(cfg.n_layers):
        names += [f"layers.{l}.{n}" for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")]
    names.append("lm_head")
    return names


def weight_shape(cfg, name):
    h, f, v = cfg.hidden, cfg.ffn, cfg.vocab
    leaf = name.split(".")[-1]
    return {
        "embed": (v, h), "lm_head": (v, h),
        "wq": (cfg.q_dim, h), "wk": (cfg.kv_dim, h), "wv": (cfg.kv_dim, h),
        "wo": (h, cfg.q_dim), "wg": (f, h), "wu": (f, h), "wd": (h, f),
    }[leaf]


def generate_weights(cfg):
    """Return {name: float32 array} for every tensor, norm gains included."""
    rng = np.random.default_rng([cfg.weight_seed_id, 0, 0])
    out = {}
    for name in weight_names(cfg):
        shape = weight_shape(cfg, name)
        draw = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
        draw *= np.float32(cfg.weight_std)
        out[name] = bf16_round(draw).reshape(shape)
    ones = np.ones(cfg.hidden, dtype=np.float32)
    for l in range(cfg.n_layers):
        out[f"layers.{l}.attn_norm"] = ones.copy()
        out[f"layers.{l}.mlp_norm"] = ones.copy()
    out["final_norm"] = ones.copy()
    return out

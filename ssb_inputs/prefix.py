"""Prefix embeddings standing in for the vision encoder + prompt.

The pages' recognizer encodes a region crop and a task prompt before
decoding (GravityOCR review, "technical details"; Appendix C counts vision
and prefill as a fixed per-crop cost).  Trained encoders are not available,
so each region's prefix is P rows of N(0, 1) values, rounded to bf16 so the
GPU's bf16 input is exact.
"""

import numpy as np

from .weights import bf16_round


def prefix_embeddings(wid, index, P, hidden):
    rng = np.random.default_rng([wid, 1, index])
    e = rng.standard_normal(P * hidden, dtype=np.float32)
    return bf16_round(e).reshape(P, hidden)

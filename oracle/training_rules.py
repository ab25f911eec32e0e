"""Training-time masking and attention rules, as rule checks (test infrastructure only).

Training itself is out of scope (it needs the pages' datasets and days of
GPU time); these two functions state the rules precisely so that tests can
enumerate them and check them against the inference-time visibility.

* Complementary masking (GravityOCR review, section 3.1 "Joint AR-Diffusion
  Training"; velog review, "training: three streams in one forward"): per
  block draw t ~ U(0, 1); the first corrupted stream masks each response
  token with probability t, the second masks exactly the complement, so
  every response token is supervised in exactly one stream.
* Attention pattern (same passages, and the blog's description of the
  attention figure): the clean stream is causal and never sees a corrupted
  stream; a corrupted block sees its own block bidirectionally and the
  clean response blocks before it, never the current or a later clean
  block, and never the other corrupted stream.  The shared image+prompt
  prefix is clean and visible to all (causal inside itself).
"""

import numpy as np


def complementary_masks(t, u):
    """Masks of the two corrupted streams for one block.

    ``u`` holds one U(0,1) draw per token of the block.  Stream 1 masks token
    i when u[i] < t; stream 2 masks the complement.
    """
    m1 = np.asarray(u) < t
    return m1, ~m1


def training_visibility(prefix_len, n_blocks, B):
    """Key-visibility matrix of one packed training sample.

    Layout along both axes: [prefix (prefix_len) | clean (n_blocks*B) |
    corrupted stream 1 (n_blocks*B) | corrupted stream 2 (n_blocks*B)].
    Returns (vis, kinds) where kinds[i] = (stream, block, index_in_response)
    with stream in {"prefix", "clean", "c1", "c2"}.
    """
    R = n_blocks * B
    T = prefix_len + 3 * R
    kinds = []
    for i in range(prefix_len):
        kinds.append(("prefix", -1, i))
    for s in ("clean", "c1", "c2"):
        for i in range(R):
            kinds.append((s, i // B, i))
    vis = np.zeros((T, T), dtype=bool)
    for qi, (qs, qb, qx) in enumerate(kinds):
        for ki, (ks, kb, kx) in enumerate(kinds):
            if ks == "prefix":
                ok = qs != "prefix" or kx <= qx
            elif qs == "prefix":
                ok = False
            elif qs == "clean":
                ok = ks == "clean" and kx <= qx
            else:  # corrupted query
                ok = (ks == "clean" and kb < qb) or (ks == qs and kb == qb)
            vis[qi, ki] = ok
    return vis, kinds

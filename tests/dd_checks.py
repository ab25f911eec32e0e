"""Shared checks of direct block-diffusion GPU tests (not a test module)."""

import numpy as np

from oracle import argmax_excluding, select_positions


def softmax_conf(logits, mask_id):
    """Softmax probability of the greedy token, [M] excluded, in float64."""
    z = np.asarray(logits, dtype=np.float64).copy()
    z[mask_id] = -np.inf
    return 1.0 / np.exp(z - z.max()).sum()


def decisions_safe(step_conf, step_of, tau, delta):
    """No decision of the block lies within delta of the threshold or of a fallback tie."""
    B = len(step_of)
    for k, conf in enumerate(step_conf):
        und = [j for j in range(B) if step_of[j] >= k]
        if any(abs(conf[j] - tau) <= delta for j in und):
            return False
        if not any(conf[j] >= tau for j in und) and len(und) > 1:
            top = sorted((conf[j] for j in und), reverse=True)
            if top[0] - top[1] <= delta:
                return False
    return True


def check_block_against_own_outputs(ex, toks, tau, B, mask_id, conf_rtol=1e-5):
    """Decisions and tokens of a GPU block, replayed from the GPU's own numbers.

    The commit rule re-evaluated in float32 on the GPU's confidences gives the
    GPU's step indices exactly; committed tokens are the greedy tokens of the
    step that committed them; with logits, the greedy tokens are the argmax of
    the GPU's logits and the confidences their float64 softmax within conf_rtol.
    """
    conf, stok, step_of = ex["conf"], ex["tok"], ex["step_of"]
    tau32 = float(np.float32(tau))
    for k in range(conf.shape[0]):
        und = [step_of[j] >= k for j in range(B)]
        got = [j for j in range(B) if step_of[j] == k]
        assert got == select_positions(und, [float(c) for c in conf[k]], tau32), f"step {k}"
        for j in got:
            assert toks[j] == stok[k][j]
    if "logits" in ex:
        lg = ex["logits"].cpu().numpy()
        for k in range(conf.shape[0]):
            for j in range(B):
                assert stok[k][j] == argmax_excluding(lg[k][j], mask_id)[0]
                c = softmax_conf(lg[k][j], mask_id)
                assert abs(conf[k][j] - c) <= conf_rtol * c, (k, j, conf[k][j], c)

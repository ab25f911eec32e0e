"""GPU parity of stochastic self-speculative decoding (tiny fp32 decoder)
against the CPU oracle, through the C ABI.  Uniforms are seeded inputs,
rounded to float32 and given to both sides.

Bars:
  * draft and verify logits within max-abs 2e-2 of the float64 oracle (fp32
    arithmetic lands below 1e-4);
  * every draw and every acceptance decision of a GPU round replayed in
    float64 from the GPU's own logits: valid inverse-CDF draws, decisions
    following the rule, up to 1e-4 relative at a boundary;
  * A and the committed tokens equal to the oracle's wherever no draw or
    decision the outcome depends on lies within 2e-5 relative of a boundary;
  * at a vanishing temperature the stochastic round equals the greedy round;
  * free-running stochastic decoding equal to the oracle's where unambiguous;
    AR sampling through the same kernels.
"""

import numpy as np
import pytest
import torch

from ssb_inputs import generate_weights, prefix_embeddings, workload
from oracle import Decoder, prefill
from oracle.stochastic import probs, residual, spec_decode_sample, spec_round_sample, prefill_sample
from sample_checks import draw_safe, replay_round

pytestmark = pytest.mark.gpu

LOGIT_TOL = 2e-2
SAFE = 2e-5     # fp32 cumulative sums over 512 tokens are good to ~1e-6 relative


@pytest.fixture(scope="module")
def tiny():
    from self_speculative_block_amd.engine import Model, Pool
    wl = workload(1)
    cfg = wl.model
    w = generate_weights(cfg)
    model = Model(cfg, w, block_B=wl.block, max_rows=256, max_positions=256)
    pool = Pool(model, n_pages=64)
    yield wl, cfg, w, model, pool, Decoder(cfg, w)
    pool.close()
    model.close()


def _kv(pool, n=200):
    from self_speculative_block_amd.engine import KV
    return KV(pool, n)


def _uniforms(seed, shape):
    return np.random.default_rng([2024, seed]).random(shape).astype(np.float32)


def _oracle_round_safe(r, u, B, T, mask_id):
    """No draw or decision of an oracle round lies within SAFE of a boundary."""
    u = np.asarray(u, dtype=np.float64)
    q = [probs(r.draft_logits[j], mask_id, T) for j in range(B + 1)]
    p = [probs(r.verify_logits[j], mask_id, T) for j in range(B + 1)]
    if not draw_safe(q[0], u[0], SAFE):
        return False
    for j in range(1, min(r.A + 1, B) + 1):     # the draws the outcome depends on
        if not draw_safe(q[j], u[j], SAFE):
            return False
    for j in range(1, min(r.A + 1, B) + 1):
        d = r.d[j - 1]
        lhs, rhs = u[B + j] * q[j][d], p[j - 1][d]
        if abs(lhs - rhs) <= SAFE * max(lhs, rhs):
            return False
    w = residual(p[r.A], q[r.A + 1]) if r.A < B else p[B]
    return w.sum() > 0 and draw_safe(w, u[2 * B + 1], SAFE)


@pytest.mark.parametrize("T", [1.0, 0.05])
def test_round_sample_matches_oracle(tiny, T):
    wl, cfg, w, model, pool, orc = tiny
    B = wl.block
    exact = 0
    seen_A = set()
    for s in range(6):
        pre = prefix_embeddings(wl.wid, s, wl.prefix_len, cfg.hidden)
        kv = _kv(pool)
        kv.prefill(model.prefix_tensor(pre))
        st, _, _ = prefill(orc, pre, wl.prefix_len + 5 * (B + 2))
        for k in range(4):
            u = _uniforms(100 * s + k, 2 * B + 2)
            u_dev = torch.tensor(u, device="cuda")
            committed, A, dl, vl = kv.round_sample(B, u_dev, temperature=T, want_logits=True)
            dl, vl = dl.cpu().numpy(), vl.cpu().numpy()
            replay_round(dl, vl, u, B, T, cfg.mask_id, cfg.eos_id, committed, A)
            r = spec_round_sample(orc, st, B, u.astype(np.float64), temperature=T, keep_logits=True)
            assert np.abs(dl - r.draft_logits).max() < min(LOGIT_TOL, 1e-4)
            assert np.abs(vl - r.verify_logits).max() < min(LOGIT_TOL, 1e-4)
            if not _oracle_round_safe(r, u, B, T, cfg.mask_id):
                break
            assert committed == r.committed and A == r.A
            assert kv.state()[:2] == (st.n, st.x0)
            exact += 1
            seen_A.add(A)
        kv.close()
    assert exact >= 12 and len(seen_A) >= 2


def test_vanishing_temperature_is_greedy(tiny):
    wl, cfg, w, model, pool, orc = tiny
    B = wl.block
    same = total = 0
    for s in range(6):
        pre = model.prefix_tensor(prefix_embeddings(wl.wid, s, wl.prefix_len, cfg.hidden))
        kv_g, kv_s = _kv(pool), _kv(pool)
        kv_g.prefill(pre)
        kv_s.prefill(pre)
        for k in range(3):
            u_dev = torch.tensor(_uniforms(900 + 10 * s + k, 2 * B + 2), device="cuda")
            cg, Ag, _, _ = kv_g.round(B)
            cs, As, _, _ = kv_s.round_sample(B, u_dev, temperature=1e-6)
            total += 1
            if (cg, Ag) == (cs, As):
                same += 1
            else:
                break
        kv_g.close()
        kv_s.close()
    assert same >= total - 1 and same >= 12


def test_decode_sample_matches_oracle_and_ar_sampling_runs(tiny):
    wl, cfg, w, model, pool, orc = tiny
    B = wl.block
    T = 0.05
    agree = 0
    for s in range(8):
        pre_np = prefix_embeddings(wl.wid, s, wl.prefix_len, cfg.hidden)
        pre = model.prefix_tensor(pre_np)
        U = _uniforms(5000 + s, (40, 2 * B + 2))
        kv = _kv(pool)
        got, st = kv.decode_sample(pre, B, 40, torch.tensor(U, device="cuda"), temperature=T)
        kv.reset()
        assert 1 <= len(got) <= 40 and st.rounds >= 1 and st.forwards == 2 * st.rounds
        rounds = []
        ref = spec_decode_sample(orc, pre_np, B, 40, U.astype(np.float64), temperature=T, rounds_out=rounds)
        if got == ref:
            agree += 1
        # AR sampling: y1 drawn with the same first uniform as the self-speculative decode
        ua = torch.tensor(U[:, 0].copy(), device="cuda")
        ar, sta = kv.decode_ar_sample(pre, 40, ua, temperature=T)
        kv.close()
        assert ar[0] == got[0] and 1 <= len(ar) <= 40
        _, y1 = prefill_sample(orc, pre_np, wl.prefix_len + 4, float(U[0, 0]), temperature=T)
        assert ar[0] == y1
    assert agree >= 6

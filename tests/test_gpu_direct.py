"""GPU parity of direct block-diffusion decoding (tiny fp32 decoder, 2 layers,
hidden 128, vocab 512) against the CPU oracle, through the C ABI.

Bars:
  * every denoising step's logits within max-abs 2e-2 of the float64 oracle
    (fp32 arithmetic lands below 1e-4);
  * confidences within 1e-4 relative of the oracle's, and within 1e-5
    relative of the softmax of the GPU's own logits taken in float64;
  * the commit decisions exact given the GPU's own confidences (the rule
    re-evaluated in float32 on the host) and the committed tokens equal to
    the greedy tokens of the GPU's own logits;
  * tokens, step counts and step indices equal to the oracle's wherever no
    decision lies within 20x the observed confidence error of the threshold
    (or, for the most-confident fallback, of a tie);
  * block size 1 equals the GPU's AR decoding and tau = 0 equals the GPU's
    one-shot draft, exactly (the same kernels on the same rows);
  * EOS and budget cuts.
"""

import dataclasses

import numpy as np
import pytest
import torch

from ssb_inputs import generate_weights, prefix_embeddings, workload
from oracle import Decoder, argmax_excluding, dd_cache_write, dd_decode, dd_fill, prefill
from dd_checks import check_block_against_own_outputs, decisions_safe as _safe

pytestmark = pytest.mark.gpu

LOGIT_TOL = 2e-2


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


def _mid_tau(orc, pre, B):
    st, _, _ = prefill(orc, pre, pre.shape[0] + B + 4)
    return float(np.median(dd_fill(orc, st, B, 2.0).step_conf[0]))


def test_dd_blocks_match_oracle(tiny):
    wl, cfg, w, model, pool, orc = tiny
    B = wl.block
    checked = 0
    for s in range(6):
        pre = prefix_embeddings(wl.wid, s, wl.prefix_len, cfg.hidden)
        tau = _mid_tau(orc, pre, B)
        kv = _kv(pool)
        kv.prefill(model.prefix_tensor(pre))
        st, _, _ = prefill(orc, pre, wl.prefix_len + 4 * B + 4)
        for blk in range(3):
            toks, n, steps, ex = kv.dd_block(B, tau, want_steps=True, want_logits=True)
            r = dd_fill(orc, st, B, tau, keep_logits=True)
            check_block_against_own_outputs(ex, toks, tau, B, cfg.mask_id)
            k = min(steps, r.steps)
            lg = ex["logits"][:k].cpu().numpy()
            err = np.abs(lg - np.stack(r.step_logits[:k])).max()
            assert err < LOGIT_TOL and err < 1e-4, err
            cerr = np.abs(ex["conf"][:k] - np.array(r.step_conf[:k])) / np.array(r.step_conf[:k])
            assert cerr.max() < 1e-4, cerr.max()
            if not _safe(r.step_conf, r.step_of, tau, 20 * cerr.max() * max(map(max, r.step_conf))):
                kv.close()
                break
            assert toks == r.tokens and steps == r.steps and ex["step_of"] == r.step_of and n == B
            checked += 1
            dd_cache_write(orc, st, r.tokens)
            assert kv.state()[:2] == (st.n, st.x0)
        else:
            kv.close()
    assert checked >= 10


def test_dd_decode_block_one_is_gpu_ar(tiny):
    wl, cfg, w, model, pool, orc = tiny
    for s in range(8):
        pre = model.prefix_tensor(prefix_embeddings(wl.wid, s, wl.prefix_len, cfg.hidden))
        kv = _kv(pool)
        ar, _ = kv.decode_ar(pre, 40)
        kv.reset()
        for tau in (0.0, 0.5):
            dd, st = kv.decode_dd(pre, 1, tau, 40)
            kv.reset()
            assert dd == ar, (s, tau)
            assert st.forwards == len(dd) - 1 and st.cache_forwards == 0
        kv.close()


def test_dd_tau_zero_block_is_gpu_draft(tiny):
    wl, cfg, w, model, pool, orc = tiny
    B = wl.block
    for s in range(4):
        pre = model.prefix_tensor(prefix_embeddings(wl.wid, s, wl.prefix_len, cfg.hidden))
        kv = _kv(pool)
        y1 = kv.prefill(pre)
        toks, n, steps, ex = kv.dd_block(B, 0.0, write_cache=False, want_steps=True)
        assert steps == 1 and ex["step_of"] == [0] * B
        assert kv.state()[:2] == (wl.prefix_len, y1)
        _, _, dl, _ = kv.round(B, want_logits=True)
        dl = dl.cpu().numpy()
        draft = [argmax_excluding(dl[j], cfg.mask_id)[0] for j in range(B)]
        assert toks == draft
        kv.close()


def test_dd_decode_matches_oracle_eos_and_budget(tiny):
    wl, cfg, w, model, pool, orc = tiny
    from self_speculative_block_amd.engine import Model, Pool
    B = 4
    agree = 0
    eos_checked = False
    for s in range(8, 20):
        pre_np = prefix_embeddings(wl.wid, s, wl.prefix_len, cfg.hidden)
        tau = _mid_tau(orc, pre_np, B)
        pre = model.prefix_tensor(pre_np)
        kv = _kv(pool)
        full, st = kv.decode_dd(pre, B, tau, 30)
        kv.reset()
        if cfg.eos_id in full:
            kv.close()
            continue
        blocks = []
        ref, rst = dd_decode(orc, pre_np, B, tau, 30, blocks_out=blocks)
        assert len(full) == 30 and st.rounds == 8 and st.cache_forwards == 7
        if all(_safe(b.step_conf, b.step_of, tau, 1e-4 * tau) for b in blocks):
            assert full == ref and st.forwards == rst.steps
            agree += 1
        for max_len in (1, 2, 5, 13):
            got, _ = kv.decode_dd(pre, B, tau, max_len)
            kv.reset()
            assert got == full[:max_len]
        ks = [i for i in range(9, 13) if full[i] not in full[:i]]
        kv.close()
        if ks and not eos_checked:
            eos_checked = True
            k = ks[0]
            cfg2 = dataclasses.replace(cfg, eos_id=full[k])
            m2 = Model(cfg2, w, block_B=wl.block, max_rows=64, max_positions=256)
            p2 = Pool(m2, n_pages=32)
            from self_speculative_block_amd.engine import KV
            kv2 = KV(p2, 200)
            out, st2 = kv2.decode_dd(m2.prefix_tensor(pre_np), B, tau, 30)
            assert out == full[: k + 1] and st2.rounds == 3 and st2.cache_forwards == 2
            kv2.close()
            p2.close()
            m2.close()
    assert agree >= 6 and eos_checked


# ---- multi-step draft schedule ----

def test_multistep_one_step_is_gpu_round(tiny):
    wl, cfg, w, model, pool, orc = tiny
    B = wl.block
    for s in range(4):
        pre = model.prefix_tensor(prefix_embeddings(wl.wid, s, wl.prefix_len, cfg.hidden))
        a, b = _kv(pool), _kv(pool)
        a.prefill(pre)
        b.prefill(pre)
        for k in range(3):
            c1, A1, k1, v1 = a.round_multistep(B, 1, 0.5, want_logits=True)
            c2, A2, _, v2 = b.round(B, want_logits=True)
            assert (c1, A1, k1) == (c2, A2, 1)
            assert torch.equal(v1, v2)
            assert a.state()[:2] == b.state()[:2]
        a.close()
        b.close()


def test_multistep_decode_is_gpu_ar_and_matches_oracle(tiny):
    from oracle import spec_round_multistep
    wl, cfg, w, model, pool, orc = tiny
    B = wl.block
    checked = 0
    for s in range(4):
        pre_np = prefix_embeddings(wl.wid, s, wl.prefix_len, cfg.hidden)
        pre = model.prefix_tensor(pre_np)
        tau = _mid_tau(orc, pre_np, B)
        kv = _kv(pool)
        ar, _ = kv.decode_ar(pre, 40)
        for steps in (2, 4):
            kv.reset()
            out, st = kv.decode_multistep(pre, B, steps, tau, 40)
            assert out == ar, (s, steps)
            assert st.rounds <= st.forwards - st.rounds <= steps * st.rounds
        # round by round against the oracle while no draft decision is near the threshold
        kv.reset()
        kv.prefill(pre)
        ost, _, _ = prefill(orc, pre_np, wl.prefix_len + 5 * (B + 2))
        for k in range(3):
            c, A, nf, vl = kv.round_multistep(B, 3, tau, want_logits=True)
            r = spec_round_multistep(orc, ost, B, 3, tau, keep_logits=True)
            if (c, A, nf) != (r.committed, r.A, r.draft_forwards):
                break          # a draft decision within rounding of the threshold
            assert np.abs(vl.cpu().numpy() - r.verify_logits).max() < 1e-4
            assert kv.state()[:2] == (ost.n, ost.x0)
            checked += 1
        kv.close()
    assert checked >= 6


def test_error_paths_of_the_decoding_modes(tiny):
    """Bad arguments of the direct-diffusion, stochastic and draft-schedule calls fail with a
    code and leave the committed state unchanged."""
    from self_speculative_block_amd import SsbError, SSB_EINVAL, SSB_ENOKV, SSB_ESTATE
    from self_speculative_block_amd.engine import KV, ar_step_batch, serve
    from self_speculative_block_amd._lib import SSB_SERVE_SPEC
    wl, cfg, w, model, pool, orc = tiny
    B = wl.block
    pre = model.prefix_tensor(prefix_embeddings(wl.wid, 0, wl.prefix_len, cfg.hidden))
    kv = _kv(pool)

    def code(fn):
        with pytest.raises(SsbError) as e:
            fn()
        return e.value.code

    u = torch.rand(2 * B + 2, device="cuda")
    assert code(lambda: kv.dd_block(B, 0.5)) == SSB_ESTATE          # no prefill yet
    assert code(lambda: kv.round_sample(B, u)) == SSB_ESTATE
    assert code(lambda: kv.round_multistep(B, 2, 0.5)) == SSB_ESTATE
    kv.prefill(pre)
    st0 = kv.state()
    assert code(lambda: kv.dd_block(0, 0.5)) == SSB_EINVAL
    assert code(lambda: kv.dd_block(B + 1, 0.5)) == SSB_EINVAL
    assert code(lambda: kv.dd_block(B, float("nan"))) == SSB_EINVAL
    assert code(lambda: kv.dd_block(B, 0.5, max_commit=0)) == SSB_EINVAL
    assert code(lambda: kv.round_sample(B, u, temperature=0.0)) == SSB_EINVAL
    assert code(lambda: kv.round_sample(B, u, temperature=float("inf"))) == SSB_EINVAL
    assert code(lambda: kv.round_sample(B, None)) == SSB_EINVAL
    assert code(lambda: kv.round_multistep(B, 0, 0.5)) == SSB_EINVAL
    assert code(lambda: kv.round_multistep(0, 1, 0.5)) == SSB_EINVAL
    assert code(lambda: kv.decode_sample(pre, B, 40, torch.rand((1, 2 * B + 2), device="cuda"))) == SSB_ESTATE
    assert kv.state() == st0
    # the sampling decode runs out of uniforms: an error, not a read past the array
    kv.reset()
    assert code(lambda: kv.decode_sample(pre, B, 40, torch.rand((1, 2 * B + 2), device="cuda"))) == SSB_EINVAL
    kv.close()
    small = KV(pool, wl.prefix_len + 4)
    small.prefill(pre)
    assert code(lambda: small.dd_block(B, 0.5)) == SSB_ENOKV
    assert code(lambda: small.round_multistep(B, 2, 0.5)) == SSB_ENOKV
    assert small.state()[0] == wl.prefix_len
    assert code(lambda: ar_step_batch(model, [small, small])) == SSB_EINVAL   # the same kv twice
    small.close()
    reqs = [{"prefix_dev": pre, "max_len": 10}]
    assert code(lambda: serve(model, pool, reqs, 0, SSB_SERVE_SPEC, B=B)) == SSB_EINVAL
    assert code(lambda: serve(model, pool, reqs, 2, 7, B=B)) == SSB_EINVAL
    assert code(lambda: serve(model, pool, reqs, 2, SSB_SERVE_SPEC, B=B, max_tokens=wl.prefix_len + 4)) == SSB_EINVAL

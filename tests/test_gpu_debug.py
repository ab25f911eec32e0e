"""Debug checks of the round's KV handling, determinism and resumability (GPU).

* NaN poisoning: with the engine's debug poisoning on, the KV slots of every
  layer at the draft window (p+1 .. p+B+1) are set to NaN between the draft
  and the verify forward, and the rolled-back slots (p+A+2 .. p+B+1) after
  accept.  The verify must rewrite its slots before reading them, and nothing
  may read a rolled-back slot before the next window rewrites it (GravityOCR
  review, Appendix B.2: verify overwrites the draft's slots in place; only
  causal state survives a round).  Poisoned rounds must therefore give the
  same tokens, state and logits, bit for bit, as unpoisoned ones, with no NaN.
* Determinism: replaying the same round gives the same bits.
* Resume: a decode stopped at a round boundary and continued with single
  rounds equals one decode call (the state between rounds is exactly the
  cache, its length and the boundary token).
"""

import dataclasses

import numpy as np
import pytest
import torch

from ssb_inputs import generate_weights, plant_accept_lengths, prefix_embeddings, workload
from oracle import build_plant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", params=["tiny", "full1"])
def setup(request):
    from self_speculative_block_amd.engine import KV, Model, Pool
    if request.param == "tiny":
        wl = workload(1)
        cfg = wl.model
        max_pos = 256
    else:
        wl = workload(2)
        cfg = dataclasses.replace(wl.model, n_layers=1)
        max_pos = wl.prefix_len + 400
    B, P = wl.block, wl.prefix_len
    model = Model(cfg, generate_weights(cfg), block_B=B, max_rows=512, max_positions=max_pos)
    pool = Pool(model, n_pages=8 * (max_pos // 16 + 2))
    kv = KV(pool, max_pos - 8)
    pre_dev = model.prefix_tensor(prefix_embeddings(wl.wid, 3, P, cfg.hidden))
    y1 = kv.prefill(pre_dev)
    cont = [y1]
    for _ in range(3 * (B + 2) + 2):
        cont.append(kv.ar_step()[0])
    kv.rewind(P, y1)
    yield dict(wl=wl, cfg=cfg, B=B, P=P, model=model, pool=pool, kv=kv, pre_dev=pre_dev, y1=y1, cont=cont)
    model.set_debug(False)
    kv.close()
    pool.close()
    model.close()


def _planted(s, c, a):
    cfg = s["cfg"]
    return torch.tensor(build_plant(s["cont"], c, a, s["B"], cfg.vocab, cfg.mask_id), dtype=torch.int32,
                        device="cuda")


def _rounds(s, astars, poison):
    """Consecutive rounds from the prefilled state with planted accept lengths; per round the
    committed tokens, A, state and both logits."""
    kv, model, B = s["kv"], s["model"], s["B"]
    kv.rewind(s["P"], s["y1"])
    model.set_debug(poison)
    try:
        out, c = [], 1
        for a in astars:
            toks, A, dl, vl = kv.round(B, planted_dev=_planted(s, c, a), want_logits=True)
            out.append((toks, A, kv.state(), dl, vl))
            c += len(toks)
        return out
    finally:
        model.set_debug(False)


def test_poisoned_rounds_equal_unpoisoned(setup):
    s = setup
    B = s["B"]
    for astars in ([0], [1], [B // 2], [B], [2, 0, B], [B, 3, 1]):
        ref = _rounds(s, astars, poison=False)
        got = _rounds(s, astars, poison=True)
        for k, ((t0, a0, st0, d0, v0), (t1, a1, st1, d1, v1)) in enumerate(zip(ref, got)):
            assert (t1, a1, st1) == (t0, a0, st0), f"round {k} of {astars}"
            assert not torch.isnan(d1).any() and not torch.isnan(v1).any(), f"NaN reached the logits ({astars})"
            assert torch.equal(d1, d0) and torch.equal(v1, v0), f"round {k} of {astars}: logits changed"
            assert a1 == min(astars[k], B)


def test_poisoned_batched_round_equals_unpoisoned(setup):
    from self_speculative_block_amd.engine import KV, round_batch
    s = setup
    model, pool, cfg, B, P = s["model"], s["pool"], s["cfg"], s["B"], s["P"]
    kvs, firsts, plants = [], [], []
    for i, (a, extra) in enumerate([(0, 0), (B // 2, 5), (B, 11)]):
        kv = KV(pool, P + extra + 2 * B + 8)
        pre = model.prefix_tensor(prefix_embeddings(s["wl"].wid, 20 + i, P + extra, cfg.hidden))
        y = kv.prefill(pre)
        cont = [y] + [kv.ar_step()[0] for _ in range(B + 2)]
        kv.rewind(P + extra, y)
        kvs.append(kv)
        firsts.append((P + extra, y))
        plants.append(build_plant(cont, 1, a, B, cfg.vocab, cfg.mask_id))
    planted = torch.tensor(plants, dtype=torch.int32, device="cuda")
    results = []
    for poison in (False, True):
        for kv, (n, y) in zip(kvs, firsts):
            kv.rewind(n, y)
        model.set_debug(poison)
        try:
            res, dl, vl = round_batch(model, kvs, B, [B + 2] * 3, planted_dev=planted, want_logits=True)
        finally:
            model.set_debug(False)
        results.append((res, [kv.state() for kv in kvs], dl, vl))
    (r0, s0, d0, v0), (r1, s1, d1, v1) = results
    assert r1 == r0 and s1 == s0
    assert not torch.isnan(d1).any() and not torch.isnan(v1).any()
    assert torch.equal(d1, d0) and torch.equal(v1, v0)
    for kv in kvs:
        kv.close()


def test_round_replay_is_deterministic(setup):
    s = setup
    kv, B = s["kv"], s["B"]
    runs = []
    for _ in range(3):        # graph replays
        kv.rewind(s["P"], s["y1"])
        runs.append((kv.round(B, planted_dev=_planted(s, 1, B // 2))[:2], kv.state()))
    assert runs[1] == runs[0] and runs[2] == runs[0]
    logits = []
    for _ in range(2):        # eager, with logits
        kv.rewind(s["P"], s["y1"])
        toks, A, dl, vl = kv.round(B, planted_dev=_planted(s, 1, B // 2), want_logits=True)
        assert (toks, A) == runs[0][0]
        logits.append((dl, vl))
    assert torch.equal(logits[0][0], logits[1][0]) and torch.equal(logits[0][1], logits[1][1])


def test_decode_resumes_across_calls(setup):
    """Decode to a round boundary, then continue with single planted rounds: the output equals
    one decode call.  A* is planted; rounds commit A* + 2 tokens, so the boundary after K rounds
    is 1 + sum(A*_k + 2) tokens."""
    s = setup
    kv, cfg, B = s["kv"], s["cfg"], s["B"]
    ar = s["cont"]
    L = len(ar) - (B + 2)          # every planted draft stays inside the AR continuation
    if cfg.eos_id in ar[:L]:
        L = ar.index(cfg.eos_id) + 1
    astar = plant_accept_lengths(s["wl"].wid, 7, L, B, 0.8)
    cont_dev = torch.tensor(ar, dtype=torch.int32, device="cuda")
    kv.reset()
    full, _ = kv.decode(s["pre_dev"], B, L, cont_dev=cont_dev, astar=astar)
    K, L1 = 0, 1
    while K < len(astar) and L1 + int(astar[K]) + 2 < L:
        L1 += min(int(astar[K]), B) + 2
        K += 1
    if K == 0:
        pytest.skip("the first round already reaches the length")
    kv.reset()
    out, _ = kv.decode(s["pre_dev"], B, L1, cont_dev=cont_dev, astar=astar[:K])
    assert out == full[:L1]
    assert kv.state()[:2] == (s["P"] + L1 - 1, out[-1])
    k = K
    while len(out) < L and out[-1] != cfg.eos_id:
        a = int(astar[k]) if k < len(astar) else B
        toks, A, _, _ = kv.round(B, max_commit=L - len(out), planted_dev=_planted(s, len(out), a))
        out += toks
        k += 1
    assert out == full


def test_poison_hook_control(setup):
    """Control of the poisoning: NaN written into slots the next window rewrites first leaves the
    round unchanged bit for bit; NaN in a committed slot the round reads makes it fail with
    SSB_EHIP (NaN logits), and the kv's state stays as it was."""
    from self_speculative_block_amd._lib import SSB_EHIP, SsbError
    s = setup
    kv, B, P = s["kv"], s["B"], s["P"]
    ref = _rounds(s, [B // 2], poison=False)[0]
    kv.rewind(P, s["y1"])
    kv.poison(P, P + B + 1)                  # the draft window's slots: rewritten before any read
    toks, A, dl, vl = kv.round(B, planted_dev=_planted(s, 1, B // 2), want_logits=True)
    assert (toks, A, kv.state()) == ref[:3]
    assert torch.equal(dl, ref[3]) and torch.equal(vl, ref[4])
    kv.rewind(P, s["y1"])
    kv.poison(P - 1, P)                      # the last committed slot: every window row reads it
    with pytest.raises(SsbError) as e:
        kv.round(B, planted_dev=_planted(s, 1, B // 2))
    assert e.value.code == SSB_EHIP
    assert kv.state()[:2] == (P, s["y1"])
    kv.reset()                               # drop the poisoned cache; later tests prefill again
    assert kv.prefill(s["pre_dev"]) == s["y1"]


def test_graphs_do_not_outlive_their_pool():
    """Captured round graphs bake in the pool's device buffer.  A pool freed and followed by a new
    pool (often at the same host address, with a different buffer) must not replay them: rounds in
    the new pool give the same results as in the first one."""
    from self_speculative_block_amd.engine import KV, Model, Pool
    wl = workload(1)
    cfg, B, P = wl.model, wl.block, wl.prefix_len
    model = Model(cfg, generate_weights(cfg), block_B=B, max_rows=64, max_positions=256)
    pre_dev = model.prefix_tensor(prefix_embeddings(wl.wid, 5, P, cfg.hidden))
    results = []
    for n_pages in (40, 24, 40):
        pool = Pool(model, n_pages=n_pages)
        kv = KV(pool, 200)
        kv.prefill(pre_dev)
        got = [kv.round(B)[:2] for _ in range(3)]        # graph capture, then replays
        got.append(kv.ar_step()[0])
        results.append(got)
        kv.close()
        pool.close()
    assert results[1] == results[0] and results[2] == results[0]
    model.close()


def _other_token(t, cfg):
    u = (t + 7) % cfg.vocab
    return (u + 1) % cfg.vocab if u == cfg.mask_id else u


def test_verify_rows_see_only_earlier_window_rows(setup):
    """Causal verify visibility on the GPU (GravityOCR review, section 3.2: verify row i attends
    to the cache and window rows <= i).  Changing the planted draft d_j leaves verify rows
    0..j-1 bit-identical and changes row j; the draft forward runs before planting and is
    unchanged."""
    s = setup
    kv, cfg, B, P = s["kv"], s["cfg"], s["B"], s["P"]
    base = build_plant(s["cont"], 1, B, B, cfg.vocab, cfg.mask_id)
    for j in sorted({1, B // 2, B}):
        pert = list(base)
        pert[j - 1] = _other_token(pert[j - 1], cfg)
        outs = []
        for plant in (base, pert):
            kv.rewind(P, s["y1"])
            outs.append(kv.round(B, planted_dev=torch.tensor(plant, dtype=torch.int32, device="cuda"),
                                 want_logits=True))
        (_, _, d0, v0), (_, _, d1, v1) = outs
        assert torch.equal(d0, d1)
        assert torch.equal(v0[:j], v1[:j]), f"a verify row before {j} saw d_{j}"
        assert not torch.equal(v0[j], v1[j])


def test_batched_requests_are_isolated(setup):
    """In a batched round, changing one request's planted drafts changes nothing, bit for bit, in
    another request's draft and verify logits."""
    from self_speculative_block_amd.engine import KV, round_batch
    s = setup
    model, pool, cfg, B, P = s["model"], s["pool"], s["cfg"], s["B"], s["P"]
    kvs, firsts, plants = [], [], []
    for i in range(2):
        kv = KV(pool, P + 2 * B + 8)
        y = kv.prefill(model.prefix_tensor(prefix_embeddings(s["wl"].wid, 40 + i, P, cfg.hidden)))
        cont = [y] + [kv.ar_step()[0] for _ in range(B + 2)]
        kv.rewind(P, y)
        kvs.append(kv)
        firsts.append(y)
        plants.append(build_plant(cont, 1, B, B, cfg.vocab, cfg.mask_id))
    pert = [list(plants[0]), [_other_token(t, cfg) for t in plants[1]]]
    outs = []
    for pl in (plants, pert):
        for kv, y in zip(kvs, firsts):
            kv.rewind(P, y)
        res, dl, vl = round_batch(model, kvs, B, [B + 2] * 2, planted_dev=torch.tensor(pl, dtype=torch.int32,
                                                                                      device="cuda"), want_logits=True)
        outs.append((res, dl, vl))
    rows0 = slice(0, B + 1)
    assert outs[0][0][0] == outs[1][0][0]
    assert torch.equal(outs[0][1][rows0], outs[1][1][rows0]) and torch.equal(outs[0][2][rows0], outs[1][2][rows0])
    assert not torch.equal(outs[0][2][B + 2:], outs[1][2][B + 2:])   # request 1's verify rows did change
    for kv in kvs:
        kv.close()

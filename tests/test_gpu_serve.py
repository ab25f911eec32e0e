"""Continuous batching and the batched AR step on the GPU (tiny fp32 decoder),
through the C ABI.

Bars:
  * a batched AR step gives every request the token of its own AR step (exact);
  * serving a queue under any cap on running requests (1 .. 64) gives every
    request the output of its own AR decode, in AR mode and in
    self-speculative mode, with and without planted drafts (exact); planted
    accept lengths are realised (rounds per request);
  * every served output against the oracle's greedy AR decode of the same
    prefix: equal, or departing only where the oracle's top-2 margin is below
    1e-2 (every departure of the teacher-forced comparison; GravityOCR review,
    Appendix B.3);
  * per-request and aggregate accounting (tokens, prefills, launches).
"""

import numpy as np
import pytest
import torch

from ssb_inputs import generate_weights, prefix_embeddings, workload
from oracle import Decoder, ar_decode, teacher_forced_argmax

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny():
    from self_speculative_block_amd.engine import Model, Pool
    wl = workload(1)
    cfg = wl.model
    w = generate_weights(cfg)
    model = Model(cfg, w, block_B=wl.block, max_rows=64 * (wl.block + 1), max_positions=256)
    pool = Pool(model, n_pages=80 * 12)
    ORACLE["orc"] = Decoder(cfg, w)
    yield wl, cfg, model, pool
    pool.close()
    model.close()


ORACLE = {}


def _queue(wl, cfg, model, n, lens):
    return [{"prefix_dev": model.prefix_tensor(prefix_embeddings(wl.wid, i, wl.prefix_len, cfg.hidden)),
             "pre": prefix_embeddings(wl.wid, i, wl.prefix_len, cfg.hidden), "max_len": lens[i]} for i in range(n)]


def _check_against_oracle(reqs, outs, near_tie=1e-2):
    """Each served output equals the oracle's greedy AR decode, or departs from the oracle's
    prediction only at near-ties; returns the number of outputs identical to the oracle's."""
    orc = ORACLE["orc"]
    same = 0
    for q, o in zip(reqs, outs):
        key = (q["pre"].tobytes(), q["max_len"])
        if key not in ORACLE:
            ORACLE[key] = ar_decode(orc, q["pre"], q["max_len"])
        if o == ORACLE[key]:
            same += 1
            continue
        preds, margins = teacher_forced_argmax(orc, q["pre"], o)
        for t in range(len(o)):
            if o[t] != preds[t]:
                assert margins[t] < near_tie, (t, o[t], preds[t], margins[t])
        # a shorter or longer output must end at an EOS or the request's budget
        assert len(o) == q["max_len"] or o[-1] == orc.cfg.eos_id
    return same


def _ar_outputs(pool, reqs):
    from self_speculative_block_amd.engine import KV
    kv = KV(pool, 200)
    outs = []
    for q in reqs:
        kv.reset()
        outs.append(kv.decode_ar(q["prefix_dev"], q["max_len"])[0])
    kv.close()
    return outs


def test_batched_ar_step_equals_single_steps(tiny):
    from self_speculative_block_amd.engine import KV, ar_step_batch
    wl, cfg, model, pool = tiny
    pres = [model.prefix_tensor(prefix_embeddings(wl.wid, i, wl.prefix_len, cfg.hidden)) for i in range(5)]
    single = []
    for p in pres:
        kv = KV(pool, 200)
        kv.prefill(p)
        single.append([kv.ar_step()[0] for _ in range(6)])
        kv.close()
    kvs = [KV(pool, 200) for _ in pres]
    for kv, p in zip(kvs, pres):
        kv.prefill(p)
    got = [ar_step_batch(model, kvs) for _ in range(6)]
    for r in range(5):
        assert [g[r] for g in got] == single[r]
    for kv in kvs:
        kv.close()


@pytest.mark.parametrize("cap", [1, 3, 8, 64])
def test_serve_ar_and_spec_equal_ar_decode(tiny, cap):
    from self_speculative_block_amd.engine import serve
    from self_speculative_block_amd._lib import SSB_SERVE_AR, SSB_SERVE_SPEC
    wl, cfg, model, pool = tiny
    n = 70 if cap == 64 else 12
    lens = [int(x) for x in np.random.default_rng([3, cap]).integers(1, 48, n)]
    reqs = _queue(wl, cfg, model, n, lens)
    ref = _ar_outputs(pool, reqs)
    out, info, st = serve(model, pool, reqs, cap, SSB_SERVE_AR)
    assert out == ref
    assert st["prefills"] == n and st["tokens"] == sum(len(o) for o in ref)
    assert st["steps"] >= max(len(o) for o in ref) - 1 and st["mean_running"] <= cap
    assert all(info[i]["rounds"] == len(ref[i]) - 1 for i in range(n))
    out, info, st = serve(model, pool, reqs, cap, SSB_SERVE_SPEC, B=wl.block)
    assert out == ref
    assert st["tokens"] == sum(len(o) for o in ref)
    same = _check_against_oracle(reqs, out)
    assert same >= 0.9 * n, f"{same} of {n} served outputs identical to the oracle's"


def test_serve_spec_with_planted_drafts(tiny):
    from self_speculative_block_amd.engine import serve
    from self_speculative_block_amd._lib import SSB_SERVE_SPEC
    wl, cfg, model, pool = tiny
    B = wl.block
    n = 10
    lens = [40] * n
    reqs = _queue(wl, cfg, model, n, lens)
    ref = _ar_outputs(pool, reqs)
    for i, q in enumerate(reqs):
        q["cont_dev"] = torch.tensor(ref[i], dtype=torch.int32, device="cuda")
        q["astar"] = [(i + k) % (B + 1) for k in range(40)]
    out, info, st = serve(model, pool, reqs, 4, SSB_SERVE_SPEC, B=B)
    assert out == ref
    _check_against_oracle(reqs, out)
    for i in range(n):
        if cfg.eos_id in ref[i]:
            continue
        # rounds commit A + 2 tokens each (the last one may be cut by the budget)
        c, k = 1, 0
        while c < 40:
            c += (i + k) % (B + 1) + 2
            k += 1
        assert info[i]["rounds"] == k, i

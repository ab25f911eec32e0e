"""GPU parity of the full-width decoder (bf16 weights, fp16 activations and KV cache, fp32
accumulation) against the float64 oracle, at the round microbenchmark's shape: hidden 1024, 16
query heads over 4 KV heads of 64, SwiGLU 4096, vocab 60000; n = 1280 cached positions; B = 32;
batch 1 (the launch configuration bench.py times), plus ragged batched rounds.  Stacks of 1 and
24 layers.

Bars, the same at every stack depth:
  * logits within max-abs 2e-2 of the oracle;
  * argmax decisions (a0, d_j, a_j, y1) equal wherever the oracle's top-2 margin exceeds twice
    the logit error measured on the same rows (a flip needs a smaller margin), and at least 1e-2;
    accept lengths and committed tokens exact when no decision on the accepted path is that close;
  * teacher-forced tokens: every position where a GPU-decoded sequence departs from the oracle's
    prediction for it sits at an oracle top-2 margin below 1e-2 (GravityOCR review, Appendix B.3:
    divergences are traced to near-ties);
  * GPU self-speculative decoding identical to GPU AR decoding (exact);
  * a batched round identical, request by request, to single rounds (exact), and each request's
    logits, accept length and tokens against the oracle at its own ragged state (one layer).

The oracle's 1280-position prefill of the 24-layer stack takes 10-20 s on the host, so each
stack is one module fixture.
"""

import numpy as np
import pytest
import torch

from ssb_inputs import generate_weights, prefix_embeddings, workload
from oracle import Decoder, ar_step, build_plant, dd_fill, prefill, spec_round, teacher_forced_argmax
from oracle.model import argmax_excluding
from dd_checks import check_block_against_own_outputs
from sample_checks import replay_round
from round_checks import check_round

pytestmark = pytest.mark.gpu

LOGIT_TOL = 2e-2      # max-abs logit bar at every stack depth
NEAR_TIE = 1e-2       # oracle top-2 margin below which either token is acceptable
B = 32


def _copy_state(st):
    from oracle.decode import DecodeState
    return DecodeState(cache=st.cache.copy(), n=st.n, x0=st.x0)


def _am(logits, mask_id):
    return argmax_excluding(np.asarray(logits, dtype=np.float64), mask_id)


@pytest.fixture(scope="module", params=[1, 24], ids=["1layer", "24layers"])
def full(request):
    import dataclasses
    from self_speculative_block_amd.engine import KV, Model, Pool
    wl = workload(2)
    cfg = dataclasses.replace(wl.model, n_layers=request.param)
    P = wl.prefix_len
    w = generate_weights(cfg)
    orc = Decoder(cfg, w)
    model = Model(cfg, w, block_B=64, max_rows=2048, max_positions=P + 400)
    del w
    pool = Pool(model, n_pages=6 * (P + 400) // 16)
    pre = prefix_embeddings(wl.wid, 0, P, cfg.hidden)
    pre_dev = model.prefix_tensor(pre)
    kv = KV(pool, P + 300)
    y1 = kv.prefill(pre_dev)
    st, y1_orc, margin = prefill(orc, pre, P + 300)
    # oracle AR continuation y2..y35 from the prefilled state (plants the drafts)
    st_ar = _copy_state(st)
    cont = [y1_orc]
    margins = [margin]
    for _ in range(B + 3):
        y, mg = ar_step(orc, st_ar)
        cont.append(y)
        margins.append(mg)
    # the logit error measured on one unplanted round (draft rows, the oracle's own state) sets the
    # near-tie threshold of the decision checks: max(1e-2, twice the measured error)
    kv.rewind(P, y1_orc)
    _, _, dl0, _ = kv.round(B, want_logits=True)
    r0 = spec_round(orc, _copy_state(st), B, keep_logits=True)
    meas = float(np.abs(dl0.cpu().numpy() - r0.draft_logits).max())
    print(f"\n[{cfg.n_layers} layers] draft-logit max-abs error vs the oracle {meas:.5f}", flush=True)
    kv.rewind(P, y1)
    yield dict(wl=wl, cfg=cfg, P=P, orc=orc, model=model, pool=pool, pre=pre, pre_dev=pre_dev, kv=kv,
               y1=y1, st=st, y1_orc=y1_orc, cont=cont, cont_margins=margins, st_ar=st_ar,
               tol=LOGIT_TOL, meas=meas, tie=max(NEAR_TIE, 2 * meas))
    kv.close()
    pool.close()
    model.close()


def test_draft_logit_error_within_bar(full):
    assert full["meas"] < LOGIT_TOL, full["meas"]


def test_prefill_first_token_matches_oracle(full):
    if full["cont_margins"][0] >= full["tie"]:
        assert full["y1"] == full["y1_orc"]


@pytest.mark.parametrize("astar", [20, 0, 32])
def test_round_logits_accept_and_commit_match_oracle(full, astar):
    cfg, P, kv, orc = full["cfg"], full["P"], full["kv"], full["orc"]
    y1, cont = full["y1_orc"], full["cont"]
    if full["y1"] != y1:
        pytest.skip("the prefill token is an oracle near-tie")
    plant = build_plant(cont, 1, astar, B, cfg.vocab, cfg.mask_id)
    # GPU: state (n = P, x0 = y1), planted drafts, logits of both forwards
    kv.rewind(P, y1)
    planted = torch.tensor(plant, dtype=torch.int32, device="cuda")     # -1 keeps the draft's token
    committed, A, dl, vl = kv.round(B, planted_dev=planted, want_logits=True)
    st = full["st"]
    st.n, st.x0 = P, y1
    res = check_round(cfg, orc, st, B, plant, committed, A, dl.cpu().numpy(), vl.cpu().numpy(), full["tol"])
    if full["y1"] == y1 and res["same_rows"] >= 1:
        assert res["same_rows"] > min(astar, B)       # planted rows always agree
    if not res["tie"]:
        assert A == min(astar, B)
        assert kv.state()[:2] == (st.n, st.x0)


def test_spec_decode_equals_ar_decode_and_oracle(full):
    kv, pre_dev, cfg = full["kv"], full["pre_dev"], full["cfg"]
    max_len = 96
    kv.reset()
    spec, stats = kv.decode(pre_dev, B, max_len)
    kv.reset()
    ar, _ = kv.decode_ar(pre_dev, max_len)
    assert spec == ar
    assert stats.rounds >= 1
    # the oracle's greedy continuation agrees up to the first oracle near-tie
    ref, margins = full["cont"], full["cont_margins"]
    for k, (g, o) in enumerate(zip(ar, ref)):
        if margins[k] <= full["tie"]:
            break
        assert g == o, f"AR token {k}"
    kv.reset()
    assert kv.prefill(pre_dev) == full["y1"]


@pytest.mark.parametrize("astar", [20, 32])
def test_fused_layer_tail_equals_three_launches(full, astar):
    """Decode windows of at most 48 rows run each layer's O, gate|up and down as one fused launch
    (two grid barriers inside); the three-launch form must give the same bits: tokens, state and
    both forwards' logits, for a round and for an AR step."""
    cfg, P, kv, model = full["cfg"], full["P"], full["kv"], full["model"]
    y1 = full["y1"]
    plant = torch.tensor(build_plant(full["cont"], 1, astar, B, cfg.vocab, cfg.mask_id), dtype=torch.int32,
                         device="cuda")
    outs = []
    for unfused in (False, True):
        model.set_debug(False, unfused=unfused)
        kv.rewind(P, y1)
        c, A, dl, vl = kv.round(B, planted_dev=plant, want_logits=True)
        st = kv.state()
        kv.rewind(P, y1)
        tok, lg = kv.ar_step(want_logits=True)
        outs.append((c, A, dl, vl, st, tok, lg))
    model.set_debug(False, unfused=False)
    (c0, A0, d0, v0, s0, t0, l0), (c1, A1, d1, v1, s1, t1, l1) = outs
    assert (c0, A0, s0, t0) == (c1, A1, s1, t1)
    assert torch.equal(d0, d1) and torch.equal(v0, v1), "round logits differ between fused and unfused tails"
    assert torch.equal(l0, l1), "AR-step logits differ between fused and unfused tails"
    kv.rewind(P, y1)


@pytest.mark.parametrize("Bs", [16, 24])
def test_spec_decode_other_block_sizes_equal_ar(full, Bs):
    """Windows of 17 and 25 rows take other GEMM row tiles than the 33-row window (QKV and O in
    16-row blocks, gate|up in one 32-row block): self-speculative decoding still equals AR
    decoding token for token."""
    kv, pre_dev = full["kv"], full["pre_dev"]
    kv.reset()
    spec, stats = kv.decode(pre_dev, Bs, 64)
    kv.reset()
    ar, _ = kv.decode_ar(pre_dev, 64)
    assert spec == ar
    assert stats.rounds >= 1
    kv.reset()
    assert kv.prefill(pre_dev) == full["y1"]


@pytest.mark.parametrize("Bb,R", [(32, 4), (32, 8), (64, 4), (32, 16), (64, 16), (24, 8)])
def test_batched_round_equals_single_rounds(full, Bb, R):
    """A ragged batched round (R requests of different lengths, one launch per stage) gives each
    request exactly what its own single round gives: tokens, accept length and state, and its
    draft and verify logits bit for bit.  132 rows run the GEMMs' parallel grid; 260 and 264 rows
    the looped form (several 48-row blocks per workgroup); 528 rows the large-tile exact form for
    QKV, 1040 rows for all four layer GEMMs."""
    from self_speculative_block_amd.engine import KV, round_batch
    cfg, model, pool = full["cfg"], full["model"], full["pool"]
    wl5 = workload(5)
    lens = {4: [1088, 1000, 1100, 1200], 8: [600, 520, 700, 650, 480, 560, 610, 530],
            16: [300, 260, 340, 280, 320, 250, 310, 270, 330, 290, 260, 350, 240, 300, 280, 320]}[R]
    kvs, firsts, conts = [], [], []
    for i, P in enumerate(lens):
        pre = prefix_embeddings(wl5.wid, i, P, cfg.hidden)
        kv = KV(pool, P + 2 * Bb + 8)
        pre_dev = model.prefix_tensor(pre)
        y = kv.prefill(pre_dev)
        c = [y]
        for _ in range(Bb + 2):
            c.append(kv.ar_step()[0])
        kv.rewind(P, y)
        kvs.append(kv)
        firsts.append(y)
        conts.append(c)
    astars = ([0, Bb // 2, Bb, 3, 5, 1, Bb - 1, 7] * 2)[:R]
    budgets = ([Bb + 2, Bb + 2, 5, Bb + 2, Bb + 2, 3, Bb + 2, Bb + 2] * 2)[:R]
    plants = [build_plant(conts[r], 1, astars[r], Bb, cfg.vocab, cfg.mask_id) for r in range(R)]
    planted = torch.tensor(plants, dtype=torch.int32, device="cuda")
    got = round_batch(model, kvs, Bb, budgets, planted_dev=planted)          # graph replay
    states = [kv.state() for kv in kvs]
    for r, kv in enumerate(kvs):
        kv.rewind(lens[r], firsts[r])
    got_l, dl, vl = round_batch(model, kvs, Bb, budgets, planted_dev=planted, want_logits=True)
    assert got_l == got
    assert [kv.state() for kv in kvs] == states
    for r, kv in enumerate(kvs):
        kv.rewind(lens[r], firsts[r])
        c, A, dls, vls = kv.round(Bb, max_commit=budgets[r], planted_dev=planted[r], want_logits=True)
        assert (c, A) == got[r], f"request {r}"
        assert kv.state() == states[r]
        assert A == min(astars[r], Bb)
        assert c == conts[r][1: 1 + min(A + 2, budgets[r])]
        rows = slice(r * (Bb + 1), (r + 1) * (Bb + 1))
        assert torch.equal(dl[rows], dls), f"request {r}: draft logits differ from its single round"
        assert torch.equal(vl[rows], vls), f"request {r}: verify logits differ from its single round"
    if cfg.n_layers == 1 and R == 16:
        # each request against the oracle at its own ragged state (lengths 240-350, one layer)
        orc = full["orc"]
        dl_np, vl_np = dl.cpu().numpy(), vl.cpu().numpy()
        for r in range(R):
            st = _oracle_prefill_cached(full, wl5.wid, r, lens[r], Bb)
            if st.x0 != firsts[r]:
                assert full["batch_margins"][(wl5.wid, r)] < full["tie"], f"request {r}: prefill token"
                continue
            rows = slice(r * (Bb + 1), (r + 1) * (Bb + 1))
            check_round(cfg, orc, st, Bb, plants[r], got[r][0], got[r][1], dl_np[rows], vl_np[rows], full["tol"],
                        budget=budgets[r])
    for kv in kvs:
        kv.close()


def _oracle_prefill_cached(full, wid, i, P, Bb):
    """The oracle's state after prefilling request i's prefix (cached per prefix; a copy)."""
    cache = full.setdefault("batch_states", {})
    key = (wid, i)
    if key not in cache or cache[key].cache.K.shape[1] < P + 2 * Bb + 8:
        pre = prefix_embeddings(wid, i, P, full["cfg"].hidden)
        st, _, margin = prefill(full["orc"], pre, P + 2 * 64 + 8)
        cache[key] = st
        full.setdefault("batch_margins", {})[key] = margin
    return _copy_state(cache[key])


def _top2_of_logits(lg, mask_id):
    """Per row of float32 logits, the mask id excluded: the largest value, the lowest id holding it,
    and the largest value left once that id is removed (equal to the first when it occurs twice)."""
    z = np.array(lg, dtype=np.float32, copy=True)
    z[:, mask_id] = -np.inf
    rows = np.arange(len(z))
    i1 = np.argmax(z, axis=1)                 # first occurrence: the lowest id
    v1 = z[rows, i1]
    z[rows, i1] = -np.inf
    return i1, v1, z.max(axis=1)


def test_lm_head_records_equal_exact_top2_of_logits(full):
    """The LM head's per-group records (each of 8 lanes scans 8 columns, merged across the lanes and
    then across the vocabulary groups) give, row for row, exactly the top-1 value, its lowest id and
    the runner-up value of the logits the same launch writes: a teacher-forced forward of 33 tokens
    (the round's row count), compared with a plain sort of the returned logits."""
    from self_speculative_block_amd.engine import KV
    cfg, pool = full["cfg"], full["pool"]
    kv = KV(pool, full["P"] + 64)
    kv.prefill(full["pre_dev"])
    am, t1, t2, lg = kv.forward_tokens(full["cont"][:B + 1], full["P"], want_logits=True)
    kv.close()
    i1, v1, v2 = _top2_of_logits(lg.cpu().numpy(), cfg.mask_id)
    assert list(am) == [int(i) for i in i1]
    assert np.array_equal(np.asarray(t1, dtype=np.float32), v1)
    assert np.array_equal(np.asarray(t2, dtype=np.float32), v2)
    kv = full["kv"]
    kv.reset()
    assert kv.prefill(full["pre_dev"]) == full["y1"]


def test_tall_forward_logits_match_oracle(full):
    """A teacher-forced forward of 200 rows after the prefill runs as a tall forward: the large-tile
    GEMMs on fragment-major activations, the folded two-stream attention, the 128 x 256 gate|up
    blocks. Its logits, every row and every id, against the oracle's forward of the same rows on
    the same prefilled cache, at the logit bar."""
    from oracle.decode import causal_visibility
    from self_speculative_block_amd.engine import KV
    cfg, pool, orc, P = full["cfg"], full["pool"], full["orc"], full["P"]
    M = 200
    toks = [int(t) for t in np.random.default_rng(17).integers(0, cfg.vocab - 2, M)]
    kv = KV(pool, P + M + 8)
    kv.prefill(full["pre_dev"])
    _, _, _, lg = kv.forward_tokens(toks, P, want_logits=True)
    kv.close()
    st = _copy_state(full["st"])
    pos = P + np.arange(M)
    ref = orc.forward(st.cache, orc.embed_tokens(toks), pos, causal_visibility(pos, P + M))
    err = float(np.abs(lg.cpu().numpy() - ref).max())
    print(f"\n[{cfg.n_layers} layers] tall forward of {M} rows: logit max-abs error vs the oracle {err:.5f}",
          flush=True)
    assert err < LOGIT_TOL, err


def test_teacher_forced_tokens_match_oracle(full):
    """GravityOCR review, Appendix B.3: a decoded sequence is judged position by position; a
    position where the GPU's token differs from the oracle's greedy prediction for it (given the
    same history) must sit at an oracle top-2 margin below 1e-2.  Eight seeded prefixes: the
    microbenchmark's 1280 positions and seven 256-position prefixes; 64 tokens each, decoded by
    GPU self-speculative rounds (B = 32).  A sequence with no such position is exactly what the
    oracle's own greedy decode produces; the share of such sequences is the identity rate."""
    from self_speculative_block_amd.engine import KV
    cfg, model, pool, orc = full["cfg"], full["model"], full["pool"], full["orc"]
    N = 64
    prefixes = [full["pre"]] + [prefix_embeddings(3, 1000 + i, 256, cfg.hidden) for i in range(7)]
    identical, positions, flips = 0, 0, []
    kv = KV(pool, full["P"] + N + 2 * B + 8)
    for i, pre in enumerate(prefixes):
        kv.reset()
        toks, _ = kv.decode(model.prefix_tensor(pre), B, N)
        preds, margins = teacher_forced_argmax(orc, pre, toks)
        bad = [(t, toks[t], preds[t], margins[t]) for t in range(len(toks)) if toks[t] != preds[t]]
        for t, g, o, mg in bad:
            flips.append((i, t, mg))
            assert mg < NEAR_TIE, f"prefix {i} position {t}: GPU {g} vs oracle {o} at margin {mg:.4f}"
        identical += not bad
        positions += len(toks)
    kv.close()
    print(f"\n[{cfg.n_layers} layers] teacher-forced: {positions} positions over {len(prefixes)} prefixes, "
          f"{len(flips)} departures (margins {[round(m, 4) for _, _, m in flips]}), "
          f"identical sequences {identical}/{len(prefixes)}", flush=True)
    kv = full["kv"]
    kv.reset()
    assert kv.prefill(full["pre_dev"]) == full["y1"]


def test_direct_diffusion_block(full):
    """Direct block diffusion at full width, B = 32.  The random-init decoder's
    confidences all sit near 1/vocab, so the threshold is the median of the
    first step's confidences (about half the block qualifies at once).
    Every stack: decisions and tokens replayed exactly from the GPU's own
    confidences and logits; tau = 0 gives the GPU's one-shot draft.  One
    layer: each step's logits and confidences against the oracle for as long
    as both sides have committed the same tokens."""
    cfg, P, kv, orc = full["cfg"], full["P"], full["kv"], full["orc"]
    y1 = full["y1_orc"]
    if full["y1"] != y1:
        pytest.skip("the prefill token is an oracle near-tie")
    kv.rewind(P, y1)
    toks0, _, steps0, ex0 = kv.dd_block(B, 0.0, write_cache=False, want_steps=True)
    assert steps0 == 1
    _, _, dl, _ = kv.round(B, want_logits=True)
    dl = dl.cpu().numpy()
    assert toks0 == [argmax_excluding(dl[j], cfg.mask_id)[0] for j in range(B)]
    tau = float(np.median(ex0["conf"][0]))
    kv.rewind(P, y1)
    toks, n, steps, ex = kv.dd_block(B, tau, want_steps=True, want_logits=True)
    assert 1 <= steps <= B and n == B
    check_block_against_own_outputs(ex, toks, tau, B, cfg.mask_id, conf_rtol=1e-4)
    assert kv.state()[:2] == (P + B, toks[-1])
    if cfg.n_layers == 1:
        st = full["st"]
        st.n, st.x0 = P, y1
        r = dd_fill(orc, st, B, tau, keep_logits=True)
        lg = ex["logits"].cpu().numpy()
        for k in range(min(steps, r.steps)):
            err = np.abs(lg[k] - r.step_logits[k]).max()
            assert err < full["tol"], (k, err)
            rel = np.abs(ex["conf"][k] - np.array(r.step_conf[k])) / np.array(r.step_conf[k])
            assert rel.max() < 0.1, (k, rel.max())
            same = all((ex["step_of"][j] == k) == (r.step_of[j] == k) for j in range(B)) and \
                all(toks[j] == r.tokens[j] for j in range(B) if r.step_of[j] == k)
            if not same:
                break
    kv.rewind(P, y1)


def test_direct_diffusion_block_one_is_ar(full):
    kv, pre_dev = full["kv"], full["pre_dev"]
    kv.reset()
    ar, _ = kv.decode_ar(pre_dev, 24)
    kv.reset()
    dd, st = kv.decode_dd(pre_dev, 1, 0.5, 24)
    assert dd == ar and st.forwards == len(dd) - 1
    kv.reset()
    assert kv.prefill(pre_dev) == full["y1"]


@pytest.mark.parametrize("T", [1.0, 0.05])
def test_stochastic_round_full_width(full, T):
    """Stochastic rounds at full width, B = 32: every draw and acceptance decision
    replayed in float64 from the GPU's own logits; with one layer, logits against
    the oracle given the same uniforms."""
    from oracle.stochastic import spec_round_sample
    cfg, P, kv, orc = full["cfg"], full["P"], full["kv"], full["orc"]
    y1 = full["y1_orc"]
    if full["y1"] != y1:
        pytest.skip("the prefill token is an oracle near-tie")
    for k in range(3):
        u = np.random.default_rng([31, k, int(T * 100)]).random(2 * B + 2).astype(np.float32)
        kv.rewind(P, y1)
        committed, A, dl, vl = kv.round_sample(B, torch.tensor(u, device="cuda"), temperature=T,
                                               want_logits=True)
        dl, vl = dl.cpu().numpy(), vl.cpu().numpy()
        assert 0 <= A <= B and len(committed) == A + 2
        replay_round(dl, vl, u, B, T, cfg.mask_id, cfg.eos_id, committed, A)
        assert kv.state()[:2] == (P + A + 2, committed[-1])
        if cfg.n_layers == 1:
            st = full["st"]
            st.n, st.x0 = P, y1
            r = spec_round_sample(orc, st, B, u.astype(np.float64), temperature=T, keep_logits=True)
            assert np.abs(dl - r.draft_logits).max() < full["tol"]
            # verify row j sees a0, d_1..d_j: comparable while both sides drew the same tokens
            same = [committed[0]] + committed[1: A + 1] == [r.a0] + r.d[:A]
            rows = A + 1 if same else (1 if committed[0] == r.a0 else 0)
            if rows:
                assert np.abs(vl[:rows] - r.verify_logits[:rows]).max() < full["tol"]
    kv.rewind(P, y1)


def test_multistep_draft_full_width(full):
    """Draft schedules at full width: one step equals the one-shot round exactly
    (tokens and verify logits), and three steps decode AR-identically."""
    cfg, P, kv, pre_dev = full["cfg"], full["P"], full["kv"], full["pre_dev"]
    y1 = full["y1"]
    kv.rewind(P, y1)
    c1, A1, k1, v1 = kv.round_multistep(B, 1, 0.5, want_logits=True)
    kv.rewind(P, y1)
    c2, A2, _, v2 = kv.round(B, want_logits=True)
    assert (c1, A1, k1) == (c2, A2, 1) and torch.equal(v1, v2)
    kv.reset()
    ar, _ = kv.decode_ar(pre_dev, 48)
    kv.reset()
    out, st = kv.decode_multistep(pre_dev, B, 3, 0.5, 48)
    assert out == ar and st.forwards <= 4 * st.rounds
    kv.reset()
    assert kv.prefill(pre_dev) == y1


def test_serve_continuous_batching_full_width(full):
    """Four queued requests served two at a time, AR and self-speculative (B = 32,
    planted drafts): every output equals the request's own AR decode."""
    from self_speculative_block_amd.engine import KV, serve
    from self_speculative_block_amd._lib import SSB_SERVE_AR, SSB_SERVE_SPEC
    cfg, model, pool = full["cfg"], full["model"], full["pool"]
    wl5 = workload(5)
    reqs = [{"prefix_dev": model.prefix_tensor(prefix_embeddings(wl5.wid, i, 1088, cfg.hidden)), "max_len": L}
            for i, L in enumerate([40, 12, 64, 25])]
    kv = KV(pool, 1088 + 80)
    ref = []
    for q in reqs:
        kv.reset()
        ref.append(kv.decode_ar(q["prefix_dev"], q["max_len"])[0])
    kv.close()
    out, _, st = serve(model, pool, reqs, 2, SSB_SERVE_AR)
    assert out == ref and st["prefills"] == 4
    for i, q in enumerate(reqs):
        q["cont_dev"] = torch.tensor(ref[i], dtype=torch.int32, device="cuda")
        q["astar"] = [(7 * i + 5 * k) % (B + 1) for k in range(64)]
    out, _, st = serve(model, pool, reqs, 2, SSB_SERVE_SPEC, B=B)
    assert out == ref

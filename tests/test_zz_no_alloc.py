"""ssb_round_noalloc (the round for callers that cannot allocate device memory) against ssb_round,
through the C ABI, on a two-layer model of the benchmark's width (hidden 1024, 16 query heads over
4 KV heads, SwiGLU 4096, vocab 60000; bf16 weights).

Both calls start from the same kv state with the same planted drafts; the committed tokens, the
accept length and the kv state after the call must be identical (bar: integers, bit-exact).  Three
calls in a row with shrinking windows (B = 64, 32, 8: the three-launch and fused layer tails) reuse
the same scratch array, and a window too large for it is rejected with SSB_EINVAL, state unchanged.
"""

import dataclasses

import pytest
import torch

from ssb_inputs import generate_weights, prefix_embeddings, workload
from oracle import build_plant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def two_layer():
    from self_speculative_block_amd.engine import KV, Model, Pool
    wl = workload(2)
    cfg = dataclasses.replace(wl.model, n_layers=2)
    model = Model(cfg, generate_weights(cfg), block_B=64, max_rows=2048, max_positions=4096, max_batch=1,
                  sampling=False)
    pool = Pool(model, n_pages=4096 // 16 + 64)
    yield cfg, model, pool
    pool.close()
    model.close()


def test_round_noalloc_equals_round(two_layer):
    from self_speculative_block_amd.engine import KV
    cfg, model, pool = two_layer
    P = 600
    kv = KV(pool, P + 2 * 64 + 8)
    y1 = kv.prefill(model.prefix_tensor(prefix_embeddings(2, 5, P, cfg.hidden)))
    cont = [y1] + [kv.ar_step()[0] for _ in range(66)]
    for B, astar in ((64, 40), (32, 20), (8, 8)):          # each call's window smaller than the last
        plant = torch.tensor(build_plant(cont, 1, astar, B, cfg.vocab, cfg.mask_id), dtype=torch.int32,
                             device="cuda")
        kv.rewind(P, y1)
        ref_c, ref_A, _, _ = kv.round(B, planted_dev=plant)
        ref_state = kv.state()
        kv.rewind(P, y1)
        got_c, got_A = kv.round_noalloc(B, planted_dev=plant)
        assert (got_c, got_A) == (ref_c, ref_A), f"B={B}"
        assert kv.state() == ref_state, f"B={B}"
        assert got_A == min(astar, B)
    # an unplanted round, and a budget cut
    kv.rewind(P, y1)
    ref = kv.round(16, max_commit=5)[:2]
    st = kv.state()
    kv.rewind(P, y1)
    assert kv.round_noalloc(16, max_commit=5) == ref
    assert kv.state() == st
    kv.close()


def test_round_noalloc_rejects_a_window_beyond_its_scratch(two_layer):
    from self_speculative_block_amd.engine import KV
    from self_speculative_block_amd._lib import SSB_EINVAL, SsbError
    cfg, model, pool = two_layer
    P = 3600                      # B = 64 over 3,666 positions needs more than 16 MiB of scratch
    kv = KV(pool, P + 2 * 64 + 8)
    y1 = kv.prefill(model.prefix_tensor(prefix_embeddings(2, 6, P, cfg.hidden)))
    before = kv.state()
    with pytest.raises(SsbError) as err:
        kv.round_noalloc(64)
    assert err.value.code == SSB_EINVAL and "scratch" in str(err.value)
    assert kv.state() == before
    c, A = kv.round_noalloc(8)    # a small window still fits
    kv.rewind(P, y1)
    assert kv.round(8)[:2] == (c, A)
    kv.close()

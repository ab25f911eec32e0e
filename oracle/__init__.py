"""CPU oracle for the self-speculative decoding round — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU engine
(``self_speculative_block_amd``) never imports it and shares no code with it;
the two meet only in the seeded data of ``ssb_inputs``.

Everything here is plain numpy in float64 by default (float32 on request),
written for readability rather than speed.  Each function cites the passage
of the pages it follows.  Pages: "GravityOCR review" (the chapter-by-chapter
review of arXiv:2609.26638v1), "velog review" (the paper summary with full
tables) and "Trillion Labs blog" (the earlier blog post).

Pin status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py``; the training-time rules (complementary masks and
the three-stream attention predicate) are rule checks only and are pinned
by brute-force enumeration.  Nothing in this package is "parity unpinned".
"""

from .model import Decoder, KVCache, rms_norm, rope, silu, attend, argmax_excluding
from .decode import (
    DecodeState, RoundResult, prefill, ar_step, ar_decode, spec_round, spec_decode,
    draft_visibility, verify_visibility, causal_visibility, accept_length, commit_tokens,
    build_plant, tpf, teacher_forced_argmax,
)
from .training_rules import complementary_masks, training_visibility
from .direct import (confidence, select_positions, BlockResult, dd_fill, dd_cache_write, dd_release,
                     DDStats, dd_tpf, dd_decode, MultiStepRoundResult, spec_round_multistep,
                     spec_decode_multistep)

__all__ = [
    "Decoder", "KVCache", "rms_norm", "rope", "silu", "attend", "argmax_excluding",
    "DecodeState", "RoundResult", "prefill", "ar_step", "ar_decode", "spec_round",
    "spec_decode", "draft_visibility", "verify_visibility", "causal_visibility",
    "accept_length", "commit_tokens", "build_plant", "tpf", "teacher_forced_argmax",
    "complementary_masks", "training_visibility",
    "confidence", "select_positions", "BlockResult", "dd_fill", "dd_cache_write", "dd_release",
    "DDStats", "dd_tpf", "dd_decode", "MultiStepRoundResult", "spec_round_multistep",
    "spec_decode_multistep",
]

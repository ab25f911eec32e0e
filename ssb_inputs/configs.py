"""Model sizes and workload shapes.

The decoder is a pre-norm Llama-style stack (RMSNorm, RoPE, GQA attention,
SwiGLU MLP, untied embedding and LM head, no biases).  The pages describe a
GLM-OCR-based region recognizer whose language decoder, LM head and one
added [M] embedding row are shared by the AR and block-diffusion modes
(GravityOCR review, section 3.1 "AR-to-Diffusion Conversion"); they do not
give its architecture, so the sizes below are the synthetic stand-ins the
workloads are quoted on.

Workload shapes follow the pages' measurement workloads: block size 32
(review, "technical details"), text crops of mean 73 output tokens, table
crops of mean 872 (Table 4), about 18 concurrent regions per page
(Appendix C), and the decode round of section 3.2 / Appendix B.2.
"""

from dataclasses import dataclass, field, asdict
from typing import Tuple


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    mask_id: int
    eos_id: int
    dtype: str            # "f32" or "bf16": storage/arithmetic type of the GPU engine
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    weight_std: float = 0.02
    weight_seed_id: int = 0   # first entry of the weight generator's seed

    def as_dict(self):
        return asdict(self)

    @property
    def q_dim(self):
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim

    def layer_params(self):
        h, f = self.hidden, self.ffn
        return h * (self.q_dim + 2 * self.kv_dim) + self.q_dim * h + 3 * h * f + 2 * h

    def streamed_params(self):
        """Parameters one forward pass reads: all layers, final norm, LM head."""
        return self.n_layers * self.layer_params() + self.hidden + self.vocab * self.hidden

    def kv_bytes_per_position(self, elem_bytes):
        return self.n_layers * 2 * self.kv_dim * elem_bytes


TINY = ModelConfig(
    name="tiny_fp32", n_layers=2, hidden=128, n_heads=4, n_kv_heads=4, head_dim=32,
    ffn=512, vocab=512, mask_id=511, eos_id=510, dtype="f32", weight_seed_id=1,
)

DECODER_1B = ModelConfig(
    name="decoder_24x1024_bf16", n_layers=24, hidden=1024, n_heads=16, n_kv_heads=4,
    head_dim=64, ffn=4096, vocab=60000, mask_id=59999, eos_id=59998, dtype="bf16",
    weight_seed_id=2,
)

MODELS = {m.name: m for m in (TINY, DECODER_1B)}


@dataclass(frozen=True)
class Workload:
    wid: int                  # first entry of every seed of this workload
    name: str
    model: ModelConfig
    block: int                # B
    prefix_len: int           # P
    n_regions: int = 1
    max_len: int = 0          # output cap (0: per-region target length)
    length_mean: Tuple[float, ...] = ()
    length_cap: int = 0
    length_mix: Tuple[Tuple[str, int, float, int], ...] = ()   # (kind, count, mean, cap)
    plant_p: float = 0.0      # geometric success probability of the first planted mismatch
    full_accept_p: float = 0.0
    reps: int = 0
    warmup: int = 0
    blocks_extra: Tuple[int, ...] = field(default_factory=tuple)
    page_tokens: int = 16


WORKLOADS = {
    1: Workload(wid=1, name="tiny_fp32_equivalence", model=TINY, block=8, prefix_len=64,
                n_regions=200, max_len=64),
    2: Workload(wid=2, name="round_microbench_b32_n1280", model=DECODER_1B, block=32,
                prefix_len=1280, n_regions=1, plant_p=1.0 / 20.0, reps=1000, warmup=50),
    3: Workload(wid=3, name="text_regions", model=DECODER_1B, block=32, prefix_len=1088,
                n_regions=256, length_mix=(("text", 256, 73.0, 512),), plant_p=1.0 / 20.0),
    4: Workload(wid=4, name="table_regions", model=DECODER_1B, block=32, prefix_len=1088,
                n_regions=64, length_mix=(("table", 64, 872.0, 4096),), plant_p=1.0 / 20.0,
                full_accept_p=0.05),
    5: Workload(wid=5, name="batched_page", model=DECODER_1B, block=32, prefix_len=1088,
                n_regions=16,
                length_mix=(("text", 12, 73.0, 512), ("table", 3, 872.0, 4096),
                            ("formula", 1, 200.0, 1024)),
                plant_p=1.0 / 20.0, blocks_extra=(64,)),
}


def workload(wid):
    return WORKLOADS[wid]

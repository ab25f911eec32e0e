"""Seeded synthetic inputs shared by the CPU oracle and the HIP engine.

This package holds data only: model sizes, seeded weight draws, prefix
embeddings standing in for the vision+prompt prefix, target lengths and the
planted-draft schedule.  It contains none of the decoding method's
arithmetic, so the oracle (``oracle/``) and the GPU engine
(``self_speculative_block_amd``) can both read it without sharing code.

Every random draw uses ``numpy.random.default_rng([workload_id, purpose,
index])`` with purpose 0 = weights, 1 = prefix, 2 = length, 3 = plant,
4 = forced full accept.
"""

from .configs import ModelConfig, Workload, MODELS, WORKLOADS, workload
from .weights import generate_weights, weight_names, bf16_round
from .prefix import prefix_embeddings
from .schedule import target_lengths, plant_accept_lengths, region_kinds

__all__ = [
    "ModelConfig", "Workload", "MODELS", "WORKLOADS", "workload",
    "generate_weights", "weight_names", "bf16_round",
    "prefix_embeddings", "target_lengths", "plant_accept_lengths", "region_kinds",
]

"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

Holds model shapes, random BF16 and 4-bit weights and random token ids only -- none of the
model's arithmetic -- so that the oracle and the HIP path share nothing but their
inputs.
"""
from .configs import ModelConfig, PRESETS, get_config
from .weights import (INIT_STD, tensor_manifest, bf16_round, bf16_bits_to_f32,
                      make_weights)
from .prompts import make_prompt, make_drafts
from .q4 import Q4_GROUP, q4_nbytes, q4_draw, make_q4_weights

__all__ = ["ModelConfig", "PRESETS", "get_config", "INIT_STD", "tensor_manifest",
           "bf16_round", "bf16_bits_to_f32", "make_weights", "make_prompt", "make_drafts",
           "Q4_GROUP", "q4_nbytes", "q4_draw", "make_q4_weights"]

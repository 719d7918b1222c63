"""Model shapes for the synthetic hybrid Gated-DeltaNet + attention workloads.

The pages describe a 24-layer hybrid of 18 DeltaNet layers and 6 full-attention
layers (luce-megakernel announcement, page 1, the paragraph on why the model is
not a vanilla transformer).  They give no dimensions, so every size below is a
stated workload shape, not a fact from the pages:

* ``tiny``         4 layers (3 DeltaNet + 1 attention), hidden 256 -- the small case.
* ``hybrid_0p8b``  24 layers in a repeating 3 DeltaNet : 1 attention pattern,
                   hidden 1024, 16 DeltaNet heads of 128, 8 Q / 2 KV heads of 128,
                   SwiGLU FFN 3584, vocabulary 151936 tied -- the decode/prefill
                   workload.
* ``hybrid_27b``   the 27B-scale shape of the pages' second system (64 layers,
                   hidden 5120); only its shape lives here.

Layer ``l`` is attention when ``l % period == attn_slot`` and DeltaNet otherwise.
This module holds sizes only: no arithmetic of the model.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict, replace


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    ffn: int
    vocab: int
    dn_heads: int
    dn_dk: int
    dn_dv: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    period: int = 4
    attn_slot: int = 3
    rms_eps: float = 1e-6
    l2_eps: float = 1e-6
    rope_theta: float = 10000.0
    max_ctx: int = 1024
    tied: bool = True

    def is_attention(self, layer: int) -> bool:
        return layer % self.period == self.attn_slot

    @property
    def n_attention_layers(self) -> int:
        return sum(1 for l in range(self.n_layers) if self.is_attention(l))

    @property
    def n_deltanet_layers(self) -> int:
        return self.n_layers - self.n_attention_layers

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)

    def as_dict(self) -> dict:
        return asdict(self)


PRESETS = {
    "tiny": ModelConfig(
        name="tiny", n_layers=4, hidden=256, ffn=768, vocab=4096,
        dn_heads=4, dn_dk=64, dn_dv=64, n_q_heads=4, n_kv_heads=2, head_dim=64,
        max_ctx=256),
    "hybrid_0p8b": ModelConfig(
        name="hybrid_0p8b", n_layers=24, hidden=1024, ffn=3584, vocab=151936,
        dn_heads=16, dn_dk=128, dn_dv=128, n_q_heads=8, n_kv_heads=2, head_dim=128,
        max_ctx=2048),
    "hybrid_27b": ModelConfig(
        name="hybrid_27b", n_layers=64, hidden=5120, ffn=17408, vocab=151936,
        dn_heads=32, dn_dk=128, dn_dv=128, n_q_heads=24, n_kv_heads=4, head_dim=128,
        max_ctx=32768),
}


def get_config(name: str, **overrides) -> ModelConfig:
    cfg = PRESETS[name]
    return cfg.with_(**overrides) if overrides else cfg

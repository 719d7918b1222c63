"""Seeded random-init BF16 weights for the synthetic hybrid models.

Both the GPU path and the CPU oracle consume the exact same BF16 bit patterns
produced here.  The pages report BF16 weights with FP32 accumulation (luce-
megakernel announcement, page 1, kernel-design bullets); the values themselves
are random because no trained checkpoint is used.

Recipe (fixed, so any reader can regenerate the same bits):

* one generator ``numpy.random.default_rng([seed, 0])`` walks the tensor
  manifest in order;
* every matrix is ``standard_normal(shape, float32) * 0.02``, rounded to BF16
  with round-to-nearest-even;
* every norm gain is 1.0, or ``1 + gain_noise * standard_normal`` when
  ``gain_noise > 0`` (drawn from the same generator at the gain's slot in the
  manifest), then rounded the same way.

Tensor names and shapes (row-major ``[out][in]``)::

    embed                [vocab, hidden]        (also the tied LM head)
    l{i}.norm1           [hidden]
    DeltaNet layer:
      l{i}.dn.wqkv       [3*H*d, hidden]        rows: q heads, then k heads, then v heads
      l{i}.dn.wa         [H, hidden]            decay-gate logits
      l{i}.dn.wb         [H, hidden]            write-strength logits
      l{i}.dn.wo         [hidden, H*dv]
    attention layer:
      l{i}.attn.wq       [nq*hd, hidden]
      l{i}.attn.wk       [nkv*hd, hidden]
      l{i}.attn.wv       [nkv*hd, hidden]
      l{i}.attn.wo       [hidden, nq*hd]
    l{i}.norm2           [hidden]
    l{i}.ffn.wg          [ffn, hidden]
    l{i}.ffn.wu          [ffn, hidden]
    l{i}.ffn.wd          [hidden, ffn]
    final_norm           [hidden]

This module only draws numbers and rounds them to the storage format; it holds
none of the model's arithmetic.
"""
from __future__ import annotations

import numpy as np

from .configs import ModelConfig

INIT_STD = 0.02


def tensor_manifest(cfg: ModelConfig) -> list[tuple[str, tuple[int, ...], str]]:
    """Ordered list of (name, shape, kind) with kind in {"matrix", "gain"}."""
    H, dk, dv = cfg.dn_heads, cfg.dn_dk, cfg.dn_dv
    D = cfg.hidden
    out = [("embed", (cfg.vocab, D), "matrix")]
    for l in range(cfg.n_layers):
        out.append((f"l{l}.norm1", (D,), "gain"))
        if cfg.is_attention(l):
            out.append((f"l{l}.attn.wq", (cfg.n_q_heads * cfg.head_dim, D), "matrix"))
            out.append((f"l{l}.attn.wk", (cfg.n_kv_heads * cfg.head_dim, D), "matrix"))
            out.append((f"l{l}.attn.wv", (cfg.n_kv_heads * cfg.head_dim, D), "matrix"))
            out.append((f"l{l}.attn.wo", (D, cfg.n_q_heads * cfg.head_dim), "matrix"))
        else:
            out.append((f"l{l}.dn.wqkv", (H * dk * 2 + H * dv, D), "matrix"))
            out.append((f"l{l}.dn.wa", (H, D), "matrix"))
            out.append((f"l{l}.dn.wb", (H, D), "matrix"))
            out.append((f"l{l}.dn.wo", (D, H * dv), "matrix"))
        out.append((f"l{l}.norm2", (D,), "gain"))
        out.append((f"l{l}.ffn.wg", (cfg.ffn, D), "matrix"))
        out.append((f"l{l}.ffn.wu", (cfg.ffn, D), "matrix"))
        out.append((f"l{l}.ffn.wd", (D, cfg.ffn), "matrix"))
    out.append(("final_norm", (D,), "gain"))
    return out


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 BF16 bit patterns, round to nearest, ties to even.

    Inputs must be finite (the generator never produces inf/NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    r = (bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 BF16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_weights(cfg: ModelConfig, seed: int, gain_noise: float = 0.0) -> dict[str, np.ndarray]:
    """Return {name: uint16 BF16 bits} in manifest order (dicts keep insertion order)."""
    rng = np.random.default_rng([seed, 0])
    w: dict[str, np.ndarray] = {}
    for name, shape, kind in tensor_manifest(cfg):
        if kind == "matrix":
            a = rng.standard_normal(shape, dtype=np.float32)
            a *= np.float32(INIT_STD)
        else:
            if gain_noise > 0.0:
                a = np.float32(1.0) + np.float32(gain_noise) * rng.standard_normal(shape, dtype=np.float32)
            else:
                a = np.ones(shape, dtype=np.float32)
        w[name] = bf16_round(a)
        del a
    return w

"""Seeded random 4-bit weights (the Q4G32 storage format) for the 27B-scale hybrid.

The pages' second system runs a 27B-scale hybrid from 4-bit block-quantised weights (the
megakernel follow-up posts, page 3: the quantisation-support and speed paragraphs).  No trained
checkpoint is available, so the codes and block parameters are drawn at random in the storage
format itself; both the GPU path and the CPU oracle read the same bytes.

Q4G32 format of a row-major matrix W[R][K] (K a multiple of 32), R*K*5/8 bytes:

* codes, R*K/2 bytes: row r's codes are bytes [r*K/2, (r+1)*K/2).  Columns 8i .. 8i+7 of a row sit in
  the four bytes at offset 4i, read as one little-endian 32-bit word v: column 8i + 2j (j = 0..3)
  is the nibble at bits 4j .. 4j+3 of v, column 8i + 2j + 1 the nibble at bits 16 + 4j .. 19 + 4j;
* block parameters, after all codes: group g (columns 32g .. 32g+31) of row r has two IEEE
  binary16 values (d, m), d first, at byte R*K/2 + 4*(r*K/32 + g);
* the weight is d*q + m, q being the 4-bit code (0..15).

Recipe (fixed): one generator ``numpy.random.default_rng([seed, 3])`` walks the tensor manifest in
order.  For a matrix: the codes are ``R*K/2`` uniformly random bytes (``Generator.bytes``), then
``d = fp16(0.02 * 0.27 * (1 + 0.1 n1))`` and ``m = fp16(-7.5 d + 0.02 * 0.05 n2)`` per group with n1,
n2 standard normal (float32), drawn as one array of shape [R*K/32, 2].  This is roughly the spread
of groups of 32 draws from N(0, 0.02^2) (range about 4.1 sigma) with uniform codes in place of
bell-shaped ones.  Norm gains are BF16 bits exactly as in ``weights.make_weights`` (1.0, or
1 + gain_noise * n drawn from the same generator at the gain's slot).

This module only draws numbers and writes them in the storage format; it holds none of the
model's arithmetic.
"""
from __future__ import annotations

import numpy as np

from .configs import ModelConfig
from .weights import tensor_manifest, bf16_round

Q4_GROUP = 32
Q4_D_SCALE = 0.02 * 0.27


def q4_nbytes(R: int, K: int) -> int:
    """Bytes of a Q4G32 matrix of logical shape [R][K]."""
    assert K % Q4_GROUP == 0, "Q4G32 needs K divisible by 32"
    return R * K // 2 + R * (K // Q4_GROUP) * 4


def q4_draw(rng: np.random.Generator, R: int, K: int) -> np.ndarray:
    """One random Q4G32 matrix [R][K] -> uint8 buffer of q4_nbytes(R, K)."""
    ncode = R * K // 2
    ng = R * (K // Q4_GROUP)
    out = np.empty(ncode + ng * 4, dtype=np.uint8)
    out[:ncode] = np.frombuffer(rng.bytes(ncode), dtype=np.uint8)
    n = rng.standard_normal((ng, 2), dtype=np.float32)
    d = (np.float32(Q4_D_SCALE) * (np.float32(1.0) + np.float32(0.1) * n[:, 0])).astype(np.float16)
    m = (np.float32(-7.5) * d.astype(np.float32) + np.float32(0.02 * 0.05) * n[:, 1]).astype(np.float16)
    dm = np.empty((ng, 2), dtype=np.float16)
    dm[:, 0] = d
    dm[:, 1] = m
    out[ncode:] = dm.reshape(-1).view(np.uint8)
    return out


def make_q4_weights(cfg: ModelConfig, seed: int, gain_noise: float = 0.0) -> dict[str, np.ndarray]:
    """{name: uint8 Q4G32 buffer for matrices, uint16 BF16 bits for gains}, manifest order."""
    rng = np.random.default_rng([seed, 3])
    w: dict[str, np.ndarray] = {}
    for name, shape, kind in tensor_manifest(cfg):
        if kind == "matrix":
            w[name] = q4_draw(rng, shape[0], shape[1])
        else:
            if gain_noise > 0.0:
                a = np.float32(1.0) + np.float32(gain_noise) * rng.standard_normal(shape, dtype=np.float32)
            else:
                a = np.ones(shape, dtype=np.float32)
            w[name] = bf16_round(a)
    return w

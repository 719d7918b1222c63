"""Decoding of 4-bit block-quantised weights (Q4G32), written from the format definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages' 27B-scale system runs from 4-bit weights in blocks with a per-block scale (megakernel
follow-up posts, page 3, quantisation-support paragraph); the block layout used here is groups of
32 consecutive columns of a row, each with an FP16 scale d and an FP16 offset m, weight = d*q + m
for the 4-bit code q.  Byte layout of a matrix W[R][K]:

* codes first, row-major, K/2 bytes per row.  In row r, columns 8i .. 8i+7 occupy the 32-bit
  little-endian word at byte r*K/2 + 4i; in that word, column 8i + 2j (j = 0, 1, 2, 3) is the
  nibble starting at bit 4j and column 8i + 2j + 1 the nibble starting at bit 16 + 4j;
* then (d, m) pairs of IEEE binary16 values, row-major over (row, group), 4 bytes per group.

Every decoded value d*q + m is exact in float64 (an 11-bit significand times a 4-bit integer,
plus an 11-bit significand), so the oracle's weights are the stored weights exactly.
"""
from __future__ import annotations

import numpy as np

GROUP = 32


def q4g32_split(buf: np.ndarray, R: int, K: int):
    """Views of a Q4G32 buffer: (code words [R][K/8] uint32, params [R][K/32][2] float16)."""
    assert K % GROUP == 0
    buf = np.asarray(buf, dtype=np.uint8)
    ncode = R * K // 2
    assert buf.size == ncode + R * (K // GROUP) * 4, "Q4G32 buffer size does not match its shape"
    words = buf[:ncode].view("<u4").reshape(R, K // 8)
    params = buf[ncode:].view("<f2").reshape(R, K // GROUP, 2)
    return words, params


def q4g32_codes(words: np.ndarray) -> np.ndarray:
    """Code words [..., n] -> codes [..., 8n] in column order (the nibble placement above)."""
    words = np.asarray(words, dtype=np.uint32)
    q = np.empty(words.shape + (8,), dtype=np.uint8)
    for j in range(4):
        q[..., 2 * j] = (words >> np.uint32(4 * j)) & np.uint32(0xF)
        q[..., 2 * j + 1] = (words >> np.uint32(16 + 4 * j)) & np.uint32(0xF)
    return q.reshape(words.shape[:-1] + (words.shape[-1] * 8,))


def q4g32_dequant_rows(buf: np.ndarray, R: int, K: int, rows, dtype=np.float64) -> np.ndarray:
    """Rows `rows` (an index array or slice) of the Q4G32 matrix W[R][K], decoded to `dtype`."""
    words, params = q4g32_split(buf, R, K)
    q = q4g32_codes(words[rows]).astype(dtype)
    p = params[rows].astype(dtype)
    d = p[..., 0]
    m = p[..., 1]
    w = q.reshape(q.shape[:-1] + (K // GROUP, GROUP)) * d[..., None] + m[..., None]
    return w.reshape(q.shape)


def q4g32_dequant(buf: np.ndarray, R: int, K: int, dtype=np.float64) -> np.ndarray:
    """The whole Q4G32 matrix W[R][K] decoded to `dtype`."""
    return q4g32_dequant_rows(buf, R, K, slice(None), dtype)

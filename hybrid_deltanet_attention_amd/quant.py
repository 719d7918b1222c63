"""Host quantizer to the 4-bit Q4G32 weight format that MK_Q4G32 models load.

The pages' 27B-scale system decodes from 4-bit block-quantised weights (megakernel follow-up posts,
page 3, quantisation-support paragraph).  Q4G32 keeps, for every group of 32 consecutive columns of
a row, an FP16 scale d and an FP16 offset m; a weight is d*q + m with a 4-bit code q.

Layout of a matrix W[R][K] (K a multiple of 32), R*K*5/8 bytes, as `mk_load_weights` expects it:
codes first (row-major, K/2 bytes per row; columns 8i .. 8i+7 of a row in the little-endian 32-bit
word at byte 4i of the row, column 8i+2j in the nibble at bit 4j and column 8i+2j+1 in the nibble at
bit 16+4j), then the (d, m) binary16 pairs, row-major over (row, group).  The nibble placement puts
the codes of two neighbouring columns 16 bits apart, so one AND/OR turns a word into two BF16
values 128 + q for the kernel's packed dot products.

Quantisation of a group: m = fp16(min), d = fp16((max - min) / 15), q = clip(rint((w - m) / d), 0, 15)
(q = 0 when d = 0).  The reconstruction error is at most d/2 plus the FP16 rounding of d and m.
"""
from __future__ import annotations

import numpy as np

GROUP = 32


def q4g32_nbytes(R: int, K: int) -> int:
    if K % GROUP:
        raise ValueError(f"Q4G32 needs the column count to be a multiple of {GROUP}, got {K}")
    return R * K // 2 + R * (K // GROUP) * 4


def pack_q4g32(q: np.ndarray, d: np.ndarray, m: np.ndarray) -> np.ndarray:
    """Codes q [R][K] (0..15) and per-group d, m [R][K/32] (float16) -> the Q4G32 byte buffer."""
    q = np.asarray(q, dtype=np.uint32)
    R, K = q.shape
    nb = q4g32_nbytes(R, K)
    g = q.reshape(R, K // 8, 8)
    words = np.zeros((R, K // 8), dtype=np.uint32)
    for j in range(4):
        words |= g[..., 2 * j] << np.uint32(4 * j)
        words |= g[..., 2 * j + 1] << np.uint32(16 + 4 * j)
    out = np.empty(nb, dtype=np.uint8)
    ncode = R * K // 2
    out[:ncode] = words.astype("<u4").reshape(-1).view(np.uint8)
    dm = np.empty((R, K // GROUP, 2), dtype="<f2")
    dm[..., 0] = np.asarray(d, dtype=np.float16)
    dm[..., 1] = np.asarray(m, dtype=np.float16)
    out[ncode:] = dm.reshape(-1).view(np.uint8)
    return out


def quantize_q4g32(w: np.ndarray) -> np.ndarray:
    """Float matrix [R][K] -> Q4G32 buffer (min/max per group of 32 columns)."""
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("quantize_q4g32 takes a 2-D matrix")
    R, K = w.shape
    q4g32_nbytes(R, K)
    g = w.reshape(R, K // GROUP, GROUP)
    lo = g.min(axis=-1)
    hi = g.max(axis=-1)
    m16 = lo.astype(np.float16)
    d16 = ((hi - lo) / np.float32(15.0)).astype(np.float16)
    d = d16.astype(np.float32)[..., None]
    m = m16.astype(np.float32)[..., None]
    safe = np.where(d > 0, d, np.float32(1.0))
    q = np.where(d > 0, np.clip(np.rint((g - m) / safe), 0, 15), 0).astype(np.uint32)
    return pack_q4g32(q.reshape(R, K), d16, m16)

"""Causal grouped-query softmax attention, two independent ways.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages call the attention layers standard multi-head attention and say the
kernel fuses the QKV projection, RoPE, the causal softmax and the output
projection (luce-megakernel announcement, page 1, layer-pattern paragraph and
kernel-design bullets).  The model run here has 8 query heads sharing 2 key/value
heads; query head i reads key/value head i // (n_q / n_kv), so MHA is the case
n_kv = n_q.  Scores are scaled by 1/sqrt(head_dim), position t attends to
positions 0..t (itself included), and softmax subtracts the row maximum.
"""
from __future__ import annotations

import numpy as np

from .primitives import softmax


def attend_one(q, Kc, Vc):
    """One query position over a cache, head by head.

    q [nq, hd]; Kc, Vc [nkv, L, hd] holding the L visible positions -> o [nq, hd]."""
    nq, hd = q.shape
    nkv = Kc.shape[0]
    group = nq // nkv
    o = np.empty_like(q)
    for i in range(nq):
        g = i // group
        s = Kc[g] @ q[i] / np.sqrt(hd)
        p = softmax(s)
        o[i] = p @ Vc[g]
    return o


def causal_attention(Q, K, V):
    """Whole sequence with the full masked score matrix.

    Q [T, nq, hd]; K, V [T, nkv, hd] -> O [T, nq, hd]."""
    T, nq, hd = Q.shape
    nkv = K.shape[1]
    group = nq // nkv
    mask = np.tril(np.ones((T, T), dtype=bool))
    O = np.empty_like(Q)
    for i in range(nq):
        g = i // group
        s = (Q[:, i, :] @ K[:, g, :].T) / np.sqrt(hd)
        s = np.where(mask, s, -np.inf)
        O[:, i, :] = softmax(s, axis=-1) @ V[:, g, :]
    return O


KV_DTYPES = ("f32", "f16", "q8")
Q8_BLOCK = 32


def kv_round(x, kv: str):
    """Values a key or value row takes once stored in the KV cache.

    The pages keep the 27B model's cache in fp16 up to about 80K positions and in an 8-bit format
    above (Reddit follow-up on the 27B model, "Limits" paragraph).  "f32": unchanged.  "f16": the
    IEEE binary16 value nearest the float32 value (ties to even).  "q8": blocks of 32 consecutive
    values along the last axis share a float32 scale s = max|x| / 127; each value is stored as the
    integer code rint(x / s) (ties to even; 0 when s = 0) and read back as code * s.  The rounding
    decisions are taken in float32, the precision of the cache; the result is returned in x's dtype."""
    x = np.asarray(x)
    if kv == "f32":
        return x
    x32 = x.astype(np.float32)
    if kv == "f16":
        return x32.astype(np.float16).astype(x.dtype)
    if kv != "q8":
        raise ValueError(f"unknown KV cache type {kv!r}")
    hd = x.shape[-1]
    if hd % Q8_BLOCK:
        raise ValueError("q8 cache rows need a multiple of 32 values")
    b = x32.reshape(*x.shape[:-1], hd // Q8_BLOCK, Q8_BLOCK)
    s = np.max(np.abs(b), axis=-1, keepdims=True) / np.float32(127.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        code = np.where(s > 0, np.rint(b / np.where(s > 0, s, np.float32(1.0))), np.float32(0.0))
    return (code * s).reshape(x.shape).astype(x.dtype)


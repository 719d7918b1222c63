"""Elementwise and normalisation primitives of the model, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def bf16_decode(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """BF16 bit patterns (uint16) -> values: a BF16 is the top half of an IEEE float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(dtype)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis (the gain multiplies after normalising)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def l2norm(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(sum(x^2) + eps) over the last axis (per head)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def sigmoid(z):
    """1 / (1 + e^-z), evaluated without overflow for either sign of z."""
    z = np.asarray(z)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(z):
    """log(1 + e^z) = max(z, 0) + log1p(e^-|z|)."""
    z = np.asarray(z)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def silu(z):
    """z * sigmoid(z)."""
    return z * sigmoid(z)


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def rope_angles(head_dim: int, theta: float, positions, dtype=np.float64):
    """cos, sin of angle pos * theta^(-2i/head_dim) for i < head_dim/2; shape [..., head_dim/2]."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * inv_freq
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE: element i pairs with element i + head_dim/2 and the pair turns by its angle.

    x: [..., head_dim]; cos/sin broadcast against [..., head_dim/2]."""
    half = x.shape[-1] // 2
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)

"""Seeded token sequences: prompts and speculative drafts.

The pages time a 520-token prompt and 128 generated tokens on real text
(luce-megakernel announcement, page 1, results table).  No text corpus is used
here: token ids are uniform over the vocabulary, which keeps the shapes of the
pages' runs (prompt length, number of decode steps) without their data.
"""
from __future__ import annotations

import numpy as np


def make_prompt(vocab: int, n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 1])
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def make_drafts(vocab: int, k: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 2])
    return rng.integers(0, vocab, size=k, dtype=np.int64).astype(np.int32)

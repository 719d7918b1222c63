"""Agreement metrics between a candidate's logits/state and the oracle's.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages score an engine against a reference by how often the top token
matches and by the mean KL divergence in nats (Reddit follow-up on the 27B
megakernel, page 3, decode-accuracy table); relative L2 is added because with
random weights the softmax is nearly flat and KL alone is a weak check.
"""
from __future__ import annotations

import numpy as np


def rel_l2(candidate, reference) -> float:
    c = np.asarray(candidate, dtype=np.float64)
    r = np.asarray(reference, dtype=np.float64)
    return float(np.linalg.norm((c - r).ravel()) / max(np.linalg.norm(r.ravel()), 1e-300))


def _log_softmax(z):
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    return z - m - np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True))


def mean_kl(ref_logits, cand_logits) -> float:
    """Mean over rows of KL(p_ref || p_cand) in nats."""
    lr = _log_softmax(np.atleast_2d(ref_logits))
    lc = _log_softmax(np.atleast_2d(cand_logits))
    kl = np.sum(np.exp(lr) * (lr - lc), axis=-1)
    return float(np.mean(kl))


def top1_agreement(ref_logits, cand_logits) -> float:
    r = np.argmax(np.atleast_2d(ref_logits), axis=-1)
    c = np.argmax(np.atleast_2d(cand_logits), axis=-1)
    return float(np.mean(r == c))

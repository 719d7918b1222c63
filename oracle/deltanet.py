"""Gated delta rule (the DeltaNet mixer's learned recurrence), in four independent forms.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the mixer only as linear attention with a learned recurrence whose
cost grows linearly with context (luce-megakernel announcement, page 1, the
paragraph on the hybrid layer pattern) and say its recurrence runs in FP32
registers (same page, kernel-design bullets).  The recurrence itself is the gated
delta rule of Gated DeltaNet (Yang, Kautz, Hatamizadeh, ICLR 2025):

    A_t = alpha_t (I - beta_t k_t k_t^T)
    S_t = S_{t-1} A_t + beta_t v_t k_t^T          S in R^{dv x dk}
    o_t = S_t q_t                                  (read after the update)

with k, q already L2-normalised.  Shapes: a leading head axis is allowed
everywhere (``[..., dk]`` etc.).

Forms:
* ``delta_step`` / ``delta_recurrent`` -- the recurrence above, literally, with the
  dk x dk transition matrix built each step.
* ``delta_explicit_product`` -- brute force: S_t = S_0 A_1...A_t +
  sum_j beta_j v_j k_j^T A_{j+1}...A_t for every t (tiny sizes only).
* ``delta_parallel`` -- the whole sequence at once.  Writing
  u_t = beta_t (v_t - alpha_t S_{t-1} k_t), the recurrence becomes
  S_t = alpha_t S_{t-1} + u_t k_t^T, so with gamma_t = prod_{i<=t} alpha_i and
  G_tj = gamma_t / gamma_j:
      (I + strict_lower(diag(beta) (K K^T * G))) U = diag(beta) (V - diag(gamma) K S_0^T)
      O   = diag(gamma) Q S_0^T + lower(Q K^T * G) U          (lower includes the diagonal)
      S_T = gamma_T S_0 + U^T diag(gamma_T / gamma) K
  G is formed as exp(g_t - g_j) from cumulative log-decays, never as a ratio.
* ``delta_chunked`` -- ``delta_parallel`` applied chunk by chunk with the state
  carried between chunks (the chunkwise algorithm a multi-token kernel uses).
"""
from __future__ import annotations

import numpy as np

from .primitives import sigmoid, softplus


def gates(a, b):
    """alpha = exp(-softplus(a)) in (0, 1), beta = sigmoid(b) in (0, 1); one scalar per head per token."""
    return np.exp(-softplus(a)), sigmoid(b)


def delta_step(S, q, k, v, alpha, beta):
    """One token: S [..., dv, dk], q/k [..., dk], v [..., dv], alpha/beta [...] -> (S_new, o)."""
    dk = k.shape[-1]
    eye = np.eye(dk, dtype=S.dtype)
    a = np.asarray(alpha, dtype=S.dtype)[..., None, None]
    b = np.asarray(beta, dtype=S.dtype)[..., None, None]
    A = a * (eye - b * (k[..., :, None] * k[..., None, :]))
    S_new = S @ A + b * (v[..., :, None] * k[..., None, :])
    o = (S_new @ q[..., :, None])[..., 0]
    return S_new, o


def delta_recurrent(S0, Q, K, V, alpha, beta):
    """Sequence of steps.  Q/K [T, ..., dk], V [T, ..., dv], alpha/beta [T, ...] -> (O [T, ..., dv], S_T)."""
    S = np.array(S0, copy=True)
    outs = []
    for t in range(Q.shape[0]):
        S, o = delta_step(S, Q[t], K[t], V[t], alpha[t], beta[t])
        outs.append(o)
    return np.stack(outs), S


def delta_explicit_product(S0, Q, K, V, alpha, beta):
    """Brute force over matrix products, single head: S0 [dv, dk], Q/K [T, dk], V [T, dv], alpha/beta [T]."""
    T, dk = K.shape
    eye = np.eye(dk, dtype=S0.dtype)
    A = [alpha[t] * (eye - beta[t] * np.outer(K[t], K[t])) for t in range(T)]
    outs, S_t = [], None
    for t in range(T):
        P = eye.copy()
        for i in range(t + 1):
            P = P @ A[i]
        S_t = S0 @ P
        for j in range(t + 1):
            Pj = eye.copy()
            for i in range(j + 1, t + 1):
                Pj = Pj @ A[i]
            S_t = S_t + beta[j] * np.outer(V[j], K[j]) @ Pj
        outs.append(S_t @ Q[t])
    return np.stack(outs), S_t


def delta_parallel(S0, Q, K, V, alpha, beta):
    """Whole-sequence form for one head: S0 [dv, dk], Q/K [T, dk], V [T, dv], alpha/beta [T]."""
    T = K.shape[0]
    g = np.cumsum(np.log(alpha))                 # log gamma_t
    lower = np.tril(np.ones((T, T), dtype=bool))
    strict = np.tril(np.ones((T, T), dtype=bool), -1)
    # gamma_t / gamma_j for j <= t; the upper triangle is masked to exp(-inf) = 0 before
    # exponentiating, so its positive log differences never overflow
    G = np.exp(np.where(lower, g[:, None] - g[None, :], -np.inf))
    gamma = np.exp(g)
    KK = np.where(strict, (K @ K.T) * G, 0.0)
    M = np.eye(T, dtype=K.dtype) + beta[:, None] * KK
    rhs = beta[:, None] * (V - gamma[:, None] * (K @ S0.T))
    U = np.linalg.solve(M, rhs)
    QK = np.where(lower, (Q @ K.T) * G, 0.0)
    O = gamma[:, None] * (Q @ S0.T) + QK @ U
    decay_to_end = np.exp(g[-1] - g)             # gamma_T / gamma_j
    S_T = gamma[-1] * S0 + U.T @ (decay_to_end[:, None] * K)
    return O, S_T


def delta_chunked(S0, Q, K, V, alpha, beta, chunk: int):
    """``delta_parallel`` on consecutive chunks of ``chunk`` tokens, carrying the state (one head)."""
    T = K.shape[0]
    S = np.array(S0, copy=True)
    outs = []
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        O, S = delta_parallel(S, Q[c0:c1], K[c0:c1], V[c0:c1], alpha[c0:c1], beta[c0:c1])
        outs.append(O)
    return np.concatenate(outs, axis=0), S

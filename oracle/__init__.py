"""CPU oracle for the hybrid Gated-DeltaNet + full-attention decoder.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
never calls it and shares no code with it: the two meet only through the seeded
inputs of the ``synth`` package.

What it computes: the plain, unfused forward pass of the model the pages run as
one kernel (luce-megakernel announcement, page 1: 24 layers, 18 DeltaNet layers
with a learned linear recurrence and 6 full-attention layers, BF16 weights with
FP32 accumulation).  The pages give no equations; the readings used here are:

* DeltaNet mixer: the gated delta rule ``S <- alpha*S(I - beta*k k^T) + beta*v k^T``,
  ``o = S q`` with L2-normalised q and k, ``beta = sigmoid(w_b.x)``,
  ``alpha = exp(-softplus(w_a.x))`` (Gated DeltaNet, Yang, Kautz and
  Hatamizadeh, ICLR 2025), S in R^{dv x dk}, read after the update, S_0 = 0,
  no 1/sqrt(dk) on q.
* Attention: grouped-query causal softmax attention with rotate-half RoPE
  (theta 10000), scale 1/sqrt(head_dim), KV cache holds rotated keys.
* Block: pre-norm residual, RMSNorm (eps 1e-6, gain after normalising), SwiGLU
  FFN, final RMSNorm, tied LM head, greedy argmax with the lowest index on ties.

* 4-bit weights (the 27B-scale model): groups of 32 columns with an FP16 scale d and
  offset m, weight = d*q + m (``quant.py`` decodes the byte layout; the decoded values
  are exact in float64, so the oracle runs on the stored weights exactly).

Everything runs in float64 by default (``dtype`` may be set to float32 for the
float32-vs-float64 gap check).  Functions that run the model two independent
ways -- ``Oracle.step`` (token by token, recurrent DeltaNet, KV cache) and
``Oracle.forward`` (whole sequence, parallel DeltaNet form, full causal score
matrix) -- are pinned against each other and against closed forms in
``tests/test_oracle_*.py``.
"""
from .primitives import rmsnorm, l2norm, sigmoid, softplus, silu, rope_angles, rope, softmax, bf16_decode
from .deltanet import (gates, delta_step, delta_recurrent, delta_explicit_product,
                       delta_parallel, delta_chunked)
from .attention import attend_one, causal_attention, kv_round, KV_DTYPES
from .model import Oracle
from .metrics import rel_l2, mean_kl, top1_agreement
from .quant import q4g32_dequant, q4g32_dequant_rows

__all__ = ["rmsnorm", "l2norm", "sigmoid", "softplus", "silu", "rope_angles", "rope", "softmax",
           "bf16_decode", "gates", "delta_step", "delta_recurrent", "delta_explicit_product",
           "delta_parallel", "delta_chunked", "attend_one", "causal_attention", "kv_round", "KV_DTYPES", "Oracle",
           "rel_l2", "mean_kl", "top1_agreement", "q4g32_dequant", "q4g32_dequant_rows"]

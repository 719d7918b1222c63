"""Shared helpers of the GPU tests: run the HIP library and the oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np

import synth


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device")
    return torch


def new_model(cfg, weights, grid=None, weight_dtype=None, kv_dtype=None, max_verify_k=0):
    from hybrid_deltanet_attention_amd import Model
    from hybrid_deltanet_attention_amd.binding import MK_BF16, MK_F32
    m = Model(cfg, device=0, weight_dtype=MK_BF16 if weight_dtype is None else weight_dtype,
              kv_dtype=MK_F32 if kv_dtype is None else kv_dtype, max_verify_k=max_verify_k)
    m.mk_load_weights(weights)
    if grid is not None:
        m.mk_set_grid(grid)
    return m


def run_teacher_forced(m, prompt, fed, want_logits=True):
    """mk_prefill(prompt) then one mk_decode_step per token in ``fed`` (the oracle's tokens).

    Returns (prefill logits, prefill next token, [decode logits], [decode next tokens])."""
    torch = torch_cuda()
    vocab = m.cfg.vocab
    d_prompt = torch.tensor(np.asarray(prompt, dtype=np.int32), device="cuda")
    d_next = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_logits = torch.empty(vocab, dtype=torch.float32, device="cuda") if want_logits else None
    m.mk_prefill(d_prompt, len(prompt), d_next, d_logits)
    m.mk_sync()
    pre_logits = d_logits.cpu().numpy().copy() if want_logits else None
    pre_next = int(d_next.item())
    d_fed = torch.tensor(np.asarray(fed, dtype=np.int32), device="cuda")
    out_l, out_n = [], []
    for t in range(len(fed)):
        m.mk_decode_step(d_fed[t:t + 1], d_next, d_logits)
        if want_logits:
            out_l.append(d_logits.cpu().numpy().copy())
        out_n.append(int(d_next.item()))
    m.mk_sync()
    return pre_logits, pre_next, out_l, out_n


def oracle_reference(cfg, weights, prompt, n_steps, cache_bytes=None, kv="f32"):
    from oracle import Oracle
    o = Oracle(cfg, weights, kv=kv)
    if cache_bytes is not None:
        o.W.cache_left = cache_bytes  # keep every decoded 4-bit matrix (wide models)
    fed, logits, last = o.greedy(prompt, n_steps)
    return o, fed, logits, last

"""The 0.8B-shaped hybrid at full size: pp512 prefill then 128 teacher-forced decode steps vs the oracle.

The oracle runs the prompt with its whole-sequence form and the decode steps token by token, in
fp64; the GPU runs the same tokens in the launch configuration the benchmark times (default grid,
one launch per token).  Bars: logits relative L2 <= 1e-2 at every step, top-1 agreement >= 99 %,
mean KL <= 1e-3 nats, DeltaNet state relative L2 <= 1e-3 per layer after the 128 steps.
"""
import time

import numpy as np
import pytest

import synth
from oracle.metrics import rel_l2, mean_kl, top1_agreement
from gpu_util import new_model, run_teacher_forced, oracle_reference

pytestmark = pytest.mark.gpu


def test_0p8b_prompt512_decode128():
    cfg = synth.get_config("hybrid_0p8b")
    W = synth.make_weights(cfg, 0)
    prompt = synth.make_prompt(cfg.vocab, 512, 0)
    t0 = time.time()
    o, fed, ref_logits, ref_last = oracle_reference(cfg, W, prompt, 128)
    print(f"oracle done in {time.time() - t0:.1f}s", flush=True)
    m = new_model(cfg, W)
    pre_l, pre_n, dec_l, dec_n = run_teacher_forced(m, prompt, fed)
    e_pre = rel_l2(pre_l, ref_last)
    errs = [rel_l2(g, r) for g, r in zip(dec_l, ref_logits)]
    G = np.stack(dec_l)
    print(f"prefill logits rel-L2 {e_pre:.2e}; decode max {max(errs):.2e} mean {np.mean(errs):.2e}; "
          f"top1 {top1_agreement(ref_logits, G):.4f}; KL {mean_kl(ref_logits, G):.2e}", flush=True)
    assert e_pre <= 1e-2
    assert pre_n == int(np.argmax(pre_l))
    assert max(errs) <= 1e-2
    assert top1_agreement(ref_logits, G) >= 0.99
    assert mean_kl(ref_logits, G) <= 1e-3
    assert all(dec_n[t] == int(np.argmax(dec_l[t])) for t in range(len(dec_l)))
    worst = 0.0
    for l in range(cfg.n_layers):
        if not cfg.is_attention(l):
            e = rel_l2(m.mk_read_state(l), o.S[l])
            worst = max(worst, e)
            assert e <= 1e-3, f"layer {l} state rel-L2 {e:.2e}"
    T = 512 + 128
    kv = m.mk_read_state(3)
    ek = rel_l2(kv[0][:, :T], o.Kc[3][:, :T])
    print(f"worst DeltaNet state rel-L2 {worst:.2e}; layer 3 K rel-L2 {ek:.2e}", flush=True)
    assert ek <= 1e-3
    m.close()

"""Decode at long context: the 0.8B shape with a 32,768-position KV cache.

A 30,000-token prompt runs through the GPU prefill (the oracle's whole-sequence form at 30K tokens
is out of reach on the host).  The GPU's DeltaNet states and KV caches are then handed to the
oracle (mk_read_state), and both decode the same tokens from there, the oracle choosing them:
logits relative L2 <= 1e-2 at every step, top-1 agreement on every step, DeltaNet state relative
L2 <= 1e-3 after the steps.  This checks split-K attention over ~1,900 16-position items per KV
head and the combine of that many partials per output.
"""
import time

import numpy as np
import pytest

import synth
from oracle import Oracle
from oracle.metrics import rel_l2
from gpu_util import new_model, torch_cuda

pytestmark = pytest.mark.gpu


def test_0p8b_32k_context_decode():
    torch = torch_cuda()
    cfg = synth.get_config("hybrid_0p8b", max_ctx=32768)
    W = synth.make_weights(cfg, 0)
    T = 30000
    prompt = synth.make_prompt(cfg.vocab, T, 11)
    m = new_model(cfg, W)
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    t0 = time.time()
    m.mk_prefill(torch.tensor(prompt, device="cuda"), T, nxt)
    m.mk_sync()
    print(f"GPU prefill of {T} tokens: {time.time() - t0:.2f}s", flush=True)
    o = Oracle(cfg, W)
    for l in range(cfg.n_layers):
        st = m.mk_read_state(l)
        if cfg.is_attention(l):
            o.Kc[l][:] = st[0]
            o.Vc[l][:] = st[1]
        else:
            o.S[l] = st.astype(np.float64)
    o.pos = T
    tok = int(nxt.item())
    d_tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_log = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    errs = []
    for s in range(6):
        d_tok.fill_(tok)
        m.mk_decode_step(d_tok, nxt, d_log)
        ref = o.step(tok)
        g = d_log.cpu().numpy()
        errs.append(rel_l2(g, ref))
        assert int(nxt.item()) == int(np.argmax(g))
        assert int(np.argmax(g)) == int(np.argmax(ref)) or abs(ref[np.argmax(g)] - ref.max()) <= 1e-4 * np.abs(ref).max()
        tok = int(np.argmax(ref))
    print(f"decode logits rel-L2 per step: {' '.join(f'{e:.2e}' for e in errs)}", flush=True)
    assert max(errs) <= 1e-2
    for l in range(cfg.n_layers):
        if not cfg.is_attention(l):
            e = rel_l2(m.mk_read_state(l), o.S[l])
            assert e <= 1e-3, f"layer {l} state rel-L2 {e:.2e}"
    assert m.mk_get_position() == T + 6
    m.close()

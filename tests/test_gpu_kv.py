"""Compact KV caches (MK_F16, MK_Q8) against the oracle with the same cache type.

The follow-up post on the 27B megakernel keeps its KV cache in fp16 up to about 80K positions and
in an 8-bit format above (Reddit follow-up, page 3, "Limits" paragraph).  Here a context's whole
cache is binary16, or int8 codes with one FP32 scale per 32 values; keys and values are rounded to
the cache type as they enter the cache, and attention (the entering position included) reads the
stored values.  The oracle rounds the same way (oracle.attention.kv_round), so the bars are the FP32
cache's: logits relative L2 <= 1e-2 at every step, top-1 >= 99 %, mean KL <= 1e-3 nats, DeltaNet state
and KV relative L2 <= 1e-3 -- except that int8 entries may differ by one code where the two sides'
inputs straddle a rounding boundary (at most one step each, at most 1 % of them).  The verify launch must equal sequential decode launches bit for bit with
a compact cache too.  Long contexts: a 30,000-token binary16 cache and a 96,000-token int8 cache built
by the GPU prefill are handed to the oracle, and both decode the same tokens from there.
"""
import time

import numpy as np
import pytest

import synth
from oracle import Oracle
from oracle.metrics import rel_l2
from gpu_util import new_model, torch_cuda
from test_gpu_parity import _check_run, kv_cache_close
from test_gpu_verify import _check_against_decode

pytestmark = pytest.mark.gpu

MK_F16, MK_Q8, MK_Q4G32 = 3, 6, 5
KVS = [MK_F16, MK_Q8]
IDS = ["f16", "q8"]


@pytest.mark.parametrize("kv", KVS, ids=IDS)
def test_tiny_prefill_then_decode(kv):
    cfg = synth.get_config("tiny")
    W = synth.make_weights(cfg, 30)
    _check_run(cfg, W, synth.make_prompt(cfg.vocab, 40, 30), 24, kv_dtype=kv)


@pytest.mark.parametrize("kv", KVS, ids=IDS)
def test_tiny_multi_chunk_items_odd_grid(kv):
    # an 8,192-position cache: each split-K attention item walks 4 chunks of 16 positions
    cfg = synth.get_config("tiny", max_ctx=8192)
    W = synth.make_weights(cfg, 31)
    _check_run(cfg, W, synth.make_prompt(cfg.vocab, 150, 31), 20, grid=37, kv_dtype=kv)


@pytest.mark.parametrize("kv", KVS, ids=IDS)
def test_tiny_many_items_per_workgroup(kv):
    # an 8,192-position cache (items of 4 chunks) on a grid of 8 after a 1,500-token prompt: each
    # workgroup walks about 6 items, 24 chunks, in passes of three and one chunk, and its six chunk
    # buffers wrap around several times.  Decode against the oracle, then the verify launch (which
    # takes the chunks one at a time) against decode launches, bit for bit.
    cfg = synth.get_config("tiny", max_ctx=8192)
    W = synth.make_weights(cfg, 36)
    prompt = synth.make_prompt(cfg.vocab, 1500, 36)
    _check_run(cfg, W, prompt, 8, grid=8, kv_dtype=kv)
    assert _check_against_decode(cfg, W, prompt, lambda c: c, 5, grid=8, label="many items", kv_dtype=kv) == 5


@pytest.mark.parametrize("kv", KVS, ids=IDS)
def test_head_dim_96_prompt_through_decode(kv):
    # head_dim 96: rows that do not fill the 1 KB staging slots evenly; the prompt runs through the
    # decode kernel (the matrix-core prefill attention takes head sizes 64 and 128)
    cfg = synth.get_config("tiny", head_dim=96, n_q_heads=4, n_kv_heads=2, max_ctx=128)
    W = synth.make_weights(cfg, 32)
    _check_run(cfg, W, synth.make_prompt(cfg.vocab, 35, 32), 16, kv_dtype=kv)


@pytest.mark.parametrize("kv", KVS, ids=IDS)
def test_q4_weights_with_compact_cache(kv):
    cfg = synth.get_config("tiny")
    W = synth.make_q4_weights(cfg, 33)
    _check_run(cfg, W, synth.make_prompt(cfg.vocab, 20, 33), 16, weight_dtype=MK_Q4G32, kv_dtype=kv)


@pytest.mark.parametrize("kv", KVS, ids=IDS)
def test_verify_equals_decode_bitwise(kv):
    cfg = synth.get_config("tiny", max_ctx=512)
    W = synth.make_weights(cfg, 34)
    prompt = synth.make_prompt(cfg.vocab, 45, 34)
    assert _check_against_decode(cfg, W, prompt, lambda c: c, 5, label="greedy", kv_dtype=kv) == 5

    def plant(c):
        d = list(c)
        d[2] = (d[2] + 1) % cfg.vocab
        return d
    assert _check_against_decode(cfg, W, prompt, plant, 5, grid=37, label="mismatch@2", kv_dtype=kv) == 2


@pytest.mark.parametrize("kv", KVS, ids=IDS)
def test_state_read_write_keeps_stored_values(kv):
    """read_state gives the stored values (exact binary16, or int8 code times scale); writing them
    back and reading again changes nothing beyond the scale's last bit"""
    torch = torch_cuda()
    cfg = synth.get_config("tiny")
    W = synth.make_weights(cfg, 35)
    m = new_model(cfg, W, kv_dtype=kv)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    m.mk_prefill(torch.tensor(synth.make_prompt(cfg.vocab, 30, 35), device="cuda"), 30, tok)
    m.mk_sync()
    a = m.mk_read_state(3)
    K = a[0][:, :30].astype(np.float64)
    if kv == MK_F16:
        assert np.array_equal(K, K.astype(np.float16).astype(np.float64))
    else:
        b = K.reshape(*K.shape[:-1], -1, 32)
        sc = np.abs(b).max(-1, keepdims=True) / 127
        q = np.where(sc > 0, b / np.where(sc > 0, sc, 1), 0)
        assert np.max(np.abs(q - np.rint(q))) < 1e-4
    m.mk_write_state(3, a)
    b2 = m.mk_read_state(3)
    assert rel_l2(b2, a) <= 1e-6
    m.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kv,T", [(MK_F16, 30000), (MK_Q8, 96000)], ids=["f16-30k", "q8-96k"])
def test_0p8b_long_context_decode(kv, T):
    torch = torch_cuda()
    max_ctx = 32768 if T <= 32000 else 98304
    cfg = synth.get_config("hybrid_0p8b", max_ctx=max_ctx)
    W = synth.make_weights(cfg, 0)
    prompt = synth.make_prompt(cfg.vocab, T, 12)
    m = new_model(cfg, W, kv_dtype=kv)
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    t0 = time.time()
    m.mk_prefill(torch.tensor(prompt, device="cuda"), T, nxt)
    m.mk_sync()
    print(f"GPU prefill of {T} tokens ({IDS[KVS.index(kv)]} cache): {time.time() - t0:.2f}s", flush=True)
    o = Oracle(cfg, W, kv=IDS[KVS.index(kv)])
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
    for s in range(4):
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
        st = m.mk_read_state(l)
        if cfg.is_attention(l):
            kvn = IDS[KVS.index(kv)]
            kv_cache_close(st[0][:, :T + 4], o.Kc[l][:, :T + 4], kvn, f"layer {l} K")
            kv_cache_close(st[1][:, :T + 4], o.Vc[l][:, :T + 4], kvn, f"layer {l} V")
        else:
            e = rel_l2(st, o.S[l])
            assert e <= 1e-3, f"layer {l} rel-L2 {e:.2e}"
    assert m.mk_get_position() == T + 4
    m.close()

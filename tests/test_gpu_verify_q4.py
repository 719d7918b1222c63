"""mk_verify_k with 4-bit (Q4G32) weights: the pending token and up to 5 drafts in one launch.

Against the 4-bit decode kernel (bitwise): the verify launch packs every position's activations as
the decode kernel packs them and forms every sum in its order, so its choices, accepted count,
DeltaNet states and KV entries must equal those of k + 1 (choices) and a + 1 (state) sequential
4-bit decode launches exactly.  Against the oracle (Oracle.verify, pinned to the whole-sequence form):
choices and accepted count, and the rolled-back state to the decode bars, on the tiny shape and on a
4-layer slice at the 27B-scale width whose 30,000-token context (DeltaNet states and a binary16 KV
cache built on the GPU) is handed to the oracle, as the speculative-verify workload has it (Reddit
follow-up on the 27B megakernel, page 3: drafts checked against a long code context).
"""
import numpy as np
import pytest

import synth
from oracle import Oracle
from oracle.metrics import rel_l2
from gpu_util import torch_cuda
from test_gpu_parity import kv_cache_close
from test_gpu_verify import _check_against_decode, _verify_model, _dev

pytestmark = pytest.mark.gpu

MK_Q4G32, MK_F32, MK_F16, MK_Q8 = 5, 2, 3, 6


@pytest.mark.parametrize("seed", [0, 1])
def test_q4_tiny_equals_decode_bitwise(seed):
    cfg = synth.get_config("tiny")
    W = synth.make_q4_weights(cfg, seed)
    prompt = synth.make_prompt(cfg.vocab, 14, seed)
    assert _check_against_decode(cfg, W, prompt, lambda c: c, 5, label="q4 greedy", weight_dtype=MK_Q4G32) == 5

    def plant(c):
        d = list(c)
        d[3] = (d[3] + 1) % cfg.vocab
        return d
    assert _check_against_decode(cfg, W, prompt, plant, 5, label="q4 mismatch@3", weight_dtype=MK_Q4G32) == 3
    _check_against_decode(cfg, W, prompt, lambda c: synth.make_drafts(cfg.vocab, len(c), seed), 5, label="q4 random",
                          weight_dtype=MK_Q4G32)


def test_q4_ragged_odd_grid_and_f16_cache():
    cfg = synth.get_config("tiny", hidden=224, ffn=352, dn_heads=3, dn_dk=32, dn_dv=32, n_q_heads=6,
                           n_kv_heads=3, head_dim=32, vocab=1000, n_layers=5, max_ctx=96)
    W = synth.make_q4_weights(cfg, 5, gain_noise=0.1)
    prompt = synth.make_prompt(cfg.vocab, 21, 5)
    assert _check_against_decode(cfg, W, prompt, lambda c: c, 4, grid=37, label="q4 ragged",
                                 weight_dtype=MK_Q4G32) == 4
    assert _check_against_decode(cfg, W, prompt, lambda c: c, 5, label="q4 f16 kv", kv_dtype=MK_F16,
                                 weight_dtype=MK_Q4G32) == 5


def _oracle_from_gpu(cfg, W, m, T, kv="f32", cache_bytes=None):
    o = Oracle(cfg, W, kv=kv)
    if cache_bytes is not None:
        o.W.cache_left = cache_bytes
    for l in range(cfg.n_layers):
        st = m.mk_read_state(l)
        if cfg.is_attention(l):
            o.Kc[l][:] = st[0]
            o.Vc[l][:] = st[1]
        else:
            o.S[l] = st.astype(np.float64)
    o.pos = T
    return o


def _verify_vs_oracle(cfg, W, prompt, seed, kv_dtype=MK_F32, kv="f32", cache_bytes=None, grid=None,
                      decode_steps=0):
    """GPU prompt (decode launches), state handed to the oracle; greedy, planted and random drafts
    scored by one verify launch each (from the same handed-off state) and by Oracle.verify; then,
    with decode_steps, that many teacher-forced decode launches from the same state against the
    oracle's steps (logits relative L2 <= 1e-2, the fused argmax of the launch's own logits)"""
    torch = torch_cuda()
    mv = _verify_model(cfg, W, 5, grid, kv_dtype, MK_Q4G32)
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    T = len(prompt)

    def gpu_prompt():
        mv.mk_reset()
        mv.mk_prefill(_dev(prompt), T, nxt)
        mv.mk_sync()
        return int(nxt.item())

    pend = gpu_prompt()
    o = _oracle_from_gpu(cfg, W, mv, T, kv, cache_bytes)
    start = o.snapshot()
    cont, t = [], pend
    for _ in range(5):
        t = o.argmax(o.step(t))
        cont.append(t)
    cases = {"greedy": cont, "planted@1": cont[:1] + [(cont[1] + 3) % cfg.vocab] + cont[2:],
             "random": [int(x) for x in synth.make_drafts(cfg.vocab, 5, seed)]}
    for label, drafts in cases.items():
        o.restore(start)
        r = o.verify([pend] + drafts)
        assert gpu_prompt() == pend
        out = torch.full((6,), -7, dtype=torch.int32, device="cuda")
        acc = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        mv.mk_verify_k(_dev([pend] + drafts), 5, out, acc)
        mv.mk_sync()
        y, a = [int(v) for v in out.cpu().numpy()], int(acc.item())
        print(f"[q4 verify {cfg.name} T={T} {label}] gpu {y} a={a} oracle {r['y']} a={r['a']}", flush=True)
        for i, (g, ref) in enumerate(zip(y[: a + 1], r["y"][: a + 1])):
            if g != ref:
                lg = r["logits"][i]
                assert abs(lg[g] - lg[ref]) <= 1e-4 * np.abs(lg).max(), f"{label}: choice {i} {g} vs {ref}"
        assert a == r["a"], f"{label}: accepted {a} vs oracle {r['a']}"
        P = o.pos
        for l in range(cfg.n_layers):
            st = mv.mk_read_state(l)
            if cfg.is_attention(l):
                kv_cache_close(st[0][:, T - 2:P], o.Kc[l][:, T - 2:P], kv, f"{label} layer {l} K")
                kv_cache_close(st[1][:, T - 2:P], o.Vc[l][:, T - 2:P], kv, f"{label} layer {l} V")
            else:
                e = rel_l2(st, o.S[l])
                assert e <= 1e-3, f"{label}: layer {l} state rel-L2 {e:.2e}"
        assert mv.mk_get_position() == P
    if decode_steps:
        o.restore(start)
        assert gpu_prompt() == pend
        d_tok = torch.zeros(1, dtype=torch.int32, device="cuda")
        d_next = torch.zeros(1, dtype=torch.int32, device="cuda")
        d_lg = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
        t = pend
        for i in range(decode_steps):
            d_tok.fill_(t)
            mv.mk_decode_step(d_tok, d_next, d_lg)
            mv.mk_sync()
            g = d_lg.cpu().numpy()
            ref = o.step(t)
            e = rel_l2(g, ref)
            print(f"[q4 decode {cfg.name} T={T} step {i}] logits rel-L2 {e:.2e}", flush=True)
            assert e <= 1e-2, f"decode step {i}: logits rel-L2 {e:.2e}"
            assert int(d_next.item()) == int(np.argmax(g))
            t = o.argmax(ref)
    mv.close()


def test_q4_tiny_against_oracle_verify():
    cfg = synth.get_config("tiny")
    W = synth.make_q4_weights(cfg, 7)
    _verify_vs_oracle(cfg, W, [int(t) for t in synth.make_prompt(cfg.vocab, 12, 7)], 7)


@pytest.mark.timeout(1200)
def test_q4_27b_width_slice_30k_context_against_oracle_verify():
    cfg = synth.get_config("hybrid_27b", n_layers=4, max_ctx=32768)
    W = synth.make_q4_weights(cfg, 0)
    prompt = [int(t) for t in synth.make_prompt(cfg.vocab, 30000, 13)]
    # the decode steps run the shape-specialised 4-bit kernel, whose attention takes the binary16
    # chunks two at a time
    _verify_vs_oracle(cfg, W, prompt, 13, kv_dtype=MK_F16, kv="f16", cache_bytes=1 << 36, decode_steps=3)


@pytest.mark.timeout(900)
def test_q4_27b_width_slice_int8_cache_against_oracle():
    # an int8 cache at 27B width: an 8,192-position cache (attention items of 4 chunks, which the
    # shape-specialised 4-bit decode kernel takes two at a time) after a 2,000-token prompt; verify
    # and decode against the oracle from the handed-off context
    cfg = synth.get_config("hybrid_27b", n_layers=4, max_ctx=8192)
    W = synth.make_q4_weights(cfg, 2)
    prompt = [int(t) for t in synth.make_prompt(cfg.vocab, 2000, 14)]
    _verify_vs_oracle(cfg, W, prompt, 14, kv_dtype=MK_Q8, kv="q8", cache_bytes=1 << 36, decode_steps=3)

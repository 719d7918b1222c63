"""The MFMA prefill path (mk_prefill) against the oracle's whole-sequence form.

Prefill leaves the DeltaNet state and the KV cache exactly where token-by-token decode would, and
returns the last position's logits and greedy token.  Cases: a prompt alone (state and cache
checked right after prefill), a prompt longer than one prefill chunk (1024 tokens), a prefill that
continues a context built by an earlier prefill and decode steps, a head grouping the prefill
attention tiling does not cover (handled token by token), three query heads per KV head on the
matrix-core attention (a partly filled head group), DeltaNet key widths that do not fill the chunk
kernels' tiles or exceed them, and 4-bit (Q4G32) weights: every GEMM over 2K columns against the
weights expanded to BF16 high and low parts, the last prompt token through one 4-bit decode launch.
Bars as in test_gpu_parity.
"""
import numpy as np
import pytest

import synth
from oracle import Oracle
from oracle.metrics import rel_l2
from gpu_util import new_model, torch_cuda

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-2
STATE_TOL = 1e-3


def _prefill(m, tokens, want_logits=True):
    torch = torch_cuda()
    d_tok = torch.tensor(np.asarray(tokens, dtype=np.int32), device="cuda")
    d_next = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_logits = torch.empty(m.cfg.vocab, dtype=torch.float32, device="cuda") if want_logits else None
    m.mk_prefill(d_tok, len(tokens), d_next, d_logits)
    m.mk_sync()
    return (d_logits.cpu().numpy() if want_logits else None), int(d_next.item())


def _decode(m, tokens):
    torch = torch_cuda()
    d_next = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_logits = torch.empty(m.cfg.vocab, dtype=torch.float32, device="cuda")
    out = []
    for t in tokens:
        d_tok = torch.tensor([int(t)], dtype=torch.int32, device="cuda")
        m.mk_decode_step(d_tok, d_next, d_logits)
        out.append(d_logits.cpu().numpy().copy())
    m.mk_sync()
    return out


def _check_state(m, cfg, fwd, T):
    for l in range(cfg.n_layers):
        st = m.mk_read_state(l)
        if cfg.is_attention(l):
            K, V = fwd["KV"][l]
            assert rel_l2(st[0][:, :T], K) <= STATE_TOL, f"layer {l} K"
            assert rel_l2(st[1][:, :T], V) <= STATE_TOL, f"layer {l} V"
        else:
            e = rel_l2(st, fwd["S"][l])
            print(f"  layer {l} state rel-L2 {e:.2e}", flush=True)
            assert e <= STATE_TOL, f"layer {l} state rel-L2 {e:.2e}"


@pytest.mark.parametrize("name,n", [("tiny", 16), ("tiny", 200), ("hybrid_0p8b", 520)])
def test_prefill_state_and_logits(name, n):
    cfg = synth.get_config(name)
    W = synth.make_weights(cfg, 0)
    prompt = synth.make_prompt(cfg.vocab, n, 0)
    fwd = Oracle(cfg, W).forward(prompt, logits="last")
    m = new_model(cfg, W)
    lg, nxt = _prefill(m, prompt)
    e = rel_l2(lg, fwd["logits"])
    print(f"[{name} prefill {n}] logits rel-L2 {e:.2e}", flush=True)
    assert e <= LOGIT_TOL
    assert nxt == int(np.argmax(lg))
    assert m.mk_get_position() == n
    _check_state(m, cfg, fwd, n)
    m.close()


def test_prefill_longer_than_one_chunk():
    cfg = synth.get_config("tiny", max_ctx=1200)
    W = synth.make_weights(cfg, 1)
    prompt = synth.make_prompt(cfg.vocab, 1100, 1)
    fwd = Oracle(cfg, W).forward(prompt, logits="last")
    m = new_model(cfg, W)
    lg, nxt = _prefill(m, prompt)
    assert rel_l2(lg, fwd["logits"]) <= LOGIT_TOL
    assert nxt == int(np.argmax(lg))
    _check_state(m, cfg, fwd, 1100)
    m.close()


def test_prefill_continues_a_context():
    """prefill 16 -> 4 decode steps -> prefill 8 more -> 4 decode steps == one whole-sequence pass"""
    cfg = synth.get_config("tiny")
    W = synth.make_weights(cfg, 2)
    a = synth.make_prompt(cfg.vocab, 16, 2)
    b = synth.make_prompt(cfg.vocab, 4, 3)
    c = synth.make_prompt(cfg.vocab, 8, 4)
    d = synth.make_prompt(cfg.vocab, 4, 5)
    seq = np.concatenate([a, b, c, d])
    o = Oracle(cfg, W)
    full = o.forward(seq, logits="all")
    m = new_model(cfg, W)
    _prefill(m, a, want_logits=False)
    dec1 = _decode(m, b)
    lg, _ = _prefill(m, c)
    dec2 = _decode(m, d)
    L = full["logits"]
    for t in range(4):
        assert rel_l2(dec1[t], L[16 + t]) <= LOGIT_TOL
        assert rel_l2(dec2[t], L[28 + t]) <= LOGIT_TOL
    assert rel_l2(lg, L[27]) <= LOGIT_TOL
    assert m.mk_get_position() == 32
    _check_state(m, cfg, full, 32)
    m.close()


def test_prefill_head_grouping_outside_the_tiling():
    # 6 query heads over 2 KV heads (3 per group): prefill runs token by token through decode
    cfg = synth.get_config("tiny", n_q_heads=6, n_kv_heads=2, head_dim=48)
    W = synth.make_weights(cfg, 5)
    prompt = synth.make_prompt(cfg.vocab, 12, 5)
    fwd = Oracle(cfg, W).forward(prompt, logits="last")
    m = new_model(cfg, W)
    lg, nxt = _prefill(m, prompt)
    assert rel_l2(lg, fwd["logits"]) <= LOGIT_TOL
    _check_state(m, cfg, fwd, 12)
    m.close()


@pytest.mark.parametrize("heads,dk,dv", [(3, 48, 40), (2, 96, 64), (2, 192, 64)])
def test_prefill_key_widths(heads, dk, dv):
    # keys narrower than the chunk kernels' 64 / 128-wide tiles (zero-padded columns), and keys wider
    # than 128 (token-by-token recurrence with its own normalisation pass); 100 tokens = one whole
    # chunk and a ragged one
    cfg = synth.get_config("tiny", dn_heads=heads, dn_dk=dk, dn_dv=dv)
    W = synth.make_weights(cfg, 7)
    prompt = synth.make_prompt(cfg.vocab, 100, 7)
    fwd = Oracle(cfg, W).forward(prompt, logits="last")
    m = new_model(cfg, W)
    lg, nxt = _prefill(m, prompt)
    e = rel_l2(lg, fwd["logits"])
    print(f"[dn heads {heads} dk {dk} dv {dv}] logits rel-L2 {e:.2e}", flush=True)
    assert e <= LOGIT_TOL
    assert nxt == int(np.argmax(lg))
    _check_state(m, cfg, fwd, 100)
    m.close()


def test_prefill_mfma_attention_partial_head_group():
    # 6 query heads over 2 KV heads at head size 64: the matrix-core attention's group of four query
    # heads is partly filled (three heads live)
    cfg = synth.get_config("tiny", n_q_heads=6, n_kv_heads=2, head_dim=64)
    W = synth.make_weights(cfg, 6)
    prompt = synth.make_prompt(cfg.vocab, 150, 6)
    fwd = Oracle(cfg, W).forward(prompt, logits="last")
    m = new_model(cfg, W)
    lg, nxt = _prefill(m, prompt)
    e = rel_l2(lg, fwd["logits"])
    print(f"[6q/2kv hd64 prefill 150] logits rel-L2 {e:.2e}", flush=True)
    assert e <= LOGIT_TOL
    assert nxt == int(np.argmax(lg))
    _check_state(m, cfg, fwd, 150)
    m.close()


MK_Q4G32 = 5


@pytest.mark.parametrize("n,max_ctx", [(16, None), (200, None), (1100, 1200)])
def test_prefill_q4_state_and_logits(n, max_ctx):
    # 4-bit weights: 16 tokens (one partial DeltaNet chunk), 200 (several chunks), 1100 (two prefill
    # chunks of up to 1024 tokens before the last token's decode launch)
    cfg = synth.get_config("tiny") if max_ctx is None else synth.get_config("tiny", max_ctx=max_ctx)
    W = synth.make_q4_weights(cfg, 11)
    prompt = synth.make_prompt(cfg.vocab, n, 11)
    fwd = Oracle(cfg, W).forward(prompt, logits="last")
    m = new_model(cfg, W, weight_dtype=MK_Q4G32)
    lg, nxt = _prefill(m, prompt)
    e = rel_l2(lg, fwd["logits"])
    print(f"[tiny 4-bit prefill {n}] logits rel-L2 {e:.2e}", flush=True)
    assert e <= LOGIT_TOL
    assert nxt == int(np.argmax(lg))
    assert m.mk_get_position() == n
    _check_state(m, cfg, fwd, n)
    m.close()

"""mk_verify_k: one launch scores the pending token and k drafts and keeps the accepted prefix.

Against the decode kernel (bitwise): the verify launch forms every sum in the decode kernel's order,
so its greedy choices, accepted count, DeltaNet states and KV entries must equal those of k + 1
(choices) and a + 1 (state) sequential decode launches exactly, at the same grid size.
Against the oracle (Oracle.verify, pinned to the whole-sequence form): choices and accepted count,
and the rolled-back state to the decode bars (state relative L2 <= 1e-3).
"""
import numpy as np
import pytest

import synth
from oracle.metrics import rel_l2
from gpu_util import new_model, torch_cuda

pytestmark = pytest.mark.gpu

STATE_TOL = 1e-3


def _verify_model(cfg, W, max_k, grid=None, kv_dtype=2, weight_dtype=1):
    from hybrid_deltanet_attention_amd import Model
    m = Model(cfg, device=0, max_verify_k=max_k, kv_dtype=kv_dtype, weight_dtype=weight_dtype)
    m.mk_load_weights(W)
    if grid is not None:
        m.mk_set_grid(grid)
    return m


def _dev(a):
    torch = torch_cuda()
    return torch.tensor(np.asarray(a, dtype=np.int32), device="cuda")


def _prefill(m, prompt):
    torch = torch_cuda()
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    m.mk_prefill(_dev(prompt), len(prompt), nxt)
    m.mk_sync()
    return int(nxt.item())


def _decode_tokens(m, toks):
    """one decode launch per token; returns the greedy choice after each"""
    torch = torch_cuda()
    d = _dev(toks)
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = []
    for t in range(len(toks)):
        m.mk_decode_step(d[t:t + 1], nxt)
        out.append(int(nxt.item()))
    m.mk_sync()
    return out


def _verify(m, toks):
    torch = torch_cuda()
    k = len(toks) - 1
    out = torch.full((k + 1,), -7, dtype=torch.int32, device="cuda")
    acc = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    m.mk_verify_k(_dev(toks), k, out, acc)
    m.mk_sync()
    return [int(v) for v in out.cpu().numpy()], int(acc.item())


def _accepted(toks, y):
    a = 0
    while a < len(toks) - 1 and toks[a + 1] == y[a]:
        a += 1
    return a


def _same_state(mv, mr, cfg, pos, what):
    for l in range(cfg.n_layers):
        a, b = mv.mk_read_state(l), mr.mk_read_state(l)
        if cfg.is_attention(l):
            a, b = a[:, :, :pos], b[:, :, :pos]
        assert np.array_equal(a, b), f"{what}: layer {l} differs from sequential decode"


def _check_against_decode(cfg, W, prompt, drafts_of, k, grid=None, label="", kv_dtype=2, weight_dtype=1):
    """drafts_of(greedy continuation) -> drafts; verify == sequential decode, bitwise"""
    mr = new_model(cfg, W, grid, weight_dtype=weight_dtype, kv_dtype=kv_dtype)
    mv = _verify_model(cfg, W, max(k, 1), grid, kv_dtype, weight_dtype)
    pend = _prefill(mr, prompt)
    assert _prefill(mv, prompt) == pend
    # greedy continuation from the reference (k tokens after the pending one)
    cont = _decode_tokens(mr, [pend])
    while len(cont) < k:
        cont += _decode_tokens(mr, cont[-1:])
    drafts = [int(d) for d in drafts_of(cont[:k])]
    toks = [pend] + drafts
    # reference choices: k + 1 decode launches over [pending, d1..dk]
    mr.mk_reset()
    _prefill(mr, prompt)
    y_ref = _decode_tokens(mr, toks)
    a_ref = _accepted(toks, y_ref)
    y, a = _verify(mv, toks)
    print(f"[{cfg.name} {label} k={k} grid={mv.mk_get_grid()}] drafts {drafts} choices {y} accepted {a}", flush=True)
    assert y == y_ref, f"{label}: verify choices {y} != decode choices {y_ref}"
    assert a == a_ref
    # reference state: only the accepted tokens decoded
    mr.mk_reset()
    _prefill(mr, prompt)
    _decode_tokens(mr, toks[: a + 1])
    pos = len(prompt) + a + 1
    assert mv.mk_get_position() == pos == mr.mk_get_position()
    _same_state(mv, mr, cfg, pos, label)
    mr.close()
    mv.close()
    return a


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_greedy_drafts_all_accepted(seed):
    cfg = synth.get_config("tiny")
    W = synth.make_weights(cfg, seed)
    prompt = synth.make_prompt(cfg.vocab, 16, seed)
    for k in (5, 3, 1):
        a = _check_against_decode(cfg, W, prompt, lambda c: c, k, label="greedy")
        assert a == k


def test_tiny_random_drafts():
    cfg = synth.get_config("tiny")
    W = synth.make_weights(cfg, 2)
    prompt = synth.make_prompt(cfg.vocab, 21, 2)
    _check_against_decode(cfg, W, prompt, lambda c: synth.make_drafts(cfg.vocab, len(c), 2), 5, label="random")


@pytest.mark.parametrize("j", [0, 2, 4])
def test_tiny_planted_mismatch(j):
    cfg = synth.get_config("tiny")
    W = synth.make_weights(cfg, 3)
    prompt = synth.make_prompt(cfg.vocab, 12, 3)

    def plant(c):
        d = list(c)
        d[j] = (d[j] + 1) % cfg.vocab
        return d
    a = _check_against_decode(cfg, W, prompt, plant, 5, label=f"mismatch@{j}")
    assert a == j


def test_tiny_k0_and_odd_grid():
    cfg = synth.get_config("tiny")
    W = synth.make_weights(cfg, 4)
    prompt = synth.make_prompt(cfg.vocab, 9, 4)
    assert _check_against_decode(cfg, W, prompt, lambda c: c[:0], 0, label="k=0") == 0
    assert _check_against_decode(cfg, W, prompt, lambda c: c, 4, grid=37, label="grid 37") == 4


def test_tiny_multi_chunk_attention_items():
    """a cache of 8,192 positions: split-K attention items of 4 chunks, merged inside the item"""
    cfg = synth.get_config("tiny", max_ctx=8192)
    W = synth.make_weights(cfg, 10)
    prompt = synth.make_prompt(cfg.vocab, 150, 10)
    assert _check_against_decode(cfg, W, prompt, lambda c: c, 5, label="cpi 4 greedy") == 5
    _check_against_decode(cfg, W, prompt, lambda c: synth.make_drafts(cfg.vocab, len(c), 10), 5, label="cpi 4 random")


def test_tiny_ragged_shapes():
    cfg = synth.get_config("tiny", hidden=200, ffn=328, dn_heads=3, dn_dk=32, dn_dv=48, n_q_heads=6,
                           n_kv_heads=3, head_dim=40, vocab=1000, n_layers=5, max_ctx=80)
    W = synth.make_weights(cfg, 5)
    prompt = synth.make_prompt(cfg.vocab, 30, 5)
    assert _check_against_decode(cfg, W, prompt, lambda c: c, 5, label="ragged") == 5


def test_tiny_session_mixes_verify_decode_prefill():
    """verify, decode and prefill calls in any order keep one consistent sequence"""
    cfg = synth.get_config("tiny")
    W = synth.make_weights(cfg, 6)
    prompt = synth.make_prompt(cfg.vocab, 14, 6)
    extra = synth.make_prompt(cfg.vocab, 7, 60)
    mr = new_model(cfg, W)
    mv = _verify_model(cfg, W, 5)
    stream = []  # tokens fed to the model after the prompt, in order
    pend = _prefill(mv, prompt)
    assert _prefill(mr, prompt) == pend
    # 1: greedy drafts (taken from the reference), all accepted
    cont = _decode_tokens(mr, [pend])
    for _ in range(2):
        cont += _decode_tokens(mr, cont[-1:])
    mr.mk_reset()
    _prefill(mr, prompt)
    y, a = _verify(mv, [pend] + cont[:3])
    assert a == 3 and y[:3] == cont[:3]
    stream += [pend] + cont[:3]
    pend = y[a]
    # 2: random drafts
    d = [int(x) for x in synth.make_drafts(cfg.vocab, 5, 61)]
    y, a = _verify(mv, [pend] + d)
    stream += [pend] + d[:a]
    pend = y[a]
    # 3: two decode steps
    out = _decode_tokens(mv, [pend])
    stream += [pend]
    pend = out[0]
    out = _decode_tokens(mv, [pend])
    stream += [pend]
    pend = out[0]
    # 4: partial acceptance, then a prefill continuing the context
    y, a = _verify(mv, [pend, 1, 2])
    stream += [pend] + [1, 2][:a]
    nxt_v = _prefill(mv, extra)
    # reference: the same tokens through decode only, then the same prefill
    _decode_tokens(mr, stream)
    nxt_r = _prefill(mr, extra)
    assert nxt_v == nxt_r
    pos = len(prompt) + len(stream) + len(extra)
    assert mv.mk_get_position() == pos == mr.mk_get_position()
    _same_state(mv, mr, cfg, pos, "session")
    mr.close()
    mv.close()


def test_tiny_against_oracle_verify():
    """choices, accepted count and rolled-back state vs Oracle.verify (greedy, planted, random drafts)"""
    from oracle import Oracle
    cfg = synth.get_config("tiny")
    W = synth.make_weights(cfg, 8)
    prompt = [int(t) for t in synth.make_prompt(cfg.vocab, 10, 8)]
    o = Oracle(cfg, W)
    fwd = o.forward(prompt, logits="last")
    pend = int(np.argmax(fwd["logits"]))
    # the oracle's greedy continuation
    o.load_state(fwd)
    cont, t = [], pend
    for _ in range(5):
        t = o.argmax(o.step(t))
        cont.append(t)
    cases = {"greedy": cont, "planted@1": cont[:1] + [(cont[1] + 5) % cfg.vocab] + cont[2:],
             "random": [int(x) for x in synth.make_drafts(cfg.vocab, 5, 8)]}
    for label, drafts in cases.items():
        o.load_state(fwd)
        r = o.verify([pend] + drafts)
        mv = _verify_model(cfg, W, 5)
        assert _prefill(mv, prompt) == pend
        y, a = _verify(mv, [pend] + drafts)
        print(f"[oracle {label}] gpu {y} a={a} oracle {r['y']} a={r['a']}", flush=True)
        # a choice may differ only where the oracle's two best logits are within rounding of each other
        for i, (g, ref) in enumerate(zip(y[: a + 1], r["y"][: a + 1])):
            if g != ref:
                lg = r["logits"][i]
                assert abs(lg[g] - lg[ref]) <= 1e-4 * np.abs(lg).max(), f"{label}: choice {i} {g} vs {ref}"
        assert a == r["a"], f"{label}: accepted {a} vs oracle {r['a']}"
        for l in range(cfg.n_layers):
            st = mv.mk_read_state(l)
            if cfg.is_attention(l):
                P = o.pos
                e = max(rel_l2(st[0][:, :P], o.Kc[l][:, :P]), rel_l2(st[1][:, :P], o.Vc[l][:, :P]))
            else:
                e = rel_l2(st, o.S[l])
            assert e <= STATE_TOL, f"{label}: layer {l} rel-L2 {e:.2e}"
        assert mv.mk_get_position() == o.pos
        mv.close()


def test_errors():
    from hybrid_deltanet_attention_amd import MkError
    torch = torch_cuda()
    cfg = synth.get_config("tiny")
    W = synth.make_weights(cfg, 9)
    out = torch.zeros(8, dtype=torch.int32, device="cuda")
    acc = torch.zeros(1, dtype=torch.int32, device="cuda")
    m0 = new_model(cfg, W)  # created with max_verify_k = 0
    with pytest.raises(MkError) as e:
        m0.mk_verify_k(_dev([1, 2]), 1, out, acc)
    assert e.value.code == -1
    m0.close()
    mv = _verify_model(cfg, W, 3)
    with pytest.raises(MkError) as e:
        mv.mk_verify_k(_dev([1, 2, 3, 4, 5]), 4, out, acc)  # k above max_verify_k
    assert e.value.code == -1
    # a token id outside the vocabulary is reported at the next synchronisation, nothing is written
    _prefill(mv, [3, 4, 5])
    mv.mk_verify_k(_dev([1, cfg.vocab + 3]), 1, out, acc)
    with pytest.raises(MkError) as e:
        mv.mk_sync()
    assert e.value.code == -1
    mv.mk_reset()
    # a context that cannot take k + 1 more positions
    _prefill(mv, synth.make_prompt(cfg.vocab, cfg.max_ctx - 3, 9))
    with pytest.raises(MkError) as e:
        mv.mk_verify_k(_dev([1, 2, 3, 4]), 3, out, acc)
    assert e.value.code == -6
    y, a = _verify(mv, [1, 2, 3])  # exactly fills the context
    assert mv.mk_get_position() == cfg.max_ctx - 3 + a + 1
    mv.close()


def test_0p8b_greedy_and_random_drafts():
    """the full 0.8B shape in the benchmark's launch configuration"""
    cfg = synth.get_config("hybrid_0p8b")
    W = synth.make_weights(cfg, 0)
    prompt = synth.make_prompt(cfg.vocab, 64, 0)
    assert _check_against_decode(cfg, W, prompt, lambda c: c, 5, label="0.8B greedy") == 5
    _check_against_decode(cfg, W, prompt, lambda c: synth.make_drafts(cfg.vocab, len(c), 0), 5, label="0.8B random")

"""Edge cases of the HIP path against the oracle: exact argmax ties, extreme DeltaNet gates, and the
0.8B speculative verify from a handed-off state.

* Ties.  The tied LM head makes logit j the dot product of embedding row j with the final hidden
  vector, so two equal embedding rows give two equal logits.  With every odd row a copy of the even
  row before it, every maximum is a tie, and the greedy choice must be the lower (even) index
  (lowest index among equal maxima, the argmax rule of the decode, prefill and verify kernels and of
  the oracle).  The GPU reduces both rows of a pair through the same arithmetic, so their logits
  must be bitwise equal too.
* Gate extremes.  The decay and write-strength rows scaled by 32 (exact in BF16) push the gate
  logits to about +-10 (tiny) and +-20 (0.8B): alpha = exp(-softplus(a)) spans 1e-9 .. 1 and
  beta = sigmoid(b) spans 0 .. 1, so inside a 64-token prefill chunk the cumulative decay
  underflows FP32 many times over.  The prefill's log-space decays and the decode update must
  still match the oracle to the usual bars.
* Verify at 0.8B.  A 512-token GPU prefill is handed to the oracle (mk_read_state); greedy,
  partly wrong and random drafts are scored by one mk_verify_k launch and by Oracle.verify.
"""
import numpy as np
import pytest

import synth
from oracle import Oracle
from oracle.metrics import rel_l2
from gpu_util import new_model, run_teacher_forced, torch_cuda
from test_gpu_parity import _check_run

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-2
STATE_TOL = 1e-3


def _twin_rows(W):
    """every odd embedding row a copy of the even row before it"""
    W = dict(W)
    E = W["embed"].copy()
    E[1::2] = E[0::2][: E[1::2].shape[0]]
    W["embed"] = E
    return W


def _lowest_argmax(lg):
    m = lg.max()
    return int(np.flatnonzero(lg == m)[0])


def _dev(a):
    torch = torch_cuda()
    return torch.tensor(np.asarray(a, dtype=np.int32), device="cuda")


def test_argmax_ties_decode_prefill_verify():
    from hybrid_deltanet_attention_amd import Model
    torch = torch_cuda()
    cfg = synth.get_config("tiny")
    W = _twin_rows(synth.make_weights(cfg, 12))
    prompt = synth.make_prompt(cfg.vocab, 40, 12)
    o = Oracle(cfg, W)
    fed, ref_logits, ref_last = o.greedy(prompt, 16)
    assert all(t % 2 == 0 for t in fed), "the oracle's greedy choices are the even twins"

    m = new_model(cfg, W)
    pre_l, pre_n, dec_l, dec_n = run_teacher_forced(m, prompt, fed)
    print(f"[ties] prefill choice {pre_n}, decode choices {dec_n}", flush=True)
    for lg, n, what in [(pre_l, pre_n, "prefill")] + [(g, c, f"decode {t}") for t, (g, c) in
                                                      enumerate(zip(dec_l, dec_n))]:
        assert np.array_equal(lg[0::2], lg[1::2]), f"{what}: twin rows must give bitwise-equal logits"
        assert n == _lowest_argmax(lg), f"{what}: choice {n} is not the lowest index of the maximum"
        assert n % 2 == 0, f"{what}: choice {n} is the higher twin"
    assert pre_n == fed[0]
    assert rel_l2(pre_l, ref_last) <= LOGIT_TOL
    assert max(rel_l2(g, r) for g, r in zip(dec_l, ref_logits)) <= LOGIT_TOL
    assert dec_n[:-1] == [int(t) for t in fed[1:]], "decode choices must equal the oracle's"
    m.close()

    # verify: the pending token and five drafts -- the greedy continuation (all accepted), then the
    # same with the second draft replaced by the higher twin of the right token (one accepted)
    mv = Model(cfg, device=0, max_verify_k=5)
    mv.mk_load_weights(W)
    greedy = [int(t) for t in fed[1:6]]
    for drafts, want_a in [(greedy, 5), (greedy[:1] + [greedy[1] + 1] + greedy[2:], 1)]:
        mv.mk_reset()
        nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
        mv.mk_prefill(_dev(prompt), len(prompt), nxt)
        mv.mk_sync()
        assert int(nxt.item()) == fed[0]
        out = torch.full((6,), -7, dtype=torch.int32, device="cuda")
        acc = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        mv.mk_verify_k(_dev([int(fed[0])] + drafts), 5, out, acc)
        mv.mk_sync()
        y, a = [int(v) for v in out.cpu().numpy()], int(acc.item())
        print(f"[ties verify] drafts {drafts} choices {y} accepted {a}", flush=True)
        assert a == want_a, f"accepted {a}, expected {want_a}"
        assert all(v % 2 == 0 for v in y[: a + 1]), "verify chose a higher twin"
        assert y[: a + 1] == [int(t) for t in fed[1: a + 2]]
    mv.close()


def _gate_scaled(cfg, seed, scale=32.0):
    W = synth.make_weights(cfg, seed)
    for l in range(cfg.n_layers):
        if cfg.is_attention(l):
            continue
        for n in ("wa", "wb"):
            name = f"l{l}.dn.{n}"
            W[name] = synth.bf16_round(synth.bf16_bits_to_f32(W[name]) * np.float32(scale))
    return W


def _gate_range(cfg, W, prompt):
    """the oracle's gate logits over the prompt at the first DeltaNet layer (for the log line)"""
    o = Oracle(cfg, W)
    h = o.W.rows("embed", np.asarray(prompt))
    h = h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + cfg.rms_eps)
    a = h @ o.W["l0.dn.wa"].T
    b = h @ o.W["l0.dn.wb"].T
    return float(np.abs(a).max()), float(np.abs(b).max())


def test_gate_extremes_tiny_chunked_prefill_and_decode():
    cfg = synth.get_config("tiny")
    W = _gate_scaled(cfg, 13)
    prompt = synth.make_prompt(cfg.vocab, 200, 13)
    print(f"[gates tiny] max |a| {_gate_range(cfg, W, prompt)[0]:.1f}, max |b| {_gate_range(cfg, W, prompt)[1]:.1f}",
          flush=True)
    _check_run(cfg, W, prompt, 24)


def test_gate_extremes_0p8b_chunked_prefill_and_decode():
    cfg = synth.get_config("hybrid_0p8b", max_ctx=512)
    W = _gate_scaled(cfg, 14)
    prompt = synth.make_prompt(cfg.vocab, 150, 14)
    print(f"[gates 0.8B] max |a| {_gate_range(cfg, W, prompt)[0]:.1f}, max |b| {_gate_range(cfg, W, prompt)[1]:.1f}",
          flush=True)
    _check_run(cfg, W, prompt, 6)


def test_0p8b_verify_against_oracle_from_handed_off_state():
    from hybrid_deltanet_attention_amd import Model
    torch = torch_cuda()
    cfg = synth.get_config("hybrid_0p8b")
    W = synth.make_weights(cfg, 15)
    prompt = synth.make_prompt(cfg.vocab, 512, 15)
    mv = Model(cfg, device=0, max_verify_k=5)
    mv.mk_load_weights(W)
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")

    def gpu_prefill():
        mv.mk_reset()
        mv.mk_prefill(_dev(prompt), len(prompt), nxt)
        mv.mk_sync()
        return int(nxt.item())

    pend = gpu_prefill()
    o = Oracle(cfg, W)
    for l in range(cfg.n_layers):
        st = mv.mk_read_state(l)
        if cfg.is_attention(l):
            o.Kc[l][:] = st[0]
            o.Vc[l][:] = st[1]
        else:
            o.S[l] = st.astype(np.float64)
    o.pos = len(prompt)
    start = o.snapshot()
    cont, t = [], pend
    for _ in range(5):
        t = o.argmax(o.step(t))
        cont.append(t)
    cases = {"greedy": cont, "planted@2": cont[:2] + [(cont[2] + 9) % cfg.vocab] + cont[3:],
             "random": [int(x) for x in synth.make_drafts(cfg.vocab, 5, 15)]}
    for label, drafts in cases.items():
        o.restore(start)
        r = o.verify([pend] + drafts)
        assert gpu_prefill() == pend
        out = torch.full((6,), -7, dtype=torch.int32, device="cuda")
        acc = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        mv.mk_verify_k(_dev([pend] + drafts), 5, out, acc)
        mv.mk_sync()
        y, a = [int(v) for v in out.cpu().numpy()], int(acc.item())
        print(f"[0.8B verify {label}] gpu {y} a={a} oracle {r['y']} a={r['a']}", flush=True)
        for i, (g, ref) in enumerate(zip(y[: a + 1], r["y"][: a + 1])):
            if g != ref:
                lg = r["logits"][i]
                assert abs(lg[g] - lg[ref]) <= 1e-4 * np.abs(lg).max(), f"{label}: choice {i} {g} vs {ref}"
        assert a == r["a"], f"{label}: accepted {a} vs oracle {r['a']}"
        worst = 0.0
        for l in range(cfg.n_layers):
            st = mv.mk_read_state(l)
            if cfg.is_attention(l):
                P = o.pos
                e = max(rel_l2(st[0][:, :P], o.Kc[l][:, :P]), rel_l2(st[1][:, :P], o.Vc[l][:, :P]))
            else:
                e = rel_l2(st, o.S[l])
            worst = max(worst, e)
            assert e <= STATE_TOL, f"{label}: layer {l} rel-L2 {e:.2e}"
        print(f"  worst state/KV rel-L2 {worst:.2e}", flush=True)
        assert mv.mk_get_position() == o.pos
    mv.close()

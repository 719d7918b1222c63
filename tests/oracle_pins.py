"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
closed form, a hand-worked example, brute force, an invariant, or its own
independent second form.  The functions look up oracle routines through their
modules at call time so that ``test_oracle_mutations.py`` can plant a mistake in
the oracle and check that some pin catches it.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle.primitives as prim
import oracle.deltanet as dn
import oracle.attention as att
import oracle.model as om
import oracle.quant as oq
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ------------------------------------------------------------------ primitives
def pin_rmsnorm_closed_form():
    # mean of squares of [1,-2,2,4] is 25/4, so the RMS is 5/2 (eps = 0)
    x = np.array([1.0, -2.0, 2.0, 4.0])
    g = np.array([1.0, 2.0, 3.0, 4.0])
    _close(prim.rmsnorm(x, g, 0.0), [0.4, -1.6, 2.4, 6.4], 1e-15, "rmsnorm")
    # a constant vector c normalises to sign(c) * g up to eps
    _close(prim.rmsnorm(np.full(8, -3.0), np.arange(1.0, 9.0), 1e-6), -np.arange(1.0, 9.0), 1e-6, "rmsnorm const")


def pin_l2norm_closed_form():
    _close(prim.l2norm(np.array([3.0, 4.0]), 0.0), [0.6, 0.8], 1e-15, "l2norm")
    _close(prim.l2norm(np.array([[0.0, 5.0], [-8.0, 6.0]]), 0.0), [[0.0, 1.0], [-0.8, 0.6]], 1e-15, "l2norm rows")


def pin_gate_closed_forms():
    # softplus(0) = ln 2 -> alpha = 1/2 ; sigmoid(0) = 1/2
    a, b = dn.gates(np.array([0.0]), np.array([0.0]))
    _close(a, [0.5], 1e-15, "alpha(0)")
    _close(b, [0.5], 1e-15, "beta(0)")
    # softplus(ln(e-1)) = ln(e) = 1 -> alpha = 1/e ; sigmoid(ln 3) = 3/4
    a, b = dn.gates(np.array([math.log(math.e - 1.0)]), np.array([math.log(3.0)]))
    _close(a, [1.0 / math.e], 1e-15, "alpha(ln(e-1))")
    _close(b, [0.75], 1e-15, "beta(ln 3)")
    # limits: alpha -> 1 and beta -> 0 as the logits go to -inf; alpha -> 0, beta -> 1 at +inf
    a, b = dn.gates(np.array([-800.0, 800.0]), np.array([-800.0, 800.0]))
    _close(a, [1.0, 0.0], 1e-300, "alpha limits")
    _close(b, [0.0, 1.0], 1e-300, "beta limits")
    _close(prim.silu(np.array([1.0, 0.0])), [1.0 / (1.0 + math.exp(-1.0)), 0.0], 1e-15, "silu")


def pin_bf16_decode():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x4049], dtype=np.uint16)
    _close(prim.bf16_decode(bits), [1.0, -2.0, 1.0078125, 0.0, 3.140625], 0.0, "bf16 decode")


def pin_rope_pairing_and_sign():
    # head_dim 4, theta 1e4: frequencies 1 and 0.01; element i pairs with i + 2
    cos, sin = prim.rope_angles(4, 10000.0, 1)
    x = np.array([1.0, 2.0, 3.0, 4.0])
    c1, s1, c2, s2 = math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01)
    want = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    _close(prim.rope(x, cos, sin), want, 1e-14, "rope hd=4 pos=1")
    # position 0 is the identity
    cos0, sin0 = prim.rope_angles(8, 10000.0, 0)
    y = np.arange(8.0)
    _close(prim.rope(y, cos0, sin0), y, 0.0, "rope pos 0")


def pin_rope_relativity():
    rng = np.random.default_rng(7)
    hd = 16
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)

    def score(m, n):
        cm, sm = prim.rope_angles(hd, 10000.0, m)
        cn, sn = prim.rope_angles(hd, 10000.0, n)
        return float(prim.rope(q, cm, sm) @ prim.rope(k, cn, sn))

    for m, n, d in [(5, 2, 11), (40, 39, 100), (3, 3, 7)]:
        assert abs(score(m, n) - score(m + d, n + d)) < 1e-11, "rope scores must depend on m - n only"
    cm, sm = prim.rope_angles(hd, 10000.0, 123)
    assert abs(np.linalg.norm(prim.rope(q, cm, sm)) - np.linalg.norm(q)) < 1e-12, "rope preserves norm"


# -------------------------------------------------------------------- deltanet
def pin_deltanet_hand_example():
    with open(os.path.join(GOLDEN, "deltanet_two_step.json")) as f:
        g = json.load(f)
    S = np.array(g["S0"])
    for i, st in enumerate(g["steps"]):
        S, o = dn.delta_step(S, np.array(st["q"]), np.array(st["k"]), np.array(st["v"]),
                             st["alpha"], st["beta"])
        _close(S, st["S"], 1e-14, f"hand step {i} S")
        _close(o, st["o"], 1e-14, f"hand step {i} o")


def pin_deltanet_exact_recall():
    """alpha = beta = 1, S0 = 0, orthonormal keys: the state stores each key->value pair exactly,
    and querying with a stored key returns its value (so q carries no 1/sqrt(dk) scale)."""
    rng = np.random.default_rng(11)
    dk, dv, n = 8, 5, 6
    Kq, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Kq[:, :n].T.copy()
    V = rng.standard_normal((n, dv))
    S = np.zeros((dv, dk))
    for t in range(n):
        S, o = dn.delta_step(S, K[t], K[t], V[t], 1.0, 1.0)
        _close(o, V[t], 1e-12, f"recall readout t={t}")
    for j in range(n):
        _close(S @ K[j], V[j], 1e-12, f"recall of pair {j}")


def pin_deltanet_last_write():
    """beta = 1, unit key, any alpha: right after a write, S_t k_t = v_t."""
    rng = np.random.default_rng(12)
    dk, dv = 6, 4
    S = rng.standard_normal((dv, dk))
    for t in range(5):
        k = prim.l2norm(rng.standard_normal(dk), 0.0)
        v = rng.standard_normal(dv)
        alpha = float(rng.uniform(0.1, 1.0))
        S, _ = dn.delta_step(S, k, k, v, alpha, 1.0)
        _close(S @ k, v, 1e-12, f"last write t={t}")


def pin_deltanet_gate_limits():
    rng = np.random.default_rng(13)
    dk, dv = 5, 3
    S0 = rng.standard_normal((dv, dk))
    k = prim.l2norm(rng.standard_normal(dk), 0.0)
    q = rng.standard_normal(dk)
    v = rng.standard_normal(dv)
    S, _ = dn.delta_step(S0, q, k, v, 0.0, 0.7)
    _close(S, 0.7 * np.outer(v, k), 1e-14, "alpha = 0 forgets everything")
    S, _ = dn.delta_step(S0, q, k, v, 0.3, 0.0)
    _close(S, 0.3 * S0, 1e-14, "beta = 0 only decays")
    S, o = dn.delta_step(S0, q, k, v, 1.0, 0.0)
    _close(S, S0, 0.0, "alpha = 1, beta = 0 keeps S")
    _close(o, S0 @ q, 1e-14, "readout uses the updated S")
    for alpha, beta in [(0.9, 0.4), (0.5, 1.0), (0.2, 0.05)]:
        S, _ = dn.delta_step(S0, q, k, v, alpha, beta)
        lhs = np.linalg.norm(S, 2)
        rhs = alpha * np.linalg.norm(S0, 2) + beta * np.linalg.norm(v)
        assert lhs <= rhs + 1e-12, "spectral-norm bound ||S_t|| <= alpha ||S_t-1|| + beta ||v||"


def _random_sequence(rng, T, dk, dv):
    Q = prim.l2norm(rng.standard_normal((T, dk)), 1e-6)
    K = prim.l2norm(rng.standard_normal((T, dk)), 1e-6)
    V = rng.standard_normal((T, dv))
    alpha, beta = dn.gates(rng.standard_normal(T), rng.standard_normal(T))
    S0 = rng.standard_normal((dv, dk))
    return S0, Q, K, V, alpha, beta


def pin_deltanet_forms_agree():
    """recurrent == explicit product == parallel (one chunk) == chunked, fp64, T <= 16."""
    rng = np.random.default_rng(14)
    for T, dk, dv in [(1, 4, 3), (7, 6, 5), (16, 8, 8)]:
        S0, Q, K, V, alpha, beta = _random_sequence(rng, T, dk, dv)
        O_r, S_r = dn.delta_recurrent(S0, Q, K, V, alpha, beta)
        O_e, S_e = dn.delta_explicit_product(S0, Q, K, V, alpha, beta)
        O_p, S_p = dn.delta_parallel(S0, Q, K, V, alpha, beta)
        _close(O_e, O_r, 1e-11, f"explicit vs recurrent O (T={T})")
        _close(S_e, S_r, 1e-11, f"explicit vs recurrent S (T={T})")
        _close(O_p, O_r, 1e-11, f"parallel vs recurrent O (T={T})")
        _close(S_p, S_r, 1e-11, f"parallel vs recurrent S (T={T})")
        for C in (1, 3, 4, 5):
            O_c, S_c = dn.delta_chunked(S0, Q, K, V, alpha, beta, C)
            _close(O_c, O_r, 1e-11, f"chunk {C} vs recurrent O (T={T})")
            _close(S_c, S_r, 1e-11, f"chunk {C} vs recurrent S (T={T})")


def pin_deltanet_long_decay_stable():
    """alpha ~ 0.5 over 200 tokens: the parallel form stays finite (decays taken in log space)."""
    rng = np.random.default_rng(15)
    S0, Q, K, V, _, beta = _random_sequence(rng, 200, 4, 4)
    alpha = np.full(200, 0.5)
    O_r, S_r = dn.delta_recurrent(S0, Q, K, V, alpha, beta)
    O_c, S_c = dn.delta_chunked(S0, Q, K, V, alpha, beta, 64)
    assert np.all(np.isfinite(O_c)) and np.all(np.isfinite(S_c))
    _close(O_c, O_r, 1e-10, "chunk 64 vs recurrent, strong decay")
    _close(S_c, S_r, 1e-10, "chunk 64 vs recurrent S, strong decay")


# ------------------------------------------------------------------- attention
def pin_attention_closed_forms():
    e = math.e
    q = np.array([[2.0, 0.0, 0.0, 0.0]])                     # 1 head, hd = 4
    Kc = np.array([[[1.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]]])
    Vc = np.array([[[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]]])
    # scores (2*1)/sqrt(4) = 1 and 0 -> weights e/(1+e), 1/(1+e)
    _close(att.attend_one(q, Kc, Vc), [[e / (1 + e), 1 / (1 + e), 0.0, 0.0]], 1e-15, "two-key softmax")
    rng = np.random.default_rng(16)
    v0 = rng.standard_normal((1, 1, 8))
    _close(att.attend_one(rng.standard_normal((3, 8)), rng.standard_normal((1, 1, 8)), v0),
           np.repeat(v0[0], 3, axis=0), 1e-15, "one key -> its value")
    k_same = np.repeat(rng.standard_normal((1, 1, 8)), 5, axis=1)
    V5 = rng.standard_normal((1, 5, 8))
    _close(att.attend_one(rng.standard_normal((2, 8)), k_same, V5),
           np.repeat(V5[0].mean(axis=0, keepdims=True), 2, axis=0), 1e-14, "equal keys -> mean value")


def pin_attention_gqa_grouping():
    """query head i reads kv head i // (nq/nkv); brute-force scalar loops on a small case."""
    rng = np.random.default_rng(17)
    nq, nkv, L, hd = 4, 2, 3, 2
    q = rng.standard_normal((nq, hd))
    Kc = rng.standard_normal((nkv, L, hd))
    Vc = rng.standard_normal((nkv, L, hd))
    got = att.attend_one(q, Kc, Vc)
    for i in range(nq):
        g = i // (nq // nkv)
        s = [sum(q[i, d] * Kc[g, j, d] for d in range(hd)) / math.sqrt(hd) for j in range(L)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = sum(w)
        want = [sum(w[j] / z * Vc[g, j, d] for j in range(L)) for d in range(hd)]
        _close(got[i], want, 1e-14, f"head {i}")


def pin_attention_forms_agree():
    """full masked matrix == one query at a time over a growing cache; future keys are invisible."""
    rng = np.random.default_rng(18)
    T, nq, nkv, hd = 9, 6, 3, 4
    Q = rng.standard_normal((T, nq, hd))
    K = rng.standard_normal((T, nkv, hd))
    V = rng.standard_normal((T, nkv, hd))
    O = att.causal_attention(Q, K, V)
    Kc = np.transpose(K, (1, 0, 2))
    Vc = np.transpose(V, (1, 0, 2))
    for t in range(T):
        _close(O[t], att.attend_one(Q[t], Kc[:, : t + 1], Vc[:, : t + 1]), 1e-14, f"row {t}")
    K2, V2 = K.copy(), V.copy()
    K2[5:] += 3.0
    V2[5:] -= 1.0
    _close(att.causal_attention(Q, K2, V2)[:5], O[:5], 0.0, "causal mask")


# ----------------------------------------------------------------------- model
def _tiny(**kw):
    return synth.get_config("tiny", **kw)


def pin_model_layer_pattern():
    c = synth.get_config("hybrid_0p8b")
    kinds = ["A" if c.is_attention(l) else "D" for l in range(c.n_layers)]
    assert kinds.count("D") == 18 and kinds.count("A") == 6, "18 DeltaNet + 6 attention layers"
    assert "".join(kinds[:8]) == "DDDADDDA"
    t = _tiny()
    assert ["A" if t.is_attention(l) else "D" for l in range(4)] == ["D", "D", "D", "A"]


def pin_model_incremental_equals_recompute(cfg=None, seed=0, gain_noise=0.0, T=12):
    """token-by-token (recurrent DeltaNet + KV cache) == whole sequence (parallel DeltaNet + full
    masked attention): logits at every position, final DeltaNet states, rotated K and V."""
    cfg = cfg or _tiny()
    W = synth.make_weights(cfg, seed, gain_noise=gain_noise)
    toks = synth.make_prompt(cfg.vocab, T, seed)
    o = om.Oracle(cfg, W)
    fwd = o.forward(toks, logits="all")
    step_logits = np.stack([o.step(t) for t in toks])
    _close(step_logits, fwd["logits"], 1e-10, "logits O1 vs O2")
    for l, S in fwd["S"].items():
        _close(o.S[l], S, 1e-10, f"state layer {l}")
    for l, (K, V) in fwd["KV"].items():
        _close(o.Kc[l][:, :T], K, 1e-12, f"K layer {l}")
        _close(o.Vc[l][:, :T], V, 1e-12, f"V layer {l}")


def pin_model_gain_noise():
    pin_model_incremental_equals_recompute(seed=3, gain_noise=0.1, T=8)


def pin_model_mha_special_case():
    pin_model_incremental_equals_recompute(cfg=_tiny(n_kv_heads=4), seed=1, T=6)


def pin_model_causal():
    cfg = _tiny()
    W = synth.make_weights(cfg, 2)
    o = om.Oracle(cfg, W)
    toks = synth.make_prompt(cfg.vocab, 10, 2)
    a = o.forward(toks)["logits"]
    toks2 = toks.copy()
    toks2[6:] = (toks2[6:] + 17) % cfg.vocab
    b = o.forward(toks2)["logits"]
    _close(b[:6], a[:6], 0.0, "earlier logits ignore later tokens")
    assert np.max(np.abs(b[6:] - a[6:])) > 1e-6


def pin_model_continuation():
    """forward(prompt) then step() == forward(prompt + continuation) at the continued positions."""
    cfg = _tiny()
    W = synth.make_weights(cfg, 4)
    toks = synth.make_prompt(cfg.vocab, 11, 4)
    o = om.Oracle(cfg, W)
    full = o.forward(toks, logits="all")
    part = o.forward(toks[:7], logits="last")
    _close(part["logits"], full["logits"][6], 1e-10, "last-only logits")
    o.load_state(part)
    for t in range(7, 11):
        _close(o.step(toks[t]), full["logits"][t], 1e-10, f"continued position {t}")


def _verify_setup(seed, n_prompt, n_greedy):
    cfg = _tiny()
    W = synth.make_weights(cfg, seed)
    prompt = synth.make_prompt(cfg.vocab, n_prompt, seed)
    o = om.Oracle(cfg, W)
    # the greedy continuation, from the whole-sequence form (one forward pass per prefix)
    seq = list(prompt)
    for _ in range(n_greedy):
        seq.append(int(np.argmax(o.forward(seq, logits="last")["logits"])))
    return cfg, W, o, [int(t) for t in prompt], seq[n_prompt:]


def _check_rolled_back(o, kept, what):
    """o's state and cache == the whole-sequence form over the kept tokens"""
    ref = o.forward(kept, logits="last")
    assert o.pos == len(kept), f"{what}: position {o.pos} vs {len(kept)}"
    for l, S in ref["S"].items():
        _close(o.S[l], S, 1e-10, f"{what}: state layer {l}")
    for l, (K, V) in ref["KV"].items():
        _close(o.Kc[l][:, : len(kept)], K, 1e-12, f"{what}: K layer {l}")
        _close(o.Vc[l][:, : len(kept)], V, 1e-12, f"{what}: V layer {l}")


def pin_verify_accepts_greedy_drafts():
    """drafts equal to the greedy continuation are all accepted; the choices are that continuation"""
    cfg, W, o, prompt, cont = _verify_setup(5, 9, 6)
    o.load_state(o.forward(prompt[:-1], logits="last"))
    pending = prompt[-1]
    k = 4
    r = o.verify([pending] + cont[:k])
    assert r["a"] == k, f"accepted {r['a']} of {k} greedy drafts"
    assert r["y"] == cont[: k + 1], "greedy choices"
    _check_rolled_back(o, prompt + cont[:k], "all accepted")


def pin_verify_planted_mismatch():
    """a draft that differs from the greedy choice at index j stops acceptance at a = j and
    discards the state of every later position"""
    cfg, W, o, prompt, cont = _verify_setup(6, 8, 5)
    for j in (0, 2):
        o.load_state(o.forward(prompt[:-1], logits="last"))
        drafts = list(cont[:4])
        drafts[j] = (drafts[j] + 1) % cfg.vocab
        r = o.verify([prompt[-1]] + drafts)
        assert r["a"] == j, f"planted mismatch at {j}: accepted {r['a']}"
        assert r["y"][: j + 1] == cont[: j + 1]
        _check_rolled_back(o, prompt + cont[:j], f"mismatch at {j}")


def pin_verify_k0_is_one_step():
    cfg, W, o, prompt, cont = _verify_setup(7, 6, 1)
    o.load_state(o.forward(prompt[:-1], logits="last"))
    r = o.verify([prompt[-1]])
    assert r["a"] == 0 and r["y"] == cont[:1]
    _check_rolled_back(o, prompt, "k = 0")


def _micro_model(name):
    """One of the hand-worked one-layer models of tests/golden/micro_models.json: its config and
    its weights as BF16 bit patterns (every stored value must be exact in BF16)."""
    with open(os.path.join(GOLDEN, "micro_models.json")) as f:
        g = json.load(f)
    m = g["models"][name]
    cfg = synth.get_config("tiny").with_(name="micro", **g["config_common"], **m["config"])
    W = {}
    for wname, shape, _ in synth.tensor_manifest(cfg):
        vals = np.asarray(m["weights"][wname], dtype=np.float32)
        assert vals.shape == tuple(shape), f"{wname}: {vals.shape} vs manifest {shape}"
        W[wname] = synth.bf16_round(vals)
        assert np.array_equal(prim.bf16_decode(W[wname]), vals.astype(np.float64)), f"{wname} not BF16-exact"
    return cfg, W, g["tokens"], m


def pin_micro_model_deltanet_golden():
    """A one-layer DeltaNet model run by hand (tests/golden/micro_models.json): logits and state
    after each of two tokens, through both the token-by-token and the whole-sequence forms, and
    the FFN and head stages on the hand values."""
    cfg, W, toks, m = _micro_model("deltanet")
    o = om.Oracle(cfg, W)
    for t, st in zip(toks, m["steps"]):
        _close(o.step(t), st["logits"], 1e-12, f"micro deltanet logits (token {t})")
        _close(o.S[0][0], st["S"], 1e-12, f"micro deltanet state (token {t})")
        _close(o._ffn(0, np.array(st["x1"])), st["x2"], 1e-12, f"micro deltanet FFN (token {t})")
        _close(o._head(np.array(st["x2"])), st["logits"], 1e-12, f"micro deltanet head (token {t})")
    fwd = o.forward(toks)
    _close(fwd["logits"], [st["logits"] for st in m["steps"]], 1e-12, "micro deltanet forward logits")
    _close(fwd["S"][0][0], m["steps"][-1]["S"], 1e-12, "micro deltanet forward state")


def pin_micro_model_attention_golden():
    """A one-layer attention model run by hand: logits after each of two tokens (so RoPE turns the
    second query and key), the rotated key cache and the values, through both forms."""
    cfg, W, toks, m = _micro_model("attention")
    o = om.Oracle(cfg, W)
    for t, st in zip(toks, m["steps"]):
        _close(o.step(t), st["logits"], 1e-12, f"micro attention logits (token {t})")
        _close(o._ffn(0, np.array(st["x1"])), st["x2"], 1e-12, f"micro attention FFN (token {t})")
    _close(o.Kc[0][0, :2], m["kv_cache"]["K"], 1e-12, "micro attention K cache")
    _close(o.Vc[0][0, :2], m["kv_cache"]["V"], 1e-12, "micro attention V cache")
    fwd = o.forward(toks)
    _close(fwd["logits"], [st["logits"] for st in m["steps"]], 1e-12, "micro attention forward logits")
    _close(fwd["KV"][0][0][0], m["kv_cache"]["K"], 1e-12, "micro attention forward K")


def pin_model_without_residual_writes():
    """With every mixer output projection and every FFN down projection zero, no layer writes to
    the residual stream, so the logits are the tied head on the normalised embedding alone:
    logits = E (E[tok] / rms(E[tok]) * g_final), whatever the other weights.  Distinct random
    gains make the final gain distinguishable from the layers' ones."""
    cfg = _tiny()
    W = synth.make_weights(cfg, 8, gain_noise=0.3)
    for name in W:
        if name.endswith(".wo") or name.endswith(".ffn.wd"):
            W[name] = np.zeros_like(W[name])
    E = prim.bf16_decode(W["embed"])
    gf = prim.bf16_decode(W["final_norm"])
    toks = synth.make_prompt(cfg.vocab, 5, 8)
    o = om.Oracle(cfg, W)
    fwd = o.forward(toks)
    for i, t in enumerate(toks):
        x = E[t]
        want = E @ (x / math.sqrt(float(np.mean(x * x)) + cfg.rms_eps) * gf)
        _close(o.step(t), want, 1e-12, f"head on the embedding (token {t})")
        _close(fwd["logits"][i], want, 1e-12, f"forward head on the embedding (position {i})")


def pin_ffn_linear_in_up_projection():
    """SwiGLU multiplies silu(W_g h) by the linear W_u h, so the FFN's residual contribution is
    linear in W_u (doubling W_u doubles it) and vanishes when W_u = 0, but not when W_g is merely
    scaled (silu is not linear)."""
    cfg = _tiny()
    W = synth.make_weights(cfg, 9)
    x = np.random.default_rng(19).standard_normal(cfg.hidden)
    base = om.Oracle(cfg, W)._ffn(0, x) - x
    W2 = dict(W)
    W2["l0.ffn.wu"] = synth.bf16_round(prim.bf16_decode(W["l0.ffn.wu"]).astype(np.float32) * 2)
    _close(om.Oracle(cfg, W2)._ffn(0, x) - x, 2 * base, 1e-12, "FFN linear in W_u")
    W3 = dict(W)
    W3["l0.ffn.wu"] = np.zeros_like(W["l0.ffn.wu"])
    _close(om.Oracle(cfg, W3)._ffn(0, x) - x, np.zeros_like(x), 0.0, "W_u = 0 makes the FFN inert")
    W4 = dict(W)
    W4["l0.ffn.wg"] = synth.bf16_round(prim.bf16_decode(W["l0.ffn.wg"]).astype(np.float32) * 2)
    assert np.max(np.abs(om.Oracle(cfg, W4)._ffn(0, x) - x - 2 * base)) > 1e-6 * np.max(np.abs(base)), \
        "the gate enters through silu, not linearly"


def pin_kv_f16_rounding():
    """binary16 keeps 10 fraction bits: 1 + 2^-11 lies halfway between 1 and 1 + 2^-10 and goes to
    the even neighbour 1; 1 + 3 * 2^-11 lies halfway between 1 + 2^-10 and 1 + 2^-9 and goes to
    1 + 2^-9; 65504 is the largest finite value; 2^-24 is the smallest subnormal and 2^-26 rounds
    to 0."""
    x = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65504.0, -3.0, 2.0 ** -24, 2.0 ** -26])
    _close(att.kv_round(x, "f16"), [1.0, 1 + 2.0 ** -9, 65504.0, -3.0, 2.0 ** -24, 0.0], 0.0, "f16 cache rounding")
    _close(att.kv_round(x, "f32"), x, 0.0, "f32 cache keeps the values")


def pin_kv_q8_hand_example():
    """int8 cache rows: blocks of 32 share s = max|x| / 127 and store rint(x / s), ties to even.
    Block 0 has max 127, so s = 1 and the codes are the values rounded (0.5 -> 0, 1.5 -> 2,
    2.5 -> 2, -63.5 -> -64); block 1 is zero; block 2 is block 0 times 2^-7 (same codes, s = 2^-7);
    block 3 has a single nonzero value -4 (s = 4 / 127, code -127)."""
    row = np.zeros(128)
    row[:6] = [127.0, -63.5, 0.5, 1.5, 2.5, -0.5]
    row[64:70] = row[:6] * 2.0 ** -7
    row[100] = -4.0
    want = np.zeros(128)
    want[:6] = [127.0, -64.0, 0.0, 2.0, 2.0, -0.0]
    want[64:70] = want[:6] * 2.0 ** -7
    want[100] = -4.0
    got = att.kv_round(row, "q8")
    _close(got, want, 1e-6, "q8 hand example")
    rng = np.random.default_rng(23)
    x = rng.standard_normal((5, 64)) * np.array([1.0, 1e-3, 30.0, 1.0, 7.0])[:, None]
    y = att.kv_round(x, "q8")
    s = np.abs(x.reshape(5, 2, 32)).max(-1) / 127
    assert np.all(np.abs(y - x).reshape(5, 2, 32) <= s[..., None] * (0.5 + 1e-6)), "q8 error above half a step"


def pin_model_kv_cache_types():
    """with an f16 or q8 cache, token-by-token decode still equals the whole-sequence form (both
    round keys and values as they enter the cache), the cache holds representable values only,
    and the logits move away from the f32 cache's by a small amount"""
    cfg = _tiny()
    W = synth.make_weights(cfg, 24)
    toks = synth.make_prompt(cfg.vocab, 10, 24)
    base = om.Oracle(cfg, W).forward(toks)["logits"]
    for kv in ("f16", "q8"):
        o = om.Oracle(cfg, W, kv=kv)
        fwd = o.forward(toks, logits="all")
        step_logits = np.stack([o.step(t) for t in toks])
        _close(step_logits, fwd["logits"], 1e-10, f"{kv}: logits O1 vs O2")
        for l, (K, V) in fwd["KV"].items():
            _close(o.Kc[l][:, :10], K, 1e-12, f"{kv}: K layer {l}")
            _close(o.Vc[l][:, :10], V, 1e-12, f"{kv}: V layer {l}")
            if kv == "f16":
                assert np.array_equal(K, K.astype(np.float16).astype(np.float64)), "f16 cache holds binary16 values"
            else:
                b = K.reshape(*K.shape[:-1], -1, 32)
                sc = np.abs(b).max(-1, keepdims=True) / 127
                q = np.where(sc > 0, b / np.where(sc > 0, sc, 1), 0)
                assert np.max(np.abs(q - np.rint(q))) < 1e-4, "q8 cache holds code * scale"
        d = float(np.max(np.abs(fwd["logits"] - base)))
        assert 0.0 < d < 1e-2 * float(np.max(np.abs(base))), f"{kv}: cache rounding moves logits by {d:.2e}"


def pin_argmax_lowest_index():
    lg = np.array([0.1, 0.7, 0.3, 0.7, -1.0])
    assert om.Oracle.argmax(lg) == 1


def pin_fp32_vs_fp64_gap():
    """The oracle's own rounding is far below the GPU tolerances (logits 1e-2, state 1e-3)."""
    import oracle.metrics as mt
    cfg = _tiny()
    W = synth.make_weights(cfg, 0)
    toks = synth.make_prompt(cfg.vocab, 16, 0)
    o64 = om.Oracle(cfg, W, np.float64)
    o32 = om.Oracle(cfg, W, np.float32)
    l64 = np.stack([o64.step(t) for t in toks])
    l32 = np.stack([o32.step(t) for t in toks])
    assert mt.rel_l2(l32, l64) < 1e-5
    for l in o64.S:
        assert mt.rel_l2(o32.S[l], o64.S[l]) < 1e-5



# ------------------------------------------------------------ 4-bit weights
def pin_q4g32_hand_example():
    """A hand-built byte image decodes to the values its codes and block parameters define."""
    with open(os.path.join(GOLDEN, "q4g32_hand.json")) as f:
        g = json.load(f)
    buf = np.frombuffer(bytes.fromhex(g["codes_hex"] + g["params_hex"]), dtype=np.uint8)
    W = oq.q4g32_dequant(buf, g["rows"], g["cols"])
    j = np.arange(32)
    want0 = np.concatenate([0.5 * (j % 16) - 2.0, 0.25 * (j % 16) + 1.0])
    want1 = np.concatenate([2.0 * (15 - j % 16) - 16.0, np.full(32, 0.5)])
    _close(W, np.stack([want0, want1]), 0.0, "q4g32 hand example")
    # single rows through the row path
    _close(oq.q4g32_dequant_rows(buf, 2, 64, np.array([1])), want1[None], 0.0, "q4g32 row 1")


def pin_q4g32_quantizer_roundtrip():
    """The library's host quantizer against the oracle's decoder: every weight comes back within
    half a step (plus the FP16 rounding of d and m), constant groups come back exactly, and the
    group extremes map to codes 0 and 15."""
    from hybrid_deltanet_attention_amd.quant import quantize_q4g32
    rng = np.random.default_rng(5)
    R, K = 6, 128
    w = (rng.standard_normal((R, K)) * 0.02).astype(np.float32)
    w[2, 32:64] = np.float32(0.375)  # a constant group: d = 0, every weight equals m
    buf = quantize_q4g32(w)
    W = oq.q4g32_dequant(buf, R, K)
    g = w.reshape(R, K // 32, 32).astype(np.float64)
    d = (g.max(-1) - g.min(-1)) / 15.0
    bound = 0.5 * d + 16 * d * 2.0 ** -11 + np.abs(g.min(-1)) * 2.0 ** -11
    err = np.abs(W.reshape(R, K // 32, 32) - g).max(-1)
    assert np.all(err <= bound + 1e-12), f"q4g32 round trip error {err.max():.3e} over its bound"
    _close(W[2, 32:64], np.full(32, 0.375), 0.0, "constant group")
    words, _ = oq.q4g32_split(buf, R, K)
    q = oq.q4g32_codes(words).reshape(R, K // 32, 32)
    live = np.ones((R, K // 32), bool)
    live[2, 1] = False
    assert np.all(q.max(-1)[live] == 15) and np.all(q.min(-1)[live] == 0), "group extremes must map to 15 and 0"
    assert np.all(q[2, 1] == 0), "a constant group has code 0 throughout"


def pin_q4g32_model_equals_bf16_model():
    """A model whose 4-bit weights decode to BF16-exact values gives the same logits as the model
    built from those BF16 values (the oracle's lazy decode, row lookup and blocked LM head)."""
    from hybrid_deltanet_attention_amd.quant import pack_q4g32
    cfg = synth.get_config("tiny").with_(n_layers=2, attn_slot=1, period=2, vocab=512, max_ctx=16)
    rng = np.random.default_rng(9)
    q4, bf = {}, {}
    for name, shape, kind in synth.tensor_manifest(cfg):
        if kind == "gain":
            bf[name] = q4[name] = synth.bf16_round(np.ones(shape, np.float32))
            continue
        R, K = shape
        q = rng.integers(0, 16, size=(R, K))
        d = np.where(rng.random((R, K // 32)) < 0.5, 2.0 ** -8, 2.0 ** -7)
        m = -8.0 * d
        q4[name] = pack_q4g32(q, d.astype(np.float16), m.astype(np.float16))
        vals = (q.reshape(R, K // 32, 32) - 8.0) * d[..., None]
        bf[name] = synth.bf16_round(vals.reshape(R, K).astype(np.float32))
    a = om.Oracle(cfg, q4)
    a.W.cache_left = 0  # decode on every use
    b = om.Oracle(cfg, bf)
    toks = [3, 17, 400]
    fa, fb = a.forward(toks), b.forward(toks)
    _close(fa["logits"], fb["logits"], 0.0, "q4 vs bf16 forward logits")
    _close(a.W.lin("embed", fa["logits"][:, :cfg.hidden], block=100),
           fa["logits"][:, :cfg.hidden] @ b.W["embed"].T, 1e-12, "blocked LM head")
    a.load_state(fa)
    b.load_state(fb)
    _close(a.step(5), b.step(5), 0.0, "q4 vs bf16 step logits")

ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]

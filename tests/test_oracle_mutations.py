"""Plant a plausible mistake in the oracle (on the CPU) and check that some pin catches it.

Each mutation is a wrong variant of one oracle routine: a dropped term, a wrong
sign, a swapped operand or index.  A pin set that passes on a mutant would not
be able to tell that mistake from the real method.
"""
import numpy as np
import pytest

import oracle.primitives as prim
import oracle.deltanet as dn
import oracle.attention as att
import oracle.model as om
import oracle.quant as oq
from oracle_pins import ALL_PINS


def _step_no_alpha(S, q, k, v, alpha, beta):
    return _REAL_STEP(S, q, k, v, np.ones_like(np.asarray(alpha, dtype=float)), beta)


def _step_transposed(S, q, k, v, alpha, beta):
    St, _ = _REAL_STEP(np.swapaxes(S, -1, -2), q, k, v, alpha, beta)
    St = np.swapaxes(St, -1, -2)
    return St, (St @ q[..., :, None])[..., 0]


def _step_read_before_update(S, q, k, v, alpha, beta):
    S_new, _ = _REAL_STEP(S, q, k, v, alpha, beta)
    return S_new, (S @ q[..., :, None])[..., 0]


def _step_q_scaled(S, q, k, v, alpha, beta):
    return _REAL_STEP(S, q / np.sqrt(q.shape[-1]), k, v, alpha, beta)


def _gates_beta_swapped(a, b):
    return np.exp(-prim.softplus(a)), prim.sigmoid(-b)


def _gates_alpha_no_exp(a, b):
    return 1.0 / (1.0 + prim.softplus(a)), prim.sigmoid(b)


def _rope_interleaved(x, cos, sin):
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * cos - x2 * sin
    out[..., 1::2] = x2 * cos + x1 * sin
    return out


def _rope_sign(x, cos, sin):
    return _REAL_ROPE(x, cos, -sin)


def _rms_no_gain(x, g, eps):
    return _REAL_RMS(x, np.ones_like(g), eps)


def _rms_no_mean(x, g, eps):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * g


def _attend_no_scale(q, Kc, Vc):
    return _REAL_ATTEND(q * np.sqrt(q.shape[-1]), Kc, Vc)


def _attend_wrong_group(q, Kc, Vc):
    # head i -> kv head i % nkv (interleaved) instead of contiguous groups
    nq, hd = q.shape
    nkv = Kc.shape[0]
    o = np.empty_like(q)
    for i in range(nq):
        s = Kc[i % nkv] @ q[i] / np.sqrt(hd)
        p = prim.softmax(s)
        o[i] = p @ Vc[i % nkv]
    return o


def _parallel_no_s0_decay(S0, Q, K, V, alpha, beta):
    O, S_T = _REAL_PAR(S0, Q, K, V, alpha, beta)
    g = np.cumsum(np.log(alpha))
    return O, S_T - np.exp(g[-1]) * S0 + S0


def _verify_variant(keep_extra=0, shift=0, rollback=True):
    def verify(self, tokens):
        tokens = [int(t) for t in tokens]
        start = self.snapshot()
        logits = np.stack([self.step(t) for t in tokens])
        y = [self.argmax(lg) for lg in logits]
        a = 0
        while a + shift < len(tokens) - 1 and tokens[a + 1] == y[a + shift]:
            a += 1
        if rollback:
            self.restore(start)
            for t in tokens[: max(0, min(len(tokens), a + 1 + keep_extra))]:
                self.step(t)
        return {"y": y, "a": a, "logits": logits}
    return verify


def _q4_codes_halves_swapped(words):
    words = np.asarray(words, dtype=np.uint32)
    return _REAL_Q4_CODES((words >> np.uint32(16)) | (words << np.uint32(16)))


def _q4_codes_nibbles_in_order(words):
    # columns taken as the 8 nibbles in bit order (no even / odd split across the half-words)
    words = np.asarray(words, dtype=np.uint32)
    q = np.stack([(words >> np.uint32(4 * j)) & np.uint32(0xF) for j in range(8)], axis=-1).astype(np.uint8)
    return q.reshape(words.shape[:-1] + (words.shape[-1] * 8,))


def _q4_split_params_swapped(buf, R, K):
    words, params = _REAL_Q4_SPLIT(buf, R, K)
    return words, params[..., ::-1]


def _ffn_silu_on_up(self, l, x):
    c = self.cfg
    h = prim.rmsnorm(x, self.W[f"l{l}.norm2"], c.rms_eps)
    gte = h @ self.W[f"l{l}.ffn.wg"].T
    up = h @ self.W[f"l{l}.ffn.wu"].T
    return x + (gte * prim.silu(up)) @ self.W[f"l{l}.ffn.wd"].T


def _head_no_final_norm(self, x):
    return self.W.lin("embed", x)


def _head_layer_gain(self, x):
    last = self.cfg.n_layers - 1
    return self.W.lin("embed", prim.rmsnorm(x, self.W[f"l{last}.norm2"], self.cfg.rms_eps))


def _dn_project_variant(swap_gates=False, swap_qk=False):
    def project(self, l, h):
        c = self.cfg
        H, dk, dv = c.dn_heads, c.dn_dk, c.dn_dv
        qkv = h @ self.W[f"l{l}.dn.wqkv"].T
        q = qkv[..., : H * dk].reshape(*h.shape[:-1], H, dk)
        k = qkv[..., H * dk: 2 * H * dk].reshape(*h.shape[:-1], H, dk)
        v = qkv[..., 2 * H * dk:].reshape(*h.shape[:-1], H, dv)
        if swap_qk:
            q, k = k, q
        a = h @ self.W[f"l{l}.dn.w{'b' if swap_gates else 'a'}"].T
        b = h @ self.W[f"l{l}.dn.w{'a' if swap_gates else 'b'}"].T
        alpha, beta = dn.gates(a, b)
        return prim.l2norm(q, c.l2_eps), prim.l2norm(k, c.l2_eps), v, alpha, beta
    return project


def _attn_project_variant(rope_v=False, swap_kv=False, q_unrotated=False):
    def project(self, l, h, positions):
        c = self.cfg
        q = (h @ self.W[f"l{l}.attn.wq"].T).reshape(*h.shape[:-1], c.n_q_heads, c.head_dim)
        k = (h @ self.W[f"l{l}.attn.wk"].T).reshape(*h.shape[:-1], c.n_kv_heads, c.head_dim)
        v = (h @ self.W[f"l{l}.attn.wv"].T).reshape(*h.shape[:-1], c.n_kv_heads, c.head_dim)
        if swap_kv:
            k, v = v, k
        cos, sin = prim.rope_angles(c.head_dim, c.rope_theta, positions, self.dtype)
        cos, sin = cos[..., None, :], sin[..., None, :]
        qr = q if q_unrotated else prim.rope(q, cos, sin)
        vr = prim.rope(v, cos, sin) if rope_v else v
        return qr, prim.rope(k, cos, sin), vr
    return project


def _kv_round_variant(mode):
    def kv_round(x, kv):
        x = np.asarray(x)
        if kv == "f16" and mode == "f16_truncated":
            b = x.astype(np.float32).astype(np.float16)
            up = np.abs(b.astype(np.float32)) > np.abs(x.astype(np.float32))
            b = np.where(up, np.nextafter(b, np.float16(0)), b)
            return b.astype(x.dtype)
        if kv == "q8" and mode in ("q8_floor", "q8_row_scale"):
            x32 = x.astype(np.float32)
            if mode == "q8_row_scale":
                s = np.max(np.abs(x32), axis=-1, keepdims=True) / np.float32(127)
                return (np.rint(x32 / np.where(s > 0, s, 1)) * s).astype(x.dtype)
            b = x32.reshape(*x.shape[:-1], -1, 32)
            s = np.max(np.abs(b), axis=-1, keepdims=True) / np.float32(127)
            return (np.floor(b / np.where(s > 0, s, 1)) * s).reshape(x.shape).astype(x.dtype)
        return _REAL_KV_ROUND(x, kv)
    return kv_round


_REAL_Q4_CODES = oq.q4g32_codes
_REAL_Q4_SPLIT = oq.q4g32_split
_REAL_STEP = dn.delta_step
_REAL_ROPE = prim.rope
_REAL_RMS = prim.rmsnorm
_REAL_ATTEND = att.attend_one
_REAL_PAR = dn.delta_parallel
_REAL_KV_ROUND = att.kv_round

# (label, [(module, attribute), ...], replacement)
MUTANTS = [
    ("deltanet: alpha dropped", [(dn, "delta_step"), (om, "delta_step")], _step_no_alpha),
    ("deltanet: S transposed", [(dn, "delta_step"), (om, "delta_step")], _step_transposed),
    ("deltanet: read before update", [(dn, "delta_step"), (om, "delta_step")], _step_read_before_update),
    ("deltanet: q scaled by 1/sqrt(dk)", [(dn, "delta_step"), (om, "delta_step")], _step_q_scaled),
    ("gates: beta sign flipped", [(dn, "gates"), (om, "gates")], _gates_beta_swapped),
    ("gates: alpha without exp", [(dn, "gates"), (om, "gates")], _gates_alpha_no_exp),
    ("rope: interleaved pairs", [(prim, "rope"), (om, "rope")], _rope_interleaved),
    ("rope: sine sign", [(prim, "rope"), (om, "rope")], _rope_sign),
    ("rmsnorm: gain dropped", [(prim, "rmsnorm"), (om, "rmsnorm")], _rms_no_gain),
    ("rmsnorm: sum instead of mean", [(prim, "rmsnorm"), (om, "rmsnorm")], _rms_no_mean),
    ("attention: no 1/sqrt(hd)", [(att, "attend_one"), (om, "attend_one")], _attend_no_scale),
    ("attention: interleaved GQA groups", [(att, "attend_one"), (om, "attend_one")], _attend_wrong_group),
    ("parallel form: S0 not decayed", [(dn, "delta_parallel"), (om, "delta_parallel")], _parallel_no_s0_decay),
    ("verify: no rollback", [(om.Oracle, "verify")], _verify_variant(rollback=False)),
    ("verify: rollback keeps the accepted drafts only", [(om.Oracle, "verify")], _verify_variant(keep_extra=-1)),
    ("verify: rollback keeps one token too many", [(om.Oracle, "verify")], _verify_variant(keep_extra=1)),
    ("verify: draft compared with the next choice", [(om.Oracle, "verify")], _verify_variant(shift=1)),
    ("ffn: silu on up instead of gate", [(om.Oracle, "_ffn")], _ffn_silu_on_up),
    ("head: final RMSNorm dropped", [(om.Oracle, "_head")], _head_no_final_norm),
    ("head: a layer gain in place of the final gain", [(om.Oracle, "_head")], _head_layer_gain),
    ("deltanet: alpha and beta from swapped wa/wb rows", [(om.Oracle, "_dn_project")],
     _dn_project_variant(swap_gates=True)),
    ("deltanet: q and k slices of wqkv swapped", [(om.Oracle, "_dn_project")], _dn_project_variant(swap_qk=True)),
    ("attention: RoPE applied to v", [(om.Oracle, "_attn_project")], _attn_project_variant(rope_v=True)),
    ("attention: k and v swapped", [(om.Oracle, "_attn_project")], _attn_project_variant(swap_kv=True)),
    ("attention: q left unrotated", [(om.Oracle, "_attn_project")], _attn_project_variant(q_unrotated=True)),
    ("kv cache: f16 truncated", [(att, "kv_round"), (om, "kv_round")], _kv_round_variant("f16_truncated")),
    ("kv cache: q8 codes floored", [(att, "kv_round"), (om, "kv_round")], _kv_round_variant("q8_floor")),
    ("kv cache: q8 one scale per row", [(att, "kv_round"), (om, "kv_round")], _kv_round_variant("q8_row_scale")),
    ("q4: code half-words swapped", [(oq, "q4g32_codes")], _q4_codes_halves_swapped),
    ("q4: nibbles read in bit order", [(oq, "q4g32_codes")], _q4_codes_nibbles_in_order),
    ("q4: scale and offset swapped", [(oq, "q4g32_split")], _q4_split_params_swapped),
]


@pytest.mark.parametrize("label,targets,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_some_pin_catches(label, targets, repl, monkeypatch):
    for mod, attr in targets:
        monkeypatch.setattr(mod, attr, repl)
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, np.linalg.LinAlgError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {label}"

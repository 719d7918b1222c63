"""The whole hybrid decoder, token by token (``Oracle.step``) and whole-sequence (``Oracle.forward``).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Layer pattern (luce-megakernel announcement, page 1, layer-pattern paragraph):
18 DeltaNet layers and 6 full-attention layers out of 24, placed here as a
repeating 3:1 pattern, layer l being attention when l % period == attn_slot.
Each layer is pre-norm residual:

    x += Mixer(RMSNorm(x; g1))         Mixer = gated DeltaNet or GQA attention
    x += W_d (silu(W_g h) * (W_u h)),  h = RMSNorm(x; g2)

followed after the last layer by ``logits = E . RMSNorm(x; g_f)`` with the input
embedding E reused as the LM head, and greedy argmax (lowest index on ties).

The two entry points share only the per-token primitives; ``step`` carries a
recurrent DeltaNet state and a KV cache, ``forward`` uses the parallel DeltaNet
form and the full causal score matrix, so they check each other.
"""
from __future__ import annotations

import numpy as np

from .primitives import bf16_decode, rmsnorm, l2norm, silu, rope_angles, rope
from .deltanet import gates, delta_step, delta_parallel
from .attention import attend_one, causal_attention, kv_round, KV_DTYPES
from .quant import q4g32_dequant, q4g32_dequant_rows


def matrix_shape(cfg, name: str) -> tuple:
    """Logical [rows, cols] of a weight matrix by name (rows = outputs, cols = inputs)."""
    D = cfg.hidden
    if name == "embed":
        return (cfg.vocab, D)
    part = name.split(".", 1)[1]
    H, dk, dv, hd = cfg.dn_heads, cfg.dn_dk, cfg.dn_dv, cfg.head_dim
    shapes = {"dn.wqkv": (2 * H * dk + H * dv, D), "dn.wa": (H, D), "dn.wb": (H, D), "dn.wo": (D, H * dv),
              "attn.wq": (cfg.n_q_heads * hd, D), "attn.wk": (cfg.n_kv_heads * hd, D),
              "attn.wv": (cfg.n_kv_heads * hd, D), "attn.wo": (D, cfg.n_q_heads * hd),
              "ffn.wg": (cfg.ffn, D), "ffn.wu": (cfg.ffn, D), "ffn.wd": (D, cfg.ffn)}
    return shapes[part]


class Weights:
    """Weight values by name.  BF16 tensors (uint16 bit patterns) are decoded once; 4-bit Q4G32
    matrices (uint8 buffers) are decoded when used, and kept only while the decoded total stays
    under `cache_bytes` (the 27B-scale matrices would not fit otherwise)."""

    def __init__(self, cfg, weight_bits: dict, dtype, cache_bytes: int = 1 << 31):
        self.cfg = cfg
        self.dtype = dtype
        self.dec = {}
        self.q4 = {}
        self.cache_left = cache_bytes
        for name, bits in weight_bits.items():
            if np.asarray(bits).dtype == np.uint8:
                self.q4[name] = (bits, matrix_shape(cfg, name))
            else:
                self.dec[name] = bf16_decode(bits, dtype)

    def __getitem__(self, name):
        if name in self.dec:
            return self.dec[name]
        buf, (R, K) = self.q4[name]
        w = q4g32_dequant(buf, R, K, self.dtype)
        if w.nbytes <= self.cache_left:
            self.cache_left -= w.nbytes
            self.dec[name] = w
        return w

    def rows(self, name, idx):
        """Selected rows of a matrix (the embedding lookup)."""
        if name in self.dec:
            return self.dec[name][idx].copy()
        buf, (R, K) = self.q4[name]
        return q4g32_dequant_rows(buf, R, K, idx, self.dtype)

    def lin(self, name, x, block: int = 16384):
        """x @ W.T; a 4-bit matrix is decoded whole and kept when it fits the cache budget, else
        decoded a block of rows at a time (each output is still one row's dot product)."""
        if name in self.dec or name not in self.q4:
            return x @ self[name].T
        buf, (R, K) = self.q4[name]
        if R * K * np.dtype(self.dtype).itemsize <= self.cache_left:
            return x @ self[name].T
        out = np.empty(x.shape[:-1] + (R,), dtype=np.result_type(x, self.dtype))
        for r0 in range(0, R, block):
            r1 = min(R, r0 + block)
            out[..., r0:r1] = x @ q4g32_dequant_rows(buf, R, K, slice(r0, r1), self.dtype).T
        return out


class Oracle:
    """kv: the KV cache's storage type ("f32", "f16" or "q8", see ``attention.kv_round``); keys and
    values are rounded to it when they enter the cache, so attention, including the current
    position's own key and value, always sees the stored values."""

    def __init__(self, cfg, weight_bits: dict, dtype=np.float64, kv: str = "f32"):
        if kv not in KV_DTYPES:
            raise ValueError(f"unknown KV cache type {kv!r}")
        self.cfg = cfg
        self.dtype = dtype
        self.kv = kv
        self.W = Weights(cfg, weight_bits, dtype)
        self.reset()

    # ---------------------------------------------------------------- state
    def reset(self):
        c = self.cfg
        self.pos = 0
        self.S = {}
        self.Kc = {}
        self.Vc = {}
        for l in range(c.n_layers):
            if c.is_attention(l):
                self.Kc[l] = np.zeros((c.n_kv_heads, c.max_ctx, c.head_dim), self.dtype)
                self.Vc[l] = np.zeros((c.n_kv_heads, c.max_ctx, c.head_dim), self.dtype)
            else:
                self.S[l] = np.zeros((c.dn_heads, c.dn_dv, c.dn_dk), self.dtype)

    def load_state(self, fwd: dict):
        """Continue token by token from the end of a ``forward`` result."""
        self.reset()
        T = fwd["n_tokens"]
        for l, S in fwd["S"].items():
            self.S[l] = np.array(S, copy=True)
        for l, (K, V) in fwd["KV"].items():
            self.Kc[l][:, :T] = K
            self.Vc[l][:, :T] = V
        self.pos = T

    # ------------------------------------------------------------ per layer
    def _dn_project(self, l, h):
        c = self.cfg
        H, dk, dv = c.dn_heads, c.dn_dk, c.dn_dv
        qkv = h @ self.W[f"l{l}.dn.wqkv"].T
        q = qkv[..., : H * dk].reshape(*h.shape[:-1], H, dk)
        k = qkv[..., H * dk: 2 * H * dk].reshape(*h.shape[:-1], H, dk)
        v = qkv[..., 2 * H * dk:].reshape(*h.shape[:-1], H, dv)
        a = h @ self.W[f"l{l}.dn.wa"].T
        b = h @ self.W[f"l{l}.dn.wb"].T
        alpha, beta = gates(a, b)
        return l2norm(q, c.l2_eps), l2norm(k, c.l2_eps), v, alpha, beta

    def _attn_project(self, l, h, positions):
        c = self.cfg
        q = (h @ self.W[f"l{l}.attn.wq"].T).reshape(*h.shape[:-1], c.n_q_heads, c.head_dim)
        k = (h @ self.W[f"l{l}.attn.wk"].T).reshape(*h.shape[:-1], c.n_kv_heads, c.head_dim)
        v = (h @ self.W[f"l{l}.attn.wv"].T).reshape(*h.shape[:-1], c.n_kv_heads, c.head_dim)
        cos, sin = rope_angles(c.head_dim, c.rope_theta, positions, self.dtype)
        cos = cos[..., None, :]
        sin = sin[..., None, :]
        return rope(q, cos, sin), rope(k, cos, sin), v

    def _ffn(self, l, x):
        c = self.cfg
        h = rmsnorm(x, self.W[f"l{l}.norm2"], c.rms_eps)
        gte = h @ self.W[f"l{l}.ffn.wg"].T
        up = h @ self.W[f"l{l}.ffn.wu"].T
        return x + (silu(gte) * up) @ self.W[f"l{l}.ffn.wd"].T

    def _head(self, x):
        xf = rmsnorm(x, self.W["final_norm"], self.cfg.rms_eps)
        return self.W.lin("embed", xf)

    # --------------------------------------------------- one token (O1 form)
    def step(self, tok: int) -> np.ndarray:
        """Run one token at the current position, update state and cache, return logits [vocab]."""
        c = self.cfg
        p = self.pos
        if p >= c.max_ctx:
            raise ValueError("context full")
        x = self.W.rows("embed", int(tok))
        for l in range(c.n_layers):
            h = rmsnorm(x, self.W[f"l{l}.norm1"], c.rms_eps)
            if c.is_attention(l):
                q, k, v = self._attn_project(l, h, p)
                self.Kc[l][:, p] = kv_round(k, self.kv)
                self.Vc[l][:, p] = kv_round(v, self.kv)
                o = attend_one(q, self.Kc[l][:, : p + 1], self.Vc[l][:, : p + 1])
                x = x + o.reshape(-1) @ self.W[f"l{l}.attn.wo"].T
            else:
                q, k, v, alpha, beta = self._dn_project(l, h)
                self.S[l], o = delta_step(self.S[l], q, k, v, alpha, beta)
                x = x + o.reshape(-1) @ self.W[f"l{l}.dn.wo"].T
            x = self._ffn(l, x)
        self.pos = p + 1
        return self._head(x)

    # ------------------------------------------------ whole sequence (O2 form)
    def forward(self, tokens, logits: str = "all") -> dict:
        """Fresh state, whole sequence at once.  Returns logits ("all" [T, vocab] or "last" [vocab]),
        the final DeltaNet state per layer, and the rotated K / V per attention layer [nkv, T, hd]."""
        c = self.cfg
        tokens = np.asarray(tokens)
        T = tokens.shape[0]
        positions = np.arange(T)
        X = self.W.rows("embed", tokens)
        S_out, KV_out = {}, {}
        for l in range(c.n_layers):
            Hn = rmsnorm(X, self.W[f"l{l}.norm1"], c.rms_eps)
            if c.is_attention(l):
                Q, K, V = self._attn_project(l, Hn, positions)
                K, V = kv_round(K, self.kv), kv_round(V, self.kv)
                O = causal_attention(Q, K, V)
                KV_out[l] = (np.transpose(K, (1, 0, 2)).copy(), np.transpose(V, (1, 0, 2)).copy())
                X = X + O.reshape(T, -1) @ self.W[f"l{l}.attn.wo"].T
            else:
                Q, K, V, alpha, beta = self._dn_project(l, Hn)
                O = np.empty((T, c.dn_heads, c.dn_dv), self.dtype)
                S_l = np.empty((c.dn_heads, c.dn_dv, c.dn_dk), self.dtype)
                S0 = np.zeros((c.dn_dv, c.dn_dk), self.dtype)
                for hh in range(c.dn_heads):
                    O[:, hh], S_l[hh] = delta_parallel(S0, Q[:, hh], K[:, hh], V[:, hh],
                                                       alpha[:, hh], beta[:, hh])
                S_out[l] = S_l
                X = X + O.reshape(T, -1) @ self.W[f"l{l}.dn.wo"].T
            X = self._ffn(l, X)
        out = {"n_tokens": T, "S": S_out, "KV": KV_out}
        out["logits"] = self._head(X) if logits == "all" else self._head(X[-1])
        return out

    # ------------------------------------------------------ speculative verify
    def snapshot(self) -> dict:
        return {"pos": self.pos, "S": {l: S.copy() for l, S in self.S.items()},
                "Kc": {l: K.copy() for l, K in self.Kc.items()}, "Vc": {l: V.copy() for l, V in self.Vc.items()}}

    def restore(self, snap: dict):
        self.pos = snap["pos"]
        self.S = {l: S.copy() for l, S in snap["S"].items()}
        self.Kc = {l: K.copy() for l, K in snap["Kc"].items()}
        self.Vc = {l: V.copy() for l, V in snap["Vc"].items()}

    def verify(self, tokens) -> dict:
        """Score the pending token and k drafts, tokens = [t0, d1..dk], from the current position.

        Speculative decoding keeps the main model's greedy output exactly (Reddit follow-up on the
        27B model, speculative-decoding paragraph): y_i is the greedy choice after feeding
        tokens[0..i-1] one by one, the accepted count a is the longest prefix with d_i == y_i, and
        the state and cache end as if only tokens[0..a] had been decoded (position advanced by
        a + 1).  The caller emits y_1..y_{a+1}; y_{a+1} becomes the next pending token.
        Returns {"y": [k+1] ints, "a": int, "logits": [k+1, vocab]}."""
        tokens = [int(t) for t in tokens]
        if not tokens:
            raise ValueError("verify needs the pending token")
        start = self.snapshot()
        logits = np.stack([self.step(t) for t in tokens])
        y = [self.argmax(lg) for lg in logits]
        a = 0
        while a < len(tokens) - 1 and tokens[a + 1] == y[a]:
            a += 1
        # roll back: the state after tokens[0..a] only
        self.restore(start)
        for t in tokens[: a + 1]:
            self.step(t)
        return {"y": y, "a": a, "logits": logits}

    # ------------------------------------------------------------- helpers
    @staticmethod
    def argmax(logits) -> int:
        """Greedy choice; numpy's argmax returns the lowest index among equal maxima."""
        return int(np.argmax(logits))

    def greedy(self, prompt, n_steps: int):
        """Prompt through ``forward``, then ``n_steps`` token-by-token greedy steps.

        Returns (tokens fed to each decode step [n_steps], logits of each decode step [n_steps, vocab],
        last-prompt-position logits)."""
        fwd = self.forward(prompt, logits="last")
        self.load_state(fwd)
        nxt = self.argmax(fwd["logits"])
        fed, outs = [], []
        for _ in range(n_steps):
            fed.append(nxt)
            lg = self.step(nxt)
            outs.append(lg)
            nxt = self.argmax(lg)
        return np.array(fed, dtype=np.int32), np.stack(outs) if outs else None, fwd["logits"]

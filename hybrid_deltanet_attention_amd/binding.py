"""ctypes binding of ``include/mk.h`` -- argument marshalling only.

Every step of the decode path runs in the HIP library; nothing here computes model math.
Functions keep the C names (``mk_create``, ``mk_decode_step``, ...); ``Model`` bundles them with
a torch-allocated workspace.  When ``libmk.so`` is missing, every call raises -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))

MK_OK = 0
MK_BF16, MK_F32, MK_F16, MK_I32, MK_Q4G32, MK_Q8 = 1, 2, 3, 4, 5, 6
STATUS = {
    0: "MK_OK", -1: "MK_E_INVALID", -2: "MK_E_SHAPE", -3: "MK_E_DTYPE", -4: "MK_E_NAME",
    -5: "MK_E_ORDER", -6: "MK_E_CTX_FULL", -7: "MK_E_NO_DEVICE", -8: "MK_E_OCCUPANCY",
    -9: "MK_E_HIP", -10: "MK_E_DEVICE_TIMEOUT", -11: "MK_E_UNSUPPORTED",
}

# every symbol include/mk.h declares
EXPORTS = ["mk_workspace_bytes", "mk_create", "mk_load_weights", "mk_check_tensors", "mk_prefill",
           "mk_decode_step", "mk_decode_step_noalloc", "mk_verify_k", "mk_reset", "mk_sync", "mk_get_position", "mk_set_position",
           "mk_state_bytes", "mk_read_state", "mk_write_state", "mk_set_grid", "mk_get_grid",
           "mk_set_trace", "mk_last_error", "mk_destroy"]
# every symbol include/mk_test.h declares (single phases for unit parity tests; not product surface)
TEST_EXPORTS = ["mk_test_gemv", "mk_test_q4_tile", "mk_test_gemv_q4", "mk_test_deltanet", "mk_test_argmax"]


class MkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class mk_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "hidden", "ffn", "vocab", "period", "attn_slot", "dn_heads", "dn_dk", "dn_dv",
        "n_q_heads", "n_kv_heads", "head_dim", "tied_embeddings", "weight_dtype", "kv_dtype",
        "max_ctx", "max_verify_k")] + [(n, ctypes.c_float) for n in ("rms_eps", "l2_eps", "rope_theta")]


class mk_tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("data", ctypes.c_void_p), ("on_device", ctypes.c_int32)]


def lib_path() -> str:
    return os.path.join(PKG, "libmk.so")


_LIB = None


def load_library():
    """Load the in-tree ``libmk.so``; raises if it was not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise MkError(-7, f"{path} is missing: build it with python -m hybrid_deltanet_attention_amd.build")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "mk_workspace_bytes": (SZ, [P]),
        "mk_create": (ctypes.c_int, [P, ctypes.c_int, P, SZ, P, P]),
        "mk_load_weights": (ctypes.c_int, [P, P, I32]),
        "mk_check_tensors": (ctypes.c_int, [P, P, I32]),
        "mk_prefill": (ctypes.c_int, [P, P, I32, P, P]),
        "mk_decode_step": (ctypes.c_int, [P, P, P, P]),
        "mk_decode_step_noalloc": (ctypes.c_int, [P, P, P, P]),
        "mk_verify_k": (ctypes.c_int, [P, P, I32, P, P]),
        "mk_reset": (ctypes.c_int, [P]),
        "mk_sync": (ctypes.c_int, [P]),
        "mk_get_position": (ctypes.c_int, [P, P]),
        "mk_set_position": (ctypes.c_int, [P, I32]),
        "mk_state_bytes": (SZ, [P, I32]),
        "mk_read_state": (ctypes.c_int, [P, I32, P]),
        "mk_write_state": (ctypes.c_int, [P, I32, P]),
        "mk_set_grid": (ctypes.c_int, [P, I32]),
        "mk_get_grid": (ctypes.c_int, [P, P]),
        "mk_set_trace": (ctypes.c_int, [P, P, SZ]),
        "mk_last_error": (ctypes.c_char_p, [P]),
        "mk_destroy": (None, [P]),
        "mk_test_gemv": (ctypes.c_int, [P, I32, I32, P, P, P]),
        "mk_test_q4_tile": (ctypes.c_int, [P, I32, I32, P, P]),
        "mk_test_gemv_q4": (ctypes.c_int, [P, I32, I32, P, P, P]),
        "mk_test_deltanet": (ctypes.c_int, [P, I32, I32, I32, ctypes.c_float, P, P, P]),
        "mk_test_argmax": (ctypes.c_int, [P, I32, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _LIB = lib
    return lib


def _err(ctx=None) -> str:
    m = load_library().mk_last_error(ctx)
    return m.decode() if m else ""


def _check(rc: int, ctx=None):
    if rc != MK_OK:
        raise MkError(rc, _err(ctx))


def mk_config_from(cfg, max_verify_k: int = 0, weight_dtype: int = MK_BF16, kv_dtype: int = MK_F32) -> mk_config:
    """Marshal a model shape (any object with the synth.ModelConfig attributes) into the C struct.
    weight_dtype: MK_BF16, or MK_Q4G32 for 4-bit block-quantised matrices; kv_dtype: MK_F32, MK_F16
    or MK_Q8 (the KV cache's element type)."""
    c = mk_config()
    for f in ("n_layers", "hidden", "ffn", "vocab", "period", "attn_slot", "dn_heads", "dn_dk",
              "dn_dv", "n_q_heads", "n_kv_heads", "head_dim", "max_ctx"):
        setattr(c, f, int(getattr(cfg, f)))
    c.tied_embeddings = 1 if getattr(cfg, "tied", True) else 0
    c.weight_dtype = int(weight_dtype)
    c.kv_dtype = int(kv_dtype)
    c.max_verify_k = max_verify_k
    c.rms_eps = float(cfg.rms_eps)
    c.l2_eps = float(cfg.l2_eps)
    c.rope_theta = float(cfg.rope_theta)
    return c


def mk_workspace_bytes(cfg) -> int:
    c = cfg if isinstance(cfg, mk_config) else mk_config_from(cfg)
    n = load_library().mk_workspace_bytes(ctypes.byref(c))
    if n == 0:
        raise MkError(-1, _err())
    return int(n)


def matrix_shapes(cfg) -> dict:
    """Logical [out, in] shape of every weight matrix of the model, by manifest name."""
    D, H, hd = cfg.hidden, cfg.dn_heads, cfg.head_dim
    out = {"embed": (cfg.vocab, D)}
    for l in range(cfg.n_layers):
        p = f"l{l}."
        if l % cfg.period == cfg.attn_slot:
            out.update({p + "attn.wq": (cfg.n_q_heads * hd, D), p + "attn.wk": (cfg.n_kv_heads * hd, D),
                        p + "attn.wv": (cfg.n_kv_heads * hd, D), p + "attn.wo": (D, cfg.n_q_heads * hd)})
        else:
            out.update({p + "dn.wqkv": (2 * H * cfg.dn_dk + H * cfg.dn_dv, D), p + "dn.wa": (H, D),
                        p + "dn.wb": (H, D), p + "dn.wo": (D, H * cfg.dn_dv)})
        out.update({p + "ffn.wg": (cfg.ffn, D), p + "ffn.wu": (cfg.ffn, D), p + "ffn.wd": (D, cfg.ffn)})
    return out


def _tensor_array(weights: dict, keep: list, q4_shapes: dict | None = None):
    """weights: name -> numpy uint16 array (host) or torch uint16/int16/bfloat16 CUDA tensor; with
    q4_shapes, a flat uint8 array (host) or CUDA tensor is a Q4G32 matrix of that logical shape."""
    arr = (mk_tensor * len(weights))()
    for i, (name, w) in enumerate(weights.items()):
        t = arr[i]
        nb = name.encode()
        keep.append(nb)
        t.name = nb
        if isinstance(w, np.ndarray):
            a = np.ascontiguousarray(w)
            keep.append(a)
            t.dtype = MK_BF16 if a.dtype == np.uint16 else (MK_F32 if a.dtype == np.float32 else 0)
            t.data = a.ctypes.data
            t.on_device = 0
            shape = a.shape
            if a.dtype == np.uint8 and q4_shapes is not None and name in q4_shapes:
                t.dtype = MK_Q4G32
                shape = q4_shapes[name]
        else:  # torch tensor
            import torch
            a = w.contiguous()
            keep.append(a)
            t.dtype = MK_BF16 if a.dtype in (torch.bfloat16, torch.uint16, torch.int16) else 0
            t.data = a.data_ptr()
            t.on_device = 1 if a.is_cuda else 0
            shape = tuple(a.shape)
            if a.dtype == torch.uint8 and q4_shapes is not None and name in q4_shapes:
                t.dtype = MK_Q4G32
                shape = q4_shapes[name]
        t.ndim = len(shape)
        for d in range(4):
            t.shape[d] = int(shape[d]) if d < len(shape) else 0
    return arr


def mk_check_tensors(cfg, weights: dict, weight_dtype: int = MK_BF16) -> None:
    c = mk_config_from(cfg, weight_dtype=weight_dtype)
    keep: list = []
    arr = _tensor_array(weights, keep, matrix_shapes(cfg) if weight_dtype == MK_Q4G32 else None)
    _check(load_library().mk_check_tensors(ctypes.byref(c), arr, len(weights)))


class Model:
    """A context on one device: workspace (torch uint8 tensor), stream, loaded weights."""

    def __init__(self, cfg, device: int = 0, stream=None, max_verify_k: int = 0, weight_dtype: int = MK_BF16,
                 kv_dtype: int = MK_F32):
        import torch
        self.lib = load_library()
        self.cfg = cfg
        self.weight_dtype = int(weight_dtype)
        self.kv_dtype = int(kv_dtype)
        self.c = mk_config_from(cfg, max_verify_k, weight_dtype, kv_dtype)
        self.device = device
        nbytes = mk_workspace_bytes(self.c)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=f"cuda:{device}")
        self.stream = stream if stream is not None else torch.cuda.current_stream(device)
        ctx = ctypes.c_void_p()
        rc = self.lib.mk_create(ctypes.byref(self.c), device, ctypes.c_void_p(self.workspace.data_ptr()),
                                nbytes, ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(ctx))
        _check(rc)
        self.ctx = ctx

    # ---- C entry points, same names
    def mk_load_weights(self, weights: dict):
        keep: list = []
        arr = _tensor_array(weights, keep, matrix_shapes(self.cfg) if self.weight_dtype == MK_Q4G32 else None)
        _check(self.lib.mk_load_weights(self.ctx, arr, len(weights)), self.ctx)

    def mk_prefill(self, d_tokens, n: int, d_next, d_logits=None):
        _check(self.lib.mk_prefill(self.ctx, _ptr(d_tokens), int(n), _ptr(d_next), _ptr(d_logits)), self.ctx)

    def mk_decode_step(self, d_tok, d_next, d_logits=None):
        _check(self.lib.mk_decode_step(self.ctx, _ptr(d_tok), _ptr(d_next), _ptr(d_logits)), self.ctx)

    def mk_decode_step_noalloc(self, d_tok, d_next, d_logits=None):
        _check(self.lib.mk_decode_step_noalloc(self.ctx, _ptr(d_tok), _ptr(d_next), _ptr(d_logits)), self.ctx)

    def mk_verify_k(self, d_tokens, k: int, d_out, d_n_accepted):
        _check(self.lib.mk_verify_k(self.ctx, _ptr(d_tokens), int(k), _ptr(d_out), _ptr(d_n_accepted)), self.ctx)

    def mk_reset(self):
        _check(self.lib.mk_reset(self.ctx), self.ctx)

    def mk_sync(self):
        _check(self.lib.mk_sync(self.ctx), self.ctx)

    def mk_get_position(self) -> int:
        v = ctypes.c_int32()
        _check(self.lib.mk_get_position(self.ctx, ctypes.byref(v)), self.ctx)
        return v.value

    def mk_set_position(self, pos: int):
        _check(self.lib.mk_set_position(self.ctx, int(pos)), self.ctx)

    def mk_read_state(self, layer: int) -> np.ndarray:
        n = self.lib.mk_state_bytes(self.ctx, layer)
        if n == 0:
            raise MkError(-1, "layer out of range")
        buf = np.empty(n // 4, dtype=np.float32)
        _check(self.lib.mk_read_state(self.ctx, layer, buf.ctypes.data), self.ctx)
        c = self.cfg
        if c.is_attention(layer):
            return buf.reshape(2, c.n_kv_heads, c.max_ctx, c.head_dim)
        return buf.reshape(c.dn_heads, c.dn_dv, c.dn_dk)

    def mk_write_state(self, layer: int, arr: np.ndarray):
        a = np.ascontiguousarray(arr, dtype=np.float32)
        if a.nbytes != self.lib.mk_state_bytes(self.ctx, layer):
            raise MkError(-2, "state size mismatch")
        _check(self.lib.mk_write_state(self.ctx, layer, a.ctypes.data), self.ctx)

    def mk_set_grid(self, n: int):
        _check(self.lib.mk_set_grid(self.ctx, int(n)), self.ctx)

    def mk_get_grid(self) -> int:
        v = ctypes.c_int32()
        _check(self.lib.mk_get_grid(self.ctx, ctypes.byref(v)), self.ctx)
        return v.value

    def mk_set_trace(self, d_trace=None):
        nbytes = 0 if d_trace is None else d_trace.numel() * d_trace.element_size()
        _check(self.lib.mk_set_trace(self.ctx, _ptr(d_trace), nbytes), self.ctx)

    def close(self):
        if getattr(self, "ctx", None):
            self.lib.mk_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


# ---- test-only single phases (include/mk_test.h): device tensors in, device tensors out; the
# current torch stream.  Argument marshalling only.
def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def mk_test_gemv(d_W, R: int, K: int, d_x, d_y):
    _check(load_library().mk_test_gemv(_ptr(d_W), R, K, _ptr(d_x), _ptr(d_y), _stream()))


def mk_test_q4_tile(d_src, R: int, K: int, d_tiles):
    _check(load_library().mk_test_q4_tile(_ptr(d_src), R, K, _ptr(d_tiles), _stream()))


def mk_test_gemv_q4(d_tiles, R: int, K: int, d_x, d_y):
    _check(load_library().mk_test_gemv_q4(_ptr(d_tiles), R, K, _ptr(d_x), _ptr(d_y), _stream()))


def mk_test_deltanet(d_in, H: int, dk: int, dv: int, l2eps: float, d_S, d_o):
    _check(load_library().mk_test_deltanet(_ptr(d_in), H, dk, dv, l2eps, _ptr(d_S), _ptr(d_o), _stream()))


def mk_test_argmax(d_v, n: int, d_idx):
    _check(load_library().mk_test_argmax(_ptr(d_v), n, _ptr(d_idx), _stream()))

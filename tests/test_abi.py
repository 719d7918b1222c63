"""CPU checks of the C-ABI library: it loads, exports every function include/mk.h declares, and its
host-side validation (configuration, tensor manifest, device discovery) answers with the documented
status codes.  No kernel runs here."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import synth
from hybrid_deltanet_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mk.h")
TEST_HEADER = os.path.join(ROOT, "include", "mk_test.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.lib_path()):
        from hybrid_deltanet_attention_amd.build import build
        build()
    return B.load_library()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"\b(mk_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 15
    assert sorted(names) == sorted(B.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_exports_every_test_only_function(lib):
    # the single-phase entry points for unit parity tests, declared apart from the product surface
    names = declared_functions(TEST_HEADER)
    assert sorted(names) == sorted(B.TEST_EXPORTS)
    assert not set(names) & set(declared_functions())
    for n in names:
        assert hasattr(lib, n), n


def test_test_only_functions_reject_bad_arguments(lib):
    # argument checks answer MK_E_INVALID (-1) before anything is launched (no device needed)
    assert lib.mk_test_gemv(None, 4, 8, None, None, None) == -1
    assert lib.mk_test_gemv_q4(None, 4, 32, None, None, None) == -1
    assert lib.mk_test_q4_tile(None, 4, 33, None, None) == -1
    assert lib.mk_test_deltanet(None, 1, 512, 8, 1e-6, None, None, None) == -1
    assert lib.mk_test_argmax(None, 9000, None, None) == -1


def test_exported_symbols_are_plain_c(lib):
    # C linkage: the dynamic symbol table holds the plain names
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", B.lib_path()], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in declared_functions() + declared_functions(TEST_HEADER):
        assert n in syms, n


def _cfg(name="tiny", **kw):
    return B.mk_config_from(synth.get_config(name, **kw))


def test_workspace_bytes_grows_with_context(lib):
    a = B.mk_workspace_bytes(_cfg(max_ctx=128))
    b = B.mk_workspace_bytes(_cfg(max_ctx=256))
    assert 0 < a < b
    # the 0.8B shape: weights alone are ~1.2 GB of BF16
    big = B.mk_workspace_bytes(_cfg("hybrid_0p8b"))
    assert big > 1.17e9


@pytest.mark.parametrize("field,value", [
    ("n_layers", 0), ("hidden", 100), ("n_kv_heads", 3), ("head_dim", 6), ("attn_slot", 4),
    ("weight_dtype", 2), ("kv_dtype", 1), ("max_ctx", 0), ("tied_embeddings", 0), ("dn_dk", 512),
])
def test_bad_config_is_rejected(lib, field, value):
    c = _cfg()
    setattr(c, field, value)
    assert lib.mk_workspace_bytes(ctypes.byref(c)) == 0
    assert lib.mk_last_error(None)


def test_bad_eps_is_rejected(lib):
    c = _cfg()
    c.rms_eps = 0.0
    assert lib.mk_workspace_bytes(ctypes.byref(c)) == 0


def _manifest(cfg):
    return {n: np.zeros(shape, dtype=np.uint16) for n, shape, _ in synth.tensor_manifest(cfg)}


def test_tensor_manifest_accepted(lib):
    cfg = synth.get_config("tiny")
    B.mk_check_tensors(cfg, _manifest(cfg))


def _status(cfg, tensors):
    with pytest.raises(B.MkError) as e:
        B.mk_check_tensors(cfg, tensors)
    return e.value.code


def test_tensor_errors(lib):
    cfg = synth.get_config("tiny")
    t = _manifest(cfg)
    bad = dict(t)
    bad["l0.dn.wqkv"] = np.zeros((10, cfg.hidden), dtype=np.uint16)
    assert _status(cfg, bad) == -2                    # MK_E_SHAPE
    bad = dict(t)
    bad["l0.dn.wqkv"] = t["l0.dn.wqkv"].astype(np.float32)
    assert _status(cfg, bad) == -3                    # MK_E_DTYPE
    bad = dict(t)
    del bad["final_norm"]
    assert _status(cfg, bad) == -4                    # MK_E_NAME (missing)
    bad = dict(t)
    bad["l0.attn.wq"] = np.zeros((4, 4), dtype=np.uint16)  # layer 0 is DeltaNet
    assert _status(cfg, bad) == -4                    # MK_E_NAME (unknown)
    assert "l0.attn.wq" in B._err()


def test_create_without_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a HIP device is present")
    c = _cfg()
    need = lib.mk_workspace_bytes(ctypes.byref(c))
    ctx = ctypes.c_void_p()
    rc = lib.mk_create(ctypes.byref(c), 0, ctypes.c_void_p(1 << 20), need, None, ctypes.byref(ctx))
    assert rc == -7 and not ctx.value                 # MK_E_NO_DEVICE
    assert b"device" in lib.mk_last_error(None)


def test_create_argument_checks(lib):
    c = _cfg()
    need = lib.mk_workspace_bytes(ctypes.byref(c))
    ctx = ctypes.c_void_p()
    assert lib.mk_create(ctypes.byref(c), 0, None, need, None, ctypes.byref(ctx)) == -1
    assert lib.mk_create(ctypes.byref(c), 0, ctypes.c_void_p(1 << 20), need - 1, None, ctypes.byref(ctx)) == -1
    assert lib.mk_create(ctypes.byref(c), 0, ctypes.c_void_p((1 << 20) + 4), need, None, ctypes.byref(ctx)) == -1
    assert lib.mk_create(ctypes.byref(c), 0, ctypes.c_void_p(1 << 20), need, None, None) == -1


def test_null_context_calls_fail_cleanly(lib):
    assert lib.mk_decode_step(None, None, None, None) == -1
    assert lib.mk_prefill(None, None, 0, None, None) == -1
    assert lib.mk_reset(None) == -1
    assert lib.mk_sync(None) == -1
    assert lib.mk_verify_k(None, None, 0, None, None) in (-1, -11)
    assert lib.mk_state_bytes(None, 0) == 0
    lib.mk_destroy(None)


def test_q4_config_and_tensor_checks(lib):
    """4-bit weights: the matrices must come as MK_Q4G32 (gains as MK_BF16), widths must be
    multiples of 32, and speculative verify stays BF16-only."""
    import synth
    from hybrid_deltanet_attention_amd import binding as b
    cfg = synth.get_config("tiny")
    W = synth.make_q4_weights(cfg, 0)
    b.mk_check_tensors(cfg, W, weight_dtype=b.MK_Q4G32)
    with pytest.raises(b.MkError) as e:
        b.mk_check_tensors(cfg, synth.make_weights(cfg, 0), weight_dtype=b.MK_Q4G32)
    assert e.value.code == -3 and "MK_Q4G32" in str(e.value)
    with pytest.raises(b.MkError) as e:
        b.mk_check_tensors(cfg, W)  # a 4-bit buffer offered to a BF16 model
    assert e.value.code == -3
    q4 = b.mk_workspace_bytes(b.mk_config_from(cfg, weight_dtype=b.MK_Q4G32))
    bf = b.mk_workspace_bytes(b.mk_config_from(cfg))
    assert q4 < bf, "4-bit weights take less workspace"
    for bad in (dict(hidden=200), dict(ffn=776)):
        with pytest.raises(b.MkError):
            b.mk_workspace_bytes(b.mk_config_from(synth.get_config("tiny", **bad), weight_dtype=b.MK_Q4G32))
    # speculative verify with 4-bit weights: the verify records and DeltaNet snapshots add workspace
    assert b.mk_workspace_bytes(b.mk_config_from(cfg, max_verify_k=1, weight_dtype=b.MK_Q4G32)) > q4
    # 27B-scale: 14.08 GB of 4-bit weights (0.625 B per weight) plus state, cache and records, and the
    # prefill's scratch: the largest matrix expanded to BF16 high and low parts (2 x 17,408 rows of
    # 2 x 5,120 values, 0.71 GB) and activation rows twice as wide as the BF16 path's
    c27 = synth.get_config("hybrid_27b", max_ctx=2048)
    n = b.mk_workspace_bytes(b.mk_config_from(c27, weight_dtype=b.MK_Q4G32))
    wq = 2 * 17408 * (2 * 5120) * 2
    assert 14.0e9 + wq < n < 14.6e9 + wq + 0.5e9

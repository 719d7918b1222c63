"""mk_decode_step_noalloc -- the decode step with its exchange records in the library's static device
array -- against mk_decode_step through the C ABI: the same kernel on the same inputs, so tokens,
logits, DeltaNet states and KV entries must be bit-identical.

Two calls in a row share the one array: first the 0.8B-shaped model (about 9 MB of records), then
the tiny model (well under 1 MB) at an odd grid, whose records sit where the first model's did and
whose launch epochs repeat the first model's -- so a record left over from the first call would be
taken as current if the entry point did not clear what it uses.  The second call also alternates
the two entry points on one context.  A model whose records exceed the array is refused with
MK_E_UNSUPPORTED before anything is launched.
"""
import numpy as np
import pytest

import synth
from gpu_util import torch_cuda

pytestmark = pytest.mark.gpu


def _run(cfg, W, prompt, n_steps, mode, grid=None):
    """prefill, then n_steps decode steps fed back on the device; mode: 'plain', 'noalloc' or
    'alternate' (noalloc on even steps)"""
    from hybrid_deltanet_attention_amd import Model
    torch = torch_cuda()
    m = Model(cfg, device=0)
    m.mk_load_weights(W)
    if grid is not None:
        m.mk_set_grid(grid)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    m.mk_prefill(torch.tensor(np.asarray(prompt, dtype=np.int32), device="cuda"), len(prompt), tok)
    logits, toks = [], []
    for i in range(n_steps):
        na = mode == "noalloc" or (mode == "alternate" and i % 2 == 0)
        (m.mk_decode_step_noalloc if na else m.mk_decode_step)(tok, tok, lg)
        m.mk_sync()
        logits.append(lg.cpu().numpy().copy())
        toks.append(int(tok.item()))
    states = [m.mk_read_state(l).copy() for l in range(cfg.n_layers)]
    pos = m.mk_get_position()
    m.close()
    return logits, toks, states, pos


def _same(a, b, what):
    la, ta, sa, pa = a
    lb, tb, sb, pb = b
    assert ta == tb, f"{what}: tokens {ta} vs {tb}"
    assert pa == pb, f"{what}: position {pa} vs {pb}"
    for i, (x, y) in enumerate(zip(la, lb)):
        assert np.array_equal(x, y), f"{what}: logits of step {i} differ"
    for l, (x, y) in enumerate(zip(sa, sb)):
        assert np.array_equal(x, y), f"{what}: state of layer {l} differs"


def test_noalloc_equals_decode_two_calls_second_smaller():
    big = synth.get_config("hybrid_0p8b")
    Wb = synth.make_weights(big, 21)
    pb = synth.make_prompt(big.vocab, 40, 21)
    small = synth.get_config("tiny")
    Ws = synth.make_weights(small, 22)
    ps = synth.make_prompt(small.vocab, 12, 22)
    ref_big = _run(big, Wb, pb, 12, "plain")
    ref_small = _run(small, Ws, ps, 12, "plain", grid=37)
    print(f"[noalloc] 0.8B tokens {ref_big[1]}", flush=True)
    _same(_run(big, Wb, pb, 12, "noalloc"), ref_big, "0.8B, static records")
    print("[noalloc] 0.8B bit-identical; now the tiny model on the same array", flush=True)
    _same(_run(small, Ws, ps, 12, "noalloc", grid=37), ref_small, "tiny after 0.8B, static records")
    _same(_run(small, Ws, ps, 12, "alternate", grid=37), ref_small, "tiny, alternating entry points")


def test_noalloc_refuses_records_beyond_the_array():
    from hybrid_deltanet_attention_amd import Model, MkError
    torch = torch_cuda()
    # a 131,072-position cache makes the attention partial records alone about 17 MB
    cfg = synth.get_config("tiny", max_ctx=131072)
    m = Model(cfg, device=0)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(MkError) as e:
        m.mk_decode_step_noalloc(tok, tok)
    assert e.value.code == -11 and "static scratch" in str(e.value)
    m.close()

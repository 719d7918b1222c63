"""4-bit (Q4G32) decode kernel vs the CPU oracle on the same stored weights.

The oracle decodes the same bytes exactly (float64) and runs the same model, so the bars are the
BF16 path's: logits relative L2 <= 1e-2 at every step, top-1 agreement >= 99 %, mean KL <= 1e-3
nats, DeltaNet state and KV cache relative L2 <= 1e-3.  The prompt runs through the prefill GEMMs
(weights expanded to BF16 high and low parts) and its last token through one decode launch.

Sizes: the tiny hybrid; ragged widths (columns that do not fill a 2048-column unit, odd head
counts); a 4-layer slice at the 27B-scale width (hidden 5120: 2.5 units per row; FFN 17408:
8.5 units; 24 Q / 4 KV heads, 151,936-row tied LM head).  The full 64-layer 27B-scale model runs
on the GPU with the same weight generator, so its first four layers hold exactly the slice's
tensors: after the same prompt their DeltaNet states and KV entries must equal the slice's bit
for bit, and two runs must agree bitwise.  Deeper layers at full depth are checked only through
these properties (the float64 oracle would need minutes per token at 22.5 B weights).
"""
import numpy as np
import pytest

import synth
from gpu_util import new_model, run_teacher_forced, torch_cuda
from test_gpu_parity import _check_run

pytestmark = pytest.mark.gpu

MK_Q4G32 = 5


@pytest.mark.parametrize("seed", [0, 1])
def test_q4_tiny_prompt_then_decode(seed):
    cfg = synth.get_config("tiny")
    W = synth.make_q4_weights(cfg, seed)
    _check_run(cfg, W, synth.make_prompt(cfg.vocab, 16, seed), 32, weight_dtype=MK_Q4G32)


def test_q4_ragged_shapes():
    # widths that are multiples of 32 but not of the 2048-column unit, odd head counts, small grid
    cfg = synth.get_config("tiny", hidden=224, ffn=352, dn_heads=3, dn_dk=32, dn_dv=32, n_q_heads=6,
                           n_kv_heads=3, head_dim=32, vocab=1000, n_layers=5, max_ctx=64)
    W = synth.make_q4_weights(cfg, 5, gain_noise=0.1)
    _check_run(cfg, W, synth.make_prompt(cfg.vocab, 21, 5), 12, weight_dtype=MK_Q4G32)
    _check_run(cfg, W, synth.make_prompt(cfg.vocab, 9, 6), 6, grid=37, weight_dtype=MK_Q4G32)


def test_q4_long_prompt_small_grid():
    # 23 attention items per KV head and 32 combine outputs per workgroup: the combine stages its
    # partials in several rounds through the 4-bit kernel's smaller partials region
    cfg = synth.get_config("tiny", max_ctx=512)
    W = synth.make_q4_weights(cfg, 9)
    _check_run(cfg, W, synth.make_prompt(cfg.vocab, 360, 9), 8, grid=8, weight_dtype=MK_Q4G32)


def _slice_cfg(n_layers, max_ctx=64):
    return synth.get_config("hybrid_27b", n_layers=n_layers, max_ctx=max_ctx)


PROMPT_27B = 8


@pytest.mark.timeout(1200)
def test_q4_27b_width_slice_1k_context():
    """a 4-layer slice at 27B width: a 1,024-token prompt then 32 decode steps against the oracle
    (the oracle keeps the decoded slice, about 17 GB in float64, and runs the prompt in its
    whole-sequence form)"""
    cfg4 = _slice_cfg(4, max_ctx=1024 + 32)
    W4 = synth.make_q4_weights(cfg4, 0)
    prompt = synth.make_prompt(cfg4.vocab, 1024, 1)
    print("[27B width, 4 layers] prompt 1024, 32 steps", flush=True)
    _check_run(cfg4, W4, prompt, 32, weight_dtype=MK_Q4G32, oracle_cache=1 << 36)


def test_q4_27b_full_depth_against_slice():
    cfg4 = _slice_cfg(4)
    prompt = synth.make_prompt(cfg4.vocab, PROMPT_27B, 0)
    # the full-depth model: its first four layers are the slice's tensors (same generator, manifest
    # order); feed it the same tokens
    torch = torch_cuda()
    cfg = _slice_cfg(64)
    W = synth.make_q4_weights(cfg, 0)
    m = new_model(cfg, W, weight_dtype=MK_Q4G32)
    del W
    d_prompt = torch.tensor(np.asarray(prompt, dtype=np.int32), device="cuda")
    runs = []
    for rep in range(2):
        if rep:
            m.mk_reset()
        d_next = torch.zeros(1, dtype=torch.int32, device="cuda")
        d_logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
        m.mk_prefill(d_prompt, len(prompt), d_next, d_logits)
        m.mk_sync()
        lg = d_logits.cpu().numpy().copy()
        assert np.all(np.isfinite(lg)), "full-depth logits must be finite"
        assert int(d_next.item()) == int(np.argmax(lg)), "fused argmax must equal argmax of the written logits"
        runs.append((lg, {l: m.mk_read_state(l).copy() for l in range(4)}))
    assert np.array_equal(runs[0][0], runs[1][0]), "two full-depth runs must agree bitwise"
    print(f"[27B full depth] prompt logits max |.| {np.abs(runs[0][0]).max():.3f}", flush=True)
    m.close()
    # layers 0..3 after the prompt against a slice run of the same prompt
    m4 = new_model(cfg4, synth.make_q4_weights(cfg4, 0), weight_dtype=MK_Q4G32)
    d_next = torch.zeros(1, dtype=torch.int32, device="cuda")
    m4.mk_prefill(d_prompt, len(prompt), d_next, None)
    m4.mk_sync()
    for l in range(4):
        a = m4.mk_read_state(l)
        b = runs[0][1][l]
        if cfg4.is_attention(l):
            a, b = a[:, :, :PROMPT_27B], b[:, :, :PROMPT_27B]
        assert np.array_equal(a, b), f"layer {l}: full-depth state differs from the 4-layer slice"
    m4.close()

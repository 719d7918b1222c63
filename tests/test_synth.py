"""The seeded input generators: BF16 rounding, manifest, determinism."""
import numpy as np

import synth


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, 1.0 + 2.0**-9, -2.5, 3.14159265,
                  1.0 + 2.0**-7 + 2.0**-8], dtype=np.float32)
    # 1+2^-8 is a tie between 1.0 (0x3F80, even) and 0x3F81 -> 0x3F80
    # 1+3*2^-8 is a tie between 0x3F81 and 0x3F82 (even) -> 0x3F82
    # 1+2^-7+2^-8 = 0x3F81 + half -> tie, odd 0x3F81 rounds up to 0x3F82
    want = np.array([0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020, 0x4049, 0x3F82], dtype=np.uint16)
    assert np.array_equal(synth.bf16_round(f), want)
    back = synth.bf16_bits_to_f32(want)
    assert back[0] == 1.0 and back[4] == -2.5


def test_manifest_tiny_and_0p8b_sizes():
    t = synth.get_config("tiny")
    n = sum(int(np.prod(s)) for _, s, k in synth.tensor_manifest(t) if k == "matrix")
    assert n == 4_397_056
    c = synth.get_config("hybrid_0p8b")
    n = sum(int(np.prod(s)) for _, s, k in synth.tensor_manifest(c) if k == "matrix")
    assert n == 587_137_024


def test_weights_deterministic_and_scaled():
    t = synth.get_config("tiny")
    a = synth.make_weights(t, 5)
    b = synth.make_weights(t, 5)
    c = synth.make_weights(t, 6)
    assert all(np.array_equal(a[k], b[k]) for k in a)
    assert not np.array_equal(a["embed"], c["embed"])
    e = synth.bf16_bits_to_f32(a["embed"])
    assert abs(float(e.std()) - 0.02) < 1e-3
    assert np.all(synth.bf16_bits_to_f32(a["l0.norm1"]) == 1.0)
    g = synth.bf16_bits_to_f32(synth.make_weights(t, 3, gain_noise=0.1)["l0.norm1"])
    assert 0.05 < float(g.std()) < 0.15


def test_prompts():
    p = synth.make_prompt(4096, 16, 0)
    assert p.dtype == np.int32 and p.shape == (16,) and p.min() >= 0 and p.max() < 4096
    assert np.array_equal(p, synth.make_prompt(4096, 16, 0))
    assert not np.array_equal(p, synth.make_prompt(4096, 16, 1))


def test_q4_weights_deterministic_and_sized():
    cfg = synth.get_config("tiny")
    a = synth.make_q4_weights(cfg, 0)
    b = synth.make_q4_weights(cfg, 0)
    c = synth.make_q4_weights(cfg, 1)
    for name, shape, kind in synth.tensor_manifest(cfg):
        if kind == "matrix":
            assert a[name].dtype == np.uint8 and a[name].size == synth.q4_nbytes(*shape) == shape[0] * shape[1] * 5 // 8
        else:
            assert a[name].dtype == np.uint16 and a[name].shape == shape
        assert np.array_equal(a[name], b[name])
    assert not np.array_equal(a["embed"], c["embed"])
    # block parameters: d near 0.0054, m near -7.5 d
    R, K = cfg.vocab, cfg.hidden
    dm = a["embed"][R * K // 2:].view("<f2").reshape(-1, 2).astype(np.float64)
    assert 0.004 < dm[:, 0].mean() < 0.007 and np.all(dm[:, 0] > 0)
    assert abs((dm[:, 1] + 7.5 * dm[:, 0]).mean()) < 1e-4

"""Host-side pieces of bench.py that need no GPU: the argument contract, the algorithmic byte
count of a decode launch, and the energy-counter reader's failure path."""
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_0p8b():
    # 587,137,024 BF16 parameters outside the embedding-as-head (incl. gains) plus the tied head,
    # the DeltaNet state read and written, and 12,288 bytes of FP32 KV per visible position
    cfg = synth.get_config("hybrid_0p8b")
    a = bench.algorithmic_bytes(cfg, 1000)
    assert a["state"] == 18 * 16 * 128 * 128 * 4 * 2
    assert a["kv"] == 12288 * 1000
    assert a["lm_head"] == 2 * 151936 * 1024 + 6 * 1024
    per_dn = 2 * ((2 * 16 * 128 + 16 * 128 + 2 * 16) * 1024 + 1024 * 2048 + 3 * 3584 * 1024) + 8 * 1024
    per_att = 2 * ((8 + 4) * 128 * 1024 + 1024 * 1024 + 3 * 3584 * 1024) + 8 * 1024
    assert a["weights"] == 18 * per_dn + 6 * per_att
    assert a["total"] == a["weights"] + a["lm_head"] + a["state"] + a["kv"]


def test_energy_reader_never_raises():
    read, err = bench._energy_reader()
    if read is None:
        assert isinstance(err, str) and err
    else:
        j, _ = read()
        assert j >= 0


def test_prefill_flops_0p8b_pp520():
    # the prefill's algorithmic work at pp520: GEMMs 2 x 431,554,560 layer weights x 520 tokens,
    # chunked DeltaNet about 9.96 MFLOP per full 64-token chunk and head (8 full chunks + one of 8
    # tokens, 16 heads, 18 layers), causal attention 2 x 2 x 128 x (520 x 521 / 2) x 8 heads x 6
    # layers, and the LM head on one row
    cfg = synth.get_config("hybrid_0p8b")
    f = bench.prefill_flops(cfg, 520)
    assert f["gemm"] == 2 * 520 * 431554560
    assert f["attention"] == 2 * 2 * 128 * (520 * 521 / 2) * 8 * 6
    assert f["lm_head"] == 2 * 151936 * 1024
    full = 2 * 64 * 64 * 128 * 2 + 2 * 64 * 128 * 128 * 3 + 64 * 64 * 128 + 2 * 64 * 64 * 128
    assert full == 9961472
    tail = 2 * 8 * 8 * 128 * 2 + 2 * 8 * 128 * 128 * 3 + 8 * 8 * 128 + 2 * 8 * 8 * 128
    assert f["deltanet"] == 18 * 16 * (8 * full + tail)
    assert abs(f["total"] / 1e9 - 475.65) < 0.01

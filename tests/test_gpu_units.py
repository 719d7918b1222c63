"""Single phases of the decode step on the GPU (include/mk_test.h) against the oracle's own
primitives, so that a parity failure can be pinned to one phase.  Each test export runs the decode
kernels' device code for that phase: the BF16 GEMV, the 4-bit GEMV, the gated delta rule on the
state rows, and the final greedy pick.

Bars: the BF16 GEMV multiplies exact BF16 weights by x split into BF16 high and low parts
(x - hi - lo = O(2^-17 |x|)) and sums in FP32, so relative L2 errors stay near 1e-6 (bar 1e-5); with
small integer weights and inputs every product and partial sum is exact in FP32, so the result must
equal the integer dot product exactly.  The 4-bit GEMV quantises x per 32-column block to 16-bit
integers (step max|x| / 30000), about 1e-5 relative (bar 1e-4).  The delta rule runs in FP32 against
the oracle's float64 (bar 1e-5).  The greedy pick is exact: largest value, lowest index on ties.
"""
import numpy as np
import pytest

import synth
from oracle import deltanet as odn
from oracle import primitives as prim
from oracle import quant as oq
from oracle.metrics import rel_l2
from gpu_util import torch_cuda

pytestmark = pytest.mark.gpu


def _dev(a):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _out(n, dtype):
    torch = torch_cuda()
    return torch.full((n,), float("nan") if dtype == "f" else -7, dtype=torch.float32 if dtype == "f" else torch.int32,
                      device="cuda")


def _host(t):
    torch = torch_cuda()
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("R,K", [(4, 8), (37, 200), (6176, 1024), (1024, 3584), (257, 5120)])
def test_gemv_bf16_against_float64(R, K):
    from hybrid_deltanet_attention_amd import binding as B
    rng = np.random.default_rng([R, K, 1])
    Wb = synth.bf16_round(rng.standard_normal((R, K)).astype(np.float32) * np.float32(0.02))
    x = rng.standard_normal(K).astype(np.float32)
    ref = prim.bf16_decode(Wb) @ x.astype(np.float64)
    y = _out(R, "f")
    B.mk_test_gemv(_dev(Wb), R, K, _dev(x), y)
    g = _host(y)
    e = rel_l2(g, ref)
    print(f"[gemv bf16 {R}x{K}] rel-L2 {e:.2e}", flush=True)
    assert np.all(np.isfinite(g)) and e <= 1e-5


def test_gemv_bf16_exact_on_integers():
    # integer weights in [-8, 8] (exact in BF16) and integer inputs in [-64, 64] (hi = x, lo = 0):
    # every product and partial sum is an integer below 2^24, so the FP32 result is exact
    from hybrid_deltanet_attention_amd import binding as B
    R, K = 97, 2056
    rng = np.random.default_rng(5)
    Wf = rng.integers(-8, 9, size=(R, K)).astype(np.float32)
    x = rng.integers(-64, 65, size=K).astype(np.float32)
    y = _out(R, "f")
    B.mk_test_gemv(_dev(synth.bf16_round(Wf)), R, K, _dev(x), y)
    ref = (Wf.astype(np.int64) @ x.astype(np.int64)).astype(np.float32)
    assert np.array_equal(_host(y), ref)


@pytest.mark.parametrize("R,K", [(4, 32), (37, 224), (4096, 5120), (515, 17408)])
def test_gemv_q4_against_float64(R, K):
    from hybrid_deltanet_attention_amd import binding as B
    rng = np.random.default_rng([R, K, 2])
    buf = synth.q4_draw(rng, R, K)
    x = rng.standard_normal(K).astype(np.float32)
    ref = oq.q4g32_dequant(buf, R, K) @ x.astype(np.float64)
    torch = torch_cuda()
    tiles = torch.zeros(((R + 3) // 4 * 4 * K * 5) // 8, dtype=torch.uint8, device="cuda")
    B.mk_test_q4_tile(_dev(buf), R, K, tiles)
    y = _out(R, "f")
    B.mk_test_gemv_q4(tiles, R, K, _dev(x), y)
    g = _host(y)
    e = rel_l2(g, ref)
    print(f"[gemv q4 {R}x{K}] rel-L2 {e:.2e}", flush=True)
    assert np.all(np.isfinite(g)) and e <= 1e-4


@pytest.mark.parametrize("H,dk,dv", [(16, 128, 128), (3, 48, 40), (2, 192, 64), (1, 256, 256)])
def test_deltanet_rows_against_float64(H, dk, dv):
    from hybrid_deltanet_attention_amd import binding as B
    rng = np.random.default_rng([H, dk, dv])
    q = rng.standard_normal((H, dk)).astype(np.float32)
    k = rng.standard_normal((H, dk)).astype(np.float32)
    v = rng.standard_normal((H, dv)).astype(np.float32)
    a = (rng.standard_normal(H) * 2).astype(np.float32)
    b = (rng.standard_normal(H) * 2).astype(np.float32)
    S = (rng.standard_normal((H, dv, dk)) * 0.1).astype(np.float32)
    inp = np.concatenate([q.ravel(), k.ravel(), v.ravel(), a, b]).astype(np.float32)
    l2eps = 1e-6
    alpha, beta = odn.gates(a.astype(np.float64), b.astype(np.float64))
    S_ref, o_ref = odn.delta_step(S.astype(np.float64), prim.l2norm(q.astype(np.float64), l2eps),
                                  prim.l2norm(k.astype(np.float64), l2eps), v.astype(np.float64), alpha, beta)
    dS = _dev(S)
    o = _out(H * dv, "f")
    B.mk_test_deltanet(_dev(inp), H, dk, dv, l2eps, dS, o)
    Sg, og = _host(dS), _host(o)
    es, eo = rel_l2(Sg, S_ref), rel_l2(og, o_ref.ravel())
    print(f"[deltanet H={H} dk={dk} dv={dv}] state rel-L2 {es:.2e} output {eo:.2e}", flush=True)
    assert es <= 1e-5 and eo <= 1e-5


@pytest.mark.parametrize("n", [1, 100, 8192])
def test_argmax_lowest_index_on_ties(n):
    from hybrid_deltanet_attention_amd import binding as B
    rng = np.random.default_rng(n)
    v = rng.standard_normal(n).astype(np.float32)
    if n > 1:
        v[rng.integers(0, n, size=3)] = -np.inf
        top = np.float32(v.max() + 1)
        ties = np.sort(rng.choice(n, size=min(n, 5), replace=False))
        v[ties] = top  # several equal maxima: the lowest index must win
    idx = _out(1, "i")
    B.mk_test_argmax(_dev(v), n, idx)
    want = int(np.flatnonzero(v == v.max())[0])
    assert int(_host(idx)[0]) == want

"""Benchmark: batch-1 decode of the 0.8B-shaped hybrid (one kernel launch per token) and pp520 prefill.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload (synthetic, seeded): the 0.8B-shaped hybrid -- 24 layers in a 3 DeltaNet : 1 attention
pattern, hidden 1024, 16 DeltaNet heads of 128, 8 Q / 2 KV attention heads of 128, SwiGLU 3584,
vocabulary 151936 tied -- with BF16 weights ~N(0, 0.02) from seed 0 and a 512-token uniform
random prompt.  After the prompt, W untimed decode steps, then K timed decode steps, each one
launch of the decode kernel with the token fed back on the device.  The pages time the same
shapes (pp520, tg128) on a real checkpoint and real text (luce-megakernel announcement, page 1,
results table); random ids and random weights stand in for them here.

Prints ONE JSON line.  ``value`` is decode tokens/s on the one GPU.  ``roofline`` prices the
decode kernel's algorithmic bytes per launch (weights + LM head + DeltaNet state read and write +
KV cache) against the 8 TB/s HBM peak, using the kernel's average duration measured with events
on the stream it is launched on.  ``cpu_baseline`` times the CPU oracle (fp64, token by token) on
a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
PROMPT = 512
PP = 520
SEED = 0
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL = "mk_decode_kernel"
# measured HBM traffic of the decode kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE), valid only for the
# kernel source it was measured on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_0p8b_traffic.json")
KERNEL_SOURCES = ["hybrid_deltanet_attention_amd/csrc/mk_decode.hip", "hybrid_deltanet_attention_amd/csrc/mk_device.h",
                  "hybrid_deltanet_attention_amd/csrc/mk_internal.h"]
COPY_BYTES = 1 << 30


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode launch from the committed counter summary, or None when the kernel
    source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return int(t["bytes_per_launch"])


def _counter_rows(d):
    import csv
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    return rows


def _mean_counter(rows, kernel_sub, counter):
    v = [float(r["Counter_Value"]) for r in rows if kernel_sub in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not v:
        raise SystemExit(f"no {counter} rows for a kernel named like {kernel_sub}")
    return float(np.mean(v)), len(v)


def summarize_pmc(dirs: dict) -> dict:
    """dirs: {"fetch": d, "write": d, "copy_fetch": d, "copy_write": d} (rocprofv3 -d output folders).
    FETCH_SIZE and WRITE_SIZE read KiB per dispatch; each is scaled by bytes/KiB that the same counter
    reports for a plain 1 GiB device-to-device copy."""
    cf, _ = _mean_counter(_counter_rows(dirs["copy_fetch"]), "opy", "FETCH_SIZE")
    cw, _ = _mean_counter(_counter_rows(dirs["copy_write"]), "opy", "WRITE_SIZE")
    kf, nf = _mean_counter(_counter_rows(dirs["fetch"]), KERNEL, "FETCH_SIZE")
    kw, nw = _mean_counter(_counter_rows(dirs["write"]), KERNEL, "WRITE_SIZE")
    sf, sw = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    return {"kernel": KERNEL, "source_sha256": kernel_source_hash(),
            "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw, "dispatches": [nf, nw],
            "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": COPY_BYTES,
            "fetch_scale": sf, "write_scale": sw,
            "bytes_per_launch": int(kf * 1024 * sf + kw * 1024 * sw)}


SIMDS = 1024  # 256 compute units x 4 SIMDs
MFMA_COUNTERS = ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_VALU_MFMA_BUSY_CYCLES",
                 "SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"]


def _kernel_durations(trace_dir):
    """kernel name -> (calls, average ns) from a rocprofv3 --kernel-trace --stats csv folder"""
    import csv
    out = {}
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                out[r["Name"]] = (int(r["Calls"]), float(r["AverageNs"]))
    if not out:
        raise SystemExit(f"no *kernel_stats.csv under {trace_dir}")
    return out


def _is_kernel(name: str, k: str) -> bool:
    """a profiler's kernel name (with namespace, template arguments and signature) is kernel k"""
    return any(pre + k + post in " " + name for pre in (" ", "::") for post in ("<", "("))


def summarize_mfma(pmc_dir, trace_dir, kernels=("pf_gemm_kernel", "pf_dn_cscan_mfma_kernel", "pf_dn_cprep_kernel",
                                                 "pf_attn_mfma_kernel"), clock_ghz: float = 2.4) -> str:
    """Matrix-core counters per prefill kernel family.  MFMA FLOP = MOPS x 512.  SQ_VALU_MFMA_BUSY_CYCLES
    counts matrix-core cycles at the peak rate (here 0.5 cycle per MOP, 1024 BF16 FLOP per SIMD and
    cycle), summed over the 1024 SIMDs, so busy / (cycles x 1024) is the fraction of the matrix-core
    peak a kernel reaches.  Two cycle counts: GRBM_GUI_ACTIVE (the csv sums it over the 8 XCDs;
    rocprof's MfmaUtil takes the largest, about the sum / 8) and the kernel's average duration from
    the kernel trace of the same command x the 2.4 GHz clock."""
    rows = _counter_rows(pmc_dir)
    durs = _kernel_durations(trace_dir)
    lines = [f"{'kernel (all template instances)':26s} {'disp':>5s} {'MFMA GFLOP':>11s} {'BF16 MOPS':>9s} "
             f"{'util(GUI) %':>11s} {'util(dur) %':>11s} {'avg us':>8s} {'MFMA TFLOP/s':>12s}"]
    for k in kernels:
        per = {}
        for r in rows:
            if _is_kernel(r["Kernel_Name"], k):
                d = per.setdefault(r["Dispatch_Id"], {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if not per:
            continue
        n = len(per)
        mean = lambda c: float(np.mean([d.get(c, 0.0) for d in per.values()]))
        mops_bf, mops_f32 = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16"), mean("SQ_INSTS_VALU_MFMA_MOPS_F32")
        busy, gui = mean("SQ_VALU_MFMA_BUSY_CYCLES"), mean("GRBM_GUI_ACTIVE")
        flop = (mops_bf + mops_f32) * 512
        calls = sum(c for name, (c, _) in durs.items() if _is_kernel(name, k))
        ns = sum(c * a for name, (c, a) in durs.items() if _is_kernel(name, k)) / max(calls, 1)
        u_gui = 100.0 * busy / (gui / 8 * SIMDS) if gui else float("nan")
        u_dur = 100.0 * busy / (ns * clock_ghz * SIMDS) if ns else float("nan")
        lines.append(f"{k:26s} {n:5d} {flop / 1e9:11.3f} {mops_bf / max(mops_bf + mops_f32, 1):9.2f} {u_gui:11.2f} "
                     f"{u_dur:11.2f} {ns / 1e3:8.2f} {flop / (ns * 1e-9) / 1e12 if ns else float('nan'):12.2f}")
    return "\n".join(lines)


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, 4 times: the reference for the byte counters."""
    import torch
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "reps": 4}), flush=True)


KV_BYTES = {"f32": 4.0, "f16": 2.0, "q8": 1.0 + 4.0 / 32}  # per cached value (int8: code + a scale per 32)


def algorithmic_bytes(cfg, L: int, wb: float = 2.0, kv: str = "f32") -> dict:
    """Bytes one decode launch must move at context length L (positions 0..L-1 visible); wb is the
    bytes per weight of the matrices (2 for BF16, 0.625 for 4-bit codes with an FP16 scale and
    offset per 32 weights); kv the KV cache's element type."""
    D, H = cfg.hidden, cfg.dn_heads
    w = 0
    state = 0
    kvb = 0
    for l in range(cfg.n_layers):
        if cfg.is_attention(l):
            rows_in = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
            kout = cfg.n_q_heads * cfg.head_dim
            kvb += 2 * cfg.n_kv_heads * cfg.head_dim * KV_BYTES[kv] * L  # K and V: L-1 positions read, 1 written
        else:
            rows_in = 2 * H * cfg.dn_dk + H * cfg.dn_dv + 2 * H
            kout = H * cfg.dn_dv
            state += 2 * H * cfg.dn_dv * cfg.dn_dk * 4       # read + write
        w += wb * (rows_in * D + D * kout + 3 * cfg.ffn * D) + 2 * 4 * D
    head = wb * cfg.vocab * D + 4 * D + wb * D               # tied LM head, final gain, embedding row
    return {"weights": w, "lm_head": head, "state": state, "kv": kvb, "total": w + head + state + kvb}


def prefill_flops(cfg, T: int, chunk: int = 64) -> dict:
    """Algorithmic floating-point work of a T-token prefill: the projection and FFN GEMMs
    (2 T x every layer weight), the chunked DeltaNet per (chunk of c tokens, head) -- K K^T, Q K^T,
    K S0^T, Q S0^T, U^T K, the triangular solve and lower(Q K^T) U -- causal attention (scores and
    P V over the visible positions), and the LM head on the last row only."""
    D, H, dk, dv = cfg.hidden, cfg.dn_heads, cfg.dn_dk, cfg.dn_dv
    gemm = dn = att = 0.0
    chunks = [min(chunk, T - c0) for c0 in range(0, T, chunk)]
    for l in range(cfg.n_layers):
        if cfg.is_attention(l):
            rows_in = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
            kout = cfg.n_q_heads * cfg.head_dim
            att += 2 * 2 * cfg.head_dim * (T * (T + 1) / 2) * cfg.n_q_heads
        else:
            rows_in = 2 * H * dk + H * dv + 2 * H
            kout = H * dv
            for c in chunks:
                dn += H * (2 * c * c * dk * 2 + 2 * c * dk * dv * 3 + c * c * dv + 2 * c * c * dv)
        gemm += 2.0 * T * (rows_in * D + D * kout + 3 * cfg.ffn * D)
    head = 2.0 * cfg.vocab * D
    return {"gemm": gemm, "deltanet": dn, "attention": att, "lm_head": head, "total": gemm + dn + att + head}


def stream_reference(n_bytes: int = 1 << 31, reps: int = 10) -> dict:
    """Streaming rates this GPU reaches on plain library kernels, the practical ceiling the decode
    kernel's rate is also put against: a device-to-device copy (read + write bytes) and a sum
    reduction (read bytes) over n_bytes, best of reps, timed with events."""
    import torch
    a = torch.empty(n_bytes // 2, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    res = {}
    for label, fn, moved in (("copy", lambda: b.copy_(a), 2 * n_bytes), ("sum", lambda: a.sum(dtype=torch.float32), n_bytes)):
        fn()
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / 1e3)
        res[label + "_GBs"] = round(moved / best / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    res["bytes"] = n_bytes
    res["best"] = max(res["copy_GBs"], res["sum_GBs"])
    return res


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(cfg, W, n_prompt=PP, n_steps=6, n_single=2) -> dict:
    """The oracle as it stands (fp64 NumPy) on this host: the pp520 prompt through its
    whole-sequence form (timed as the oracle's prefill), then n_steps token-by-token decode steps
    at positions 520.. (the GPU decode leg runs at 521..648), all BLAS threads; then n_single more
    decode steps with BLAS held to one thread."""
    from oracle import Oracle
    import synth
    t0 = time.perf_counter()
    o = Oracle(cfg, W)
    t_load = time.perf_counter() - t0
    prompt = synth.make_prompt(cfg.vocab, n_prompt, SEED)
    t0 = time.perf_counter()
    fwd = o.forward(prompt, logits="last")
    t_pre = time.perf_counter() - t0
    o.load_state(fwd)
    tok = int(np.argmax(fwd["logits"]))
    tok = int(np.argmax(o.step(tok)))  # first step pays one-off costs (page-in of the decoded weights)
    t1 = time.perf_counter()
    for _ in range(n_steps):
        tok = int(np.argmax(o.step(tok)))
    dt = time.perf_counter() - t1
    threads = _blas_threads()
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t2 = time.perf_counter()
            for _ in range(n_single):
                tok = int(np.argmax(o.step(tok)))
            single = {"value": round(n_single / (time.perf_counter() - t2), 3), "unit": "tok/s", "cores": 1,
                      "sample": f"{n_single} decode steps at positions {n_prompt + n_steps + 1}.."}
    except Exception as ex:
        single = {"status": f"threadpoolctl unavailable: {type(ex).__name__}"}
    return {"value": round(n_steps / dt, 3), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_steps} fp64 token-by-token decode steps at positions {n_prompt + 1}..{n_prompt + n_steps} "
                      f"after the {n_prompt}-token prompt, 0.8B shape; weight decode to fp64 took {t_load:.1f} s "
                      f"(not timed); host os.cpu_count()={os.cpu_count()}",
            "prefill": {"value": round(n_prompt / t_pre, 2), "unit": "tok/s", "workload": f"pp{n_prompt}",
                        "s": round(t_pre, 2), "form": "whole-sequence (batched matmuls, parallel DeltaNet, "
                                                       "full causal scores), logits of the last row"},
            "single_thread": single}


def _energy_reader():
    """A function returning the board's energy accumulator in joules (amdsmi), or an error string."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        if len(handles) != 1:
            return None, f"{len(handles)} GPUs visible to amdsmi; cannot tell which one runs the kernel"
        h = handles[0]

        def read():
            e = amdsmi.amdsmi_get_energy_count(h)
            return e["energy_accumulator"] * e["counter_resolution"] * 1e-6, e["timestamp"]
        read()
        return read, None
    except Exception as ex:  # no amdsmi, no permission, no counter on this board
        return None, f"energy counter unavailable: {type(ex).__name__}: {ex}"


def energy_leg(m, prompt, tok, n_steps: int, min_seconds: float = 4.0) -> dict:
    """Tokens per joule of the decode loop from the board energy accumulator (whole board, idle
    power included).  The accumulator advances in coarse steps, so the window spans at least
    min_seconds: rounds of (512-token prefill, n_steps one-launch decode steps), repeated.  The
    prefills are inside the window (about 1 % of its time) and count no tokens."""
    import torch
    read, err = _energy_reader()
    if read is None:
        return {"status": err}
    torch.cuda.synchronize()
    time.sleep(0.25)
    ei0, _ = read()
    ti0 = time.perf_counter()
    time.sleep(2.0)
    ei1, _ = read()
    idle_w = (ei1 - ei0) / (time.perf_counter() - ti0)
    e0, _ = read()
    t0 = time.perf_counter()
    steps = rounds = 0
    while time.perf_counter() - t0 < min_seconds:
        m.mk_reset()
        m.mk_prefill(prompt[:PROMPT], PROMPT, tok)
        for _ in range(n_steps):
            m.mk_decode_step(tok, tok)
        m.mk_sync()
        steps += n_steps
        rounds += 1
    t1 = time.perf_counter()
    e1, _ = read()
    joules = e1 - e0
    secs = t1 - t0
    return {"tok_per_J": round(steps / joules, 3) if joules > 0 else None,
            "avg_power_W": round(joules / secs, 1),
            "idle_power_W": round(idle_w, 1),
            "steps": steps, "rounds": rounds, "seconds": round(secs, 3),
            "context": f"positions {PROMPT}..{PROMPT + n_steps - 1}, a 512-token prefill before each round",
            "counter": "amdsmi energy accumulator, whole board"}


def long_context_leg(cfg_name: str, W, ctx: int, n_steps: int, kv: str = "f32") -> dict:
    """Decode at a long context: a ctx-token prompt through the GPU prefill, then n_steps timed
    one-launch decode steps with the KV cache that large (same weights; the cache holds the next
    multiple of 32,768 positions and stores kv: "f32", "f16" or "q8")."""
    import torch
    import synth
    from hybrid_deltanet_attention_amd import Model
    from hybrid_deltanet_attention_amd.binding import MK_F32, MK_F16, MK_Q8
    max_ctx = 32768 * ((ctx + 64 + 32767) // 32768)
    cfg = synth.get_config(cfg_name, max_ctx=max_ctx)
    dev = torch.device("cuda:0")
    m = Model(cfg, device=0, kv_dtype={"f32": MK_F32, "f16": MK_F16, "q8": MK_Q8}[kv])
    m.mk_load_weights(W)
    prompt = torch.tensor(synth.make_prompt(cfg.vocab, ctx, SEED + 7), device=dev)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    t0 = time.perf_counter()
    m.mk_prefill(prompt, ctx, tok)
    m.mk_sync()
    pre_s = time.perf_counter() - t0
    for _ in range(4):
        m.mk_decode_step(tok, tok)
    m.mk_sync()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]
    for i in range(n_steps):
        ev[i][0].record(m.stream)
        m.mk_decode_step(tok, tok)
        ev[i][1].record(m.stream)
    m.mk_sync()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    region = ev[0][0].elapsed_time(ev[-1][1]) / 1e3
    L0 = ctx + 5
    bytes_per = float(np.mean([algorithmic_bytes(cfg, L0 + i, kv=kv)["total"] for i in range(n_steps)]))
    gbs = bytes_per / (us * 1e-6) / 1e9
    m.close()
    return {"context": ctx, "kv": kv, "max_ctx": max_ctx, "prefill_s": round(pre_s, 3),
            "us_per_launch": round(us, 2), "tok_per_s": round(n_steps / region, 1), "bytes_per_launch": int(bytes_per),
            "achieved_GBs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}


def q4_27b_verify_leg(W, ctx: int, n_launch: int, k: int = 5) -> dict:
    """Speculative verify of the 27B-scale 4-bit hybrid against a long context: the pending token and k
    random drafts scored per mk_verify_k launch at position ctx of a 32,768-position binary16 KV cache
    (the pages keep fp16 KV up to about 80K).  The context is a ctx-token random prompt through the
    4-bit prefill (timed: the GEMMs on the weights expanded to BF16 high and low parts, the last
    token through one decode launch).  Random drafts are almost always rejected, so each launch
    advances one position; its cost is the same whatever is accepted."""
    import torch
    import synth
    from hybrid_deltanet_attention_amd import Model
    from hybrid_deltanet_attention_amd.binding import MK_Q4G32, MK_F16
    cfg = synth.get_config("hybrid_27b", max_ctx=32768)
    assert ctx + 4 * n_launch + 8 <= cfg.max_ctx
    m = Model(cfg, device=0, weight_dtype=MK_Q4G32, max_verify_k=k, kv_dtype=MK_F16)
    m.mk_load_weights(W)
    rng = np.random.default_rng([SEED, 21])
    dev = torch.device("cuda:0")
    prompt = torch.tensor(synth.make_prompt(cfg.vocab, ctx, SEED + 21), device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    m.mk_prefill(prompt[:64], 64, nxt)  # first-use costs out of the timing
    m.mk_sync()
    m.mk_reset()
    t0 = time.perf_counter()
    m.mk_prefill(prompt, ctx, nxt)
    m.mk_sync()
    pre_s = time.perf_counter() - t0
    print(f"[bench] 27B-scale 4-bit: {ctx}-token prefill in {pre_s:.2f} s", file=sys.stderr, flush=True)
    toks = torch.tensor(rng.integers(0, cfg.vocab, size=(n_launch + 2, k + 1)), dtype=torch.int32, device=dev)
    out = torch.zeros((n_launch + 2, k + 1), dtype=torch.int32, device=dev)
    acc = torch.zeros(n_launch + 2, dtype=torch.int32, device=dev)
    for i in range(2):
        m.mk_verify_k(toks[i], k, out[i], acc[i:i + 1])
    m.mk_sync()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_launch)]
    torch.cuda.synchronize()
    for i in range(n_launch):
        ev[i][0].record(m.stream)
        m.mk_verify_k(toks[i + 2], k, out[i + 2], acc[i + 2:i + 3])
        ev[i][1].record(m.stream)
    m.mk_sync()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    a = acc[2:].cpu().numpy()
    # algorithmic bytes of a pass: the weights once, the KV cache read at ~ctx positions, the DeltaNet
    # state read and written; the k state snapshots the rollback needs are written as well
    b = algorithmic_bytes(cfg, ctx + k + 1, 0.625, kv="f16")
    snaps = k * b["state"] // 2
    bytes_pass = b["total"]
    gbs = bytes_pass / (us * 1e-6) / 1e9
    # plain decode launches at the same context (one position each)
    for _ in range(2):
        m.mk_decode_step(nxt, nxt)
    m.mk_sync()
    n_dec = 16
    evd = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_dec)]
    torch.cuda.synchronize()
    for i in range(n_dec):
        evd[i][0].record(m.stream)
        m.mk_decode_step(nxt, nxt)
        evd[i][1].record(m.stream)
    m.mk_sync()
    torch.cuda.synchronize()
    us_dec = float(np.mean([x.elapsed_time(y) for x, y in evd])) * 1e3
    p_dec = m.mk_get_position() - n_dec // 2
    bytes_dec = algorithmic_bytes(cfg, p_dec, 0.625, kv="f16")["total"]
    m.close()
    return {"workload": f"hybrid_27b 4-bit verify, pending token + {k} random drafts at position {ctx} "
                        f"(32,768-position binary16 KV cache, context from a {ctx}-token 4-bit prefill)",
            "prefill_s": round(pre_s, 2), "prefill_tok_per_s": round(ctx / pre_s, 1),
            "us_per_pass": round(us, 1), "positions_per_pass": k + 1, "mean_accepted": round(float(a.mean()), 3),
            "tok_per_s_measured": round(float((a + 1).sum()) / (n_launch * us * 1e-6), 1),
            "tok_per_s_all_accepted": round((k + 1) / (us * 1e-6), 1), "launches": n_launch,
            "bytes_per_pass": int(bytes_pass), "snapshot_bytes": int(snaps), "achieved_GBs": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "decode_at_context": {"position": int(p_dec), "us_per_launch": round(us_dec, 1),
                                  "tok_per_s": round(1e6 / us_dec, 1), "bytes_per_launch": int(bytes_dec),
                                  "frac": round(bytes_dec / (us_dec * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}}


def q4_27b_leg(ctx: int, n_steps: int, verify_ctx: int = 30000) -> dict:
    """The 27B-scale hybrid from 4-bit Q4G32 weights (64 layers, hidden 5120, 0.625 B per weight,
    14.08 GB): a ctx-token random prompt through the decode kernel (one launch per token), then
    n_steps timed one-launch decode steps.  Weights are drawn in the storage format (seeded)."""
    import torch
    import synth
    from hybrid_deltanet_attention_amd import Model
    from hybrid_deltanet_attention_amd.binding import MK_Q4G32
    cfg = synth.get_config("hybrid_27b", max_ctx=2048)
    assert ctx + n_steps + 8 <= cfg.max_ctx
    print(f"[bench] 27B-scale 4-bit: generating weights", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    W = synth.make_q4_weights(cfg, SEED)
    gen_s = time.perf_counter() - t0
    m = Model(cfg, device=0, weight_dtype=MK_Q4G32)
    m.mk_load_weights(W)
    print(f"[bench] 27B-scale 4-bit: weights drawn in {gen_s:.1f} s and loaded", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    prompt = torch.tensor(synth.make_prompt(cfg.vocab, ctx, SEED + 11), device=dev)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    m.mk_prefill(prompt[:64], 64, tok)  # first-use costs out of the timing
    m.mk_sync()
    m.mk_reset()
    t0 = time.perf_counter()
    m.mk_prefill(prompt, ctx, tok)
    m.mk_sync()
    pre_s = time.perf_counter() - t0
    for _ in range(4):
        m.mk_decode_step(tok, tok)
    m.mk_sync()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]
    torch.cuda.synchronize()
    for i in range(n_steps):
        ev[i][0].record(m.stream)
        m.mk_decode_step(tok, tok)
        ev[i][1].record(m.stream)
    m.mk_sync()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    region = ev[0][0].elapsed_time(ev[-1][1]) / 1e3
    L0 = ctx + 5
    bytes_per = float(np.mean([algorithmic_bytes(cfg, L0 + i, 0.625)["total"] for i in range(n_steps)]))
    gbs = bytes_per / (us * 1e-6) / 1e9
    m.close()
    del m
    torch.cuda.empty_cache()
    ver = None
    if verify_ctx > 0:
        print(f"[bench] 27B-scale 4-bit: verify at position {verify_ctx}", file=sys.stderr, flush=True)
        ver = q4_27b_verify_leg(W, verify_ctx, 16)
    del W
    return {"workload": f"hybrid_27b 4-bit (Q4G32) batch-1 decode after a {ctx}-token prompt",
            "layers": cfg.n_layers, "hidden": cfg.hidden, "ffn": cfg.ffn, "weights_GB": 14.08,
            "prompt_s": round(pre_s, 3), "prompt_tok_per_s": round(ctx / pre_s, 1), "us_per_launch": round(us, 2), "tok_per_s": round(n_steps / region, 1),
            "steps": n_steps, "bytes_per_launch": int(bytes_per), "achieved_GBs": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "verify": ver}


def verify_leg(cfg, W, m_dec, prompt, tok, k: int, n_launch: int) -> dict:
    """mk_verify_k timing at the decode workload: the pending token and k drafts per launch, after the
    512-token prompt.  Greedy drafts are the model's own continuation (from decode launches), so every
    launch accepts all k; random drafts are almost always rejected.  Tokens are prepared on the
    device before the timed loop, so the launches run back to back."""
    import torch
    from hybrid_deltanet_attention_amd import Model
    dev = torch.device("cuda:0")
    # greedy continuation g[0..]: g[0] is the pending token after the prompt
    m_dec.mk_reset()
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    m_dec.mk_prefill(prompt[:PROMPT], PROMPT, nxt)
    n_g = (k + 1) * n_launch
    g = torch.zeros(n_g, dtype=torch.int32, device=dev)
    g[0:1].copy_(nxt)
    for i in range(1, n_g):
        m_dec.mk_decode_step(g[i - 1:i], g[i:i + 1])
    m_dec.mk_sync()
    mv = Model(cfg, device=0, max_verify_k=k)
    mv.mk_load_weights(W)
    stream = mv.stream
    out = torch.zeros((n_launch, k + 1), dtype=torch.int32, device=dev)
    acc = torch.zeros(n_launch, dtype=torch.int32, device=dev)
    rnd = torch.tensor(np.random.default_rng([SEED, 2]).integers(0, cfg.vocab, size=(n_launch, k + 1)),
                       dtype=torch.int32, device=dev)
    res = {}
    for label, src in (("greedy_drafts", None), ("random_drafts", rnd)):
        mv.mk_reset()
        mv.mk_prefill(prompt[:PROMPT], PROMPT, nxt)
        for i in range(2):  # warm-up launches, then back to the prompt's end
            mv.mk_verify_k(g[0:k + 1], k, out[0], acc[0:1])
        mv.mk_reset()
        mv.mk_prefill(prompt[:PROMPT], PROMPT, nxt)
        mv.mk_sync()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_launch)]
        torch.cuda.synchronize()
        for i in range(n_launch):
            toks = g[i * (k + 1):(i + 1) * (k + 1)] if src is None else src[i]
            ev[i][0].record(stream)
            mv.mk_verify_k(toks, k, out[i], acc[i:i + 1])
            ev[i][1].record(stream)
        mv.mk_sync()
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
        region = ev[0][0].elapsed_time(ev[-1][1]) / 1e3
        a = acc.cpu().numpy()
        emitted = int((a + 1).sum())
        res[label] = {"us_per_launch": round(us, 2), "mean_accepted": round(float(a.mean()), 3),
                      "tok_per_s": round(emitted / region, 1), "launches": n_launch}
        if src is None:
            res[label]["all_accepted"] = bool((a == k).all())
    mv.close()
    return {"k": k, "positions_per_launch": k + 1, "context": f"after the {PROMPT}-token prompt", **res}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_line(cfg, pp_s: float) -> dict:
    f = prefill_flops(cfg, PP)
    weight_bytes = algorithmic_bytes(cfg, 0)["weights"] + algorithmic_bytes(cfg, 0)["lm_head"]
    achieved = f["total"] / pp_s / 1e12
    return {"workload": f"pp{PP}", "value": round(PP / pp_s, 1), "unit": "tok/s", "ms": round(pp_s * 1e3, 3),
            "roofline": {"bound": "mfma", "dtype": "bf16", "achieved": round(achieved, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                         "gflop": round(f["total"] / 1e9, 2),
                         "gflop_parts": {k: round(v / 1e9, 3) for k, v in f.items() if k != "total"},
                         "hbm_floor_us": round(weight_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 1)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the pp520 prefill timing (profiling runs)")
    ap.add_argument("--config", default="hybrid_0p8b")
    ap.add_argument("--long-context", type=int, default=30000,
                    help="prompt length of the long-context decode legs: a binary16 cache at this length and an "
                         "int8 cache at 96,000 positions (the pages keep fp16 to about 80K, 8-bit above); 0 skips them")
    ap.add_argument("--verify-k", type=int, default=5, help="drafts per mk_verify_k launch in the verify leg; 0 skips it")
    ap.add_argument("--q4-steps", type=int, default=64,
                    help="timed decode steps of the 27B-scale 4-bit leg (1,024-token prompt); 0 skips it")
    ap.add_argument("--energy-steps", type=int, default=1280,
                    help="decode steps of the energy (tok/J) leg; 0 skips it")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (reference for rocprofv3 byte counters)")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_DIR", "TRACE_DIR"),
                    help="matrix-core counter summary of the prefill kernels from a rocprofv3 --pmc folder and a "
                         "--kernel-trace --stats folder of the same command")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn four rocprofv3 --pmc output folders into the traffic summary JSON")
    args = ap.parse_args()
    if args.summarize_mfma:
        print(summarize_mfma(*args.summarize_mfma))
        return
    if args.summarize_pmc:
        f, w, cf, cw = args.summarize_pmc
        print(json.dumps(summarize_pmc({"fetch": f, "write": w, "copy_fetch": cf, "copy_write": cw}), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the decode path is batch-1 on a single device and "
              "this build has no multi-GPU path (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from hybrid_deltanet_attention_amd import Model

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    cfg = synth.get_config(args.config)
    assert PROMPT + args.warmup + args.steps <= cfg.max_ctx and PP + 1 <= cfg.max_ctx
    print(f"[bench] generating {cfg.name} weights (seed {SEED})", file=sys.stderr, flush=True)
    W = synth.make_weights(cfg, SEED)
    m = Model(cfg, device=0)
    m.mk_load_weights(W)
    stream = m.stream
    dev = torch.device("cuda:0")
    prompt = torch.tensor(synth.make_prompt(cfg.vocab, PP, SEED), device=dev)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)

    # ---- prefill pp520 (fresh context each time), median of 3 after one warm run
    pp_times = []
    for r in range(0 if args.no_prefill else 4):
        m.mk_reset()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        m.mk_prefill(prompt, PP, tok)
        e1.record(stream)
        m.mk_sync()
        if r:
            pp_times.append(e0.elapsed_time(e1) / 1e3)
    pp_s = float(np.median(pp_times)) if pp_times else float("nan")
    print(f"[bench] prefill pp{PP}: {PP / pp_s:.0f} tok/s", file=sys.stderr, flush=True)

    # ---- decode: 512-token prompt, W warm-up steps, K timed steps (token fed back on device)
    m.mk_reset()
    m.mk_prefill(prompt[:PROMPT], PROMPT, tok)
    for _ in range(args.warmup):
        m.mk_decode_step(tok, tok)
    m.mk_sync()
    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        starts[i].record(stream)
        m.mk_decode_step(tok, tok)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    m.mk_sync()
    per_launch = [s.elapsed_time(e) / 1e3 for s, e in zip(starts, ends)]
    region = starts[0].elapsed_time(ends[-1]) / 1e3
    avg_launch = float(np.mean(per_launch))
    L0 = PROMPT + args.warmup + 1
    bytes_per = np.mean([algorithmic_bytes(cfg, L0 + i)["total"] for i in range(K)])
    achieved = bytes_per / avg_launch / 1e9
    tok_s = K / region
    print(f"[bench] decode: {tok_s:.0f} tok/s, {avg_launch * 1e6:.1f} us/launch, "
          f"{achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of 8 TB/s), wall {wall:.3f}s",
          file=sys.stderr, flush=True)

    stream_ref = stream_reference()
    print(f"[bench] streaming reference: {stream_ref}", file=sys.stderr, flush=True)

    out = {
        "metric": "batch-1 decode tok/s + % HBM roofline (0.8B hybrid bf16); pp520 prefill tok/s",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(region / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} batch-1 decode after a {PROMPT}-token prompt, one launch per token",
                   "layers": cfg.n_layers, "deltanet_layers": cfg.n_deltanet_layers,
                   "attention_layers": cfg.n_attention_layers, "hidden": cfg.hidden, "ffn": cfg.ffn,
                   "vocab": cfg.vocab, "weights": "bf16 N(0,0.02) seed 0", "prompt_tokens": PROMPT,
                   "grid_workgroups": m.mk_get_grid()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "bytes_per_launch": int(bytes_per), "avg_launch_us": round(avg_launch * 1e6, 2),
                     "measured_stream": stream_ref,
                     "frac_of_measured_stream": round(achieved / stream_ref["best"], 4)},
        "prefill": None if not pp_times else prefill_line(cfg, pp_s),
        "launches_per_token": 1,
    }
    if args.verify_k > 0:
        out["verify"] = verify_leg(cfg, W, m, prompt, tok, args.verify_k, 64)
        out["verify"]["decode_us_per_launch"] = round(avg_launch * 1e6, 2)
        print(f"[bench] verify: {out['verify']}", file=sys.stderr, flush=True)
    if args.long_context > 0:
        out["long_context"] = [long_context_leg(args.config, W, min(args.long_context, 32768 - 64), 32, "f16"),
                               long_context_leg(args.config, W, 96000, 32, "q8")]
        print(f"[bench] long context: {out['long_context']}", file=sys.stderr, flush=True)
    if args.energy_steps > 0:
        n_e = min(args.energy_steps, cfg.max_ctx - PROMPT)
        out["energy"] = energy_leg(m, prompt, tok, n_e)
        print(f"[bench] energy: {out['energy']}", file=sys.stderr, flush=True)
    m.close()
    del m
    torch.cuda.empty_cache()
    if args.q4_steps > 0:
        out["q4_27b"] = q4_27b_leg(1024, args.q4_steps)
        print(f"[bench] 27B-scale 4-bit: {out['q4_27b']}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, W)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

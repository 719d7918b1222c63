// Batch-1 decode step of the hybrid Gated-DeltaNet + attention decoder as ONE persistent kernel
// launch on gfx950 (luce-megakernel announcement, page 1: the whole forward in one dispatch, a
// grid-wide sync instead of kernel boundaries, BF16 weights with FP32 accumulation, the DeltaNet
// recurrence in FP32 registers, QKV + RoPE + causal softmax + output projection fused).
//
// Grid: one 512-lane workgroup per compute unit (regular launch; one workgroup fits per CU and the
// grid is no larger than the CU count, so all workgroups are resident together).  Inside a
// workgroup, waves 0..3 stream (every weight, state and KV copy), waves 4..7 poll exchange
// records, and all eight compute out of LDS (the polling waves also update the DeltaNet state rows
// and store their rows and records, and every wave forms a share of the attention P.V).
//
// Exchanges between phases use no barrier, fence or counter.  A phase publishes its outputs as
// 8-byte records (FP32 value, launch epoch) with device-coherent stores; the next phase polls
// exactly the records it needs until their epoch matches.  Each record is written once per launch,
// so nothing is ever cleared.  Per DeltaNet layer there are five exchanges (in-projection, mixer
// output, residual, FFN hidden, residual), per attention layer six (plus the split-K partials).
//
// Weights never depend on activations, so each phase's weights are copied global -> LDS with
// asynchronous LDS-DMA before the workgroup waits for the phase's inputs; the copies run during
// the exchange latency.  A streaming wave waits for exactly the copies it needs (vmcnt counts
// loads, stores and LDS-DMA in issue order), and workgroup barriers order LDS only, so copies for
// later phases stay in flight across them.  Every wait is bounded: a wait that gives up sets
// ctl->err and every workgroup leaves the kernel.

#include "mk_device.h"

constexpr int ATT_PASS = MK_ATT_PASS;

namespace {

// ------------------------------------------------------------------------------------------
// the megakernel.  The body is compiled once per model shape it is specialised for (every size a
// compile-time constant, so divisions and trip counts fold) and once generically (sizes read from
// the parameters); the host picks the instance that matches the model.
// ------------------------------------------------------------------------------------------
template <int D_, int FFN_, int H_, int DK_, int DV_, int NQ_, int NKV_, int HD_, int KVT>
__device__ __forceinline__ void decode_body(const MkDecodeParams& p0) {
  // Every wave at the highest issue priority.  Measured on the 0.8B shape: 579 -> 568 us per token,
  // the same whether only the streaming waves, only the polling waves, or all of them are raised
  // (priority 3 / 1, 2 / 1, 3 / 2, 3 / 3: 570-571 us), so the relative order of the two roles is
  // not what it changes; the 4-bit decode and the verify kernels measured no faster with it.
  __builtin_amdgcn_s_setprio(3);
  MkDecodeParams p = p0;
  // each instance serves one KV cache type and compiles only that type's row code
  p.kvt = KVT;
  if (D_) p.D = D_;
  if (FFN_) p.ffn = FFN_;
  if (H_) p.H = H_;
  if (DK_) p.dk = DK_;
  if (DV_) p.dv = DV_;
  if (NQ_) p.nq = NQ_;
  if (NKV_) p.nkv = NKV_;
  if (HD_) p.hd = HD_;
  extern __shared__ float lds_raw[];
  LS float* lds = (LS float*)lds_raw;
  const int NW = (int)gridDim.x, w = (int)blockIdx.x;
  Lds s;
  s.desc = (LS MkLayerDev*)(lds + p.lds_desc);
  s.gain = (LS uint16_t*)(lds + p.lds_gain);
  s.rope = lds + p.lds_rope;
  s.x = lds + p.lds_x;
  s.xn = (LS u32*)(lds + p.lds_xn);
  s.vec = lds + p.lds_vec;
  s.att = lds + p.lds_att;
  s.att_cap = MK_RED_CAP;
  s.scr = lds + p.lds_scr;
  s.flag = (LS int*)(lds + p.lds_flag);
  s.stA = (LS u32x4*)g_stage;
  s.stB = (LS u32x4*)g_stage + MK_STAGE_A_SLOTS * SLOT;
  s.a_slots = MK_STAGE_A_SLOTS;
  const int D = p.D;

  Ctx cx;
  cx.ctl = p.ctl;
  cx.epoch = p.ctl->step;
  const int pos = p.ctl->pos;
  const int tok = p.tok[0];
  // a bad token id or a full context is reported through ctl->err; every workgroup sees the same
  // values, so all of them leave before touching memory
  if (tok < 0 || tok >= p.vocab || pos < 0 || pos >= p.max_ctx) {
    if (w == 0 && tid() == 0) set_err(cx, 2u);
    return;
  }
  Tracer tr{(LS unsigned long long*)(lds + p.lds_trace), p.trace ? p.trace + (size_t)w * MK_TRACE_EVENTS : nullptr,
            0};
  tr.mark();

  // launch-start loads (nothing else is in flight yet): descriptors, embedding row, RoPE row,
  // layer 0's gains
  {
    const int nw = p.n_layers * (int)(sizeof(MkLayerDev) / 4);
    const MK_G u32* dsrc = (const MK_G u32*)p.layers;
    for (int i = tid(); i < nw; i += MK_NT) ((LS u32*)s.desc)[i] = dsrc[i];
    for (int i = tid(); i < D; i += MK_NT) s.x[i] = bf16f(p.embed[(size_t)tok * D + i]);
    const int half = p.hd / 2;
    for (int i = tid(); i < half; i += MK_NT) {
      s.rope[i] = p.rope_cos[(size_t)pos * half + i];
      s.rope[half + i] = p.rope_sin[(size_t)pos * half + i];
    }
    for (int i = tid(); i < 2 * D; i += MK_NT) s.gain[i] = p.gain0[i];
    if (tid() == 0) *s.flag = 0;
  }
  wg_bar();

  // this workgroup's rows of the residual-sized projections (out-projection, down projection)
  const int d0 = split(D, NW, w), d1 = split(D, NW, w + 1);
  // FFN hidden range (gate/up row pairs)
  const int j0 = split(p.ffn, NW, w), j1 = split(p.ffn, NW, w + 1);

  // layer 0's input rows go out first
  Gemv gin;
  int P0, P1;
  {
    const MkLayerDev L0 = layer_desc(s.desc, 0);
    pair_range(L0.rows_in, NW, w, P0, P1);
    gin.init(L0.w_in + (size_t)2 * P0 * D, min(2 * P1, L0.rows_in) - 2 * P0, D);
    gemv_stage(gin, s.stA, A_UNITS);
    if (streamer()) wait_vm<0>();
  }
  wg_bar();

  for (int l = 0; l < p.n_layers; ++l) {
    const MkLayerDev L = layer_desc(s.desc, l);
    const LS uint16_t* gl = s.gain + (size_t)(l & 1) * 2 * D;
    // stage A holds this layer's input rows (waited for before the barrier that ended the last gather)
    rmsnorm(s.x, gl, s.xn, D, p.rms_eps, tr);
    tr.mark();
    int K;  // mixer output width
    Gemv gout, ggu;
    ggu.init(L.w_gu + (size_t)2 * j0 * D, 2 * (j1 - j0), D);
    int cntA;
    if (L.kind == MK_LAYER_DN) {
      K = p.H * p.dv;
      MK_G mk_u64* dst = L.ll_in + 2 * P0;
      gemv<false, false, false>(gin, s.xn, s.stA, A_UNITS, s.att, tr,
                                [&](int r, float v, float) { ll_put(dst + r, cx.epoch, v); });
      tr.mark();
      // state rows and the out-projection units -> stage B; gate/up units -> stage A
      const int s0 = split(K, NW, w), s1 = split(K, NW, w + 1);
      const int rps = 64 / (p.dk >> 2);
      const int sslots = min((s1 - s0 + rps - 1) / rps, MK_STAGE_B_SLOTS / 2);
      const int boff = (sslots + 3) & ~3;
      gout.init(L.w_out + (size_t)d0 * K, d1 - d0, K);
      state_stage(p, L, s0, s1, s.stB, sslots);
      gemv_stage(gout, s.stB + boff * SLOT, (MK_STAGE_B_SLOTS - boff) / USLOTS);
      // the polling waves update the state rows while the streaming waves issue the gate/up
      // units -> stage A (free since the in-projection)
      cntA = 0;
      if (!dn_state<true>(p, L, cx, s, s0, s1, sslots, 0, tr, [&] { cntA = gemv_stage(ggu, s.stA, A_UNITS); }))
        return;
      tr.mark();
      // mixer output -> out-projection rows + residual -> records
      {
        const bool ok = gather_vec(cx, L.ll_o, K, s.vec);
        if (wg_bar_or(s, !ok)) return;
        to_hl(s.vec, K);
        wg_bar();
      }
      tr.mark();
      gemv<false, false, false>(gout, (const LS u32*)s.vec, s.stB + boff * SLOT, (MK_STAGE_B_SLOTS - boff) / USLOTS, s.att, tr,
                                [&](int r, float v, float) { ll_put(L.ll_x1 + d0 + r, cx.epoch, s.x[d0 + r] + v); });
    } else {
      K = p.nq * p.hd;
      att_qkv(p, L, cx, s, gin, P0, pos, tr);
      tr.mark();
      // K/V rows of the first chunks of the work items -> stage A (free until the gate/up units),
      // the out-projection units -> stage B.  Compact caches whose chunk buffers fit 2 ATT_PASS
      // times in stage A take their chunks ATT_PASS at a time (att_items_multi).
      const int boff = 0;
      const bool multi = KVT != MK_KV_F32 && 2 * ATT_PASS * kv_buf_slots(p.hd, p.kvt) <= s.a_slots;
      const int first = multi ? ATT_PASS : max(1, kv_nbuf(p.hd, p.kvt, s.a_slots) - 1);
      for (int kc = 0; kc < first; ++kc) {
        const int cn = att_chunk_at(p, NW, w, pos, kc);
        if (cn >= 0) kv_stage(p, L, cn, pos, s.stA + kc * kv_buf_slots(p.hd, p.kvt) * SLOT);
      }
      gout.init(L.w_out + (size_t)d0 * K, d1 - d0, K);
      gemv_stage(gout, s.stB + boff * SLOT, (MK_STAGE_B_SLOTS - boff) / USLOTS);
      if (multi ? !att_items_multi<ATT_PASS>(p, L, cx, s, NW, w, pos, 0, tr) : !att_items(p, L, cx, s, NW, w, pos, 0, tr))
        return;
      cntA = gemv_stage(ggu, s.stA, A_UNITS);
      tr.mark();
      const int o0 = split(K, NW, w), o1 = split(K, NW, w + 1);
      if (!att_combine(p, L, cx, s, o0, o1, pos)) return;
      tr.mark();
      {
        const bool ok = gather_vec(cx, L.ll_o, K, s.vec);
        if (wg_bar_or(s, !ok)) return;
        to_hl(s.vec, K);
        wg_bar();
      }
      tr.mark();
      gemv<false, false, false>(gout, (const LS u32*)s.vec, s.stB + boff * SLOT, (MK_STAGE_B_SLOTS - boff) / USLOTS, s.att, tr,
                                [&](int r, float v, float) { ll_put(L.ll_x1 + d0 + r, cx.epoch, s.x[d0 + r] + v); });
    }
    tr.mark();
    // down-projection units and the next layer's (or the final) gains -> stage B
    Gemv gdn;
    gdn.init(L.w_down + (size_t)d0 * p.ffn, d1 - d0, p.ffn);
    const int cntB = gemv_stage(gdn, s.stB, MK_STAGE_B_SLOTS / USLOTS);
    {
      const bool ok = gather_vec(cx, L.ll_x1, D, s.x);
      if (streamer()) wait_vm_n(cntB);  // gate/up units (stage A)
      if (wg_bar_or(s, !ok)) return;
    }
    tr.mark();
    rmsnorm(s.x, gl + D, s.xn, D, p.rms_eps, tr);
    gemv<true, false, false>(ggu, s.xn, s.stA, A_UNITS, s.att, tr, [&](int j, float gv, float uv) {
      ll_put(L.ll_h + j0 + j, cx.epoch, gv / (1.0f + expf(-gv)) * uv);
    });
    tr.mark();
    // next layer's input rows (or the LM head's) -> stage A
    const MK_G uint16_t* Ln_g12 = nullptr;
    if (l + 1 < p.n_layers) {
      const MkLayerDev Ln = layer_desc(s.desc, l + 1);
      pair_range(Ln.rows_in, NW, w, P0, P1);
      gin.init(Ln.w_in + (size_t)2 * P0 * D, min(2 * P1, Ln.rows_in) - 2 * P0, D);
      Ln_g12 = Ln.g12;
    } else {
      pair_range(p.vocab, NW, w, P0, P1);
      gin.init(p.embed + (size_t)2 * P0 * D, min(2 * P1, p.vocab) - 2 * P0, D);
    }
    cntA = gemv_stage(gin, s.stA, A_UNITS);
    {
      // the next layer's gains (or the final norm's) ride along with the FFN hidden poll
      const MK_G uint16_t* gsrc = l + 1 < p.n_layers ? Ln_g12 : p.g_final;
      const int gn = (l + 1 < p.n_layers ? 2 : 1) * D;
      GainCopy gc;
      if (!streamer()) gains_issue(gsrc, gn, gc);
      const bool ok = gather_hl(cx, L.ll_h, p.ffn, (LS u32*)s.vec);
      if (!streamer()) gains_store(gsrc, gn, gc, s.gain + (size_t)((l + 1) & 1) * 2 * D);
      if (streamer()) wait_vm_n(cntA);  // down units (stage B)
      if (wg_bar_or(s, !ok)) return;
    }
    tr.mark();
    gemv<false, false, false>(gdn, (const LS u32*)s.vec, s.stB, MK_STAGE_B_SLOTS / USLOTS, s.att, tr,
                              [&](int r, float v, float) { ll_put(L.ll_x2 + d0 + r, cx.epoch, s.x[d0 + r] + v); });
    tr.mark();
    {
      const bool ok = gather_vec(cx, L.ll_x2, D, s.x);
      if (streamer()) wait_vm<0>();  // next input rows (stage A)
      if (wg_bar_or(s, !ok)) return;
    }
    tr.mark();
  }

  // final norm + tied LM head + argmax (lowest index among equal maxima)
  rmsnorm(s.x, s.gain + (size_t)(p.n_layers & 1) * 2 * D, s.xn, D, p.rms_eps, tr);
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  const int v0 = 2 * P0;
  gemv<false, true, true>(gin, s.xn, s.stA, A_UNITS, s.att, tr, [&](int r, float v, float) {
    const int idx = v0 + r;
    if (p.logits) p.logits[idx] = v;
    if (v > best || (v == best && idx < bidx)) {
      best = v;
      bidx = idx;
    }
  });
  tr.mark();
  // workgroup argmax: fixed tree over lanes then waves in order
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ob = __shfl_xor(best, m, 64);
    const int oi = __shfl_xor(bidx, m, 64);
    if (ob > best || (ob == best && oi < bidx)) {
      best = ob;
      bidx = oi;
    }
  }
  if (lane() == 0) {
    s.scr[wave()] = best;
    s.scr[MK_NWAVE + wave()] = __int_as_float(bidx);
  }
  wg_bar();
  if (tid() == 0) {
    for (int i = 0; i < MK_NWAVE; ++i) {
      const float ob = s.scr[i];
      const int oi = __float_as_int(s.scr[MK_NWAVE + i]);
      if (ob > best || (ob == best && oi < bidx)) {
        best = ob;
        bidx = oi;
      }
    }
    ll_put(p.ll_am + 2 * w, cx.epoch, best);
    ll_put(p.ll_am + 2 * w + 1, cx.epoch, __int_as_float(bidx));
  }
  tr.mark();
  if (w != 0) {
    tr.flush();
    return;
  }
  // workgroup 0 reduces the per-workgroup winners and publishes the token
  {
    const bool ok = gather_vec(cx, p.ll_am, 2 * NW, s.vec);
    if (wg_bar_or(s, !ok)) return;
  }
  if (wave() == 0) {
    float b;
    int bi;
    wave_argmax(s.vec, NW, b, bi);
    if (lane() == 0) {
      p.next[0] = bi;
      p.ctl->pos = pos + 1;
      p.ctl->step = cx.epoch + 1u;
    }
  }
  tr.mark();
  tr.flush();
}

}  // namespace

// generic shape
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_kernel(MkDecodeParams p) {
  decode_body<0, 0, 0, 0, 0, 0, 0, 0, MK_KV_F32>(p);
}
// hidden 1024, FFN 3584, 16 DeltaNet heads of 128, 8 Q / 2 KV heads of 128 (the 0.8B-shaped hybrid)
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_kernel_h1024(MkDecodeParams p) {
  decode_body<1024, 3584, 16, 128, 128, 8, 2, 128, MK_KV_F32>(p);
}
// hidden 256, FFN 768, 4 DeltaNet heads of 64, 4 Q / 2 KV heads of 64 (the tiny hybrid)
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_kernel_h256(MkDecodeParams p) {
  decode_body<256, 768, 4, 64, 64, 4, 2, 64, MK_KV_F32>(p);
}
// binary16 and int8 KV caches: generic shape, and the 0.8B-shaped hybrid
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_kernel_f16(MkDecodeParams p) {
  decode_body<0, 0, 0, 0, 0, 0, 0, 0, MK_KV_F16>(p);
}
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_kernel_q8(MkDecodeParams p) {
  decode_body<0, 0, 0, 0, 0, 0, 0, 0, MK_KV_Q8>(p);
}
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_kernel_h1024_f16(MkDecodeParams p) {
  decode_body<1024, 3584, 16, 128, 128, 8, 2, 128, MK_KV_F16>(p);
}
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_kernel_h1024_q8(MkDecodeParams p) {
  decode_body<1024, 3584, 16, 128, 128, 8, 2, 128, MK_KV_Q8>(p);
}

namespace {
template <int D_, int FFN_, int H_, int DK_, int DV_, int NQ_, int NKV_, int HD_>
bool shape_is(const MkDecodeParams& p) {
  return p.D == D_ && p.ffn == FFN_ && p.H == H_ && p.dk == DK_ && p.dv == DV_ && p.nq == NQ_ && p.nkv == NKV_ &&
         p.hd == HD_;
}
typedef void (*DecodeKernel)(MkDecodeParams);
DecodeKernel pick_kernel(const MkDecodeParams& p) {
  const bool h1024 = shape_is<1024, 3584, 16, 128, 128, 8, 2, 128>(p);
  if (p.kvt == MK_KV_F16) return h1024 ? mk_decode_kernel_h1024_f16 : mk_decode_kernel_f16;
  if (p.kvt == MK_KV_Q8) return h1024 ? mk_decode_kernel_h1024_q8 : mk_decode_kernel_q8;
  if (h1024) return mk_decode_kernel_h1024;
  if (shape_is<256, 768, 4, 64, 64, 4, 2, 64>(p)) return mk_decode_kernel_h256;
  return mk_decode_kernel;
}
}  // namespace

// ------------------------------------------------------------------------------------------
// load-time helper kernels
// ------------------------------------------------------------------------------------------
__global__ void mk_permute_rows_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                       const int32_t* __restrict__ perm, int64_t rows, int64_t cols) {
  // dst row perm[r] <- src row r
  const int64_t r = blockIdx.x;
  if (r >= rows) return;
  const uint16_t* s = src + r * cols;
  uint16_t* d = dst + (int64_t)perm[r] * cols;
  for (int64_t c = threadIdx.x; c < cols; c += blockDim.x) d[c] = s[c];
}

__global__ void mk_zero_kernel(uint32_t* __restrict__ dst, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = 0u;
}

__global__ void mk_set_ctl_kernel(MkCtl* ctl, int32_t pos, int reset_err, int bump_step) {
  if (threadIdx.x == 0) {
    if (pos >= 0) ctl->pos = pos;
    if (ctl->step == 0u) ctl->step = 1u;
    if (bump_step) ctl->step += 1u;
    if (reset_err) ctl->err = 0u;
  }
}

extern "C" int mk_launch_decode(const MkDecodeParams* p, int n_wg, void* stream) {
  hipLaunchKernelGGL(pick_kernel(*p), dim3(n_wg), dim3(MK_NT), (size_t)p->lds_floats * 4, (hipStream_t)stream, *p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_launch_permute_rows(const uint16_t* src, uint16_t* dst, const int32_t* d_perm, int64_t rows,
                                      int64_t cols, void* stream) {
  if (rows <= 0) return 0;
  hipLaunchKernelGGL(mk_permute_rows_kernel, dim3((unsigned)rows), dim3(256), 0, (hipStream_t)stream, src, dst, d_perm,
                     rows, cols);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_launch_zero(void* dst, int64_t bytes, void* stream) {
  if (bytes <= 0) return 0;
  hipLaunchKernelGGL(mk_zero_kernel, dim3(1024), dim3(256), 0, (hipStream_t)stream, (uint32_t*)dst, bytes / 4);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_launch_set_ctl(MkCtl* ctl, int32_t pos, int reset_err, int bump_step, void* stream) {
  hipLaunchKernelGGL(mk_set_ctl_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, ctl, pos, reset_err, bump_step);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_decode_max_blocks_per_cu(const MkDecodeParams* p, int lds_bytes) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, pick_kernel(*p), MK_NT, lds_bytes) != hipSuccess) return 0;
  return nb;
}

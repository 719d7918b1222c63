// Batch-1 decode step of the hybrid Gated-DeltaNet + attention decoder from 4-bit block-quantised
// weights (Q4G32), as ONE persistent kernel launch on gfx950: the pages' 27B-scale system runs the
// same layer pattern from 4-bit weights, one fused launch per token (megakernel follow-up posts,
// page 3, quantisation-support and speed paragraphs; news-aggregator page, the 27B megakernel).
//
// Same grid, wave roles and exchange records as the BF16 decode kernel (mk_decode.hip).  What
// differs is sized for wide models whose weights dominate every phase:
//  * every GEMV streams its 4-bit units through registers on all eight waves (mk_q4.h); weights
//    are not staged in LDS;
//  * the LDS keeps the residual, one vector region (normalised activations, gathered mixer output
//    or FFN hidden -- never live together), the unit partials and two layer descriptors (the next
//    one is fetched by the polling waves during a gather); RMSNorm gains are read from global
//    memory;
//  * a small static stage holds the DeltaNet state rows and the split-K attention KV chunks,
//    copied with LDS-DMA before the waits that precede their use, as in the BF16 kernel.

#include "mk_q4.h"

namespace {

constexpr int Q4_STAGE_A = 32;  // KV chunk buffers (1 KB slots)
constexpr int Q4_STAGE_B = 16;  // DeltaNet state rows
__shared__ __attribute__((aligned(1024))) u32x4 g_stage_q4[(Q4_STAGE_A + Q4_STAGE_B) * SLOT];

template <int D_, int FFN_, int H_, int DK_, int DV_, int NQ_, int NKV_, int HD_>
__device__ __forceinline__ void decode_q4_body(const MkDecodeParams& p0) {
  MkDecodeParams p = p0;
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
  s.desc = (LS MkLayerDev*)(lds + p.lds_desc);  // [2]: layer l in slot l & 1
  s.gain = nullptr;
  s.rope = lds + p.lds_rope;
  s.x = lds + p.lds_x;
  s.vec = lds + p.lds_vec;
  s.xn = (LS u32*)s.vec;  // normalised activations share the vector region
  s.att = lds + p.lds_att;
  s.att_cap = Q4_RED_CAP;
  s.scr = lds + p.lds_scr;
  s.flag = (LS int*)(lds + p.lds_flag);
  s.stA = (LS u32x4*)g_stage_q4;
  s.stB = (LS u32x4*)g_stage_q4 + Q4_STAGE_A * SLOT;
  s.a_slots = Q4_STAGE_A;
  const int D = p.D;

  Ctx cx;
  cx.ctl = p.ctl;
  cx.epoch = p.ctl->step;
  const int pos = p.ctl->pos;
  const int tok = p.tok[0];
  if (tok < 0 || tok >= p.vocab || pos < 0 || pos >= p.max_ctx) {
    if (w == 0 && tid() == 0) set_err(cx, 2u);
    return;
  }
  Tracer tr{(LS unsigned long long*)(lds + p.lds_trace), p.trace ? p.trace + (size_t)w * MK_TRACE_EVENTS : nullptr,
            0};
  tr.mark();

  // launch start: the token's embedding row (decoded), the RoPE row
  q4_embed_row(p.embed, p.vocab, D, tok, s.x);
  {
    const int half = p.hd / 2;
    for (int i = tid(); i < half; i += MK_NT) {
      s.rope[i] = p.rope_cos[(size_t)pos * half + i];
      s.rope[half + i] = p.rope_sin[(size_t)pos * half + i];
    }
    if (tid() == 0) *s.flag = 0;
    const MK_G u32* dsrc = (const MK_G u32*)p.layers;
    for (int i = tid(); i < (int)(sizeof(MkLayerDev) / 4); i += MK_NT) ((LS u32*)s.desc)[i] = dsrc[i];
  }
  wg_bar();

  const int d0 = split(D, NW, w), d1 = split(D, NW, w + 1);
  const int j0 = split(p.ffn, NW, w), j1 = split(p.ffn, NW, w + 1);
  for (int l = 0; l < p.n_layers; ++l) {
    const MkLayerDev L = layer_desc(s.desc, l & 1);
    rmsnorm_gg(s.x, L.g12, s.xn, D, p.rms_eps, tr);
    tr.mark();
    int P0, P1;
    pair_range(L.rows_in, NW, w, P0, P1);
    GemvQ4 gin;
    gin.init(L.w_in, L.rows_in, 2 * P0, min(2 * P1, L.rows_in) - 2 * P0, D);
    int K;  // mixer output width
    if (L.kind == MK_LAYER_DN) {
      K = p.H * p.dv;
      MK_G mk_u64* dst = L.ll_in + 2 * P0;
      gemv_q4<false, false>(gin, s.xn, s.att, tr, [&](int r, float v, float) { ll_put(dst + r, cx.epoch, v); });
      tr.mark();
      // this workgroup's state rows -> stage B while the in-projection records travel
      const int s0 = split(K, NW, w), s1 = split(K, NW, w + 1);
      const int rps = 64 / (p.dk >> 2);
      const int sslots = min((s1 - s0 + rps - 1) / rps, Q4_STAGE_B);
      state_stage(p, L, s0, s1, s.stB, sslots);
      if (!dn_state(p, L, cx, s, s0, s1, sslots, 0, tr)) return;
      tr.mark();
    } else {
      K = p.nq * p.hd;
      att_qkv_run(p, L, cx, s, P0, pos, [&](auto epi) { gemv_q4<true, false>(gin, s.xn, s.att, tr, epi); });
      tr.mark();
      // K/V rows of the first work items -> stage A
      for (int kc = 0; kc + 1 < kv_nbuf(p.hd, s.a_slots) || kc == 0; ++kc) {
        const int cn = att_chunk_at(p, NW, w, pos, kc);
        if (cn >= 0) kv_stage(p, L, cn, pos, s.stA + kc * kv_buf_slots(p.hd) * SLOT);
      }
      if (!att_items(p, L, cx, s, NW, w, pos, 0, tr)) return;
      tr.mark();
      const int o0 = split(K, NW, w), o1 = split(K, NW, w + 1);
      if (!att_combine(p, L, cx, s, o0, o1, pos)) return;
      tr.mark();
    }
    // mixer output -> out-projection rows + residual -> records
    {
      const bool ok = gather_vec(cx, L.ll_o, K, s.vec);
      if (wg_bar_or(s, !ok)) return;
      to_hl(s.vec, K);
      wg_bar();
    }
    tr.mark();
    {
      GemvQ4 gout;
      gout.init(L.w_out, D, d0, d1 - d0, K);
      gemv_q4<false, false>(gout, (const LS u32*)s.vec, s.att, tr,
                            [&](int r, float v, float) { ll_put(L.ll_x1 + d0 + r, cx.epoch, s.x[d0 + r] + v); });
    }
    tr.mark();
    {
      // the polling threads fetch the next layer's descriptor under this gather's latency
      constexpr int NDW = (int)(sizeof(MkLayerDev) / 4);
      const int di = tid() - NCT;
      const bool fetch = !streamer() && di < NDW && l + 1 < p.n_layers;
      u32 dw = 0u;
      if (fetch) dw = ((const MK_G u32*)(p.layers + l + 1))[di];
      const bool ok = gather_vec(cx, L.ll_x1, D, s.x);
      if (fetch) ((LS u32*)(s.desc + ((l + 1) & 1)))[di] = dw;
      if (wg_bar_or(s, !ok)) return;
    }
    tr.mark();
    rmsnorm_gg(s.x, L.g12 + D, s.xn, D, p.rms_eps, tr);
    {
      GemvQ4 ggu;
      ggu.init(L.w_gu, 2 * p.ffn, 2 * j0, 2 * (j1 - j0), D);
      gemv_q4<true, false>(ggu, s.xn, s.att, tr, [&](int j, float gv, float uv) {
        ll_put(L.ll_h + j0 + j, cx.epoch, gv / (1.0f + expf(-gv)) * uv);
      });
    }
    tr.mark();
    {
      const bool ok = gather_hl(cx, L.ll_h, p.ffn, (LS u32*)s.vec);
      if (wg_bar_or(s, !ok)) return;
    }
    tr.mark();
    {
      GemvQ4 gdn;
      gdn.init(L.w_down, D, d0, d1 - d0, p.ffn);
      gemv_q4<false, false>(gdn, (const LS u32*)s.vec, s.att, tr,
                            [&](int r, float v, float) { ll_put(L.ll_x2 + d0 + r, cx.epoch, s.x[d0 + r] + v); });
    }
    tr.mark();
    {
      const bool ok = gather_vec(cx, L.ll_x2, D, s.x);
      if (wg_bar_or(s, !ok)) return;
    }
    tr.mark();
  }

  // final norm + tied LM head + argmax (lowest index among equal maxima)
  rmsnorm_gg(s.x, p.g_final, s.xn, D, p.rms_eps, tr);
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  {
    int P0, P1;
    pair_range(p.vocab, NW, w, P0, P1);
    GemvQ4 gl;
    gl.init(p.embed, p.vocab, 2 * P0, min(2 * P1, p.vocab) - 2 * P0, D);
    const int v0 = 2 * P0;
    gemv_q4<false, true>(gl, s.xn, s.att, tr, [&](int r, float v, float) {
      const int idx = v0 + r;
      if (p.logits) p.logits[idx] = v;
      if (v > best || (v == best && idx < bidx)) {
        best = v;
        bidx = idx;
      }
    });
  }
  tr.mark();
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
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_q4_kernel(MkDecodeParams p) {
  decode_q4_body<0, 0, 0, 0, 0, 0, 0, 0>(p);
}
// hidden 5120, FFN 17408, 32 DeltaNet heads of 128, 24 Q / 4 KV heads of 128 (the 27B-scale hybrid)
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_q4_kernel_h5120(MkDecodeParams p) {
  decode_q4_body<5120, 17408, 32, 128, 128, 24, 4, 128>(p);
}

namespace {
typedef void (*DecodeKernel)(MkDecodeParams);
DecodeKernel pick_q4_kernel(const MkDecodeParams& p) {
  if (p.D == 5120 && p.ffn == 17408 && p.H == 32 && p.dk == 128 && p.dv == 128 && p.nq == 24 && p.nkv == 4 &&
      p.hd == 128)
    return mk_decode_q4_kernel_h5120;
  return mk_decode_q4_kernel;
}
}  // namespace

extern "C" int mk_launch_decode_q4(const MkDecodeParams* p, int n_wg, void* stream) {
  hipLaunchKernelGGL(pick_q4_kernel(*p), dim3(n_wg), dim3(MK_NT), (size_t)p->lds_floats * 4, (hipStream_t)stream, *p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_decode_q4_max_blocks_per_cu(const MkDecodeParams* p, int lds_bytes) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, pick_q4_kernel(*p), MK_NT, lds_bytes) != hipSuccess) return 0;
  return nb;
}

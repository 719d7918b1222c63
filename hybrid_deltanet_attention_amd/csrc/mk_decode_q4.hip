// Batch-1 decode step of the hybrid Gated-DeltaNet + attention decoder from 4-bit block-quantised
// weights (Q4G32), as ONE persistent kernel launch on gfx950: the pages' 27B-scale system runs the
// same layer pattern from 4-bit weights, one fused launch per token (megakernel follow-up posts,
// page 3, quantisation-support and speed paragraphs; news-aggregator page, the 27B megakernel).
//
// Same grid, wave roles and exchange records as the BF16 decode kernel (mk_decode.hip).  What
// differs is sized for wide models whose weights dominate every phase:
//  * every GEMV streams its 4-bit units through registers on all eight waves (mk_q4.h); weights
//    are not staged in LDS.  Before each exchange the streaming waves take and load their first
//    units of the GEMV that follows it, so HBM keeps streaming while the records travel; every
//    wave then polls the residual and FFN-hidden records (the streaming waves' polls queue behind
//    their primed loads, which the GEMV needs first anyway); the mixer output, one round of polls
//    for the polling waves alone, stays with them;
//  * the LDS keeps the residual, one vector region (normalised activations, gathered mixer output
//    or FFN hidden -- never live together), the unit partials and two layer descriptors (the next
//    one is fetched by the polling waves during a gather); RMSNorm gains are read from global
//    memory;
//  * a small static stage holds the DeltaNet state rows and the split-K attention KV chunks,
//    copied with LDS-DMA before the waits that precede their use, as in the BF16 kernel.

#include "mk_q4.h"

namespace {

// Poll loads in flight per thread in the residual and FFN-hidden gathers, which every wave takes
// part in: a streaming wave's polls queue behind the units it primed for the next GEMV, whose data
// is needed right after the gather anyway, and the gathers of wide vectors then take one round of
// polls (or, for the FFN hidden vector of a 27B-scale model, two instead of five).  Measured on the
// 27B-scale shape: 4,755 us per token with the polling waves alone, 4,530 with every wave in all
// four gathers, 4,515 with 12 polls in flight for the FFN hidden gather (16: 4,556), 4,430 with
// the mixer-output gather (4,096 records: one round either way) back on the polling waves.
constexpr int Q4_PB = 8;
constexpr int Q4_PB_FFN = 12;
constexpr int Q4_STAGE_A = 32;  // KV chunk buffers (1 KB slots)
constexpr int Q4_STAGE_B = 16;  // DeltaNet state rows
__shared__ __attribute__((aligned(1024))) u32x4 g_stage_q4[(Q4_STAGE_A + Q4_STAGE_B) * SLOT];

template <int D_, int FFN_, int H_, int DK_, int DV_, int NQ_, int NKV_, int HD_, int KVT>
__device__ __forceinline__ void decode_q4_body(const MkDecodeParams& p0) {
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
  s.desc = (LS MkLayerDev*)(lds + p.lds_desc);  // [2]: layer l in slot l & 1
  s.gain = nullptr;
  s.rope = lds + p.lds_rope;
  s.x = lds + p.lds_x;
  s.vec = lds + p.lds_vec;
  s.xn = (LS u32*)s.vec;  // packed activations (q4_pack) share the vector region
  s.att = lds + p.lds_att;
  s.att_cap = Q4_RED_CAP;
  s.scr = lds + p.lds_scr;
  s.flag = (LS int*)(lds + p.lds_flag);
  s.stA = (LS u32x4*)g_stage_q4;
  s.stB = (LS u32x4*)g_stage_q4 + Q4_STAGE_A * SLOT;
  s.a_slots = Q4_STAGE_A;
  // GEMV unit counters, alternating from one GEMV to the next (in-projection, gate/up and LM head
  // on c0; out and down projections on c1), so a GEMV can be primed before the previous one's
  // counter is cleared
  LS int* c0 = s.flag + 1;
  LS int* c1 = s.flag + 2;
  Q4Ring q;
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
  q4_embed_row(p.embed, D, tok, s.x);
  {
    const int half = p.hd / 2;
    for (int i = tid(); i < half; i += MK_NT) {
      s.rope[i] = p.rope_cos[(size_t)pos * half + i];
      s.rope[half + i] = p.rope_sin[(size_t)pos * half + i];
    }
    if (tid() == 0) {
      *s.flag = 0;
      *c0 = 0;
      *c1 = 0;
    }
    const MK_G u32* dsrc = (const MK_G u32*)p.layers;
    for (int i = tid(); i < (int)(sizeof(MkLayerDev) / 4); i += MK_NT) ((LS u32*)s.desc)[i] = dsrc[i];
  }
  wg_bar();

  // row slices in whole 4-row blocks of the tiled matrices: residual-sized projections (out, down)
  // and FFN hidden pairs (one block = gate and up rows of two hidden units)
  const int d0 = 4 * split(D >> 2, NW, w), d1 = 4 * split(D >> 2, NW, w + 1);
  const int j0 = 2 * split(p.ffn >> 1, NW, w), j1 = 2 * split(p.ffn >> 1, NW, w + 1);
  // this workgroup's in-projection rows of a layer: whole 4-row blocks; P0 = first row pair
  auto in_slice = [&](const MkLayerDev& Lx, GemvQ4& g, int& P0) {
    const int nbi = (Lx.rows_in + 3) >> 2;
    const int B0 = split(nbi, NW, w), B1 = split(nbi, NW, w + 1);
    P0 = 2 * B0;
    g.init(Lx.w_in, B0, max(0, min(4 * B1, Lx.rows_in) - 4 * B0), D);
  };
  auto head_slice = [&](GemvQ4& g, int& v0) {
    const int nbv = (p.vocab + 3) >> 2;
    const int B0 = split(nbv, NW, w), B1 = split(nbv, NW, w + 1);
    v0 = 4 * B0;
    g.init(p.embed, B0, max(0, min(4 * B1, p.vocab) - 4 * B0), D);
  };
  {
    // layer 0's in-projection units, while the first norm runs
    GemvQ4 g;
    int P0;
    in_slice(layer_desc(s.desc, 0), g, P0);
    if (streamer()) gemv_q4_prime(g, c0, q);
  }
  // input-norm gains of the layer about to start: loaded ahead of the gather that precedes the norm
  Q4Gains<D_ ? (D_ / 4 + NPT - 1) / NPT : Q4_GAIN_IT> gin_g;
  gains_gg_issue(layer_desc(s.desc, 0).g12, D, gin_g);
  for (int l = 0; l < p.n_layers; ++l) {
    const MkLayerDev L = layer_desc(s.desc, l & 1);
    rmsnorm_gg(s.x, gin_g, s.vec, D, p.rms_eps, tr);
    q4_pack(s.vec, D);
    tr.mark();
    int P0;
    GemvQ4 gin;
    in_slice(L, gin, P0);
    int K;  // mixer output width
    if (L.kind == MK_LAYER_DN) {
      K = p.H * p.dv;
      MK_G mk_u64* dst = L.ll_in + 2 * P0;
      gemv_q4<false, false>(gin, s.xn, s.att, c0, q, streamer(), tr,
                            [&](int r, float v, float) { ll_put(dst + r, cx.epoch, v); });
      tr.mark();
      // this workgroup's state rows -> stage B while the in-projection records travel
      const int s0 = split(K, NW, w), s1 = split(K, NW, w + 1);
      const int rps = 64 / (p.dk >> 2);
      const int sslots = min((s1 - s0 + rps - 1) / rps, Q4_STAGE_B);
      state_stage(p, L, s0, s1, s.stB, sslots);
      if (!dn_state<false>(p, L, cx, s, s0, s1, sslots, 0, tr, [] {})) return;
      tr.mark();
    } else {
      K = p.nq * p.hd;
      att_qkv_run(p, L, cx, s, P0, pos,
                  [&](auto epi) { gemv_q4<true, false>(gin, s.xn, s.att, c0, q, streamer(), tr, epi); });
      tr.mark();
      // K/V rows of the first chunks of the work items -> stage A.  In the shape-specialised
      // instances, compact caches whose chunk buffers fit four times in the stage take their chunks
      // two at a time (att_items_multi; the generic instance would spill registers with both walks).
      const bool multi = D_ != 0 && KVT != MK_KV_F32 && 4 * kv_buf_slots(p.hd, p.kvt) <= s.a_slots;
      const int first = multi ? 2 : max(1, kv_nbuf(p.hd, p.kvt, s.a_slots) - 1);
      for (int kc = 0; kc < first; ++kc) {
        const int cn = att_chunk_at(p, NW, w, pos, kc);
        if (cn >= 0) kv_stage(p, L, cn, pos, s.stA + kc * kv_buf_slots(p.hd, p.kvt) * SLOT);
      }
      if (multi ? !att_items_multi<2>(p, L, cx, s, NW, w, pos, 0, tr) : !att_items(p, L, cx, s, NW, w, pos, 0, tr))
        return;
      tr.mark();
      const int o0 = split(K, NW, w), o1 = split(K, NW, w + 1);
      if (!att_combine(p, L, cx, s, o0, o1, pos)) return;
      tr.mark();
    }
    // mixer output -> out-projection rows + residual -> records
    GemvQ4 gout;
    gout.init(L.w_out, d0 >> 2, d1 - d0, K);
    if (streamer()) gemv_q4_prime(gout, c1, q);
    {
      const bool ok = gather_vec(cx, L.ll_o, K, s.vec);
      if (wg_bar_or(s, !ok)) return;
      q4_pack(s.vec, K);
    }
    tr.mark();
    gemv_q4<false, false>(gout, (const LS u32*)s.vec, s.att, c1, q, streamer(), tr,
                          [&](int r, float v, float) { ll_put(L.ll_x1 + d0 + r, cx.epoch, s.x[d0 + r] + v); });
    tr.mark();
    GemvQ4 ggu;
    ggu.init(L.w_gu, j0 >> 1, 2 * (j1 - j0), D);
    if (streamer()) gemv_q4_prime(ggu, c0, q);
    {
      // the polling threads fetch the next layer's descriptor under this gather's latency
      constexpr int NDW = (int)(sizeof(MkLayerDev) / 4);
      const int di = tid() - NCT;
      const bool fetch = !streamer() && di < NDW && l + 1 < p.n_layers;
      u32 dw = 0u;
      if (fetch) dw = ((const MK_G u32*)(p.layers + l + 1))[di];
      const bool ok = gather_vec_all<false, Q4_PB>(cx, L.ll_x1, D, s.x);
      if (fetch) ((LS u32*)(s.desc + ((l + 1) & 1)))[di] = dw;
      if (wg_bar_or(s, !ok)) return;
    }
    tr.mark();
    rmsnorm_gg(s.x, L.g12 + D, s.vec, D, p.rms_eps, tr);
    q4_pack(s.vec, D);
    gemv_q4<true, false>(ggu, s.xn, s.att, c0, q, streamer(), tr, [&](int j, float gv, float uv) {
      ll_put(L.ll_h + j0 + j, cx.epoch, gv / (1.0f + expf(-gv)) * uv);
    });
    tr.mark();
    GemvQ4 gdn;
    gdn.init(L.w_down, d0 >> 2, d1 - d0, p.ffn);
    if (streamer()) gemv_q4_prime(gdn, c1, q);
    {
      const bool ok = gather_vec_all<false, Q4_PB_FFN>(cx, L.ll_h, p.ffn, s.vec);
      if (wg_bar_or(s, !ok)) return;
      q4_pack(s.vec, p.ffn);
    }
    tr.mark();
    gemv_q4<false, false>(gdn, (const LS u32*)s.vec, s.att, c1, q, streamer(), tr,
                          [&](int r, float v, float) { ll_put(L.ll_x2 + d0 + r, cx.epoch, s.x[d0 + r] + v); });
    tr.mark();
    // the next layer's input-norm gains (polling threads) and in-projection units (or the LM
    // head's; streaming threads) while the residual travels
    {
      GemvQ4 g;
      int i0;
      if (l + 1 < p.n_layers) {
        const MkLayerDev Ln = layer_desc(s.desc, (l + 1) & 1);
        gains_gg_issue(Ln.g12, D, gin_g);
        in_slice(Ln, g, i0);
      } else {
        head_slice(g, i0);
      }
      if (streamer()) gemv_q4_prime(g, c0, q);
    }
    {
      const bool ok = gather_vec_all<false, Q4_PB>(cx, L.ll_x2, D, s.x);
      if (wg_bar_or(s, !ok)) return;
    }
    tr.mark();
  }

  // final norm + tied LM head + argmax (lowest index among equal maxima)
  rmsnorm_gg(s.x, p.g_final, s.vec, D, p.rms_eps, tr);
  q4_pack(s.vec, D);
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  {
    GemvQ4 gl;
    int v0;
    head_slice(gl, v0);
    gemv_q4<false, true>(gl, s.xn, s.att, c0, q, streamer(), tr, [&](int r, float v, float) {
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
  decode_q4_body<0, 0, 0, 0, 0, 0, 0, 0, MK_KV_F32>(p);
}
// hidden 5120, FFN 17408, 32 DeltaNet heads of 128, 24 Q / 4 KV heads of 128 (the 27B-scale hybrid)
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_q4_kernel_h5120(MkDecodeParams p) {
  decode_q4_body<5120, 17408, 32, 128, 128, 24, 4, 128, MK_KV_F32>(p);
}
// binary16 and int8 KV caches
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_q4_kernel_f16(MkDecodeParams p) {
  decode_q4_body<0, 0, 0, 0, 0, 0, 0, 0, MK_KV_F16>(p);
}
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_q4_kernel_q8(MkDecodeParams p) {
  decode_q4_body<0, 0, 0, 0, 0, 0, 0, 0, MK_KV_Q8>(p);
}
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_q4_kernel_h5120_f16(MkDecodeParams p) {
  decode_q4_body<5120, 17408, 32, 128, 128, 24, 4, 128, MK_KV_F16>(p);
}
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_q4_kernel_h5120_q8(MkDecodeParams p) {
  decode_q4_body<5120, 17408, 32, 128, 128, 24, 4, 128, MK_KV_Q8>(p);
}

namespace {
typedef void (*DecodeKernel)(MkDecodeParams);
DecodeKernel pick_q4_kernel(const MkDecodeParams& p) {
  const bool h5120 = p.D == 5120 && p.ffn == 17408 && p.H == 32 && p.dk == 128 && p.dv == 128 && p.nq == 24 &&
                     p.nkv == 4 && p.hd == 128;
  if (p.kvt == MK_KV_F16) return h5120 ? mk_decode_q4_kernel_h5120_f16 : mk_decode_q4_kernel_f16;
  if (p.kvt == MK_KV_Q8) return h5120 ? mk_decode_q4_kernel_h5120_q8 : mk_decode_q4_kernel_q8;
  return h5120 ? mk_decode_q4_kernel_h5120 : mk_decode_q4_kernel;
}
}  // namespace

// Load time: a Q4G32 matrix in its input layout (codes, then (d, m) words) -> the tiled layout of
// mk_q4.h.  One thread per (4-row block, 32-column block); rows past R are zero.
__global__ void mk_q4_tile_kernel(const uint8_t* __restrict__ src, int64_t R, int64_t K, uint8_t* __restrict__ dst) {
  const int64_t G = K >> 5, nt = ((R + 3) >> 2) * G;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nt; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = t / G, g = t - b * G;
    u32x4 out[5];
    u32 pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = 4 * b + r;
      out[r] = u32x4{0u, 0u, 0u, 0u};
      pw[r] = 0u;
      if (row < R) {
        out[r] = *(const u32x4*)(src + row * (K >> 1) + g * 16);
        pw[r] = *(const u32*)(src + R * (K >> 1) + (row * G + g) * 4);
      }
    }
    out[4] = u32x4{pw[0], pw[1], pw[2], pw[3]};
    // segment s of row block b: five planes of ng 16-byte pieces
    const int64_t s = g >> 6, l = g & 63, ng = G - 64 * s < 64 ? G - 64 * s : 64;
    uint8_t* seg = dst + (b * G + 64 * s) * Q4_TILE;
#pragma unroll
    for (int i = 0; i < 5; ++i) *(u32x4*)(seg + i * ng * 16 + l * 16) = out[i];
  }
}

extern "C" int mk_launch_q4_tile(const void* src, int64_t R, int64_t K, void* dst, void* stream) {
  if (R <= 0) return 0;
  hipLaunchKernelGGL(mk_q4_tile_kernel, dim3(1024), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)src, R, K,
                     (uint8_t*)dst);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_launch_decode_q4(const MkDecodeParams* p, int n_wg, void* stream) {
  hipLaunchKernelGGL(pick_q4_kernel(*p), dim3(n_wg), dim3(MK_NT), (size_t)p->lds_floats * 4, (hipStream_t)stream, *p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_decode_q4_max_blocks_per_cu(const MkDecodeParams* p, int lds_bytes) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, pick_q4_kernel(*p), MK_NT, lds_bytes) != hipSuccess) return 0;
  return nb;
}

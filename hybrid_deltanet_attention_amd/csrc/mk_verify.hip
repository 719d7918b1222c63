// Speculative verify of the hybrid decoder as ONE persistent kernel launch on gfx950: the pending
// token and up to five drafted tokens are scored in a single pass (Reddit follow-up on the 27B
// model, "Speed" and speculative-decoding paragraphs: the speed-up comes from scoring a batch of
// drafts in one pass whose cost stays close to that of a single token, and the output equals the
// main model's greedy choices; news-aggregator page: the whole draft-and-check cycle runs fused
// in one launch).
//
// The launch runs the decode kernel's per-position arithmetic on nt = k + 1 positions at once:
//  - every GEMV streams each weight row from HBM once and applies it to all nt activation vectors;
//  - every exchange carries the records of all nt positions, so a layer still costs five (DeltaNet)
//    or six (attention) exchanges, not 5 nt;
//  - each DeltaNet state row applies the nt gated delta-rule updates in order, in registers;
//  - a split-K attention item (16 positions of one KV head) serves every position whose causal
//    window reaches it, the new positions' keys and values coming from the exchange records.
// Sums are formed in the same order as in the decode kernel, so the greedy choice after each
// position equals, bit for bit, the one a decode launch at that position would make.
//
// Accepting: workgroup 0 gathers every workgroup's per-position (max, index), takes the greedy
// choices y_1..y_nt, counts the leading drafts equal to them (a), writes the outputs, advances the
// position by a + 1 and publishes a as one more record.  Every workgroup then restores its
// DeltaNet rows to the state after position a: the pass wrote the state after each position t < nt
// - 1 to snapshot t and the final one to the main buffer, so only a copy of the workgroup's own rows
// from snapshot a is needed (by the same threads that wrote them).  KV-cache entries of rejected
// positions lie past the new position and are overwritten later.
//
// Unlike the decode kernel no weights are prefetched into LDS: the LDS holds nt positions'
// residuals and vectors instead, and all eight waves stream their GEMV units through registers.

#include "mk_q4.h"

namespace {

constexpr int VT = MK_VERIFY_MAXT;
constexpr int PBV = 16;  // poll loads in flight per thread in the verify gathers

// The verify kernel prefetches nothing into LDS, so all 512 threads poll, PBV loads each (the
// decode kernel's gathers use its 256 polling threads, 8 loads each): the nt-position record
// vectors are gathered in about as few memory round trips as the decode kernel's single-position
// ones.  (Keeping polls off the waves that store, as the decode kernel does, measured slower here:
// the extra poll rounds and the halved row parallelism cost more than the store waits they save.)
// Same contracts as gather_map / gather_vec / gather_hl.
template <typename SrcFn, typename UseFn>
__device__ __forceinline__ bool gather_map_all(const Ctx& cx, int n, SrcFn src, UseFn use) {
  const u32 e = cx.epoch;
  const int pl = tid();
  bool ok = true;
  for (int base = 0; ok && base < n; base += MK_NT * PBV) {
    u32 pending = 0;
#pragma unroll
    for (int k = 0; k < PBV; ++k)
      if (base + k * MK_NT + pl < n) pending |= 1u << k;
    // record addresses once per round, not per poll
    const MK_G mk_u64* ad[PBV];
#pragma unroll
    for (int k = 0; k < PBV; ++k) ad[k] = ((pending >> k) & 1u) ? src(base + k * MK_NT + pl) : nullptr;
    u32 spins = 0;
    while (pending) {
      mk_u64 v[PBV];
#pragma unroll
      for (int k = 0; k < PBV; ++k)
        if ((pending >> k) & 1u) v[k] = ld_dev(ad[k]);
#pragma unroll
      for (int k = 0; k < PBV; ++k)
        if (((pending >> k) & 1u) && (u32)(v[k] >> 32) == e) {
          use(base + k * MK_NT + pl, __uint_as_float((u32)v[k]));
          pending &= ~(1u << k);
        }
      if (pending) {
        ++spins;
        if (((spins & 255u) == 0 && err_seen(cx)) || spins > MK_SPIN_LIMIT) {
          if (spins > MK_SPIN_LIMIT) set_err(cx, 1u);
          ok = false;
          break;
        }
      }
    }
  }
  wait_vm<0>();
  return ok;
}

// RMSNorm of nt residuals x[t] -> xn[t] (hi/lo BF16 pairs).  Wave t forms position t's sum of
// squares exactly as every wave of the decode kernel's rmsnorm does; then all threads scale.
// Ends with a barrier.
__device__ __forceinline__ void rmsnorm_v(const LS float* x, const LS uint16_t* g, LS u32* xn, int D, float eps,
                                          int nt, LS float* rs) {
  D = uni(D);
  const int D4 = D >> 2;
  if (wave() < nt) {
    const LS f32x4* x4 = (const LS f32x4*)(x + wave() * D);
    float s = 0.f;
    for (int c0 = lane(); c0 < D4; c0 += 256) {
      f32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c0 + 64 * k < D4) v[k] = x4[c0 + 64 * k];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        s = fmaf(v[k].x, v[k].x, s);
        s = fmaf(v[k].y, v[k].y, s);
        s = fmaf(v[k].z, v[k].z, s);
        s = fmaf(v[k].w, v[k].w, s);
      }
    }
    s = wave_sum(s);
    if (lane() == 0) rs[wave()] = 1.0f / sqrtf(s / (float)D + eps);
  }
  wg_bar();
  for (int i = tid(); i < nt * D4; i += MK_NT) {
    const int t = i / D4, c = i - t * D4;
    const float r = rs[t];
    const f32x4 v = ((const LS f32x4*)(x + t * D))[c];
    const u32x2 gg = *(const LS u32x2*)(g + 4 * c);
    u32 h[4], l[4];
    split_hl(v.x * r * __uint_as_float(gg.x << 16), h[0], l[0]);
    split_hl(v.y * r * __uint_as_float(gg.x & 0xffff0000u), h[1], l[1]);
    split_hl(v.z * r * __uint_as_float(gg.y << 16), h[2], l[2]);
    split_hl(v.w * r * __uint_as_float(gg.y & 0xffff0000u), h[3], l[3]);
    LS u32* xo = xn + t * D;
    const int o = hl_word(4 * c);
    *(LS u32x2*)(xo + o) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    *(LS u32x2*)(xo + o + 4) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
  }
  wg_bar();
}

// GEMV over nt activation vectors (position t's at xin + t * xs words, hi/lo layout).  Every wave
// streams its units from HBM through registers (two units of look-ahead) and applies each to all
// nt vectors.  A row's value at a position is the same sum, in the same order, as the decode
// kernel's GEMV forms.  The streaming threads then call epi(row, t, v, 0) or, with PAIRS,
// epi(pair, t, v_even_row, v_odd_row).
//
// A wave's first two units can be loaded ahead with gemv_v_pre, before the exchange that delivers
// the GEMV's input, so that their HBM latency runs under the exchange (the loads have no address
// dependence on the input).  gemv_v then starts from them.
struct GemvPre {
  RegUnits<2> r;
};

// rows of one chunk: the unit partials of all nt positions fit MK_RED_CAP
__device__ __forceinline__ int gemv_v_rows(int S, int nt) { return max(4, (MK_RED_CAP / (S * nt)) & ~3); }

__device__ __forceinline__ void gemv_v_issue2(const Gemv& g, int RB, int s, int step, RegUnits<2>& r, int rb0) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rbi = rb0 + i * step;
#pragma unroll
    for (int k = 0; k < USLOTS; ++k) {
      const MK_G uint16_t* a = rbi < RB ? g.addr(rbi * g.S + s, k) : nullptr;
      r.c[i * USLOTS + k] = a ? ldw(a) : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ void gemv_v_pre(const Gemv& G, int nt, GemvPre& pre) {
  const int S = uni(G.S);
  Gemv g;
  g.init(uni_ptr(G.W), uni(min(gemv_v_rows(S, uni(nt)), G.R)), uni(G.K));
  const int RB = (g.R + 3) >> 2;
  SegPlan sp;
  sp.init(S, wave(), MK_NWAVE);
  if (sp.s0 < S && sp.j < RB) gemv_v_issue2(g, RB, sp.s0, sp.nj, pre.r, sp.j);
  keep_issued();
}

template <bool PAIRS, typename Epi>
__device__ __forceinline__ void gemv_v(const Gemv& G, const LS u32* xin, int xs, int nt, LS float* red,
                                       const GemvPre& pre, Epi epi) {
  const int S = uni(G.S);
  nt = uni(nt);
  const int rc = gemv_v_rows(S, nt);
  for (int r0 = 0; r0 < G.R; r0 += rc) {
    Gemv g;
    g.init(uni_ptr(G.W + (size_t)r0 * G.K), uni(min(rc, G.R - r0)), uni(G.K));
    const int RB = (g.R + 3) >> 2;
    const int blk = g.R * S;  // partials per position
    SegPlan sp;
    sp.init(S, wave(), MK_NWAVE);
    for (int s = sp.s0; s < S; s += sp.sstep) {
      int rb = sp.j;
      if (rb >= RB) continue;
      const int step = sp.nj;
      RegUnits<2> cur, nxt;
      if (r0 == 0 && s == sp.s0) {
#pragma unroll
        for (int i = 0; i < 2 * USLOTS; ++i) cur.c[i] = pre.r.c[i];
      } else {
        gemv_v_issue2(g, RB, s, step, cur, rb);
      }
      // Nothing may look outstanding in cur when the loop starts: the loads above are conditional,
      // and a register the compiler cannot place in the load queue makes it wait for every load,
      // the look-ahead ones included, before each unit.
      wait_vm<0>();
      for (; rb < RB; rb += 2 * step) {
        gemv_v_issue2(g, RB, s, step, nxt, rb + 2 * step);
        keep_issued();
        const bool h1 = rb + step < RB;
        // positions in a loop, not unrolled: the kernel's code must stay small enough for the
        // instruction cache, and each position reads its 32 bytes of activations from LDS
#pragma unroll 2
        for (int t = 0; t < nt; ++t) {
          XSlice x;
          load_x(x, xin + t * xs, s, g.K);
          const float a0 = unit_dot_x(s, g.K, cur.c, x);
          const float a1 = h1 ? unit_dot_x(s, g.K, cur.c + USLOTS, x) : 0.f;
          put_partial(g, rb * S + s, a0, red + t * blk);
          if (h1) put_partial(g, (rb + step) * S + s, a1, red + t * blk);
        }
#pragma unroll
        for (int i = 0; i < 2 * USLOTS; ++i) cur.c[i] = nxt.c[i];
      }
      // the last look-ahead loads are never used; waiting here keeps them from looking
      // outstanding to the code that follows
      wait_vm<0>();
    }
    wg_bar();
    if (streamer()) {
      // (position, row) pairs spread over the streaming threads, so the positions' epilogues run
      // side by side
      const int nr = PAIRS ? g.R / 2 : g.R;
      for (int i = tid(); i < nt * nr; i += NCT) {
        const int t = i / nr, j = i - t * nr;
        const LS float* rt = red + t * blk;
        if (PAIRS) epi(r0 / 2 + j, t, seg_sum(rt + (2 * j) * S, S), seg_sum(rt + (2 * j + 1) * S, S));
        else epi(r0 + j, t, seg_sum(rt + j * S, S), 0.f);
      }
    }
    wg_bar();  // red is reused by the next chunk
  }
}

// Gated delta rule for nt positions on rows [s0, s1) of S, read from the main buffer once.  After
// position t a row goes to snapshot t (t < nt - 1) or back to the main buffer (t = nt - 1), and
// o_t = S_t q_t goes to the records.  Every wave owns rows (local index li % 8); wave t forms
// position t's norms and gates; all in the decode kernel's order.
__device__ __forceinline__ bool dn_state_v(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx, const Lds& s,
                                           LS float* buf, LS float* nrm, int s0, int s1, int nt) {
  const int H = p.H, dk = p.dk, dv = p.dv, K = H * dv;
  const int rows_in = L.rows_in;
  const MK_G mk_u64* in = L.ll_in;
  const int off_k = H * dk, off_v = 2 * H * dk, off_a = 2 * H * dk + H * dv, off_b = off_a + H;
  const int h0 = s0 < s1 ? s0 / dv : 0, h1 = s0 < s1 ? (s1 - 1) / dv : -1;
  // this wave's first row (local index = wave) is loaded before the first gather, so its HBM
  // latency runs under the exchange
  float pre[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane() + 64 * c;
    pre[c] = (wave() < s1 - s0 && e < dk) ? L.S[(size_t)(s0 + wave()) * dk + e] : 0.f;
  }
  for (int h = h0; h <= h1; ++h) {
    const int i0 = max(s0, h * dv) - h * dv, i1 = min(s1, (h + 1) * dv) - h * dv;
    const int nv = i1 - i0;
    const int per = 2 * dk + 2 + nv;  // per position: q, k, a, b, this workgroup's v rows
    const bool ok = gather_map_all(cx, nt * per, [=](int f) {
      const int t = f / per, g = f - t * per;
      const MK_G mk_u64* b = in + (size_t)t * rows_in;
      if (g < dk) return b + h * dk + g;
      if (g < 2 * dk) return b + off_k + h * dk + (g - dk);
      if (g == 2 * dk) return b + off_a + h;
      if (g == 2 * dk + 1) return b + off_b + h;
      return b + off_v + h * dv + i0 + (g - 2 * dk - 2);
    }, [=](int f, float v) { buf[f] = v; });
    if (wg_bar_or(s, !ok)) return false;
    // wave t: position t's norms and gates -> nrm[4 t ..]
    if (wave() < nt) {
      const int t = wave();
      const LS float* q = buf + t * per;
      const LS float* k = q + dk;
      float qq = 0.f, kk = 0.f;
      for (int e = lane(); e < dk; e += 64) {
        qq = fmaf(q[e], q[e], qq);
        kk = fmaf(k[e], k[e], kk);
      }
      qq = wave_sum(qq);
      kk = wave_sum(kk);
      if (lane() == 0) {
        nrm[4 * t] = 1.0f / sqrtf(qq + p.l2_eps);
        nrm[4 * t + 1] = 1.0f / sqrtf(kk + p.l2_eps);
        nrm[4 * t + 2] = expf(-softplusf_(q[2 * dk]));
        nrm[4 * t + 3] = sigmoidf_(q[2 * dk + 1]);
      }
    }
    wg_bar();
    const int lo = h * dv + i0 - s0, hi = h * dv + i1 - s0;
    for (int li = lo + ((wave() - lo % MK_NWAVE) + MK_NWAVE) % MK_NWAVE; li < hi; li += MK_NWAVE) {
      const int row = s0 + li;
      float sr[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = lane() + 64 * c;
        sr[c] = li == wave() ? pre[c] : (e < dk ? L.S[(size_t)row * dk + e] : 0.f);
      }
#pragma unroll 1
      for (int t = 0; t < nt; ++t) {
        const float sq = nrm[4 * t], sk = nrm[4 * t + 1], al = nrm[4 * t + 2], be = nrm[4 * t + 3];
        const LS float* q = buf + t * per;
        const LS float* k = q + dk;
        const LS float* vr = q + 2 * dk + 2;
        float kd = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e = lane() + 64 * c;
          if (e < dk) kd = fmaf(sr[c], k[e] * sk, kd);
        }
        kd = wave_sum(kd);
        const float u = be * (vr[row - h * dv - i0] - al * kd);
        MK_G float* dst = t + 1 < nt ? L.Ssnap + (size_t)t * p.snap_stride : L.S;
        float od = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e = lane() + 64 * c;
          if (e < dk) {
            const float nv2 = fmaf(u, k[e] * sk, al * sr[c]);
            sr[c] = nv2;
            dst[(size_t)row * dk + e] = nv2;
            od = fmaf(nv2, q[e] * sq, od);
          }
        }
        od = wave_sum(od);
        if (lane() == 0) ll_put(L.ll_o + (size_t)t * K + row, cx.epoch, od);
      }
    }
    wg_bar();  // buf is reused by the next head
  }
  return true;
}

// One q/k/v row pair (RoPE pair order) of position t: rotate q and k at position pos + t, append k
// and v to an FP32 cache at pos + t (compact caches are appended by the attention items), publish.
__device__ __forceinline__ void att_qkv_v_put(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx,
                                              const Lds& s, int P, int t, int pos, float x1, float x2) {
  const int hd = p.hd, half = hd / 2, rows_in = L.rows_in;
  const int nqp = p.nq * half, nkp = p.nkv * half;
  MK_G mk_u64* llq = L.ll_in + (size_t)t * rows_in;
  MK_G mk_u64* llk = llq + p.nq * hd;
  MK_G mk_u64* llv = llk + p.nkv * hd;
  const LS float* rp = s.rope + t * hd;
  if (P < nqp + nkp) {
    const bool isq = P < nqp;
    const int Q = isq ? P : P - nqp;
    const int hh = Q / half, m = Q - hh * half;
    const float c = rp[m], sv = rp[half + m];
    const float y1 = x1 * c - x2 * sv;
    const float y2 = x2 * c + x1 * sv;
    if (isq) {
      ll_put(llq + hh * hd + m, cx.epoch, y1);
      ll_put(llq + hh * hd + m + half, cx.epoch, y2);
    } else {
      const size_t co = ((size_t)hh * p.max_ctx + pos + t) * hd + m;
      ll_put(llk + hh * hd + m, cx.epoch, y1);
      ll_put(llk + hh * hd + m + half, cx.epoch, y2);
      if (p.kvt == MK_KV_F32) {  // compact rows are appended by the attention items
        L.Kc[co] = y1;
        L.Kc[co + half] = y2;
      }
    }
  } else {
    const int Q = P - nqp - nkp;
    const int hh = Q / half, m = Q - hh * half;
    const size_t co = ((size_t)hh * p.max_ctx + pos + t) * hd + m;
    ll_put(llv + hh * hd + m, cx.epoch, x1);
    ll_put(llv + hh * hd + m + half, cx.epoch, x2);
    if (p.kvt == MK_KV_F32) {
      L.Vc[co] = x1;
      L.Vc[co + half] = x2;
    }
  }
}

// q/k/v rows (RoPE pair order) for nt positions: rotate q and k at position pos + t, append k and v
// to the cache at pos + t, publish all three.
__device__ __forceinline__ void att_qkv_v(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx, const Lds& s,
                                          const Gemv& g, const GemvPre& pre, int P0, int pos, int nt) {
  gemv_v<true>(g, s.xn, p.D, nt, s.att, pre, [&](int pl, int t, float x1, float x2) {
    att_qkv_v_put(p, L, cx, s, P0 + pl, t, pos, x1, x2);
  });
}

// Split-K attention items over positions 0 .. pos + nt - 1, with the decode kernel's items: (block
// of att_cpi 16-position chunks, KV head g).  A chunk serves the positions t >= tmin whose window
// reaches it; keys and values of positions already in the cache (< pos) are loaded by the streaming
// waves, those of this launch's positions come from the records.  Per served position and query
// head the chunk's (max, sum, acc) are formed exactly as a decode chunk forms them and merged into
// the position's running values for the item in chunk order, with the decode kernel's formula; a
// position publishes its (max, sum, acc[hd]) at its last chunk of the item.
// TWO_PARTS: the score parts go two at a time (qk_parts2x2; more loads in flight, more registers),
// else one at a time (qk_part2); the products and sums are the same either way.  ONE_PART: the
// instance for shapes whose scores are one part (att_parts == 1) with hd / 4 a multiple of 8 (so
// eight-group steps are qk_part2's own), without the code for the other cases.
template <bool TWO_PARTS, bool ONE_PART = false>
__device__ __forceinline__ bool att_items_v(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx, const Lds& s,
                                            LS float* sc, int NW, int w, int pos, int nt) {
  const int hd = p.hd, nkv = p.nkv, gs = p.nq / p.nkv, C = ATT_C, rows_in = L.rows_in, cpi = p.att_cpi;
  const int Lmax = pos + nt;
  const int nch = (Lmax + C - 1) / C;
  const int items = ((nch + cpi - 1) / cpi) * nkv;
  const float scale = 1.0f / sqrtf((float)hd);
  LS float* qv = sc;                   // [nt][gs][hd]
  LS float* kc = qv + nt * gs * hd;    // [C][hd]
  LS float* vc = kc + C * hd;          // [C][hd]
  LS float* pb = vc + C * hd;          // [nt][gs][C] probabilities (unnormalised)
  LS float* mf = pb + nt * gs * C;     // [nt][gs][2] this chunk's merge factors (running acc, chunk acc)
  LS float* racc = mf + 2 * nt * gs;   // [nt][gs][hd] running acc of the item
  LS float* rml = racc + nt * gs * hd; // [2 (chunk parity)][nt][gs][2] running max and sum
  const int np = ONE_PART ? 1 : att_parts(gs, hd), gpp = (hd >> 2) / np;
  // partial scores [np][2 nh] in the GEMV partials region, each written and read by one thread (at
  // most MK_VERIFY_MAXT * MK_NT + MK_NT floats: np * gs * 16 <= MK_NT)
  LS float* sp = s.att;
  static_assert(MK_VERIFY_MAXT * MK_NT + MK_NT <= MK_RED_CAP, "partial scores exceed the GEMV partials region");
  const MK_G mk_u64* llq = L.ll_in;
  const MK_G mk_u64* llk = L.ll_in + p.nq * hd;
  const MK_G mk_u64* llv = llk + nkv * hd;
  const size_t tstride = (size_t)p.max_items * gs * (hd + 2);  // partial records per position
  const int h4 = hd >> 2;
  // Keys and values of the positions already in the cache, loaded by every thread one chunk ahead into
  // registers (raw cache words; up to ATT_C * 64 four-value groups per chunk)
  constexpr int KVR = (ATT_C * 64 + MK_NT - 1) / MK_NT;
  // (each cache type loads into registers of its own width, so that no load's destination has to be
  // assembled into a wider vector -- which would make the wave wait for the load right away)
  u32x4 rk[KVR], rv[KVR];
  u32x2 rk2[KVR], rv2[KVR];
  u32 rk1[KVR], rv1[KVR];
  float rks[KVR], rvs[KVR];
  int pf_n = 0;  // four-value groups held for the chunk to come (per workgroup)
  auto kv_fetch = [&](int itn, int cn) {
    pf_n = 0;
    if (itn >= items) return;
    const int g = itn - (itn / nkv) * nkv, j0 = cn * C;
    pf_n = max(0, min(pos, min(Lmax, j0 + C)) - j0) * h4;
#pragma unroll
    for (int e = 0; e < KVR; ++e) {
      const int x = tid() + e * MK_NT;
      if (x < pf_n) {
        const int jj = x / h4, d = (x - jj * h4) * 4;
        const size_t gi = ((size_t)g * p.max_ctx + j0 + jj) * hd + d;
        if (p.kvt == MK_KV_F32) {
          rk[e] = *(const MK_G u32x4*)(L.Kc + gi);
          rv[e] = *(const MK_G u32x4*)(L.Vc + gi);
        } else if (p.kvt == MK_KV_F16) {
          rk2[e] = *(const MK_G u32x2*)((const MK_G _Float16*)L.Kc + gi);
          rv2[e] = *(const MK_G u32x2*)((const MK_G _Float16*)L.Vc + gi);
        } else {
          rk1[e] = *(const MK_G u32*)((const MK_G signed char*)L.Kc + gi);
          rv1[e] = *(const MK_G u32*)((const MK_G signed char*)L.Vc + gi);
          rks[e] = L.Ks[gi / MK_KV_Q8_BLOCK];
          rvs[e] = L.Vs[gi / MK_KV_Q8_BLOCK];
        }
      }
    }
  };
  // the held groups -> kc / vc rows in FP32 (the decode kernel's expansion of the same rows)
  auto kv_stash = [&]() {
#pragma unroll
    for (int e = 0; e < KVR; ++e) {
      const int x = tid() + e * MK_NT;
      if (x < pf_n) {
        const int jj = x / h4, d = (x - jj * h4) * 4;
        f32x4 kk, vv;
        if (p.kvt == MK_KV_F32) {
          kk = f32x4{__uint_as_float(rk[e].x), __uint_as_float(rk[e].y), __uint_as_float(rk[e].z),
                     __uint_as_float(rk[e].w)};
          vv = f32x4{__uint_as_float(rv[e].x), __uint_as_float(rv[e].y), __uint_as_float(rv[e].z),
                     __uint_as_float(rv[e].w)};
        } else if (p.kvt == MK_KV_F16) {
          kk = f32x4{half_bits_f32(rk2[e].x & 0xffffu), half_bits_f32(rk2[e].x >> 16), half_bits_f32(rk2[e].y & 0xffffu),
                     half_bits_f32(rk2[e].y >> 16)};
          vv = f32x4{half_bits_f32(rv2[e].x & 0xffffu), half_bits_f32(rv2[e].x >> 16), half_bits_f32(rv2[e].y & 0xffffu),
                     half_bits_f32(rv2[e].y >> 16)};
        } else {
          const float ks = rks[e], vs = rvs[e];
          kk = f32x4{i8_f32(rk1[e], 0) * ks, i8_f32(rk1[e], 1) * ks, i8_f32(rk1[e], 2) * ks, i8_f32(rk1[e], 3) * ks};
          vv = f32x4{i8_f32(rv1[e], 0) * vs, i8_f32(rv1[e], 1) * vs, i8_f32(rv1[e], 2) * vs, i8_f32(rv1[e], 3) * vs};
        }
        *(LS f32x4*)(kc + jj * hd + d) = kk;
        *(LS f32x4*)(vc + jj * hd + d) = vv;
      }
    }
  };
  int gq = -1;  // KV head whose queries are in qv
  int k = 0;    // chunk sequence number in this workgroup (running-value parity)
  if (w < items) kv_fetch(w, (w / nkv) * cpi);
  for (int it = w; it < items; it += NW) {
    const int blk = it / nkv, g = it - blk * nkv;
    const int c0 = blk * cpi, c1 = min(nch, c0 + cpi);
    for (int c = c0; c < c1; ++c, ++k) {
      const int j0 = c * C;
      const int tmin = max(0, j0 - pos);
      const int jend = min(Lmax, j0 + C);
      const int jnew = max(j0, pos);
      const int nnew = max(0, jend - jnew);
      kv_stash();
      const int nqr = g != gq ? nt * gs * hd : 0;  // queries: once per KV head
      gq = g;
      const int nkvr = nnew * hd;
      bool ok = true;
      if (nqr + 2 * nkvr > 0) {
        ok = gather_map_all(cx, nqr + 2 * nkvr, [=](int f) {
          if (f < nqr) {
            const int tt = f / (gs * hd), r = f - tt * gs * hd;
            return llq + (size_t)tt * rows_in + g * gs * hd + r;
          }
          f -= nqr;
          const int sel = f >= nkvr ? 1 : 0;
          f -= sel * nkvr;
          const int jj = f / hd, d = f - jj * hd;
          return (sel ? llv : llk) + (size_t)(jnew + jj - pos) * rows_in + g * hd + d;
        }, [=](int f, float v) {
          if (f < nqr) {
            qv[f] = v;
          } else {
            f -= nqr;
            const int sel = f >= nkvr ? 1 : 0;
            f -= sel * nkvr;
            const int jj = f / hd, d = f - jj * hd;
            (sel ? vc : kc)[(jnew - j0 + jj) * hd + d] = v;
          }
        });
      }
      // the next chunk's cached rows load while this one is processed (after the gather, whose
      // final wait would otherwise drain them)
      if (c + 1 < c1) kv_fetch(it, c + 1);
      else kv_fetch(it + NW, ((it + NW) / nkv) * cpi);
      if (wg_bar_or(s, !ok)) return false;
      // this launch's positions in the chunk take the cache's values and are appended (barriers inside)
      if (p.kvt != MK_KV_F32 && nnew > 0)
        kv_round_append(p, L, kc + (jnew - j0) * hd, vc + (jnew - j0) * hd, nnew, pb, g, jnew);
      // scores, softmax numerators, row max and sum: one thread per (position, head, slot) of the
      // first half of the rows and the row of the same slot one half further on (so the key row is
      // loaded once for both), whole 16-lane rows.  The slot-0 thread of each row also forms the
      // row's merge with the item's running values (the decode kernel's formula) -> merge factors,
      // and the running or published (max, sum).
      const LS float* rin = rml + (k & 1) * 2 * nt * gs;   // running (max, sum) before this chunk
      LS float* rout = rml + ((k + 1) & 1) * 2 * nt * gs;  // ... and after it
      const bool first = c == c0;
      const int nrow = (nt - tmin) * gs * C;
      const int nh = ((nrow / C + 1) / 2) * C;  // rows of the first half (whole 16-lane rows)
      // row f (< nrow) = (position tmin + f / (gs C), head, slot)
      auto row_of = [&](int f, int& tt, int& ii, int& jq) {
        f = min(f, nrow - 1);
        tt = f / (gs * C);
        const int r = f - tt * gs * C;
        ii = r / C;
        jq = r - ii * C;
      };
      // scores, softmax numerators, row max and sum: one thread per row f of the first half and the
      // row f + nh of the same slot (one key row serves both), whole 16-lane rows.  A thread forms the
      // decode kernel's key-dimension parts of its two dot products one after another (qk_part2),
      // keeps them in the GEMV partials region and adds them in the decode kernel's tree
      for (int b0 = 0; b0 < nh; b0 += MK_NT) {
        int fr[2];
        fr[0] = b0 + tid();
        fr[1] = fr[0] + nh;
        float a[2] = {0.f, 0.f};
        int tt[2], ii[2], jq[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) row_of(fr[u], tt[u], ii[u], jq[u]);
        if (fr[0] < nh) {
          const int sst = 2 * nh;
          const LS float* kr = kc + jq[0] * hd;
          const LS float* qr0 = qv + ((tmin + tt[0]) * gs + ii[0]) * hd;
          const LS float* qr1 = qv + ((tmin + tt[1]) * gs + ii[1]) * hd;
          if (ONE_PART) {
            qk_part2_w<8>(kr, qr0, qr1, jq[0], 0, gpp, a[0], a[1]);  // gpp = hd / 4, a multiple of 8 here
            sp[fr[0]] = a[0];
            sp[fr[1]] = a[1];
          } else if (np == 1 || !TWO_PARTS) {
            for (int part = 0; part < np; ++part) {
              qk_part2(kr, qr0, qr1, jq[0], part, gpp, a[0], a[1]);
              sp[part * sst + fr[0]] = a[0];
              sp[part * sst + fr[1]] = a[1];
            }
          } else {
            for (int part = 0; part + 1 < np; part += 2) {  // np is a power of two
              float ap[4];
              qk_parts2x2(kr, qr0, qr1, jq[0], part, gpp, ap);
              sp[part * sst + fr[0]] = ap[0];
              sp[part * sst + fr[1]] = ap[1];
              sp[(part + 1) * sst + fr[0]] = ap[2];
              sp[(part + 1) * sst + fr[1]] = ap[3];
            }
          }
          a[0] = att_part_sum(sp + fr[0], sst, np);
          a[1] = att_part_sum(sp + fr[1], sst, np);
        }
        for (int u = 0; u < 2; ++u) {
          const int t = tmin + tt[u], i = ii[u], jj = jq[u];
          const int nj = min(pos + t + 1, j0 + C) - j0;
          const bool valid = fr[0] < nh && fr[u] < nrow && jj < nj;
          const float scv = valid ? a[u] * scale : -INFINITY;
          const float m = row_max16(scv);
          const float e = valid ? expf(scv - m) : 0.f;
          const float l = row_sum16(e);
          if (fr[0] < nh && fr[u] < nrow) {
            const int ti = t * gs + i;
            pb[ti * C + jj] = e;
            if (jj == 0) {
              // position t's chunks of this item: c0 .. its last visible chunk
              const bool last = c + 1 == min(c1, (pos + t) / C + 1);
              float M = m, S = l, fr0 = 0.f, fr1 = 1.f;
              if (!first) {
                const float Mr = rin[2 * ti], Sr = rin[2 * ti + 1];
                const float Mn = fmaxf(Mr, M);
                const float f = expf(Mr - Mn), f1 = expf(M - Mn);
                S = fmaf(Sr, f, S * f1);
                M = Mn;
                fr0 = f;
                fr1 = f1;
              }
              mf[2 * ti] = fr0;
              mf[2 * ti + 1] = fr1;
              if (last) {
                MK_G mk_u64* part = L.ll_part + (size_t)t * tstride + (size_t)it * gs * (hd + 2) + i * (hd + 2);
                ll_put(part, cx.epoch, M);
                ll_put(part + 1, cx.epoch, S);
              } else {
                rout[2 * ti] = M;
                rout[2 * ti + 1] = S;
              }
            }
          }
        }
      }
      wg_bar();
      {
        // weighted values: thread (d, tg) keeps column d of the chunk's values in registers and
        // produces the (position, head) rows tg, tg + NG, ...; each output adds its 16 products in
        // slot order, then merges with the item's running acc by the row's factors
        const int NG = MK_NT / hd, nrows = (nt - tmin) * gs;
        const int d = tid() % hd, tg = tid() / hd;
        if (tg < NG) {
          float vcol[ATT_C];
#pragma unroll
          for (int jj = 0; jj < ATT_C; ++jj) vcol[jj] = vc[jj * hd + d];
          for (int rr = tg; rr < nrows; rr += NG) {
            const int tt = rr / gs, i = rr - tt * gs;
            const int t = tmin + tt;
            const int ti = t * gs + i;
            const int nj = min(pos + t + 1, j0 + C) - j0;
            f32x4 pw[ATT_C / 4];
#pragma unroll
            for (int q = 0; q < ATT_C / 4; ++q) pw[q] = *(const LS f32x4*)(pb + ti * C + 4 * q);
            float acc = 0.f;
            if (nj >= ATT_C) {
#pragma unroll
              for (int q = 0; q < ATT_C / 4; ++q) {
                acc = fmaf(pw[q].x, vcol[4 * q + 0], acc);
                acc = fmaf(pw[q].y, vcol[4 * q + 1], acc);
                acc = fmaf(pw[q].z, vcol[4 * q + 2], acc);
                acc = fmaf(pw[q].w, vcol[4 * q + 3], acc);
              }
            } else {
#pragma unroll
              for (int q = 0; q < ATT_C / 4; ++q) {
                acc = fmaf(pw[q].x, 4 * q + 0 < nj ? vcol[4 * q + 0] : 0.f, acc);
                acc = fmaf(pw[q].y, 4 * q + 1 < nj ? vcol[4 * q + 1] : 0.f, acc);
                acc = fmaf(pw[q].z, 4 * q + 2 < nj ? vcol[4 * q + 2] : 0.f, acc);
                acc = fmaf(pw[q].w, 4 * q + 3 < nj ? vcol[4 * q + 3] : 0.f, acc);
              }
            }
            if (!first) acc = fmaf(racc[ti * hd + d], mf[2 * ti], acc * mf[2 * ti + 1]);
            const bool last = c + 1 == min(c1, (pos + t) / C + 1);
            if (last) {
              MK_G mk_u64* part = L.ll_part + (size_t)t * tstride + (size_t)it * gs * (hd + 2) + i * (hd + 2);
              ll_put(part + 2 + d, cx.epoch, acc);
            } else {
              racc[ti * hd + d] = acc;
            }
          }
        }
      }
      wg_bar();  // LDS is reused by the next chunk
    }
  }
  return true;
}

// log-sum-exp merge (in chunk order) of every position's partials for outputs o[o0..o1) -> records;
// one gather serves all positions.  Position t (at pos + t) merges (pos + t) / 16 + 1 chunks; its
// staging block of vn outputs starts after the blocks of positions 0..t-1.  cap: floats of LDS
// staging available.
// items per KV head that position t (at pos + t) merges
__device__ __forceinline__ int comb_nch(int pos, int t, int cpi) {
  const int nch = (pos + t + ATT_C) / ATT_C;
  return (nch + cpi - 1) / cpi;
}
// items of positions 0 .. t-1 together
__device__ __forceinline__ int comb_before(int pos, int t, int cpi) {
  int n = 0;
  for (int u = 0; u < t; ++u) n += comb_nch(pos, u, cpi);
  return n;
}
__device__ __forceinline__ bool att_combine_v(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx,
                                              const Lds& s, LS float* stage, int cap, int o0, int o1, int pos,
                                              int nt) {
  const int hd = p.hd, nkv = p.nkv, gs = p.nq / p.nkv, K = p.nq * hd, cpi = p.att_cpi;
  const int nown = o1 - o0;
  if (nown <= 0) return true;
  const int tot = comb_before(pos, nt, cpi);
  const size_t tstride = (size_t)p.max_items * gs * (hd + 2);
  const int vpp = max(1, cap / (3 * tot));
  for (int v0 = 0; v0 < nown; v0 += vpp) {
    const int vn = min(vpp, nown - v0);
    const bool ok = gather_map_all(cx, vn * 3 * tot, [=](int f) {
      const int cf = f / (3 * vn);  // chunk slots of the positions before, in units of vn * 3 records
      int t = 0;
      while (t + 1 < nt && comb_before(pos, t + 1, cpi) <= cf) ++t;
      f -= 3 * vn * comb_before(pos, t, cpi);
      const int n = comb_nch(pos, t, cpi);
      const int which = f % 3;
      const int vc = f / 3;
      const int v = vc / n, c = vc - v * n;
      const int fo = o0 + v0 + v;
      const int i = fo / hd, d = fo - i * hd;
      const int g = i / gs, il = i - g * gs;
      const MK_G mk_u64* rec = L.ll_part + (size_t)t * tstride + ((size_t)(c * nkv + g) * gs + il) * (hd + 2);
      return rec + (which == 2 ? 2 + d : which);
    }, [=](int f, float v) { stage[f] = v; });
    if (wg_bar_or(s, !ok)) return false;
    if (streamer()) {
      for (int pr = wave(); pr < nt * vn; pr += NCW) {
        const int t = pr / vn, v = pr - t * vn;
        const int n = comb_nch(pos, t, cpi);
        const LS float* bp = stage + 3 * vn * comb_before(pos, t, cpi) + (size_t)v * n * 3;
        float M = -INFINITY;
        for (int c = lane(); c < n; c += 64) M = fmaxf(M, bp[3 * c]);
        M = wave_max(M);
        float num = 0.f, den = 0.f;
        for (int c = lane(); c < n; c += 64) {
          const float e = expf(bp[3 * c] - M);
          den = fmaf(e, bp[3 * c + 1], den);
          num = fmaf(e, bp[3 * c + 2], num);
        }
        num = wave_sum(num);
        den = wave_sum(den);
        if (lane() == 0) ll_put(L.ll_o + (size_t)t * K + o0 + v0 + v, cx.epoch, num / den);
      }
    }
    wg_bar();
  }
  return true;
}

// BF16 gains (n values, n a multiple of 8) -> LDS, by every thread, between barriers
__device__ __forceinline__ void load_gains(const MK_G uint16_t* src, int n, LS uint16_t* dst) {
  for (int i = tid(); i < (n >> 3); i += MK_NT) *(LS u32x4*)(dst + 8 * i) = *(const MK_G u32x4*)(src + 8 * i);
}

// Workgroup 0 takes the greedy choices y_1..y_nt from every workgroup's per-position (max, index)
// records, counts the accepted drafts a, writes the outputs and the new position and publishes a;
// then every workgroup restores its DeltaNet rows to the state after position a.  Shared by the BF16
// and 4-bit verify kernels.
__device__ __forceinline__ void verify_accept_rollback(const MkDecodeParams& p, const Ctx& cx, const Lds& s,
                                                       const LS int* toks, int NW, int w, int pos, int nt,
                                                       Tracer& tr) {
  // workgroup 0: greedy choices, accepted count, outputs, new position
  if (w == 0) {
    wg_bar();  // the running-argmax cells are read before the gather reuses the region
    const bool ok = gather_vec_all<false, PBV>(cx, p.ll_am, nt * 2 * NW, s.vec);
    if (wg_bar_or(s, !ok)) return;
    // wave t: position t's choice
    if (wave() < nt) {
      float b;
      int bi;
      wave_argmax(s.vec + wave() * 2 * NW, NW, b, bi);
      if (lane() == 0) {
        p.vout[wave()] = bi;
        ((LS int*)s.scr)[wave()] = bi;
      }
    }
    wg_bar();
    if (tid() == 0) {
      int a = 0;
      while (a + 1 < nt && toks[a + 1] == ((LS int*)s.scr)[a]) ++a;
      *p.vacc = a;
      ll_put(p.ll_acc, cx.epoch, __int_as_float(a));
      p.ctl->pos = pos + a + 1;
    }
  }
  tr.mark();
  // every workgroup: the accepted count, then its DeltaNet rows back to the state after position a
  {
    const bool ok = gather_vec_all<false, PBV>(cx, p.ll_acc, 1, s.scr);
    if (wg_bar_or(s, !ok)) return;
  }
  const int a = uni(__float_as_int(s.scr[0]));
  if (a + 1 < nt) {
    const int K = p.H * p.dv, dk = p.dk;
    const int s0 = split(K, NW, w), s1 = split(K, NW, w + 1);
    // The threads that wrote each snapshot element in dn_state_v copy it.  Loads for CB layers are
    // issued before their stores: a load issued after a store would wait for that store too.
    constexpr int CB = 8;
    for (int li = wave(); li < s1 - s0; li += MK_NWAVE) {
      const size_t ro = (size_t)(s0 + li) * dk;
      for (int l0 = 0; l0 < p.n_layers; l0 += CB) {
        float v[CB][4];
#pragma unroll
        for (int i = 0; i < CB; ++i) {
          const int l = l0 + i;
          const MkLayerDev L = layer_desc(s.desc, min(l, p.n_layers - 1));
          const bool dn = l < p.n_layers && L.kind == MK_LAYER_DN;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = lane() + 64 * c;
            v[i][c] = (dn && e < dk) ? L.Ssnap[(size_t)a * p.snap_stride + ro + e] : 0.f;
          }
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
          const int l = l0 + i;
          const MkLayerDev L = layer_desc(s.desc, min(l, p.n_layers - 1));
          const bool dn = l < p.n_layers && L.kind == MK_LAYER_DN;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = lane() + 64 * c;
            if (dn && e < dk) L.S[ro + e] = v[i][c];
          }
        }
      }
    }
  }
  tr.mark();
  tr.flush();
  if (w == 0) {
    wait_vm<0>();
    wg_bar();
    if (tid() == 0) p.ctl->step = cx.epoch + 1u;
  }
}

template <int D_, int FFN_, int H_, int DK_, int DV_, int NQ_, int NKV_, int HD_, bool KV_COMPACT>
__device__ __forceinline__ void verify_body(const MkDecodeParams& p0) {
  MkDecodeParams p = p0;
  if (!KV_COMPACT) p.kvt = MK_KV_F32;
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
  const int nt = uni(p.nt);
  Lds s;
  s.desc = (LS MkLayerDev*)(lds + p.lds_desc);
  s.gain = (LS uint16_t*)(lds + p.lds_gain);
  s.rope = lds + p.lds_rope;
  s.x = lds + p.lds_x;
  s.vec = lds + p.lds_vec;
  s.xn = (LS u32*)s.vec;  // normalised activations share the vector region (never live together)
  s.att = lds + p.lds_att;
  s.att_cap = MK_RED_CAP;
  s.scr = lds + p.lds_scr;
  s.flag = (LS int*)(lds + p.lds_flag);
  s.stA = nullptr;
  s.a_slots = 0;
  s.stB = nullptr;
  LS int* toks = (LS int*)(lds + p.lds_xn);  // the verify carve keeps the tokens in the xn slot
  const int D = p.D, F = p.ffn;
  const int vcap = uni(p.vec_floats);  // floats of the vector region

  Ctx cx;
  cx.ctl = p.ctl;
  cx.epoch = p.ctl->step;
  const int pos = p.ctl->pos;
  // bad token ids or a context that cannot take nt more positions: every workgroup sees the same
  // values and leaves before touching memory
  bool bad = nt < 1 || nt > VT || pos < 0 || pos + nt > p.max_ctx;
  for (int t = 0; t < VT; ++t)
    if (t < nt) {
      const int tk = p.vtok[t];
      bad = bad || tk < 0 || tk >= p.vocab;
    }
  if (bad) {
    if (w == 0 && tid() == 0) set_err(cx, 2u);
    return;
  }
  Tracer tr{(LS unsigned long long*)(lds + p.lds_trace), p.trace ? p.trace + (size_t)w * MK_TRACE_EVENTS : nullptr,
            0};
  tr.mark();
  {
    const int nw = p.n_layers * (int)(sizeof(MkLayerDev) / 4);
    const MK_G u32* dsrc = (const MK_G u32*)p.layers;
    for (int i = tid(); i < nw; i += MK_NT) ((LS u32*)s.desc)[i] = dsrc[i];
    if (tid() < nt) toks[tid()] = p.vtok[tid()];
    for (int i = tid(); i < nt * D; i += MK_NT) {
      const int t = i / D, c = i - t * D;
      s.x[i] = bf16f(p.embed[(size_t)p.vtok[t] * D + c]);
    }
    const int half = p.hd / 2;
    for (int i = tid(); i < nt * half; i += MK_NT) {
      const int t = i / half, m = i - t * half;
      s.rope[t * p.hd + m] = p.rope_cos[(size_t)(pos + t) * half + m];
      s.rope[t * p.hd + half + m] = p.rope_sin[(size_t)(pos + t) * half + m];
    }
    if (tid() == 0) *s.flag = 0;
  }

  const int d0 = split(D, NW, w), d1 = split(D, NW, w + 1);
  const int j0 = split(F, NW, w), j1 = split(F, NW, w + 1);
  int P0, P1;
  // the in-projection (or LM-head) rows of layer l
  auto input_rows = [&](int l, Gemv& g) {
    if (l < p.n_layers) {
      const MkLayerDev Ln = layer_desc(s.desc, l);
      pair_range(Ln.rows_in, NW, w, P0, P1);
      g.init(Ln.w_in + (size_t)2 * P0 * D, min(2 * P1, Ln.rows_in) - 2 * P0, D);
    } else {
      pair_range(p.vocab, NW, w, P0, P1);
      g.init(p.embed + (size_t)2 * P0 * D, min(2 * P1, p.vocab) - 2 * P0, D);
    }
  };
  wg_bar();  // descriptors
  GemvPre pre;  // the next GEMV's first units, loaded before the exchange that precedes it
  Gemv gin;
  input_rows(0, gin);
  gemv_v_pre(gin, nt, pre);
  for (int l = 0; l < p.n_layers; ++l) {
    const MkLayerDev L = layer_desc(s.desc, l);
    load_gains(L.g12, 2 * D, s.gain);
    wg_bar();
    tr.mark();
    rmsnorm_v(s.x, s.gain, s.xn, D, p.rms_eps, nt, s.scr);
    tr.mark();
    int K;
    Gemv gout;
    if (L.kind == MK_LAYER_DN) {
      K = p.H * p.dv;
      MK_G mk_u64* dst = L.ll_in + 2 * P0;
      const int rin = L.rows_in;
      gemv_v<false>(gin, s.xn, D, nt, s.att, pre,
                    [&](int r, int t, float v, float) { ll_put(dst + (size_t)t * rin + r, cx.epoch, v); });
      tr.mark();
      gout.init(L.w_out + (size_t)d0 * K, d1 - d0, K);
      gemv_v_pre(gout, nt, pre);
      const int s0 = split(K, NW, w), s1 = split(K, NW, w + 1);
      if (!dn_state_v(p, L, cx, s, s.vec, s.scr, s0, s1, nt)) return;
    } else {
      K = p.nq * p.hd;
      att_qkv_v(p, L, cx, s, gin, pre, P0, pos, nt);
      tr.mark();
      gout.init(L.w_out + (size_t)d0 * K, d1 - d0, K);
      gemv_v_pre(gout, nt, pre);
      if (!att_items_v<!KV_COMPACT>(p, L, cx, s, s.vec, NW, w, pos, nt)) return;
      const int o0 = split(K, NW, w), o1 = split(K, NW, w + 1);
      if (!att_combine_v(p, L, cx, s, s.vec, vcap, o0, o1, pos, nt)) return;
    }
    tr.mark();
    // mixer outputs of every position -> out-projection rows + residual -> records
    {
      const bool ok = gather_vec_all<false, PBV>(cx, L.ll_o, nt * K, s.vec);
      if (wg_bar_or(s, !ok)) return;
      for (int t = 0; t < nt; ++t) to_hl(s.vec + t * K, K);
      wg_bar();
    }
    tr.mark();
    gemv_v<false>(gout, (const LS u32*)s.vec, K, nt, s.att, pre, [&](int r, int t, float v, float) {
      ll_put(L.ll_x1 + (size_t)t * D + d0 + r, cx.epoch, s.x[t * D + d0 + r] + v);
    });
    tr.mark();
    Gemv ggu;
    ggu.init(L.w_gu + (size_t)2 * j0 * D, 2 * (j1 - j0), D);
    gemv_v_pre(ggu, nt, pre);
    {
      const bool ok = gather_vec_all<false, PBV>(cx, L.ll_x1, nt * D, s.x);
      if (wg_bar_or(s, !ok)) return;
    }
    tr.mark();
    rmsnorm_v(s.x, s.gain + D, s.xn, D, p.rms_eps, nt, s.scr);
    tr.mark();
    gemv_v<true>(ggu, s.xn, D, nt, s.att, pre, [&](int j, int t, float gv, float uv) {
      ll_put(L.ll_h + (size_t)t * F + j0 + j, cx.epoch, gv / (1.0f + expf(-gv)) * uv);
    });
    tr.mark();
    Gemv gdn;
    gdn.init(L.w_down + (size_t)d0 * F, d1 - d0, F);
    gemv_v_pre(gdn, nt, pre);
    {
      const bool ok = gather_vec_all<true, PBV>(cx, L.ll_h, nt * F, s.vec);
      if (wg_bar_or(s, !ok)) return;
    }
    tr.mark();
    gemv_v<false>(gdn, (const LS u32*)s.vec, F, nt, s.att, pre, [&](int r, int t, float v, float) {
      ll_put(L.ll_x2 + (size_t)t * D + d0 + r, cx.epoch, s.x[t * D + d0 + r] + v);
    });
    tr.mark();
    input_rows(l + 1, gin);
    gemv_v_pre(gin, nt, pre);
    {
      const bool ok = gather_vec_all<false, PBV>(cx, L.ll_x2, nt * D, s.x);
      if (wg_bar_or(s, !ok)) return;
    }
  }

  tr.mark();
  // final norm + tied LM head + per-position argmax (lowest index among equal maxima)
  load_gains(p.g_final, D, s.gain);
  wg_bar();
  rmsnorm_v(s.x, s.gain, s.xn, D, p.rms_eps, nt, s.scr);
  {
    const Gemv ghead = gin;  // the LM-head rows, first units already loaded
    // running argmax per (position, streaming thread) in LDS, after the normalised activations
    LS float* amv = s.vec + nt * D;
    LS int* ami = (LS int*)(amv + nt * NCT);
    for (int i = tid(); i < nt * NCT; i += MK_NT) {
      amv[i] = -INFINITY;
      ami[i] = 0x7fffffff;
    }
    wg_bar();
    const int v0 = 2 * P0;
    gemv_v<false>(ghead, s.xn, D, nt, s.att, pre, [&](int r, int t, float v, float) {
      const int idx = v0 + r;
      const int c = t * NCT + tid();
      if (v > amv[c] || (v == amv[c] && idx < ami[c])) {
        amv[c] = v;
        ami[c] = idx;
      }
    });
    tr.mark();
    // wave t: the workgroup's winner for position t (largest value, lowest index)
    if (wave() < nt) {
      const int t = wave();
      float b = -INFINITY;
      int bi = 0x7fffffff;
      for (int i = lane(); i < NCT; i += 64) {
        const float ob = amv[t * NCT + i];
        const int oi = ami[t * NCT + i];
        if (ob > b || (ob == b && oi < bi)) {
          b = ob;
          bi = oi;
        }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ob = __shfl_xor(b, m, 64);
        const int oi = __shfl_xor(bi, m, 64);
        if (ob > b || (ob == b && oi < bi)) {
          b = ob;
          bi = oi;
        }
      }
      if (lane() == 0) {
        ll_put(p.ll_am + (size_t)t * 2 * NW + 2 * w, cx.epoch, b);
        ll_put(p.ll_am + (size_t)t * 2 * NW + 2 * w + 1, cx.epoch, __int_as_float(bi));
      }
    }
  }
  verify_accept_rollback(p, cx, s, toks, NW, w, pos, nt, tr);
}

// ================================================================ 4-bit (Q4G32) speculative verify
// The same launch for 4-bit weights: the 4-bit decode kernel's arithmetic on nt positions (the
// activations of every position packed per 32-column block as that kernel packs them, the same
// unit sums, wave reduction and segment order; DeltaNet rows, attention items and combine as in
// the BF16 verify above), so every choice equals, bit for bit, the one a 4-bit decode launch makes.
// At the 27B-scale widths nt positions' residuals and FFN hidden vectors do not fit a workgroup's
// LDS, so:
//  - the residual lives in the exchange records (the mixer and FFN outputs are published as the
//    residual after the add, as in decode); a workgroup keeps only its own rows per position (xr),
//    and gathers a position's whole residual when its RMSNorm scale is formed;
//  - every GEMV runs over column groups of whole 2048-column segments, as many as the packed
//    activations of all nt positions fit the vector region; a group's activations are gathered (or
//    normalised) and packed, its units applied to every position, and a row's segment partials
//    summed in segment order once all groups are done.  Every weight is read once.
constexpr int Q4V_CTR = 1;  // the GEMV unit counter sits after the abort flag

// words of packed activations for n columns (n a multiple of 32)
__device__ __forceinline__ int q4v_pw(int n) { return (n >> 5) * Q4_XW; }

// segments per column group: every position's columns of the group side by side, nt * cols <= cap
// (each position's columns are packed in place, so position t's packed words start at t * cols),
// and no more columns than one q4_pack call takes
__device__ __forceinline__ int q4v_group_segs(int cap, int nt) {
  return max(1, min(cap / (nt * Q4_COLS), 8 * MK_NT * Q4_PACK_IT / Q4_COLS));
}

// rows of one chunk: the segment partials of all nt positions fit MK_RED_CAP (whole 4-row blocks)
__device__ __forceinline__ int q4v_rows(int S, int nt) { return max(4, (MK_RED_CAP / (S * nt)) & ~3); }

// Unit sources of a (row chunk, column group): units u = rb * Sg + (s - sg0), s in [sg0, sg0 + Sg).
struct Q4SrcV {
  __amdgpu_buffer_rsrc_t rt;
  int U, G, Sg, sg0;
  __device__ __forceinline__ void init(const GemvQ4& g, int sg0_, int Sg_) {
    const MK_G uint8_t* T = uni_ptr(g.T);
    const int R = uni(g.R), RB = (R + 3) >> 2;
    G = uni(g.K) >> 5;
    sg0 = uni(sg0_);
    Sg = uni(Sg_);
    U = RB * Sg;
    rt = __builtin_amdgcn_make_buffer_rsrc((void*)T, 0, RB * G * Q4_TILE, 0x00020000);
  }
  __device__ __forceinline__ void issue(Q4Unit& r, int u) const {
    constexpr int OOB = 0x7ffffff0;  // past the resource: the load returns zeros
    const int rb = u / Sg, s = sg0 + (u - rb * Sg);
    const int ng = min(64, G - 64 * s);
    const bool live = u < U && lane() < ng;
    const int o = rb * G * Q4_TILE + s * 64 * Q4_TILE + lane() * 16;
    const int pl = ng * 16;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      r.c[k] = __builtin_amdgcn_raw_buffer_load_b128(rt, live ? o + k * pl : OOB, 0, 2 /* nt */);
    r.p = __builtin_amdgcn_raw_buffer_load_b128(rt, live ? o + 4 * pl : OOB, 0, 2 /* nt */);
  }
};

__device__ __forceinline__ int q4v_grab(LS int* ctr) {
  int v = 0;
  if (lane() == 0) v = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return __builtin_amdgcn_readfirstlane(v);
}

// Partials of the units of rows [0, g.R) x segments [sg0, sg0 + Sg) for nt positions -> red[t][row][s]
// (S segments per row).  Position t's packed activations of the group start at P + t * pstride
// words; xp_t is shifted back so that column c's block is found at (c >> 5) * Q4_XW.  All eight
// waves take units from the LDS counter, Q4_RING in flight each (as gemv_q4_partials).
__device__ __forceinline__ void q4v_partials(const GemvQ4& g, int sg0, int Sg, const LS u32* P, int pstride, int nt,
                                             LS float* red, LS int* ctr) {
  Q4SrcV src;
  src.init(g, sg0, Sg);
  const int R = uni(g.R), K = uni(g.K), S = uni(g.S), U = src.U;
  const int blk = R * S;
  const LS u32* xb = P - (sg0 * Q4_COLS >> 5) * Q4_XW;
  Q4Ring q;
#pragma unroll
  for (int k = 0; k < Q4_RING; ++k) {
    q.uk[k] = q4v_grab(ctr);
    src.issue(q.r[k], q.uk[k]);
  }
  while (q.uk[0] < U) {
#pragma unroll
    for (int k = 0; k < Q4_RING; ++k) {
      const bool live = q.uk[k] < U;
      if (live) {
        const int u = q.uk[k], rb = u / Sg, s = sg0 + (u - rb * Sg);
#pragma unroll 1
        for (int t = 0; t < nt; ++t) {
          Q4X x;
          q4_load_x(x, xb + t * pstride, s, K);
          const float a0 = q4_row(q.r[k].c[0], q.r[k].p.x, x);
          const float a1 = q4_row(q.r[k].c[1], q.r[k].p.y, x);
          const float a2 = q4_row(q.r[k].c[2], q.r[k].p.z, x);
          const float a3 = q4_row(q.r[k].c[3], q.r[k].p.w, x);
          const float v = reduce_rows4(a0, a1, a2, a3);
          if ((lane() & 15) == 0) {
            const int row = rb * 4 + (lane() >> 4);
            if (row < R) red[t * blk + row * S + s] = v;
          }
        }
      }
      q.uk[k] = live ? q4v_grab(ctr) : U;
      src.issue(q.r[k], q.uk[k]);
    }
  }
  wait_vm<0>();  // the ring's last loads read zeros; wait for them before the registers are reused
}

// W . x_t over a workgroup's rows for nt positions.  pack(c0, n, P) fills the packed activations of
// columns [c0, c0 + n) of every position (position t's at P + t * n words), ends
// with a barrier and returns false when a wait gave up (the same in every thread); epi(row, t, v, 0)
// or, PAIRS, epi(pair, t, v_even, v_odd) runs on the streaming threads once a row chunk's groups are
// done.  Returns false when a pack failed.
// PACKED: pack() gathers words that are already packed, position t's at P + t (n / 32) Q4_XW, so a
// column group takes 0.625 of the LDS of FP32 values and groups are that much wider.
template <bool PAIRS, bool PACKED = false, typename Pack, typename Epi>
__device__ __forceinline__ bool gemv_q4_v(const GemvQ4& G, int nt, LS float* P, int pcap, LS float* red, LS int* ctr,
                                          Pack pack, Epi epi) {
  const int S = uni(G.S), K = uni(G.K);
  nt = uni(nt);
  // one group when every position's columns fit (then they are packed once for all row chunks)
  const int gs = PACKED ? (nt * (K >> 5) * Q4_XW <= pcap ? S : min(S, max(1, pcap / (nt * (Q4_COLS >> 5) * Q4_XW))))
                        : (nt * K <= pcap && K <= 8 * MK_NT * Q4_PACK_IT ? S : min(S, q4v_group_segs(pcap, nt)));
  const int ngroups = (S + gs - 1) / gs;
  const int rc = q4v_rows(S, nt);
  for (int r0 = 0; r0 == 0 || r0 < G.R; r0 += rc) {
    GemvQ4 g = G;
    g.T = G.T + (size_t)(r0 >> 2) * (size_t)(K >> 5) * Q4_TILE;
    g.R = max(0, min(rc, G.R - r0));
    for (int gi = 0; gi < ngroups; ++gi) {
      const int sg0 = gi * gs, Sg = min(gs, S - sg0);
      const int c0 = sg0 * Q4_COLS, n = min(K, (sg0 + Sg) * Q4_COLS) - c0;
      const int pstride = PACKED ? (n >> 5) * Q4_XW : n;  // position t's packed words start at t * pstride
      if ((ngroups > 1 || r0 == 0) && !pack(c0, n, P)) return false;  // one group: packed once
      if (g.R > 0) q4v_partials(g, sg0, Sg, (const LS u32*)P, pstride, nt, red, ctr);
      wg_bar();
      if (tid() == 0) *ctr = 0;  // the next grab comes after at least one more barrier
    }
    if (streamer()) {
      const int nr = PAIRS ? g.R / 2 : g.R, blk = g.R * S;
      for (int i = tid(); i < nt * nr; i += NCT) {
        const int t = i / nr, j = i - t * nr;
        const LS float* rt = red + t * blk;
        if (PAIRS) epi(r0 / 2 + j, t, seg_sum(rt + (2 * j) * S, S), seg_sum(rt + (2 * j + 1) * S, S));
        else epi(r0 + j, t, seg_sum(rt + j * S, S), 0.f);
      }
    }
    wg_bar();  // red (and P, for the next chunk's groups) are reused
  }
  return true;
}

// Columns [c0, c0 + n) of a 4-bit embedding row -> dst[0..n) in FP32 (q4_embed_row's values).
__device__ __forceinline__ void q4_embed_cols(const MK_G uint16_t* E, int D, int tok, int c0, int n, LS float* dst) {
  const int G = D >> 5;
  const MK_G uint8_t* rowb = (const MK_G uint8_t*)E + (size_t)(tok >> 2) * (size_t)G * Q4_TILE;
  const int r = tok & 3;
  for (int i = tid() + (c0 >> 3); i < ((c0 + n) >> 3); i += MK_NT) {
    const int gi = i >> 2, s = gi >> 6, l = gi & 63, ng = min(64, G - 64 * s);
    const MK_G uint8_t* seg = rowb + (size_t)s * 64 * Q4_TILE;
    const u32 v = *(const MK_G u32*)(seg + r * ng * 16 + l * 16 + 4 * (i & 3));
    const u32 pw = *(const MK_G u32*)(seg + 4 * ng * 16 + l * 16 + 4 * r);
    const float d = f16_lo(pw), m = f16_hi(pw);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[8 * i - c0 + 2 * j] = fmaf(d, (float)((v >> (4 * j)) & 15u), m);
      dst[8 * i - c0 + 2 * j + 1] = fmaf(d, (float)((v >> (16 + 4 * j)) & 15u), m);
    }
  }
}

// Columns [c0, c0 + n) of every position's vector -> dst + t * n: records src[t][stride] (one gather
// for all positions), or, for the first layer's residual (src == nullptr), the embedding rows of the
// tokens.  Every thread calls it; ends with a barrier; false when a wait gave up.
__device__ __forceinline__ bool q4v_gather(const Ctx& cx, const Lds& s, const MK_G uint16_t* E, int D,
                                          const LS int* toks, const MK_G mk_u64* src, int stride, int nt, int c0,
                                          int n, LS float* dst) {
  bool ok = true;
  if (src) {
    ok = gather_map_all(cx, nt * n, [=](int f) {
      const int t = f / n;
      return src + (size_t)t * stride + c0 + (f - t * n);
    }, [=](int f, float v) { dst[f] = v; });
  } else {
    for (int t = 0; t < nt; ++t) q4_embed_cols(E, D, toks[t], c0, n, dst + t * n);
  }
  return !wg_bar_or(s, !ok);
}

// RMSNorm scales of nt residuals, rs[t] = 1 / sqrt(mean x_t^2 + eps), and this workgroup's residual
// rows [d0, d1) of each position -> xr[t * rstride ..].  whole: the residuals came in one gather and
// are left at P + t * D.  The residuals come in chunks of whole
// 1024-value strides of the 4-bit decode kernel's rmsnorm_gg (all positions per gather); wave t
// carries position t's running per-lane sum through the chunks in exactly that kernel's order, so the
// scale is bit-identical.
__device__ __forceinline__ bool q4v_norm_scales(const Ctx& cx, const Lds& s, const MK_G uint16_t* E, int D,
                                                const LS int* toks, const MK_G mk_u64* src, int nt, float eps,
                                                LS float* P, int pcap, LS float* rs, LS float* xr, int rstride,
                                                int d0, int d1, bool& whole) {
  const int D4 = D >> 2;
  const int ch = max(1024, (pcap / nt) / 1024 * 1024);
  whole = ch >= D;  // one gather: every position's residual is left at P + t * D
  float sq = 0.f;
  for (int a = 0; a < D; a += ch) {
    const int n = min(ch, D - a);
    if (!q4v_gather(cx, s, E, D, toks, src, D, nt, a, n, P)) return false;
    if (wave() < nt) {
      const LS f32x4* x4 = (const LS f32x4*)(P + wave() * n) - (a >> 2);  // indexed by the residual's f32x4
      for (int c0 = (a >> 2) + lane(); c0 < min((a + n) >> 2, D4); c0 += 256) {
        f32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[k] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (c0 + 64 * k < D4) v[k] = x4[c0 + 64 * k];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          sq = fmaf(v[k].x, v[k].x, sq);
          sq = fmaf(v[k].y, v[k].y, sq);
          sq = fmaf(v[k].z, v[k].z, sq);
          sq = fmaf(v[k].w, v[k].w, sq);
        }
      }
    }
    const int nr = d1 - d0;
    for (int i = tid(); i < nt * nr; i += MK_NT) {
      const int t = i / nr, r = i - t * nr, col = d0 + r;
      if (col >= a && col < a + n) xr[t * rstride + r] = P[t * n + col - a];
    }
    wg_bar();
  }
  if (wave() < nt) {
    sq = wave_sum(sq);
    if (lane() == 0) rs[wave()] = 1.0f / sqrtf(sq / (float)D + eps);
  }
  wg_bar();
  return true;
}

// Packed normalised activations of columns [c0, c0 + n) for every position (position t at P + t * n):
// x * rs[t] * g, as rmsnorm_gg scales, then q4_pack.  resident: the norm left every whole residual
// in P, so all columns need no second gather.
__device__ __forceinline__ bool q4v_pack_norm(const Ctx& cx, const Lds& s, const MK_G uint16_t* E, int D,
                                              const LS int* toks, const MK_G mk_u64* src, int nt,
                                              const MK_G uint16_t* g, const LS float* rs, int c0, int n, LS float* P,
                                              bool resident) {
  if (!(resident && c0 == 0 && n == D) && !q4v_gather(cx, s, E, D, toks, src, D, nt, c0, n, P)) return false;
  const int n4 = n >> 2;
  for (int i = tid(); i < nt * n4; i += MK_NT) {
    const int t = i / n4, c = i - t * n4;
    const float r = rs[t];
    const f32x4 v = ((LS f32x4*)P)[i];
    const u32x2 gg = *(const MK_G u32x2*)(g + c0 + 4 * c);
    ((LS f32x4*)P)[i] = f32x4{v.x * r * __uint_as_float(gg.x << 16), v.y * r * __uint_as_float(gg.x & 0xffff0000u),
                              v.z * r * __uint_as_float(gg.y << 16), v.w * r * __uint_as_float(gg.y & 0xffff0000u)};
  }
  wg_bar();
  for (int t = 0; t < nt; ++t) q4_pack(P + t * n, n);
  return true;
}

// Packed activations of columns [c0, c0 + n) (n a multiple of 32) for every position from records
// that already hold packed words -- position t's at src + t * stride, block b's Q4_XW words at
// b * Q4_XW -- to P + t * pw, pw = (n / 32) Q4_XW (the packed stride of gemv_q4_v<.., true>).  Every
// thread calls it; ends with a barrier.
__device__ __forceinline__ bool q4v_gather_packed(const Ctx& cx, const Lds& s, const MK_G mk_u64* src, int stride,
                                                  int nt, int c0, int n, LS float* P) {
  const int pw = (n >> 5) * Q4_XW, w0 = (c0 >> 5) * Q4_XW;
  const bool ok = gather_map_all(cx, nt * pw, [=](int f) {
    const int t = f / pw;
    return src + (size_t)t * stride + w0 + (f - t * pw);
  }, [=](int f, float v) { P[f] = v; });
  return !wg_bar_or(s, !ok);
}

// Packed record vectors: columns [c0, c0 + n) of src[t][stride] for every position (at P + t * n).
__device__ __forceinline__ bool q4v_pack_records(const Ctx& cx, const Lds& s, const MK_G mk_u64* src, int stride,
                                                 int nt, int c0, int n, LS float* P) {
  if (!q4v_gather(cx, s, nullptr, 0, nullptr, src, stride, nt, c0, n, P)) return false;
  for (int t = 0; t < nt; ++t) q4_pack(P + t * n, n);
  return true;
}

template <bool ONE_PART>
__device__ __forceinline__ void verify_q4_body(const MkDecodeParams& p) {
  extern __shared__ float lds_raw[];
  LS float* lds = (LS float*)lds_raw;
  const int NW = (int)gridDim.x, w = (int)blockIdx.x;
  const int nt = uni(p.nt);
  Lds s;
  s.desc = (LS MkLayerDev*)(lds + p.lds_desc);
  s.gain = nullptr;
  s.rope = lds + p.lds_rope;
  s.x = lds + p.lds_x;     // this workgroup's residual rows [t][rstride]
  s.vec = lds + p.lds_vec; // packed activations, gathered vectors, DeltaNet / attention / combine scratch
  s.xn = (LS u32*)s.vec;
  s.att = lds + p.lds_att; // GEMV partials
  s.att_cap = MK_RED_CAP;
  s.scr = lds + p.lds_scr;
  s.flag = (LS int*)(lds + p.lds_flag);
  s.stA = nullptr;
  s.a_slots = 0;
  s.stB = nullptr;
  LS int* toks = (LS int*)(lds + p.lds_xn);
  LS int* ctr = s.flag + Q4V_CTR;
  LS float* rs = s.scr + 2 * VT * MK_NWAVE - VT;  // RMSNorm scales, after the reduction cells
  const int D = p.D, F = p.ffn;
  const int pcap = uni(p.vec_floats);
  const int rstride = uni(p.rstride);  // residual rows per position

  Ctx cx;
  cx.ctl = p.ctl;
  cx.epoch = p.ctl->step;
  const int pos = p.ctl->pos;
  bool bad = nt < 1 || nt > VT || pos < 0 || pos + nt > p.max_ctx;
  for (int t = 0; t < VT; ++t)
    if (t < nt) {
      const int tk = p.vtok[t];
      bad = bad || tk < 0 || tk >= p.vocab;
    }
  if (bad) {
    if (w == 0 && tid() == 0) set_err(cx, 2u);
    return;
  }
  Tracer tr{(LS unsigned long long*)(lds + p.lds_trace), p.trace ? p.trace + (size_t)w * MK_TRACE_EVENTS : nullptr,
            0};
  tr.mark();
  {
    if (tid() < nt) toks[tid()] = p.vtok[tid()];
    const int half = p.hd / 2;
    for (int i = tid(); i < nt * half; i += MK_NT) {
      const int t = i / half, m = i - t * half;
      s.rope[t * p.hd + m] = p.rope_cos[(size_t)(pos + t) * half + m];
      s.rope[t * p.hd + half + m] = p.rope_sin[(size_t)(pos + t) * half + m];
    }
    if (tid() == 0) {
      *s.flag = 0;
      *ctr = 0;
    }
  }
  wg_bar();

  // the 4-bit decode kernel's row slices: residual-sized projections and FFN pairs in whole 4-row
  // blocks, in-projection and LM-head rows by 4-row blocks
  const int d0 = 4 * split(D >> 2, NW, w), d1 = min(D, 4 * split(D >> 2, NW, w + 1));
  // FFN hidden columns by whole 32-column blocks, so that each workgroup packs its own slice of the
  // down projection's input once (the 4-bit decode kernel packs the same blocks from the same values)
  const int j0 = 32 * split(F >> 5, NW, w), j1 = 32 * split(F >> 5, NW, w + 1);
  auto in_slice = [&](const MkLayerDev& Lx, GemvQ4& g, int& P0) {
    const int nbi = (Lx.rows_in + 3) >> 2;
    const int B0 = split(nbi, NW, w), B1 = split(nbi, NW, w + 1);
    P0 = 2 * B0;
    g.init(Lx.w_in, B0, max(0, min(4 * B1, Lx.rows_in) - 4 * B0), D);
  };
  const MK_G mk_u64* xsrc = nullptr;  // the residual's records (null: the embedding rows)
  bool whole = false;                 // the last norm left every whole residual in s.vec
  for (int l = 0; l < p.n_layers; ++l) {
    const MkLayerDev L = p.layers[l];  // read-only descriptors (uniform loads)
    if (!q4v_norm_scales(cx, s, p.embed, D, toks, xsrc, nt, p.rms_eps, s.vec, pcap, rs, s.x, rstride, d0, d1,
                         whole))
      return;
    tr.mark();
    auto pack_in = [&](int c0, int n, LS float* P) {
      return q4v_pack_norm(cx, s, p.embed, D, toks, xsrc, nt, L.g12, rs, c0, n, P, whole);
    };
    int P0;
    GemvQ4 gin;
    in_slice(L, gin, P0);
    int K;
    if (L.kind == MK_LAYER_DN) {
      K = p.H * p.dv;
      const int rin = L.rows_in;
      MK_G mk_u64* dst = L.ll_in + 2 * P0;
      if (!gemv_q4_v<false>(gin, nt, s.vec, pcap, s.att, ctr, pack_in,
                            [&](int r, int t, float v, float) { ll_put(dst + (size_t)t * rin + r, cx.epoch, v); }))
        return;
      tr.mark();
      const int s0 = split(K, NW, w), s1 = split(K, NW, w + 1);
      if (!dn_state_v(p, L, cx, s, s.vec, s.scr, s0, s1, nt)) return;
    } else {
      K = p.nq * p.hd;
      if (!gemv_q4_v<true>(gin, nt, s.vec, pcap, s.att, ctr, pack_in, [&](int pl, int t, float x1, float x2) {
            att_qkv_v_put(p, L, cx, s, P0 + pl, t, pos, x1, x2);
          }))
        return;
      tr.mark();
      if (!att_items_v<true, ONE_PART>(p, L, cx, s, s.vec, NW, w, pos, nt)) return;
      const int o0 = split(K, NW, w), o1 = split(K, NW, w + 1);
      if (!att_combine_v(p, L, cx, s, s.vec, pcap, o0, o1, pos, nt)) return;
    }
    tr.mark();
    // mixer outputs -> out-projection rows + residual -> records (the residual after the mixer)
    {
      GemvQ4 gout;
      gout.init(L.w_out, d0 >> 2, d1 - d0, K);
      if (!gemv_q4_v<false>(
              gout, nt, s.vec, pcap, s.att, ctr,
              [&](int c0, int n, LS float* P) { return q4v_pack_records(cx, s, L.ll_o, K, nt, c0, n, P); },
              [&](int r, int t, float v, float) {
                ll_put(L.ll_x1 + (size_t)t * D + d0 + r, cx.epoch, s.x[t * rstride + r] + v);
              }))
        return;
    }
    tr.mark();
    xsrc = L.ll_x1;
    if (!q4v_norm_scales(cx, s, p.embed, D, toks, xsrc, nt, p.rms_eps, s.vec, pcap, rs, s.x, rstride, d0, d1,
                         whole))
      return;
    {
      GemvQ4 ggu;
      ggu.init(L.w_gu, j0 >> 1, 2 * (j1 - j0), D);
      // this workgroup's FFN hidden values [t][hw] in the LM head's argmax cells (not live here)
      LS float* hb = s.att + MK_RED_CAP;
      const int hw = j1 - j0;
      if (!gemv_q4_v<true>(
              ggu, nt, s.vec, pcap, s.att, ctr,
              [&](int c0, int n, LS float* P) {
                return q4v_pack_norm(cx, s, p.embed, D, toks, xsrc, nt, L.g12 + D, rs, c0, n, P, whole);
              },
              [&](int j, int t, float gv, float uv) { hb[t * hw + j] = gv / (1.0f + expf(-gv)) * uv; }))
        return;
      // pack the slice (blocks are packed independently, so position t's blocks follow t - 1's) and
      // publish the packed words: position t's at ll_h + t * F, block b's at b * Q4_XW
      if (hw > 0) {
        q4_pack(hb, nt * hw);
        const int pw = (hw >> 5) * Q4_XW;
        for (int i = tid(); i < nt * pw; i += MK_NT) {
          const int t = i / pw, r = i - t * pw;
          ll_put(L.ll_h + (size_t)t * F + (j0 >> 5) * Q4_XW + r, cx.epoch, hb[t * pw + r]);
        }
      }
    }
    tr.mark();
    {
      GemvQ4 gdn;
      gdn.init(L.w_down, d0 >> 2, d1 - d0, F);
      if (!gemv_q4_v<false, true>(
              gdn, nt, s.vec, pcap, s.att, ctr,
              [&](int c0, int n, LS float* P) { return q4v_gather_packed(cx, s, L.ll_h, F, nt, c0, n, P); },
              [&](int r, int t, float v, float) {
                ll_put(L.ll_x2 + (size_t)t * D + d0 + r, cx.epoch, s.x[t * rstride + r] + v);
              }))
        return;
    }
    tr.mark();
    xsrc = L.ll_x2;
  }

  // final norm + tied LM head + per-position argmax (lowest index among equal maxima)
  if (!q4v_norm_scales(cx, s, p.embed, D, toks, xsrc, nt, p.rms_eps, s.vec, pcap, rs, s.x, rstride, d0, d1, whole))
    return;
  {
    LS float* amv = s.att + MK_RED_CAP;  // running argmax per (position, streaming thread)
    LS int* ami = (LS int*)(amv + nt * NCT);
    for (int i = tid(); i < nt * NCT; i += MK_NT) {
      amv[i] = -INFINITY;
      ami[i] = 0x7fffffff;
    }
    wg_bar();
    const int nbv = (p.vocab + 3) >> 2;
    const int B0 = split(nbv, NW, w), B1 = split(nbv, NW, w + 1);
    const int v0 = 4 * B0;
    GemvQ4 gl;
    gl.init(p.embed, B0, max(0, min(4 * B1, p.vocab) - 4 * B0), D);
    const bool hok = gemv_q4_v<false>(
        gl, nt, s.vec, pcap, s.att, ctr,
        [&](int c0, int n, LS float* P) {
          return q4v_pack_norm(cx, s, p.embed, D, toks, xsrc, nt, p.g_final, rs, c0, n, P, whole);
        },
        [&](int r, int t, float v, float) {
                       const int idx = v0 + r;
                       const int c = t * NCT + tid();
          if (v > amv[c] || (v == amv[c] && idx < ami[c])) {
            amv[c] = v;
            ami[c] = idx;
          }
        });
    if (!hok) return;
    tr.mark();
    if (wave() < nt) {
      const int t = wave();
      float b = -INFINITY;
      int bi = 0x7fffffff;
      for (int i = lane(); i < NCT; i += 64) {
        const float ob = amv[t * NCT + i];
        const int oi = ami[t * NCT + i];
        if (ob > b || (ob == b && oi < bi)) {
          b = ob;
          bi = oi;
        }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ob = __shfl_xor(b, m, 64);
        const int oi = __shfl_xor(bi, m, 64);
        if (ob > b || (ob == b && oi < bi)) {
          b = ob;
          bi = oi;
        }
      }
      if (lane() == 0) {
        ll_put(p.ll_am + (size_t)t * 2 * NW + 2 * w, cx.epoch, b);
        ll_put(p.ll_am + (size_t)t * 2 * NW + 2 * w + 1, cx.epoch, __int_as_float(bi));
      }
    }
  }
  // the rollback walks every layer's descriptor: the table goes to the tail of the vector region,
  // which is free from here on
  {
    const int nw = p.n_layers * (int)(sizeof(MkLayerDev) / 4);
    const MK_G u32* dsrc = (const MK_G u32*)p.layers;
    for (int i = tid(); i < nw; i += MK_NT) ((LS u32*)s.desc)[i] = dsrc[i];
  }
  wg_bar();
  verify_accept_rollback(p, cx, s, toks, NW, w, pos, nt, tr);
}

}  // namespace

__global__ void __launch_bounds__(MK_NT, 1) mk_verify_kernel(MkDecodeParams p) {
  verify_body<0, 0, 0, 0, 0, 0, 0, 0, false>(p);
}
// hidden 1024, FFN 3584, 16 DeltaNet heads of 128, 8 Q / 2 KV heads of 128 (the 0.8B-shaped hybrid)
__global__ void __launch_bounds__(MK_NT, 1) mk_verify_kernel_h1024(MkDecodeParams p) {
  verify_body<1024, 3584, 16, 128, 128, 8, 2, 128, false>(p);
}
// binary16 or int8 KV cache
__global__ void __launch_bounds__(MK_NT, 1) mk_verify_kernel_kvc(MkDecodeParams p) {
  verify_body<0, 0, 0, 0, 0, 0, 0, 0, true>(p);
}

namespace {
typedef void (*VerifyKernel)(MkDecodeParams);
VerifyKernel pick_verify(const MkDecodeParams& p) {
  if (p.kvt != MK_KV_F32) return mk_verify_kernel_kvc;
  if (p.D == 1024 && p.ffn == 3584 && p.H == 16 && p.dk == 128 && p.dv == 128 && p.nq == 8 && p.nkv == 2 &&
      p.hd == 128)
    return mk_verify_kernel_h1024;
  return mk_verify_kernel;
}
}  // namespace

// 4-bit weights (any KV cache type); the second instance serves shapes whose attention scores are one
// part (the 27B-scale shape among them) without the code for several
__global__ void __launch_bounds__(MK_NT, 1) mk_verify_q4_kernel(MkDecodeParams p) { verify_q4_body<false>(p); }
__global__ void __launch_bounds__(MK_NT, 1) mk_verify_q4_kernel_1p(MkDecodeParams p) { verify_q4_body<true>(p); }

namespace {
VerifyKernel pick_verify_q4(const MkDecodeParams& p) {
  return att_parts(p.nq / p.nkv, p.hd) == 1 && (p.hd / 4) % 8 == 0 ? mk_verify_q4_kernel_1p : mk_verify_q4_kernel;
}
}  // namespace

extern "C" int mk_launch_verify_q4(const MkDecodeParams* p, int n_wg, void* stream) {
  hipLaunchKernelGGL(pick_verify_q4(*p), dim3(n_wg), dim3(MK_NT), (size_t)p->lds_floats * 4, (hipStream_t)stream, *p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_verify_q4_max_blocks_per_cu(const MkDecodeParams* p, int lds_bytes) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, pick_verify_q4(*p), MK_NT, lds_bytes) != hipSuccess) return 0;
  return nb;
}

extern "C" int mk_launch_verify(const MkDecodeParams* p, int n_wg, void* stream) {
  hipLaunchKernelGGL(pick_verify(*p), dim3(n_wg), dim3(MK_NT), (size_t)p->lds_floats * 4, (hipStream_t)stream, *p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_verify_max_blocks_per_cu(const MkDecodeParams* p, int lds_bytes) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, pick_verify(*p), MK_NT, lds_bytes) != hipSuccess) return 0;
  return nb;
}

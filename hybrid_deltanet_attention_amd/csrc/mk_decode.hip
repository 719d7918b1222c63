// Batch-1 decode step of the hybrid Gated-DeltaNet + attention decoder as ONE persistent kernel
// launch on gfx950 (luce-megakernel announcement, page 1: the whole forward in one dispatch, a
// grid-wide sync instead of kernel boundaries, BF16 weights with FP32 accumulation, the DeltaNet
// recurrence in FP32 registers, QKV + RoPE + causal softmax + output projection fused).
//
// Grid: one 512-lane workgroup per compute unit.  Every phase splits its rows over the grid; a
// phase's outputs are published as 8-byte exchange records (FP32 value in the low word, the
// launch epoch in the high word) written with device-coherent stores, and the next phase polls
// exactly the records it needs.  A record carries its own readiness, so there is no separate
// barrier, no L2 writeback/invalidate fence and no atomic counter on the critical path.  Each
// exchange buffer is written once per launch, so records never need clearing.
//
// Every wait is bounded: a wait that gives up sets ctl->err and every workgroup leaves the kernel.

#include <hip/hip_runtime.h>
#include "mk_internal.h"

typedef unsigned int u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));

namespace {

__device__ __forceinline__ int tid() { return (int)threadIdx.x; }
__device__ __forceinline__ int lane() { return (int)threadIdx.x & 63; }
__device__ __forceinline__ int wave() { return (int)threadIdx.x >> 6; }

// contiguous balanced split of n items over parts: part i gets [split(n,parts,i), split(n,parts,i+1))
__device__ __forceinline__ int split(int n, int parts, int i) {
  return (int)(((long long)n * i) / parts);
}

__device__ __forceinline__ void ll_put(mk_u64* p, u32 epoch, float v) {
  __hip_atomic_store(p, ((mk_u64)epoch << 32) | (mk_u64)__float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ mk_u64 ll_get(const mk_u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float bf_lo(u32 w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(u32 w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Fixed-order workgroup sum; every thread receives the same value.
__device__ __forceinline__ float block_sum(float v, float* scr) {
  v = wave_sum(v);
  if (lane() == 0) scr[wave()] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < MK_NWAVE; ++i) s += scr[i];
  __syncthreads();
  return s;
}

__device__ __forceinline__ void block_sum2(float& a, float& b, float* scr) {
  a = wave_sum(a);
  b = wave_sum(b);
  if (lane() == 0) {
    scr[wave()] = a;
    scr[MK_NWAVE + wave()] = b;
  }
  __syncthreads();
  float sa = 0.f, sb = 0.f;
#pragma unroll
  for (int i = 0; i < MK_NWAVE; ++i) {
    sa += scr[i];
    sb += scr[MK_NWAVE + i];
  }
  __syncthreads();
  a = sa;
  b = sb;
}

struct Ctx {
  MkCtl* ctl;
  u32 epoch;
};

// Poll n exchange records; record f lives at src(f) and its value goes to dst[f] (LDS).
// All threads of the workgroup call it; returns false (and sets ctl->err) if a wait gave up.
template <typename SrcFn>
__device__ __forceinline__ bool ll_gather(const Ctx& cx, int n, SrcFn src, float* dst) {
  constexpr int B = 4;
  bool ok = true;
  for (int base = 0; base < n && ok; base += MK_NT * B) {
    u32 pending = 0;
#pragma unroll
    for (int b = 0; b < B; ++b)
      if (base + b * MK_NT + tid() < n) pending |= 1u << b;
    u32 spins = 0;
    while (pending) {
      mk_u64 v[B];
#pragma unroll
      for (int b = 0; b < B; ++b)
        if ((pending >> b) & 1u) v[b] = ll_get(src(base + b * MK_NT + tid()));
#pragma unroll
      for (int b = 0; b < B; ++b)
        if (((pending >> b) & 1u) && (u32)(v[b] >> 32) == cx.epoch) {
          dst[base + b * MK_NT + tid()] = __uint_as_float((u32)v[b]);
          pending &= ~(1u << b);
        }
      if (pending) {
        ++spins;
        if ((spins & 255u) == 0 &&
            __hip_atomic_load(&cx.ctl->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
          ok = false;
          break;
        }
        if (spins > MK_SPIN_LIMIT) {
          __hip_atomic_store(&cx.ctl->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = false;
          break;
        }
      }
    }
  }
  return ok;
}

// Contiguous records src[0..n) -> dst[0..n).
__device__ __forceinline__ bool ll_gather_vec(const Ctx& cx, const mk_u64* src, int n, float* dst) {
  return ll_gather(cx, n, [=](int f) { return src + f; }, dst);
}

// Dot products of R rows of a row-major BF16 matrix (row stride K) with xin[0..K) (FP32, LDS).
// Work unit = (row, 512-column segment); units are dealt to the 8 waves round robin, each lane
// handles 8 consecutive columns with one 16-byte nontemporal load.  The per-row result is
// the segment sums added in segment order, so it does not depend on how rows are split over
// workgroups.  Rows are processed in blocks of RB; for each block, epi(row0, nrows) runs after
// the block's results are in out[0..nrows) (LDS), with the workgroup synchronised.
template <int RB, typename Epi>
__device__ __forceinline__ void gemv(const uint16_t* __restrict__ W, int R, int K, const float* xin,
                                     float* red, float* out, Epi epi) {
  constexpr int UB = 8;
  const int S = (K + 511) >> 9;
  const int w = wave(), l = lane();
  for (int rb = 0; rb < R; rb += RB) {
    const int nr = min(RB, R - rb);
    const int U = nr * S;
    const int nu = (U > w) ? (U - w + MK_NWAVE - 1) / MK_NWAVE : 0;
    const uint16_t* Wb = W + (size_t)rb * K;
    for (int i0 = 0; i0 < nu; i0 += UB) {
      u32x4 wv[UB];
#pragma unroll
      for (int b = 0; b < UB; ++b) {
        const int u = w + MK_NWAVE * (i0 + b);
        const int r = u / S, s = u - r * S;
        const int k = s * 512 + l * 8;
        if (i0 + b < nu && k < K)
          wv[b] = __builtin_nontemporal_load((const u32x4*)(Wb + (size_t)r * K + k));
        else
          wv[b] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int b = 0; b < UB; ++b) {
        const int u = w + MK_NWAVE * (i0 + b);
        const int r = u / S, s = u - r * S;
        const int k = s * 512 + l * 8;
        float acc = 0.f;
        if (k < K) {
          const float4 x0 = *(const float4*)(xin + k);
          const float4 x1 = *(const float4*)(xin + k + 4);
          acc = bf_lo(wv[b].x) * x0.x;
          acc = fmaf(bf_hi(wv[b].x), x0.y, acc);
          acc = fmaf(bf_lo(wv[b].y), x0.z, acc);
          acc = fmaf(bf_hi(wv[b].y), x0.w, acc);
          acc = fmaf(bf_lo(wv[b].z), x1.x, acc);
          acc = fmaf(bf_hi(wv[b].z), x1.y, acc);
          acc = fmaf(bf_lo(wv[b].w), x1.z, acc);
          acc = fmaf(bf_hi(wv[b].w), x1.w, acc);
        }
        acc = wave_sum(acc);
        if (i0 + b < nu && l == 0) red[u] = acc;
      }
    }
    __syncthreads();
    for (int r = tid(); r < nr; r += MK_NT) {
      float s = 0.f;
      for (int j = 0; j < S; ++j) s += red[r * S + j];
      out[r] = s;
    }
    __syncthreads();
    epi(rb, nr);
    __syncthreads();
  }
}

__device__ __forceinline__ void rmsnorm_lds(const float* x, const float* __restrict__ g, float* xn, int D,
                                            float eps, float* scr) {
  float s = 0.f;
  for (int i = tid(); i < D; i += MK_NT) s += x[i] * x[i];
  s = block_sum(s, scr);
  const float r = 1.0f / sqrtf(s / (float)D + eps);
  for (int i = tid(); i < D; i += MK_NT) xn[i] = x[i] * r * g[i];
  __syncthreads();
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ __forceinline__ float softplusf_(float z) { return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z))); }

struct Lds {
  float* x;    // residual [D]
  float* xn;   // normalised input [max K]
  float* vec;  // gathered vector / misc
  float* red;  // gemv unit partials
  float* out;  // gemv row results
  float* scr;  // reductions
};

// ------------------------------------------------------------------------------------------
// DeltaNet phases
// ------------------------------------------------------------------------------------------

// in-projection rows [q; k; v; a; b] of the normalised residual -> exchange records
__device__ __forceinline__ void dn_in_proj(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx,
                                           const Lds& s, int NW, int w) {
  const int R = 2 * p.H * p.dk + p.H * p.dv + 2 * p.H;
  const int r0 = split(R, NW, w), r1 = split(R, NW, w + 1);
  mk_u64* dst = L.ll_in;
  gemv<128>(L.w_in + (size_t)r0 * p.D, r1 - r0, p.D, s.xn, s.red, s.out, [&](int rb, int nr) {
    for (int r = tid(); r < nr; r += MK_NT) ll_put(dst + r0 + rb + r, cx.epoch, s.out[r]);
  });
}

// gated delta rule on this workgroup's rows of S, readout o = S q (after the update)
__device__ __forceinline__ bool dn_state(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx,
                                         const Lds& s, int NW, int w) {
  const int H = p.H, dk = p.dk, dv = p.dv;
  const int R = H * dv;
  const int r0 = split(R, NW, w), r1 = split(R, NW, w + 1);
  if (r0 >= r1) return true;
  const int h0 = r0 / dv, h1 = (r1 - 1) / dv;
  float* q = s.vec;
  float* k = s.vec + dk;
  float* ab = s.vec + 2 * dk;
  float* vr = s.vec + 2 * dk + 2;
  const mk_u64* in = L.ll_in;
  const int off_k = H * dk, off_v = 2 * H * dk, off_a = 2 * H * dk + H * dv, off_b = off_a + H;
  for (int h = h0; h <= h1; ++h) {
    const int i0 = max(r0, h * dv) - h * dv, i1 = min(r1, (h + 1) * dv) - h * dv;
    const int nv = i1 - i0;
    // one gather for q_h, k_h, a_h, b_h and this workgroup's v rows
    const int n = 2 * dk + 2 + nv;
    const bool ok = ll_gather(cx, n, [=](int f) {
      if (f < dk) return in + h * dk + f;
      if (f < 2 * dk) return in + off_k + h * dk + (f - dk);
      if (f == 2 * dk) return in + off_a + h;
      if (f == 2 * dk + 1) return in + off_b + h;
      return in + off_v + h * dv + i0 + (f - 2 * dk - 2);
    }, s.vec);
    if (__syncthreads_or(!ok)) return false;
    float qq = 0.f, kk = 0.f;
    for (int e = tid(); e < dk; e += MK_NT) {
      qq += q[e] * q[e];
      kk += k[e] * k[e];
    }
    block_sum2(qq, kk, s.scr);
    const float sq = 1.0f / sqrtf(qq + p.l2_eps);
    const float sk = 1.0f / sqrtf(kk + p.l2_eps);
    const float alpha = expf(-softplusf_(ab[0]));
    const float beta = sigmoidf_(ab[1]);
    float* Sh = L.S + (size_t)h * dv * dk;
    for (int i = i0 + wave(); i < i1; i += MK_NWAVE) {
      float* row = Sh + (size_t)i * dk;
      float sr[4];
      float kd = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e = lane() + 64 * t;
        sr[t] = (e < dk) ? row[e] : 0.f;
        if (e < dk) kd = fmaf(sr[t], k[e] * sk, kd);
      }
      kd = wave_sum(kd);
      const float u = beta * (vr[i - i0] - alpha * kd);
      float od = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e = lane() + 64 * t;
        if (e < dk) {
          sr[t] = fmaf(u, k[e] * sk, alpha * sr[t]);
          row[e] = sr[t];
          od = fmaf(sr[t], q[e] * sq, od);
        }
      }
      od = wave_sum(od);
      if (lane() == 0) ll_put(L.ll_mid + h * dv + i, cx.epoch, od);
    }
    __syncthreads();
  }
  return true;
}

// x_new[r] = x[r] + Wout[r] . vec  for this workgroup's rows -> exchange records
__device__ __forceinline__ void out_proj_residual(const MkDecodeParams& p, const uint16_t* Wout, int K,
                                                  mk_u64* dst, const Ctx& cx, const Lds& s, int NW, int w) {
  const int r0 = split(p.D, NW, w), r1 = split(p.D, NW, w + 1);
  gemv<128>(Wout + (size_t)r0 * K, r1 - r0, K, s.vec, s.red, s.out, [&](int rb, int nr) {
    for (int r = tid(); r < nr; r += MK_NT) ll_put(dst + r0 + rb + r, cx.epoch, s.x[r0 + rb + r] + s.out[r]);
  });
}

// ------------------------------------------------------------------------------------------
// attention phases
// ------------------------------------------------------------------------------------------

// q/k/v rows in RoPE pair order; rotate q and k at position pos; append k, v to the cache
__device__ __forceinline__ void att_qkv(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx,
                                        const Lds& s, int NW, int w, int pos) {
  const int hd = p.hd, half = hd / 2;
  const int NP = (p.nq + 2 * p.nkv) * half;
  const int p0 = split(NP, NW, w), p1 = split(NP, NW, w + 1);
  const float* cs = p.rope_cos + (size_t)pos * half;
  const float* sn = p.rope_sin + (size_t)pos * half;
  mk_u64* llq = L.ll_in;
  mk_u64* llk = L.ll_in + p.nq * hd;
  mk_u64* llv = llk + p.nkv * hd;
  gemv<128>(L.w_in + (size_t)2 * p0 * p.D, 2 * (p1 - p0), p.D, s.xn, s.red, s.out, [&](int rb, int nr) {
    for (int t = tid(); t < nr / 2; t += MK_NT) {
      const int P = p0 + rb / 2 + t;
      const float x1 = s.out[2 * t], x2 = s.out[2 * t + 1];
      int sec, hh, m;
      if (P < p.nq * half) {
        sec = 0; hh = P / half; m = P - hh * half;
      } else if (P < (p.nq + p.nkv) * half) {
        sec = 1; hh = (P - p.nq * half) / half; m = (P - p.nq * half) - hh * half;
      } else {
        sec = 2; hh = (P - (p.nq + p.nkv) * half) / half; m = (P - (p.nq + p.nkv) * half) - hh * half;
      }
      float y1 = x1, y2 = x2;
      if (sec < 2) {
        const float c = cs[m], sv = sn[m];
        y1 = x1 * c - x2 * sv;
        y2 = x2 * c + x1 * sv;
      }
      if (sec == 0) {
        ll_put(llq + hh * hd + m, cx.epoch, y1);
        ll_put(llq + hh * hd + m + half, cx.epoch, y2);
      } else if (sec == 1) {
        ll_put(llk + hh * hd + m, cx.epoch, y1);
        ll_put(llk + hh * hd + m + half, cx.epoch, y2);
        float* kc = L.Kc + ((size_t)hh * p.max_ctx + pos) * hd;
        kc[m] = y1;
        kc[m + half] = y2;
      } else {
        ll_put(llv + hh * hd + m, cx.epoch, y1);
        ll_put(llv + hh * hd + m + half, cx.epoch, y2);
        float* vc = L.Vc + ((size_t)hh * p.max_ctx + pos) * hd;
        vc[m] = y1;
        vc[m + half] = y2;
      }
    }
  });
}

// split-K partial softmax attention: work item = (kv head g, chunk of MK_ATT_CHUNK positions)
// emits (running max m, sum l, acc[hd]) for each query head of group g
__device__ __forceinline__ bool att_partial(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx,
                                            const Lds& s, int NW, int w, int pos) {
  const int hd = p.hd, nkv = p.nkv, gs = p.nq / p.nkv;
  const int Lpos = pos + 1;
  const int nch = (Lpos + MK_ATT_CHUNK - 1) / MK_ATT_CHUNK;
  const int items = nch * nkv;
  const float scale = 1.0f / sqrtf((float)hd);
  float* qv = s.vec;                 // [gs][hd]
  float* kp = s.vec + gs * hd;       // [hd] key at pos
  float* vp = kp + hd;               // [hd] value at pos
  float* sc = vp + hd;               // [gs][MK_ATT_CHUNK]
  float* ml = sc + gs * MK_ATT_CHUNK;  // [gs][2]
  const mk_u64* llq = L.ll_in;
  const mk_u64* llk = L.ll_in + p.nq * hd;
  const mk_u64* llv = llk + nkv * hd;
  for (int it = w; it < items; it += NW) {
    const int c = it / nkv, g = it - c * nkv;
    const int j0 = c * MK_ATT_CHUNK, j1 = min(Lpos, j0 + MK_ATT_CHUNK);
    const bool has_pos = (j1 == Lpos);
    const int n = gs * hd + (has_pos ? 2 * hd : 0);
    const bool ok = ll_gather(cx, n, [=](int f) {
      if (f < gs * hd) return llq + g * gs * hd + f;
      if (f < gs * hd + hd) return llk + g * hd + (f - gs * hd);
      return llv + g * hd + (f - gs * hd - hd);
    }, s.vec);
    if (__syncthreads_or(!ok)) return false;
    const float* Kg = L.Kc + (size_t)g * p.max_ctx * hd;
    const float* Vg = L.Vc + (size_t)g * p.max_ctx * hd;
    for (int jj = wave(); jj < j1 - j0; jj += MK_NWAVE) {
      const int j = j0 + jj;
      const float* kr = (j == pos) ? kp : Kg + (size_t)j * hd;
      float kreg[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e = lane() + 64 * t;
        kreg[t] = (e < hd) ? kr[e] : 0.f;
      }
      for (int i = 0; i < gs; ++i) {
        float d = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int e = lane() + 64 * t;
          if (e < hd) d = fmaf(kreg[t], qv[i * hd + e], d);
        }
        d = wave_sum(d);
        if (lane() == 0) sc[i * MK_ATT_CHUNK + jj] = d * scale;
      }
    }
    __syncthreads();
    if (tid() < gs) {
      const int i = tid();
      float m = -INFINITY;
      for (int jj = 0; jj < j1 - j0; ++jj) m = fmaxf(m, sc[i * MK_ATT_CHUNK + jj]);
      float l = 0.f;
      for (int jj = 0; jj < j1 - j0; ++jj) {
        const float e = expf(sc[i * MK_ATT_CHUNK + jj] - m);
        sc[i * MK_ATT_CHUNK + jj] = e;
        l += e;
      }
      ml[2 * i] = m;
      ml[2 * i + 1] = l;
    }
    __syncthreads();
    mk_u64* part = L.ll_mid + (size_t)it * gs * (hd + 2);
    for (int t = tid(); t < gs * hd; t += MK_NT) {
      const int i = t / hd, d = t - i * hd;
      float a = 0.f;
      for (int jj = 0; jj < j1 - j0; ++jj) {
        const int j = j0 + jj;
        const float vv = (j == pos) ? vp[d] : Vg[(size_t)j * hd + d];
        a = fmaf(sc[i * MK_ATT_CHUNK + jj], vv, a);
      }
      ll_put(part + i * (hd + 2) + 2 + d, cx.epoch, a);
    }
    if (tid() < 2 * gs) ll_put(part + (tid() >> 1) * (hd + 2) + (tid() & 1), cx.epoch, ml[tid()]);
    __syncthreads();
  }
  return true;
}

// combine the chunk partials of this workgroup's slice of o (log-sum-exp merge in chunk order)
__device__ __forceinline__ bool att_combine(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx,
                                            const Lds& s, int NW, int w, int pos) {
  const int hd = p.hd, nkv = p.nkv, gs = p.nq / p.nkv;
  const int Lpos = pos + 1;
  const int nch = (Lpos + MK_ATT_CHUNK - 1) / MK_ATT_CHUNK;
  const int N = p.nq * hd;
  const int o0 = split(N, NW, w), o1 = split(N, NW, w + 1);
  const int nown = o1 - o0;
  if (nown <= 0) return true;
  // staged in LDS in passes of at most `cap` (value, chunk) pairs
  const int cap = 2048;
  const mk_u64* part = L.ll_mid;
  // each pass handles `vpp` owned values fully
  const int vpp = max(1, cap / nch);
  for (int v0 = 0; v0 < nown; v0 += vpp) {
    const int vn = min(vpp, nown - v0);
    const int n = vn * nch * 3;
    const bool ok = ll_gather(cx, n, [=](int f) {
      const int which = f % 3;
      const int vc = f / 3;
      const int v = vc / nch, c = vc - v * nch;
      const int fo = o0 + v0 + v;
      const int i = fo / hd, d = fo - i * hd;
      const int g = i / gs, il = i - g * gs;
      const mk_u64* rec = part + ((size_t)(c * nkv + g) * gs + il) * (hd + 2);
      return rec + (which == 2 ? 2 + d : which);
    }, s.vec);
    if (__syncthreads_or(!ok)) return false;
    for (int v = tid(); v < vn; v += MK_NT) {
      const float* base = s.vec + (size_t)v * nch * 3;
      float M = -INFINITY;
      for (int c = 0; c < nch; ++c) M = fmaxf(M, base[3 * c]);
      float num = 0.f, den = 0.f;
      for (int c = 0; c < nch; ++c) {
        const float e = expf(base[3 * c] - M);
        den = fmaf(e, base[3 * c + 1], den);
        num = fmaf(e, base[3 * c + 2], num);
      }
      ll_put(L.ll_o + o0 + v0 + v, cx.epoch, num / den);
    }
    __syncthreads();
  }
  return true;
}

// ------------------------------------------------------------------------------------------
// FFN phases
// ------------------------------------------------------------------------------------------

// gate/up rows interleaved; h_j = silu(g_j) * u_j for this workgroup's j range
__device__ __forceinline__ void ffn_gate_up(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx,
                                            const Lds& s, int NW, int w) {
  const int j0 = split(p.ffn, NW, w), j1 = split(p.ffn, NW, w + 1);
  gemv<128>(L.w_gu + (size_t)2 * j0 * p.D, 2 * (j1 - j0), p.D, s.xn, s.red, s.out, [&](int rb, int nr) {
    for (int t = tid(); t < nr / 2; t += MK_NT) {
      const float g = s.out[2 * t], u = s.out[2 * t + 1];
      const float h = g / (1.0f + expf(-g)) * u;
      ll_put(L.ll_h + j0 + rb / 2 + t, cx.epoch, h);
    }
  });
}

}  // namespace

// ------------------------------------------------------------------------------------------
// the megakernel
// ------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_kernel(MkDecodeParams p) {
  extern __shared__ float lds[];
  const int NW = (int)gridDim.x, w = (int)blockIdx.x;
  Lds s;
  s.x = lds + p.lds_x;
  s.xn = lds + p.lds_xn;
  s.vec = lds + p.lds_vec;
  s.red = lds + p.lds_red;
  s.out = lds + p.lds_out;
  s.scr = lds + p.lds_scr;

  Ctx cx;
  cx.ctl = p.ctl;
  cx.epoch = p.ctl->step;
  const int pos = p.ctl->pos;
  const int tok = p.tok[0];
  // a bad token id or a full context is reported through ctl->err; every workgroup sees the
  // same values, so all of them leave before touching memory
  if (tok < 0 || tok >= p.vocab || pos < 0 || pos >= p.max_ctx) {
    if (w == 0 && tid() == 0) __hip_atomic_store(&p.ctl->err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  // embedding row (BF16 -> FP32), computed redundantly by every workgroup
  for (int i = tid(); i < p.D; i += MK_NT) {
    const u32 b = p.embed[(size_t)tok * p.D + i];
    s.x[i] = __uint_as_float(b << 16);
  }
  __syncthreads();

  for (int l = 0; l < p.n_layers; ++l) {
    const MkLayerDev& L = p.layers[l];
    rmsnorm_lds(s.x, L.g1, s.xn, p.D, p.rms_eps, s.scr);
    if (L.kind == MK_LAYER_DN) {
      dn_in_proj(p, L, cx, s, NW, w);
      if (!dn_state(p, L, cx, s, NW, w)) return;
      const int K = p.H * p.dv;
      if (__syncthreads_or(!ll_gather_vec(cx, L.ll_mid, K, s.vec))) return;
      out_proj_residual(p, L.w_out, K, L.ll_x1, cx, s, NW, w);
    } else {
      att_qkv(p, L, cx, s, NW, w, pos);
      if (!att_partial(p, L, cx, s, NW, w, pos)) return;
      if (!att_combine(p, L, cx, s, NW, w, pos)) return;
      const int K = p.nq * p.hd;
      if (__syncthreads_or(!ll_gather_vec(cx, L.ll_o, K, s.vec))) return;
      out_proj_residual(p, L.w_out, K, L.ll_x1, cx, s, NW, w);
    }
    if (__syncthreads_or(!ll_gather_vec(cx, L.ll_x1, p.D, s.x))) return;
    rmsnorm_lds(s.x, L.g2, s.xn, p.D, p.rms_eps, s.scr);
    ffn_gate_up(p, L, cx, s, NW, w);
    if (__syncthreads_or(!ll_gather_vec(cx, L.ll_h, p.ffn, s.vec))) return;
    out_proj_residual(p, L.w_down, p.ffn, L.ll_x2, cx, s, NW, w);
    if (__syncthreads_or(!ll_gather_vec(cx, L.ll_x2, p.D, s.x))) return;
  }

  // final norm + tied LM head + argmax (lowest index among equal maxima)
  rmsnorm_lds(s.x, p.g_final, s.xn, p.D, p.rms_eps, s.scr);
  const int v0 = split(p.vocab, NW, w), v1 = split(p.vocab, NW, w + 1);
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  gemv<256>(p.embed + (size_t)v0 * p.D, v1 - v0, p.D, s.xn, s.red, s.out, [&](int rb, int nr) {
    for (int r = tid(); r < nr; r += MK_NT) {
      const float v = s.out[r];
      const int idx = v0 + rb + r;
      if (p.logits) p.logits[idx] = v;
      if (v > best || (v == best && idx < bidx)) {
        best = v;
        bidx = idx;
      }
    }
  });
  // workgroup argmax: fixed tree over lanes then waves
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
  __syncthreads();
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
  if (w != 0) return;
  // workgroup 0 reduces the per-workgroup winners and publishes the token
  __syncthreads();
  const bool ok = ll_gather_vec(cx, p.ll_am, 2 * NW, s.vec);
  if (__syncthreads_or(!ok)) return;
  if (tid() == 0) {
    float b = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = 0; i < NW; ++i) {
      const float ob = s.vec[2 * i];
      const int oi = __float_as_int(s.vec[2 * i + 1]);
      if (ob > b || (ob == b && oi < bi)) {
        b = ob;
        bi = oi;
      }
    }
    p.next[0] = bi;
    p.ctl->pos = pos + 1;
    p.ctl->step = cx.epoch + 1u;
  }
}

// ------------------------------------------------------------------------------------------
// small helper kernels
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

__global__ void mk_bf16_to_f32_kernel(const uint16_t* __restrict__ src, float* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = __uint_as_float((u32)src[i] << 16);
}

__global__ void mk_zero_kernel(uint32_t* __restrict__ dst, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = 0u;
}

__global__ void mk_set_ctl_kernel(MkCtl* ctl, int32_t pos, int reset_err) {
  if (threadIdx.x == 0) {
    if (pos >= 0) ctl->pos = pos;
    if (ctl->step == 0u) ctl->step = 1u;
    if (reset_err) ctl->err = 0u;
  }
}

extern "C" int mk_decode_lds_bytes(const MkDecodeParams* p) { return p->lds_floats * 4; }

extern "C" int mk_launch_decode(const MkDecodeParams* p, int n_wg, void* stream) {
  hipLaunchKernelGGL(mk_decode_kernel, dim3(n_wg), dim3(MK_NT), (size_t)p->lds_floats * 4,
                     (hipStream_t)stream, *p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_launch_permute_rows(const uint16_t* src, uint16_t* dst, const int32_t* d_perm, int64_t rows,
                                      int64_t cols, void* stream) {
  if (rows <= 0) return 0;
  hipLaunchKernelGGL(mk_permute_rows_kernel, dim3((unsigned)rows), dim3(256), 0, (hipStream_t)stream, src, dst,
                     d_perm, rows, cols);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_launch_bf16_to_f32(const uint16_t* src, float* dst, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(mk_bf16_to_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     src, dst, n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_launch_zero(void* dst, int64_t bytes, void* stream) {
  if (bytes <= 0) return 0;
  const int64_t words = bytes / 4;
  hipLaunchKernelGGL(mk_zero_kernel, dim3(1024), dim3(256), 0, (hipStream_t)stream, (uint32_t*)dst, words);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_launch_set_ctl(MkCtl* ctl, int32_t pos, int reset_err, void* stream) {
  hipLaunchKernelGGL(mk_set_ctl_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, ctl, pos, reset_err);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_decode_max_blocks_per_cu(int lds_bytes) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, mk_decode_kernel, MK_NT, lds_bytes) != hipSuccess) return 0;
  return nb;
}

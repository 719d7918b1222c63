// 4-bit block-quantised weights (Q4G32) in the persistent decode kernel: the GEMV over them, the
// embedding row and RMSNorm with gains read from global memory.
//
// The pages' 27B-scale system decodes from 4-bit weights in blocks with a per-block scale
// (megakernel follow-up posts, page 3, quantisation-support paragraph).  Here a block is 32
// consecutive columns of a row with an FP16 scale d and offset m: w = d q + m.  A matrix W[R][K]
// is its codes (K/2 bytes per row; in the little-endian word at byte 4i of a row, column 8i + 2j
// is the nibble at bit 4j and column 8i + 2j + 1 the nibble at bit 16 + 4j) followed by its (d, m)
// pairs, one 32-bit word per (row, block), d in the low half.
#pragma once

#include "mk_device.h"

namespace {

constexpr int Q4_COLS = 2048;    // columns of a 4-bit GEMV unit (32 per lane)
constexpr int Q4_RED_CAP = 2048; // unit partials held in LDS per row chunk

// (d, m) words of a Q4G32 matrix with R rows and K columns whose codes start at W
__device__ __forceinline__ const MK_G u32* q4_params(const MK_G uint16_t* W, int R, int K) {
  return (const MK_G u32*)((const MK_G uint8_t*)W + (size_t)R * (size_t)(K >> 1));
}

// ---------------------------------------------------------------------------------- GEMV
// out[r] = W[r] . x over a workgroup's slice of rows.  A unit is 4 rows x 2048 columns: lane l
// holds columns 32 l .. 32 l + 31 of the unit's segment -- 16 bytes of codes and one (d, m) word
// per row -- and the hi/lo BF16 pairs of its 32 activations.  One AND/OR turns a code word into
// BF16 pairs (128 + q_even, 128 + q_odd) (BF16 0x4300 is 128 and its low 7 bits are the
// significand), so v_dot2c_f32_bf16 forms sum_j (128 + q_j) x_j exactly per product with FP32
// accumulation, and a block contributes  d * sum_j (128 + q_j) x_j + (m - 128 d) * sum_j x_j.
// Units are numbered segment-major (u = s * RB + rb) and split into contiguous, balanced ranges
// over all eight waves; a wave reloads its activations only when its range crosses a segment.
// Row partials are reduced over the wave in the same fixed order as the BF16 GEMV, and a row's
// value adds its segment partials in segment order.
struct GemvQ4 {
  const MK_G uint8_t* C;  // codes of the slice's first row
  const MK_G u32* P;      // (d, m) words of the slice's first row
  int R, K, S;            // rows, columns, 2048-column segments
  // rows [row0, row0 + R) of the matrix whose codes start at W and that has Rtot rows, K columns
  __device__ __forceinline__ void init(const MK_G uint16_t* W, int Rtot, int row0, int R_, int K_) {
    K = K_;
    R = R_;
    C = (const MK_G uint8_t*)W + (size_t)row0 * (size_t)(K_ >> 1);
    P = q4_params(W, Rtot, K_) + (size_t)row0 * (size_t)(K_ >> 5);
    S = (K_ + Q4_COLS - 1) / Q4_COLS;
  }
  __device__ __forceinline__ int chunk_rows() const { return max(4, (Q4_RED_CAP / S) & ~3); }
};

// this lane's part of one unit: codes of its 32 columns in each of the 4 rows, and their (d, m)
struct Q4Unit {
  u32x4 c[4];
  u32 p[4];
};

// Loads of unit (rb, s) for this lane.  Rows past R and columns past K read row 0 / column 0 of the
// slice (always inside the matrix); their results are never used (rows past R are not stored,
// columns past K meet zero activations).
__device__ __forceinline__ void q4_issue(const GemvQ4& g, int rb, int s, Q4Unit& u) {
  const int col = s * Q4_COLS + lane() * 32;
  const int cc = col < g.K ? col : 0;
  const size_t kb = (size_t)(g.K >> 1), kg = (size_t)(g.K >> 5);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = rb * 4 + k;
    const size_t rr = row < g.R ? (size_t)row : 0;
    u.c[k] = __builtin_nontemporal_load((const MK_G u32x4*)(g.C + rr * kb + (cc >> 1)));
    u.p[k] = __builtin_nontemporal_load(g.P + rr * kg + (cc >> 5));
  }
}

// this lane's 32 activations of segment s (hi/lo pairs, 8 words per 8 columns) and their sum
struct Q4X {
  u32x4 w[8];
  float sum;
};
__device__ __forceinline__ void q4_load_x(Q4X& x, const LS u32* hl, int s, int K) {
  const int col = s * Q4_COLS + lane() * 32;
#pragma unroll
  for (int i = 0; i < 8; ++i) x.w[i] = u32x4{0u, 0u, 0u, 0u};
  if (col < K) {
    const LS u32x4* p = (const LS u32x4*)(hl + (col >> 3) * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) x.w[i] = p[i];
  }
  // sum of hi + lo over the 32 columns, through the dot unit with weights (1, 1)
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a = dot2(x.w[i].x, 0x3F803F80u, a);
    a = dot2(x.w[i].y, 0x3F803F80u, a);
    a = dot2(x.w[i].z, 0x3F803F80u, a);
    a = dot2(x.w[i].w, 0x3F803F80u, a);
  }
  x.sum = a;
}

__device__ __forceinline__ float f16_lo(u32 w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(u32 w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// one row's 32 weights of this lane . its 32 activations
__device__ __forceinline__ float q4_row(u32x4 c, u32 pw, const Q4X& x) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32 v = c[i];
    const u32x4 xh = x.w[2 * i], xl = x.w[2 * i + 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32 b = ((v >> (4 * j)) & 0x000F000Fu) | 0x43004300u;
      acc = dot2(b, xh[j], acc);
      acc = dot2(b, xl[j], acc);
    }
  }
  const float d = f16_lo(pw), m = f16_hi(pw);
  return fmaf(d, acc, fmaf(-128.0f, d, m) * x.sum);
}

__device__ __forceinline__ void q4_put_partial(const GemvQ4& g, int rb, int s, float v, LS float* red) {
  if ((lane() & 15) == 0) {
    const int row = rb * 4 + (lane() >> 4);
    if (row < g.R) red[row * g.S + s] = v;
  }
}

// Unit partials of one row chunk -> red[row * S + segment], all eight waves streaming.
__device__ __forceinline__ void gemv_q4_partials(const GemvQ4& g0, const LS u32* xin, LS float* red) {
  GemvQ4 g = g0;
  g.C = uni_ptr(g0.C);
  g.P = uni_ptr(g0.P);
  g.R = uni(g0.R);
  g.K = uni(g0.K);
  g.S = uni(g0.S);
  const int RB = (g.R + 3) >> 2, U = RB * g.S;
  const int u0 = split(U, MK_NWAVE, wave()), u1 = split(U, MK_NWAVE, wave() + 1);
  if (u0 >= u1) return;
  Q4X x;
  int xs = -1;
  auto issue2 = [&](Q4Unit (&r)[2], int u) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ui = u + i;
      if (ui < u1) {
        const int s = ui / RB;
        q4_issue(g, ui - s * RB, s, r[i]);
      }
    }
  };
  auto unit = [&](const Q4Unit& r, int u) {
    const int s = u / RB, rb = u - s * RB;
    if (s != xs) {
      q4_load_x(x, xin, s, g.K);
      xs = s;
    }
    const float a0 = q4_row(r.c[0], r.p[0], x);
    const float a1 = q4_row(r.c[1], r.p[1], x);
    const float a2 = q4_row(r.c[2], r.p[2], x);
    const float a3 = q4_row(r.c[3], r.p[3], x);
    q4_put_partial(g, rb, s, reduce_rows4(a0, a1, a2, a3), red);
  };
  Q4Unit cur[2], nxt[2];
  issue2(cur, u0);
  // nothing may look outstanding in cur when the loop starts (conditional loads; see the BF16 GEMV)
  wait_vm<0>();
  for (int u = u0; u < u1; u += 2) {
    issue2(nxt, u + 2);
    keep_issued();
    unit(cur[0], u);
    if (u + 1 < u1) unit(cur[1], u + 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) cur[i] = nxt[i];
  }
  // the look-ahead loads past the range were never issued; wait for any still counted
  wait_vm<0>();
}

// W . x over the slice, then epi(row, value, 0) (or, PAIRS, epi(pair, row 2 pair, row 2 pair + 1))
// by the streaming threads (their stores stay off the polling waves' queues).
template <bool PAIRS, bool EPI_ALL, typename Epi>
__device__ __forceinline__ void gemv_q4(const GemvQ4& G, const LS u32* xin, LS float* red, Tracer& tr, Epi epi) {
  const int rc = G.chunk_rows();
  for (int r0 = 0; r0 < G.R; r0 += rc) {
    GemvQ4 g = G;
    g.C = G.C + (size_t)r0 * (size_t)(G.K >> 1);
    g.P = G.P + (size_t)r0 * (size_t)(G.K >> 5);
    g.R = min(rc, G.R - r0);
    gemv_q4_partials(g, xin, red);
    tr.mark();
    wg_bar();
    tr.mark();
    const int stride = EPI_ALL ? MK_NT : NCT;
    if (EPI_ALL || streamer()) {
      if (PAIRS) {
        for (int t = tid(); t < g.R / 2; t += stride)
          epi(r0 / 2 + t, seg_sum(red + (2 * t) * g.S, g.S), seg_sum(red + (2 * t + 1) * g.S, g.S));
      } else {
        for (int t = tid(); t < g.R; t += stride) epi(r0 + t, seg_sum(red + t * g.S, g.S), 0.f);
      }
    }
    if (r0 + rc < G.R) wg_bar();  // red is reused by the next chunk
  }
}

// Row `tok` of a Q4G32 matrix [vocab][D] -> x[0..D) in FP32 (d q + m: exact in FP32 for these
// widths), one code word (8 columns) per thread.
__device__ __forceinline__ void q4_embed_row(const MK_G uint16_t* E, int vocab, int D, int tok, LS float* x) {
  const MK_G u32* codes = (const MK_G u32*)((const MK_G uint8_t*)E + (size_t)tok * (size_t)(D >> 1));
  const MK_G u32* par = q4_params(E, vocab, D) + (size_t)tok * (size_t)(D >> 5);
  for (int i = tid(); i < (D >> 3); i += MK_NT) {
    const u32 v = codes[i];
    const u32 pw = par[i >> 2];
    const float d = f16_lo(pw), m = f16_hi(pw);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = fmaf(d, (float)((v >> (4 * j)) & 15u), m);
      x[8 * i + 2 * j + 1] = fmaf(d, (float)((v >> (16 + 4 * j)) & 15u), m);
    }
  }
}

// RMSNorm as in rmsnorm(), the BF16 gains read from global memory (issued before the sum of
// squares so their latency overlaps it).  D <= 4 * MK_NT * Q4_GAIN_IT.
constexpr int Q4_GAIN_IT = 4;
__device__ __forceinline__ void rmsnorm_gg(const LS float* x, const MK_G uint16_t* g, LS u32* xn, int D, float eps,
                                           Tracer& tr) {
  D = uni(D);
  const int D4 = D >> 2;
  u32x2 gg[Q4_GAIN_IT];
#pragma unroll
  for (int k = 0; k < Q4_GAIN_IT; ++k) {
    const int c = tid() + k * MK_NT;
    gg[k] = c < D4 ? *(const MK_G u32x2*)(g + 4 * c) : u32x2{0u, 0u};
  }
  const LS f32x4* x4 = (const LS f32x4*)x;
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
  const float r = 1.0f / sqrtf(s / (float)D + eps);
  tr.mark();
#pragma unroll
  for (int k = 0; k < Q4_GAIN_IT; ++k) {
    const int c = tid() + k * MK_NT;
    if (c < D4) {
      const f32x4 v = x4[c];
      u32 h[4], l[4];
      split_hl(v.x * r * __uint_as_float(gg[k].x << 16), h[0], l[0]);
      split_hl(v.y * r * __uint_as_float(gg[k].x & 0xffff0000u), h[1], l[1]);
      split_hl(v.z * r * __uint_as_float(gg[k].y << 16), h[2], l[2]);
      split_hl(v.w * r * __uint_as_float(gg[k].y & 0xffff0000u), h[3], l[3]);
      const int o = hl_word(4 * c);
      *(LS u32x2*)(xn + o) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      *(LS u32x2*)(xn + o + 4) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
    }
  }
  tr.mark();
  wg_bar();
}

}  // namespace

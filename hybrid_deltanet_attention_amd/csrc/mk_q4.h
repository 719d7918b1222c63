// 4-bit block-quantised weights (Q4G32) in the persistent decode kernel: the GEMV over them, the
// embedding row, RMSNorm with gains read from global memory and the activation packing.
//
// The pages' 27B-scale system decodes from 4-bit weights in blocks with a per-block scale
// (megakernel follow-up posts, page 3, quantisation-support paragraph).  Here a block is 32
// consecutive columns of a row with an FP16 scale d and offset m: w = d q + m.  A matrix W[R][K]
// is its codes (K/2 bytes per row; in the little-endian word at byte 4i of a row, column 8i + 2j
// is the nibble at bit 4j and column 8i + 2j + 1 the nibble at bit 16 + 4j) followed by its (d, m)
// pairs, one 32-bit word per (row, block), d in the low half.
//
// In the workspace every 4-bit matrix is tiled (mk_launch_q4_tile): rows are taken four at a time
// (the last block padded with zero rows); row block b takes G * 80 bytes at b G 80 (G = K / 32
// column blocks), in segments of 64 column blocks (the last may be shorter, n blocks).  Segment s
// of row block b starts at byte s * 64 * 80 of the row block and holds five planes of n * 16
// bytes: plane k < 4 is row 4b + k's 16 code bytes of each column block in order, plane 4 the four
// rows' (d, m) words of each column block.  A GEMV unit is one segment of one row block: five
// 16-byte loads per lane, each wave-wide load one contiguous plane, the unit one 5 KB span.
#pragma once

#include "mk_device.h"

namespace {

constexpr int Q4_COLS = 2048;    // columns of a 4-bit GEMV unit (32 per lane)
constexpr int Q4_RED_CAP = 2048; // unit partials held in LDS per row chunk

constexpr int Q4_TILE = 80;  // bytes per (4-row block, 32-column block) tile

// ---------------------------------------------------------------------------------- GEMV
// out[r] = W[r] . x over a workgroup's slice of rows.  A unit is 4 rows x 2048 columns: lane l
// holds columns 32 l .. 32 l + 31 of the unit's segment (one 32-column block): 16 bytes of codes
// and one (d, m) word per row.  The activations come as 16-bit integers per block,
// T_j = rint(x_j / s_g) with s_g = max_j |x_j| / 30000, split into four signed 4-bit digits laid
// out like the codes (q4_pack), so v_dot8_i32_i4 forms sum_j (q_j - 8) D_kj for eight columns at a
// time in exact integer arithmetic, and a block contributes
//   d s_g sum_j (q_j - 8) T_j + (m + 8 d) sum_j x_j.
// Units are numbered row-block-major (u = rb * S + s), so that the workgroup streams its slice of
// rows front to back; the eight waves take them in that order from a workgroup counter in LDS, so
// they finish together whatever each wave's memory latency, and
// each wave keeps Q4_RING units' loads in flight (buffer loads: a unit past the last or a column
// past K reads zeros without touching memory, so every iteration issues the same loads).  A unit's
// partial does not depend on which wave computes it.  Row partials are reduced over the wave in
// the fixed order of the BF16 GEMV, and a row's value adds its segment partials in segment order.
constexpr int Q4_XW = 20;   // LDS words per 32-column block of packed activations
constexpr int Q4_RING = 4;  // units in flight per wave
constexpr float Q4_TMAX = 30000.0f;

struct GemvQ4 {
  const MK_G uint8_t* T;  // tiles of the slice's first row block
  int R, K, S;            // rows, columns, 2048-column segments
  // rows [4 b0, 4 b0 + R) of the tiled matrix at W with K columns
  __device__ __forceinline__ void init(const MK_G uint16_t* W, int b0, int R_, int K_) {
    K = K_;
    R = R_;
    T = (const MK_G uint8_t*)W + (size_t)b0 * (size_t)(K_ >> 5) * Q4_TILE;
    S = (K_ + Q4_COLS - 1) / Q4_COLS;
  }
  __device__ __forceinline__ int chunk_rows() const { return max(4, (Q4_RED_CAP / S) & ~3); }
};

// this lane's part of one unit: codes of its 32 columns in each of the 4 rows, and their (d, m)
struct Q4Unit {
  u32x4 c[4];
  u32x4 p;
};

// this lane's block of packed activations: digit words [8-column word i][digit k], s_g, sum x
struct Q4X {
  u32x4 w[4];
  float s, sum;
};
__device__ __forceinline__ void q4_load_x(Q4X& x, const LS u32* xp, int s, int K) {
  const int col = s * Q4_COLS + lane() * 32;
#pragma unroll
  for (int i = 0; i < 4; ++i) x.w[i] = u32x4{0u, 0u, 0u, 0u};
  x.s = 0.f;
  x.sum = 0.f;
  if (col < K) {
    const LS u32* b = xp + (col >> 5) * Q4_XW;
#pragma unroll
    for (int i = 0; i < 4; ++i) x.w[i] = ((const LS u32x4*)b)[i];
    const u32x2 g = *(const LS u32x2*)(b + 16);
    x.s = __uint_as_float(g.x);
    x.sum = __uint_as_float(g.y);
  }
}

__device__ __forceinline__ float f16_lo(u32 w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(u32 w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// one row's 32 weights of this lane . its 32 activations
__device__ __forceinline__ float q4_row(u32x4 c, u32 pw, const Q4X& x) {
  int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = (int)(c[i] ^ 0x88888888u);  // codes q - 8 as signed nibbles
    a0 = __builtin_amdgcn_sdot8(v, (int)x.w[i].x, a0, false);
    a1 = __builtin_amdgcn_sdot8(v, (int)x.w[i].y, a1, false);
    a2 = __builtin_amdgcn_sdot8(v, (int)x.w[i].z, a2, false);
    a3 = __builtin_amdgcn_sdot8(v, (int)x.w[i].w, a3, false);
  }
  const int S = a0 + (a1 << 4) + (a2 << 8) + (a3 << 12);  // sum (q - 8) T, |S| < 2^23
  const float d = f16_lo(pw), m = f16_hi(pw);
  return fmaf(d * x.s, (float)S, fmaf(8.0f, d, m) * x.sum);
}

__device__ __forceinline__ void q4_put_partial(const GemvQ4& g, int rb, int s, float v, LS float* red) {
  if ((lane() & 15) == 0) {
    const int row = rb * 4 + (lane() >> 4);
    if (row < g.R) red[row * g.S + s] = v;
  }
}

// A wave's units in flight: their loads and unit numbers.
struct Q4Ring {
  Q4Unit r[Q4_RING];
  int uk[Q4_RING];
};

// Unit sources of one row chunk (uniform values).
struct Q4Src {
  __amdgpu_buffer_rsrc_t rt;
  int RB, U, G, S, K, R;
  __device__ __forceinline__ void init(const GemvQ4& g0) {
    const MK_G uint8_t* T = uni_ptr(g0.T);
    R = uni(g0.R);
    K = uni(g0.K);
    S = uni(g0.S);
    RB = (R + 3) >> 2;
    U = RB * S;
    G = K >> 5;
    rt = __builtin_amdgcn_make_buffer_rsrc((void*)T, 0, RB * G * Q4_TILE, 0x00020000);
  }
  __device__ __forceinline__ int grab(LS int* ctr) const {
    int v = 0;
    if (lane() == 0) v = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return __builtin_amdgcn_readfirstlane(v);
  }
  // loads of unit u (zeros for u >= U or column blocks past K)
  __device__ __forceinline__ void issue(Q4Unit& r, int u) const {
    constexpr int OOB = 0x7ffffff0;  // past the resource: the load returns zeros
    const int rb = u / S, s = u - rb * S;
    const int ng = min(64, G - 64 * s);  // column blocks in this segment
    const bool live = u < U && lane() < ng;
    const int o = rb * G * Q4_TILE + s * 64 * Q4_TILE + lane() * 16;
    const int pl = ng * 16;  // plane bytes
#pragma unroll
    for (int k = 0; k < 4; ++k)
      r.c[k] = __builtin_amdgcn_raw_buffer_load_b128(rt, live ? o + k * pl : OOB, 0, 2 /* nt */);
    r.p = __builtin_amdgcn_raw_buffer_load_b128(rt, live ? o + 4 * pl : OOB, 0, 2 /* nt */);
  }
};

// The first Q4_RING units of g's first row chunk for this wave: taken from the counter and their
// loads issued.  Weights do not depend on activations, so a wave primes the next GEMV before it
// waits for that GEMV's inputs.
__device__ __forceinline__ void gemv_q4_prime(const GemvQ4& g, LS int* ctr, Q4Ring& q) {
  GemvQ4 c0 = g;
  c0.R = min(g.R, g.chunk_rows());
  Q4Src src;
  src.init(c0);
#pragma unroll
  for (int k = 0; k < Q4_RING; ++k) {
    q.uk[k] = src.grab(ctr);
    src.issue(q.r[k], q.uk[k]);
  }
}

// Unit partials of one row chunk -> red[row * S + segment], all eight waves streaming; ctr is the
// LDS unit counter (zero before the first grab; gemv_q4 clears it again after the partials).
// primed: this wave's ring already holds its first units (gemv_q4_prime).
__device__ __forceinline__ void gemv_q4_partials(const GemvQ4& g0, const LS u32* xin, LS float* red, LS int* ctr,
                                                 Q4Ring& q, bool primed) {
  Q4Src src;
  src.init(g0);
  GemvQ4 g = g0;
  g.R = src.R;
  g.K = src.K;
  g.S = src.S;
  const int U = src.U;
  Q4X x;
  int xs = -1;
  auto unit = [&](const Q4Unit& r, int u) {
    const int rb = u / g.S, s = u - rb * g.S;
    if (s != xs) {
      q4_load_x(x, xin, s, g.K);
      xs = s;
    }
    const float a0 = q4_row(r.c[0], r.p.x, x);
    const float a1 = q4_row(r.c[1], r.p.y, x);
    const float a2 = q4_row(r.c[2], r.p.z, x);
    const float a3 = q4_row(r.c[3], r.p.w, x);
    q4_put_partial(g, rb, s, reduce_rows4(a0, a1, a2, a3), red);
  };
  if (!primed) {
#pragma unroll
    for (int k = 0; k < Q4_RING; ++k) {
      q.uk[k] = src.grab(ctr);
      src.issue(q.r[k], q.uk[k]);
    }
  }
  // each wave's grabs increase, so once its oldest unit is past U every later one is too
  while (q.uk[0] < U) {
#pragma unroll
    for (int k = 0; k < Q4_RING; ++k) {
      const bool live = q.uk[k] < U;
      if (live) unit(q.r[k], q.uk[k]);
      q.uk[k] = live ? src.grab(ctr) : U;
      src.issue(q.r[k], q.uk[k]);
    }
  }
  // the last loads of the ring read zeros; wait for them before the registers are reused
  wait_vm<0>();
}

// W . x over the slice, then epi(row, value, 0) (or, PAIRS, epi(pair, row 2 pair, row 2 pair + 1))
// by the streaming threads (their stores stay off the polling waves' queues).
// q / primed: as for gemv_q4_partials (the prime covers the first row chunk).
template <bool PAIRS, bool EPI_ALL, typename Epi>
__device__ __forceinline__ void gemv_q4(const GemvQ4& G, const LS u32* xin, LS float* red, LS int* ctr, Q4Ring& q,
                                        bool primed, Tracer& tr, Epi epi) {
  const int rc = G.chunk_rows();
  // at least one pass, also for an empty slice: the counter must be cleared behind the prime's
  // grabs and the primed loads waited for
  for (int r0 = 0; r0 == 0 || r0 < G.R; r0 += rc) {
    GemvQ4 g = G;
    g.T = G.T + (size_t)(r0 >> 2) * (size_t)(G.K >> 5) * Q4_TILE;  // rc is a multiple of 4
    g.R = max(0, min(rc, G.R - r0));
    gemv_q4_partials(g, xin, red, ctr, q, primed && r0 == 0);
    tr.mark();
    wg_bar();
    if (tid() == 0) *ctr = 0;  // the next use comes after at least one more barrier
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

// Row `tok` of the tiled 4-bit embedding [vocab][D] -> x[0..D) in FP32 (d q + m: exact in FP32
// for these widths), one code word (8 columns) per thread.
__device__ __forceinline__ void q4_embed_row(const MK_G uint16_t* E, int D, int tok, LS float* x) {
  const int G = D >> 5;
  const MK_G uint8_t* rowb = (const MK_G uint8_t*)E + (size_t)(tok >> 2) * (size_t)G * Q4_TILE;
  const int r = tok & 3;
  for (int i = tid(); i < (D >> 3); i += MK_NT) {
    const int gi = i >> 2, s = gi >> 6, l = gi & 63, ng = min(64, G - 64 * s);
    const MK_G uint8_t* seg = rowb + (size_t)s * 64 * Q4_TILE;
    const u32 v = *(const MK_G u32*)(seg + r * ng * 16 + l * 16 + 4 * (i & 3));
    const u32 pw = *(const MK_G u32*)(seg + 4 * ng * 16 + l * 16 + 4 * r);
    const float d = f16_lo(pw), m = f16_hi(pw);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = fmaf(d, (float)((v >> (4 * j)) & 15u), m);
      x[8 * i + 2 * j + 1] = fmaf(d, (float)((v >> (16 + 4 * j)) & 15u), m);
    }
  }
}

// x -> xf = x / sqrt(mean x^2 + eps) * g in FP32 (packed for the GEMV by q4_pack).  Every wave
// sums the squares itself (same order in every wave); the polling threads read the BF16 gains
// from global memory (issued before the sum) and write xf, so the streaming waves, whose queues
// may hold the next GEMV's primed loads, issue no load here.  D <= 4 * NPT * Q4_GAIN_IT.
constexpr int Q4_GAIN_IT = 8;
// gains held by the polling threads, IT pieces of 4 each (D <= 4 * NPT * IT)
template <int IT = Q4_GAIN_IT>
struct Q4Gains {
  u32x2 gg[IT];
};
// the polling threads' loads of the gains g[0..D) (a caller may issue them early, before a gather)
template <int IT>
__device__ __forceinline__ void gains_gg_issue(const MK_G uint16_t* g, int D, Q4Gains<IT>& gn) {
  const int D4 = uni(D) >> 2;
  const int pl = tid() - NCT;
  if (!streamer()) {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int c = pl + k * NPT;
      gn.gg[k] = c < D4 ? *(const MK_G u32x2*)(g + 4 * c) : u32x2{0u, 0u};
    }
  }
}
template <int IT>
__device__ __forceinline__ void rmsnorm_gg(const LS float* x, const Q4Gains<IT>& gn, LS float* xf, int D, float eps,
                                           Tracer& tr) {
  D = uni(D);
  const int D4 = D >> 2;
  const int pl = tid() - NCT;
  const u32x2(&gg)[IT] = gn.gg;
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
  if (!streamer()) {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int c = pl + k * NPT;
      if (c < D4) {
        const f32x4 v = x4[c];
        ((LS f32x4*)xf)[c] =
            f32x4{v.x * r * __uint_as_float(gg[k].x << 16), v.y * r * __uint_as_float(gg[k].x & 0xffff0000u),
                  v.z * r * __uint_as_float(gg[k].y << 16), v.w * r * __uint_as_float(gg[k].y & 0xffff0000u)};
      }
    }
  }
  tr.mark();
  wg_bar();
}
__device__ __forceinline__ void rmsnorm_gg(const LS float* x, const MK_G uint16_t* g, LS float* xf, int D, float eps,
                                           Tracer& tr) {
  Q4Gains<> gn;
  gains_gg_issue(g, D, gn);
  rmsnorm_gg(x, gn, xf, D, eps, tr);
}

// FP32 v[0..n) (n a multiple of 32) -> in place, the GEMV's packed activations: block g of 32
// columns takes words [20 g, 20 g + 20): 16 digit words (8-column word i, digit k at 4 i + k; in a
// digit word, column 2t's digit is the nibble at bit 4t and column 2t + 1's the nibble at bit
// 16 + 4t, as in the code words), then s_g and sum_j x_j.  T_j = rint(x_j / s_g), |T_j| <= 30000,
// is written as sum_k D_k 16^k with digits D_k in [-8, 7]: the nibbles of T + 0x8888, each XOR 8.
// A quad of lanes handles a block (8 columns per lane); all blocks are read before any is written
// (the packed form is smaller, so block g's words overlap only blocks <= g).  Between barriers,
// by all threads; n <= 8 * MK_NT * Q4_PACK_IT.
constexpr int Q4_PACK_IT = 5;
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
}
__device__ __forceinline__ float quad_sum(float v) {
  v = v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ void q4_pack(LS float* v, int n) {
  n = uni(n);
  const int n8 = n >> 3;
  u32x4 dg[Q4_PACK_IT];
  u32x2 gp[Q4_PACK_IT];
#pragma unroll
  for (int it = 0; it < Q4_PACK_IT; ++it) {
    const int i = it * MK_NT + tid();
    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f}, b = a;
    if (i < n8) {
      a = ((const LS f32x4*)v)[2 * i];
      b = ((const LS f32x4*)v)[2 * i + 1];
    }
    const float mx = quad_max(fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                                    fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w)))));
    const float sm = quad_sum(((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w)));
    const float inv = mx > 0.f ? Q4_TMAX / mx : 0.f;
    // rint(x * inv) + 0x8888 from the bits of x * inv + 1.5 * 2^23 (round to nearest even)
    auto u16 = [&](float e) { return __float_as_uint(fmaf(e, inv, 12582912.0f)) + (0x8888u - 0x4B400000u); };
    u32 P0 = u16(a.x) | (u16(a.y) << 16), P1 = u16(a.z) | (u16(a.w) << 16);
    u32 P2 = u16(b.x) | (u16(b.y) << 16), P3 = u16(b.z) | (u16(b.w) << 16);
    // 4 x 4 nibble transpose in both 16-bit halves: row t (P_t) holds the digits of columns 2t and
    // 2t + 1; afterwards row k holds digit k of every column
    u32 t;
    t = ((P0 >> 8) ^ P2) & 0x00FF00FFu; P2 ^= t; P0 ^= t << 8;
    t = ((P1 >> 8) ^ P3) & 0x00FF00FFu; P3 ^= t; P1 ^= t << 8;
    t = ((P0 >> 4) ^ P1) & 0x0F0F0F0Fu; P1 ^= t; P0 ^= t << 4;
    t = ((P2 >> 4) ^ P3) & 0x0F0F0F0Fu; P3 ^= t; P2 ^= t << 4;
    dg[it] = u32x4{P0 ^ 0x88888888u, P1 ^ 0x88888888u, P2 ^ 0x88888888u, P3 ^ 0x88888888u};
    gp[it] = u32x2{__float_as_uint(mx * (1.0f / Q4_TMAX)), __float_as_uint(sm)};
  }
  wg_bar();
#pragma unroll
  for (int it = 0; it < Q4_PACK_IT; ++it) {
    const int i = it * MK_NT + tid();
    if (i < n8) {
      LS u32* b = (LS u32*)v + (i >> 2) * Q4_XW;
      ((LS u32x4*)b)[i & 3] = dg[it];
      if ((i & 3) == 0) *(LS u32x2*)(b + 16) = gp[it];
    }
  }
  wg_bar();
}

}  // namespace

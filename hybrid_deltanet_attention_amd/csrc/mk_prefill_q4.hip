// Prefill with 4-bit (Q4G32) weights on the BF16 matrix-core GEMMs of mk_prefill.hip.
//
// The pages' 27B-scale system runs from 4-bit block-quantised weights and builds its long contexts
// by prefill (megakernel follow-up posts, page 3, "Speed" and quantisation-support paragraphs).  A
// weight w = d q + m (FP16 d and m, 4-bit q) is an FP32 value of up to about 16 significant bits:
// not a BF16 value, but exactly (to 2^-17 relative) the sum of a BF16 high part and a BF16 low
// part.  Each matrix is expanded just before its GEMM into rows [W_hi | W_lo] of 2K BF16 values,
// and the activations of the K-column product into [A_hi | A_hi] and [A_lo | 0], so that the
// unchanged hi/lo GEMM over 2K columns forms
//     A_hi W_hi + A_lo W_hi + A_hi W_lo
// (the dropped A_lo W_lo is below FP32 rounding of the sum).  The expansion of one matrix (at most
// 2 FFN x hidden rows) reuses one scratch region, layer after layer.
//
// The tiled 4-bit layout (mk_q4.h): row block b (rows 4b .. 4b + 3) of a matrix with K columns
// starts at byte b * G * 80 (G = K / 32 column blocks) and is cut into segments of 64 column blocks
// (the last one n <= 64 blocks); a segment holds five planes of n * 16 bytes: plane r < 4 the
// 16 code bytes of row 4b + r per column block, plane 4 the four rows' (d, m) words (d in the low
// half).  In a row's code word i of a block, column 8i + 2j is the nibble at bit 4j and column
// 8i + 2j + 1 the nibble at bit 16 + 4j.

#include <hip/hip_runtime.h>

#include "mk_q4.h"

namespace {

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const u32 u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// one thread per (row n < N, 32-column block g): Wd[n][c] = BF16 high part of w(n, c),
// Wd[n][K + c] = BF16 low part of w - high, for the block's 32 columns.  w = fmaf(d, q, m), the
// decode kernel's value of the same weight (d q is exact in FP32).
__global__ void pf_q4_expand_kernel(const uint8_t* __restrict__ T, int N, int K, uint16_t* __restrict__ Wd) {
  const int G = K >> 5;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)N * G) return;
  const int n = (int)(idx / G), g = (int)(idx - (size_t)n * G);
  const int rb = n >> 2, r = n & 3, s = g >> 6, l = g & 63, ng = min(64, G - 64 * s);
  const uint8_t* seg = T + (size_t)rb * G * Q4_TILE + (size_t)s * 64 * Q4_TILE;
  const u32x4 c = *(const u32x4*)(seg + (size_t)r * ng * 16 + l * 16);
  const u32 pw = *(const u32*)(seg + (size_t)4 * ng * 16 + l * 16 + 4 * r);
  const float d = f16_lo(pw), m = f16_hi(pw);
  uint16_t* hi = Wd + (size_t)n * 2 * K + 32 * g;
  uint16_t* lo = hi + K;
  const u32 cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint16_t h[8], o[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float w0 = fmaf(d, (float)((cw[i] >> (4 * j)) & 15u), m);
      const float w1 = fmaf(d, (float)((cw[i] >> (16 + 4 * j)) & 15u), m);
      h[2 * j] = bf16_rne(w0);
      h[2 * j + 1] = bf16_rne(w1);
      o[2 * j] = bf16_rne(w0 - __uint_as_float((u32)h[2 * j] << 16));
      o[2 * j + 1] = bf16_rne(w1 - __uint_as_float((u32)h[2 * j + 1] << 16));
    }
    u32x4 hv, ov;
    hv.x = h[0] | ((u32)h[1] << 16);
    hv.y = h[2] | ((u32)h[3] << 16);
    hv.z = h[4] | ((u32)h[5] << 16);
    hv.w = h[6] | ((u32)h[7] << 16);
    ov.x = o[0] | ((u32)o[1] << 16);
    ov.y = o[2] | ((u32)o[3] << 16);
    ov.z = o[4] | ((u32)o[5] << 16);
    ov.w = o[6] | ((u32)o[7] << 16);
    *(u32x4*)(hi + 8 * i) = hv;
    *(u32x4*)(lo + 8 * i) = ov;
  }
}

// X[t] = the 4-bit embedding row of token tok[t] in FP32 (the decode kernel's values); ids outside
// [0, vocab) set ctl->err = 2 and give a zero row.  One 256-thread workgroup per token.
__global__ void __launch_bounds__(256) pf_embed_q4_kernel(const int32_t* __restrict__ tok, int T,
                                                          const uint8_t* __restrict__ E, int D, int vocab,
                                                          float* __restrict__ X, MkCtl* ctl) {
  const int t = blockIdx.x;
  if (t >= T) return;
  const int id = tok[t];
  float* x = X + (size_t)t * D;
  if (id < 0 || id >= vocab) {
    if (threadIdx.x == 0) __hip_atomic_store(&ctl->err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = threadIdx.x; i < D; i += blockDim.x) x[i] = 0.f;
    return;
  }
  const int G = D >> 5, r = id & 3;
  const uint8_t* rowb = E + (size_t)(id >> 2) * G * Q4_TILE;
  for (int i = threadIdx.x; i < (D >> 3); i += blockDim.x) {
    const int g = i >> 2, s = g >> 6, l = g & 63, ng = min(64, G - 64 * s);
    const uint8_t* seg = rowb + (size_t)s * 64 * Q4_TILE;
    const u32 v = *(const u32*)(seg + (size_t)r * ng * 16 + l * 16 + 4 * (i & 3));
    const u32 pw = *(const u32*)(seg + (size_t)4 * ng * 16 + l * 16 + 4 * r);
    const float d = f16_lo(pw), m = f16_hi(pw);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = fmaf(d, (float)((v >> (4 * j)) & 15u), m);
      x[8 * i + 2 * j + 1] = fmaf(d, (float)((v >> (16 + 4 * j)) & 15u), m);
    }
  }
}

// rows t < T of the split activations (leading dimension ld): Ahi[t][K + j] = Ahi[t][j] and
// Alo[t][K + j] = 0 for j < K, so that [A_hi | A_hi] + [A_lo | 0] meets [W_hi | W_lo].
__global__ void __launch_bounds__(256) pf_widen_kernel(uint16_t* __restrict__ Ahi, uint16_t* __restrict__ Alo, int ld,
                                                       int K) {
  const size_t row = (size_t)blockIdx.x * ld;
  for (int j = threadIdx.x; j < (K >> 3); j += blockDim.x) {
    *(u32x4*)(Ahi + row + K + 8 * j) = *(const u32x4*)(Ahi + row + 8 * j);
    *(u32x4*)(Alo + row + K + 8 * j) = u32x4{0u, 0u, 0u, 0u};
  }
}

}  // namespace

extern "C" int mk_pf_q4_expand(const void* T, int N, int K, uint16_t* Wd, void* stream) {
  const size_t n = (size_t)N * (K >> 5);
  hipLaunchKernelGGL(pf_q4_expand_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     (const uint8_t*)T, N, K, Wd);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_pf_embed_q4(const int32_t* tok, int T, const void* E, int D, int vocab, float* X, MkCtl* ctl,
                              void* stream) {
  hipLaunchKernelGGL(pf_embed_q4_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, tok, T, (const uint8_t*)E, D, vocab,
                     X, ctl);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_pf_widen(uint16_t* Ahi, uint16_t* Alo, int ld, int T, int K, void* stream) {
  hipLaunchKernelGGL(pf_widen_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, Ahi, Alo, ld, K);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

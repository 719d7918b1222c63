// Single-phase kernels for unit parity tests (include/mk_test.h; not part of the product surface).
// Each runs one phase of the decode step through the decode kernels' own device functions on
// caller buffers, so a parity failure can be pinned to that phase:
//   * the BF16 GEMV (activations split into BF16 hi + lo, v_dot2c, the unit reduction tree and the
//     segment order: gemv in mk_device.h);
//   * the 4-bit GEMV (activation packing and the v_dot8 unit sums: q4_pack and gemv_q4 in mk_q4.h);
//   * the gated delta rule on every row of every head (dn_head and dn_row in mk_device.h);
//   * the greedy choice over (value, index) pairs (wave_argmax: largest value, lowest index on ties).
// A workgroup is 512 lanes, as in the decode kernels, so every helper sees the wave roles it was
// written for.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "mk.h"
#include "mk_q4.h"
#include "mk_test.h"

namespace {

// y[r] = W[r] . x for rows split over the grid; W is BF16 [R][K] row-major, K a multiple of 8.
// LDS: x as hi/lo pairs (K floats), then the unit partials (MK_RED_CAP floats).
__global__ void __launch_bounds__(MK_NT, 1) mk_test_gemv_kernel(const uint16_t* W, int R, int K, const float* x,
                                                                float* y) {
  extern __shared__ float lds_raw[];
  LS float* lds = (LS float*)lds_raw;
  LS float* xv = lds;
  LS float* red = lds + K;
  const int NW = gridDim.x, w = blockIdx.x;
  for (int i = tid(); i < K; i += MK_NT) xv[i] = x[i];
  wg_bar();
  to_hl(xv, K);
  wg_bar();
  const int r0 = split(R, NW, w), r1 = split(R, NW, w + 1);
  Gemv g;
  g.init((const MK_G uint16_t*)(W + (size_t)r0 * K), r1 - r0, K);
  Tracer tr{nullptr, nullptr, 0};
  gemv<false, true, true>(g, (const LS u32*)xv, nullptr, 0, red, tr, [&](int r, float v, float) { y[r0 + r] = v; });
}

// y[r] = W[r] . x for a tiled 4-bit matrix (rows split over the grid in whole 4-row blocks).
// LDS: x packed in place (K floats), the unit partials (Q4_RED_CAP floats), the unit counter.
__global__ void __launch_bounds__(MK_NT, 1) mk_test_gemv_q4_kernel(const uint16_t* T, int R, int K, const float* x,
                                                                   float* y) {
  extern __shared__ float lds_raw[];
  LS float* lds = (LS float*)lds_raw;
  LS float* xv = lds;
  LS float* red = lds + K;
  LS int* ctr = (LS int*)(red + Q4_RED_CAP);
  const int NW = gridDim.x, w = blockIdx.x;
  for (int i = tid(); i < K; i += MK_NT) xv[i] = x[i];
  if (tid() == 0) *ctr = 0;
  wg_bar();
  q4_pack(xv, K);
  const int RB = (R + 3) >> 2;
  const int b0 = split(RB, NW, w), b1 = split(RB, NW, w + 1);
  GemvQ4 g;
  g.init((const MK_G uint16_t*)T, b0, max(0, min(4 * b1, R) - 4 * b0), K);
  Q4Ring q;
  Tracer tr{nullptr, nullptr, 0};
  gemv_q4<false, true>(g, (const LS u32*)xv, red, ctr, q, false, tr,
                       [&](int r, float v, float) { y[4 * b0 + r] = v; });
}

// One token of the gated delta rule on every head: in = [q H*dk | k H*dk | v H*dv | a H | b H] (the
// in-projection's outputs), S [H][dv][dk] updated in place, o [H*dv] = S' q^ per row.  Workgroup h
// takes head h; wave j takes rows j, j + 8, ...
__global__ void __launch_bounds__(MK_NT, 1) mk_test_deltanet_kernel(const float* in, int H, int dk, int dv, float l2eps,
                                                                    float* S, float* o) {
  extern __shared__ float lds_raw[];
  LS float* lds = (LS float*)lds_raw;
  LS float* q = lds;
  LS float* k = lds + dk;
  LS float* ab = lds + 2 * dk;
  const int h = blockIdx.x;
  for (int e = tid(); e < dk; e += MK_NT) {
    q[e] = in[(size_t)h * dk + e];
    k[e] = in[(size_t)H * dk + h * dk + e];
  }
  if (tid() == 0) {
    ab[0] = in[(size_t)2 * H * dk + H * dv + h];
    ab[1] = in[(size_t)2 * H * dk + H * dv + H + h];
  }
  wg_bar();
  const DnHead hs = dn_head(q, k, ab, dk, l2eps);
  for (int i = wave(); i < dv; i += MK_NWAVE) {
    MK_G float* Srow = (MK_G float*)(S + ((size_t)h * dv + i) * dk);
    float sr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int e = lane() + 64 * t;
      sr[t] = e < dk ? Srow[e] : 0.f;
    }
    const float od = dn_row(sr, q, k, hs, in[(size_t)2 * H * dk + h * dv + i], Srow, dk);
    if (lane() == 0) o[(size_t)h * dv + i] = od;
  }
}

// idx = the index of the largest v[i] (lowest index among equal maxima), over n <= 8192 values: the
// pairs go to LDS as the decode kernel's per-workgroup records do, one wave picks.
__global__ void __launch_bounds__(MK_NT, 1) mk_test_argmax_kernel(const float* v, int n, int32_t* idx) {
  extern __shared__ float lds_raw[];
  LS float* rec = (LS float*)lds_raw;
  for (int i = tid(); i < n; i += MK_NT) {
    rec[2 * i] = v[i];
    rec[2 * i + 1] = __int_as_float(i);
  }
  wg_bar();
  if (wave() == 0) {
    float b;
    int bi;
    wave_argmax(rec, n, b, bi);
    if (lane() == 0) *idx = bi;
  }
}

int launched() { return hipGetLastError() == hipSuccess ? MK_OK : MK_E_HIP; }

}  // namespace

extern "C" int mk_test_gemv(const uint16_t* d_W, int32_t R, int32_t K, const float* d_x, float* d_y, void* stream) {
  if (!d_W || !d_x || !d_y || R <= 0 || K <= 0 || K % 8 || K + MK_RED_CAP > 36 * 1024) return MK_E_INVALID;
  const int grid = std::min(256, (R + 3) / 4);
  hipLaunchKernelGGL(mk_test_gemv_kernel, dim3(grid), dim3(MK_NT), (size_t)(K + MK_RED_CAP) * 4, (hipStream_t)stream, d_W,
                     R, K, d_x, d_y);
  return launched();
}

extern "C" int mk_test_q4_tile(const void* d_src, int32_t R, int32_t K, void* d_tiles, void* stream) {
  if (!d_src || !d_tiles || R <= 0 || K <= 0 || K % 32) return MK_E_INVALID;
  return mk_launch_q4_tile(d_src, R, K, d_tiles, stream) ? MK_E_HIP : MK_OK;
}

extern "C" int mk_test_gemv_q4(const void* d_tiles, int32_t R, int32_t K, const float* d_x, float* d_y, void* stream) {
  if (!d_tiles || !d_x || !d_y || R <= 0 || K <= 0 || K % 32 || K > 8 * MK_NT * Q4_PACK_IT ||
      K + Q4_RED_CAP + 4 > 36 * 1024)
    return MK_E_INVALID;
  const int grid = std::min(256, (R + 3) / 4);
  hipLaunchKernelGGL(mk_test_gemv_q4_kernel, dim3(grid), dim3(MK_NT), (size_t)(K + Q4_RED_CAP + 4) * 4,
                     (hipStream_t)stream, (const uint16_t*)d_tiles, R, K, d_x, d_y);
  return launched();
}

extern "C" int mk_test_deltanet(const float* d_in, int32_t H, int32_t dk, int32_t dv, float l2eps, float* d_S,
                                float* d_o, void* stream) {
  if (!d_in || !d_S || !d_o || H <= 0 || dk <= 0 || dk > 256 || dv <= 0) return MK_E_INVALID;
  hipLaunchKernelGGL(mk_test_deltanet_kernel, dim3(H), dim3(MK_NT), (size_t)(2 * dk + 4) * 4, (hipStream_t)stream, d_in,
                     H, dk, dv, l2eps, d_S, d_o);
  return launched();
}

extern "C" int mk_test_argmax(const float* d_v, int32_t n, int32_t* d_idx, void* stream) {
  if (!d_v || !d_idx || n <= 0 || n > 8192) return MK_E_INVALID;
  hipLaunchKernelGGL(mk_test_argmax_kernel, dim3(1), dim3(MK_NT), (size_t)n * 8, (hipStream_t)stream, d_v, n, d_idx);
  return launched();
}

/* Test-only entry points of libmk.so: single phases of the decode step for unit parity tests.
 *
 * Not part of the product surface (include/mk.h is).  Each call runs one phase through the decode
 * kernels' own device code on caller-owned device buffers, enqueued on `stream` (a hipStream_t, or
 * NULL for the default stream); nothing is retained past the call.  Every call returns MK_OK, or
 * MK_E_INVALID (a NULL pointer or a size outside the documented range; nothing is launched) or
 * MK_E_HIP (the launch failed).  The phases follow the method as the library's decode step
 * computes it (luce-megakernel announcement, page 1, kernel-design bullets; the gated delta rule
 * as given with the method's formula).
 */
#ifndef MK_TEST_H
#define MK_TEST_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* y[r] = sum_k W[r][k] x[k], r < R, with the decode kernel's BF16 GEMV: x split into BF16 high and
 * low parts, two v_dot2c products per weight pair, the fixed unit reduction and segment order.
 * W: BF16 bits [R][K] row-major; x: FP32 [K]; y: FP32 [R].  K a multiple of 8, at most 32768. */
int mk_test_gemv(const uint16_t* d_W, int32_t R, int32_t K, const float* d_x, float* d_y, void* stream);

/* Tiles a 4-bit (MK_Q4G32) matrix from its input layout (include/mk.h, MK_Q4G32: all codes
 * row-major, then the (d, m) words) into the device layout the 4-bit kernels read.  d_tiles holds
 * ceil(R / 4) * 4 * K * 5 / 8 bytes.  K a multiple of 32. */
int mk_test_q4_tile(const void* d_src, int32_t R, int32_t K, void* d_tiles, void* stream);

/* y = W x for a tiled 4-bit matrix with the decode kernel's 4-bit GEMV: x packed per 32-column
 * block as 16-bit integers, v_dot8 products, the fixed unit reduction and segment order.
 * K a multiple of 32, at most 20480. */
int mk_test_gemv_q4(const void* d_tiles, int32_t R, int32_t K, const float* d_x, float* d_y, void* stream);

/* One token of the gated delta rule on every head, as the decode kernel's DeltaNet rows compute it:
 * d_in = [q H*dk | k H*dk | v H*dv | a H | b H] (raw in-projection outputs), q and k L2-normalised
 * (eps l2eps), alpha = exp(-softplus(a)), beta = sigmoid(b), S [H][dv][dk] updated in place to
 * alpha S (I - beta k k^T) + beta v k^T, d_o [H*dv] = S q read after the update.  dk <= 256. */
int mk_test_deltanet(const float* d_in, int32_t H, int32_t dk, int32_t dv, float l2eps, float* d_S, float* d_o,
                     void* stream);

/* *d_idx = the index of the largest of d_v[0..n) (the lowest index among equal maxima), with the
 * decode kernel's final greedy pick over (value, index) records.  n <= 8192. */
int mk_test_argmax(const float* d_v, int32_t n, int32_t* d_idx, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MK_TEST_H */

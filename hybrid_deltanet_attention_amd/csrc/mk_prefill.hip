// Prefill of a prompt chunk (positions p0 .. p0 + T - 1) on gfx950, as a short sequence of kernels
// per layer (luce-megakernel announcement, page 1: the same model as the decode path; its results
// table quotes pp520 prefill).  Where decode is a matrix-vector product per weight byte, prefill
// multiplies a T-row activation block by every weight matrix, so the projections and the FFN run on
// the MFMA matrix cores:
//
//   * activations are FP32; before a GEMM they are split into a BF16 high part and a BF16 low part
//     (x = hi + lo to about 2^-16 relative), and the GEMM accumulates hi.W + lo.W in FP32 against
//     the exact BF16 weights, so prefill keeps FP32-grade accuracy;
//   * v_mfma_f32_32x32x16_bf16: a 256-thread workgroup computes a 128 x 128 output tile, each wave a
//     64 x 64 block of 2 x 2 MFMA tiles, operands loaded straight from global memory (the tiles that
//     share weight rows are placed on the same XCD so they share its L2);
//   * the DeltaNet recurrence runs in its chunked form (64-token chunks): the parts that do not
//     depend on the state, for all chunks at once, then one state-carrying pass over the chunks;
//   * causal attention is an online-softmax loop over the KV cache (previous context included).
//
// The DeltaNet state and the KV cache are left exactly as token-by-token decode would leave them.

#include <hip/hip_runtime.h>
#include "mk_internal.h"
#include <algorithm>

typedef unsigned int u32;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// LDS is read through native vector types: loads of HIP's float4 / float2 structs are split and
// merged again late in code generation, which drops what the compiler knows about the access and
// makes it wait for every outstanding LDS-DMA copy -- the next block's prefetch included -- first.
typedef float f32x2 __attribute__((ext_vector_type(2)));

namespace {


__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((u32)h << 16); }
// round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f2bf(float f) {
  u32 u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ void split_store(float v, uint16_t* hi, uint16_t* lo, size_t i) {
  const uint16_t h = f2bf(v);
  hi[i] = h;
  lo[i] = f2bf(v - bf16f(h));
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum over each 16-lane row; every lane of the row gets it
__device__ __forceinline__ float row_sum16(float v) {
  v = dpp_add<0xB1>(v);
  v = dpp_add<0x4E>(v);
  v = dpp_add<0x141>(v);
  v = dpp_add<0x140>(v);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ __forceinline__ float softplusf_(float z) { return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z))); }

// ------------------------------------------------------------------------ embedding, norms
__global__ void pf_embed_kernel(const int32_t* __restrict__ tok, int T, const uint16_t* __restrict__ embed, int D,
                                int vocab, float* __restrict__ X, MkCtl* ctl) {
  const int t = blockIdx.x;
  if (t >= T) return;
  const int id = tok[t];
  if (id < 0 || id >= vocab) {
    if (threadIdx.x == 0) __hip_atomic_store(&ctl->err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = threadIdx.x; i < D; i += blockDim.x) X[(size_t)t * D + i] = 0.f;
    return;
  }
  for (int i = threadIdx.x; i < D; i += blockDim.x) X[(size_t)t * D + i] = bf16f(embed[(size_t)id * D + i]);
}

// rows of X -> rmsnorm(x) * g, split into BF16 hi/lo (one 256-thread workgroup per row)
__global__ void __launch_bounds__(256) pf_rms_split_kernel(const float* __restrict__ X, int D,
                                                           const uint16_t* __restrict__ g, float eps,
                                                           uint16_t* __restrict__ Ahi, uint16_t* __restrict__ Alo,
                                                           int lda) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const float* x = X + (size_t)t * D;
  float s = 0.f;
  for (int i = threadIdx.x; i < D; i += 256) s = fmaf(x[i], x[i], s);
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  s = red[0] + red[1] + red[2] + red[3];
  const float r = 1.0f / sqrtf(s / (float)D + eps);
  for (int i = threadIdx.x; i < D; i += 256) split_store(x[i] * r * bf16f(g[i]), Ahi, Alo, (size_t)t * lda + i);
}

// ------------------------------------------------------------------------ MFMA GEMM
// C[M x N] (+)= (Ahi + Alo)[M x K] . W[N x K]^T.  K is a multiple of 8.
// EPI 0: C = v;  EPI 1: C += v (residual);  EPI 2: columns (2c, 2c + 1) are (gate c, up c):
// H[:, c] = silu(gate) * up, stored split into BF16 hi/lo;  EPI 3: split-K partial, stored to
// P[split][M][N] (K split into ksplit ranges of whole chunks; pf_splitk_add_kernel adds the partials
// to C in split order, so the result does not depend on timing).
//
// A workgroup (4 waves, 2 x 2) computes a BM x BN tile; each wave a (BM/2) x (BN/2) block of 32 x 32
// MFMA tiles.  K advances in chunks of 64 through a ring of STAGES LDS buffers filled with LDS-DMA
// (a wave copy is 8 rows x 128 bytes); a wave waits only for its own copies of the chunk it is about
// to use, and the barriers order LDS only, so later chunks stay in flight.
constexpr int BK = 64;
// LDS ring depth: two stages (one chunk loads while the other is used).  Deeper rings measured no
// faster: 64-wide chunks already halve the barriers per product, and two 32 KB stages of a 64 x 128
// tile leave room for two workgroups per CU
template <int BM>
constexpr int gemm_stages() { return 2; }

__device__ __forceinline__ void lds_bar() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// at most n outstanding, rounded down to a supported count (waiting for more is always correct)
__device__ __forceinline__ void wait_vm_n(int n) {
  n = __builtin_amdgcn_readfirstlane(n);
  if (n >= 32) wait_vm<32>();
  else if (n >= 16) wait_vm<16>();
  else if (n >= 12) wait_vm<12>();
  else if (n >= 8) wait_vm<8>();
  else if (n >= 6) wait_vm<6>();
  else if (n >= 4) wait_vm<4>();
  else if (n >= 3) wait_vm<3>();
  else if (n >= 2) wait_vm<2>();
  else if (n >= 1) wait_vm<1>();
  else wait_vm<0>();
}

// Waves per workgroup in rows x columns of the tile: eight waves (4 x 2 for 128-row tiles, 2 x 4
// for 64 x 128) where each still gets whole 32 x 32 blocks and the tile's copies split evenly,
// else 2 x 2.  More waves per CU hide the LDS-read and barrier latency of the others.
template <int BM, int BN>
constexpr bool gemm_eight() { return (BM >= 128 || BN >= 128) && ((2 * (BM / 8) + BN / 8) % 8) == 0; }
template <int BM, int BN>
constexpr int gemm_wr() { return gemm_eight<BM, BN>() ? (BM >= 128 ? 4 : 2) : 2; }
template <int BM, int BN>
constexpr int gemm_wc() { return gemm_eight<BM, BN>() ? (BM >= 128 ? 2 : 4) : 2; }
template <int BM, int BN>
constexpr int gemm_threads() { return 64 * gemm_wr<BM, BN>() * gemm_wc<BM, BN>(); }

template <int BM, int BN, int EPI>
__global__ void __launch_bounds__((gemm_threads<BM, BN>())) pf_gemm_kernel(
    const uint16_t* __restrict__ Ahi, const uint16_t* __restrict__ Alo, int lda, int M, int K,
    const uint16_t* __restrict__ W, int N, float* __restrict__ C, int ldc, uint16_t* __restrict__ Hhi,
    uint16_t* __restrict__ Hlo, int ldh, int ksplit) {
  constexpr int WR = gemm_wr<BM, BN>(), WC = gemm_wc<BM, BN>(), NWV = WR * WC;
  constexpr int TI = BM / (32 * WR), TJ = BN / (32 * WC);  // 32 x 32 tiles per wave in each direction
  constexpr int AC = BM / 8, BC = BN / 8;                // 1 KB copies per tile per chunk
  constexpr int CPW = (2 * AC + BC) / NWV;                 // copies per wave per chunk
  static_assert(TI >= 1 && TJ >= 1 && CPW * NWV == 2 * AC + BC, "tile does not split over the waves");
  constexpr int SB = (2 * BM + BN) * BK * 2;           // bytes per stage
  constexpr int STAGES = gemm_stages<BM>();
  static_assert(BK == 64, "the LDS chunk swizzle assumes eight 16-byte k-chunks per row");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int mb = (M + BM - 1) / BM, nb = (N + BN - 1) / BN;
  const int items = mb * nb * ksplit, per = (items + 7) / 8;
  const int w = blockIdx.x;
  // work items of one column block (same weight rows) go to one XCD (workgroup w runs on XCD w % 8)
  const int item = (w % 8) * per + w / 8;
  if (item >= items) return;
  const int tile = item / ksplit, split = item - tile * ksplit;
  const int m0 = (tile % mb) * BM, n0 = (tile / mb) * BN;
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int wr = wv / WC, wc = wv % WC;  // this wave's (BM / WR) x (BN / WC) block
  const int nk = (K + BK - 1) / BK, kper = (nk + ksplit - 1) / ksplit;
  const int cbeg = split * kper, nchunk = max(0, min(nk, cbeg + kper) - cbeg);
  // Copy q (0 .. 2AC + BC) of a chunk: tile part (A hi, A lo, B) and 8-row group; wave wv issues
  // copies wv * CPW .. + CPW.  Rows past M / N read the last row instead (their results are never
  // stored), so every copy has live lanes and each wave issues exactly CPW copies per chunk -- the
  // waits below count on that.  Columns past K are left out; a chunk that has them was zeroed by the
  // same wave first (its own 1 KB blocks only, so no other wave's copy can be overwritten).
  auto issue = [&](int chunk) {  // chunk: index within this work item's K range
    char* st = smem + (size_t)(chunk % STAGES) * SB;
    const int k0 = (cbeg + chunk) * BK;
    const bool part_k = k0 + BK > K;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int q = wv * CPW + i;
      const int part = q < AC ? 0 : (q < 2 * AC ? 1 : 2);
      const int grp = part == 0 ? q : (part == 1 ? q - AC : q - 2 * AC);
      const int r = grp * 8 + (l >> 3);
      // lane l fills LDS position (row r, 16-byte slot l & 7) with the row's k-chunk
      // (l & 7) ^ (r & 7): eight consecutive rows then spread one chunk over all banks
      const int k = k0 + (((l & 7) ^ (r & 7)) * 8);
      const uint16_t* src;
      if (part < 2) src = (part == 0 ? Ahi : Alo) + (size_t)min(m0 + r, M - 1) * lda + k;
      else src = W + (size_t)min(n0 + r, N - 1) * K + k;
      char* dst = st + (part == 0 ? 0 : (part == 1 ? BM * BK * 2 : 2 * BM * BK * 2)) + grp * 1024;
      if (part_k) {
        ((u32x4*)dst)[l] = u32x4{0u, 0u, 0u, 0u};
        __builtin_amdgcn_s_waitcnt(0xC07F);
      }
      if (k < K) __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
  };
  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};
#pragma unroll
  for (int c = 0; c < STAGES - 1; ++c)
    if (c < nchunk) issue(c);
  for (int c = 0; c < nchunk; ++c) {
    // this wave's copies of chunk c are done once at most (later chunks issued) copies remain
    const int later = min(STAGES - 2, nchunk - 1 - c);
    if (later >= 4) wait_vm<4 * CPW>();
    else if (later == 3) wait_vm<3 * CPW>();
    else if (later == 2) wait_vm<2 * CPW>();
    else if (later == 1) wait_vm<CPW>();
    else wait_vm<0>();
    lds_bar();
    // chunk c + STAGES - 1 reuses the buffer of chunk c - 1, which every wave has finished
    const int cn = c + STAGES - 1;
    if (cn < nchunk) issue(cn);
    const char* st = smem + (size_t)(c % STAGES) * SB;
    const char* sah = st;
    const char* sal = st + BM * BK * 2;
    const char* sb = st + 2 * BM * BK * 2;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kc = ks * 2 + (l >> 5);  // this lane's 8-wide k-chunk of the row
      bf16x8 fh[TI], fl[TI], fb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int r = wr * (BM / WR) + i * 32 + (l & 31);
        const int kb = (kc ^ (r & 7)) * 16;
        fh[i] = *(const bf16x8*)(sah + r * (BK * 2) + kb);
        fl[i] = *(const bf16x8*)(sal + r * (BK * 2) + kb);
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int r = wc * (BN / WC) + j * 32 + (l & 31);
        fb[j] = *(const bf16x8*)(sb + r * (BK * 2) + (kc ^ (r & 7)) * 16);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fh[i], fb[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl[i], fb[j], acc[i][j], 0, 0, 0);
        }
    }
  }
  // result: accumulator r of lane l sits at row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wr * (BM / WR) + i * 32 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        const int col = n0 + wc * (BN / WC) + j * 32 + (l & 31);
        const float v = acc[i][j][r];
        if (EPI == 2) {
          // the odd neighbour lane holds the up value of the same hidden unit
          const float u = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
          if ((l & 1) == 0 && row < M && col + 1 < N) {
            const float h = v / (1.0f + expf(-v)) * u;
            split_store(h, Hhi, Hlo, (size_t)row * ldh + (col >> 1));
          }
        } else if (EPI == 3) {
          if (row < M && col < N) C[((size_t)split * M + row) * N + col] = v;
        } else if (row < M && col < N) {
          float* cp = C + (size_t)row * ldc + col;
          if (EPI == 1) *cp += v;
          else *cp = v;
        }
      }
}

// One workgroup per row r: C[r] += the ksplit partials, added in split order.  With a gain g the
// updated row is then RMS-normalised (eps, gain after normalising) into the split-bf16 operand
// (Ahi, Alo) of the next projection, so the residual add and the next block's norm share one pass.
__global__ void __launch_bounds__(256) pf_splitk_add_kernel(const float* __restrict__ P, int ksplit, int M, int N,
                                                            float* __restrict__ C, int ldc,
                                                            const uint16_t* __restrict__ g, float eps,
                                                            uint16_t* __restrict__ Ahi, uint16_t* __restrict__ Alo,
                                                            int lda) {
  __shared__ float red[4];
  const int r = blockIdx.x;  // N is a multiple of 4
  float* c = C + (size_t)r * ldc;
  float ss = 0.f;
  for (int j = threadIdx.x * 4; j < N; j += 1024) {
    f32x4 acc = *(const f32x4*)(c + j);
    for (int sp = 0; sp < ksplit; ++sp) {
      const f32x4 v = *(const f32x4*)(P + ((size_t)sp * M + r) * N + j);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    *(f32x4*)(c + j) = acc;
    ss = fmaf(acc.x, acc.x, fmaf(acc.y, acc.y, fmaf(acc.z, acc.z, fmaf(acc.w, acc.w, ss))));
  }
  if (!g) return;
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  ss = red[0] + red[1] + red[2] + red[3];
  const float rn = 1.0f / sqrtf(ss / (float)N + eps);
  for (int j = threadIdx.x * 4; j < N; j += 1024) {
    const f32x4 a = *(const f32x4*)(c + j);  // this thread's own store above
    const size_t o = (size_t)r * lda + j;
    split_store(a.x * rn * bf16f(g[j]), Ahi, Alo, o);
    split_store(a.y * rn * bf16f(g[j + 1]), Ahi, Alo, o + 1);
    split_store(a.z * rn * bf16f(g[j + 2]), Ahi, Alo, o + 2);
    split_store(a.w * rn * bf16f(g[j + 3]), Ahi, Alo, o + 3);
  }
}

// ------------------------------------------------------------------------ DeltaNet
// per (token, head): q, k L2-normalised -> QK[t][h][0..dk) = q, [dk..2dk) = k; AB[t][h] = (log alpha, beta)
__global__ void __launch_bounds__(64) pf_dn_prep_kernel(const float* __restrict__ Y, int ldy, int H, int dk, int dv,
                                                        float l2eps, float* __restrict__ QK, float* __restrict__ AB) {
  const int t = blockIdx.x / H, h = blockIdx.x % H;
  const float* y = Y + (size_t)t * ldy;
  const float* q = y + h * dk;
  const float* k = y + H * dk + h * dk;
  float qq = 0.f, kk = 0.f;
  for (int e = threadIdx.x; e < dk; e += 64) {
    qq = fmaf(q[e], q[e], qq);
    kk = fmaf(k[e], k[e], kk);
  }
  qq = wave_sum(qq);
  kk = wave_sum(kk);
  const float sq = 1.0f / sqrtf(qq + l2eps), sk = 1.0f / sqrtf(kk + l2eps);
  float* o = QK + ((size_t)t * H + h) * 2 * dk;
  for (int e = threadIdx.x; e < dk; e += 64) {
    o[e] = q[e] * sq;
    o[dk + e] = k[e] * sk;
  }
  if (threadIdx.x == 0) {
    const int off_a = 2 * H * dk + H * dv;
    AB[((size_t)t * H + h) * 2] = -softplusf_(y[off_a + h]);  // log alpha
    AB[((size_t)t * H + h) * 2 + 1] = sigmoidf_(y[off_a + H + h]);
  }
}

// Gated delta rule over T tokens, row-parallel.  A workgroup (4 waves, one per SIMD) owns 8 rows of
// one head's state: 2 rows per wave, 32 lanes per row, NE = dk / 32 consecutive key elements per
// lane, the row in registers; a row sum is a 16-lane DPP reduction plus one permlane16 swap.  Tokens
// go through LDS in chunks of TC: while a chunk is processed the next chunk's q, k, gates and v are
// already loading into registers.  o = S q is read after each update.
constexpr int TC = 32;
__device__ __forceinline__ float sum32(float v) {
  v = row_sum16(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int NE>
__global__ void __launch_bounds__(256) pf_dn_scan_kernel(float* __restrict__ S, const float* __restrict__ QK,
                                                         const float* __restrict__ AB, const float* __restrict__ Y,
                                                         int ldy, int T, int H, int dk, int dv,
                                                         uint16_t* __restrict__ Ohi, uint16_t* __restrict__ Olo,
                                                         int ldo) {
  constexpr int DKM = 32 * NE;  // key width held per row
  constexpr int RW = 8;         // rows per workgroup
  __shared__ __attribute__((aligned(16))) float sqk[2][TC][2 * DKM];
  __shared__ float sab[2][TC][2];
  __shared__ float sv[2][TC][RW];
  const int rbs = (dv + RW - 1) / RW;
  const int h = blockIdx.x / rbs, r0 = (blockIdx.x % rbs) * RW;
  const int tid = threadIdx.x, l = tid & 63, wv = tid >> 6;
  const int rl = wv * 2 + (l >> 5), c = l & 31;  // local row, lane within the row
  const int i = r0 + rl;
  const bool valid = i < dv;
  float* srow = S + ((size_t)h * dv + (valid ? i : 0)) * dk;
  float s[NE];
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    const int e = NE * c + j;
    s[j] = (valid && e < dk) ? srow[e] : 0.f;
  }
  const int off_v = 2 * H * dk + h * dv + r0;
  constexpr int QK_PER = (TC * 2 * DKM + 255) / 256;
  float rq[QK_PER], rab = 0.f, rvv = 0.f;
  auto fetch = [&](int t0) {
#pragma unroll
    for (int x = 0; x < QK_PER; ++x) {
      const int f = tid + 256 * x;
      const int tt = f / (2 * DKM), e = f % (2 * DKM);
      const int t = t0 + tt;
      const bool isk = e >= DKM;
      const int ee = isk ? e - DKM : e;
      rq[x] = (tt < TC && t < T && ee < dk) ? QK[((size_t)t * H + h) * 2 * dk + (isk ? dk : 0) + ee] : 0.f;
    }
    {
      const int t = t0 + (tid >> 1);
      rab = (tid < 2 * TC && t < T) ? AB[((size_t)t * H + h) * 2 + (tid & 1)] : 0.f;
    }
    {
      const int tt = tid / RW, rr = tid % RW, t = t0 + tt;
      rvv = (tt < TC && t < T && r0 + rr < dv) ? Y[(size_t)t * ldy + off_v + rr] : 0.f;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int x = 0; x < QK_PER; ++x) {
      const int f = tid + 256 * x;
      const int tt = f / (2 * DKM), e = f % (2 * DKM);
      if (tt < TC) sqk[buf][tt][e] = rq[x];
    }
    if (tid < 2 * TC) sab[buf][tid >> 1][tid & 1] = rab;
    if (tid / RW < TC) sv[buf][tid / RW][tid % RW] = rvv;
  };
  fetch(0);
  stash(0);
  __syncthreads();
  for (int t0 = 0, buf = 0; t0 < T; t0 += TC, buf ^= 1) {
    if (t0 + TC < T) fetch(t0 + TC);
    const int nt = min(TC, T - t0);
    // the next step's operands are read from LDS while the current step computes
    float q[NE], k[NE], a, b, v;
    auto lds_step = [&](int tt, float* qo, float* ko, float& ao, float& bo, float& vo) {
      const float* qp = &sqk[buf][tt][NE * c];
      const float* kp = &sqk[buf][tt][DKM + NE * c];
      if constexpr (NE % 4 == 0) {
#pragma unroll
        for (int j = 0; j < NE; j += 4) {
          const f32x4 x = *(const f32x4*)(qp + j);
          const f32x4 y = *(const f32x4*)(kp + j);
          qo[j] = x.x; qo[j + 1] = x.y; qo[j + 2] = x.z; qo[j + 3] = x.w;
          ko[j] = y.x; ko[j + 1] = y.y; ko[j + 2] = y.z; ko[j + 3] = y.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < NE; ++j) {
          qo[j] = qp[j];
          ko[j] = kp[j];
        }
      }
      ao = expf(sab[buf][tt][0]);
      bo = sab[buf][tt][1];
      vo = sv[buf][tt][rl];
    };
    auto step = [&](int tt, const float* qv, const float* kv, float av, float bv, float vv) {
      float kd = 0.f;
#pragma unroll
      for (int j = 0; j < NE; ++j) kd = fmaf(s[j], kv[j], kd);
      kd = sum32(kd);
      const float u = bv * (vv - av * kd);
      float od = 0.f;
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        s[j] = fmaf(u, kv[j], av * s[j]);
        od = fmaf(s[j], qv[j], od);
      }
      od = sum32(od);
      if (c == 0 && valid) split_store(od, Ohi, Olo, (size_t)(t0 + tt) * ldo + h * dv + i);
    };
    // two steps per round with ping-pong operands: the reads for step t + 1 are in flight while
    // step t computes, in straight-line code (TC is even, so every read stays inside the chunk; a
    // step past the chunk's last token is skipped)
    float q2[NE], k2[NE], a2, b2, v2;
    lds_step(0, q, k, a, b, v);
    for (int tt = 0; tt < nt; tt += 2) {
      lds_step(tt + 1, q2, k2, a2, b2, v2);
      step(tt, q, k, a, b, v);
      if (tt + 2 < TC) lds_step(tt + 2, q, k, a, b, v);
      if (tt + 1 < nt) step(tt + 1, q2, k2, a2, b2, v2);
    }
    __syncthreads();
    if (t0 + TC < T) stash(buf ^ 1);
    __syncthreads();
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const int e = NE * c + j;
      if (e < dk) srow[e] = s[j];
    }
  }
}

// ---- chunked (UT) form of the gated delta rule
// Gated DeltaNet (Yang, Kautz, Hatamizadeh, ICLR 2025), chunkwise algorithm; derived here from the
// recurrence S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T in row form (S is dv x dk).
// Within a chunk of C tokens with state S0 on entry, gamma_t = prod_{i<=t} alpha_i and
// G_tj = gamma_t / gamma_j (exp of a difference of cumulative log alphas, never above 1 for j <= t):
//   (I + M) U = diag(beta) (V - diag(gamma) K S0^T),   M = strict lower part of diag(beta) (K K^T o G)
//   O   = diag(gamma) Q S0^T + (lower part incl. diagonal of Q K^T o G) U
//   S_C = gamma_C S0 + U^T diag(gamma_C / gamma) K
// (rows of K, Q, V, U, O are tokens).  Everything that does not involve S0 -- K K^T, Q K^T, the
// decays and W = (I + M)^{-1} diag(beta) -- is computed for all chunks in parallel
// (pf_dn_cprep_kernel); the pass that carries the state runs chunk after chunk, each workgroup on
// 16 rows of one head's state (pf_dn_cscan_mfma_kernel).
constexpr int PC = 64;                          // tokens per chunk
constexpr int PC_BLK = 2 * PC * PC + 2 * PC + 4;  // per (chunk, head): W, Bt [PC][PC], gam, dlt [PC], gamma_C

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b, float acc) {
  acc = fmaf(a.x, b.x, acc);
  acc = fmaf(a.y, b.y, acc);
  acc = fmaf(a.z, b.z, acc);
  return fmaf(a.w, b.w, acc);
}

// FP32 matrix-core helpers (v_mfma_f32_16x16x4_f32: exact FP32 products, FP32 sums).
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// c + A B^T over NK shared columns, A and B given by this lane's row (arow: M-side row lane % 16,
// brow: N-side row lane % 16).  Within each 16-column block, lane group lk = lane / 16 reads its
// four contiguous columns 4 lk .. 4 lk + 3 with one 16-byte load and feeds them to four MFMAs (the
// k-th MFMA of the block takes column 4 lk + k from every lane group: a partition of the block).
// Two accumulators alternate between blocks so consecutive MFMAs do not wait for each other.
template <int NK>
__device__ __forceinline__ f32x4 mfma_rows(const float* arow, const float* brow, f32x4 c) {
  const int lk = (threadIdx.x & 63) >> 4;
  f32x4 acc[2] = {c, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int m = 0; m < NK / 16; ++m) {
    const f32x4 a = *(const f32x4*)(arow + 16 * m + 4 * lk);
    const f32x4 b = *(const f32x4*)(brow + 16 * m + 4 * lk);
    f32x4& d = acc[m & 1];
    d = mfma4(a.x, b.x, d);
    d = mfma4(a.y, b.y, d);
    d = mfma4(a.z, b.z, d);
    d = mfma4(a.w, b.w, d);
  }
  return acc[0] + acc[1];
}
// 16 x 16 blocks in LDS (row strides lda, ldb) on one wave: c + A B, with lane (lr = lane % 16,
// lk = lane / 16) holding rows 4 lk .. 4 lk + 3 of column lr of the result (the MFMA's output
// layout); the s-th MFMA takes k = 4 s + lk from every lane
__device__ __forceinline__ f32x4 mm16(const float* A, int lda, const float* B, int ldb, f32x4 c) {
  const int lr = threadIdx.x & 15, lk = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int s = 0; s < 4; ++s) c = mfma4(A[lr * lda + 4 * s + lk], B[(4 * s + lk) * ldb + lr], c);
  return c;
}
// store / load a block in that layout (stores scaled by f)
__device__ __forceinline__ void put16(float* D, int ld, f32x4 v, float f) {
  const int lr = threadIdx.x & 15, lk = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) D[(4 * lk + r) * ld + lr] = f * v[r];
}
__device__ __forceinline__ f32x4 get16(const float* D, int ld) {
  const int lr = threadIdx.x & 15, lk = (threadIdx.x & 63) >> 4;
  f32x4 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = D[(4 * lk + r) * ld + lr];
  return v;
}
// Per (chunk c, head h): the chunk's L2-normalised q and k (written to QK for the state pass, head
// major: QK[h][t][q | k], so a head's chunk is one contiguous 64 KB block), then
// W = (I + M)^{-1} diag(beta) and Bt = lower(Q K^T o G) incl. the diagonal (both [t][j]),
// gam_t = gamma_t, dlt_t = gamma_last / gamma_t, gamma_last.  Tokens past the end of the prompt
// have k = q = 0 and beta = 0, so their rows and columns come out zero.
template <int DKM>
__global__ void __launch_bounds__(256) pf_dn_cprep_kernel(const float* __restrict__ Y, int ldy, int T, int H, int dk,
                                                          int dv, float l2eps, float* __restrict__ QK,
                                                          float* __restrict__ CH) {
  __shared__ __attribute__((aligned(16))) float sk[PC][DKM + 4];
  __shared__ __attribute__((aligned(16))) float sq[PC][DKM + 4];
  __shared__ float sm[PC][PC + 1];  // M, strictly lower
  __shared__ float sx[PC][PC + 1];  // (I + M)^{-1}
  __shared__ float sg[PC], sbeta[PC];
  const int h = blockIdx.x % H, c = blockIdx.x / H;
  const int t0 = c * PC, Cn = min(PC, T - t0);
  const int tid = threadIdx.x;
  const int n4 = dk >> 2;
  if (dk < DKM) {  // key columns past dk take part in the products as zeros
    for (int f = tid; f < PC * (DKM + 4); f += 256) {
      (&sk[0][0])[f] = 0.f;
      (&sq[0][0])[f] = 0.f;
    }
    __syncthreads();
  }
  {
    // every load of the chunk is issued before the first is used
    constexpr int NL = PC * DKM / 4 / 256;
    f32x4 rq[NL], rk[NL];
#pragma unroll
    for (int x = 0; x < NL; ++x) {
      const int f = tid + 256 * x, t = f / n4, e = (f - t * n4) * 4;
      rq[x] = f32x4{0.f, 0.f, 0.f, 0.f};
      rk[x] = rq[x];
      if (t < Cn) {
        const float* src = Y + (size_t)(t0 + t) * ldy + h * dk;
        rq[x] = *(const f32x4*)(src + e);
        rk[x] = *(const f32x4*)(src + H * dk + e);
      }
    }
#pragma unroll
    for (int x = 0; x < NL; ++x) {
      const int f = tid + 256 * x, t = f / n4, e = (f - t * n4) * 4;
      if (t < PC) {
        *(f32x4*)&sq[t][e] = rq[x];
        *(f32x4*)&sk[t][e] = rk[x];
      }
    }
  }
  if (tid < PC) {  // log alpha = -softplus(a), beta = sigmoid(b)
    const bool in = tid < Cn;
    const float* ab = Y + (size_t)(t0 + (in ? tid : 0)) * ldy + 2 * H * dk + H * dv + h;
    sg[tid] = in ? -softplusf_(ab[0]) : 0.f;
    sbeta[tid] = in ? sigmoidf_(ab[H]) : 0.f;
  }
  __syncthreads();
  {
    // L2 normalisation: two lanes per (token, q or k) row, each summing every other 4-element group
    const int row = tid >> 1, t = row >> 1, half = tid & 1;
    float* v = (row & 1) ? &sk[t][0] : &sq[t][0];
    float ss = 0.f;
#pragma unroll
    for (int e = 4 * half; e < DKM; e += 8) ss = dot4(*(const f32x4*)(v + e), *(const f32x4*)(v + e), ss);
    ss += __shfl_xor(ss, 1);
    const float rn = 1.0f / sqrtf(ss + l2eps);
    float* o = QK + ((size_t)h * T + t0 + t) * 2 * dk + ((row & 1) ? dk : 0);
#pragma unroll
    for (int e = 4 * half; e < DKM; e += 8) {
      const f32x4 a = *(const f32x4*)(v + e);
      const f32x4 b = f32x4{a.x * rn, a.y * rn, a.z * rn, a.w * rn};
      *(f32x4*)(v + e) = b;
      if (t < Cn && e < dk) *(f32x4*)(o + e) = b;
    }
  }
  __syncthreads();
  if (tid == 0) {  // cumulative log alpha, inclusive
    float a = 0.f;
    for (int t = 0; t < PC; ++t) {
      a += sg[t];
      sg[t] = a;
    }
  }
  // K K^T and Q K^T on and below the diagonal, 16 x 16 blocks on the matrix cores: task = (matrix,
  // lower-triangle block); a lane holds rows 16 bt + 4 lk + r of column 16 bj + lr
  const int wv = tid >> 6, lane64 = tid & 63, lr = lane64 & 15, lk = lane64 >> 4;
  f32x4 acc[5];
#pragma unroll
  for (int x = 0; x < 5; ++x) {
    const int task = wv + 4 * x, mat = task / 10, bb = task - mat * 10;
    const int bt = bb >= 6 ? 3 : (bb >= 3 ? 2 : (bb >= 1 ? 1 : 0)), bj = bb - bt * (bt + 1) / 2;
    acc[x] = mfma_rows<DKM>(mat ? &sq[16 * bt + lr][0] : &sk[16 * bt + lr][0], &sk[16 * bj + lr][0],
                            f32x4{0.f, 0.f, 0.f, 0.f});
  }
  __syncthreads();  // cumulative log alphas are in place
  float* blk = CH + ((size_t)c * H + h) * PC_BLK;
  float* gW = blk;
  float* gBt = blk + PC * PC;
  float* gGam = blk + 2 * PC * PC;
  float* gDlt = gGam + PC;
#pragma unroll
  for (int x = 0; x < 5; ++x) {
    const int task = wv + 4 * x, mat = task / 10, bb = task - mat * 10;
    const int bt = bb >= 6 ? 3 : (bb >= 3 ? 2 : (bb >= 1 ? 1 : 0)), bj = bb - bt * (bt + 1) / 2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * bt + 4 * lk + r, j = 16 * bj + lr;
      const float dec = j <= t ? expf(sg[t] - sg[j]) : 0.f;
      if (mat == 0) sm[t][j] = j < t ? sbeta[t] * dec * acc[x][r] : 0.f;
      else gBt[t * PC + j] = j <= t ? dec * acc[x][r] : 0.f;
    }
  }
  // blocks above the diagonal
  for (int f = tid; f < PC * PC; f += 256) {
    const int t = f / PC, j = f - t * PC;
    if ((j >> 4) > (t >> 4)) {
      sm[t][j] = 0.f;
      gBt[f] = 0.f;
    }
  }
  if (tid < PC) {
    const float last = sg[Cn - 1];
    gGam[tid] = expf(sg[tid]);
    gDlt[tid] = expf(last - sg[tid]);
    if (tid == 0) gDlt[PC] = expf(last);
  }
  __syncthreads();
  // W = (I + M)^{-1} diag(beta), M strictly lower.  X = (I + M)^{-1} by blocks of 16 on the matrix
  // cores.  Diagonal block N = M_ii (nilpotent, N^16 = 0), one wave each:
  //   (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8)
  // (the factors are polynomials in N, so they commute).  Then block row by block row
  //   X_ij = -X_ii T_ij,  T_ij = sum_{j <= m < i} M_im X_mj,  one wave per j.
  // The waves' 16 x 16 scratch blocks reuse the query tile, which is no longer read.
  float* scr = &sq[0][0] + wv * 3 * 256;
  {
    float* X = scr;           // running product
    float* Pw = scr + 256;    // N^(2^p)
    const float* Nb = &sm[16 * wv][16 * wv];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane64 + 64 * q, rr = e >> 4, cc = e & 15;
      X[e] = (rr == cc ? 1.f : 0.f) - Nb[rr * (PC + 1) + cc];
    }
    const float* A = Nb;
    int ld = PC + 1;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const f32x4 sq2 = mm16(A, ld, A, ld, f32x4{0.f, 0.f, 0.f, 0.f});  // N^(2^(p+1))
      put16(Pw, 16, sq2, 1.f);
      A = Pw;
      ld = 16;
      put16(X, 16, mm16(X, 16, Pw, 16, get16(X, 16)), 1.f);  // X (I + N^(2^(p+1)))
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane64 + 64 * q, rr = e >> 4, cc = e & 15;
      sx[16 * wv + rr][16 * wv + cc] = X[e];
    }
  }
  __syncthreads();
  for (int i = 1; i < 4; ++i) {
    const int j = wv;
    if (j < i) {
      f32x4 t4 = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int m = j; m < i; ++m) t4 = mm16(&sm[16 * i][16 * m], PC + 1, &sx[16 * m][16 * j], PC + 1, t4);
      put16(scr, 16, t4, 1.f);
      put16(&sx[16 * i][16 * j], PC + 1, mm16(&sx[16 * i][16 * i], PC + 1, scr, 16, f32x4{0.f, 0.f, 0.f, 0.f}), -1.f);
    }
    __syncthreads();
  }
  for (int f = tid; f < PC * PC; f += 256) {
    const int t = f / PC, j = f - t * PC;
    gW[f] = j <= t ? sx[t][j] * sbeta[j] : 0.f;
  }
}

// The state-carrying pass, chunk after chunk with state S0 on entry:
//   Z = K S0^T, P = Q S0^T, R = V - diag(gam) Z, U = W R,
//   O = diag(gam) P + Bt U -> outputs (hi/lo BF16), S <- gamma_C S0 + (diag(dlt) U)^T K.
constexpr int CS_NT = 512;
// On the FP32 matrix cores (v_mfma_f32_16x16x4_f32: exact FP32 products, FP32 sums): workgroup =
// (head, 16 state rows), 8 waves.  The products are formed transposed, rows of
// the state as the 16-row M side:
//   Z^T = S0 K^T, P^T = S0 Q^T           waves 0-3 / 4-7, one 16-token block each
//   R^T = V^T - Z^T diag(gam)            waves 0-3, in registers -> LDS
//   U^T = R^T W^T                        waves 0-3
//   O^T = P^T diag(gam) + U^T Bt^T       waves 4-7 -> outputs (hi/lo BF16)
//   S   = gamma_C S0 + (U^T diag(dlt)) K one 16-column block of keys per wave
// Per chunk the operands move through LDS once per MFMA fragment instead of once per output.
constexpr int CM_RW = 16;
template <int DKM>
__global__ void __launch_bounds__(CS_NT) pf_dn_cscan_mfma_kernel(float* __restrict__ S, const float* __restrict__ QK,
                                                                 const float* __restrict__ CH,
                                                                 const float* __restrict__ Y, int ldy, int T, int H,
                                                                 int dk, int dv, uint16_t* __restrict__ Ohi,
                                                                 uint16_t* __restrict__ Olo, int ldo) {
  constexpr int RW = CM_RW, LK = DKM + 4, LC = PC + 4;
  __shared__ __attribute__((aligned(16))) float sk[PC][LK];
  __shared__ __attribute__((aligned(16))) float sq[PC][LK];
  __shared__ __attribute__((aligned(16))) float sw[PC][LC];
  __shared__ __attribute__((aligned(16))) float sbt[PC][LC];
  __shared__ __attribute__((aligned(16))) float ss[RW][LK];
  __shared__ __attribute__((aligned(16))) float sr[RW][LC];
  __shared__ __attribute__((aligned(16))) float su[RW][LC];
  __shared__ float sv[PC][RW];
  __shared__ __attribute__((aligned(16))) float sgam[PC];
  __shared__ __attribute__((aligned(16))) float sdlt[PC + 4];
  // workgroup b takes head b % H and row block b / H: the row blocks of one head share an XCD
  // (workgroups are dealt to the 8 XCDs round-robin), so that head's chunk operands are fetched
  // into one L2 rather than into eight
  const int h = blockIdx.x % H, r0 = (blockIdx.x / H) * RW;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, lr = l & 15, lk = l >> 4;
  const int n4 = dk >> 2;
  if (dk < DKM) {  // key columns past dk take part in the products as zeros
    for (int f = tid; f < PC * LK; f += CS_NT) {
      (&sk[0][0])[f] = 0.f;
      (&sq[0][0])[f] = 0.f;
    }
    for (int f = tid; f < RW * LK; f += CS_NT) (&ss[0][0])[f] = 0.f;
    __syncthreads();
  }
  for (int f = tid; f < RW * n4; f += CS_NT) {
    const int i = f / n4, e = (f - i * n4) * 4;
    *(f32x4*)&ss[i][e] = r0 + i < dv ? *(const f32x4*)(S + ((size_t)h * dv + r0 + i) * dk + e)
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int off_v = 2 * H * dk + h * dv + r0;
  const int nc = (T + PC - 1) / PC;
  // a chunk's operands are loaded into registers two chunks ahead (two register sets, used in
  // turn; the chunk index is clamped so every set is always loaded and the load counts stay uniform).
  // Every load is unconditional -- rows past the chunk and rows past dv read a valid row and are
  // zeroed when stashed: a register whose load sits behind a branch cannot be placed in the in-order
  // load count, and the wait before its use then also drains the loads of the later chunks.
  constexpr int NL = PC * DKM / 4 / CS_NT, NM = PC * PC / 4 / CS_NT, NV = PC * RW / CS_NT;
  struct Ops {
    f32x4 rq[NL], rk[NL], rw[NM], rb[NM];
    float rg, rv[NV];
  };
  Ops oa, ob;
  auto fetch = [&](Ops& o, int c) {
    c = min(c, nc - 1);
    f32x4(&rq)[NL] = o.rq;
    f32x4(&rk)[NL] = o.rk;
    f32x4(&rw)[NM] = o.rw;
    f32x4(&rb)[NM] = o.rb;
    float& rg = o.rg;
    float(&rv)[NV] = o.rv;
    const int t0 = c * PC, Cn = min(PC, T - t0);
    const float* blk = CH + ((size_t)c * H + h) * PC_BLK;
#pragma unroll
    for (int x = 0; x < NL; ++x) {
      const int f = tid + CS_NT * x, tt = min(f / n4, Cn - 1), e = (f - (f / n4) * n4) * 4;
      const float* src = QK + ((size_t)h * T + t0 + tt) * 2 * dk;
      rq[x] = *(const f32x4*)(src + e);
      rk[x] = *(const f32x4*)(src + dk + e);
    }
#pragma unroll
    for (int x = 0; x < NM; ++x) {
      const int f = tid + CS_NT * x;
      rw[x] = *(const f32x4*)(blk + 4 * f);
      rb[x] = *(const f32x4*)(blk + PC * PC + 4 * f);
    }
    rg = blk[2 * PC * PC + min(tid, 2 * PC)];  // gam [0, PC), dlt [PC, 2 PC], gamma_C last
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const int f = tid + CS_NT * x, tt = min(f / RW, Cn - 1), i = min(f - (f / RW) * RW, dv - 1 - r0);
      rv[x] = Y[(size_t)(t0 + tt) * ldy + off_v + i];
    }
  };
  auto stash = [&](const Ops& o, int Cn) {
    const f32x4(&rq)[NL] = o.rq;
    const f32x4(&rk)[NL] = o.rk;
    const f32x4(&rw)[NM] = o.rw;
    const f32x4(&rb)[NM] = o.rb;
    const float rg = o.rg;
    const float(&rv)[NV] = o.rv;
#pragma unroll
    for (int x = 0; x < NL; ++x) {
      const int f = tid + CS_NT * x, tt = f / n4, e = (f - tt * n4) * 4;
      const bool in = tt < Cn;
      if (tt < PC) {
        *(f32x4*)&sq[tt][e] = in ? rq[x] : f32x4{0.f, 0.f, 0.f, 0.f};
        *(f32x4*)&sk[tt][e] = in ? rk[x] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int x = 0; x < NM; ++x) {
      const int f = tid + CS_NT * x, tt = f / (PC / 4), jj = (f - tt * (PC / 4)) * 4;
      *(f32x4*)&sw[tt][jj] = rw[x];
      *(f32x4*)&sbt[tt][jj] = rb[x];
    }
    if (tid < PC) sgam[tid] = rg;
    else if (tid <= 2 * PC) sdlt[tid - PC] = rg;
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const int f = tid + CS_NT * x, tt = f / RW, i = f - tt * RW;
      sv[tt][i] = (tt < Cn && r0 + i < dv) ? rv[x] : 0.f;
    }
  };
  const int nb = wv & 3, tok = 16 * nb + lr;  // this wave's 16-token block, this lane's token
  fetch(oa, 0);
  fetch(ob, 1);
  auto chunk = [&](int c, Ops& o) {
    const int t0 = c * PC, Cn = min(PC, T - t0);
    stash(o, Cn);
    __syncthreads();
    fetch(o, c + 2);
    // Z^T (waves 0-3) or P^T (waves 4-7) for tokens 16 nb ..: lane holds rows 4 lk + r, token tok
    const f32x4 zp = mfma_rows<DKM>(&ss[lr][0], wv < 4 ? &sk[tok][0] : &sq[tok][0], f32x4{0.f, 0.f, 0.f, 0.f});
    if (wv < 4) {
      const float g = sgam[tok];
#pragma unroll
      for (int r = 0; r < 4; ++r) sr[4 * lk + r][tok] = sv[tok][4 * lk + r] - g * zp[r];
    }
    __syncthreads();
    if (wv < 4) {
      const f32x4 u = mfma_rows<PC>(&sr[lr][0], &sw[tok][0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) su[4 * lk + r][tok] = u[r];
    }
    __syncthreads();
    if (wv >= 4) {
      const float g = sgam[tok];
      const f32x4 o = mfma_rows<PC>(&su[lr][0], &sbt[tok][0], f32x4{g * zp[0], g * zp[1], g * zp[2], g * zp[3]});
      if (tok < Cn) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 4 * lk + r;
          if (r0 + row < dv) split_store(o[r], Ohi, Olo, (size_t)(t0 + tok) * ldo + h * dv + r0 + row);
        }
      }
    }
    // state update: key columns 16 eb .. 16 eb + 15 per wave (tokens past the prompt have u = 0)
    for (int eb = wv; eb < DKM / 16; eb += 8) {
      const int e = 16 * eb + lr;
      const float gc = sdlt[PC];
      f32x4 acc[2];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[0][r] = gc * ss[4 * lk + r][e];
      acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < PC / 16; ++m) {
        const int tb = 16 * m + 4 * lk;  // this lane group's four tokens of the block
        const f32x4 uu = *(const f32x4*)&su[lr][tb], dd = *(const f32x4*)&sdlt[tb];
        f32x4& d = acc[m & 1];
        d = mfma4(dd.x * uu.x, sk[tb][e], d);
        d = mfma4(dd.y * uu.y, sk[tb + 1][e], d);
        d = mfma4(dd.z * uu.z, sk[tb + 2][e], d);
        d = mfma4(dd.w * uu.w, sk[tb + 3][e], d);
      }
      const f32x4 st = acc[0] + acc[1];
#pragma unroll
      for (int r = 0; r < 4; ++r) ss[4 * lk + r][e] = st[r];
    }
    __syncthreads();  // ss, sk and the chunk matrices are rewritten by the next chunk
  };
  for (int c = 0; c < nc; c += 2) {
    chunk(c, oa);
    if (c + 1 < nc) chunk(c + 1, ob);
  }
  for (int f = tid; f < RW * n4; f += CS_NT) {
    const int ri = f / n4, e = (f - ri * n4) * 4;
    if (r0 + ri < dv) *(f32x4*)(S + ((size_t)h * dv + r0 + ri) * dk + e) = *(const f32x4*)&ss[ri][e];
  }
}

// ------------------------------------------------------------------------ attention
// q/k/v columns of Y are in RoPE pair order per head (2m, 2m + 1) = (dim m, dim m + hd/2).  Rotate q
// and k at positions p0 + t, write q to Q[t][head][hd] in natural order and k and v to the rows
// kv_pos0 + t of K / V ([head][kv_stride][hd]: the FP32 cache itself, or the chunk's rows when the
// cache is compact).
__global__ void pf_att_rope_kernel(const float* __restrict__ Y, int ldy, int p0, int nq, int nkv, int hd,
                                   const float* __restrict__ rcos, const float* __restrict__ rsin, float* __restrict__ Q,
                                   float* __restrict__ K, float* __restrict__ V, int kv_stride, int kv_pos0) {
  const int t = blockIdx.x;
  const int half = hd / 2, pos = p0 + t, kp = kv_pos0 + t;
  const float* y = Y + (size_t)t * ldy;
  const int npairs = (nq + 2 * nkv) * half;
  for (int P = threadIdx.x; P < npairs; P += blockDim.x) {
    const float x1 = y[2 * P], x2 = y[2 * P + 1];
    const int hh = P / half, m = P - hh * half;
    if (hh < nq + nkv) {
      const float c = rcos[(size_t)pos * half + m], sv = rsin[(size_t)pos * half + m];
      const float y1 = x1 * c - x2 * sv, y2 = x2 * c + x1 * sv;
      if (hh < nq) {
        float* qo = Q + ((size_t)t * nq + hh) * hd;
        qo[m] = y1;
        qo[m + half] = y2;
      } else {
        float* ko = K + ((size_t)(hh - nq) * kv_stride + kp) * hd;
        ko[m] = y1;
        ko[m + half] = y2;
      }
    } else {
      float* vo = V + ((size_t)(hh - nq - nkv) * kv_stride + kp) * hd;
      vo[m] = x1;
      vo[m + half] = x2;
    }
  }
}

// A compact KV cache's rows at positions p0 .. p0 + T - 1 from the chunk's FP32 rows [nkv][T][hd]:
// binary16 (nearest), or int8 codes with one scale per 32 values (s = max|x| / 127, code =
// rint(x / s)), exactly as the decode kernels form them.  One workgroup per (position, KV head); a
// block of 32 values is 32 consecutive lanes of one wave.
__global__ void __launch_bounds__(256) pf_kv_pack_kernel(const float* __restrict__ Kf, const float* __restrict__ Vf,
                                                         int T, int hd, int kvt, void* __restrict__ Kc,
                                                         void* __restrict__ Vc, float* __restrict__ Ks,
                                                         float* __restrict__ Vs, int max_ctx, int p0) {
  const int t = blockIdx.x, g = blockIdx.y;
  const size_t src = ((size_t)g * T + t) * hd, dst = ((size_t)g * max_ctx + p0 + t) * hd;
  for (int e0 = 0; e0 < 2 * hd; e0 += blockDim.x) {
    const int e = e0 + (int)threadIdx.x;  // every lane of a block of 32 takes part in its reduction
    const bool in = e < 2 * hd;
    const int v = e >= hd ? 1 : 0, d = e - v * hd;
    const float x = in ? (v ? Vf : Kf)[src + d] : 0.f;
    if (kvt == MK_KV_F16) {
      if (in) ((_Float16*)(v ? Vc : Kc))[dst + d] = (_Float16)x;
    } else {
      float m = fabsf(x);
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
      const float sc = m / 127.0f;
      if (in) {
        ((signed char*)(v ? Vc : Kc))[dst + d] = (signed char)(int)(sc > 0.f ? rintf(x / sc) : 0.f);
        if ((d & (MK_KV_Q8_BLOCK - 1)) == 0) (v ? Vs : Ks)[dst / MK_KV_Q8_BLOCK + d / MK_KV_Q8_BLOCK] = sc;
      }
    }
  }
}

// Causal attention for the chunk's queries over cache positions 0 .. p0 + t.  A workgroup (4 waves)
// takes one KV head g and QB = 16 / gs consecutive queries of every query head of its group: 16
// (head, query) rows.  Keys go through LDS in blocks of 32 positions (LDS-DMA, double-buffered, the
// next block in flight while the current one is used).  Per block: scores with one thread per
// (row, key pair), the block's max and sum per row over a 16-lane DPP row, then P.V with one thread
// per (row, 8 dims); the running max / sum / output are rescaled per block (online softmax).
constexpr int KB = 32;
constexpr int HDM = 256;  // largest head size
template <int DPL>  // head dims per lane in P.V (a power of two >= hd / 16)
__global__ void __launch_bounds__(256) pf_attention_kernel(const float* __restrict__ Q, const float* __restrict__ Kc,
                                                           const float* __restrict__ Vc, int T, int p0, int nq, int nkv,
                                                           int hd, int max_ctx, uint16_t* __restrict__ Ohi,
                                                           uint16_t* __restrict__ Olo, int ldo) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int lpp = hd >> 2, pps = 64 / lpp, nsl = (KB + pps - 1) / pps;  // lanes / keys per 1 KB slot
  float* skv = sm;                                  // [2 buffers][2 (K, V)][nsl slots][256 floats]
  float* sq = sm + 2 * 2 * nsl * 256;               // [16][hd]
  float* sp = sq + 16 * HDM;                        // [16][KB]
  float* sc = sp + 16 * KB;                         // [16] rescale of the running output
  const int gs = nq / nkv, QB = 16 / gs;
  const int nqb = (T + QB - 1) / QB;
  const int g = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const int tid = threadIdx.x, l = tid & 63, wv = tid >> 6;
  const int jend = p0 + min(T, (qb + 1) * QB);  // keys this workgroup needs: [0, jend)
  const int nblk = (jend + KB - 1) / KB;
  const float scale = 1.0f / sqrtf((float)hd);
  auto issue = [&](int blk) {
    float* base = skv + (size_t)(blk & 1) * 2 * nsl * 256;
    for (int q = wv; q < 2 * nsl; q += 4) {
      const int isv = q >= nsl, sl = q - isv * nsl;
      const int kk = sl * pps + l / lpp, j = blk * KB + kk;
      const float* src = (isv ? Vc : Kc) + ((size_t)g * max_ctx + min(j, jend - 1)) * hd + (l % lpp) * 4;
      if (l < pps * lpp && kk < KB)
        __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)(base + q * 256),
                                         16, 0, 0);
    }
  };
  const int ncopy = wv < 2 * nsl ? (2 * nsl - wv + 3) / 4 : 0;  // copies this wave issues per block
  issue(0);
  // queries of the 16 rows, pre-scaled
  for (int x = tid; x < 16 * hd; x += 256) {
    const int row = x / hd, e = x % hd;
    const int hq = g * gs + row / QB, tq = qb * QB + row % QB;
    sq[row * HDM + e] = tq < T ? Q[((size_t)tq * nq + hq) * hd + e] * scale : 0.f;
  }
  // P.V mapping: thread -> (row, 8 dims); score mapping: thread -> (row, keys 2c, 2c + 1)
  const int prow = tid >> 4, pc = tid & 15;
  const int tq_p = qb * QB + prow % QB;
  const int jmax = p0 + min(tq_p, T - 1);
  float acc[DPL];
#pragma unroll
  for (int x = 0; x < DPL; ++x) acc[x] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  for (int blk = 0; blk < nblk; ++blk) {
    if (blk + 1 < nblk) {
      issue(blk + 1);
      wait_vm_n(ncopy);  // this block's copies are done once only the next block's remain
    } else {
      wait_vm<0>();
    }
    lds_bar();
    const float* kb = skv + (size_t)(blk & 1) * 2 * nsl * 256;
    const float* vb = kb + nsl * 256;
    const int j0 = blk * KB;
    // scores of keys 2pc and 2pc + 1 for row prow
    float s2[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kk = 2 * pc + u, j = j0 + kk;
      float a = -INFINITY;
      if (j <= jmax) {
        const float* kr = kb + (kk / pps) * 256 + (kk % pps) * hd;
        const float* qr = sq + prow * HDM;
        const int n4 = hd >> 2, st0 = kk % n4;  // staggered start: the keys of a row hit different banks
        float d = 0.f;
        for (int d0 = 0; d0 < n4; d0 += 8) {
          f32x4 kv[8], qv[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            int e = d0 + x + st0;
            e = (e >= n4 ? e - n4 : e) * 4;
            kv[x] = f32x4{0.f, 0.f, 0.f, 0.f};
            qv[x] = kv[x];
            if (d0 + x < n4) {
              kv[x] = *(const f32x4*)(kr + e);
              qv[x] = *(const f32x4*)(qr + e);
            }
          }
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            d = fmaf(kv[x].x, qv[x].x, d);
            d = fmaf(kv[x].y, qv[x].y, d);
            d = fmaf(kv[x].z, qv[x].z, d);
            d = fmaf(kv[x].w, qv[x].w, d);
          }
        }
        a = d;
      }
      s2[u] = a;
    }
    // block max and the running rescale, per 16-lane row (one row = one query row)
    float bm = fmaxf(s2[0], s2[1]);
    bm = fmaxf(bm, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(bm), __float_as_int(bm), 0xB1, 0xF, 0xF, false)));
    bm = fmaxf(bm, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(bm), __float_as_int(bm), 0x4E, 0xF, 0xF, false)));
    bm = fmaxf(bm, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(bm), __float_as_int(bm), 0x141, 0xF, 0xF, false)));
    bm = fmaxf(bm, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(bm), __float_as_int(bm), 0x140, 0xF, 0xF, false)));
    const float mn = fmaxf(m, bm);                 // finite: key 0 of block 0 is always visible
    const float corr = expf(m - mn);
    const float e0 = expf(s2[0] - mn), e1 = expf(s2[1] - mn);
    lsum = fmaf(lsum, corr, row_sum16(e0 + e1));
    m = mn;
    sp[prow * KB + 2 * pc] = e0;
    sp[prow * KB + 2 * pc + 1] = e1;
    lds_bar();
    // P.V for row prow, dims pc * DPL .. + DPL (four keys' values loaded before they are used)
    const int nvalid = min(KB, jend - j0);
    const bool live = pc * DPL < hd;
#pragma unroll
    for (int x = 0; x < DPL; ++x) acc[x] *= corr;
    for (int k0 = 0; k0 < nvalid; k0 += 4) {
      float pk[4], vv[4][DPL];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = k0 + u;
        pk[u] = kk < nvalid ? sp[prow * KB + kk] : 0.f;
        const float* vr = vb + (kk / pps) * 256 + (kk % pps) * hd + pc * DPL;
#pragma unroll
        for (int x = 0; x < DPL; x += (DPL >= 4 ? 4 : 2)) {
          if (DPL >= 4) {
            const f32x4 t4 = (kk < nvalid && live) ? *(const f32x4*)(vr + x) : f32x4{0.f, 0.f, 0.f, 0.f};
            vv[u][x] = t4.x;
            vv[u][x + 1] = t4.y;
            vv[u][x + 2] = t4.z;
            vv[u][x + 3] = t4.w;
          } else {
            const f32x2 t2 = (kk < nvalid && live) ? *(const f32x2*)(vr + x) : f32x2{0.f, 0.f};
            vv[u][x] = t2.x;
            vv[u][x + 1] = t2.y;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int x = 0; x < DPL; ++x) acc[x] = fmaf(pk[u], vv[u][x], acc[x]);
    }
    lds_bar();  // this block's buffer is refilled next iteration, sp rewritten
  }
  const int hq = g * gs + prow / QB;
  if (tq_p < T) {
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int x = 0; x < DPL; ++x) {
      const int e = pc * DPL + x;
      if (e < hd) split_store(acc[x] * inv, Ohi, Olo, (size_t)tq_p * ldo + hq * hd + e);
    }
  }
}

// ------------------------------------------------------------------------ attention on MFMA
// Causal attention for the chunk's queries over cache positions 0 .. p0 + t on
// v_mfma_f32_32x32x16_bf16, every operand split into BF16 hi + lo and each product formed as
// hi.hi + hi.lo + lo.hi (the lo.lo term is below 2^-16 relative).  A workgroup (4 waves) takes one
// KV head g, 32 consecutive queries and up to 4 query heads of the group, one per wave.  Key blocks
// of 32 positions go through LDS as BF16 hi/lo, keys as [key][dim] and values transposed as
// [dim][key]; the next block's loads are in flight while the current one is used.  Per block and
// wave:
//   S^T = K Q^T (32 keys x 32 queries): a lane holds 16 keys of one query, so the query's max and
//   sum take its 16 registers and the partner lane l ^ 32;
//   online softmax: m' = max(m, max_j s), P = exp(S - m'), l' = l e^(m - m') + sum P, O *= e^(m - m');
//   O += P V (32 queries x HD in HD / 32 accumulator tiles), P through LDS as BF16 hi/lo.
__device__ __forceinline__ void split8(const float (&v)[8], bf16x8& h, bf16x8& lo) {
  u32x4 hw, lw;
  uint16_t hb[8], lb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hb[i] = f2bf(v[i]);
    lb[i] = f2bf(v[i] - bf16f(hb[i]));
  }
  hw = u32x4{hb[0] | ((u32)hb[1] << 16), hb[2] | ((u32)hb[3] << 16), hb[4] | ((u32)hb[5] << 16), hb[6] | ((u32)hb[7] << 16)};
  lw = u32x4{lb[0] | ((u32)lb[1] << 16), lb[2] | ((u32)lb[3] << 16), lb[4] | ((u32)lb[5] << 16), lb[6] | ((u32)lb[7] << 16)};
  h = __builtin_bit_cast(bf16x8, hw);
  lo = __builtin_bit_cast(bf16x8, lw);
}

template <int HD, int KVT>
__global__ void __launch_bounds__(256) pf_attn_mfma_kernel(const float* __restrict__ Q, const void* __restrict__ Kc,
                                                           const void* __restrict__ Vc, const float* __restrict__ Ks,
                                                           const float* __restrict__ Vs, int T, int p0, int nq, int nkv,
                                                           int max_ctx, uint16_t* __restrict__ Ohi,
                                                           uint16_t* __restrict__ Olo, int ldo, int nsplit,
                                                           float* __restrict__ part) {
  constexpr int KS = HD / 16;         // k-steps of S^T
  constexpr int DT = HD / 32;         // accumulator tiles of O
  constexpr int LPT = 32 * HD / 256;  // floats of K (and of V) per thread and block
  static_assert(LPT % 4 == 0, "whole 16-byte loads");
  extern __shared__ __attribute__((aligned(16))) float sm[];
  uint16_t* Kh = (uint16_t*)sm;     // [32][HD]
  uint16_t* Kl = Kh + 32 * HD;
  uint16_t* Vh = Kl + 32 * HD;      // [HD][32]
  uint16_t* Vl = Vh + HD * 32;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  char* wb = (char*)(Vl + HD * 32) + wv * (4 * 32 * 32 + 2 * 32 * 4);
  uint16_t* Ph = (uint16_t*)wb;     // [32 queries][32 keys]
  uint16_t* Pl = Ph + 32 * 32;
  float* cr = (float*)(Pl + 32 * 32);  // [32] rescale of the running output
  float* lsm = cr + 32;                // [32] final sums
  const int gs = nq / nkv, nquad = (gs + 3) / 4, ntile = (T + 31) / 32;
  int b = blockIdx.x;
  const int split = b % nsplit;
  b /= nsplit;
  const int tile = b % ntile;
  b /= ntile;
  const int quad = b % nquad, g = b / nquad;
  const int il = quad * 4 + wv;
  const bool live = il < gs;
  const int hq = g * gs + min(il, gs - 1);
  const int t0 = tile * 32;
  const int tq = t0 + (l & 31);                   // this lane's query
  const int jend = p0 + min(T, t0 + 32);          // keys [0, jend)
  const int Pq = tq < T ? p0 + tq : jend - 1;     // its last visible key (rows past T see all)
  const int nall = (jend + 31) / 32;
  // key blocks of this split: [kb0, kb0 + nblk)
  const int kper = (nall + nsplit - 1) / nsplit;
  const int kb0 = min(nall, split * kper), nblk = min(nall, kb0 + kper) - kb0;
  const float scale = 1.0f / sqrtf((float)HD);
  const int hi32 = l >> 5;
  // Q fragments: B operand of S^T (column = query, k = dims)
  bf16x8 qh[KS], ql[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float v[8];
    const float* qp = Q + ((size_t)min(tq, T - 1) * nq + hq) * HD + ks * 16 + hi32 * 8;
    const f32x4 a = *(const f32x4*)qp, c = *(const f32x4*)(qp + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
    split8(v, qh[ks], ql[ks]);
  }
  // K / V block loads: thread -> LPT / 4 pieces of K and of V
  f32x4 kr[LPT / 4], vr[LPT / 4];
  auto load_blk = [&](int blk) {
#pragma unroll
    for (int i = 0; i < LPT / 4; ++i) {
      const int e = (i * 256 + tid) * 4;
      const int key = e / HD, d = e - key * HD;
      const int j = min(blk * 32 + key, jend - 1);
      const size_t gi = ((size_t)g * max_ctx + j) * HD + d;
      if (KVT == MK_KV_F32) {
        kr[i] = *(const f32x4*)((const float*)Kc + gi);
        vr[i] = *(const f32x4*)((const float*)Vc + gi);
      } else if (KVT == MK_KV_F16) {
        const _Float16* kh = (const _Float16*)Kc + gi;
        const _Float16* vh = (const _Float16*)Vc + gi;
        kr[i] = f32x4{(float)kh[0], (float)kh[1], (float)kh[2], (float)kh[3]};
        vr[i] = f32x4{(float)vh[0], (float)vh[1], (float)vh[2], (float)vh[3]};
      } else {
        const u32 kq = *(const u32*)((const signed char*)Kc + gi), vq = *(const u32*)((const signed char*)Vc + gi);
        const float ks = Ks[gi / MK_KV_Q8_BLOCK], vs = Vs[gi / MK_KV_Q8_BLOCK];
        kr[i] = f32x4{(float)(int)(signed char)kq * ks, (float)(int)(signed char)(kq >> 8) * ks,
                      (float)(int)(signed char)(kq >> 16) * ks, (float)(int)(signed char)(kq >> 24) * ks};
        vr[i] = f32x4{(float)(int)(signed char)vq * vs, (float)(int)(signed char)(vq >> 8) * vs,
                      (float)(int)(signed char)(vq >> 16) * vs, (float)(int)(signed char)(vq >> 24) * vs};
      }
    }
  };
  auto store_blk = [&]() {
#pragma unroll
    for (int i = 0; i < LPT / 4; ++i) {
      const int e = (i * 256 + tid) * 4;
      const int key = e / HD, d = e - key * HD;
      const float kv[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
      const float vv[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
      uint16_t kh[4], kl[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        kh[x] = f2bf(kv[x]);
        kl[x] = f2bf(kv[x] - bf16f(kh[x]));
        const uint16_t h = f2bf(vv[x]);
        Vh[(d + x) * 32 + key] = h;
        Vl[(d + x) * 32 + key] = f2bf(vv[x] - bf16f(h));
      }
      *(u32x2*)(Kh + key * HD + d) = u32x2{kh[0] | ((u32)kh[1] << 16), kh[2] | ((u32)kh[3] << 16)};
      *(u32x2*)(Kl + key * HD + d) = u32x2{kl[0] | ((u32)kl[1] << 16), kl[2] | ((u32)kl[3] << 16)};
    }
  };
  f32x16 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] = f32x16{};
  float m = -INFINITY, lsum = 0.f;
  if (nblk > 0) {
    load_blk(kb0);
    store_blk();
  }
  lds_bar();
  for (int kb = kb0; kb < kb0 + nblk; ++kb) {
    if (kb + 1 < kb0 + nblk) load_blk(kb + 1);  // in flight during this block
    if (live) {
      f32x16 st = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int kd = ks * 16 + hi32 * 8;
        const bf16x8 kh = *(const bf16x8*)(Kh + (l & 31) * HD + kd);
        const bf16x8 kl = *(const bf16x8*)(Kl + (l & 31) * HD + kd);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qh[ks], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, ql[ks], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl, qh[ks], st, 0, 0, 0);
      }
      // register r: key kb*32 + 8 (r / 4) + 4 (l / 32) + r % 4 of query tq
      float mloc = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = kb * 32 + 8 * (r >> 2) + 4 * hi32 + (r & 3);
        st[r] = j <= Pq ? st[r] * scale : -INFINITY;
        mloc = fmaxf(mloc, st[r]);
      }
      const float mb = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float mn = fmaxf(m, mb);  // finite: key 0 is visible to every query
      const float corr = expf(m - mn);
      float ls = 0.f;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        uint16_t h[4], lo[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float pv = expf(st[r4 * 4 + x] - mn);  // 0 for masked keys
          ls += pv;
          h[x] = f2bf(pv);
          lo[x] = f2bf(pv - bf16f(h[x]));
        }
        const int o = (l & 31) * 32 + 8 * r4 + 4 * hi32;
        *(u32x2*)(Ph + o) = u32x2{h[0] | ((u32)h[1] << 16), h[2] | ((u32)h[3] << 16)};
        *(u32x2*)(Pl + o) = u32x2{lo[0] | ((u32)lo[1] << 16), lo[2] | ((u32)lo[3] << 16)};
      }
      lsum = fmaf(lsum, corr, ls + __shfl_xor(ls, 32, 64));
      m = mn;
      if (l < 32) cr[l] = corr;
      __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's P and rescale writes are done
      asm volatile("" ::: "memory");
      // O rows (queries) of register r: 8 (r / 4) + 4 (l / 32) + r % 4
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 c4 = *(const f32x4*)(cr + 8 * r4 + 4 * hi32);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          O[dt][r4 * 4 + 0] *= c4.x;
          O[dt][r4 * 4 + 1] *= c4.y;
          O[dt][r4 * 4 + 2] *= c4.z;
          O[dt][r4 * 4 + 3] *= c4.w;
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int kq = s2 * 16 + hi32 * 8;
        const bf16x8 ph = *(const bf16x8*)(Ph + (l & 31) * 32 + kq);
        const bf16x8 pl = *(const bf16x8*)(Pl + (l & 31) * 32 + kq);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 vh = *(const bf16x8*)(Vh + (dt * 32 + (l & 31)) * 32 + kq);
          const bf16x8 vl = *(const bf16x8*)(Vl + (dt * 32 + (l & 31)) * 32 + kq);
          O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph, vh, O[dt], 0, 0, 0);
          O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph, vl, O[dt], 0, 0, 0);
          O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pl, vh, O[dt], 0, 0, 0);
        }
      }
    }
    lds_bar();  // every wave is done with this block's K / V
    if (kb + 1 < kb0 + nblk) {
      store_blk();
      lds_bar();
    }
  }
  if (!live) return;
  if (nsplit > 1) {
    // unnormalised partial of this split: per query row (max, sum, O[HD]); a split without keys
    // leaves (-inf, 0, 0)
    float* pp = part + ((size_t)(tile * nq + hq) * nsplit + split) * 32 * (HD + 2);
    if (l < 32) {
      pp[l * (HD + 2)] = m;
      pp[l * (HD + 2) + 1] = lsum;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * hi32 + (r & 3);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) pp[row * (HD + 2) + 2 + dt * 32 + (l & 31)] = O[dt][r];
    }
    return;
  }
  if (l < 32) lsm[l] = lsum;
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const f32x4 l4 = *(const f32x4*)(lsm + 8 * r4 + 4 * hi32);
    const float inv[4] = {1.0f / l4.x, 1.0f / l4.y, 1.0f / l4.z, 1.0f / l4.w};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int t = t0 + 8 * r4 + 4 * hi32 + x;
      if (t < T) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          split_store(O[dt][r4 * 4 + x] * inv[x], Ohi, Olo, (size_t)t * ldo + hq * HD + dt * 32 + (l & 31));
      }
    }
  }
}

// Key-split partials -> output: per (query, head), splits merged in order:
// M = max_s m_s, O = sum_s e^(m_s - M) O_s / sum_s e^(m_s - M) l_s; written as BF16 hi/lo.
__global__ void __launch_bounds__(256) pf_attn_merge_kernel(const float* __restrict__ part, int T, int nq, int hd,
                                                            int nsplit, uint16_t* __restrict__ Ohi,
                                                            uint16_t* __restrict__ Olo, int ldo) {
  const int t = blockIdx.x, hq = blockIdx.y;
  if (t >= T) return;
  const int tile = t >> 5, row = t & 31;
  const float* base = part + ((size_t)(tile * nq + hq) * nsplit) * 32 * (hd + 2) + (size_t)row * (hd + 2);
  const size_t sstride = (size_t)32 * (hd + 2);
  float M = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, base[sp * sstride]);
  float den = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) den = fmaf(expf(base[sp * sstride] - M), base[sp * sstride + 1], den);
  const float inv = 1.0f / den;
  for (int d = threadIdx.x; d < hd; d += 256) {
    float num = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) num = fmaf(expf(base[sp * sstride] - M), base[sp * sstride + 2 + d], num);
    split_store(num * inv, Ohi, Olo, (size_t)t * ldo + hq * hd + d);
  }
}

// ------------------------------------------------------------------------ LM head on one row
// x -> rmsnorm(x) * g -> logits = E . xn over rows [w * rpw, ...); per-workgroup (max, index) with
// the lowest index among equal maxima
__global__ void __launch_bounds__(256) pf_lmhead_kernel(const float* __restrict__ x, int D,
                                                        const uint16_t* __restrict__ g, float eps,
                                                        const uint16_t* __restrict__ E, int vocab,
                                                        float* __restrict__ logits, float* __restrict__ part) {
  extern __shared__ float xs[];
  __shared__ float red[8];
  __shared__ int redi[4];
  float s = 0.f;
  for (int i = threadIdx.x; i < D; i += 256) s = fmaf(x[i], x[i], s);
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  s = red[0] + red[1] + red[2] + red[3];
  const float r = 1.0f / sqrtf(s / (float)D + eps);
  for (int i = threadIdx.x; i < D; i += 256) xs[i] = x[i] * r * bf16f(g[i]);
  __syncthreads();
  const int rpw = (vocab + gridDim.x - 1) / gridDim.x;
  const int v0 = blockIdx.x * rpw, v1 = min(vocab, v0 + rpw);
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  // each wave takes 4 rows at a time: their loads are in flight together and their four wave
  // reductions overlap; rows are visited in increasing order within a wave
  constexpr int RW = 4;
  for (int vb = v0 + wv * RW; vb < v1; vb += 4 * RW) {
    float a[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) a[i] = 0.f;
    for (int k = l * 8; k < D; k += 512) {
      u32x4 wq[RW];
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const int v = min(vb + i, v1 - 1);
        wq[i] = *(const u32x4*)(E + (size_t)v * D + k);
      }
      float xk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xk[j] = xs[k + j];
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        a[i] = fmaf(__uint_as_float(wq[i].x << 16), xk[0], a[i]);
        a[i] = fmaf(__uint_as_float(wq[i].x & 0xffff0000u), xk[1], a[i]);
        a[i] = fmaf(__uint_as_float(wq[i].y << 16), xk[2], a[i]);
        a[i] = fmaf(__uint_as_float(wq[i].y & 0xffff0000u), xk[3], a[i]);
        a[i] = fmaf(__uint_as_float(wq[i].z << 16), xk[4], a[i]);
        a[i] = fmaf(__uint_as_float(wq[i].z & 0xffff0000u), xk[5], a[i]);
        a[i] = fmaf(__uint_as_float(wq[i].w << 16), xk[6], a[i]);
        a[i] = fmaf(__uint_as_float(wq[i].w & 0xffff0000u), xk[7], a[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < RW; ++i) a[i] = wave_sum(a[i]);
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int v = vb + i;
      if (v < v1) {
        if (logits && l == 0) logits[v] = a[i];
        if (a[i] > best || (a[i] == best && v < bidx)) {
          best = a[i];
          bidx = v;
        }
      }
    }
  }
  __syncthreads();
  if (l == 0) {
    red[4 + wv] = best;
    redi[wv] = bidx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 0; i < 4; ++i)
      if (red[4 + i] > best || (red[4 + i] == best && redi[i] < bidx)) {
        best = red[4 + i];
        bidx = redi[i];
      }
    part[2 * blockIdx.x] = best;
    part[2 * blockIdx.x + 1] = __int_as_float(bidx);
  }
}

__global__ void pf_finish_kernel(const float* __restrict__ part, int n, int32_t* __restrict__ next, MkCtl* ctl,
                                 int32_t pos) {
  // one wave: lanes over the partial winners, then a shuffle tree (largest value, lowest index)
  const int l = threadIdx.x;
  float b = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = l; i < n; i += 64) {
    const float v = part[2 * i];
    const int vi = __float_as_int(part[2 * i + 1]);
    if (v > b || (v == b && vi < bi)) {
      b = v;
      bi = vi;
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
  if (l == 0) {
    next[0] = bi;
    ctl->pos = pos;
  }
}

}  // namespace

// ------------------------------------------------------------------------ launchers
#define MK_LAUNCH_OK() (hipGetLastError() == hipSuccess ? 0 : -1)

extern "C" int mk_pf_embed(const int32_t* tok, int T, const uint16_t* embed, int D, int vocab, float* X, MkCtl* ctl,
                           void* stream) {
  hipLaunchKernelGGL(pf_embed_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, tok, T, embed, D, vocab, X, ctl);
  return MK_LAUNCH_OK();
}

extern "C" int mk_pf_rms_split(const float* X, int T, int D, const uint16_t* g, float eps, uint16_t* Ahi,
                               uint16_t* Alo, int lda, void* stream) {
  hipLaunchKernelGGL(pf_rms_split_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, X, D, g, eps, Ahi, Alo, lda);
  return MK_LAUNCH_OK();
}

template <int BM, int BN>
static int launch_gemm(int epi, const uint16_t* Ahi, const uint16_t* Alo, int lda, int M, int K, const uint16_t* W, int N,
                       float* C, int ldc, uint16_t* Hhi, uint16_t* Hlo, int ldh, int ksplit, hipStream_t s) {
  const int items = ((M + BM - 1) / BM) * ((N + BN - 1) / BN) * ksplit;
  const int grid = ((items + 7) / 8) * 8;
  const size_t lds = (size_t)gemm_stages<BM>() * (2 * BM + BN) * BK * 2;
  if (epi == 0)
    hipLaunchKernelGGL((pf_gemm_kernel<BM, BN, 0>), dim3(grid), dim3(gemm_threads<BM, BN>()), lds, s, Ahi, Alo, lda, M, K, W, N, C, ldc,
                       Hhi, Hlo, ldh, ksplit);
  else if (epi == 1)
    hipLaunchKernelGGL((pf_gemm_kernel<BM, BN, 1>), dim3(grid), dim3(gemm_threads<BM, BN>()), lds, s, Ahi, Alo, lda, M, K, W, N, C, ldc,
                       Hhi, Hlo, ldh, ksplit);
  else if (epi == 2)
    hipLaunchKernelGGL((pf_gemm_kernel<BM, BN, 2>), dim3(grid), dim3(gemm_threads<BM, BN>()), lds, s, Ahi, Alo, lda, M, K, W, N, C, ldc,
                       Hhi, Hlo, ldh, ksplit);
  else
    hipLaunchKernelGGL((pf_gemm_kernel<BM, BN, 3>), dim3(grid), dim3(gemm_threads<BM, BN>()), lds, s, Ahi, Alo, lda, M, K, W, N, C, ldc,
                       Hhi, Hlo, ldh, ksplit);
  return MK_LAUNCH_OK();
}

// number of K ranges for a split-K residual GEMM: enough workgroups for the chip, at least four
// BK-column K steps per range, and the partials within p_floats
static int splitk_parts(int M, int K, int N, int big, size_t p_floats) {
  const int nk = (K + BK - 1) / BK;
  int ks = std::min(std::max(1, 256 / big), std::max(1, nk / 4));
  while (ks > 1 && (size_t)ks * M * N > p_floats) --ks;
  return ks;
}

extern "C" int mk_pf_gemm(int epi, const uint16_t* Ahi, const uint16_t* Alo, int lda, int M, int K, const uint16_t* W,
                          int N, float* C, int ldc, uint16_t* Hhi, uint16_t* Hlo, int ldh, float* P, size_t p_floats,
                          void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int big = ((M + 127) / 128) * ((N + 127) / 128);
  if (big >= 200) {
    // whole rounds of 256 workgroups times the tile area: a ragged last row block (M = 520 is four
    // 128-row blocks and 8 rows) can cost a second round of 128 x 128 tiles, where 64 x 128 tiles
    // fill two rounds of half the work
    const int half = ((M + 63) / 64) * ((N + 127) / 128);
    if ((half + 255) / 256 * 64 < (big + 255) / 256 * 128)
      return launch_gemm<64, 128>(epi, Ahi, Alo, lda, M, K, W, N, C, ldc, Hhi, Hlo, ldh, 1, s);
    return launch_gemm<128, 128>(epi, Ahi, Alo, lda, M, K, W, N, C, ldc, Hhi, Hlo, ldh, 1, s);
  }
  // too few large tiles to fill the chip: a residual update splits K over workgroups (partials in P,
  // added to C in split order); other epilogues use small tiles
  if (epi == 1 && P && N % 4 == 0) {
    const int ks = splitk_parts(M, K, N, big, p_floats);
    if (ks > 1) {
      launch_gemm<128, 128>(3, Ahi, Alo, lda, M, K, W, N, P, N, Hhi, Hlo, ldh, ks, s);
      hipLaunchKernelGGL(pf_splitk_add_kernel, dim3(M), dim3(256), 0, s, P, ks, M, N, C, ldc, nullptr, 0.f, nullptr,
                         nullptr, 0);
      return MK_LAUNCH_OK();
    }
  }
  return launch_gemm<64, 64>(epi, Ahi, Alo, lda, M, K, W, N, C, ldc, Hhi, Hlo, ldh, 1, s);
}

extern "C" int mk_pf_gemm_res(const uint16_t* Ahi, const uint16_t* Alo, int lda, int M, int K, const uint16_t* W,
                              int N, float* C, int ldc, float* P, size_t p_floats, const uint16_t* g, float eps,
                              uint16_t* Nhi, uint16_t* Nlo, int ldn, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int big = ((M + 127) / 128) * ((N + 127) / 128);
  const int ks = (big < 200 && P && N % 4 == 0) ? splitk_parts(M, K, N, big, p_floats) : 1;
  if (ks > 1) {
    launch_gemm<128, 128>(3, Ahi, Alo, lda, M, K, W, N, P, N, nullptr, nullptr, 0, ks, s);
    hipLaunchKernelGGL(pf_splitk_add_kernel, dim3(M), dim3(256), 0, s, P, ks, M, N, C, ldc, g, eps, Nhi, Nlo, ldn);
    return MK_LAUNCH_OK();
  }
  int rc = mk_pf_gemm(1, Ahi, Alo, lda, M, K, W, N, C, ldc, nullptr, nullptr, 0, nullptr, 0, stream);
  if (g) rc |= mk_pf_rms_split(C, M, N, g, eps, Nhi, Nlo, ldn, stream);
  return rc;
}

extern "C" int mk_pf_dn_scan(float* S, float* QK, float* AB, const float* Y, int ldy, int T, int H, int dk, int dv,
                             float l2eps, uint16_t* Ohi, uint16_t* Olo, int ldo, float* CH, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (dk <= 128) {
    // chunked form: all chunks' W, Bt and decays in parallel, then the state pass
    const int nc = (T + PC - 1) / PC;
    const dim3 g1(nc * H), g2(H * ((dv + CM_RW - 1) / CM_RW));
    if (dk <= 64) {
      hipLaunchKernelGGL(pf_dn_cprep_kernel<64>, g1, dim3(256), 0, s, Y, ldy, T, H, dk, dv, l2eps, QK, CH);
      hipLaunchKernelGGL(pf_dn_cscan_mfma_kernel<64>, g2, dim3(CS_NT), 0, s, S, QK, CH, Y, ldy, T, H, dk, dv, Ohi, Olo,
                         ldo);
    } else {
      hipLaunchKernelGGL(pf_dn_cprep_kernel<128>, g1, dim3(256), 0, s, Y, ldy, T, H, dk, dv, l2eps, QK, CH);
      hipLaunchKernelGGL(pf_dn_cscan_mfma_kernel<128>, g2, dim3(CS_NT), 0, s, S, QK, CH, Y, ldy, T, H, dk, dv, Ohi, Olo,
                         ldo);
    }
    return MK_LAUNCH_OK();
  }
  // wider keys: normalised q, k and the gates per token, then the token-by-token row-parallel
  // recurrence
  hipLaunchKernelGGL(pf_dn_prep_kernel, dim3(T * H), dim3(64), 0, s, Y, ldy, H, dk, dv, l2eps, QK, AB);
  const dim3 grid(H * ((dv + 7) / 8));
  hipLaunchKernelGGL(pf_dn_scan_kernel<8>, grid, dim3(256), 0, s, S, QK, AB, Y, ldy, T, H, dk, dv, Ohi, Olo, ldo);
  return MK_LAUNCH_OK();
}

extern "C" int mk_pf_att_rope(const float* Y, int ldy, int T, int p0, int nq, int nkv, int hd, const float* rcos,
                              const float* rsin, float* Q, float* K, float* V, int kv_stride, int kv_pos0,
                              void* stream) {
  hipLaunchKernelGGL(pf_att_rope_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, Y, ldy, p0, nq, nkv, hd, rcos,
                     rsin, Q, K, V, kv_stride, kv_pos0);
  return MK_LAUNCH_OK();
}

extern "C" int mk_pf_kv_pack(const float* Kf, const float* Vf, int T, int nkv, int hd, int kvt, void* Kc, void* Vc,
                             float* Ks, float* Vs, int max_ctx, int p0, void* stream) {
  hipLaunchKernelGGL(pf_kv_pack_kernel, dim3(T, nkv), dim3(256), 0, (hipStream_t)stream, Kf, Vf, T, hd, kvt, Kc, Vc,
                     Ks, Vs, max_ctx, p0);
  return MK_LAUNCH_OK();
}

extern "C" int mk_pf_attention(const float* Q, const void* Kc, const void* Vc, int kvt, const float* Ks,
                               const float* Vs, int T, int p0, int nq, int nkv, int hd, int max_ctx, uint16_t* Ohi,
                               uint16_t* Olo, int ldo, float* P, size_t p_floats, void* stream) {
  if (hd == 64 || hd == 128) {
    // MFMA path: workgroups = KV heads x groups of 4 query heads x 32-query tiles x key splits.
    // Split the keys when that brings the grid nearer one workgroup per compute unit (256), as far
    // as the partial buffer holds (its partials are merged before anything else uses it).
    const int gs = nq / nkv, ntile = (T + 31) / 32;
    const int base_wg = nkv * ((gs + 3) / 4) * ntile;
    const size_t per_split = (size_t)ntile * nq * 32 * (hd + 2);
    int nsplit = std::max(1, std::min(256 / base_wg, (p0 + T + 31) / 32));
    nsplit = (int)std::min<size_t>((size_t)nsplit, std::max<size_t>(1, p_floats / per_split));
    if (!P) nsplit = 1;
    const dim3 grid(base_wg * nsplit);
    const size_t lds = (size_t)4 * 32 * hd * 2 + 4 * (4 * 32 * 32 + 2 * 32 * 4);
    hipStream_t st = (hipStream_t)stream;
#define MK_PF_ATT(HDV, KVTV)                                                                                        \
  hipLaunchKernelGGL((pf_attn_mfma_kernel<HDV, KVTV>), grid, dim3(256), lds, st, Q, Kc, Vc, Ks, Vs, T, p0, nq, nkv, \
                     max_ctx, Ohi, Olo, ldo, nsplit, P)
    if (hd == 64) {
      if (kvt == MK_KV_F16) MK_PF_ATT(64, MK_KV_F16);
      else if (kvt == MK_KV_Q8) MK_PF_ATT(64, MK_KV_Q8);
      else MK_PF_ATT(64, MK_KV_F32);
    } else {
      if (kvt == MK_KV_F16) MK_PF_ATT(128, MK_KV_F16);
      else if (kvt == MK_KV_Q8) MK_PF_ATT(128, MK_KV_Q8);
      else MK_PF_ATT(128, MK_KV_F32);
    }
#undef MK_PF_ATT
    if (nsplit > 1)
      hipLaunchKernelGGL(pf_attn_merge_kernel, dim3(T, nq), dim3(hd <= 128 ? 128 : 256), 0, st, P, T, nq, hd, nsplit, Ohi,
                         Olo, ldo);
    return MK_LAUNCH_OK();
  }
  if (kvt != MK_KV_F32) return -1;  // compact caches take the matrix-core path or token-by-token decode
  const int gs = nq / nkv, QB = 16 / gs;
  const int lpp = hd / 4, pps = 64 / lpp, nsl = (KB + pps - 1) / pps;
  const size_t lds = ((size_t)2 * 2 * nsl * 256 + 16 * HDM + 16 * KB + 16) * 4;
  const dim3 grid(nkv * ((T + QB - 1) / QB));
  hipStream_t s = (hipStream_t)stream;
  const int dpl = (hd + 15) / 16;
  const float* Kf = (const float*)Kc;
  const float* Vf = (const float*)Vc;
  if (dpl <= 2)
    hipLaunchKernelGGL(pf_attention_kernel<2>, grid, dim3(256), lds, s, Q, Kf, Vf, T, p0, nq, nkv, hd, max_ctx, Ohi, Olo, ldo);
  else if (dpl <= 4)
    hipLaunchKernelGGL(pf_attention_kernel<4>, grid, dim3(256), lds, s, Q, Kf, Vf, T, p0, nq, nkv, hd, max_ctx, Ohi, Olo, ldo);
  else if (dpl <= 8)
    hipLaunchKernelGGL(pf_attention_kernel<8>, grid, dim3(256), lds, s, Q, Kf, Vf, T, p0, nq, nkv, hd, max_ctx, Ohi, Olo, ldo);
  else
    hipLaunchKernelGGL(pf_attention_kernel<16>, grid, dim3(256), lds, s, Q, Kf, Vf, T, p0, nq, nkv, hd, max_ctx, Ohi, Olo,
                       ldo);
  return MK_LAUNCH_OK();
}

extern "C" int mk_pf_lmhead(const float* x, int D, const uint16_t* g, float eps, const uint16_t* E, int vocab,
                            float* logits, float* part, int nwg, void* stream) {
  hipLaunchKernelGGL(pf_lmhead_kernel, dim3(nwg), dim3(256), (size_t)D * 4, (hipStream_t)stream, x, D, g, eps, E, vocab,
                     logits, part);
  return MK_LAUNCH_OK();
}

extern "C" int mk_pf_finish(const float* part, int nwg, int32_t* next, MkCtl* ctl, int32_t pos, void* stream) {
  hipLaunchKernelGGL(pf_finish_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, part, nwg, next, ctl, pos);
  return MK_LAUNCH_OK();
}

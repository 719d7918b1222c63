// Device building blocks of the persistent decode and verify kernels: wave roles, exchange
// records and their gathers, the BF16 hi/lo GEMV, RMSNorm, the DeltaNet state rows, split-K
// attention items and their combine.  Included by mk_decode.hip and mk_verify.hip; everything
// here has internal linkage, so each translation unit keeps its own copy.
#pragma once

#include <hip/hip_runtime.h>
#include "mk_internal.h"
#include <type_traits>

typedef unsigned int u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
// Native vector types for LDS accesses: loads of HIP's float4 / uint2 structs are split and merged
// again late in code generation, which drops what the compiler knows about the accessed LDS object
// and makes it wait for every outstanding LDS-DMA copy before the read.
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// LDS pointers are kept in address space 3 so every access is a ds_* instruction
#if defined(__HIP_DEVICE_COMPILE__)
#define LS __attribute__((address_space(3)))
#else
#define LS
#endif

namespace {


constexpr int NCW = MK_NCW;          // streaming waves 0..NCW-1
constexpr int NCT = MK_NCT;          // streaming threads
constexpr int NPT = MK_NT - MK_NCT;  // polling threads
constexpr int SLOT = 64;             // u32x4 per 1 KB LDS slot
constexpr int USLOTS = 4;            // slots per GEMV unit: 4 rows x 512 BF16 columns
constexpr int A_UNITS = MK_STAGE_A_SLOTS / USLOTS;
constexpr int PB = 8;                // poll loads in flight per lane
constexpr int ATT_C = MK_ATT_CHUNK;

// Compiler-only barrier: memory operations issued before it stay before it.
__device__ __forceinline__ void keep_issued() { asm volatile("" ::: "memory"); }

// Thread index the compiler cannot treat as loop-invariant: per-lane address arithmetic is
// recomputed where it is used instead of being hoisted out of the layer loop and kept live.
__device__ __forceinline__ int tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
__device__ __forceinline__ int lane() { return tid() & 63; }
__device__ __forceinline__ int wave() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }
__device__ __forceinline__ bool streamer() { return wave() < NCW; }

// Values that are the same in every lane, made scalar again after a call boundary (arguments of
// out-of-line functions arrive in vector registers).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ T* uni_ptr(T* p) {
  const unsigned long long v = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v), hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return (T*)(((unsigned long long)hi << 32) | lo);
}

// contiguous balanced split of n items over parts: part i gets [split(n,parts,i), split(n,parts,i+1))
__device__ __forceinline__ int split(int n, int parts, int i) { return (int)(((long long)n * i) / parts); }

// Workgroup barrier ordering LDS only: it waits for this wave's LDS operations but not for its
// global loads, stores or LDS-DMA copies.
__device__ __forceinline__ void wg_bar() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  keep_issued();
  __builtin_amdgcn_s_barrier();
  keep_issued();
}

// vmcnt(N): at most N of this wave's vector memory operations still outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// at most n outstanding (rounded down to a supported count: waiting for more is always correct)
__device__ __forceinline__ void wait_vm_n(int n) {
  n = __builtin_amdgcn_readfirstlane(n);
  if (n >= 63) wait_vm<63>();
  else if (n >= 48) wait_vm<48>();
  else if (n >= 32) wait_vm<32>();
  else if (n >= 24) wait_vm<24>();
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

__device__ __forceinline__ void ll_put(MK_G mk_u64* p, u32 epoch, float v) {
  __hip_atomic_store(p, ((mk_u64)epoch << 32) | (mk_u64)__float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ mk_u64 ld_dev(const MK_G mk_u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float bf_lo(u32 w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(u32 w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((u32)h << 16); }

__device__ __forceinline__ u32x4 ldw(const MK_G uint16_t* p) { return __builtin_nontemporal_load((const MK_G u32x4*)p); }

// Asynchronous global -> LDS copy (gfx950 LDS DMA): lane l's 16 bytes land at dst + 16 l; tracked
// by vmcnt like a load.  Lanes that are switched off copy nothing.
__device__ __forceinline__ void dma16(const MK_G void* src, LS void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// The LDS regions that LDS-DMA fills (the two prefetch stages) live in their own static array; every
// other LDS region lives in the dynamic array and is written only by ds_* stores.  The compiler can
// then prove that reads of the dynamic regions never race a copy and issues them without waiting.
// Reads of the stage regions go through the asm blocks below: left to the compiler, each would wait
// for every outstanding vector-memory operation of the wave, the prefetches for later phases
// included.  That the copies a read needs have landed is ensured by the explicit vmcnt waits before
// the barrier that precedes the read.  Each block waits for its own reads.
__shared__ __attribute__((aligned(1024))) u32x4 g_stage[(MK_STAGE_A_SLOTS + MK_STAGE_B_SLOTS) * SLOT];

__device__ __forceinline__ u32 lds_addr(const LS void* p) { return (u32)(size_t)p; }

// four 16-byte reads at p, p + 1 KB, p + 2 KB, p + 3 KB (one GEMV unit)
__device__ __forceinline__ void stage_unit(const LS u32x4* p, u32x4 (&w)[USLOTS]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\t"
      "ds_read_b128 %3, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3])
      : "v"(lds_addr(p))
      : "memory");
}
// two units
__device__ __forceinline__ void stage_units2(const LS u32x4* p, const LS u32x4* q, u32x4 (&w)[USLOTS],
                                             u32x4 (&v)[USLOTS]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %9\n\t"
      "ds_read_b128 %5, %9 offset:1024\n\t"
      "ds_read_b128 %6, %9 offset:2048\n\t"
      "ds_read_b128 %7, %9 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(lds_addr(p)), "v"(lds_addr(q))
      : "memory");
}
// four floats at independent addresses
__device__ __forceinline__ void stage_f32x4(const LS float* a, const LS float* b, const LS float* c,
                                            const LS float* d, float (&o)[4]) {
  asm volatile(
      "ds_read_b32 %0, %4\n\t"
      "ds_read_b32 %1, %5\n\t"
      "ds_read_b32 %2, %6\n\t"
      "ds_read_b32 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(lds_addr(a)), "v"(lds_addr(b)), "v"(lds_addr(c)), "v"(lds_addr(d))
      : "memory");
}
// eight float4 at independent addresses
__device__ __forceinline__ void stage_f4x8(const LS float* const (&a)[8], f32x4 (&o)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(lds_addr(a[0])), "v"(lds_addr(a[1])), "v"(lds_addr(a[2])), "v"(lds_addr(a[3])), "v"(lds_addr(a[4])),
        "v"(lds_addr(a[5])), "v"(lds_addr(a[6])), "v"(lds_addr(a[7]))
      : "memory");
}

// four float4 at independent addresses
__device__ __forceinline__ void stage_f4x4(const LS float* const (&a)[4], f32x4 (&o)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(lds_addr(a[0])), "v"(lds_addr(a[1])), "v"(lds_addr(a[2])), "v"(lds_addr(a[3]))
      : "memory");
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF,
                                                              false)));
}

// Sum over each 16-lane row (quad swaps, half-row mirror, row mirror); every lane of the row ends
// with the row's total.  Fixed order, so every call site is deterministic.
__device__ __forceinline__ float row_sum16(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xF>(v);  // row_mirror
  return v;
}
__device__ __forceinline__ float row_max16(float v) {
  v = dpp_max<0xB1>(v);
  v = dpp_max<0x4E>(v);
  v = dpp_max<0x141>(v);
  v = dpp_max<0x140>(v);
  return v;
}
// Full-wave sum: row sums, then row broadcasts; the total lands in lane 63 and is broadcast.
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
  v = row_max16(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x142, 0xA, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x143, 0xC, 0xF, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

struct Ctx {
  MK_G MkCtl* ctl;
  u32 epoch;
};

__device__ __forceinline__ void set_err(const Ctx& cx, u32 code) {
  __hip_atomic_store(&cx.ctl->err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool err_seen(const Ctx& cx) {
  return __hip_atomic_load(&cx.ctl->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

struct Lds {
  LS MkLayerDev* desc;  // every layer's descriptor
  LS uint16_t* gain;    // BF16 RMSNorm gains [2 (layer parity)][2][D]
  LS float* rope;       // cos [hd/2], sin [hd/2] at this launch's position
  LS float* x;          // residual [D]
  LS u32* xn;           // normalised residual [D], hi/lo BF16 pairs
  LS float* vec;        // gathered mixer output / FFN hidden, argmax records
  LS float* att;        // gathered DeltaNet / attention inputs, combine staging, GEMV unit partials
  int att_cap;          // floats of the att region available to the combine staging
  LS float* scr;        // small reductions
  LS int* flag;         // set once a wait gave up
  LS u32x4* stA;        // prefetch stage A
  LS u32x4* stB;        // prefetch stage B
  int a_slots;          // 1 KB slots of stage A
};

// Workgroup barrier that also tells every thread whether any thread passed bad == true.  A wait
// that gives up is final for the launch, so the flag is only ever raised.
__device__ __forceinline__ bool wg_bar_or(const Lds& s, bool bad) {
  if (bad) *s.flag = 1;
  wg_bar();
  return *s.flag != 0;
}

struct Tracer {
  LS unsigned long long* lbuf;   // timestamps are kept in LDS while the kernel runs ...
  MK_G unsigned long long* buf;  // ... and copied here at the end (null: tracing off)
  int n;
  // wall-clock stamps of lane 0 of wave 0 (a streaming wave)
  __device__ __forceinline__ void mark() {
    if (buf) {
      if (threadIdx.x == 0 && n < MK_TRACE_EVENTS) lbuf[n] = wall_clock64();
      ++n;
    }
  }
  __device__ __forceinline__ void flush() {
    if (buf) {
      wg_bar();
      for (int i = tid(); i < MK_TRACE_EVENTS; i += MK_NT) buf[i] = i < n ? lbuf[i] : 0ull;
    }
  }
};

// GEMV activations are held as BF16 hi + lo pairs (see the GEMV section).
__device__ __forceinline__ u32 bf16_rne_bits(float f) {
  const u32 u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
// v -> (hi, lo) BF16 bit patterns with v = hi + lo + O(2^-17 |v|)
__device__ __forceinline__ void split_hl(float v, u32& h, u32& l) {
  h = bf16_rne_bits(v);
  l = bf16_rne_bits(v - __uint_as_float(h << 16));
}
// word offsets (u32) of the hi and lo pair holding column c, c even
__device__ __forceinline__ int hl_word(int c) { return (c >> 3) * 8 + ((c & 7) >> 1); }
// columns c, c + 1 (c even) -> hi/lo pair words
__device__ __forceinline__ void put_hl2(LS u32* hl, int c, float v0, float v1) {
  u32 h0, l0, h1, l1;
  split_hl(v0, h0, l0);
  split_hl(v1, h1, l1);
  const int o = hl_word(c);
  hl[o] = h0 | (h1 << 16);
  hl[o + 4] = l0 | (l1 << 16);
}

// ------------------------------------------------------------------------ exchanges (polling waves)
// Poll n records, record f at src(f); use(f, value) once its epoch matches.  Polling threads keep
// PB loads in flight each.  Every thread calls it; streaming threads return at once.
template <typename SrcFn, typename UseFn>
__device__ __forceinline__ bool gather_map(const Ctx& cx, int n, SrcFn src, UseFn use) {
  if (streamer()) return true;
  const u32 e = cx.epoch;
  const int pl = tid() - NCT;
  bool ok = true;
  for (int base = 0; ok && base < n; base += NPT * PB) {
    u32 pending = 0;
#pragma unroll
    for (int k = 0; k < PB; ++k)
      if (base + k * NPT + pl < n) pending |= 1u << k;
    u32 spins = 0;
    while (pending) {
      mk_u64 v[PB];
#pragma unroll
      for (int k = 0; k < PB; ++k)
        if ((pending >> k) & 1u) v[k] = ld_dev(src(base + k * NPT + pl));
#pragma unroll
      for (int k = 0; k < PB; ++k)
        if (((pending >> k) & 1u) && (u32)(v[k] >> 32) == e) {
          use(base + k * NPT + pl, __uint_as_float((u32)v[k]));
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
  // Every poll load has been used (or abandoned) by now; the wait, free here, tells the compiler
  // so.  Loads it cannot match with a use look outstanding to it, and a later reuse of their
  // registers would wait for all vector-memory operations, prefetch copies included.
  wait_vm<0>();
  return ok;
}

// Contiguous records src[0..n) -> dst[0..n), two records per 16-byte device-coherent load.  Each
// 8-byte record is read whole (it sits in one aligned 8-byte word), so a pair is complete once
// both halves carry the epoch.
template <bool HL>
__device__ __forceinline__ bool gather_vec_impl(MK_G MkCtl* ctl, u32 epoch, const MK_G mk_u64* src, int n,
                                                LS float* dst) {
  Ctx cx;
  cx.ctl = uni_ptr(ctl);
  cx.epoch = (u32)uni((int)epoch);
  src = uni_ptr(src);
  n = uni(n);
  const u32 e = cx.epoch;
  const int pl = tid() - NCT;
  const int np = (n + 1) >> 1;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, np * 16, 0x00020000);
  bool ok = true;
  for (int base = 0; ok && base < np; base += NPT * PB) {
    u32 pending = 0;
#pragma unroll
    for (int k = 0; k < PB; ++k)
      if (base + k * NPT + pl < np) pending |= 1u << k;
    u32 spins = 0;
    while (pending) {
      u32x4 v[PB];
#pragma unroll
      for (int k = 0; k < PB; ++k)
        if ((pending >> k) & 1u)
          v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (base + k * NPT + pl) * 16, 0, 16 /* sc1 */);
#pragma unroll
      for (int k = 0; k < PB; ++k) {
        const int j = base + k * NPT + pl;
        const bool two = 2 * j + 1 < n;
        if (((pending >> k) & 1u) && v[k].y == e && (!two || v[k].w == e)) {
          if (HL) {
            put_hl2((LS u32*)dst, 2 * j, __uint_as_float(v[k].x), two ? __uint_as_float(v[k].z) : 0.f);
          } else {
            dst[2 * j] = __uint_as_float(v[k].x);
            if (two) dst[2 * j + 1] = __uint_as_float(v[k].z);
          }
          pending &= ~(1u << k);
        }
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
  wait_vm<0>();  // as in gather_map
  return ok;
}

__device__ __forceinline__ bool gather_vec(const Ctx& cx, const MK_G mk_u64* src, int n, LS float* dst) {
  if (streamer()) return true;
  return gather_vec_impl<false>(cx.ctl, cx.epoch, src, n, dst);
}
// the same into the GEMV activation layout (hi/lo BF16 pairs); n even
__device__ __forceinline__ bool gather_hl(const Ctx& cx, const MK_G mk_u64* src, int n, LS u32* dst) {
  if (streamer()) return true;
  return gather_vec_impl<true>(cx.ctl, cx.epoch, src, n, (LS float*)dst);
}
// The same gather by all MK_NT threads with PBX polls in flight each, for kernels whose streaming
// waves hold no prefetch copies while they wait.
template <bool HL, int PBX>
__device__ __forceinline__ bool gather_vec_all(const Ctx& cx, const MK_G mk_u64* src, int n, LS float* dst) {
  src = uni_ptr(src);
  n = uni(n);
  const u32 e = cx.epoch;
  const int pl = tid();
  const int np = (n + 1) >> 1;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, np * 16, 0x00020000);
  bool ok = true;
  for (int base = 0; ok && base < np; base += MK_NT * PBX) {
    u32 pending = 0;
#pragma unroll
    for (int k = 0; k < PBX; ++k)
      if (base + k * MK_NT + pl < np) pending |= 1u << k;
    u32 spins = 0;
    while (pending) {
      u32x4 v[PBX];
#pragma unroll
      for (int k = 0; k < PBX; ++k)
        if ((pending >> k) & 1u)
          v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (base + k * MK_NT + pl) * 16, 0, 16 /* sc1 */);
#pragma unroll
      for (int k = 0; k < PBX; ++k) {
        const int j = base + k * MK_NT + pl;
        const bool two = 2 * j + 1 < n;
        if (((pending >> k) & 1u) && v[k].y == e && (!two || v[k].w == e)) {
          if (HL) {
            put_hl2((LS u32*)dst, 2 * j, __uint_as_float(v[k].x), two ? __uint_as_float(v[k].z) : 0.f);
          } else {
            dst[2 * j] = __uint_as_float(v[k].x);
            if (two) dst[2 * j + 1] = __uint_as_float(v[k].z);
          }
          pending &= ~(1u << k);
        }
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

// FP32 v[0..n) (n a multiple of 8) -> the GEMV activation layout in place, by all threads: each
// group of 8 values is rewritten as its hi and lo pairs.  Between barriers.
__device__ __forceinline__ void to_hl(LS float* v, int n) {
  for (int gidx = tid(); gidx < (n >> 3); gidx += MK_NT) {
    LS f32x4* p = (LS f32x4*)(v + 8 * gidx);
    const f32x4 a = p[0], b = p[1];
    u32 h[8], l[8];
    split_hl(a.x, h[0], l[0]);
    split_hl(a.y, h[1], l[1]);
    split_hl(a.z, h[2], l[2]);
    split_hl(a.w, h[3], l[3]);
    split_hl(b.x, h[4], l[4]);
    split_hl(b.y, h[5], l[5]);
    split_hl(b.z, h[6], l[6]);
    split_hl(b.w, h[7], l[7]);
    LS u32x4* q = (LS u32x4*)p;
    q[0] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    q[1] = u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
  }
}

// ------------------------------------------------------------------------ GEMV
// out[r] = W[r] . x for the R rows of a workgroup's slice (row stride K).  A unit is 4 rows x 512
// columns (4 KB of BF16): slot k (1 KB) is row k's 512 columns, contiguous in memory, and lane l holds
// columns 8l .. 8l+7 of all four rows, so a lane needs only its own 8 activations.  Activations are
// kept in LDS as BF16 hi + lo pairs (x = hi + lo to about 2^-17 relative): per group of 8 columns,
// 16 bytes of hi pairs then 16 bytes of lo pairs.  Products go through v_dot2c_f32_bf16 (exact BF16
// products, FP32 accumulation), two per weight pair.  A unit's four row partials are reduced over the
// wave in a fixed order (lane-half swaps, then a 16-lane DPP row sum) and parked in LDS; a row's
// value adds its 512-column segment partials in segment order, so it does not depend on how rows
// are split over workgroups.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct Gemv {
  const MK_G uint16_t* W;
  int R, K, S;  // rows, columns, 512-column segments
  __device__ __forceinline__ void init(const MK_G uint16_t* W_, int R_, int K_) {
    W = W_;
    R = R_;
    K = K_;
    S = (K + 511) >> 9;
  }
  __device__ __forceinline__ int units() const { return ((R + 3) >> 2) * S; }
  __device__ __forceinline__ int chunk_rows() const { return max(4, (MK_RED_CAP / S) & ~3); }
  // this lane's 16 bytes of slot k (row 4 rb + k) of unit u; null outside the matrix
  __device__ __forceinline__ const MK_G uint16_t* addr(int u, int k) const {
    const int rb = u / S, s = u - rb * S;
    const int row = rb * 4 + k;
    const int col = s * 512 + lane() * 8;
    return (row < R && col < K) ? W + (size_t)row * K + col : nullptr;
  }
  // slot k of unit u holds a row of the matrix (uniform over the wave)
  __device__ __forceinline__ bool live(int u, int k) const { return (u / S) * 4 + k < R; }
};

// Units staged for g: the first min(units of its first row chunk, cap) units.
__device__ __forceinline__ int staged_units(const Gemv& g, int cap) {
  Gemv c0 = g;
  c0.R = min(g.R, g.chunk_rows());
  return min(c0.units(), cap);
}

// First units of g -> stage slots [4u, 4u + 4): streaming wave c copies slot c of every unit.
// Returns the number of copies this wave issued.
__device__ __forceinline__ int gemv_stage_impl(const MK_G uint16_t* W, int R, int K, LS u32x4* stage, int cap) {
  Gemv g;
  g.init(uni_ptr(W), uni(R), uni(K));
  const int n = staged_units(g, uni(cap));
  const int c = wave();
  int cnt = 0;
  for (int u = 0; u < n; ++u) {
    if (g.live(u, c)) {
      const MK_G uint16_t* a = g.addr(u, c);
      if (a) dma16(a, stage + (u * USLOTS + c) * SLOT);
      ++cnt;  // lane 0 (the segment's first 8 columns) is always inside the matrix here
    }
  }
  return cnt;
}

__device__ __forceinline__ int gemv_stage(const Gemv& g, LS u32x4* stage, int cap) {
  if (!streamer()) return 0;
  return gemv_stage_impl(g.W, g.R, g.K, stage, cap);
}

__device__ __forceinline__ void put_partial(const Gemv& g, int u, float v, LS float* red) {
  if ((lane() & 15) == 0) {
    const int rb = u / g.S, s = u - rb * g.S;
    const int row = rb * 4 + (lane() >> 4);
    if (row < g.R) red[row * g.S + s] = v;
  }
}

// a row's segment partials added in segment order; loads are issued eight at a time
__device__ __forceinline__ float seg_sum(const LS float* p, int S) {
  float v = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = s0 + k < S ? p[s0 + k] : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (s0 + k < S) v += t[k];
  }
  return v;
}

template <int N>
struct RegUnits {
  u32x4 c[N * USLOTS];
};

// This lane's activations for 512-column segment s: hi and lo pairs of columns s*512 + 8 lane ...
struct XSlice {
  u32x4 h, l;
};
__device__ __forceinline__ void load_x(XSlice& x, const LS u32* hl, int s, int K) {
  const int col = s * 512 + lane() * 8;
  x.h = u32x4{0u, 0u, 0u, 0u};
  x.l = x.h;
  if (col < K) {
    const LS u32x4* p = (const LS u32x4*)(hl + (col >> 3) * 8);
    x.h = p[0];
    x.l = p[1];
  }
}
__device__ __forceinline__ float dot2(u32 w, u32 x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, x), acc, false);
}
// one row's 8 weights . this lane's 8 activations (hi then lo)
__device__ __forceinline__ float dot8hl(u32x4 w, const XSlice& x) {
  float a = dot2(w.x, x.h.x, 0.f);
  a = dot2(w.y, x.h.y, a);
  a = dot2(w.z, x.h.z, a);
  a = dot2(w.w, x.h.w, a);
  a = dot2(w.x, x.l.x, a);
  a = dot2(w.y, x.l.y, a);
  a = dot2(w.z, x.l.z, a);
  return dot2(w.w, x.l.w, a);
}
// Four per-lane row partials -> in every lane of 16-lane row i, row i's sum over the wave: rows 0/1
// and 2/3 trade lane halves (permlane32 swap), then rows 0/1 and 2/3 trade 16-lane rows (permlane16
// swap), then a DPP sum within each 16-lane row.
__device__ __forceinline__ float reduce_rows4(float a0, float a1, float a2, float a3) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a0), __float_as_uint(a2), false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a1), __float_as_uint(a3), false, false);
  const float p = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
  const float q = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(q), false, false);
  return row_sum16(__uint_as_float(t[0]) + __uint_as_float(t[1]));
}
// unit partial (row 4 rb + lane / 16 in 16-lane row lane / 16) from its four row slots; lanes past
// column K add nothing (their weights were never copied)
__device__ __forceinline__ float unit_dot_x(int s, int K, const u32x4* w, const XSlice& x) {
  const bool in = s * 512 + lane() * 8 < K;
  float a[USLOTS];
#pragma unroll
  for (int k = 0; k < USLOTS; ++k) a[k] = in ? dot8hl(w[k], x) : 0.f;
  return reduce_rows4(a[0], a[1], a[2], a[3]);
}

// Segment-major split of a GEMV's units over a set of NWS waves (this wave is ws): with S <= NWS
// segments, wave ws takes segment ws % S and every nj-th row block from ws / S; otherwise segments
// ws, ws + NWS, ... with every row block.  A wave keeps its segment's activations in registers.
struct SegPlan {
  int s0, sstep, j, nj;
  __device__ __forceinline__ void init(int S, int ws, int NWS) {
    if (S <= NWS) {
      s0 = ws % S;
      sstep = S;
      j = ws / S;
      nj = (NWS - s0 + S - 1) / S;
    } else {
      s0 = ws;
      sstep = NWS;
      j = 0;
      nj = 1;
    }
  }
};

// Unit partials of one row chunk -> red[row * S + segment].  Units u = rb * S + s < nst come from
// the LDS stage (every wave), the rest stream through registers (streaming waves; ALL_STREAM: all).
// xin: activations in hi/lo layout.
template <bool ALL_STREAM>
__device__ __forceinline__ void gemv_partials(const MK_G uint16_t* W, int R, int K, int nst, const LS u32* xin,
                                              const LS u32x4* stage, LS float* red) {
  Gemv g;
  g.init(uni_ptr(W), uni(R), uni(K));
  nst = uni(nst);
  const int S = g.S, RB = (g.R + 3) >> 2;
  {
    SegPlan sp;
    sp.init(S, wave(), MK_NWAVE);
    for (int s = sp.s0; s < S; s += sp.sstep) {
      if (sp.j * S + s >= nst) break;
      XSlice x;
      load_x(x, xin, s, g.K);
      for (int rb = sp.j; rb * S + s < nst; rb += 2 * sp.nj) {
        const int u0 = rb * S + s, u1 = (rb + sp.nj) * S + s;
        const bool h1 = u1 < nst;
        u32x4 w0[USLOTS], w1[USLOTS];
        if (h1) {
          stage_units2(stage + u0 * USLOTS * SLOT + lane(), stage + u1 * USLOTS * SLOT + lane(), w0, w1);
        } else {
          stage_unit(stage + u0 * USLOTS * SLOT + lane(), w0);
#pragma unroll
          for (int k = 0; k < USLOTS; ++k) w1[k] = u32x4{0u, 0u, 0u, 0u};
        }
        const float a0 = unit_dot_x(s, g.K, w0, x);
        const float a1 = h1 ? unit_dot_x(s, g.K, w1, x) : 0.f;
        put_partial(g, u0, a0, red);
        if (h1) put_partial(g, u1, a1, red);
      }
    }
  }
  if (ALL_STREAM || streamer()) {
    const int NSW = ALL_STREAM ? MK_NWAVE : NCW;
    SegPlan sp;
    sp.init(S, wave(), NSW);
    for (int s = sp.s0; s < S; s += sp.sstep) {
      // first row block of this wave's sequence whose unit is past the stage
      int rb = sp.j;
      if (rb * S + s < nst) rb += ((nst - s - rb * S + S - 1) / S + sp.nj - 1) / sp.nj * sp.nj;
      if (rb >= RB) continue;
      XSlice x;
      load_x(x, xin, s, g.K);
      const int step = sp.nj;
      auto issue2 = [&](RegUnits<2>& r, int rb0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int rbi = rb0 + i * step;
#pragma unroll
          for (int k = 0; k < USLOTS; ++k) {
            const MK_G uint16_t* a = rbi < RB ? g.addr(rbi * S + s, k) : nullptr;
            r.c[i * USLOTS + k] = a ? ldw(a) : u32x4{0u, 0u, 0u, 0u};
          }
        }
      };
      RegUnits<2> cur, nxt;
      issue2(cur, rb);
      // Nothing may look outstanding in cur when the loop starts: these loads are conditional, and
      // a register the compiler cannot place in the load queue makes it wait for every load, the
      // look-ahead ones included, before each unit.  (The stage copies this wave issued for the
      // same GEMV were waited for before the barrier that preceded it.)
      wait_vm<0>();
      for (; rb < RB; rb += 2 * step) {
        issue2(nxt, rb + 2 * step);
        keep_issued();
        const bool h1 = rb + step < RB;
        const float a0 = unit_dot_x(s, g.K, cur.c, x);
        const float a1 = h1 ? unit_dot_x(s, g.K, cur.c + USLOTS, x) : 0.f;
        put_partial(g, rb * S + s, a0, red);
        if (h1) put_partial(g, (rb + step) * S + s, a1, red);
#pragma unroll
        for (int i = 0; i < 2 * USLOTS; ++i) cur.c[i] = nxt.c[i];
      }
      // The last iteration's look-ahead loads are never used.  Waiting for them here, on the path
      // that issued them, keeps them from looking outstanding afterwards, where the compiler would
      // otherwise wait for all vector-memory operations (prefetch copies included) before reusing
      // their registers.
      wait_vm<0>();
    }
  }
}

template <bool PAIRS, bool EPI_ALL, bool ALL_STREAM, typename Epi>
__device__ __forceinline__ void gemv(const Gemv& G, const LS u32* xin, const LS u32x4* stage, int cap,
                                     LS float* red, Tracer& tr, Epi epi) {
  const int rc = G.chunk_rows();
  for (int r0 = 0; r0 < G.R; r0 += rc) {
    Gemv g;
    g.init(G.W + (size_t)r0 * G.K, min(rc, G.R - r0), G.K);
    const int nst = r0 == 0 ? min(g.units(), cap) : 0;
    gemv_partials<ALL_STREAM>(g.W, g.R, g.K, nst, xin, stage, red);
    tr.mark();
    wg_bar();
    tr.mark();
    const int stride = EPI_ALL ? MK_NT : NCT;
    if (EPI_ALL || streamer()) {
      if (PAIRS) {
        for (int t = tid(); t < g.R / 2; t += stride) epi(r0 / 2 + t, seg_sum(red + (2 * t) * g.S, g.S),
                                                          seg_sum(red + (2 * t + 1) * g.S, g.S));
      } else {
        for (int t = tid(); t < g.R; t += stride) epi(r0 + t, seg_sum(red + t * g.S, g.S), 0.f);
      }
    }
    if (r0 + rc < G.R) wg_bar();  // red is reused by the next chunk
  }
}

// x -> xn = x / sqrt(mean x^2 + eps) * g, written as hi/lo BF16 pairs (the GEMV activation layout).
// Every wave sums the squares itself (same order in every wave), so only the barrier that
// publishes xn is needed.
__device__ __forceinline__ void rmsnorm(const LS float* x, const LS uint16_t* g, LS u32* xn, int D, float eps,
                                        Tracer& tr) {
  D = uni(D);
  const int D4 = D >> 2;  // D is a multiple of 8
  const LS f32x4* x4 = (const LS f32x4*)x;
  // four float4 loads in flight per lane before any of them is used
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
  for (int c = tid(); c < D4; c += MK_NT) {
    const f32x4 v = x4[c];
    const u32x2 gg = *(const LS u32x2*)(g + 4 * c);
    u32 h[4], l[4];
    split_hl(v.x * r * __uint_as_float(gg.x << 16), h[0], l[0]);
    split_hl(v.y * r * __uint_as_float(gg.x & 0xffff0000u), h[1], l[1]);
    split_hl(v.z * r * __uint_as_float(gg.y << 16), h[2], l[2]);
    split_hl(v.w * r * __uint_as_float(gg.y & 0xffff0000u), h[3], l[3]);
    const int o = hl_word(4 * c);  // even: columns 4c .. 4c+3 fill two hi and two lo pair words
    *(LS u32x2*)(xn + o) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    *(LS u32x2*)(xn + o + 4) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
  }
  tr.mark();
  wg_bar();
}

// RMSNorm gains (BF16, n values, n a multiple of 8) -> LDS by the polling threads with plain loads:
// issued before a poll (they complete under its latency) and stored after it.  Up to GAIN_REGS
// 16-byte pieces per thread ride along; any remainder is copied after the poll.
constexpr int GAIN_REGS = 2;
struct GainCopy {
  u32x4 r[GAIN_REGS];
};
__device__ __forceinline__ void gains_issue(const MK_G uint16_t* src, int n, GainCopy& gc) {
  const int pieces = n >> 3, pl = tid() - NCT;
#pragma unroll
  for (int k = 0; k < GAIN_REGS; ++k) {
    const int i = pl + k * NPT;
    gc.r[k] = i < pieces ? *(const MK_G u32x4*)(src + 8 * i) : u32x4{0u, 0u, 0u, 0u};
  }
}
__device__ __forceinline__ void gains_store(const MK_G uint16_t* src, int n, const GainCopy& gc, LS uint16_t* dst) {
  const int pieces = n >> 3, pl = tid() - NCT;
#pragma unroll
  for (int k = 0; k < GAIN_REGS; ++k) {
    const int i = pl + k * NPT;
    if (i < pieces) *(LS u32x4*)(dst + 8 * i) = gc.r[k];
  }
  for (int i = pl + GAIN_REGS * NPT; i < pieces; i += NPT) *(LS u32x4*)(dst + 8 * i) = *(const MK_G u32x4*)(src + 8 * i);
}

__device__ __forceinline__ MkLayerDev layer_desc(const LS MkLayerDev* d, int l) {
  MkLayerDev out;
  const LS u32* src = (const LS u32*)(d + l);
  u32* dst = (u32*)&out;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(MkLayerDev) / 4); ++i) dst[i] = __builtin_amdgcn_readfirstlane(src[i]);
  return out;
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ __forceinline__ float softplusf_(float z) { return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z))); }

// ------------------------------------------------------------------------ DeltaNet
// Per-head scalars of the gated delta rule from the head's raw q, k and gate logits ab = (a, b):
// 1 / ||q|| and 1 / ||k|| (each with eps), alpha = exp(-softplus(a)), beta = sigmoid(b).  Called by a
// whole wave (the sums are wave reductions); every wave forms them identically.
struct DnHead {
  float sq, sk, alpha, beta;
};
__device__ __forceinline__ DnHead dn_head(const LS float* q, const LS float* k, const LS float* ab, int dk,
                                          float l2eps) {
  float qq = 0.f, kk = 0.f;
  for (int e = lane(); e < dk; e += 64) {
    qq = fmaf(q[e], q[e], qq);
    kk = fmaf(k[e], k[e], kk);
  }
  qq = wave_sum(qq);
  kk = wave_sum(kk);
  DnHead h;
  h.sq = 1.0f / sqrtf(qq + l2eps);
  h.sk = 1.0f / sqrtf(kk + l2eps);
  h.alpha = expf(-softplusf_(ab[0]));
  h.beta = sigmoidf_(ab[1]);
  return h;
}
// One state row through the gated delta rule, by a whole wave.  sr[t] is this lane's S[row][lane +
// 64 t]; the updated row S' = alpha S + beta (v - alpha S.k^) k^ is stored to Srow, and the row's
// output S'.q^ (read after the update) is returned in every lane.
__device__ __forceinline__ float dn_row(const float (&sr)[4], const LS float* q, const LS float* k, const DnHead& h,
                                        float v, MK_G float* Srow, int dk) {
  float kd = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int e = lane() + 64 * t;
    if (e < dk) kd = fmaf(sr[t], k[e] * h.sk, kd);
  }
  kd = wave_sum(kd);
  const float u = h.beta * (v - h.alpha * kd);
  float od = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int e = lane() + 64 * t;
    if (e < dk) {
      const float nv2 = fmaf(u, k[e] * h.sk, h.alpha * sr[t]);
      Srow[e] = nv2;
      od = fmaf(nv2, q[e] * h.sq, od);
    }
  }
  return wave_sum(od);
}

// state rows [s0, s1) -> stage slots: dk/4 lanes per row, 64/(dk/4) rows per slot.  Returns copies
// issued by this wave.
__device__ __forceinline__ int state_stage(const MkDecodeParams& p, const MkLayerDev& L, int s0, int s1,
                                           LS u32x4* stage, int max_slots) {
  if (!streamer()) return 0;
  const int lpr = p.dk >> 2, rps = 64 / lpr;
  const int nslots = min((s1 - s0 + rps - 1) / rps, max_slots);
  int cnt = 0;
  for (int j = wave(); j < nslots; j += NCW) {
    const int r = s0 + j * rps + lane() / lpr;
    if (lane() < rps * lpr && r < s1) dma16(L.S + (size_t)r * p.dk + (lane() % lpr) * 4, stage + j * SLOT);
    ++cnt;  // the slot's first row is always in range
  }
  return cnt;
}

// gated delta rule on rows [s0, s1) of S; o = S q read after the update -> records.  Rows of
// staged slots come from LDS, the rest straight from HBM.  With POLL_ROWS the polling waves own the
// rows and the streaming waves call side() once, after the first head's inputs have arrived, so
// the copies it issues enter the compute unit's queue while the rows are computed rather than
// ahead of the next gather's polls; otherwise the streaming waves own the rows and side is not
// called.
template <bool POLL_ROWS, typename Side>
__device__ __forceinline__ bool dn_state(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx, const Lds& s,
                                         int s0, int s1, int st_slots, int wait_after, Tracer& tr, Side side) {
  const int H = p.H, dk = p.dk, dv = p.dv;
  const int lpr = dk >> 2, rps = 64 / lpr;
  LS float* q = s.att;
  LS float* k = s.att + dk;
  LS float* ab = s.att + 2 * dk;
  LS float* vr = s.att + 2 * dk + 2;
  const LS float* st = (const LS float*)s.stB;
  const MK_G mk_u64* in = L.ll_in;
  const int off_k = H * dk, off_v = 2 * H * dk, off_a = 2 * H * dk + H * dv, off_b = off_a + H;
  bool first = true, side_done = false;
  // row waves: rw = 0 .. NRW - 1
  constexpr int NRW = POLL_ROWS ? MK_NWAVE - NCW : NCW;
  const bool row_wave = POLL_ROWS ? !streamer() : streamer();
  const int rw = POLL_ROWS ? wave() - NCW : wave();
  const int h0 = s0 < s1 ? s0 / dv : 0, h1 = s0 < s1 ? (s1 - 1) / dv : -1;
  for (int h = h0; h <= h1; ++h) {
    const int i0 = max(s0, h * dv) - h * dv, i1 = min(s1, (h + 1) * dv) - h * dv;
    const int nv = i1 - i0;
    const int n = 2 * dk + 2 + nv;
    const bool ok = gather_map(cx, n, [=](int f) {
      if (f < dk) return in + h * dk + f;
      if (f < 2 * dk) return in + off_k + h * dk + (f - dk);
      if (f == 2 * dk) return in + off_a + h;
      if (f == 2 * dk + 1) return in + off_b + h;
      return in + off_v + h * dv + i0 + (f - 2 * dk - 2);
    }, [=](int f, float v) { s.att[f] = v; });
    tr.mark();
    if (first && streamer()) wait_vm_n(wait_after);  // the staged state rows
    first = false;
    tr.mark();
    if (wg_bar_or(s, !ok)) return false;
    tr.mark();
    if (POLL_ROWS && !side_done) {
      if (streamer()) side();
      side_done = true;
    }
    if (row_wave) {
      const DnHead hs = dn_head(q, k, ab, dk, p.l2_eps);
      // rows of head h, local index li = row - s0, owned by row wave li % NRW
      const int lo = h * dv + i0 - s0, hi = h * dv + i1 - s0;
      // Two copies of the row loop: when every row of this head is staged the loop issues no global
      // load, so the compiler has no reason to wait on the vector-memory counter inside it -- a
      // wait there would also wait for the previous row's state stores and record store.
      auto rows = [&](auto staged_tag) {
        constexpr bool STAGED = decltype(staged_tag)::value;
        for (int li = lo + ((rw - lo % NRW) + NRW) % NRW; li < hi; li += NRW) {
          const int row = s0 + li;
          const int sl = li / rps;
          const LS float* srow = st + sl * 256 + (li % rps) * dk;
          float sr[4];
          if (STAGED) {
            const int l0 = lane();
            stage_f32x4(srow + l0, srow + (l0 + 64 < dk ? l0 + 64 : 0), srow + (l0 + 128 < dk ? l0 + 128 : 0),
                        srow + (l0 + 192 < dk ? l0 + 192 : 0), sr);
#pragma unroll
            for (int t = 0; t < 4; ++t)
              if (lane() + 64 * t >= dk) sr[t] = 0.f;
          } else {
            const bool staged = sl < st_slots;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int e = lane() + 64 * t;
              sr[t] = e < dk ? (staged ? srow[e] : L.S[(size_t)row * dk + e]) : 0.f;
            }
          }
          const float od = dn_row(sr, q, k, hs, vr[row - h * dv - i0], L.S + (size_t)row * dk, dk);
          if (lane() == 0) ll_put(L.ll_o + row, cx.epoch, od);
        }
      };
      if (lo >= hi || (hi - 1) / rps < st_slots) rows(std::true_type{});
      else rows(std::false_type{});
    }
    tr.mark();
    wg_bar();  // s.att is reused by the next head
  }
  if (first && streamer()) wait_vm_n(wait_after);
  if (POLL_ROWS && !side_done && streamer()) side();
  return true;
}

// ------------------------------------------------------------------------ attention
// KV cache rows.  A row holds the head_dim values of one position of one KV head in the cache type
// kvt: FP32, binary16, or int8 codes with one FP32 scale per 32 values kept in a separate scale row
// (Ks / Vs, hd / 32 floats per position).  Attention always works on FP32 rows in LDS: a chunk of
// FP32 rows is copied there as is; compact rows are copied there compact and then expanded.
__device__ __forceinline__ int kv_rowbytes(int hd, int kvt) {
  return kvt == MK_KV_F32 ? 4 * hd : (kvt == MK_KV_F16 ? 2 * hd : hd);
}
// 1 KB stage slots holding the K (or V) rows of one 16-position chunk
__device__ __forceinline__ int kv_slots(int hd, int kvt = MK_KV_F32) {
  const int lpp = kv_rowbytes(hd, kvt) >> 4, pps = 64 / lpp;
  return (ATT_C + pps - 1) / pps;
}
// K and V rows (and, for int8 rows, the chunk's K and V scales in one more slot) of work item `it`
// (16 positions of one KV head) -> stage slots [0, ks) (K), [ks, 2 ks) (V), 2 ks (scales: K at byte
// 0, V at byte 512); a row is copied by rowbytes / 16 lanes.  Only positions already in the cache
// (< pos) are copied; position pos comes from the exchange records.  Returns copies issued by this
// wave.
__device__ __forceinline__ int kv_stage(const MkDecodeParams& p, const MkLayerDev& L, int it, int pos,
                                        LS u32x4* stage) {
  if (!streamer()) return 0;
  const int kvt = p.kvt;
  const int rb = kv_rowbytes(p.hd, kvt), lpp = rb >> 4, pps = 64 / lpp, ks = kv_slots(p.hd, kvt);
  const int c = it / p.nkv, g = it - c * p.nkv;
  const int j0 = c * ATT_C, jend = min(pos, j0 + ATT_C);
  int cnt = 0;
  for (int q = wave(); q < 2 * ks; q += NCW) {
    const int v = q >= ks ? 1 : 0;
    const int sl = q - v * ks;
    const int j = j0 + sl * pps + lane() / lpp;
    if (lane() < pps * lpp && j < jend)
      dma16((const MK_G char*)(v ? L.Vc : L.Kc) + ((size_t)g * p.max_ctx + j) * rb + (lane() % lpp) * 16,
            stage + q * SLOT);
    if (j0 + sl * pps < jend) ++cnt;
  }
  if (kvt == MK_KV_Q8 && wave() == (2 * ks) % NCW) {
    // the chunk's scale rows are contiguous: 16 positions x hd / 32 floats for K, then for V
    const int fpp = p.hd / MK_KV_Q8_BLOCK, nl = (ATT_C * fpp + 3) >> 2;
    const int v = lane() >= 32 ? 1 : 0, l = lane() - 32 * v;
    if (l < nl && j0 + (4 * l) / fpp < jend)
      dma16((v ? L.Vs : L.Ks) + ((size_t)g * p.max_ctx + j0) * fpp + 4 * l, stage + 2 * ks * SLOT);
    if (j0 < jend) ++cnt;
  }
  return cnt;
}

// LDS reads of a stage region (asm, each waits for its own reads; see the stage notes above)
__device__ __forceinline__ u32x2 stage_b64(const LS void* p) {
  u32x2 v;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}
__device__ __forceinline__ u32 stage_b32(const LS void* p) {
  u32 v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}
__device__ __forceinline__ void stage_write_f4(LS void* p, f32x4 v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ float half_bits_f32(u32 h) {
  _Float16 x;
  __builtin_memcpy(&x, &h, 2);
  return (float)x;
}
__device__ __forceinline__ float f16_round(float x) { return (float)(_Float16)x; }
__device__ __forceinline__ float i8_f32(u32 w, int b) { return (float)(int)(signed char)(w >> (8 * b)); }

// Compact rows of a staged chunk are read where they are used and converted to FP32 in registers:
// binary16 values exactly, int8 codes times their block's FP32 scale (one multiplication), the same
// values the verify kernels form.  Staged layout of a chunk (kv_stage): K rows in slots [0, ksc), V rows
// in [ksc, 2 ksc), ppsc = 1024 / rowbytes rows per slot; int8 rows also carry a slot of scales, K at
// byte 0 and V at byte 512, hd / 32 floats per position.
struct KvCompact {
  const LS char* base;
  int rb, ppsc, ksc, fpp;
  __device__ __forceinline__ const LS char* row(int v, int jj) const {
    return base + (v * ksc + jj / ppsc) * 1024 + (jj % ppsc) * rb;
  }
  __device__ __forceinline__ const LS float* scales(int v, int jj) const {
    return (const LS float*)(base + 2 * ksc * 1024) + v * 128 + jj * fpp;
  }
};
__device__ __forceinline__ KvCompact kv_compact(int hd, int kvt, const LS u32x4* buf) {
  KvCompact c;
  c.base = (const LS char*)buf;
  c.rb = kv_rowbytes(hd, kvt);
  c.ppsc = 1024 / c.rb;
  c.ksc = kv_slots(hd, kvt);
  c.fpp = hd / MK_KV_Q8_BLOCK;
  return c;
}
// four groups of four values (elements 4 g[x] .. 4 g[x] + 3) of one compact row (scale row sr for
// int8), converted, with one wait for all the reads
template <int KVT>
__device__ __forceinline__ void kv_groups4(const LS char* r, const LS float* sr, const int (&g)[4], f32x4 (&o)[4]) {
  if (KVT == MK_KV_F16) {
    u32x2 h[4];
    asm volatile(
        "ds_read_b64 %0, %4\n\tds_read_b64 %1, %5\n\tds_read_b64 %2, %6\n\tds_read_b64 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3])
        : "v"(lds_addr(r + 8 * g[0])), "v"(lds_addr(r + 8 * g[1])), "v"(lds_addr(r + 8 * g[2])),
          "v"(lds_addr(r + 8 * g[3]))
        : "memory");
#pragma unroll
    for (int x = 0; x < 4; ++x)
      o[x] = f32x4{half_bits_f32(h[x].x & 0xffffu), half_bits_f32(h[x].x >> 16), half_bits_f32(h[x].y & 0xffffu),
                   half_bits_f32(h[x].y >> 16)};
  } else {
    u32 c[4], f[4];
    asm volatile(
        "ds_read_b32 %0, %8\n\tds_read_b32 %1, %9\n\tds_read_b32 %2, %10\n\tds_read_b32 %3, %11\n\t"
        "ds_read_b32 %4, %12\n\tds_read_b32 %5, %13\n\tds_read_b32 %6, %14\n\tds_read_b32 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3]), "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
        : "v"(lds_addr(r + 4 * g[0])), "v"(lds_addr(r + 4 * g[1])), "v"(lds_addr(r + 4 * g[2])),
          "v"(lds_addr(r + 4 * g[3])), "v"(lds_addr(sr + (4 * g[0]) / MK_KV_Q8_BLOCK)),
          "v"(lds_addr(sr + (4 * g[1]) / MK_KV_Q8_BLOCK)), "v"(lds_addr(sr + (4 * g[2]) / MK_KV_Q8_BLOCK)),
          "v"(lds_addr(sr + (4 * g[3]) / MK_KV_Q8_BLOCK))
        : "memory");
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float sc = __uint_as_float(f[x]);
      o[x] = f32x4{i8_f32(c[x], 0) * sc, i8_f32(c[x], 1) * sc, i8_f32(c[x], 2) * sc, i8_f32(c[x], 3) * sc};
    }
  }
}

// Key and value rows of this launch's positions pos0 .. pos0 + nr - 1, gathered from the exchange
// records in FP32 (row r of K at kb + r hd, of V at vb + r hd, in LDS), take the values the cache will
// hold -- so this launch uses exactly what later launches read back -- and the streaming threads
// append them to the cache.  scr: 2 nr hd / 32 floats of LDS scratch.  Contains workgroup barriers;
// every thread calls it with the same arguments.
__device__ __forceinline__ void kv_round_append(const MkDecodeParams& p, const MkLayerDev& L, LS float* kb,
                                                LS float* vb, int nr, LS float* scr, int g, int pos0) {
  const int hd = p.hd, kvt = p.kvt, nblk = hd / MK_KV_Q8_BLOCK, ne = nr * hd;
  const size_t row0 = (size_t)g * p.max_ctx + pos0;
  if (kvt == MK_KV_F16) {
    for (int e = tid(); e < 2 * ne; e += MK_NT) {
      const int v = e >= ne ? 1 : 0;
      LS float* x = (v ? vb : kb) + (e - v * ne);
      *x = f16_round(*x);
    }
    wg_bar();
    if (streamer())
      for (int e = tid(); e < 2 * ne; e += NCT) {
        const int v = e >= ne ? 1 : 0, r = e - v * ne;
        ((MK_G _Float16*)(v ? L.Vc : L.Kc))[row0 * hd + r] = (_Float16)(v ? vb : kb)[r];
      }
    return;
  }
  // int8: scale of each block of 32 = max |x| / 127, code = rint(x / scale) (0 when the block is 0)
  for (int b = tid(); b < 2 * nr * nblk; b += MK_NT) {
    const int v = b >= nr * nblk ? 1 : 0, rb = b - v * nr * nblk;
    const LS float* x = (v ? vb : kb) + rb * MK_KV_Q8_BLOCK;
    float m = 0.f;
    for (int i = 0; i < MK_KV_Q8_BLOCK; ++i) m = fmaxf(m, fabsf(x[i]));
    const float sc = m / 127.0f;
    scr[b] = sc;
    if (streamer()) (v ? L.Vs : L.Ks)[row0 * nblk + rb] = sc;
  }
  wg_bar();
  if (streamer())
    for (int e = tid(); e < 2 * ne; e += NCT) {
      const int v = e >= ne ? 1 : 0, r = e - v * ne;
      LS float* x = (v ? vb : kb) + r;
      const float sc = scr[v * nr * nblk + r / MK_KV_Q8_BLOCK];
      const float c = sc > 0.f ? rintf(*x / sc) : 0.f;
      ((MK_G signed char*)(v ? L.Vc : L.Kc))[row0 * hd + r] = (signed char)(int)c;
      *x = c * sc;
    }
  wg_bar();
}

// q/k/v rows in RoPE pair order: rotate q and k at position pos, append k and v to the cache
// `run(epi)` performs the in-projection GEMV of this workgroup's row pairs with epilogue epi.
template <typename Run>
__device__ __forceinline__ void att_qkv_run(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx, const Lds& s,
                                            int P0, int pos, Run run) {
  const int hd = p.hd, half = hd / 2;
  MK_G mk_u64* llq = L.ll_in;
  MK_G mk_u64* llk = L.ll_in + p.nq * hd;
  MK_G mk_u64* llv = llk + p.nkv * hd;
  const int nqp = p.nq * half, nkp = p.nkv * half;
  run([&](int pl, float x1, float x2) {
    const int P = P0 + pl;
    if (P < nqp + nkp) {
      const bool isq = P < nqp;
      const int Q = isq ? P : P - nqp;
      const int hh = Q / half, m = Q - hh * half;
      const float c = s.rope[m], sv = s.rope[half + m];
      const float y1 = x1 * c - x2 * sv;
      const float y2 = x2 * c + x1 * sv;
      if (isq) {
        ll_put(llq + hh * hd + m, cx.epoch, y1);
        ll_put(llq + hh * hd + m + half, cx.epoch, y2);
      } else {
        const size_t co = ((size_t)hh * p.max_ctx + pos) * hd + m;
        ll_put(llk + hh * hd + m, cx.epoch, y1);
        ll_put(llk + hh * hd + m + half, cx.epoch, y2);
        if (p.kvt == MK_KV_F32) {  // compact rows are appended by the attention item holding pos
          L.Kc[co] = y1;
          L.Kc[co + half] = y2;
        }
      }
    } else {
      const int Q = P - nqp - nkp;
      const int hh = Q / half, m = Q - hh * half;
      const size_t co = ((size_t)hh * p.max_ctx + pos) * hd + m;
      ll_put(llv + hh * hd + m, cx.epoch, x1);
      ll_put(llv + hh * hd + m + half, cx.epoch, x2);
      if (p.kvt == MK_KV_F32) {
        L.Vc[co] = x1;
        L.Vc[co + half] = x2;
      }
    }
  });
}

__device__ __forceinline__ void att_qkv(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx, const Lds& s,
                                        const Gemv& g, int P0, int pos, Tracer& tr) {
  att_qkv_run(p, L, cx, s, P0, pos,
              [&](auto epi) { gemv<true, false, false>(g, s.xn, s.stA, A_UNITS, s.att, tr, epi); });
}

// Split-K partial softmax attention.  Item = (chunk of 16 positions, KV head g); for each of the
// gs query heads of group g it emits (max m, sum l, acc[hd]) over its positions.  Scores: one thread
// per (head, position), a 16-lane DPP row per head for the max and the sum.
// KV stage slots of one 16-position chunk (K rows, V rows, and for int8 rows a slot of scales),
// rounded to whole GEMV units
__device__ __forceinline__ int kv_buf_slots(int hd, int kvt = MK_KV_F32) {
  return (2 * kv_slots(hd, kvt) + (kvt == MK_KV_Q8 ? 1 : 0) + 3) & ~3;
}
// chunk buffers in stage A (up to 3: the copies of the next two chunks run while one is used)
__device__ __forceinline__ int kv_nbuf(int hd, int kvt, int a_slots) {
  return max(1, min(3, a_slots / kv_buf_slots(hd, kvt)));
}

// Split-K attention over positions 0..pos.  A work item is (block of p.att_cpi 16-position chunks,
// KV head g); item it = block * nkv + g.  Chunk by chunk, the item computes for each of the gs query
// heads of group g the scores of its positions (one thread per (head, position), a 16-lane DPP row
// per head for the max and the sum), the softmax numerators and acc[d] = sum p v_d; chunks after
// the first of the item are merged into the running (max, sum, acc) in chunk order:
//   M' = max(M, m), f = exp(M - M'), f' = exp(m - M'), acc' = acc f + a f', sum' = sum f + l f'.
// The item publishes (M, sum, acc[hd]) per head.  With att_cpi = 1 an item is one chunk.
// Staging: stage A holds nb = kv_nbuf(hd) chunk buffers; chunk k of the workgroup's sequence uses
// buffer k % nb.  The caller has issued the copies of chunks 0 .. max(nb - 2, 0); when chunk k
// starts it issues chunk k + nb - 1 into the buffer chunk k - 1 has finished with (chunk 0 issues
// chunk nb - 1 into the last, unused buffer), then waits until only the copies of the chunks after
// k may remain (chunk 0 waits for all of them).  Queries are gathered once per KV head; the keys and
// values of position pos only by the chunk that holds it.
// ---- attention scores in key-dimension parts
// A (query, key) score is a dot product over hd dimensions, taken as hd/4 groups of four.  The
// groups are cut into np = att_parts(gs, hd) equal parts of gpp = hd/4/np groups, each summed by its
// own thread: part `part` is one fused multiply-add chain over groups part*gpp .. part*gpp + gpp - 1,
// starting at group jj mod gpp of the part and wrapping around (jj is the key's slot in its 16-position
// chunk, so the slots of a row start on different banks), four FMAs per group.  The np part sums are
// added in a fixed pairwise tree (att_part_sum).  np is the largest power of two that divides hd/4
// with np * gs * 16 <= MK_NT, so one position's scores of a chunk take at most one pass of the
// workgroup -- unless a verify launch's rows (MK_VERIFY_MAXT positions) already outnumber the
// workgroup's threads: then the parts would only add instructions to a loop that is bound by its
// issue (measured at the 27B-scale shape), and the score is one chain (np = 1).  The decode and
// verify kernels both score through these helpers, so their scores agree bit for bit.
__host__ __device__ inline int att_parts(int gs, int hd) {
  const int rows = gs * ATT_C, n4 = hd >> 2;
  int np = 1;
  if (MK_VERIFY_MAXT * rows > MK_NT) return np;
  while (2 * np * rows <= MK_NT && n4 % (2 * np) == 0) np *= 2;
  return np;
}
// one part of q . k, W groups per step (the loads of a step are in flight together; steps past the
// part's end add zero products); KSTAGE: the key row lies in an LDS-DMA stage region (read through
// asm, see g_stage)
template <bool KSTAGE, int W>
__device__ __forceinline__ float qk_part_w(const LS float* kr, const LS float* qr, int jj, int part, int gpp) {
  const int g0 = part * gpp, start = jj % gpp;
  float a = 0.f;
  for (int x0 = 0; x0 < gpp; x0 += W) {
    f32x4 kk[W], qq[W];
    const LS float* ka[W];
#pragma unroll
    for (int x = 0; x < W; ++x) {
      int gg = x0 + x + start;
      gg = gg >= gpp ? gg - gpp : gg;
      const bool in = x0 + x < gpp;
      const int dd = (g0 + gg) * 4;
      ka[x] = kr + (in ? dd : 0);
      qq[x] = in ? *(const LS f32x4*)(qr + dd) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (KSTAGE) {
      if constexpr (W == 8) stage_f4x8(ka, kk);
      else stage_f4x4(ka, kk);
    } else {
#pragma unroll
      for (int x = 0; x < W; ++x) kk[x] = *(const LS f32x4*)ka[x];
    }
#pragma unroll
    for (int x = 0; x < W; ++x) {
      if (x0 + x >= gpp) kk[x] = f32x4{0.f, 0.f, 0.f, 0.f};
      a = fmaf(kk[x].x, qq[x].x, a);
      a = fmaf(kk[x].y, qq[x].y, a);
      a = fmaf(kk[x].z, qq[x].z, a);
      a = fmaf(kk[x].w, qq[x].w, a);
    }
  }
  return a;
}
// steps of four groups (eight would hold 64 more registers in the 4-bit decode kernel, which has none
// to spare)
template <bool KSTAGE>
__device__ __forceinline__ float qk_part(const LS float* kr, const LS float* qr, int jj, int part, int gpp) {
  return qk_part_w<KSTAGE, 4>(kr, qr, jj, part, gpp);
}
// qk_part for a compact key row (binary16, or int8 codes with the scale row sr): the four values of
// a group converted as kv_groups4 converts them, in qk_part's order and steps
// element d of four compact rows r[0..3] (scale rows sr for int8), converted as kv_groups4 converts
template <int KVT>
__device__ __forceinline__ void kv_col4(const LS char* const (&r)[4], const LS float* const (&sr)[4], int d,
                                        float (&o)[4]) {
  if (KVT == MK_KV_F16) {
    u32 h[4];
    asm volatile(
        "ds_read_u16 %0, %4\n\tds_read_u16 %1, %5\n\tds_read_u16 %2, %6\n\tds_read_u16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3])
        : "v"(lds_addr(r[0] + 2 * d)), "v"(lds_addr(r[1] + 2 * d)), "v"(lds_addr(r[2] + 2 * d)),
          "v"(lds_addr(r[3] + 2 * d))
        : "memory");
#pragma unroll
    for (int x = 0; x < 4; ++x) o[x] = half_bits_f32(h[x]);
  } else {
    u32 c[4], f[4];
    const int b = d / MK_KV_Q8_BLOCK;
    asm volatile(
        "ds_read_i8 %0, %8\n\tds_read_i8 %1, %9\n\tds_read_i8 %2, %10\n\tds_read_i8 %3, %11\n\t"
        "ds_read_b32 %4, %12\n\tds_read_b32 %5, %13\n\tds_read_b32 %6, %14\n\tds_read_b32 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3]), "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
        : "v"(lds_addr(r[0] + d)), "v"(lds_addr(r[1] + d)), "v"(lds_addr(r[2] + d)), "v"(lds_addr(r[3] + d)),
          "v"(lds_addr(sr[0] + b)), "v"(lds_addr(sr[1] + b)), "v"(lds_addr(sr[2] + b)), "v"(lds_addr(sr[3] + b))
        : "memory");
#pragma unroll
    for (int x = 0; x < 4; ++x) o[x] = (float)(int)c[x] * __uint_as_float(f[x]);
  }
}
template <int KVT>
__device__ __forceinline__ float qk_part_c(const LS char* kr, const LS float* sr, const LS float* qr, int jj, int part,
                                           int gpp) {
  const int g0 = part * gpp, start = jj % gpp;
  float a = 0.f;
  for (int x0 = 0; x0 < gpp; x0 += 4) {
    f32x4 kk[4], qq[4];
    int gi[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      int gg = x0 + x + start;
      gg = gg >= gpp ? gg - gpp : gg;
      const bool in = x0 + x < gpp;
      gi[x] = g0 + (in ? gg : 0);
      qq[x] = in ? *(const LS f32x4*)(qr + 4 * gi[x]) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    kv_groups4<KVT>(kr, sr, gi, kk);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      if (x0 + x >= gpp) kk[x] = f32x4{0.f, 0.f, 0.f, 0.f};
      a = fmaf(kk[x].x, qq[x].x, a);
      a = fmaf(kk[x].y, qq[x].y, a);
      a = fmaf(kk[x].z, qq[x].z, a);
      a = fmaf(kk[x].w, qq[x].w, a);
    }
  }
  return a;
}
// the same part for two query rows against one key row (loaded once)
template <int W>
__device__ __forceinline__ void qk_part2_w(const LS float* kr, const LS float* qr0, const LS float* qr1, int jj,
                                           int part, int gpp, float& a0, float& a1) {
  const int g0 = part * gpp, start = jj % gpp;
  a0 = 0.f;
  a1 = 0.f;
  for (int x0 = 0; x0 < gpp; x0 += W) {
    f32x4 kk[W], q0[W], q1[W];
#pragma unroll
    for (int x = 0; x < W; ++x) {
      int gg = x0 + x + start;
      gg = gg >= gpp ? gg - gpp : gg;
      const int dd = (g0 + gg) * 4;
      kk[x] = f32x4{0.f, 0.f, 0.f, 0.f};
      q0[x] = kk[x];
      q1[x] = kk[x];
      if (x0 + x < gpp) {
        kk[x] = *(const LS f32x4*)(kr + dd);
        q0[x] = *(const LS f32x4*)(qr0 + dd);
        q1[x] = *(const LS f32x4*)(qr1 + dd);
      }
    }
#pragma unroll
    for (int x = 0; x < W; ++x) {
      a0 = fmaf(kk[x].x, q0[x].x, a0);
      a1 = fmaf(kk[x].x, q1[x].x, a1);
      a0 = fmaf(kk[x].y, q0[x].y, a0);
      a1 = fmaf(kk[x].y, q1[x].y, a1);
      a0 = fmaf(kk[x].z, q0[x].z, a0);
      a1 = fmaf(kk[x].z, q1[x].z, a1);
      a0 = fmaf(kk[x].w, q0[x].w, a0);
      a1 = fmaf(kk[x].w, q1[x].w, a1);
    }
  }
}
// Steps of eight groups where the part is a whole number of them (the same products in the same
// order as four-group steps), else of four (so the padding products of a part, if any, are qk_part's)
__device__ __forceinline__ void qk_part2(const LS float* kr, const LS float* qr0, const LS float* qr1, int jj, int part,
                                         int gpp, float& a0, float& a1) {
  if (gpp % 8 == 0) qk_part2_w<8>(kr, qr0, qr1, jj, part, gpp, a0, a1);
  else qk_part2_w<4>(kr, qr0, qr1, jj, part, gpp, a0, a1);
}
// parts part and part + 1 of q0 . k and q1 . k at once (four chains; a step's loads of both parts are
// in flight together): a = {part: q0, q1; part + 1: q0, q1}, each chain in qk_part's order
__device__ __forceinline__ void qk_parts2x2(const LS float* kr, const LS float* qr0, const LS float* qr1, int jj,
                                            int part, int gpp, float (&a)[4]) {
  const int start = jj % gpp;
#pragma unroll
  for (int c = 0; c < 4; ++c) a[c] = 0.f;
  for (int x0 = 0; x0 < gpp; x0 += 4) {
    f32x4 kk[2][4], q0[2][4], q1[2][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int g0 = (part + hf) * gpp;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        int gg = x0 + x + start;
        gg = gg >= gpp ? gg - gpp : gg;
        const int dd = (g0 + gg) * 4;
        kk[hf][x] = f32x4{0.f, 0.f, 0.f, 0.f};
        q0[hf][x] = kk[hf][x];
        q1[hf][x] = kk[hf][x];
        if (x0 + x < gpp) {
          kk[hf][x] = *(const LS f32x4*)(kr + dd);
          q0[hf][x] = *(const LS f32x4*)(qr0 + dd);
          q1[hf][x] = *(const LS f32x4*)(qr1 + dd);
        }
      }
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float& b0 = a[2 * hf];
        float& b1 = a[2 * hf + 1];
        b0 = fmaf(kk[hf][x].x, q0[hf][x].x, b0);
        b1 = fmaf(kk[hf][x].x, q1[hf][x].x, b1);
        b0 = fmaf(kk[hf][x].y, q0[hf][x].y, b0);
        b1 = fmaf(kk[hf][x].y, q1[hf][x].y, b1);
        b0 = fmaf(kk[hf][x].z, q0[hf][x].z, b0);
        b1 = fmaf(kk[hf][x].z, q1[hf][x].z, b1);
        b0 = fmaf(kk[hf][x].w, q0[hf][x].w, b0);
        b1 = fmaf(kk[hf][x].w, q1[hf][x].w, b1);
      }
  }
}
template <int NP>
__device__ __forceinline__ float part_tree(const LS float* p, int stride) {
  float v[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) v[i] = p[i * stride];
#pragma unroll
  for (int w = 1; w < NP; w *= 2)
#pragma unroll
    for (int i = 0; i + w < NP; i += 2 * w) v[i] += v[i + w];
  return v[0];
}
// p[0] + p[stride] + ... + p[(np - 1) stride] in the pairwise tree: (0 + 1), (2 + 3), ..., then
// (01 + 23), ..., up to the two halves
__device__ __forceinline__ float att_part_sum(const LS float* p, int stride, int np) {
  switch (np) {
    case 1: return p[0];
    case 2: return part_tree<2>(p, stride);
    case 4: return part_tree<4>(p, stride);
    case 8: return part_tree<8>(p, stride);
    case 16: return part_tree<16>(p, stride);
    default: return part_tree<32>(p, stride);
  }
}

__device__ __forceinline__ int att_items_count(const MkDecodeParams& p, int pos) {
  const int nch = (pos + ATT_C) / ATT_C;
  return ((nch + p.att_cpi - 1) / p.att_cpi) * p.nkv;
}
// chunk-level index (chunk * nkv + g) of chunk k of workgroup w's sequence (its items in order,
// each item's chunks in order); -1 past the end
__device__ __forceinline__ int att_chunk_at(const MkDecodeParams& p, int NW, int w, int pos, int k) {
  const int items = att_items_count(p, pos);
  const int nch = (pos + ATT_C) / ATT_C;
  for (int it = w; it < items; it += NW) {
    const int blk = it / p.nkv, g = it - blk * p.nkv;
    const int c0 = blk * p.att_cpi, n = min(nch, c0 + p.att_cpi) - c0;
    if (k < n) return (c0 + k) * p.nkv + g;
    k -= n;
  }
  return -1;
}
__device__ __forceinline__ bool att_items(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx, const Lds& s,
                                          int NW, int w, int pos, int wait_first, Tracer& tr) {
  const int hd = p.hd, nkv = p.nkv, gs = p.nq / p.nkv, cpi = p.att_cpi;
  const int Lpos = pos + 1;
  const int nch = (Lpos + ATT_C - 1) / ATT_C;
  const int items = att_items_count(p, pos);
  const float scale = 1.0f / sqrtf((float)hd);
  const int lpp = hd >> 2, pps = 64 / lpp, ks = kv_slots(hd);
  const int kvt = p.kvt;
  const int nb = kv_nbuf(hd, kvt, s.a_slots);
  const int kvb = kv_buf_slots(hd, kvt);
  int cnt0 = 0, cnt1 = 0, cnt2 = 0;  // copies this wave issued for the chunk in buffers 0, 1, 2
  LS float* qv = s.att;                // [gs][hd]
  LS float* kpos = qv + gs * hd;       // [hd]
  LS float* vpos = kpos + hd;          // [hd]
  LS float* pb = vpos + hd;            // [gs][16] probabilities (unnormalised)
  LS float* ml = pb + gs * ATT_C;      // [gs][2] this chunk's max and sum
  LS float* racc = ml + 2 * gs;        // [gs][hd] running acc of the item
  LS float* rml = racc + gs * hd;      // [2 (chunk parity)][gs][2] running max and sum
  const int np = att_parts(gs, hd), gpp = (hd >> 2) / np;
  LS float* sp = s.vec;                // [np][gs][16] partial scores
  const MK_G mk_u64* llq = L.ll_in;
  const MK_G mk_u64* llk = L.ll_in + p.nq * hd;
  const MK_G mk_u64* llv = llk + nkv * hd;
  (void)lpp;
  int gq = -1;  // KV head whose queries are in qv
  int k = 0;    // chunk sequence number in this workgroup (stage buffer)
  for (int it = w; it < items; it += NW) {
    const int blk = it / nkv, g = it - blk * nkv;
    const int c0 = blk * cpi, c1 = min(nch, c0 + cpi);
    for (int c = c0; c < c1; ++c, ++k) {
      const int j0 = c * ATT_C, nj = min(Lpos, j0 + ATT_C) - j0;
      const bool has_pos = j0 + nj == Lpos;
      const LS float* stf = (const LS float*)(s.stA + (k % nb) * kvb * SLOT);  // FP32 rows
      const KvCompact kc = kv_compact(hd, kvt, s.stA + (k % nb) * kvb * SLOT);  // compact rows
      int pending = 0;  // copies issued after this chunk's that may stay outstanding
      if (k > 0 || nb > 1) {
        const int kn = k + nb - 1, bn = kn % nb;
        const int cn = att_chunk_at(p, NW, w, pos, kn);
        const int nc = cn >= 0 ? kv_stage(p, L, cn, pos, s.stA + bn * kvb * SLOT) : 0;
        if (bn == 0) cnt0 = nc;
        else if (bn == 1) cnt1 = nc;
        else cnt2 = nc;
        for (int j = 1; j < nb; ++j) {
          const int b = (k + j) % nb;
          pending += b == 0 ? cnt0 : (b == 1 ? cnt1 : cnt2);
        }
      }
      const bool need_q = g != gq;
      gq = g;
      const int qoff = need_q ? 0 : gs * hd;  // records skipped
      const int n = gs * hd + (has_pos ? 2 * hd : 0) - qoff;
      const bool ok = gather_map(cx, n, [=](int f) {
        f += qoff;
        if (f < gs * hd) return llq + g * gs * hd + f;
        if (f < gs * hd + hd) return llk + g * hd + (f - gs * hd);
        return llv + g * hd + (f - gs * hd - hd);
      }, [=](int f, float v) { s.att[f + qoff] = v; });
      tr.mark();
      if (streamer()) {
        if (k == 0) wait_vm_n(wait_first);
        else wait_vm_n(pending);
      }
      tr.mark();
      if (wg_bar_or(s, !ok)) return false;
      if (kvt != MK_KV_F32 && has_pos) kv_round_append(p, L, kpos, vpos, 1, pb, g, pos);  // barriers inside
      tr.mark();
      // scores: the key-dimension parts of every (query head, slot) dot product by their own
      // threads, into the vector region (free while the items run), then added in the fixed tree
      {
        const int rows = gs * ATT_C;
        for (int task = tid(); task < np * rows; task += MK_NT) {
          const int part = task / rows, r = task - part * rows;
          const int i = r >> 4, jj = r & 15;
          if (jj < nj) {
            if (kvt == MK_KV_F32 || j0 + jj == pos) {
              const LS float* kr = j0 + jj == pos ? kpos : stf + (jj / pps) * 256 + (jj % pps) * hd;
              sp[task] = qk_part<true>(kr, qv + i * hd, jj, part, gpp);
            } else if (kvt == MK_KV_F16) {
              sp[task] = qk_part_c<MK_KV_F16>(kc.row(0, jj), nullptr, qv + i * hd, jj, part, gpp);
            } else {
              sp[task] = qk_part_c<MK_KV_Q8>(kc.row(0, jj), kc.scales(0, jj), qv + i * hd, jj, part, gpp);
            }
          }
        }
      }
      wg_bar();
      // softmax numerators, row max and sum (whole rows of 16 lanes take part in the DPP)
      const int t = tid();
      if (t < gs * ATT_C) {
        const int i = t >> 4, jj = t & 15;
        const bool valid = jj < nj;
        const float sc = valid ? att_part_sum(sp + t, gs * ATT_C, np) * scale : -INFINITY;
        const float m = row_max16(sc);
        const float e = valid ? expf(sc - m) : 0.f;
        const float l = row_sum16(e);
        pb[i * ATT_C + jj] = e;
        if (jj == 0) {
          ml[2 * i] = m;
          ml[2 * i + 1] = l;
        }
      }
      tr.mark();
      wg_bar();
      tr.mark();
      {
        // P.V by all eight waves, one (query head, dimension) output per thread and pass
        const bool first = c == c0, last = c + 1 == c1;
        const LS float* rin = rml + (k & 1) * 2 * gs;       // running (max, sum) before this chunk
        LS float* rout = rml + ((k + 1) & 1) * 2 * gs;      // ... and after it
        MK_G mk_u64* part = L.ll_part + (size_t)it * gs * (hd + 2);
        for (int o = tid(); o < gs * hd; o += MK_NT) {
          const int i = o / hd, d = o - i * hd;
          float pv[ATT_C], vv[ATT_C];
          const LS float* va[ATT_C];
#pragma unroll
          for (int jj = 0; jj < ATT_C; ++jj) {
            pv[jj] = pb[i * ATT_C + jj];  // zero beyond nj
            va[jj] = (jj < nj && j0 + jj != pos) ? stf + (ks + jj / pps) * 256 + (jj % pps) * hd + d : vpos + d;
          }
#pragma unroll
          for (int q4 = 0; q4 < ATT_C; q4 += 4) {
            float t4[4];
            if (kvt == MK_KV_F32) {
              stage_f32x4(va[q4], va[q4 + 1], va[q4 + 2], va[q4 + 3], t4);
            } else {
              // column d of four compact V rows (the slot of position pos, not staged, takes vpos)
              const LS char* vr[4] = {kc.row(1, q4), kc.row(1, q4 + 1), kc.row(1, q4 + 2), kc.row(1, q4 + 3)};
              const LS float* vs[4] = {kc.scales(1, q4), kc.scales(1, q4 + 1), kc.scales(1, q4 + 2),
                                       kc.scales(1, q4 + 3)};
              if (kvt == MK_KV_F16) kv_col4<MK_KV_F16>(vr, vs, d, t4);
              else kv_col4<MK_KV_Q8>(vr, vs, d, t4);
#pragma unroll
              for (int x = 0; x < 4; ++x)
                if (j0 + q4 + x == pos) t4[x] = vpos[d];
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) vv[q4 + x] = q4 + x < nj ? t4[x] : 0.f;
          }
          float a = 0.f;
#pragma unroll
          for (int jj = 0; jj < ATT_C; ++jj) a = fmaf(pv[jj], vv[jj], a);
          float M = ml[2 * i], S = ml[2 * i + 1];
          if (!first) {
            const float Mr = rin[2 * i], Sr = rin[2 * i + 1];
            const float Mn = fmaxf(Mr, M);
            const float f = expf(Mr - Mn), f1 = expf(M - Mn);
            a = fmaf(racc[o], f, a * f1);
            S = fmaf(Sr, f, S * f1);
            M = Mn;
          }
          if (last) {
            ll_put(part + i * (hd + 2) + 2 + d, cx.epoch, a);
            if (d == 0) {
              ll_put(part + i * (hd + 2), cx.epoch, M);
              ll_put(part + i * (hd + 2) + 1, cx.epoch, S);
            }
          } else {
            racc[o] = a;
            if (d == 0) {
              rout[2 * i] = M;
              rout[2 * i + 1] = S;
            }
          }
        }
      }
      wg_bar();  // LDS and the KV slots are reused by the next chunk
    }
  }
  if (w >= items && streamer()) wait_vm_n(wait_first);
  return true;
}

// Copies kv_stage issues for chunk-level index it in this wave (the same count, nothing issued).
__device__ __forceinline__ int kv_stage_count(const MkDecodeParams& p, int it, int pos) {
  if (!streamer()) return 0;
  const int kvt = p.kvt;
  const int rb = kv_rowbytes(p.hd, kvt), lpp = rb >> 4, pps = 64 / lpp, ks = kv_slots(p.hd, kvt);
  const int c = it / p.nkv;
  const int j0 = c * ATT_C, jend = min(pos, j0 + ATT_C);
  int cnt = 0;
  for (int q = wave(); q < 2 * ks; q += NCW) {
    const int sl = q >= ks ? q - ks : q;
    if (j0 + sl * pps < jend) ++cnt;
  }
  if (kvt == MK_KV_Q8 && wave() == (2 * ks) % NCW && j0 < jend) ++cnt;
  return cnt;
}

// ---- multi-chunk passes (compact KV caches)
// The items, chunks and per-output arithmetic of att_items, with up to B consecutive chunks of an
// item per pass: the chunks of the next pass are copied while this one is used (2 B chunk buffers
// in stage A, chunk k of the workgroup's sequence in buffer k % 2B), and each step -- scores,
// softmax rows, P.V -- covers the pass's chunks in one sweep.  The thread that owns an output takes
// the pass's chunk merges in chunk order in registers, with the formulas of att_items, so the
// results are bitwise those of att_items (and of the verify kernels).  A pass has four workgroup
// barriers where B single chunks have 4 B: at long contexts the barriers and LDS round trips of
// each chunk, not its bytes, set the time of a chunk.  The caller has issued the copies of
// sequence numbers 0 .. B - 1; a workgroup without items waits until at most wait_first of its
// copies are outstanding.
template <int B>
__device__ __forceinline__ bool att_items_multi(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx,
                                                const Lds& s, int NW, int w, int pos, int wait_first, Tracer& tr) {
  constexpr int NBUF = 2 * B;
  const int hd = p.hd, nkv = p.nkv, gs = p.nq / p.nkv, cpi = p.att_cpi;
  const int Lpos = pos + 1;
  const int nch = (Lpos + ATT_C - 1) / ATT_C;
  const int items = att_items_count(p, pos);
  const float scale = 1.0f / sqrtf((float)hd);
  const int kvt = p.kvt;
  const int kvb = kv_buf_slots(hd, kvt);
  const int rows = gs * ATT_C;
  LS float* qv = s.att;                 // [gs][hd]
  LS float* kpos = qv + gs * hd;        // [hd]
  LS float* vpos = kpos + hd;           // [hd]
  LS float* pb = vpos + hd;             // [B][gs][16] probabilities (unnormalised)
  LS float* ml = pb + B * rows;         // [B][gs][2] each chunk's max and sum
  LS float* racc = ml + 2 * B * gs;     // [gs][hd] running acc of the item
  LS float* rml = racc + gs * hd;       // [2 (pass parity)][gs][2] running max and sum
  const int np = att_parts(gs, hd), gpp = (hd >> 2) / np;
  LS float* sp = s.vec;                 // [B][np][gs][16] partial scores
  const MK_G mk_u64* llq = L.ll_in;
  const MK_G mk_u64* llk = L.ll_in + p.nq * hd;
  const MK_G mk_u64* llv = llk + nkv * hd;
  int gq = -1;      // KV head whose queries are in qv
  int k = 0;        // sequence number of the pass's first chunk
  int issued = B;   // sequence numbers whose copies have been issued
  int par = 0;      // pass parity of the running (max, sum)
  for (int it = w; it < items; it += NW) {
    const int blk = it / nkv, g = it - blk * nkv;
    const int c0 = blk * cpi, c1 = min(nch, c0 + cpi);
    for (int cp = c0, nP = 0; cp < c1; cp += nP, k += nP, par ^= 1) {
      nP = min(B, c1 - cp);  // chunks of this pass: cp .. cp + nP - 1 (sequence numbers k ..)
      // the next B chunks of the sequence -> their buffers (last used two passes ago); then wait
      // until only copies of chunks after this pass may remain
      int pending = 0;
      for (; issued < k + nP + B; ++issued) {
        const int cn = att_chunk_at(p, NW, w, pos, issued);
        if (cn < 0) break;
        kv_stage(p, L, cn, pos, s.stA + (issued % NBUF) * kvb * SLOT);
      }
      // (sequence numbers past the workgroup's last chunk were never issued: the caller's first B
      // may run past it)
      for (int q = k + nP; q < issued; ++q) {
        const int cn = att_chunk_at(p, NW, w, pos, q);
        if (cn < 0) break;
        pending += kv_stage_count(p, cn, pos);
      }
      const bool has_pos = cp + nP == nch;  // the last chunk of the pass holds position pos
      const bool need_q = g != gq;
      gq = g;
      const int qoff = need_q ? 0 : gs * hd;  // records skipped
      const int n = gs * hd + (has_pos ? 2 * hd : 0) - qoff;
      const bool ok = gather_map(cx, n, [=](int f) {
        f += qoff;
        if (f < gs * hd) return llq + g * gs * hd + f;
        if (f < gs * hd + hd) return llk + g * hd + (f - gs * hd);
        return llv + g * hd + (f - gs * hd - hd);
      }, [=](int f, float v) { s.att[f + qoff] = v; });
      tr.mark();
      // (the copies of the pass's chunks, and everything this wave issued before them, such as
      // the caller's out-projection units, are older than the `pending` most recent ones)
      if (streamer()) wait_vm_n(pending);
      tr.mark();
      if (wg_bar_or(s, !ok)) return false;
      if (has_pos) kv_round_append(p, L, kpos, vpos, 1, pb, g, pos);  // barriers inside
      tr.mark();
      // scores of every chunk of the pass, in key-dimension parts
      for (int task = tid(); task < nP * np * rows; task += MK_NT) {
        const int b = task / (np * rows), pr = task - b * (np * rows);
        const int part = pr / rows, r = pr - part * rows;
        const int i = r >> 4, jj = r & 15;
        const int j0 = (cp + b) * ATT_C, nj = min(Lpos, j0 + ATT_C) - j0;
        if (jj < nj) {
          const KvCompact kc = kv_compact(hd, kvt, s.stA + ((k + b) % NBUF) * kvb * SLOT);
          if (j0 + jj == pos) {
            sp[task] = qk_part<true>(kpos, qv + i * hd, jj, part, gpp);
          } else if (kvt == MK_KV_F16) {
            sp[task] = qk_part_c<MK_KV_F16>(kc.row(0, jj), nullptr, qv + i * hd, jj, part, gpp);
          } else {
            sp[task] = qk_part_c<MK_KV_Q8>(kc.row(0, jj), kc.scales(0, jj), qv + i * hd, jj, part, gpp);
          }
        }
      }
      wg_bar();
      // softmax numerators, row max and sum of every chunk (whole rows of 16 lanes in the DPP)
      for (int t = tid(); t < nP * rows; t += MK_NT) {
        const int b = t / rows, r = t - b * rows;
        const int i = r >> 4, jj = r & 15;
        const int j0 = (cp + b) * ATT_C, nj = min(Lpos, j0 + ATT_C) - j0;
        const bool valid = jj < nj;
        const float sc = valid ? att_part_sum(sp + b * np * rows + r, rows, np) * scale : -INFINITY;
        const float m = row_max16(sc);
        const float e = valid ? expf(sc - m) : 0.f;
        const float l = row_sum16(e);
        pb[b * rows + i * ATT_C + jj] = e;
        if (jj == 0) {
          ml[2 * (b * gs + i)] = m;
          ml[2 * (b * gs + i) + 1] = l;
        }
      }
      tr.mark();
      wg_bar();
      tr.mark();
      {
        // P.V of each chunk and the running merge in chunk order, one (query head, dimension)
        // output per thread and pass
        const bool last_pass = cp + nP == c1;
        const LS float* rin = rml + par * 2 * gs;        // running (max, sum) before this pass
        LS float* rout = rml + (par ^ 1) * 2 * gs;       // ... and after it
        MK_G mk_u64* part = L.ll_part + (size_t)it * gs * (hd + 2);
        for (int o = tid(); o < gs * hd; o += MK_NT) {
          const int i = o / hd, d = o - i * hd;
          float A = 0.f, M = 0.f, S = 0.f;
          if (cp > c0) {
            A = racc[o];
            M = rin[2 * i];
            S = rin[2 * i + 1];
          }
          for (int b = 0; b < nP; ++b) {
            const int c = cp + b, j0 = c * ATT_C, nj = min(Lpos, j0 + ATT_C) - j0;
            const KvCompact kc = kv_compact(hd, kvt, s.stA + ((k + b) % NBUF) * kvb * SLOT);
            float pv[ATT_C], vv[ATT_C];
#pragma unroll
            for (int jj = 0; jj < ATT_C; ++jj) pv[jj] = pb[b * rows + i * ATT_C + jj];  // zero beyond nj
#pragma unroll
            for (int q4 = 0; q4 < ATT_C; q4 += 4) {
              float t4[4];
              // column d of four compact V rows (the slot of position pos, not staged, takes vpos)
              const LS char* vr[4] = {kc.row(1, q4), kc.row(1, q4 + 1), kc.row(1, q4 + 2), kc.row(1, q4 + 3)};
              const LS float* vs[4] = {kc.scales(1, q4), kc.scales(1, q4 + 1), kc.scales(1, q4 + 2),
                                       kc.scales(1, q4 + 3)};
              if (kvt == MK_KV_F16) kv_col4<MK_KV_F16>(vr, vs, d, t4);
              else kv_col4<MK_KV_Q8>(vr, vs, d, t4);
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                if (j0 + q4 + x == pos) t4[x] = vpos[d];
                vv[q4 + x] = q4 + x < nj ? t4[x] : 0.f;
              }
            }
            float a = 0.f;
#pragma unroll
            for (int jj = 0; jj < ATT_C; ++jj) a = fmaf(pv[jj], vv[jj], a);
            float Mc = ml[2 * (b * gs + i)], Sc = ml[2 * (b * gs + i) + 1];
            if (c > c0) {
              const float Mn = fmaxf(M, Mc);
              const float f = expf(M - Mn), f1 = expf(Mc - Mn);
              a = fmaf(A, f, a * f1);
              Sc = fmaf(S, f, Sc * f1);
              Mc = Mn;
            }
            A = a;
            M = Mc;
            S = Sc;
          }
          if (last_pass) {
            ll_put(part + i * (hd + 2) + 2 + d, cx.epoch, A);
            if (d == 0) {
              ll_put(part + i * (hd + 2), cx.epoch, M);
              ll_put(part + i * (hd + 2) + 1, cx.epoch, S);
            }
          } else {
            racc[o] = A;
            if (d == 0) {
              rout[2 * i] = M;
              rout[2 * i + 1] = S;
            }
          }
        }
      }
      wg_bar();  // LDS and the KV buffers are reused by the next pass
    }
  }
  if (w >= items && streamer()) wait_vm_n(wait_first);
  return true;
}

// log-sum-exp merge (in item order) of the item partials for o[o0..o1) -> records
__device__ __forceinline__ bool att_combine(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx, const Lds& s,
                                            int o0, int o1, int pos) {
  const int hd = p.hd, nkv = p.nkv, gs = p.nq / p.nkv;
  const int nch = att_items_count(p, pos) / nkv;  // items per KV head
  const int nown = o1 - o0;
  if (nown <= 0) return true;
  LS float* stage = s.att;
  const int vpp = max(1, s.att_cap / (3 * nch));  // outputs staged per round
  const MK_G mk_u64* part = L.ll_part;
  for (int v0 = 0; v0 < nown; v0 += vpp) {
    const int vn = min(vpp, nown - v0);
    const int n = vn * nch * 3;
    const bool ok = gather_map(cx, n, [=](int f) {
      const int which = f % 3;
      const int vc = f / 3;
      const int v = vc / nch, c = vc - v * nch;
      const int fo = o0 + v0 + v;
      const int i = fo / hd, d = fo - i * hd;
      const int g = i / gs, il = i - g * gs;
      const MK_G mk_u64* rec = part + ((size_t)(c * nkv + g) * gs + il) * (hd + 2);
      return rec + (which == 2 ? 2 + d : which);
    }, [=](int f, float v) { stage[f] = v; });
    if (wg_bar_or(s, !ok)) return false;
    if (streamer()) {
      // a wave per output: lanes over chunks, then wave reductions (fixed order)
      for (int v = wave(); v < vn; v += NCW) {
        const LS float* base = stage + (size_t)v * nch * 3;
        float M = -INFINITY;
        for (int c = lane(); c < nch; c += 64) M = fmaxf(M, base[3 * c]);
        M = wave_max(M);
        float num = 0.f, den = 0.f;
        for (int c = lane(); c < nch; c += 64) {
          const float e = expf(base[3 * c] - M);
          den = fmaf(e, base[3 * c + 1], den);
          num = fmaf(e, base[3 * c + 2], num);
        }
        num = wave_sum(num);
        den = wave_sum(den);
        if (lane() == 0) ll_put(L.ll_o + o0 + v0 + v, cx.epoch, num / den);
      }
    }
    wg_bar();
  }
  return true;
}

// Argmax over n (value, index) pairs rec[2i], rec[2i+1] (index as float bits) by one wave: the
// largest value, the lowest index among equal values -- a total order, so the winner does not
// depend on how the pairs are split over lanes.  The result is in every lane.
__device__ __forceinline__ void wave_argmax(const LS float* rec, int n, float& b, int& bi) {
  b = -INFINITY;
  bi = 0x7fffffff;
  for (int i = lane(); i < n; i += 64) {
    const float ob = rec[2 * i];
    const int oi = __float_as_int(rec[2 * i + 1]);
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
}

// pair range [p0, p1) of the workgroup over the (R + 1) / 2 row pairs of a matrix
__device__ __forceinline__ void pair_range(int R, int NW, int w, int& p0, int& p1) {
  const int np = (R + 1) / 2;
  p0 = split(np, NW, w);
  p1 = split(np, NW, w + 1);
}

}  // namespace

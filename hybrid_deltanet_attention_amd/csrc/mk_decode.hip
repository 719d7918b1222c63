// Batch-1 decode step of the hybrid Gated-DeltaNet + attention decoder as ONE persistent kernel
// launch on gfx950 (luce-megakernel announcement, page 1: the whole forward in one dispatch, a
// grid-wide sync instead of kernel boundaries, BF16 weights with FP32 accumulation, the DeltaNet
// recurrence in FP32 registers, QKV + RoPE + causal softmax + output projection fused).
//
// Grid: one 512-lane workgroup per compute unit (regular launch; one workgroup fits per CU and the
// grid is no larger than the CU count, so all workgroups are resident together).
//
// Exchanges between phases never use a barrier, a fence or a counter.  A phase publishes its
// outputs as 8-byte records (FP32 value, launch epoch) with device-coherent stores; the next phase
// polls exactly the records it needs until their epoch matches.  Each record is written once per
// launch, so nothing is ever cleared.  Per DeltaNet layer there are five exchanges (in-projection,
// mixer output, residual, FFN hidden, residual), per attention layer six (plus the split-K
// attention partials).
//
// Every phase's first batch of weights (and the DeltaNet state rows or the KV rows an attention
// work item needs) is copied global -> LDS with asynchronous LDS-DMA loads before the workgroup
// starts polling for the phase's inputs, so HBM streaming overlaps the exchange latency.  Every
// wait is bounded: a wait that gives up sets ctl->err and every workgroup leaves the kernel.

#include <hip/hip_runtime.h>
#include "mk_internal.h"

typedef unsigned int u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
// LDS pointers are kept in address space 3 so every access is a ds_* instruction
#if defined(__HIP_DEVICE_COMPILE__)
#define LS __attribute__((address_space(3)))
#else
#define LS
#endif

namespace {

constexpr int PF_A = 8;     // GEMV units per lane in the wave's large LDS stage (8 x 1 KB)
constexpr int PF_B = 4;     // GEMV units per lane in the wave's small LDS stage (4 x 1 KB)
constexpr int PF_REG = 8;   // GEMV units per lane per register batch beyond the stage
constexpr int SR = 4;       // DeltaNet state rows per wave staged in LDS ahead of the update
constexpr int RED_CAP = 4096;
#ifndef MK_POLL_SLEEP
#define MK_POLL_SLEEP 4  // s_sleep units (64 clocks each) between failed poll rounds
#endif  // GEMV unit partials held in LDS per row block

// Compiler-only barrier: loads issued before it stay before it, so a prefetch is really in flight
// during the poll that follows (without it the compiler may sink the loads to their first use).
__device__ __forceinline__ void keep_issued() { asm volatile("" ::: "memory"); }

// Thread / lane indices the compiler cannot treat as loop-invariant: per-lane index and address
// arithmetic is recomputed where it is used instead of being hoisted out of the layer loop and kept
// live (or spilled to scratch, whose reloads would wait behind in-flight prefetches).
__device__ __forceinline__ int tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
__device__ __forceinline__ int lane() { return tid() & 63; }
__device__ __forceinline__ int lane_here() { return tid() & 63; }
__device__ __forceinline__ int wave() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

// contiguous balanced split of n items over parts: part i gets [split(n,parts,i), split(n,parts,i+1))
__device__ __forceinline__ int split(int n, int parts, int i) { return (int)(((long long)n * i) / parts); }

__device__ __forceinline__ void ll_put(MK_G mk_u64* p, u32 epoch, float v) {
  __hip_atomic_store(p, ((mk_u64)epoch << 32) | (mk_u64)__float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ mk_u64 ld_dev(const MK_G mk_u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float bf_lo(u32 w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(u32 w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ u32x4 ldw(const MK_G uint16_t* p) { return __builtin_nontemporal_load((const MK_G u32x4*)p); }

// Asynchronous global -> LDS copies (gfx950 LDS DMA): lane l's BYTES land at dst + l * BYTES, and the
// copy is tracked by vmcnt like a load.  Prefetches use these so that the compiler can neither sink
// nor drop them and no VGPRs are held across the waits that follow.
__device__ __forceinline__ void dma16(const MK_G void* src, LS void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const MK_G void* src, LS void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}
// wait until every vector memory operation of this wave (including LDS DMA) has completed
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 8 BF16 weights . 8 FP32 activations (activations 16-byte aligned)
__device__ __forceinline__ float dot8(u32x4 w, const LS float* x) {
  const float4 a = *(const LS float4*)x;
  const float4 b = *(const LS float4*)(x + 4);
  float acc = bf_lo(w.x) * a.x;
  acc = fmaf(bf_hi(w.x), a.y, acc);
  acc = fmaf(bf_lo(w.y), a.z, acc);
  acc = fmaf(bf_hi(w.y), a.w, acc);
  acc = fmaf(bf_lo(w.z), b.x, acc);
  acc = fmaf(bf_hi(w.z), b.y, acc);
  acc = fmaf(bf_lo(w.w), b.z, acc);
  acc = fmaf(bf_hi(w.w), b.w, acc);
  return acc;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  const int x = __float_as_int(v);
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, false));
}

// Full-wave sum with DPP row operations (quad swaps, row mirrors, row broadcasts); the total lands
// in lane 63 and is broadcast to every lane.  Fixed order, so every call site is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xF>(v);  // row_mirror
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Fixed-order workgroup sum; every thread receives the same value.
__device__ __forceinline__ float block_sum(float v, LS float* scr) {
  v = wave_sum(v);
  if (lane() == 0) scr[wave()] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < MK_NWAVE; ++i) s += scr[i];
  __syncthreads();
  return s;
}

__device__ __forceinline__ void block_sum2(float& a, float& b, LS float* scr) {
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
  MK_G MkCtl* ctl;
  u32 epoch;
};

__device__ __forceinline__ void set_err(const Ctx& cx, u32 code) {
  __hip_atomic_store(&cx.ctl->err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll n exchange words; word f lives at src(f), is complete when ready(word), and then
// use(f, word) consumes it.  Only the poller wave (wave 7) loads: its vector-memory counter holds
// nothing but these polls, so a completed poll is never held back by prefetch traffic issued by
// the compute waves.  Each lane keeps up to PB loads in flight per round.  All threads call it
// (the caller synchronises the workgroup afterwards); false if a wait gave up.
template <typename SrcFn, typename ReadyFn, typename UseFn>
__device__ __forceinline__ bool poll_words(const Ctx& cx, int n, SrcFn src, ReadyFn ready, UseFn use) {
  constexpr int PB = 8;
  bool ok = true;
  if (wave() != MK_NWAVE - 1) return ok;
  for (int base = 0; base < n && ok; base += 64 * PB) {
    u32 pending = 0;
#pragma unroll
    for (int b = 0; b < PB; ++b)
      if (base + b * 64 + lane() < n) pending |= 1u << b;
    u32 spins = 0;
    while (pending) {
      mk_u64 v[PB];
#pragma unroll
      for (int b = 0; b < PB; ++b)
        if ((pending >> b) & 1u) v[b] = ld_dev(src(base + b * 64 + lane()));
#pragma unroll
      for (int b = 0; b < PB; ++b)
        if (((pending >> b) & 1u) && ready(v[b])) {
          use(base + b * 64 + lane(), v[b]);
          pending &= ~(1u << b);
        }
      if (pending) {
        ++spins;
        __builtin_amdgcn_s_sleep(MK_POLL_SLEEP);
        if ((spins & 255u) == 0 &&
            __hip_atomic_load(&cx.ctl->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
          ok = false;
          break;
        }
        if (spins > MK_SPIN_LIMIT) {
          set_err(cx, 1u);
          ok = false;
          break;
        }
      }
    }
  }
  return ok;
}

// Records src(f) -> dst[f] (LDS).
template <typename SrcFn>
__device__ __forceinline__ bool ll_gather(const Ctx& cx, int n, SrcFn src, LS float* dst) {
  const u32 e = cx.epoch;
  return poll_words(cx, n, src, [=](mk_u64 v) { return (u32)(v >> 32) == e; },
                    [=](int f, mk_u64 v) { dst[f] = __uint_as_float((u32)v); });
}

// Contiguous records src[0..n) -> dst[0..n).
__device__ __forceinline__ bool ll_gather_vec(const Ctx& cx, const MK_G mk_u64* src, int n, LS float* dst) {
  return ll_gather(cx, n, [=](int f) { return src + f; }, dst);
}

struct Tracer {
  LS unsigned long long* lbuf;  // timestamps are kept in LDS while the kernel runs ...
  MK_G unsigned long long* buf; // ... and copied here at the end (null: tracing off)
  int n;
  // (wall clock, core clock) pairs, stamped by thread 0
  __device__ __forceinline__ void mark() {
    if (buf) {
      if (threadIdx.x == 0 && 2 * n + 1 < MK_TRACE_EVENTS) {
        lbuf[2 * n] = wall_clock64();
        lbuf[2 * n + 1] = clock64();
      }
      ++n;
    }
  }
  __device__ __forceinline__ void flush() {
    if (buf) {
      __syncthreads();
      const int m = min(2 * n, MK_TRACE_EVENTS);
      for (int i = tid(); i < m; i += MK_NT) buf[i] = lbuf[i];
    }
  }
};

// ------------------------------------------------------------------------ GEMV
// out[r] = W[r] . x for the R rows of a workgroup's slice (row stride K).  Work unit = (row r,
// 512-column segment s), u = r*S + s; compute wave w takes units w, w + 7, ...; lane l covers columns
// [s*512 + 8l, +8) with one 16-byte load.  A unit's partial is reduced over lanes in a fixed DPP
// order and parked in LDS; a row's value is its segment partials added in segment order.  So a
// row's result does not depend on how rows are split over workgroups.  Rows are processed in
// blocks that fit RED_CAP unit partials.  The first `npf` units of a lane come from the wave's LDS
// stage (filled earlier by gemv_stage); the rest stream through registers two batches deep.
struct Gemv {
  const MK_G uint16_t* W;
  int R, K, S, rb;  // rb = rows per block
  __device__ __forceinline__ void init(const MK_G uint16_t* W_, int R_, int K_) {
    W = W_;
    R = R_;
    K = K_;
    S = (K + 511) >> 9;
    rb = max(2, (RED_CAP / S) & ~1);
  }
  // units of this lane in the block starting at row b0
  __device__ __forceinline__ int units(int b0) const {
    const int U = min(rb, R - b0) * S;
    return (wave() < MK_NCW && U > wave()) ? (U - wave() + MK_NCW - 1) / MK_NCW : 0;
  }
  __device__ __forceinline__ const MK_G uint16_t* addr(int b0, int i) const {
    const int u = wave() + MK_NCW * i;
    const int r = u / S, s = u - r * S;
    const int k = s * 512 + lane_here() * 8;
    return k < K ? W + (size_t)(b0 + r) * K + k : nullptr;
  }
};

struct RegBatch {
  u32x4 c[PF_REG];
};

// first npf units of this lane (block 0) -> the wave's LDS stage, 1 KB per unit slot
template <int NPF>
__device__ __forceinline__ void gemv_stage(const Gemv& g, LS u32x4* stage) {
  const int n = g.units(0);  // 0 on the poller wave
#pragma unroll
  for (int b = 0; b < NPF; ++b) {
    const MK_G uint16_t* a = (b < n) ? g.addr(0, b) : nullptr;
    if (a) dma16(a, stage + b * 64);
  }
}

__device__ __forceinline__ void gemv_issue(RegBatch& rb, const Gemv& g, int b0, int i0, int n) {
#pragma unroll
  for (int b = 0; b < PF_REG; ++b) {
    const MK_G uint16_t* a = (i0 + b < n) ? g.addr(b0, i0 + b) : nullptr;
    rb.c[b] = a ? ldw(a) : u32x4{0u, 0u, 0u, 0u};
  }
}

// PAIRS == false: epi(row, value) once per row; PAIRS == true: epi(pair, v_even, v_odd) once per
// row pair (block sizes are even).  Row/pair indices are relative to the slice.
template <int NPF, bool PAIRS, typename Epi>
__device__ __forceinline__ void gemv(const Gemv& g, const LS float* xin, const LS u32x4* stage, LS float* red,
                                     Tracer& tr, Epi epi) {
  wait_vm();
  keep_issued();
  tr.mark();
  for (int b0 = 0; b0 < g.R; b0 += g.rb) {
    const int nr = min(g.rb, g.R - b0);
    const int n = g.units(b0);
    const int first = b0 == 0 ? NPF : 0;
    RegBatch cur;
    if (n > first) gemv_issue(cur, g, b0, first, n);
    keep_issued();
    auto consume = [&](int i, u32x4 wv) {
      const int u = wave() + MK_NCW * i;
      const int r = u / g.S, s = u - r * g.S;
      const int k = s * 512 + lane() * 8;
      const float d = wave_sum(k < g.K ? dot8(wv, xin + k) : 0.f);
      if (lane() == 0) red[u] = d;
    };
    if (b0 == 0) {
#pragma unroll
      for (int b = 0; b < NPF; ++b)
        if (b < n) consume(b, stage[b * 64 + lane()]);
    }
    for (int i0 = first; i0 < n; i0 += PF_REG) {
      RegBatch nxt;
      gemv_issue(nxt, g, b0, i0 + PF_REG, n);
      keep_issued();
#pragma unroll
      for (int b = 0; b < PF_REG; ++b)
        if (i0 + b < n) consume(i0 + b, cur.c[b]);
#pragma unroll
      for (int b = 0; b < PF_REG; ++b) cur.c[b] = nxt.c[b];
    }
    tr.mark();
    __syncthreads();
    tr.mark();
    if (PAIRS) {
      for (int t = tid(); t < nr / 2; t += MK_NT) {
        float v0 = 0.f, v1 = 0.f;
        for (int s = 0; s < g.S; ++s) {
          v0 += red[(2 * t) * g.S + s];
          v1 += red[(2 * t + 1) * g.S + s];
        }
        epi(b0 / 2 + t, v0, v1);
      }
    } else {
      for (int t = tid(); t < nr; t += MK_NT) {
        float v = 0.f;
        for (int s = 0; s < g.S; ++s) v += red[t * g.S + s];
        epi(b0 + t, v, 0.f);
      }
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void rmsnorm_lds(const LS float* x, const MK_G float* __restrict__ gain, LS float* xn, int D,
                                            float eps, LS float* scr) {
  float s = 0.f;
  for (int i = tid(); i < D; i += MK_NT) s += x[i] * x[i];
  s = block_sum(s, scr);
  const float r = 1.0f / sqrtf(s / (float)D + eps);
  for (int i = tid(); i < D; i += MK_NT) xn[i] = x[i] * r * gain[i];
  __syncthreads();
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ __forceinline__ float softplusf_(float z) { return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z))); }

struct Lds {
  LS float* x;     // residual [D]
  LS float* xn;    // normalised residual [D]
  LS float* vec;   // gathered mixer output / FFN hidden, argmax records
  LS float* att;   // gathered DeltaNet inputs, attention scratch, combine staging
  LS float* red;   // GEMV unit partials
  LS float* scr;   // reductions
  LS u32x4* stA;   // this wave's large prefetch stage (8 x 1 KB)
  LS u32x4* stB;   // this wave's small prefetch stage (4 x 1 KB)
};

// ------------------------------------------------------------------------ DeltaNet
// state rows [s0, s1) of this workgroup: compute wave w stages rows s0 + w + 7k (k < SR) in its large
// LDS stage, element e = lane + 64t of row k at float offset (4k + t) * 64 + lane
__device__ __forceinline__ void state_stage(const MkDecodeParams& p, const MkLayerDev& L, int s0, int s1,
                                            LS u32x4* stage) {
  LS float* st = (LS float*)stage;
  if (wave() >= MK_NCW) return;
#pragma unroll
  for (int k = 0; k < SR; ++k) {
    const int row = s0 + wave() + MK_NCW * k;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int e = lane() + 64 * t;
      if (row < s1 && e < p.dk) dma4(L.S + (size_t)row * p.dk + e, st + (4 * k + t) * 64);
    }
  }
}

// gated delta rule on rows [s0, s1) of S; o = S q read after the update -> records
__device__ __forceinline__ bool dn_state(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx, const Lds& s,
                                         int s0, int s1, Tracer& tr) {
  const int H = p.H, dk = p.dk, dv = p.dv;
  if (s0 >= s1) return true;
  const int h0 = s0 / dv, h1 = (s1 - 1) / dv;
  LS float* q = s.att;
  LS float* k = s.att + dk;
  LS float* ab = s.att + 2 * dk;
  LS float* vr = s.att + 2 * dk + 2;
  const MK_G mk_u64* in = L.ll_in;
  const int off_k = H * dk, off_v = 2 * H * dk, off_a = 2 * H * dk + H * dv, off_b = off_a + H;
  for (int h = h0; h <= h1; ++h) {
    const int i0 = max(s0, h * dv) - h * dv, i1 = min(s1, (h + 1) * dv) - h * dv;
    const int nv = i1 - i0;
    const int n = 2 * dk + 2 + nv;
    const bool ok = ll_gather(cx, n, [=](int f) {
      if (f < dk) return in + h * dk + f;
      if (f < 2 * dk) return in + off_k + h * dk + (f - dk);
      if (f == 2 * dk) return in + off_a + h;
      if (f == 2 * dk + 1) return in + off_b + h;
      return in + off_v + h * dv + i0 + (f - 2 * dk - 2);
    }, s.att);
    if (__syncthreads_or(!ok)) return false;
    wait_vm();
    tr.mark();
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
    // rows of head h owned by this compute wave: local index li = row - s0 with li % 7 == wave
    const int lo = h * dv + i0 - s0, hi = h * dv + i1 - s0;
    const LS float* st = (const LS float*)s.stA;
    const int first_li = wave() < MK_NCW ? lo + ((wave() - lo % MK_NCW) + MK_NCW) % MK_NCW : hi;
    for (int li = first_li; li < hi; li += MK_NCW) {
      const int row = s0 + li;
      const int kslot = li / MK_NCW;
      float sr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e = lane() + 64 * t;
        float v = 0.f;
        if (e < dk) v = kslot < SR ? st[(4 * kslot + t) * 64 + lane()] : L.S[(size_t)row * dk + e];
        sr[t] = v;
      }
      float kd = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e = lane() + 64 * t;
        if (e < dk) kd = fmaf(sr[t], k[e] * sk, kd);
      }
      kd = wave_sum(kd);
      const float u = beta * (vr[row - h * dv - i0] - alpha * kd);
      float od = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e = lane() + 64 * t;
        if (e < dk) {
          const float nv2 = fmaf(u, k[e] * sk, alpha * sr[t]);
          L.S[(size_t)row * dk + e] = nv2;
          od = fmaf(nv2, q[e] * sq, od);
        }
      }
      od = wave_sum(od);
      if (lane() == 0) ll_put(L.ll_o + row, cx.epoch, od);
    }
    __syncthreads();
  }
  return true;
}

// ------------------------------------------------------------------------ attention
// q/k/v rows in RoPE pair order: rotate q and k at position pos, append k and v to the cache
__device__ __forceinline__ void att_qkv(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx, const Lds& s,
                                        const Gemv& g, int P0, int pos, Tracer& tr) {
  const int hd = p.hd, half = hd / 2;
  const MK_G float* cs = p.rope_cos + (size_t)pos * half;
  const MK_G float* sn = p.rope_sin + (size_t)pos * half;
  MK_G mk_u64* llq = L.ll_in;
  MK_G mk_u64* llk = L.ll_in + p.nq * hd;
  MK_G mk_u64* llv = llk + p.nkv * hd;
  const int nqp = p.nq * half, nkp = p.nkv * half;
  gemv<PF_A, true>(g, s.xn, s.stA, s.red, tr, [&](int pl, float x1, float x2) {
    const int P = P0 + pl;
    int sec, hh, m;
    if (P < nqp) {
      sec = 0;
      hh = P / half;
      m = P - hh * half;
    } else if (P < nqp + nkp) {
      sec = 1;
      hh = (P - nqp) / half;
      m = (P - nqp) - hh * half;
    } else {
      sec = 2;
      hh = (P - nqp - nkp) / half;
      m = (P - nqp - nkp) - hh * half;
    }
    float y1 = x1, y2 = x2;
    if (sec < 2) {
      const float c = cs[m], sv = sn[m];
      y1 = x1 * c - x2 * sv;
      y2 = x2 * c + x1 * sv;
    }
    const size_t co = ((size_t)hh * p.max_ctx + pos) * hd + m;
    if (sec == 0) {
      ll_put(llq + hh * hd + m, cx.epoch, y1);
      ll_put(llq + hh * hd + m + half, cx.epoch, y2);
    } else if (sec == 1) {
      ll_put(llk + hh * hd + m, cx.epoch, y1);
      ll_put(llk + hh * hd + m + half, cx.epoch, y2);
      L.Kc[co] = y1;
      L.Kc[co + half] = y2;
    } else {
      ll_put(llv + hh * hd + m, cx.epoch, y1);
      ll_put(llv + hh * hd + m + half, cx.epoch, y2);
      L.Vc[co] = y1;
      L.Vc[co + half] = y2;
    }
  });
}

// K/V rows of one attention work item: a 4-float slice of one position per thread, two passes;
// staged in the wave's large LDS stage, slot 2 * pass + {0: K, 1: V}
constexpr int ATT_PASSES = 3;
struct AttGeo {
  int tpp, ppp;  // threads per position, positions per pass (compute threads only)
  __device__ __forceinline__ void init(int hd) {
    tpp = hd / 4;
    ppp = MK_NCT / tpp;
  }
};

__device__ __forceinline__ void kv_stage(const MkDecodeParams& p, const MkLayerDev& L, const AttGeo& ag, int it,
                                         int pos, LS u32x4* stage) {
  const int Lpos = pos + 1;
  const int c = it / p.nkv, g = it - c * p.nkv;
  const int j0 = c * MK_ATT_CHUNK, j1 = min(Lpos, j0 + MK_ATT_CHUNK);
  const int q4 = tid() % ag.tpp;
#pragma unroll
  for (int ps = 0; ps < ATT_PASSES; ++ps) {
    const int jj = tid() / ag.tpp + ps * ag.ppp;
    const int j = j0 + jj;
    if (tid() < ag.tpp * ag.ppp && j < j1 && j < pos) {
      const size_t off = ((size_t)g * p.max_ctx + j) * p.hd + 4 * q4;
      dma16(L.Kc + off, stage + (2 * ps) * 64);
      dma16(L.Vc + off, stage + (2 * ps + 1) * 64);
    }
  }
}

// split-K partial softmax attention: item = (kv head g, chunk of MK_ATT_CHUNK positions); emits
// (max m, sum l, acc[hd]) per query head of group g
__device__ __forceinline__ bool att_partial(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx,
                                            const Lds& s, int NW, int w, int pos, const AttGeo& ag) {
  const int hd = p.hd, nkv = p.nkv, gs = p.nq / p.nkv, C = MK_ATT_CHUNK;
  const int Lpos = pos + 1;
  const int nch = (Lpos + C - 1) / C;
  const int items = nch * nkv;
  const float scale = 1.0f / sqrtf((float)hd);
  LS float* qv = s.att;                  // [gs][hd]
  LS float* kpos = qv + gs * hd;         // [hd]
  LS float* vpos = kpos + hd;            // [hd]
  LS float* vst = vpos + hd;             // [C][hd]
  LS float* sp = vst + C * hd;           // [gs][C][tpp]
  LS float* sc = sp + gs * C * ag.tpp;   // [gs][C]
  LS float* ml = sc + gs * C;            // [gs][2]
  const MK_G mk_u64* llq = L.ll_in;
  const MK_G mk_u64* llk = L.ll_in + p.nq * hd;
  const MK_G mk_u64* llv = llk + nkv * hd;
  for (int it = w; it < items; it += NW) {
    if (it != w) kv_stage(p, L, ag, it, pos, s.stA);
    keep_issued();
    const int c = it / nkv, g = it - c * nkv;
    const int j0 = c * C, j1 = min(Lpos, j0 + C);
    const int nj = j1 - j0;
    const bool has_pos = (j1 == Lpos);
    const int n = gs * hd + (has_pos ? 2 * hd : 0);
    const bool ok = ll_gather(cx, n, [=](int f) {
      if (f < gs * hd) return llq + g * gs * hd + f;
      if (f < gs * hd + hd) return llk + g * hd + (f - gs * hd);
      return llv + g * hd + (f - gs * hd - hd);
    }, s.att);
    if (__syncthreads_or(!ok)) return false;
    wait_vm();
    // scores: partial dot products over 4 dims per thread, summed over the position's threads in LDS
    const int q4 = tid() % ag.tpp;
#pragma unroll
    for (int ps = 0; ps < ATT_PASSES; ++ps) {
      const int jj = tid() / ag.tpp + ps * ag.ppp;
      if (tid() < ag.tpp * ag.ppp && jj < nj) {
        const int j = j0 + jj;
        float4 kk, vv;
        if (j != pos) {
          const u32x4 kr = s.stA[(2 * ps) * 64 + lane()];
          const u32x4 vr = s.stA[(2 * ps + 1) * 64 + lane()];
          kk = float4{__uint_as_float(kr.x), __uint_as_float(kr.y), __uint_as_float(kr.z), __uint_as_float(kr.w)};
          vv = float4{__uint_as_float(vr.x), __uint_as_float(vr.y), __uint_as_float(vr.z), __uint_as_float(vr.w)};
        } else {
          kk = *(const LS float4*)(kpos + 4 * q4);
          vv = *(const LS float4*)(vpos + 4 * q4);
        }
        *(LS float4*)(vst + jj * hd + 4 * q4) = vv;
        for (int i = 0; i < gs; ++i) {
          const float4 qq = *(const LS float4*)(qv + i * hd + 4 * q4);
          float d = kk.x * qq.x;
          d = fmaf(kk.y, qq.y, d);
          d = fmaf(kk.z, qq.z, d);
          d = fmaf(kk.w, qq.w, d);
          sp[(i * C + jj) * ag.tpp + q4] = d;
        }
      }
    }
    __syncthreads();
    for (int t = tid(); t < gs * nj; t += MK_NT) {
      const int i = t / nj, jj = t - i * nj;
      float d = 0.f;
      for (int u = 0; u < ag.tpp; ++u) d += sp[(i * C + jj) * ag.tpp + u];
      sc[i * C + jj] = d * scale;
    }
    __syncthreads();
    if (tid() < gs) {
      const int i = tid();
      float m = -INFINITY;
      for (int jj = 0; jj < nj; ++jj) m = fmaxf(m, sc[i * C + jj]);
      float l = 0.f;
      for (int jj = 0; jj < nj; ++jj) {
        const float e = expf(sc[i * C + jj] - m);
        sc[i * C + jj] = e;
        l += e;
      }
      ml[2 * i] = m;
      ml[2 * i + 1] = l;
    }
    __syncthreads();
    MK_G mk_u64* part = L.ll_part + (size_t)it * gs * (hd + 2);
    for (int t = tid(); t < gs * hd; t += MK_NT) {
      const int i = t / hd, d = t - i * hd;
      float a = 0.f;
      for (int jj = 0; jj < nj; ++jj) a = fmaf(sc[i * C + jj], vst[jj * hd + d], a);
      ll_put(part + i * (hd + 2) + 2 + d, cx.epoch, a);
    }
    if (tid() < 2 * gs) ll_put(part + (tid() >> 1) * (hd + 2) + (tid() & 1), cx.epoch, ml[tid()]);
    __syncthreads();
  }
  return true;
}

// log-sum-exp merge (in chunk order) of the partials for o[o0..o1) -> records
__device__ __forceinline__ bool att_combine(const MkDecodeParams& p, const MkLayerDev& L, const Ctx& cx, const Lds& s,
                                            int o0, int o1, int pos) {
  const int hd = p.hd, nkv = p.nkv, gs = p.nq / p.nkv;
  const int nch = (pos + MK_ATT_CHUNK) / MK_ATT_CHUNK;
  const int nown = o1 - o0;
  if (nown <= 0) return true;
  LS float* stage = s.att;
  const int cap = 2048;
  const int vpp = max(1, cap / nch);
  const MK_G mk_u64* part = L.ll_part;
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
      const MK_G mk_u64* rec = part + ((size_t)(c * nkv + g) * gs + il) * (hd + 2);
      return rec + (which == 2 ? 2 + d : which);
    }, stage);
    if (__syncthreads_or(!ok)) return false;
    for (int v = tid(); v < vn; v += MK_NT) {
      const LS float* base = stage + (size_t)v * nch * 3;
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

// pair range [p0, p1) of the workgroup over the (R + 1) / 2 row pairs of a matrix
__device__ __forceinline__ void pair_range(int R, int NW, int w, int& p0, int& p1) {
  const int np = (R + 1) / 2;
  p0 = split(np, NW, w);
  p1 = split(np, NW, w + 1);
}

}  // namespace

// ------------------------------------------------------------------------------------------
// the megakernel
// ------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(MK_NT, 1) mk_decode_kernel(MkDecodeParams p) {
  extern __shared__ float lds_raw[];
  LS float* lds = (LS float*)lds_raw;
  const int NW = (int)gridDim.x, w = (int)blockIdx.x;
  Lds s;
  s.x = lds + p.lds_x;
  s.xn = lds + p.lds_xn;
  s.vec = lds + p.lds_vec;
  s.att = lds + p.lds_att;
  s.red = lds + p.lds_red;
  s.scr = lds + p.lds_scr;
  s.stA = (LS u32x4*)(lds + p.lds_stage + min(wave(), MK_NCW - 1) * MK_STAGE_FLOATS_PER_WAVE);
  s.stB = s.stA + PF_A * 64;

  Ctx cx;
  cx.ctl = p.ctl;
  cx.epoch = p.ctl->step;
  const int pos = p.ctl->pos;
  const int tok = p.tok[0];
  // a bad token id or a full context is reported through ctl->err; every workgroup sees the same
  // values, so all of them leave before touching memory
  if (tok < 0 || tok >= p.vocab || pos < 0 || pos >= p.max_ctx) {
    if (w == 0 && tid() == 0) set_err(cx, 2u);
    return;
  }
  Tracer tr{(LS unsigned long long*)(lds + p.lds_trace), p.trace ? p.trace + (size_t)w * MK_TRACE_EVENTS : nullptr, 0};
  tr.mark();
  AttGeo ag;
  ag.init(p.hd);

  // this workgroup's rows of the residual-sized projections (out-projection, down projection)
  const int d0 = split(p.D, NW, w), d1 = split(p.D, NW, w + 1);
  // FFN hidden range (gate/up row pairs)
  const int j0 = split(p.ffn, NW, w), j1 = split(p.ffn, NW, w + 1);

  // layer 0's input rows go out first
  Gemv gin;
  int P0, P1;
  {
    const MkLayerDev L0 = p.layers[0];
    pair_range(L0.rows_in, NW, w, P0, P1);
    gin.init(L0.w_in + (size_t)2 * P0 * p.D, min(2 * P1, L0.rows_in) - 2 * P0, p.D);
    gemv_stage<PF_A>(gin, s.stA);
    keep_issued();
  }
  for (int i = tid(); i < p.D; i += MK_NT) s.x[i] = __uint_as_float((u32)p.embed[(size_t)tok * p.D + i] << 16);
  __syncthreads();

  for (int l = 0; l < p.n_layers; ++l) {
    const MkLayerDev L = p.layers[l];
    rmsnorm_lds(s.x, L.g1, s.xn, p.D, p.rms_eps, s.scr);
    tr.mark();
    int K;  // mixer output width
    Gemv gout, ggu;
    ggu.init(L.w_gu + (size_t)2 * j0 * p.D, 2 * (j1 - j0), p.D);
    if (L.kind == MK_LAYER_DN) {
      K = p.H * p.dv;
      // in-projection rows -> records
      MK_G mk_u64* dst = L.ll_in + 2 * P0;
      gemv<PF_A, false>(gin, s.xn, s.stA, s.red, tr, [&](int r, float v, float) { ll_put(dst + r, cx.epoch, v); });
      tr.mark();
      // state rows and the first out-projection rows go out before q/k/v/a/b are complete
      const int s0 = split(K, NW, w), s1 = split(K, NW, w + 1);
      gout.init(L.w_out + (size_t)d0 * K, d1 - d0, K);
      state_stage(p, L, s0, s1, s.stA);
      gemv_stage<PF_B>(gout, s.stB);
      keep_issued();
      if (!dn_state(p, L, cx, s, s0, s1, tr)) return;
    } else {
      K = p.nq * p.hd;
      att_qkv(p, L, cx, s, gin, P0, pos, tr);
      tr.mark();
      // K/V rows of the first work item and the first out-projection rows go out before q/k/v
      const int items = ((pos + MK_ATT_CHUNK) / MK_ATT_CHUNK) * p.nkv;
      if (w < items) kv_stage(p, L, ag, w, pos, s.stA);
      gout.init(L.w_out + (size_t)d0 * K, d1 - d0, K);
      gemv_stage<PF_B>(gout, s.stB);
      keep_issued();
      if (!att_partial(p, L, cx, s, NW, w, pos, ag)) return;
      tr.mark();
      const int o0 = split(K, NW, w), o1 = split(K, NW, w + 1);
      gemv_stage<PF_A>(ggu, s.stA);
      keep_issued();
      if (!att_combine(p, L, cx, s, o0, o1, pos)) return;
    }
    tr.mark();
    if (L.kind == MK_LAYER_DN) {
      gemv_stage<PF_A>(ggu, s.stA);  // gate/up rows go out before the mixer output is complete
      keep_issued();
    }
    // mixer output -> out-projection rows + residual -> records
    if (__syncthreads_or(!ll_gather_vec(cx, L.ll_o, K, s.vec))) return;
    tr.mark();
    gemv<PF_B, false>(gout, s.vec, s.stB, s.red, tr,
                      [&](int r, float v, float) { ll_put(L.ll_x1 + d0 + r, cx.epoch, s.x[d0 + r] + v); });
    // down-projection rows go out before the residual is complete
    Gemv gdn;
    gdn.init(L.w_down + (size_t)d0 * p.ffn, d1 - d0, p.ffn);
    gemv_stage<PF_B>(gdn, s.stB);
    keep_issued();
    tr.mark();
    if (__syncthreads_or(!ll_gather_vec(cx, L.ll_x1, p.D, s.x))) return;
    tr.mark();
    rmsnorm_lds(s.x, L.g2, s.xn, p.D, p.rms_eps, s.scr);
    tr.mark();
    gemv<PF_A, true>(ggu, s.xn, s.stA, s.red, tr, [&](int j, float gv, float uv) {
      ll_put(L.ll_h + j0 + j, cx.epoch, gv / (1.0f + expf(-gv)) * uv);
    });
    // next layer's input rows (or the LM head's) go out before the FFN hidden is complete
    if (l + 1 < p.n_layers) {
      const MkLayerDev Ln = p.layers[l + 1];
      pair_range(Ln.rows_in, NW, w, P0, P1);
      gin.init(Ln.w_in + (size_t)2 * P0 * p.D, min(2 * P1, Ln.rows_in) - 2 * P0, p.D);
    } else {
      pair_range(p.vocab, NW, w, P0, P1);
      gin.init(p.embed + (size_t)2 * P0 * p.D, min(2 * P1, p.vocab) - 2 * P0, p.D);
    }
    gemv_stage<PF_A>(gin, s.stA);
    keep_issued();
    tr.mark();
    if (__syncthreads_or(!ll_gather_vec(cx, L.ll_h, p.ffn, s.vec))) return;
    tr.mark();
    gemv<PF_B, false>(gdn, s.vec, s.stB, s.red, tr,
                      [&](int r, float v, float) { ll_put(L.ll_x2 + d0 + r, cx.epoch, s.x[d0 + r] + v); });
    tr.mark();
    if (__syncthreads_or(!ll_gather_vec(cx, L.ll_x2, p.D, s.x))) return;
    tr.mark();
  }

  // final norm + tied LM head + argmax (lowest index among equal maxima)
  rmsnorm_lds(s.x, p.g_final, s.xn, p.D, p.rms_eps, s.scr);
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  const int v0 = 2 * P0;
  gemv<PF_A, false>(gin, s.xn, s.stA, s.red, tr, [&](int r, float v, float) {
    const int idx = v0 + r;
    if (p.logits) p.logits[idx] = v;
    if (v > best || (v == best && idx < bidx)) {
      best = v;
      bidx = idx;
    }
  });
  tr.mark();
  // workgroup argmax: fixed tree over lanes (DPP-free shuffles) then waves in order
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
  tr.mark();
  if (w != 0) {
    tr.flush();
    return;
  }
  // workgroup 0 reduces the per-workgroup winners and publishes the token
  __syncthreads();
  const MK_G mk_u64* am = p.ll_am;
  const bool ok = ll_gather(cx, 2 * NW, [=](int f) { return am + f; }, s.vec);
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
  tr.mark();
  tr.flush();
}

// ------------------------------------------------------------------------------------------
// load-time helper kernels
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

__global__ void mk_set_ctl_kernel(MkCtl* ctl, int32_t pos, int reset_err, int bump_step) {
  if (threadIdx.x == 0) {
    if (pos >= 0) ctl->pos = pos;
    if (ctl->step == 0u) ctl->step = 1u;
    if (bump_step) ctl->step += 1u;
    if (reset_err) ctl->err = 0u;
  }
}

extern "C" int mk_launch_decode(const MkDecodeParams* p, int n_wg, void* stream) {
  hipLaunchKernelGGL(mk_decode_kernel, dim3(n_wg), dim3(MK_NT), (size_t)p->lds_floats * 4, (hipStream_t)stream, *p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_launch_permute_rows(const uint16_t* src, uint16_t* dst, const int32_t* d_perm, int64_t rows,
                                      int64_t cols, void* stream) {
  if (rows <= 0) return 0;
  hipLaunchKernelGGL(mk_permute_rows_kernel, dim3((unsigned)rows), dim3(256), 0, (hipStream_t)stream, src, dst, d_perm,
                     rows, cols);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_launch_bf16_to_f32(const uint16_t* src, float* dst, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(mk_bf16_to_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, src,
                     dst, n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_launch_zero(void* dst, int64_t bytes, void* stream) {
  if (bytes <= 0) return 0;
  hipLaunchKernelGGL(mk_zero_kernel, dim3(1024), dim3(256), 0, (hipStream_t)stream, (uint32_t*)dst, bytes / 4);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_launch_set_ctl(MkCtl* ctl, int32_t pos, int reset_err, int bump_step, void* stream) {
  hipLaunchKernelGGL(mk_set_ctl_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, ctl, pos, reset_err, bump_step);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int mk_decode_max_blocks_per_cu(int lds_bytes) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, mk_decode_kernel, MK_NT, lds_bytes) != hipSuccess) return 0;
  return nb;
}

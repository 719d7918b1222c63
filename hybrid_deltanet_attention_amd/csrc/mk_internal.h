// Internal layout shared by the host runtime and the gfx950 kernels.
#pragma once

#include <stdint.h>

typedef unsigned long long mk_u64;

// Device code sees pointers into device memory as global-address-space pointers, so the compiler
// emits global (not flat) memory instructions for them; host code sees plain pointers.  The
// layout is the same either way.  Host-only translation units define MK_HOST_VIEW.
#if defined(__HIP_DEVICE_COMPILE__) && !defined(MK_HOST_VIEW)
#define MK_G __attribute__((address_space(1)))
#else
#define MK_G
#endif

// Threads per workgroup of the persistent decode grid (8 wave64s).  Waves 0..MK_NCW-1 stream: they
// issue every weight / state / KV copy and every store.  The other waves only poll exchange
// records (their vector-memory counter never holds a prefetch, so a completed poll is never held
// back behind one).  All 8 waves compute from LDS.
#define MK_NT 512
#define MK_NWAVE 8
#define MK_NCW 4
#define MK_NCT (MK_NCW * 64)
// Positions per split-K attention work item (one 16-lane DPP row per query head).
#define MK_ATT_CHUNK 16
// chunks per attention pass of the decode kernel for compact KV caches
#define MK_ATT_PASS 3
// 8-byte trace words per workgroup (pairs of wall clock, core clock).
#define MK_TRACE_EVENTS 1024
// Polls of an exchange word before a wait gives up and reports MK_E_DEVICE_TIMEOUT.
#define MK_SPIN_LIMIT (1u << 22)
// LDS prefetch stages, in 1 KB slots: A holds the in-projection / gate-up / LM-head units, B the
// state rows or KV rows plus the out-projection units, or the down-projection units.
#define MK_STAGE_A_SLOTS 56
#define MK_STAGE_B_SLOTS 32
// GEMV unit partials held in LDS per row chunk.
#define MK_RED_CAP 4096
// Prefill split-K partial buffer (floats): 256 work items of 128 x 128 outputs.
#define PF_SPLITK_FLOATS ((size_t)256 * 128 * 128)
// Largest grid the exchange buffers are sized for.
#define MK_MAX_GRID 1024
// Positions one speculative-verify launch scores (the pending token and up to 5 drafts).
#define MK_VERIFY_MAXT 6
// KV cache element types (MkDecodeParams::kvt): rows of head_dim FP32 values; rows of binary16
// values; rows of int8 codes with one FP32 scale per 32 values (value = code * scale) in Ks / Vs.
#define MK_KV_F32 0
#define MK_KV_F16 1
#define MK_KV_Q8 2
// values per int8 KV scale
#define MK_KV_Q8_BLOCK 32
// Bytes of the static exchange-record array behind mk_decode_step_noalloc (mk_noalloc.hip).
#define MK_NOALLOC_SCRATCH_BYTES (16u << 20)

// Device-resident control block (first 256 bytes of the workspace).
struct MkCtl {
  uint32_t step;   // launch epoch stamped into exchange records; starts at 1, never reused
  int32_t pos;     // next position to write
  uint32_t err;    // nonzero once a kernel gave up (1 = wait timeout, 2 = bad input)
  uint32_t pad[61];
};

enum { MK_LAYER_DN = 0, MK_LAYER_ATT = 1 };

// Per-layer device pointers (an array of these lives in the workspace).
struct MkLayerDev {
  int32_t kind;
  int32_t rows_in;               // rows of w_in
  MK_G const uint16_t* w_in;     // DeltaNet: [2*H*dk + H*dv + 2H][D] (q, k, v, a, b rows)
                                 // attention: [(nq + 2*nkv)*hd][D], rows of each head in RoPE pair order
  MK_G const uint16_t* w_out;    // [D][H*dv] or [D][nq*hd]
  MK_G const uint16_t* w_gu;     // [2*ffn][D], gate and up rows interleaved (g0, u0, g1, u1, ...)
  MK_G const uint16_t* w_down;   // [D][ffn]
  MK_G const uint16_t* g12;      // BF16 RMSNorm gains [2][D]: pre-mixer, then pre-FFN
  MK_G float* S;                 // DeltaNet: [H][dv][dk]
  MK_G float* Kc;                // attention: [nkv][max_ctx][hd] elements of the cache type (kvt)
  MK_G float* Vc;                // attention: [nkv][max_ctx][hd] elements of the cache type (kvt)
  MK_G float* Ks;                // int8 cache: scales [nkv][max_ctx][hd / 32] of Kc (else null)
  MK_G float* Vs;                // int8 cache: scales [nkv][max_ctx][hd / 32] of Vc (else null)
  MK_G mk_u64* ll_in;            // records. DeltaNet: [rows_in]; attention: q [nq*hd], k [nkv*hd], v [nkv*hd]
  MK_G mk_u64* ll_part;          // attention partial records [max_items][gs][hd + 2]
  MK_G mk_u64* ll_o;             // mixer outputs [H*dv] or [nq*hd]
  MK_G mk_u64* ll_x1;            // residual after the mixer [D]
  MK_G mk_u64* ll_h;             // FFN hidden [ffn]
  MK_G mk_u64* ll_x2;            // residual after the FFN [D]
  MK_G float* Ssnap;             // verify only: DeltaNet state after position t at Ssnap + t * snap_stride
};

struct MkDecodeParams {
  MK_G const MkLayerDev* layers;
  int32_t n_layers, D, ffn, vocab;
  int32_t H, dk, dv, nq, nkv, hd;
  int32_t max_ctx, max_items;
  int32_t att_cpi;               // 16-position chunks per split-K attention work item
  float rms_eps, l2_eps;
  MK_G const uint16_t* embed;    // [vocab][D]
  MK_G const uint16_t* g_final;  // BF16 final RMSNorm gain [D]
  MK_G const uint16_t* gain0;    // layer 0's gains (its g12)
  MK_G const float* rope_cos;    // [max_ctx][hd/2]
  MK_G const float* rope_sin;    // [max_ctx][hd/2]
  MK_G MkCtl* ctl;
  MK_G mk_u64* ll_am;            // [2 * MK_MAX_GRID] argmax records
  MK_G const int32_t* tok;       // device token to embed
  MK_G int32_t* next;            // device output token
  MK_G float* logits;            // optional [vocab]
  // optional per-workgroup phase timestamps: trace[w * MK_TRACE_EVENTS + 2e] = wall clock (100 MHz),
  // [.. + 2e + 1] = core clock
  MK_G unsigned long long* trace;
  // LDS carve (float offsets) and size
  int32_t lds_desc, lds_gain, lds_rope, lds_x, lds_xn, lds_vec, lds_att, lds_scr, lds_flag, lds_trace;
  int32_t lds_floats;
  // speculative verify (layers then points at the verify descriptors, whose records hold
  // MK_VERIFY_MAXT positions: [t][n] for every record vector of n values)
  int32_t nt;                    // positions scored: the pending token and nt - 1 drafts
  int32_t vec_floats;            // floats of the LDS vector region
  int64_t snap_stride;           // floats between DeltaNet state snapshots of consecutive positions
  MK_G const int32_t* vtok;      // [nt] device tokens
  MK_G int32_t* vout;            // [nt] greedy choice after each position
  MK_G int32_t* vacc;            // accepted drafts
  MK_G mk_u64* ll_acc;           // accepted-count record
  // weight format: 0 = BF16, 1 = Q4G32 (every matrix tiled in 80-byte (4 rows x 32 columns)
  // tiles of codes and (d, m) words; the norm gains stay BF16)
  int32_t wq4;
  // KV cache element type: MK_KV_F32, MK_KV_F16 or MK_KV_Q8
  int32_t kvt;
  // 4-bit verify: floats between the positions of a workgroup's residual rows in LDS
  int32_t rstride;
};

#ifdef __cplusplus
extern "C" {
#endif
// Launchers implemented in the .hip files (host side).
int mk_launch_decode(const MkDecodeParams* p, int n_wg, void* stream);
int mk_launch_verify(const MkDecodeParams* p, int n_wg, void* stream);
int mk_launch_decode_q4(const MkDecodeParams* p, int n_wg, void* stream);
int mk_decode_q4_max_blocks_per_cu(const MkDecodeParams* p, int lds_bytes);
// Q4G32 input layout [R][K] -> the decode kernel's tiled layout (ceil(R/4) * K/32 tiles of 80 bytes)
int mk_launch_q4_tile(const void* src, int64_t R, int64_t K, void* dst, void* stream);
int mk_verify_max_blocks_per_cu(const MkDecodeParams* p, int lds_bytes);
int mk_launch_verify_q4(const MkDecodeParams* p, int n_wg, void* stream);
int mk_verify_q4_max_blocks_per_cu(const MkDecodeParams* p, int lds_bytes);
int mk_launch_permute_rows(const uint16_t* src, uint16_t* dst, const int32_t* d_perm, int64_t rows,
                           int64_t cols, void* stream);
int mk_launch_zero(void* dst, int64_t bytes, void* stream);
int mk_launch_set_ctl(MkCtl* ctl, int32_t pos, int reset_err, int bump_step, void* stream);
int mk_decode_max_blocks_per_cu(const MkDecodeParams* p, int lds_bytes);
// device address of the static exchange-record array (mk_noalloc.hip), looked up once per device
int mk_noalloc_scratch(int device, void** out, const char** err);
// prefill kernels (mk_prefill.hip); all return 0 or -1 (launch error)
int mk_pf_embed(const int32_t* tok, int T, const uint16_t* embed, int D, int vocab, float* X, MkCtl* ctl, void* stream);
int mk_pf_rms_split(const float* X, int T, int D, const uint16_t* g, float eps, uint16_t* Ahi, uint16_t* Alo, int lda,
                    void* stream);
int mk_pf_gemm(int epi, const uint16_t* Ahi, const uint16_t* Alo, int lda, int M, int K, const uint16_t* W, int N,
               float* C, int ldc, uint16_t* Hhi, uint16_t* Hlo, int ldh, float* P, size_t p_floats, void* stream);
// residual GEMM C += A W^T; with g (else NULL) the updated rows are then RMS-normalised into (Nhi, Nlo)
int mk_pf_gemm_res(const uint16_t* Ahi, const uint16_t* Alo, int lda, int M, int K, const uint16_t* W, int N,
                   float* C, int ldc, float* P, size_t p_floats, const uint16_t* g, float eps, uint16_t* Nhi,
                   uint16_t* Nlo, int ldn, void* stream);
// DeltaNet mixer over T prompt tokens from the in-projection Y: normalised q, k (QK) and gates
// (AB, wide keys only) are produced on the way
int mk_pf_dn_scan(float* S, float* QK, float* AB, const float* Y, int ldy, int T, int H, int dk, int dv, float l2eps,
                  uint16_t* Ohi, uint16_t* Olo, int ldo, float* CH, void* stream);
// rotated k and v of the chunk's positions p0 + t -> K/V rows (kv_stride rows per head, row kv_pos0 + t)
int mk_pf_att_rope(const float* Y, int ldy, int T, int p0, int nq, int nkv, int hd, const float* rcos,
                   const float* rsin, float* Q, float* K, float* V, int kv_stride, int kv_pos0, void* stream);
// FP32 rows [nkv][T][hd] -> the compact cache (kvt MK_KV_F16 or MK_KV_Q8) at positions p0 ..
int mk_pf_kv_pack(const float* Kf, const float* Vf, int T, int nkv, int hd, int kvt, void* Kc, void* Vc, float* Ks,
                  float* Vs, int max_ctx, int p0, void* stream);
// causal attention over the cache (element type kvt; Ks / Vs the int8 scales, else NULL)
int mk_pf_attention(const float* Q, const void* Kc, const void* Vc, int kvt, const float* Ks, const float* Vs, int T,
                    int p0, int nq, int nkv, int hd, int max_ctx, uint16_t* Ohi, uint16_t* Olo, int ldo, float* P,
                    size_t p_floats, void* stream);
int mk_pf_lmhead(const float* x, int D, const uint16_t* g, float eps, const uint16_t* E, int vocab, float* logits,
                 float* part, int nwg, void* stream);
int mk_pf_finish(const float* part, int nwg, int32_t* next, MkCtl* ctl, int32_t pos, void* stream);
// 4-bit prefill (mk_prefill_q4.hip): a tiled 4-bit matrix -> rows [W_hi | W_lo] of 2K BF16 values;
// 4-bit embedding rows -> FP32; activations -> [A_hi | A_hi], [A_lo | 0]
int mk_pf_q4_expand(const void* T, int N, int K, uint16_t* Wd, void* stream);
int mk_pf_embed_q4(const int32_t* tok, int T, const void* E, int D, int vocab, float* X, MkCtl* ctl, void* stream);
int mk_pf_widen(uint16_t* Ahi, uint16_t* Alo, int ld, int T, int K, void* stream);
#ifdef __cplusplus
}
#endif

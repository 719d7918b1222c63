// Internal layout shared by the host runtime and the gfx950 kernels.
#pragma once

#include <stdint.h>

typedef unsigned long long mk_u64;

// Threads per workgroup of the persistent decode grid (8 wave64s).
#define MK_NT 512
#define MK_NWAVE 8
// Positions per split-K attention work item.
#define MK_ATT_CHUNK 16
// Polls of an exchange record before a wait gives up and reports MK_E_DEVICE_TIMEOUT.
#define MK_SPIN_LIMIT (1u << 22)

// Device-resident control block (first 256 bytes of the workspace).
struct MkCtl {
  uint32_t step;   // launch epoch stamped into exchange records; starts at 1, never reset
  int32_t pos;     // next position to write
  uint32_t err;    // nonzero once any kernel wait gave up
  uint32_t pad[61];
};

enum { MK_LAYER_DN = 0, MK_LAYER_ATT = 1 };

// Per-layer device pointers (an array of these lives in the workspace).
struct MkLayerDev {
  int32_t kind;
  int32_t kv_index;         // attention layers: index among attention layers
  const uint16_t* w_in;     // DeltaNet: [2*H*dk + H*dv + 2H][D] (q, k, v, a, b rows)
                            // attention: [(nq + 2*nkv)*hd][D], rows of each head in RoPE pair order
  const uint16_t* w_out;    // [D][H*dv] or [D][nq*hd]
  const uint16_t* w_gu;     // [2*ffn][D], gate and up rows interleaved (g0, u0, g1, u1, ...)
  const uint16_t* w_down;   // [D][ffn]
  const float* g1;          // [D]
  const float* g2;          // [D]
  float* S;                 // DeltaNet: [H][dv][dk]
  float* Kc;                // attention: [nkv][max_ctx][hd]
  float* Vc;                // attention: [nkv][max_ctx][hd]
  mk_u64* ll_in;            // DeltaNet: [2*H*dk + H*dv + 2H]; attention: q [nq*hd], k [nkv*hd], v [nkv*hd]
  mk_u64* ll_mid;           // DeltaNet: o [H*dv]; attention: partials [max_items][gs][hd + 2]
  mk_u64* ll_o;             // attention: combined o [nq*hd]
  mk_u64* ll_x1;            // [D] residual after the mixer
  mk_u64* ll_h;             // [ffn]
  mk_u64* ll_x2;            // [D] residual after the FFN
};

struct MkDecodeParams {
  const MkLayerDev* layers;
  int32_t n_layers, D, ffn, vocab;
  int32_t H, dk, dv, nq, nkv, hd;
  int32_t max_ctx, max_items;
  float rms_eps, l2_eps;
  const uint16_t* embed;        // [vocab][D]
  const float* g_final;         // [D]
  const float* rope_cos;        // [max_ctx][hd/2]
  const float* rope_sin;        // [max_ctx][hd/2]
  MkCtl* ctl;
  mk_u64* ll_am;                // [2 * max grid] argmax records
  const int32_t* tok;           // device token to embed
  int32_t* next;                // device output token
  float* logits;                // optional [vocab]
  // LDS carve (float offsets) and sizes
  int32_t lds_x, lds_xn, lds_vec, lds_red, lds_out, lds_scr, lds_floats;
};

#ifdef __cplusplus
extern "C" {
#endif
// Launchers implemented in the .hip files (host side).
int mk_launch_decode(const MkDecodeParams* p, int n_wg, void* stream);
int mk_launch_permute_rows(const uint16_t* src, uint16_t* dst, const int32_t* d_perm, int64_t rows,
                           int64_t cols, void* stream);
int mk_launch_bf16_to_f32(const uint16_t* src, float* dst, int64_t n, void* stream);
int mk_launch_zero(void* dst, int64_t bytes, void* stream);
int mk_launch_set_ctl(MkCtl* ctl, int32_t pos, int reset_err, void* stream);
int mk_decode_lds_bytes(const MkDecodeParams* p);
#ifdef __cplusplus
}
#endif

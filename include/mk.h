/*
 * mk.h -- C ABI of the batch-1 decode megakernel for a hybrid Gated-DeltaNet + full-attention
 * decoder on AMD Instinct MI355X (gfx950).
 *
 * The model is the hybrid the luce-megakernel announcement runs as one kernel launch (page 1:
 * 24 layers, 18 DeltaNet layers with a learned linear recurrence and 6 standard attention
 * layers; BF16 weights with FP32 accumulation; the DeltaNet recurrence kept in FP32 registers;
 * QKV, RoPE, causal softmax and output projection fused; a grid-wide sync in place of kernel
 * boundaries).  Layer l is attention when l % period == attn_slot, DeltaNet otherwise; blocks
 * are pre-norm residual with a SwiGLU FFN, and the input embedding doubles as the LM head.
 *
 * Conventions for every entry point:
 *  - Every call returns an int status (MK_OK == 0, negative on error).  Nothing aborts and no
 *    C++ exception crosses the ABI.  mk_last_error() describes the last failure.
 *  - Pointers named d_* are device pointers (HIP device memory of the ctx's device); pointers
 *    without the prefix are host pointers.  The library keeps no pointer past the call that
 *    received it, except the workspace given to mk_create.
 *  - Prefill, decode and verify are enqueued on the ctx's stream and return without waiting;
 *    their outputs are written to caller-owned device buffers.  mk_sync waits for them.
 *  - A ctx is bound to one device and one stream and is not thread-safe.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mk_ctx mk_ctx;

enum mk_status {
  MK_OK = 0,
  MK_E_INVALID = -1,        /* bad argument or configuration field */
  MK_E_SHAPE = -2,          /* tensor shape differs from the model's */
  MK_E_DTYPE = -3,          /* tensor element type differs from the model's */
  MK_E_NAME = -4,           /* unknown, duplicated or missing tensor name */
  MK_E_ORDER = -5,          /* call made in the wrong state (e.g. decode before weights) */
  MK_E_CTX_FULL = -6,       /* the step would pass max_ctx positions */
  MK_E_NO_DEVICE = -7,      /* no usable HIP device */
  MK_E_OCCUPANCY = -8,      /* the persistent grid cannot be co-resident on the device */
  MK_E_HIP = -9,            /* a HIP runtime call failed */
  MK_E_DEVICE_TIMEOUT = -10,/* a grid-wide wait inside a kernel gave up (bounded spin) */
  MK_E_UNSUPPORTED = -11    /* valid request this build does not implement */
};

/* MK_Q4G32: 4-bit block-quantised weights, the storage of the pages' 27B-scale model (megakernel
 * follow-up posts, page 3, quantisation-support paragraph: 4-bit weights in blocks with a scale).
 * A matrix W [R, K] (K a multiple of 32) is R*K*5/8 bytes: first the codes, K/2 bytes per row,
 * rows in order -- in row r, columns 8i .. 8i+7 sit in the little-endian 32-bit word at byte
 * r*K/2 + 4i, column 8i+2j in the nibble at bit 4j and column 8i+2j+1 in the nibble at bit 16+4j
 * (j = 0..3) -- then one 4-byte word per (row, group of 32 columns), row-major: the IEEE binary16
 * scale d in the low half, the binary16 offset m in the high half.  The weight is d*q + m for its
 * 4-bit code q.  The mk_tensor shape is the logical [R, K].
 * Values: MK_I32 (4) names int32 data such as token ids, so the 4-bit format takes the next free
 * value, 5; the numbers are part of the ABI and never change. */
enum mk_dtype { MK_BF16 = 1, MK_F32 = 2, MK_F16 = 3, MK_I32 = 4, MK_Q4G32 = 5, MK_Q8 = 6 };
/* MK_Q8 (a KV cache type): each key or value row of head_dim values is stored as int8 codes, and each
 * block of 32 consecutive values of a row has one FP32 scale s = max|x| / 127 of that block; a value
 * is stored as rint(x / s) (0 when s = 0) and read back as code * s. */

/* Model shape.  All fields are required (there is no default constructor on purpose).
 * Constraints checked by mk_workspace_bytes / mk_create: every size > 0; hidden, ffn, H*dk and
 * H*dv multiples of 8; dk, dv even and head_dim a multiple of 4, all <= 256; n_q_heads a multiple of n_kv_heads;
 * attn_slot < period; tied_embeddings == 1;
 * kv_dtype: MK_F32, MK_F16 (head_dim a multiple of 8) or MK_Q8 (head_dim a multiple of 32) -- the
 * element type of the KV cache.  The follow-up post on the 27B megakernel (page 3, "Limits"
 * paragraph) keeps its cache in fp16 up to about 80K positions and in an 8-bit format above; a
 * context picks one type for its whole cache.  Keys and values are rounded to the cache type as
 * they are appended, and attention (the appending position included) reads the stored values.
 * With 4-bit weights a compact cache needs head_dim <= 128;
 * 0 <= max_verify_k <= 5 (each unit adds one position's records, one DeltaNet state snapshot and
 * LDS; mk_create returns MK_E_OCCUPANCY if the verify kernel's LDS does not fit).
 * weight_dtype is MK_BF16 or MK_Q4G32.  MK_Q4G32 also needs hidden, ffn, H*dv and nq*head_dim to
 * be multiples of 32, hidden <= 8192, those other widths <= 20480 and max_verify_k == 0; its
 * prompts run one decode launch per
 * token (the prefill kernels take BF16 weights). */
typedef struct {
  int32_t n_layers, hidden, ffn, vocab;
  int32_t period, attn_slot;                       /* attention layers: l % period == attn_slot */
  int32_t dn_heads, dn_dk, dn_dv;                  /* DeltaNet heads and key/value head sizes   */
  int32_t n_q_heads, n_kv_heads, head_dim;         /* grouped-query attention                   */
  int32_t tied_embeddings, weight_dtype, kv_dtype;
  int32_t max_ctx;                                 /* positions the KV cache holds              */
  int32_t max_verify_k;                            /* drafts per mk_verify_k call, 0..5 (0 = none) */
  float rms_eps, l2_eps, rope_theta;
} mk_config;

/* One weight tensor for mk_load_weights.  name follows the model's manifest:
 *   embed [vocab, hidden]; per layer l: l{l}.norm1 [hidden], l{l}.norm2 [hidden],
 *   DeltaNet:  l{l}.dn.wqkv [2*H*dk + H*dv, hidden] (q heads, k heads, v heads), l{l}.dn.wa [H, hidden],
 *              l{l}.dn.wb [H, hidden], l{l}.dn.wo [hidden, H*dv];
 *   attention: l{l}.attn.wq [nq*hd, hidden], l{l}.attn.wk [nkv*hd, hidden], l{l}.attn.wv [nkv*hd, hidden],
 *              l{l}.attn.wo [hidden, nq*hd];
 *   FFN:       l{l}.ffn.wg [ffn, hidden], l{l}.ffn.wu [ffn, hidden], l{l}.ffn.wd [hidden, ffn];
 *   final_norm [hidden].
 * Row-major [out][in], contiguous.  data is a host pointer when on_device == 0, else a device
 * pointer on the ctx's device. */
typedef struct {
  const char* name;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[4];
  const void* data;
  int32_t on_device;
} mk_tensor;

/* Device bytes the caller must provide to mk_create for this configuration (weights, DeltaNet
 * state, KV cache and the kernel's exchange buffers).  Returns 0 for an invalid configuration
 * (mk_last_error(NULL) says why).  Needs no device. */
size_t mk_workspace_bytes(const mk_config* cfg);

/* Bind a context to `device`, the caller-owned workspace (>= mk_workspace_bytes, 256-byte
 * aligned, must outlive the ctx) and a HIP stream (hipStream_t, NULL = the default stream).
 * Validates cfg before touching the device.  Errors: MK_E_INVALID, MK_E_NO_DEVICE,
 * MK_E_OCCUPANCY, MK_E_HIP.  On error *out is NULL and mk_last_error(NULL) holds the message. */
int mk_create(const mk_config* cfg, int device, void* d_workspace, size_t workspace_bytes,
              void* hip_stream, mk_ctx** out);

/* Copy all model tensors into the workspace in the kernel's layout.  The follow-up post on the
 * 27B megakernel (page 3, "Since the first post" paragraph) has its loader check every tensor's
 * type and its server warm up before taking requests; this call does both.  Every manifest name must
 * appear exactly once with the manifest shape and dtype: MK_BF16 for everything, or, when the
 * config's weight_dtype is MK_Q4G32, MK_Q4G32 for the matrices (embed and every l{l}.* weight
 * matrix) and MK_BF16 for the norm gains; the whole list is checked
 * before anything is copied (MK_E_NAME / MK_E_DTYPE / MK_E_SHAPE name the offending tensor).
 * Then resets the sequence state and runs one warm-up launch.  Synchronous. */
int mk_load_weights(mk_ctx* ctx, const mk_tensor* tensors, int32_t n);

/* Same checks as mk_load_weights, for a configuration alone; needs no device or context. */
int mk_check_tensors(const mk_config* cfg, const mk_tensor* tensors, int32_t n);

/* Prefill: the prompt-processing side of the luce-megakernel announcement's results table (page 1,
 * the pp520 column: a 520-token prompt processed at once).  Runs the prompt through the same model
 * with multi-token kernels (matrix-core GEMMs, the DeltaNet recurrence in chunked form, causal
 * attention) and leaves the DeltaNet states and KV cache exactly where token-by-token decode would.
 * Process n prompt tokens d_tokens[0..n) starting at the current position; writes the greedy
 * next token (argmax of the last position's logits, lowest index on ties) to d_next[0] and, if
 * d_logits != NULL, that position's logits [vocab] as FP32.  Advances the position by n.
 * Errors: MK_E_ORDER (no weights), MK_E_INVALID (n <= 0 or null pointers), MK_E_CTX_FULL. */
int mk_prefill(mk_ctx* ctx, const int32_t* d_tokens, int32_t n, int32_t* d_next, float* d_logits);

/* One decode step as ONE kernel launch: embeds d_tok[0] at the current position, runs every
 * layer, writes the greedy next token to d_next[0] (may alias d_tok) and optional FP32 logits
 * [vocab]; advances the position by one on the device.  Errors: MK_E_ORDER, MK_E_INVALID,
 * MK_E_CTX_FULL (checked against the host's count of enqueued positions). */
int mk_decode_step(mk_ctx* ctx, const int32_t* d_tok, int32_t* d_next, float* d_logits);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): mk_decode_step with the decode kernel's scratch -- its
 * exchange records and argmax records -- held in a static device array of the library
 * (MK_NOALLOC_SCRATCH_BYTES = 16 MiB per device, kept until the process ends) instead of the
 * workspace.  It allocates nothing and makes no allocating library call; its inputs, outputs and
 * the model state (weights, DeltaNet states, KV cache, position) stay where mk_decode_step has
 * them, and its results are bit-identical to mk_decode_step's.  Every context on a device shares
 * the one array; each call clears the part it uses before launching, and calls that overlap on
 * one device (several streams, several contexts at once) race.  Errors: as mk_decode_step, plus
 * MK_E_UNSUPPORTED when the model's records exceed the array (the message gives both sizes). */
int mk_decode_step_noalloc(mk_ctx* ctx, const int32_t* d_tok, int32_t* d_next, float* d_logits);

/* Speculative verify as ONE kernel launch (Reddit follow-up on the 27B model, speculative-decoding
 * paragraph: several drafted tokens checked per pass, the main model's greedy output kept exactly).
 * d_tokens[0..k] = [pending, d1..dk] (device int32; the pending token is the last greedy choice, not
 * yet fed).  The launch runs positions pos .. pos+k and writes the greedy choice after each to
 * d_out[0..k] (device int32 [k+1]); a = the number of leading drafts with d_i == d_out[i-1] goes to
 * d_n_accepted[0].  The sequence keeps [pending, d1..da]: the position advances by a + 1 and the
 * DeltaNet states and KV cache are exactly those of a + 1 decode steps; d_out[0..a] are the tokens
 * to emit and d_out[a] is the next pending token.  Every choice equals, bit for bit, the one
 * mk_decode_step makes at that position with the same grid size.
 * Requires a context created with max_verify_k >= 1 and 0 <= k <= max_verify_k (MK_E_INVALID
 * otherwise); MK_E_CTX_FULL if k + 1 positions do not fit; a draft id outside [0, vocab) is
 * reported by the next mk_sync (MK_E_INVALID) and nothing is written.  Afterwards the host learns
 * the accepted count only through d_n_accepted; the next mk_prefill, mk_get_position or
 * full-context check synchronises to read the device's position. */
int mk_verify_k(mk_ctx* ctx, const int32_t* d_tokens, int32_t k, int32_t* d_out, int32_t* d_n_accepted);

/* Position 0, zero DeltaNet states and KV cache (weights kept).  Enqueued on the stream. */
int mk_reset(mk_ctx* ctx);

/* Wait for the stream; returns MK_E_DEVICE_TIMEOUT if a kernel reported a failed grid wait, or
 * if the device position is behind the positions enqueued since the last exact count (a launch
 * that ended early); the sequence state is then undefined until mk_reset. */
int mk_sync(mk_ctx* ctx);

/* Current position as the device holds it (synchronises). */
int mk_get_position(mk_ctx* ctx, int32_t* pos);

/* Copy one layer's recurrent state to/from host memory (synchronises).  DeltaNet layer: S as
 * FP32 [dn_heads][dn_dv][dn_dk] (row i of head h maps keys to value dimension i).  Attention
 * layer: K then V as FP32 [n_kv_heads][max_ctx][head_dim] each (keys already rotated); with a
 * compact cache the stored values decoded to FP32 on read, and FP32 values rounded to the cache
 * type (nearest binary16, or int8 blocks formed as above) on write.
 * mk_state_bytes gives the byte count for `layer`, or 0 if it is out of range. */
size_t mk_state_bytes(const mk_ctx* ctx, int32_t layer);
int mk_read_state(mk_ctx* ctx, int32_t layer, void* dst);
int mk_write_state(mk_ctx* ctx, int32_t layer, const void* src);

/* Set the sequence position to pos (0 <= pos <= max_ctx): the other half of a state hand-off, after
 * mk_write_state has restored every layer's DeltaNet state and KV entries [0, pos) of a sequence.
 * Enqueued on the stream; errors: MK_E_INVALID. */
int mk_set_position(mk_ctx* ctx, int32_t pos);

/* Number of workgroups of the persistent grid (default: one per compute unit).  Results are
 * bitwise identical for every grid size; smaller grids exist for that check and for tuning.
 * Errors: MK_E_INVALID (n < 1 or more than the device's compute units). */
int mk_set_grid(mk_ctx* ctx, int32_t n_workgroups);
int mk_get_grid(const mk_ctx* ctx, int32_t* n_workgroups);

/* Diagnostics: when d_trace != NULL, every later decode launch stores, per workgroup w, the device
 * real-time clock (100 MHz) at each phase boundary into d_trace[w * 512 + e] (uint64).  bytes must
 * cover grid * 512 * 8.  NULL turns the trace off.  Errors: MK_E_INVALID. */
int mk_set_trace(mk_ctx* ctx, void* d_trace, size_t bytes);

/* Message for the last failed call on ctx; ctx == NULL gives the calling thread's message from
 * a failed mk_workspace_bytes / mk_create / mk_check_tensors. */
const char* mk_last_error(const mk_ctx* ctx);

void mk_destroy(mk_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* MK_H */

// Host runtime behind include/mk.h: configuration checks, workspace carving, the weight loader
// (per-tensor name/type/shape checks, then repacking into the kernel's row order), sequence state
// management and kernel launches.  No torch types: plain pointers, sizes and a HIP stream.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/mk.h"
#define MK_HOST_VIEW 1
#include "mk_internal.h"

namespace {

thread_local std::string g_err;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int fail_global(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

struct TensorSpec {
  std::string name;
  std::vector<int64_t> shape;
};

bool is_attention(const mk_config& c, int l) { return l % c.period == c.attn_slot; }

// KV cache element type of the kernels for a config's kv_dtype
int kv_type(int kv_dtype) { return kv_dtype == MK_F16 ? MK_KV_F16 : (kv_dtype == MK_Q8 ? MK_KV_Q8 : MK_KV_F32); }
size_t kv_elem_bytes(int kvt) { return kvt == MK_KV_F32 ? 4 : (kvt == MK_KV_F16 ? 2 : 1); }
// stage slots of one KV chunk buffer, as the decode kernels count them (mk_device.h)
int kv_buf_slots_host(int hd, int kvt) {
  const int lpp = (int)(hd * kv_elem_bytes(kvt)) / 16, pps = 64 / lpp;
  const int ks = (MK_ATT_CHUNK + pps - 1) / pps;
  return (2 * ks + (kvt == MK_KV_Q8 ? 1 : 0) + 3) & ~3;
}

std::vector<TensorSpec> manifest(const mk_config& c) {
  std::vector<TensorSpec> m;
  const int64_t D = c.hidden, H = c.dn_heads;
  m.push_back({"embed", {c.vocab, D}});
  for (int l = 0; l < c.n_layers; ++l) {
    const std::string p = "l" + std::to_string(l) + ".";
    m.push_back({p + "norm1", {D}});
    if (is_attention(c, l)) {
      m.push_back({p + "attn.wq", {(int64_t)c.n_q_heads * c.head_dim, D}});
      m.push_back({p + "attn.wk", {(int64_t)c.n_kv_heads * c.head_dim, D}});
      m.push_back({p + "attn.wv", {(int64_t)c.n_kv_heads * c.head_dim, D}});
      m.push_back({p + "attn.wo", {D, (int64_t)c.n_q_heads * c.head_dim}});
    } else {
      m.push_back({p + "dn.wqkv", {2 * H * c.dn_dk + H * c.dn_dv, D}});
      m.push_back({p + "dn.wa", {H, D}});
      m.push_back({p + "dn.wb", {H, D}});
      m.push_back({p + "dn.wo", {D, H * c.dn_dv}});
    }
    m.push_back({p + "norm2", {D}});
    m.push_back({p + "ffn.wg", {c.ffn, D}});
    m.push_back({p + "ffn.wu", {c.ffn, D}});
    m.push_back({p + "ffn.wd", {D, c.ffn}});
  }
  m.push_back({"final_norm", {D}});
  return m;
}

std::string check_config(const mk_config* c) {
  if (!c) return "config is NULL";
  if (c->n_layers <= 0 || c->hidden <= 0 || c->ffn <= 0 || c->vocab <= 0) return "n_layers, hidden, ffn, vocab must be > 0";
  if (c->period <= 0 || c->attn_slot < 0 || c->attn_slot >= c->period) return "need 0 <= attn_slot < period";
  if (c->dn_heads <= 0 || c->dn_dk <= 0 || c->dn_dv <= 0) return "DeltaNet head sizes must be > 0";
  if (c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0) return "attention head sizes must be > 0";
  if (c->n_q_heads % c->n_kv_heads != 0) return "n_q_heads must be a multiple of n_kv_heads";
  if (c->hidden % 8 || c->ffn % 8 || (c->dn_heads * c->dn_dv) % 8 || (c->n_q_heads * c->head_dim) % 8)
    return "hidden, ffn, dn_heads*dn_dv and n_q_heads*head_dim must be multiples of 8";
  if (c->dn_dk % 4 || c->dn_dv % 2 || c->head_dim % 4) return "dn_dk and head_dim must be multiples of 4, dn_dv even";
  if (c->n_q_heads / c->n_kv_heads > 32) return "at most 32 query heads per KV head";
  if (c->dn_dk > 256 || c->dn_dv > 256 || c->head_dim > 256) return "dn_dk, dn_dv, head_dim must be <= 256";
  if (c->tied_embeddings != 1) return "only tied embeddings are supported";
  if (c->weight_dtype != MK_BF16 && c->weight_dtype != MK_Q4G32) return "weight_dtype must be MK_BF16 or MK_Q4G32";
  if (c->weight_dtype == MK_Q4G32) {
    if (c->hidden % 32 || c->ffn % 32 || (c->dn_heads * c->dn_dv) % 32 || (c->n_q_heads * c->head_dim) % 32)
      return "MK_Q4G32 needs hidden, ffn, dn_heads*dn_dv and n_q_heads*head_dim to be multiples of 32";
    if (c->hidden > 8192 || c->ffn > 20480 || c->dn_heads * c->dn_dv > 20480 || c->n_q_heads * c->head_dim > 20480)
      return "MK_Q4G32 needs hidden <= 8192 and ffn, dn_heads*dn_dv, n_q_heads*head_dim <= 20480";
  }
  if (c->kv_dtype != MK_F32 && c->kv_dtype != MK_F16 && c->kv_dtype != MK_Q8)
    return "kv_dtype must be MK_F32, MK_F16 or MK_Q8";
  if (c->kv_dtype == MK_F16 && c->head_dim % 8) return "an MK_F16 KV cache needs head_dim to be a multiple of 8";
  if (c->kv_dtype == MK_Q8 && c->head_dim % MK_KV_Q8_BLOCK)
    return "an MK_Q8 KV cache needs head_dim to be a multiple of 32";
  if (c->kv_dtype != MK_F32) {
    // the decode kernels stage compact chunks next to one FP32 chunk buffer in their KV stage
    const int kvt = kv_type(c->kv_dtype);
    const int a_slots = c->weight_dtype == MK_Q4G32 ? 32 : MK_STAGE_A_SLOTS;
    if (kv_buf_slots_host(c->head_dim, MK_KV_F32) + kv_buf_slots_host(c->head_dim, kvt) > a_slots)
      return "head_dim too large for a compact KV cache with these weights";
  }
  if (c->max_ctx <= 0 || c->max_ctx > (1 << 20)) return "max_ctx must be in [1, 2^20]";
  if (c->max_verify_k < 0 || c->max_verify_k > MK_VERIFY_MAXT - 1)
    return "max_verify_k must be in [0, " + std::to_string(MK_VERIFY_MAXT - 1) + "]";
  if (!(c->rms_eps > 0.f) || !(c->l2_eps > 0.f) || !(c->rope_theta > 0.f)) return "eps and rope_theta must be > 0";
  if (c->hidden > 16384 || c->ffn > 65536) return "hidden <= 16384 and ffn <= 65536";
  return "";
}

// ----------------------------------------------------------------------- workspace layout
struct LayerOff {
  size_t w_in, w_out, w_gu, w_down, g12, S, Kc, Vc, Ks, Vs, ll_in, ll_part, ll_o, ll_x1, ll_h, ll_x2;
  // speculative verify: records of vt positions ([t][n] per record vector) and state snapshots
  size_t v_in, v_part, v_o, v_x1, v_h, v_x2, snap;
  int64_t rows_in, k_out;
};

struct Layout {
  size_t ctl, descs, rope_cos, rope_sin, g_final, embed, ll_am, scratch, total;
  // mk_decode_step_noalloc: layer descriptors whose records point into the static scratch array,
  // and the bytes of decode records (from xchg_begin) that array must hold
  size_t ndescs, na_bytes;
  size_t state_begin, state_end;  // DeltaNet states + KV caches
  size_t xchg_begin, xchg_end;    // exchange records
  std::vector<LayerOff> layers;
  int max_items;
  // speculative verify (vt = max_verify_k + 1 positions per launch; 0 when not configured)
  int vt;
  size_t vdescs, v_am, v_acc;
  int64_t snap_stride;  // floats between the snapshots of consecutive positions
  // prefill scratch: a chunk of up to pf_T tokens
  int pf_T, pf_lda, pf_ldy, pf_ldh;
  size_t pf_x, pf_ahi, pf_alo, pf_hhi, pf_hlo, pf_y, pf_qk, pf_ab, pf_q, pf_part, pf_ch, pf_sk;
  size_t pf_wq;   // 4-bit weights: one matrix expanded to rows [W_hi | W_lo] of BF16
  size_t pf_kvf;  // compact KV caches: a chunk's rotated keys and values in FP32, [2][nkv][T][hd]
};

constexpr int PF_LM_WG = 512;  // workgroups of the prefill LM head

Layout make_layout(const mk_config& c) {
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  const int64_t D = c.hidden, H = c.dn_heads, half = c.head_dim / 2;
  const int gs = c.n_q_heads / c.n_kv_heads;
  const bool q4 = c.weight_dtype == MK_Q4G32;
  // bytes of a weight matrix [R][K]: BF16, or Q4G32 tiles (rows padded to a multiple of 4)
  auto wbytes = [&](int64_t R, int64_t K) -> size_t {
    return q4 ? (size_t)((R + 3) / 4 * 4 * K * 5 / 8) : (size_t)(R * K * 2);
  };
  L.max_items = ((c.max_ctx + MK_ATT_CHUNK - 1) / MK_ATT_CHUNK) * c.n_kv_heads;
  L.ctl = take(sizeof(MkCtl));
  L.descs = take(sizeof(MkLayerDev) * c.n_layers);
  L.rope_cos = take((size_t)c.max_ctx * half * 4);
  L.rope_sin = take((size_t)c.max_ctx * half * 4);
  L.g_final = take(D * 2);
  L.embed = take(wbytes(c.vocab, D));
  L.layers.resize(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l) {
    LayerOff& lo = L.layers[l];
    const bool att = is_attention(c, l);
    lo.rows_in = att ? (int64_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim : 2 * H * c.dn_dk + H * c.dn_dv + 2 * H;
    lo.k_out = att ? (int64_t)c.n_q_heads * c.head_dim : H * c.dn_dv;
    lo.w_in = take(wbytes(lo.rows_in, D));
    lo.w_out = take(wbytes(D, lo.k_out));
    lo.w_gu = take(wbytes(2 * (int64_t)c.ffn, D));
    lo.w_down = take(wbytes(D, c.ffn));
    lo.g12 = take(D * 4);  // BF16 [2][D]
  }
  L.state_begin = o;
  for (int l = 0; l < c.n_layers; ++l) {
    LayerOff& lo = L.layers[l];
    if (is_attention(c, l)) {
      const size_t eb = kv_elem_bytes(kv_type(c.kv_dtype));
      lo.Kc = take((size_t)c.n_kv_heads * c.max_ctx * c.head_dim * eb);
      lo.Vc = take((size_t)c.n_kv_heads * c.max_ctx * c.head_dim * eb);
      if (c.kv_dtype == MK_Q8) {
        // 16-byte copies of a chunk's scale rows may reach up to 12 bytes past the last row
        const size_t sb = (size_t)c.n_kv_heads * c.max_ctx * (c.head_dim / MK_KV_Q8_BLOCK) * 4 + 256;
        lo.Ks = take(sb);
        lo.Vs = take(sb);
      }
    } else {
      lo.S = take((size_t)H * c.dn_dv * c.dn_dk * 4);
    }
  }
  L.state_end = o;
  L.xchg_begin = o;
  for (int l = 0; l < c.n_layers; ++l) {
    LayerOff& lo = L.layers[l];
    lo.ll_in = take((size_t)lo.rows_in * 8);
    if (is_attention(c, l)) lo.ll_part = take((size_t)L.max_items * gs * (c.head_dim + 2) * 8);
    lo.ll_o = take((size_t)lo.k_out * 8);
    lo.ll_x1 = take(D * 8);
    lo.ll_h = take((size_t)c.ffn * 8);
    lo.ll_x2 = take(D * 8);
  }
  L.ll_am = take((size_t)2 * MK_MAX_GRID * 8);
  L.na_bytes = o - L.xchg_begin;  // the decode kernel's records: what mk_decode_step_noalloc keeps in static scratch
  L.vt = c.max_verify_k > 0 ? c.max_verify_k + 1 : 0;
  if (L.vt) {
    const size_t vt = (size_t)L.vt;
    for (int l = 0; l < c.n_layers; ++l) {
      LayerOff& lo = L.layers[l];
      lo.v_in = take(vt * lo.rows_in * 8);
      if (is_attention(c, l)) lo.v_part = take(vt * L.max_items * gs * (c.head_dim + 2) * 8);
      lo.v_o = take(vt * lo.k_out * 8);
      lo.v_x1 = take(vt * D * 8);
      lo.v_h = take(vt * c.ffn * 8);
      lo.v_x2 = take(vt * D * 8);
    }
    L.v_am = take(vt * 2 * MK_MAX_GRID * 8);
    L.v_acc = take(256);
  }
  L.xchg_end = o;
  if (L.vt) {
    L.vdescs = take(sizeof(MkLayerDev) * c.n_layers);
    int n_dn = 0;
    for (int l = 0; l < c.n_layers; ++l) n_dn += is_attention(c, l) ? 0 : 1;
    const int64_t per = H * c.dn_dv * c.dn_dk;
    L.snap_stride = n_dn * per;
    const size_t base = take((size_t)c.max_verify_k * L.snap_stride * 4);
    int j = 0;
    for (int l = 0; l < c.n_layers; ++l)
      if (!is_attention(c, l)) L.layers[l].snap = base + (size_t)(j++) * per * 4;
  }
  L.ndescs = take(sizeof(MkLayerDev) * c.n_layers);
  L.scratch = take(4096);
  // prefill scratch.  With 4-bit weights every GEMM runs over 2K columns ([A_hi | A_hi] and
  // [A_lo | 0] against [W_hi | W_lo]), so the activation rows are twice as wide, and one matrix at a
  // time is expanded into pf_wq.
  {
    const int64_t T = std::min(c.max_ctx, 1024);
    const int64_t kmax = std::max(std::max(D, (int64_t)c.ffn), std::max(H * c.dn_dv, (int64_t)c.n_q_heads * c.head_dim));
    const int64_t ndn = 2 * H * c.dn_dk + H * c.dn_dv + 2 * H;
    const int64_t natt = (int64_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
    const int64_t wide = q4 ? 2 : 1;
    L.pf_T = (int)T;
    L.pf_lda = (int)((wide * kmax + 7) / 8 * 8);
    L.pf_ldh = (int)(wide * c.ffn);
    L.pf_ldy = (int)((std::max(ndn, natt) + 3) / 4 * 4);  // rows 16-byte aligned
    L.pf_x = take((size_t)T * D * 4);
    L.pf_ahi = take((size_t)T * L.pf_lda * 2);
    L.pf_alo = take((size_t)T * L.pf_lda * 2);
    L.pf_hhi = take((size_t)T * L.pf_ldh * 2);
    L.pf_hlo = take((size_t)T * L.pf_ldh * 2);
    if (q4) {
      int64_t wmax = std::max(2 * (int64_t)c.ffn * D, D * (int64_t)c.ffn);
      for (const LayerOff& lo : L.layers) wmax = std::max(wmax, std::max(lo.rows_in * D, D * lo.k_out));
      L.pf_wq = take((size_t)wmax * 2 * 2);
    }
    L.pf_y = take((size_t)T * L.pf_ldy * 4);
    L.pf_qk = take((size_t)T * H * 2 * c.dn_dk * 4);
    L.pf_ab = take((size_t)T * H * 2 * 4);
    L.pf_q = take((size_t)T * c.n_q_heads * c.head_dim * 4);
    L.pf_part = take((size_t)PF_LM_WG * 2 * 4);
    // chunked DeltaNet: per (64-token chunk, head) W and Bt [64][64], two decay vectors and gamma_C
    L.pf_ch = take((size_t)((T + 63) / 64) * H * (2 * 64 * 64 + 2 * 64 + 4) * 4);
    // split-K partials of the residual GEMMs: at most 256 work items of 128 x 128 outputs
    L.pf_sk = take(PF_SPLITK_FLOATS * 4);
    if (c.kv_dtype != MK_F32) L.pf_kvf = take((size_t)2 * T * c.n_kv_heads * c.head_dim * 4);
  }
  L.total = o;
  return L;
}

// LDS carve for the decode kernel (floats) at grid size `grid`
void lds_layout(const mk_config& c, int grid, MkDecodeParams& p) {
  const int D = c.hidden;
  const int gs = c.n_q_heads / c.n_kv_heads;
  const int hd = c.head_dim, C = MK_ATT_CHUNK;
  // gathered mixer output / FFN hidden, argmax records
  // (also the attention items' partial scores: a pass of MK_ATT_PASS chunks takes at most
  // MK_ATT_PASS * MK_NT floats)
  const int vec = std::max(std::max(std::max(c.ffn, c.dn_heads * c.dn_dv), std::max(c.n_q_heads * hd, 2 * grid)),
                           MK_ATT_PASS * MK_NT);
  // gathered DeltaNet inputs (one head), attention item inputs, combine staging, GEMV unit partials
  int att = 2 * c.dn_dk + 2 + c.dn_dv;
  // attention items (a pass of up to MK_ATT_PASS chunks), running merge included
  att = std::max(att, 2 * gs * hd + 2 * hd + MK_ATT_PASS * (gs * C + 2 * gs) + 4 * gs);
  att = std::max(att, MK_RED_CAP);
  att = std::max(att, 3 * 129);  // combine staging of one output: at most 128 items per KV head (+1)
  int o = 0;
  auto take = [&](int n) {
    const int at = o;
    o += (n + 3) / 4 * 4;  // 16-byte aligned regions
    return at;
  };
  p.lds_desc = take(c.n_layers * (int)(sizeof(MkLayerDev) / 4));
  p.lds_gain = take(2 * D);  // BF16 [2][2][D]
  p.lds_rope = take(hd);
  p.lds_x = take(D);
  p.lds_xn = take(D);
  p.lds_vec = take(vec);
  p.lds_att = take(att);
  p.lds_scr = take(4 * MK_NWAVE);
  p.lds_flag = take(4);
  o = (o + 1) / 2 * 2;
  p.lds_trace = take(2 * MK_TRACE_EVENTS);
  // the prefetch stages are a static array of the kernel (MK_STAGE_A_SLOTS + MK_STAGE_B_SLOTS KB,
  // more than half the LDS of a compute unit, so one workgroup fits per unit)
  p.lds_floats = o;
}

// LDS carve for the 4-bit decode kernel (floats): two layer descriptors, no gains (read from global memory),
// the normalised activations share the vector region, unit partials hold Q4_RED_CAP floats; its
// static stage (48 KB) holds the DeltaNet state rows and the attention KV chunks.
void lds_layout_q4(const mk_config& c, int grid, MkDecodeParams& p) {
  const int D = c.hidden;
  const int gs = c.n_q_heads / c.n_kv_heads;
  const int hd = c.head_dim, C = MK_ATT_CHUNK;
  const int vec = std::max(std::max(std::max(std::max(c.ffn, D), c.dn_heads * c.dn_dv), std::max(c.n_q_heads * hd, 2 * grid)),
                           2 * MK_NT);  // (also the attention items' partial scores: passes of two chunks)
  int att = 2 * c.dn_dk + 2 + c.dn_dv;
  att = std::max(att, 2 * gs * hd + 2 * hd + 2 * (gs * C + 2 * gs) + 4 * gs);
  att = std::max(att, 2048);  // Q4_RED_CAP
  att = std::max(att, 3 * 129);
  int o = 0;
  auto take = [&](int n) {
    const int at = o;
    o += (n + 3) / 4 * 4;
    return at;
  };
  p.lds_desc = take(2 * (int)(sizeof(MkLayerDev) / 4));  // this layer's and the next one's
  p.lds_gain = 0;
  p.lds_rope = take(hd);
  p.lds_x = take(D);
  p.lds_vec = take(vec);
  p.lds_xn = p.lds_vec;
  p.lds_att = take(att);
  p.lds_scr = take(4 * MK_NWAVE);
  p.lds_flag = take(4);
  o = (o + 1) / 2 * 2;
  p.lds_trace = take(2 * MK_TRACE_EVENTS);
  p.lds_floats = o;
}

// LDS carve for the verify kernel (floats) at grid size `grid`: vt positions' residuals, RoPE rows
// and vectors; the vector region also stages DeltaNet inputs, attention items, the combine and the
// argmax records.  No prefetch stages.
void lds_layout_verify(const mk_config& c, int grid, MkDecodeParams& p) {
  const int vt = c.max_verify_k + 1;
  const int D = c.hidden;
  const int gs = c.n_q_heads / c.n_kv_heads;
  const int hd = c.head_dim, C = MK_ATT_CHUNK;
  int64_t vec = (int64_t)vt * std::max(std::max(c.ffn, c.dn_heads * c.dn_dv), std::max(c.n_q_heads * hd, D));
  vec = std::max(vec, (int64_t)vt * (2 * c.dn_dk + 2 + c.dn_dv));
  vec = std::max(vec, (int64_t)2 * vt * gs * hd + 2 * C * hd + vt * gs * C + 6 * vt * gs);  // items + merge
  vec = std::max(vec, (int64_t)3 * vt * 129);  // combine staging of one output: <= 128 items per KV head
  vec = std::max(vec, (int64_t)2 * vt * grid);
  vec = std::max(vec, (int64_t)vt * D + 2 * vt * MK_NCT);  // LM head: activations + running argmax
  int o = 0;
  auto take = [&](int64_t n) {
    const int at = o;
    o += (int)((n + 3) / 4 * 4);
    return at;
  };
  p.lds_desc = take(c.n_layers * (int)(sizeof(MkLayerDev) / 4));
  p.lds_gain = take(D);  // BF16 [2][D]
  p.lds_rope = take(vt * hd);
  p.lds_x = take((int64_t)vt * D);
  p.lds_vec = take(vec);
  p.vec_floats = (int32_t)((vec + 3) / 4 * 4);
  p.lds_att = take(MK_RED_CAP);
  p.lds_scr = take(2 * MK_VERIFY_MAXT * MK_NWAVE);
  p.lds_flag = take(4);
  p.lds_xn = take(MK_VERIFY_MAXT);  // the tokens (the normalised activations share the vector region)
  o = (o + 1) / 2 * 2;
  p.lds_trace = take(2 * MK_TRACE_EVENTS);
  p.lds_floats = o;
}

// LDS carve for the 4-bit verify kernel (floats): descriptors, RoPE rows, this workgroup's residual
// rows of each position, the GEMV partials and the LM head's running argmax, and the vector region
// (packed activations of a column group for every position; a gathered residual; DeltaNet, attention
// and combine scratch) taking what is left of the compute unit's 160 KB.  Returns "" or the reason
// the carve does not fit.
constexpr int MK_LDS_FLOATS = 160 * 1024 / 4;
std::string lds_layout_verify_q4(const mk_config& c, int grid, MkDecodeParams& p) {
  const int vt = c.max_verify_k + 1, D = c.hidden, hd = c.head_dim, C = MK_ATT_CHUNK;
  const int gs = c.n_q_heads / c.n_kv_heads;
  const int rst = 4 * ((D / 4 + grid - 1) / grid);
  int o = 0;
  auto take = [&](int64_t n) {
    const int at = o;
    o += (int)((n + 3) / 4 * 4);
    return at;
  };
  p.lds_gain = 0;
  p.lds_rope = take(vt * hd);
  p.lds_x = take((int64_t)vt * rst);
  p.rstride = rst;
  p.lds_att = take(MK_RED_CAP + 2 * vt * MK_NCT);
  p.lds_scr = take(2 * MK_VERIFY_MAXT * MK_NWAVE);
  p.lds_flag = take(4);
  p.lds_xn = take(MK_VERIFY_MAXT);
  o = (o + 1) / 2 * 2;
  p.lds_trace = take(2 * MK_TRACE_EVENTS);
  const int vec = (MK_LDS_FLOATS - o) / 4 * 4;
  p.lds_vec = take(vec);
  p.vec_floats = vec;
  p.lds_floats = o;
  // layer descriptors are read from memory; the rollback's copy of the table sits at the tail of the
  // vector region, after the argmax records it gathers there
  const int ndesc = (c.n_layers * (int)(sizeof(MkLayerDev) / 4) + 3) / 4 * 4;
  p.lds_desc = p.lds_vec + vec - ndesc;
  if ((int64_t)2 * vt * grid + ndesc > vec)
    return "4-bit verify: the layer descriptors and argmax records do not fit the vector LDS";
  int64_t need = (int64_t)vt * 2048;                                                      // one column group
  need = std::max<int64_t>(need, (int64_t)vt * (2 * c.dn_dk + 2 + c.dn_dv));              // DeltaNet inputs
  need = std::max<int64_t>(need, (int64_t)2 * vt * gs * hd + 2 * C * hd + vt * gs * C + 6 * vt * gs);  // items
  need = std::max<int64_t>(need, (int64_t)3 * vt * 129);                                  // combine staging
  need = std::max<int64_t>(need, (int64_t)2 * vt * grid);                                 // argmax records
  // a workgroup's FFN hidden slice (whole 32-column blocks) is staged in the LM head's argmax cells
  const int64_t hw = 32 * (((int64_t)c.ffn / 32 + grid - 1) / grid);
  if (vt * hw > 2 * vt * MK_NCT)
    return "4-bit verify stages " + std::to_string(hw) + " FFN hidden columns per workgroup at this grid; at most " +
           std::to_string(2 * MK_NCT) + " fit";
  if (vec < need)
    return "4-bit verify needs " + std::to_string(need * 4) + " B of vector LDS; " + std::to_string((int64_t)vec * 4) +
           " B are left";
  return "";
}

}  // namespace

struct mk_ctx {
  mk_config cfg;
  int device = 0;
  hipStream_t stream = nullptr;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  Layout lay;
  MkDecodeParams base{};
  MkDecodeParams vbase{};  // verify launches (valid when lay.vt > 0)
  MkDecodeParams nbase{};  // mk_decode_step_noalloc launches (valid when na_fits)
  char* na_scratch = nullptr;  // this device's static record array
  bool na_fits = false;
  int n_cu = 0;
  int grid = 0;
  bool loaded = false;
  // positions enqueued so far; after a verify launch only an upper bound (the device decides how
  // many drafts it keeps) until the next synchronising call reads the device's count
  int64_t pos_host = 0;
  bool pos_exact = true;
  std::string err;
};

namespace {

int fail(mk_ctx* ctx, int code, const std::string& msg) {
  if (ctx) ctx->err = msg;
  g_err = msg;
  return code;
}

#define HIPCHK(ctx, call)                                                                     \
  do {                                                                                        \
    hipError_t _e = (call);                                                                   \
    if (_e != hipSuccess)                                                                     \
      return fail((ctx), MK_E_HIP, std::string(#call) + ": " + hipGetErrorString(_e));        \
  } while (0)

// The device's position -> the host count (synchronises).  Used where the host needs the exact
// value after verify launches left it an upper bound.
int refresh_position(mk_ctx* ctx) {
  HIPCHK(ctx, hipStreamSynchronize(ctx->stream));
  MkCtl ctl;
  HIPCHK(ctx, hipMemcpy(&ctl, ctx->base.ctl, sizeof(ctl), hipMemcpyDeviceToHost));
  if (!ctl.err) ctx->pos_host = ctl.pos;
  ctx->pos_exact = true;
  return MK_OK;
}

int check_tensor_list(const mk_config& c, const mk_tensor* t, int32_t n, std::string& msg,
                      std::vector<int>* order) {
  const std::vector<TensorSpec> man = manifest(c);
  std::map<std::string, int> idx;
  for (size_t i = 0; i < man.size(); ++i) idx[man[i].name] = (int)i;
  std::vector<int> seen(man.size(), -1);
  if (n < 0 || (n > 0 && !t)) {
    msg = "tensor list is NULL or n < 0";
    return MK_E_INVALID;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (!t[i].name) {
      msg = "tensor " + std::to_string(i) + " has no name";
      return MK_E_NAME;
    }
    auto it = idx.find(t[i].name);
    if (it == idx.end()) {
      msg = std::string("unknown tensor '") + t[i].name + "'";
      return MK_E_NAME;
    }
    if (seen[it->second] >= 0) {
      msg = std::string("tensor '") + t[i].name + "' given twice";
      return MK_E_NAME;
    }
    seen[it->second] = i;
    const TensorSpec& sp = man[it->second];
    const int want = (c.weight_dtype == MK_Q4G32 && sp.shape.size() == 2) ? MK_Q4G32 : MK_BF16;
    if (t[i].dtype != want) {
      msg = std::string("tensor '") + t[i].name + "' has dtype " + std::to_string(t[i].dtype) + ", expected " +
            (want == MK_Q4G32 ? "MK_Q4G32" : "MK_BF16");
      return MK_E_DTYPE;
    }
    bool same = (int)sp.shape.size() == t[i].ndim;
    for (size_t d = 0; same && d < sp.shape.size(); ++d) same = (t[i].shape[d] == sp.shape[d]);
    if (!same) {
      std::string want = "[", got = "[";
      for (size_t d = 0; d < sp.shape.size(); ++d) want += (d ? ", " : "") + std::to_string(sp.shape[d]);
      for (int d = 0; d < t[i].ndim && d < 4; ++d) got += (d ? ", " : "") + std::to_string(t[i].shape[d]);
      msg = std::string("tensor '") + t[i].name + "' has shape " + got + "], expected " + want + "]";
      return MK_E_SHAPE;
    }
    if (!t[i].data) {
      msg = std::string("tensor '") + t[i].name + "' has no data";
      return MK_E_INVALID;
    }
  }
  for (size_t i = 0; i < man.size(); ++i)
    if (seen[i] < 0) {
      msg = "missing tensor '" + man[i].name + "'";
      return MK_E_NAME;
    }
  if (order) *order = seen;
  return MK_OK;
}

}  // namespace

extern "C" {

size_t mk_workspace_bytes(const mk_config* cfg) {
  const std::string e = check_config(cfg);
  if (!e.empty()) {
    g_err = e;
    return 0;
  }
  return make_layout(*cfg).total;
}

int mk_check_tensors(const mk_config* cfg, const mk_tensor* tensors, int32_t n) {
  const std::string e = check_config(cfg);
  if (!e.empty()) return fail_global(MK_E_INVALID, e);
  std::string msg;
  const int rc = check_tensor_list(*cfg, tensors, n, msg, nullptr);
  if (rc != MK_OK) g_err = msg;
  return rc;
}

const char* mk_last_error(const mk_ctx* ctx) { return ctx ? ctx->err.c_str() : g_err.c_str(); }

int mk_create(const mk_config* cfg, int device, void* d_workspace, size_t workspace_bytes, void* hip_stream,
              mk_ctx** out) {
  if (!out) return fail_global(MK_E_INVALID, "out is NULL");
  *out = nullptr;
  const std::string e = check_config(cfg);
  if (!e.empty()) return fail_global(MK_E_INVALID, e);
  const Layout lay = make_layout(*cfg);
  if (!d_workspace) return fail_global(MK_E_INVALID, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(d_workspace) % 256) return fail_global(MK_E_INVALID, "workspace must be 256-byte aligned");
  if (workspace_bytes < lay.total)
    return fail_global(MK_E_INVALID, "workspace too small: need " + std::to_string(lay.total) + " bytes");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return fail_global(MK_E_NO_DEVICE, "no HIP device");
  if (device < 0 || device >= ndev) return fail_global(MK_E_NO_DEVICE, "device index out of range");
  if (hipSetDevice(device) != hipSuccess) return fail_global(MK_E_NO_DEVICE, "hipSetDevice failed");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return fail_global(MK_E_HIP, "hipGetDeviceProperties failed");
  hipPointerAttribute_t pa;
  if (hipPointerGetAttributes(&pa, d_workspace) != hipSuccess || pa.type != hipMemoryTypeDevice || pa.device != device)
    return fail_global(MK_E_INVALID, "workspace is not device memory of the given device");

  mk_ctx* ctx = new mk_ctx();
  ctx->cfg = *cfg;
  ctx->device = device;
  ctx->stream = (hipStream_t)hip_stream;
  ctx->ws = (char*)d_workspace;
  ctx->ws_bytes = workspace_bytes;
  ctx->lay = lay;
  ctx->n_cu = prop.multiProcessorCount;
  ctx->grid = std::min(ctx->n_cu, MK_MAX_GRID);

  MkDecodeParams& p = ctx->base;
  p.n_layers = cfg->n_layers;
  p.D = cfg->hidden;
  p.ffn = cfg->ffn;
  p.vocab = cfg->vocab;
  p.H = cfg->dn_heads;
  p.dk = cfg->dn_dk;
  p.dv = cfg->dn_dv;
  p.nq = cfg->n_q_heads;
  p.nkv = cfg->n_kv_heads;
  p.hd = cfg->head_dim;
  p.max_ctx = cfg->max_ctx;
  p.max_items = lay.max_items;
  // at most 128 split-K attention items per KV head at full context; one chunk per item up to
  // 2,048 positions
  p.att_cpi = std::max(1, (cfg->max_ctx + 2047) / 2048);
  p.rms_eps = cfg->rms_eps;
  p.l2_eps = cfg->l2_eps;
  p.layers = (const MkLayerDev*)(ctx->ws + lay.descs);
  p.embed = (const uint16_t*)(ctx->ws + lay.embed);
  p.g_final = (const uint16_t*)(ctx->ws + lay.g_final);
  p.gain0 = (const uint16_t*)(ctx->ws + lay.layers[0].g12);
  p.rope_cos = (const float*)(ctx->ws + lay.rope_cos);
  p.rope_sin = (const float*)(ctx->ws + lay.rope_sin);
  p.ctl = (MkCtl*)(ctx->ws + lay.ctl);
  p.ll_am = (mk_u64*)(ctx->ws + lay.ll_am);
  p.wq4 = cfg->weight_dtype == MK_Q4G32 ? 1 : 0;
  p.kvt = kv_type(cfg->kv_dtype);
  if (p.wq4) lds_layout_q4(*cfg, ctx->grid, p);
  else lds_layout(*cfg, ctx->grid, p);

  const int lds_bytes = p.lds_floats * 4;
  const int fits = p.wq4 ? mk_decode_q4_max_blocks_per_cu(&p, lds_bytes) : mk_decode_max_blocks_per_cu(&p, lds_bytes);
  if (lds_bytes > (int)prop.sharedMemPerBlock || fits < 1) {
    const std::string m = "decode kernel needs " + std::to_string(lds_bytes) + " B of LDS; device offers " +
                          std::to_string(prop.sharedMemPerBlock);
    delete ctx;
    return fail_global(MK_E_OCCUPANCY, m);
  }

  // per-layer descriptors
  std::vector<MkLayerDev> descs(cfg->n_layers);
  for (int l = 0; l < cfg->n_layers; ++l) {
    const LayerOff& lo = lay.layers[l];
    MkLayerDev& d = descs[l];
    std::memset(&d, 0, sizeof(d));
    d.kind = is_attention(*cfg, l) ? MK_LAYER_ATT : MK_LAYER_DN;
    d.rows_in = (int32_t)lo.rows_in;
    d.w_in = (const uint16_t*)(ctx->ws + lo.w_in);
    d.w_out = (const uint16_t*)(ctx->ws + lo.w_out);
    d.w_gu = (const uint16_t*)(ctx->ws + lo.w_gu);
    d.w_down = (const uint16_t*)(ctx->ws + lo.w_down);
    d.g12 = (const uint16_t*)(ctx->ws + lo.g12);
    if (d.kind == MK_LAYER_ATT) {
      d.Kc = (float*)(ctx->ws + lo.Kc);
      d.Vc = (float*)(ctx->ws + lo.Vc);
      if (cfg->kv_dtype == MK_Q8) {
        d.Ks = (float*)(ctx->ws + lo.Ks);
        d.Vs = (float*)(ctx->ws + lo.Vs);
      }
      d.ll_part = (mk_u64*)(ctx->ws + lo.ll_part);
    } else {
      d.S = (float*)(ctx->ws + lo.S);
    }
    d.ll_in = (mk_u64*)(ctx->ws + lo.ll_in);
    d.ll_o = (mk_u64*)(ctx->ws + lo.ll_o);
    d.ll_x1 = (mk_u64*)(ctx->ws + lo.ll_x1);
    d.ll_h = (mk_u64*)(ctx->ws + lo.ll_h);
    d.ll_x2 = (mk_u64*)(ctx->ws + lo.ll_x2);
  }
  // speculative verify: its own records (vt positions each), snapshots and LDS carve
  std::vector<MkLayerDev> vdescs;
  if (lay.vt) {
    MkDecodeParams& v = ctx->vbase;
    v = p;
    v.layers = (const MkLayerDev*)(ctx->ws + lay.vdescs);
    v.ll_am = (mk_u64*)(ctx->ws + lay.v_am);
    v.ll_acc = (mk_u64*)(ctx->ws + lay.v_acc);
    v.snap_stride = lay.snap_stride;
    std::string why;
    if (p.wq4) why = lds_layout_verify_q4(*cfg, ctx->grid, v);
    else lds_layout_verify(*cfg, ctx->grid, v);
    const int vbytes = v.lds_floats * 4;
    if (!why.empty()) {
      delete ctx;
      return fail_global(MK_E_OCCUPANCY, why);
    }
    if (vbytes > (int)prop.sharedMemPerBlock ||
        (p.wq4 ? mk_verify_q4_max_blocks_per_cu(&v, vbytes) : mk_verify_max_blocks_per_cu(&v, vbytes)) < 1) {
      const std::string m = "verify kernel needs " + std::to_string(vbytes) + " B of LDS for max_verify_k = " +
                            std::to_string(cfg->max_verify_k) + "; device offers " +
                            std::to_string(prop.sharedMemPerBlock);
      delete ctx;
      return fail_global(MK_E_OCCUPANCY, m);
    }
    vdescs = descs;
    for (int l = 0; l < cfg->n_layers; ++l) {
      const LayerOff& lo = lay.layers[l];
      MkLayerDev& d = vdescs[l];
      d.ll_in = (mk_u64*)(ctx->ws + lo.v_in);
      d.ll_o = (mk_u64*)(ctx->ws + lo.v_o);
      d.ll_x1 = (mk_u64*)(ctx->ws + lo.v_x1);
      d.ll_h = (mk_u64*)(ctx->ws + lo.v_h);
      d.ll_x2 = (mk_u64*)(ctx->ws + lo.v_x2);
      if (d.kind == MK_LAYER_ATT) d.ll_part = (mk_u64*)(ctx->ws + lo.v_part);
      else d.Ssnap = (float*)(ctx->ws + lo.snap);
    }
  }
  // the decode kernel's records in the static scratch array (mk_decode_step_noalloc): the array's
  // device address on this device, looked up once per device with the device current
  {
    void* sp = nullptr;
    const char* serr = "";
    if (mk_noalloc_scratch(device, &sp, &serr) != 0) {
      delete ctx;
      return fail_global(MK_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + serr);
    }
    ctx->na_scratch = (char*)sp;
    ctx->na_fits = lay.na_bytes <= (size_t)MK_NOALLOC_SCRATCH_BYTES;
  }
  std::vector<MkLayerDev> ndescs;
  if (ctx->na_fits) {
    auto rebase = [&](mk_u64* q) { return q ? (mk_u64*)(ctx->na_scratch + ((char*)q - (ctx->ws + lay.xchg_begin))) : q; };
    ndescs = descs;
    for (MkLayerDev& d : ndescs) {
      d.ll_in = rebase(d.ll_in);
      d.ll_part = rebase(d.ll_part);
      d.ll_o = rebase(d.ll_o);
      d.ll_x1 = rebase(d.ll_x1);
      d.ll_h = rebase(d.ll_h);
      d.ll_x2 = rebase(d.ll_x2);
    }
    MkDecodeParams& q = ctx->nbase;
    q = p;
    q.layers = (const MkLayerDev*)(ctx->ws + lay.ndescs);
    q.ll_am = rebase(p.ll_am);
  }
  // RoPE tables: angle = pos * theta^(-2i/hd), evaluated in double, stored as float
  const int half = cfg->head_dim / 2;
  std::vector<float> cs((size_t)cfg->max_ctx * half), sn((size_t)cfg->max_ctx * half);
  for (int pos = 0; pos < cfg->max_ctx; ++pos)
    for (int i = 0; i < half; ++i) {
      const double inv = std::pow((double)cfg->rope_theta, -2.0 * i / cfg->head_dim);
      const double a = pos * inv;
      cs[(size_t)pos * half + i] = (float)std::cos(a);
      sn[(size_t)pos * half + i] = (float)std::sin(a);
    }
  int rc = MK_OK;
  auto hip_ok = [&](hipError_t er, const char* what) {
    if (er != hipSuccess && rc == MK_OK) {
      rc = MK_E_HIP;
      g_err = std::string(what) + ": " + hipGetErrorString(er);
    }
  };
  hip_ok(hipMemcpyAsync(ctx->ws + lay.descs, descs.data(), sizeof(MkLayerDev) * descs.size(), hipMemcpyHostToDevice,
                        ctx->stream), "copy layer descriptors");
  if (lay.vt)
    hip_ok(hipMemcpyAsync(ctx->ws + lay.vdescs, vdescs.data(), sizeof(MkLayerDev) * vdescs.size(),
                          hipMemcpyHostToDevice, ctx->stream), "copy verify layer descriptors");
  if (ctx->na_fits)
    hip_ok(hipMemcpyAsync(ctx->ws + lay.ndescs, ndescs.data(), sizeof(MkLayerDev) * ndescs.size(),
                          hipMemcpyHostToDevice, ctx->stream), "copy static-record layer descriptors");
  hip_ok(hipMemcpyAsync(ctx->ws + lay.rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, ctx->stream),
         "copy rope cos");
  hip_ok(hipMemcpyAsync(ctx->ws + lay.rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, ctx->stream),
         "copy rope sin");
  if (rc == MK_OK && mk_launch_zero(ctx->ws + lay.ctl, sizeof(MkCtl), ctx->stream)) rc = MK_E_HIP;
  if (rc == MK_OK && mk_launch_zero(ctx->ws + lay.state_begin, lay.state_end - lay.state_begin, ctx->stream)) rc = MK_E_HIP;
  if (rc == MK_OK && mk_launch_zero(ctx->ws + lay.xchg_begin, lay.xchg_end - lay.xchg_begin, ctx->stream)) rc = MK_E_HIP;
  if (rc == MK_OK && mk_launch_set_ctl(p.ctl, 0, 1, 0, ctx->stream)) rc = MK_E_HIP;
  if (rc == MK_OK) hip_ok(hipStreamSynchronize(ctx->stream), "synchronise after create");
  if (rc != MK_OK) {
    if (g_err.empty()) g_err = "kernel launch failed during create";
    delete ctx;
    return rc;
  }
  *out = ctx;
  return MK_OK;
}

void mk_destroy(mk_ctx* ctx) {
  if (!ctx) return;
  (void)hipStreamSynchronize(ctx->stream);
  delete ctx;
}

int mk_set_grid(mk_ctx* ctx, int32_t n) {
  if (!ctx) return fail_global(MK_E_INVALID, "ctx is NULL");
  if (n < 1 || n > ctx->n_cu || n > MK_MAX_GRID)
    return fail(ctx, MK_E_INVALID, "grid must be in [1, " + std::to_string(std::min(ctx->n_cu, MK_MAX_GRID)) + "]");
  MkDecodeParams q = ctx->base;
  if (q.wq4) lds_layout_q4(ctx->cfg, n, q);
  else lds_layout(ctx->cfg, n, q);
  if ((q.wq4 ? mk_decode_q4_max_blocks_per_cu(&q, q.lds_floats * 4) : mk_decode_max_blocks_per_cu(&q, q.lds_floats * 4)) < 1)
    return fail(ctx, MK_E_OCCUPANCY, "decode kernel does not fit at this grid size");
  MkDecodeParams v = ctx->vbase;
  if (ctx->lay.vt) {
    if (v.wq4) {
      const std::string why = lds_layout_verify_q4(ctx->cfg, n, v);
      if (!why.empty()) return fail(ctx, MK_E_OCCUPANCY, why);
    } else {
      lds_layout_verify(ctx->cfg, n, v);
    }
    if ((v.wq4 ? mk_verify_q4_max_blocks_per_cu(&v, v.lds_floats * 4) : mk_verify_max_blocks_per_cu(&v, v.lds_floats * 4)) < 1)
      return fail(ctx, MK_E_OCCUPANCY, "verify kernel does not fit at this grid size");
  }
  ctx->base = q;
  ctx->vbase = v;
  if (ctx->na_fits) {
    const MkDecodeParams keep = ctx->nbase;
    ctx->nbase = q;
    ctx->nbase.layers = keep.layers;
    ctx->nbase.ll_am = keep.ll_am;
  }
  ctx->grid = n;
  return MK_OK;
}

int mk_get_grid(const mk_ctx* ctx, int32_t* n) {
  if (!ctx || !n) return fail_global(MK_E_INVALID, "NULL argument");
  *n = ctx->grid;
  return MK_OK;
}

int mk_reset(mk_ctx* ctx) {
  if (!ctx) return fail_global(MK_E_INVALID, "ctx is NULL");
  const Layout& lay = ctx->lay;
  if (mk_launch_zero(ctx->ws + lay.state_begin, lay.state_end - lay.state_begin, ctx->stream))
    return fail(ctx, MK_E_HIP, "zero state launch failed");
  // exchange words too, so that a launch that gave up leaves nothing behind; the epoch moves on
  if (mk_launch_zero(ctx->ws + lay.xchg_begin, lay.xchg_end - lay.xchg_begin, ctx->stream))
    return fail(ctx, MK_E_HIP, "zero exchange launch failed");
  if (mk_launch_set_ctl(ctx->base.ctl, 0, 1, 1, ctx->stream)) return fail(ctx, MK_E_HIP, "set position launch failed");
  ctx->pos_host = 0;
  ctx->pos_exact = true;
  return MK_OK;
}

int mk_load_weights(mk_ctx* ctx, const mk_tensor* t, int32_t n) {
  if (!ctx) return fail_global(MK_E_INVALID, "ctx is NULL");
  const mk_config& c = ctx->cfg;
  std::string msg;
  std::vector<int> order;
  int rc = check_tensor_list(c, t, n, msg, &order);
  if (rc != MK_OK) return fail(ctx, rc, msg);
  HIPCHK(ctx, hipSetDevice(ctx->device));
  const std::vector<TensorSpec> man = manifest(c);
  const bool q4 = c.weight_dtype == MK_Q4G32;
  // bytes of a tensor as stored: BF16 gains and matrices, or Q4G32 matrices
  auto tbytes = [&](const std::vector<int64_t>& shape) -> size_t {
    if (q4 && shape.size() == 2) return (size_t)(shape[0] * shape[1] / 2 + shape[0] * (shape[1] / 32) * 4);
    size_t b = 2;
    for (int64_t d : shape) b *= (size_t)d;
    return b;
  };
  // stage host tensors through one device buffer sized for the largest tensor
  size_t max_bytes = 0;
  for (size_t i = 0; i < man.size(); ++i) max_bytes = std::max(max_bytes, tbytes(man[i].shape));
  void* stage = nullptr;
  int32_t* d_perm = nullptr;
  HIPCHK(ctx, hipMalloc(&stage, max_bytes));
  int64_t max_rows = std::max<int64_t>(2 * (int64_t)c.ffn, (int64_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim);
  if (hipMalloc(&d_perm, max_rows * 4) != hipSuccess) {
    (void)hipFree(stage);
    return fail(ctx, MK_E_HIP, "hipMalloc permutation buffer failed");
  }
  const Layout& lay = ctx->lay;
  auto src_of = [&](const mk_tensor& tt, size_t bytes, const void** out) -> int {
    if (tt.on_device) {
      *out = tt.data;
      return MK_OK;
    }
    if (hipMemcpyAsync(stage, tt.data, bytes, hipMemcpyHostToDevice, ctx->stream) != hipSuccess) return MK_E_HIP;
    *out = stage;
    return MK_OK;
  };
  auto tensor = [&](const std::string& name) -> const mk_tensor& {
    for (size_t i = 0; i < man.size(); ++i)
      if (man[i].name == name) return t[order[i]];
    return t[0];  // unreachable: the list was checked
  };
  // 4-bit matrices are assembled in their input layout in a device buffer, then tiled into place
  char* asm_buf = nullptr;
  if (q4) {
    size_t mb = 0;
    for (int l = 0; l < c.n_layers; ++l) {
      const LayerOff& lo = lay.layers[l];
      mb = std::max(mb, (size_t)(lo.rows_in * c.hidden * 5 / 8));
      mb = std::max(mb, (size_t)(c.hidden * lo.k_out * 5 / 8));
    }
    mb = std::max(mb, (size_t)(2 * (int64_t)c.ffn * c.hidden * 5 / 8));
    mb = std::max(mb, (size_t)((int64_t)c.vocab * c.hidden * 5 / 8));
    if (hipMalloc(&asm_buf, mb) != hipSuccess) {
      (void)hipFree(stage);
      (void)hipFree(d_perm);
      return fail(ctx, MK_E_HIP, "hipMalloc 4-bit assembly buffer failed");
    }
  }
  auto copy_bytes = [&](const mk_tensor& tt, size_t src_off, char* dst, size_t bytes) -> int {
    const hipMemcpyKind k = tt.on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;
    return hipMemcpyAsync(dst, (const char*)tt.data + src_off, bytes, k, ctx->stream) == hipSuccess ? MK_OK : MK_E_HIP;
  };
  // assembled matrix (asm_buf) of R rows, K columns -> its tiled region
  auto tile = [&](size_t dst_off, int64_t R, int64_t K) -> int {
    if (mk_launch_q4_tile(asm_buf, R, K, ctx->ws + dst_off, ctx->stream)) return MK_E_HIP;
    return hipStreamSynchronize(ctx->stream) == hipSuccess ? MK_OK : MK_E_HIP;  // asm_buf is reused
  };
  // a gain vector, or a whole matrix that is a region of its own
  auto copy_plain = [&](const std::string& name, size_t dst_off) -> int {
    const mk_tensor& tt = tensor(name);
    std::vector<int64_t> shape(tt.shape, tt.shape + tt.ndim);
    if (q4 && tt.ndim == 2) {
      if (copy_bytes(tt, 0, asm_buf, tbytes(shape))) return MK_E_HIP;
      return tile(dst_off, tt.shape[0], tt.shape[1]);
    }
    return copy_bytes(tt, 0, ctx->ws + dst_off, tbytes(shape));
  };
  // Matrix `name` [R][K] -> rows row0 .. row0 + R of the matrix at `base` that has Rtot rows and K
  // columns (the workspace region for BF16, the assembly buffer for Q4G32, whose input layout is
  // all rows' codes followed by all rows' (d, m) words, so the two parts move separately); with
  // perm, source row r goes to row row0 + perm[r].
  auto put_rows = [&](const std::string& name, char* base, int64_t Rtot, int64_t row0,
                      const std::vector<int32_t>* perm) -> int {
    const mk_tensor& tt = tensor(name);
    const int64_t R = tt.shape[0], K = tt.shape[1];
    // (bytes per row, source offset, destination) of each part
    struct Part {
      int64_t row_bytes;
      size_t src;
      char* dst;
    };
    std::vector<Part> parts;
    if (q4) {
      parts.push_back({K / 2, 0, base + (size_t)(row0 * (K / 2))});
      parts.push_back({(K / 32) * 4, (size_t)(R * (K / 2)), base + (size_t)(Rtot * (K / 2) + row0 * (K / 32) * 4)});
    } else {
      parts.push_back({K * 2, 0, base + (size_t)(row0 * K * 2)});
    }
    if (!perm) {
      for (const Part& pt : parts)
        if (copy_bytes(tt, pt.src, pt.dst, (size_t)(R * pt.row_bytes))) return MK_E_HIP;
      return MK_OK;
    }
    std::vector<int64_t> shape(tt.shape, tt.shape + tt.ndim);
    const void* src = nullptr;
    if (src_of(tt, tbytes(shape), &src)) return MK_E_HIP;
    if (hipMemcpyAsync(d_perm, perm->data(), R * 4, hipMemcpyHostToDevice, ctx->stream) != hipSuccess) return MK_E_HIP;
    for (const Part& pt : parts)
      if (mk_launch_permute_rows((const uint16_t*)((const char*)src + pt.src), (uint16_t*)pt.dst, d_perm, R,
                                 pt.row_bytes / 2, ctx->stream))
        return MK_E_HIP;
    // the staging buffers are reused by the next tensor
    return hipStreamSynchronize(ctx->stream) == hipSuccess ? MK_OK : MK_E_HIP;
  };
  auto mat_base = [&](size_t region) { return q4 ? asm_buf : ctx->ws + region; };

  const int64_t D = c.hidden, H = c.dn_heads;
  const int hd = c.head_dim, half = hd / 2;
  rc = copy_plain("embed", lay.embed);
  if (!rc) rc = copy_plain("final_norm", lay.g_final);
  for (int l = 0; l < c.n_layers && !rc; ++l) {
    const LayerOff& lo = lay.layers[l];
    const std::string p = "l" + std::to_string(l) + ".";
    rc = copy_plain(p + "norm1", lo.g12);
    if (!rc) rc = copy_plain(p + "norm2", lo.g12 + (size_t)D * 2);
    if (rc) break;
    if (is_attention(c, l)) {
      // rows of every head in RoPE pair order: (0, hd/2, 1, hd/2 + 1, ...)
      auto pair_perm = [&](int heads) {
        std::vector<int32_t> pm((size_t)heads * hd);
        for (int h = 0; h < heads; ++h)
          for (int d = 0; d < hd; ++d) pm[(size_t)h * hd + d] = h * hd + 2 * (d % half) + d / half;
        return pm;
      };
      const std::vector<int32_t> pq = pair_perm(c.n_q_heads), pk = pair_perm(c.n_kv_heads);
      char* base = mat_base(lo.w_in);
      rc = put_rows(p + "attn.wq", base, lo.rows_in, 0, &pq);
      if (!rc) rc = put_rows(p + "attn.wk", base, lo.rows_in, (int64_t)c.n_q_heads * hd, &pk);
      if (!rc) rc = put_rows(p + "attn.wv", base, lo.rows_in, (int64_t)(c.n_q_heads + c.n_kv_heads) * hd, &pk);
      if (!rc && q4) rc = tile(lo.w_in, lo.rows_in, D);
      if (!rc) rc = copy_plain(p + "attn.wo", lo.w_out);
    } else {
      const int64_t nqkv = 2 * H * c.dn_dk + H * c.dn_dv;
      char* base = mat_base(lo.w_in);
      rc = put_rows(p + "dn.wqkv", base, lo.rows_in, 0, nullptr);
      if (!rc) rc = put_rows(p + "dn.wa", base, lo.rows_in, nqkv, nullptr);
      if (!rc) rc = put_rows(p + "dn.wb", base, lo.rows_in, nqkv + H, nullptr);
      if (!rc && q4) rc = tile(lo.w_in, lo.rows_in, D);
      if (!rc) rc = copy_plain(p + "dn.wo", lo.w_out);
    }
    if (rc) break;
    std::vector<int32_t> pg(c.ffn), pu(c.ffn);
    for (int j = 0; j < c.ffn; ++j) {
      pg[j] = 2 * j;
      pu[j] = 2 * j + 1;
    }
    char* base = mat_base(lo.w_gu);
    rc = put_rows(p + "ffn.wg", base, 2 * (int64_t)c.ffn, 0, &pg);
    if (!rc) rc = put_rows(p + "ffn.wu", base, 2 * (int64_t)c.ffn, 0, &pu);
    if (!rc && q4) rc = tile(lo.w_gu, 2 * (int64_t)c.ffn, D);
    if (!rc) rc = copy_plain(p + "ffn.wd", lo.w_down);
  }
  const hipError_t se = hipStreamSynchronize(ctx->stream);
  (void)hipFree(stage);
  (void)hipFree(d_perm);
  if (asm_buf) (void)hipFree(asm_buf);
  if (rc) return fail(ctx, rc, "copying weights failed");
  if (se != hipSuccess) return fail(ctx, MK_E_HIP, std::string("weight copy: ") + hipGetErrorString(se));
  ctx->loaded = true;
  rc = mk_reset(ctx);
  if (rc) return rc;
  // warm-up launch (the output is discarded), then back to position 0
  int32_t* scratch_tok = (int32_t*)(ctx->ws + lay.scratch);
  HIPCHK(ctx, hipMemsetAsync(scratch_tok, 0, 64, ctx->stream));
  rc = mk_decode_step(ctx, scratch_tok, scratch_tok + 1, nullptr);
  if (rc) return rc;
  rc = mk_sync(ctx);
  if (rc) return rc;
  return mk_reset(ctx);
}

int mk_decode_step(mk_ctx* ctx, const int32_t* d_tok, int32_t* d_next, float* d_logits) {
  if (!ctx) return fail_global(MK_E_INVALID, "ctx is NULL");
  if (!ctx->loaded) return fail(ctx, MK_E_ORDER, "weights are not loaded");
  if (!d_tok || !d_next) return fail(ctx, MK_E_INVALID, "d_tok and d_next are required");
  if (ctx->pos_host + 1 > ctx->cfg.max_ctx && refresh_position(ctx) != MK_OK) return MK_E_HIP;
  if (ctx->pos_host + 1 > ctx->cfg.max_ctx) return fail(ctx, MK_E_CTX_FULL, "context is full");
  MkDecodeParams p = ctx->base;
  p.tok = d_tok;
  p.next = d_next;
  p.logits = d_logits;
  if ((p.wq4 ? mk_launch_decode_q4(&p, ctx->grid, ctx->stream) : mk_launch_decode(&p, ctx->grid, ctx->stream)))
    return fail(ctx, MK_E_HIP, "decode launch failed");
  ctx->pos_host += 1;
  return MK_OK;
}

int mk_decode_step_noalloc(mk_ctx* ctx, const int32_t* d_tok, int32_t* d_next, float* d_logits) {
  if (!ctx) return fail_global(MK_E_INVALID, "ctx is NULL");
  if (!ctx->na_fits)
    return fail(ctx, MK_E_UNSUPPORTED, "this model's decode records need " + std::to_string(ctx->lay.na_bytes) +
                                            " bytes; the static scratch array holds " +
                                            std::to_string((size_t)MK_NOALLOC_SCRATCH_BYTES));
  if (!ctx->loaded) return fail(ctx, MK_E_ORDER, "weights are not loaded");
  if (!d_tok || !d_next) return fail(ctx, MK_E_INVALID, "d_tok and d_next are required");
  if (ctx->pos_host + 1 > ctx->cfg.max_ctx && refresh_position(ctx) != MK_OK) return MK_E_HIP;
  if (ctx->pos_host + 1 > ctx->cfg.max_ctx) return fail(ctx, MK_E_CTX_FULL, "context is full");
  MkDecodeParams p = ctx->nbase;
  p.tok = d_tok;
  p.next = d_next;
  p.logits = d_logits;
  // the array holds the last call's records, possibly another context's with a matching epoch:
  // clear the part this launch polls (a fill kernel, no memset node)
  if (mk_launch_zero(ctx->na_scratch, (int64_t)ctx->lay.na_bytes, ctx->stream))
    return fail(ctx, MK_E_HIP, "clearing the static records failed");
  if ((p.wq4 ? mk_launch_decode_q4(&p, ctx->grid, ctx->stream) : mk_launch_decode(&p, ctx->grid, ctx->stream)))
    return fail(ctx, MK_E_HIP, "decode launch failed");
  ctx->pos_host += 1;
  return MK_OK;
}

int mk_prefill(mk_ctx* ctx, const int32_t* d_tokens, int32_t n, int32_t* d_next, float* d_logits) {
  if (!ctx) return fail_global(MK_E_INVALID, "ctx is NULL");
  if (!ctx->loaded) return fail(ctx, MK_E_ORDER, "weights are not loaded");
  if (!d_tokens || !d_next || n <= 0) return fail(ctx, MK_E_INVALID, "need d_tokens, d_next and n > 0");
  // the prefill kernels take the start position from the host
  if (!ctx->pos_exact && refresh_position(ctx) != MK_OK) return MK_E_HIP;
  if (ctx->pos_host + n > ctx->cfg.max_ctx) return fail(ctx, MK_E_CTX_FULL, "prompt does not fit the context");
  const mk_config& c = ctx->cfg;
  const int gs = c.n_q_heads / c.n_kv_heads;
  const int kvt = ctx->base.kvt;
  const bool q4 = ctx->base.wq4;
  // the matrix-core attention (head size 64 or 128) takes any head grouping and cache type; the
  // VALU one needs groups dividing 16 and an FP32 cache
  const bool mfma_att = c.head_dim == 64 || c.head_dim == 128;
  if (!mfma_att && (16 % gs != 0 || kvt != MK_KV_F32)) {
    // shapes the prefill attention does not cover: token by token through the decode kernel
    int32_t* scratch_tok = (int32_t*)(ctx->ws + ctx->lay.scratch) + 8;
    for (int32_t i = 0; i < n; ++i) {
      const bool last = (i == n - 1);
      const int rc = mk_decode_step(ctx, d_tokens + i, last ? d_next : scratch_tok, last ? d_logits : nullptr);
      if (rc) return rc;
    }
    return MK_OK;
  }
  const Layout& L = ctx->lay;
  char* ws = ctx->ws;
  void* st = ctx->stream;
  const int D = c.hidden, H = c.dn_heads, dk = c.dn_dk, dv = c.dn_dv, hd = c.head_dim;
  const int nq = c.n_q_heads, nkv = c.n_kv_heads, F = c.ffn;
  float* X = (float*)(ws + L.pf_x);
  uint16_t* Ahi = (uint16_t*)(ws + L.pf_ahi);
  uint16_t* Alo = (uint16_t*)(ws + L.pf_alo);
  uint16_t* Hhi = (uint16_t*)(ws + L.pf_hhi);
  uint16_t* Hlo = (uint16_t*)(ws + L.pf_hlo);
  float* Y = (float*)(ws + L.pf_y);
  float* QK = (float*)(ws + L.pf_qk);
  float* AB = (float*)(ws + L.pf_ab);
  float* Q = (float*)(ws + L.pf_q);
  const int lda = L.pf_lda, ldy = L.pf_ldy, ldh = L.pf_ldh;
  float* PK = (float*)(ws + L.pf_sk);
  const size_t PKN = PF_SPLITK_FLOATS;
  MkCtl* ctl = (MkCtl*)(ws + L.ctl);
  const float* rcos = (const float*)(ws + L.rope_cos);
  const float* rsin = (const float*)(ws + L.rope_sin);
  const uint16_t* embed = (const uint16_t*)(ws + L.embed);
  uint16_t* Wq = q4 ? (uint16_t*)(ws + L.pf_wq) : nullptr;
  // a GEMM's weights and inner size: BF16 weights as stored, or a 4-bit matrix expanded to
  // [W_hi | W_lo] with its activations (hi, lo, leading dimension ld) widened to match
  int rc = 0;
  int T = 0;  // tokens of the current chunk
  auto operand = [&](uint16_t* hi, uint16_t* lo, int ld, const uint16_t* w, int N, int K, int& KK) -> const uint16_t* {
    if (!q4) {
      KK = K;
      return w;
    }
    rc |= mk_pf_widen(hi, lo, ld, T, K, st);
    rc |= mk_pf_q4_expand(w, N, K, Wq, st);
    KK = 2 * K;
    return Wq;
  };
  // the 4-bit path leaves the last prompt token to a decode launch, which forms its logits
  const int32_t ngemm = q4 ? n - 1 : n;
  int p0 = ctx->pos_host;
  for (int c0 = 0; c0 < ngemm && !rc; c0 += T) {
    T = std::min(L.pf_T, ngemm - c0);
    if (q4) rc |= mk_pf_embed_q4(d_tokens + c0, T, embed, D, c.vocab, X, ctl, st);
    else rc |= mk_pf_embed(d_tokens + c0, T, embed, D, c.vocab, X, ctl, st);
    rc |= mk_pf_rms_split(X, T, D, (const uint16_t*)(ws + L.layers[0].g12), c.rms_eps, Ahi, Alo, lda, st);
    for (int l = 0; l < c.n_layers && !rc; ++l) {
      const LayerOff& lo = L.layers[l];
      const uint16_t* g12 = (const uint16_t*)(ws + lo.g12);
      // the next layer's input norm rides on this layer's last residual add
      const uint16_t* g_next = l + 1 < c.n_layers ? (const uint16_t*)(ws + L.layers[l + 1].g12) : nullptr;
      int K;
      const uint16_t* W = operand(Ahi, Alo, lda, (const uint16_t*)(ws + lo.w_in), (int)lo.rows_in, D, K);
      rc |= mk_pf_gemm(0, Ahi, Alo, lda, T, K, W, (int)lo.rows_in, Y, ldy, nullptr, nullptr, 0, PK, PKN, st);
      if (is_attention(c, l)) {
        float* Kc = (float*)(ws + lo.Kc);
        float* Vc = (float*)(ws + lo.Vc);
        if (kvt == MK_KV_F32) {
          rc |= mk_pf_att_rope(Y, ldy, T, p0, nq, nkv, hd, rcos, rsin, Q, Kc, Vc, c.max_ctx, p0, st);
        } else {
          // rotated rows of this chunk in FP32, then stored in the cache type
          float* Kf = (float*)(ws + L.pf_kvf);
          float* Vf = Kf + (size_t)nkv * T * hd;
          rc |= mk_pf_att_rope(Y, ldy, T, p0, nq, nkv, hd, rcos, rsin, Q, Kf, Vf, T, 0, st);
          rc |= mk_pf_kv_pack(Kf, Vf, T, nkv, hd, kvt, Kc, Vc, (float*)(ws + lo.Ks), (float*)(ws + lo.Vs), c.max_ctx,
                              p0, st);
        }
        rc |= mk_pf_attention(Q, Kc, Vc, kvt, kvt == MK_KV_Q8 ? (const float*)(ws + lo.Ks) : nullptr,
                              kvt == MK_KV_Q8 ? (const float*)(ws + lo.Vs) : nullptr, T, p0, nq, nkv, hd, c.max_ctx,
                              Ahi, Alo, lda, PK, PKN, st);
      } else {
        rc |= mk_pf_dn_scan((float*)(ws + lo.S), QK, AB, Y, ldy, T, H, dk, dv, c.l2_eps, Ahi, Alo, lda,
                            (float*)(ws + L.pf_ch), st);
      }
      W = operand(Ahi, Alo, lda, (const uint16_t*)(ws + lo.w_out), D, (int)lo.k_out, K);
      rc |= mk_pf_gemm_res(Ahi, Alo, lda, T, K, W, D, X, D, PK, PKN, g12 + D, c.rms_eps, Ahi, Alo, lda, st);
      W = operand(Ahi, Alo, lda, (const uint16_t*)(ws + lo.w_gu), 2 * F, D, K);
      rc |= mk_pf_gemm(2, Ahi, Alo, lda, T, K, W, 2 * F, nullptr, 0, Hhi, Hlo, ldh, PK, PKN, st);
      W = operand(Hhi, Hlo, ldh, (const uint16_t*)(ws + lo.w_down), D, F, K);
      rc |= mk_pf_gemm_res(Hhi, Hlo, ldh, T, K, W, D, X, D, PK, PKN, g_next, c.rms_eps, Ahi, Alo, lda, st);
    }
    p0 += T;
  }
  if (rc) return fail(ctx, MK_E_HIP, "prefill launch failed");
  if (q4) {
    // the last token: one 4-bit decode launch at position p0 (LM head and greedy choice included)
    if (ngemm > 0 && mk_launch_set_ctl(ctl, p0, 0, 0, st)) return fail(ctx, MK_E_HIP, "prefill launch failed");
    ctx->pos_host = p0;
    ctx->pos_exact = true;
    return mk_decode_step(ctx, d_tokens + n - 1, d_next, d_logits);
  }
  float* part = (float*)(ws + L.pf_part);
  rc |= mk_pf_lmhead(X + (size_t)(T - 1) * D, D, (const uint16_t*)(ws + L.g_final), c.rms_eps, embed, c.vocab,
                     d_logits, part, PF_LM_WG, st);
  rc |= mk_pf_finish(part, PF_LM_WG, d_next, ctl, p0, st);
  if (rc) return fail(ctx, MK_E_HIP, "prefill launch failed");
  ctx->pos_host = p0;
  return MK_OK;
}

int mk_set_trace(mk_ctx* ctx, void* d_trace, size_t bytes) {
  if (!ctx) return fail_global(MK_E_INVALID, "ctx is NULL");
  if (d_trace && bytes < (size_t)ctx->grid * MK_TRACE_EVENTS * 8)
    return fail(ctx, MK_E_INVALID, "trace buffer needs grid * " + std::to_string(MK_TRACE_EVENTS) + " * 8 bytes");
  ctx->base.trace = (unsigned long long*)d_trace;
  ctx->vbase.trace = (unsigned long long*)d_trace;
  ctx->nbase.trace = (unsigned long long*)d_trace;
  return MK_OK;
}

int mk_verify_k(mk_ctx* ctx, const int32_t* d_tokens, int32_t k, int32_t* d_out, int32_t* d_n_accepted) {
  if (!ctx) return fail_global(MK_E_INVALID, "ctx is NULL");
  if (!ctx->loaded) return fail(ctx, MK_E_ORDER, "weights are not loaded");
  if (!d_tokens || !d_out || !d_n_accepted) return fail(ctx, MK_E_INVALID, "d_tokens, d_out and d_n_accepted are required");
  if (ctx->lay.vt == 0) return fail(ctx, MK_E_INVALID, "the context was created with max_verify_k = 0");
  if (k < 0 || k > ctx->cfg.max_verify_k)
    return fail(ctx, MK_E_INVALID, "k must be in [0, " + std::to_string(ctx->cfg.max_verify_k) + "]");
  if (ctx->pos_host + k + 1 > ctx->cfg.max_ctx && refresh_position(ctx) != MK_OK) return MK_E_HIP;
  if (ctx->pos_host + k + 1 > ctx->cfg.max_ctx) return fail(ctx, MK_E_CTX_FULL, "the drafts do not fit the context");
  MkDecodeParams p = ctx->vbase;
  p.nt = k + 1;
  p.vtok = d_tokens;
  p.vout = d_out;
  p.vacc = d_n_accepted;
  if ((p.wq4 ? mk_launch_verify_q4(&p, ctx->grid, ctx->stream) : mk_launch_verify(&p, ctx->grid, ctx->stream)))
    return fail(ctx, MK_E_HIP, "verify launch failed");
  ctx->pos_host += k + 1;
  ctx->pos_exact = false;
  return MK_OK;
}

int mk_sync(mk_ctx* ctx) {
  if (!ctx) return fail_global(MK_E_INVALID, "ctx is NULL");
  HIPCHK(ctx, hipStreamSynchronize(ctx->stream));
  MkCtl ctl;
  HIPCHK(ctx, hipMemcpy(&ctl, ctx->base.ctl, sizeof(ctl), hipMemcpyDeviceToHost));
  if (ctl.err) {
    // clear the flag so that the next launch starts clean; the sequence state is undefined now
    if (mk_launch_set_ctl(ctx->base.ctl, -1, 1, 0, ctx->stream) == 0) (void)hipStreamSynchronize(ctx->stream);
    if (ctl.err == 2u)
      return fail(ctx, MK_E_INVALID,
                  "a decode or verify launch saw a token id outside [0, vocab) or a full context; call mk_reset");

    return fail(ctx, MK_E_DEVICE_TIMEOUT, "a grid-wide wait inside a persistent kernel gave up; call mk_reset");
  }
  // every completed launch advances the device position; a launch that left early does not
  if (ctx->pos_exact && (int64_t)ctl.pos != ctx->pos_host)
    return fail(ctx, MK_E_DEVICE_TIMEOUT,
                "the device position (" + std::to_string(ctl.pos) + ") is behind the enqueued positions (" +
                    std::to_string(ctx->pos_host) + "): a launch ended early; call mk_reset");
  return MK_OK;
}

int mk_get_position(mk_ctx* ctx, int32_t* pos) {
  if (!ctx || !pos) return fail_global(MK_E_INVALID, "NULL argument");
  HIPCHK(ctx, hipStreamSynchronize(ctx->stream));
  MkCtl ctl;
  HIPCHK(ctx, hipMemcpy(&ctl, ctx->base.ctl, sizeof(ctl), hipMemcpyDeviceToHost));
  *pos = ctl.pos;
  if (!ctl.err) {
    ctx->pos_host = ctl.pos;
    ctx->pos_exact = true;
  }
  return MK_OK;
}

int mk_set_position(mk_ctx* ctx, int32_t pos) {
  if (!ctx) return fail_global(MK_E_INVALID, "ctx is NULL");
  if (pos < 0 || pos > ctx->cfg.max_ctx) return fail(ctx, MK_E_INVALID, "position outside [0, max_ctx]");
  if (mk_launch_set_ctl(ctx->base.ctl, pos, 0, 0, ctx->stream)) return fail(ctx, MK_E_HIP, "set position launch failed");
  ctx->pos_host = pos;
  ctx->pos_exact = true;
  return MK_OK;
}

size_t mk_state_bytes(const mk_ctx* ctx, int32_t layer) {
  if (!ctx || layer < 0 || layer >= ctx->cfg.n_layers) return 0;
  const mk_config& c = ctx->cfg;
  if (is_attention(c, layer)) return (size_t)2 * c.n_kv_heads * c.max_ctx * c.head_dim * 4;
  return (size_t)c.dn_heads * c.dn_dv * c.dn_dk * 4;
}

int mk_read_state(mk_ctx* ctx, int32_t layer, void* dst) {
  if (!ctx || !dst) return fail_global(MK_E_INVALID, "NULL argument");
  if (layer < 0 || layer >= ctx->cfg.n_layers) return fail(ctx, MK_E_INVALID, "layer out of range");
  HIPCHK(ctx, hipStreamSynchronize(ctx->stream));
  const LayerOff& lo = ctx->lay.layers[layer];
  const size_t b = mk_state_bytes(ctx, layer);
  if (!is_attention(ctx->cfg, layer)) {
    HIPCHK(ctx, hipMemcpy(dst, ctx->ws + lo.S, b, hipMemcpyDeviceToHost));
    return MK_OK;
  }
  const mk_config& c = ctx->cfg;
  const int kvt = kv_type(c.kv_dtype);
  if (kvt == MK_KV_F32) {
    HIPCHK(ctx, hipMemcpy(dst, ctx->ws + lo.Kc, b / 2, hipMemcpyDeviceToHost));
    HIPCHK(ctx, hipMemcpy((char*)dst + b / 2, ctx->ws + lo.Vc, b / 2, hipMemcpyDeviceToHost));
    return MK_OK;
  }
  // compact caches: the stored values, decoded to FP32
  const size_t n = (size_t)c.n_kv_heads * c.max_ctx * c.head_dim, nb = n / MK_KV_Q8_BLOCK;
  std::vector<char> raw(n * kv_elem_bytes(kvt));
  std::vector<float> sc(kvt == MK_KV_Q8 ? nb : 0);
  for (int v = 0; v < 2; ++v) {
    HIPCHK(ctx, hipMemcpy(raw.data(), ctx->ws + (v ? lo.Vc : lo.Kc), raw.size(), hipMemcpyDeviceToHost));
    float* out = (float*)dst + v * n;
    if (kvt == MK_KV_F16) {
      const _Float16* h = (const _Float16*)raw.data();
      for (size_t i = 0; i < n; ++i) out[i] = (float)h[i];
    } else {
      HIPCHK(ctx, hipMemcpy(sc.data(), ctx->ws + (v ? lo.Vs : lo.Ks), nb * 4, hipMemcpyDeviceToHost));
      const signed char* q = (const signed char*)raw.data();
      for (size_t i = 0; i < n; ++i) out[i] = (float)q[i] * sc[i / MK_KV_Q8_BLOCK];
    }
  }
  return MK_OK;
}

int mk_write_state(mk_ctx* ctx, int32_t layer, const void* src) {
  if (!ctx || !src) return fail_global(MK_E_INVALID, "NULL argument");
  if (layer < 0 || layer >= ctx->cfg.n_layers) return fail(ctx, MK_E_INVALID, "layer out of range");
  HIPCHK(ctx, hipStreamSynchronize(ctx->stream));
  const LayerOff& lo = ctx->lay.layers[layer];
  const size_t b = mk_state_bytes(ctx, layer);
  if (!is_attention(ctx->cfg, layer)) {
    HIPCHK(ctx, hipMemcpy(ctx->ws + lo.S, src, b, hipMemcpyHostToDevice));
    return MK_OK;
  }
  const mk_config& c = ctx->cfg;
  const int kvt = kv_type(c.kv_dtype);
  if (kvt == MK_KV_F32) {
    HIPCHK(ctx, hipMemcpy(ctx->ws + lo.Kc, src, b / 2, hipMemcpyHostToDevice));
    HIPCHK(ctx, hipMemcpy(ctx->ws + lo.Vc, (const char*)src + b / 2, b / 2, hipMemcpyHostToDevice));
    return MK_OK;
  }
  // compact caches: FP32 values -> the cache type (nearest binary16; int8 blocks as the kernels form them)
  const size_t n = (size_t)c.n_kv_heads * c.max_ctx * c.head_dim, nb = n / MK_KV_Q8_BLOCK;
  std::vector<char> raw(n * kv_elem_bytes(kvt));
  std::vector<float> sc(kvt == MK_KV_Q8 ? nb : 0);
  for (int v = 0; v < 2; ++v) {
    const float* in = (const float*)src + v * n;
    if (kvt == MK_KV_F16) {
      _Float16* h = (_Float16*)raw.data();
      for (size_t i = 0; i < n; ++i) h[i] = (_Float16)in[i];
    } else {
      signed char* q = (signed char*)raw.data();
      for (size_t bi = 0; bi < nb; ++bi) {
        float m = 0.f;
        for (int i = 0; i < MK_KV_Q8_BLOCK; ++i) m = std::fmax(m, std::fabs(in[bi * MK_KV_Q8_BLOCK + i]));
        const float s = m / 127.0f;
        sc[bi] = s;
        for (int i = 0; i < MK_KV_Q8_BLOCK; ++i)
          q[bi * MK_KV_Q8_BLOCK + i] = (signed char)(int)(s > 0.f ? std::nearbyint(in[bi * MK_KV_Q8_BLOCK + i] / s) : 0.f);
      }
      HIPCHK(ctx, hipMemcpy(ctx->ws + (v ? lo.Vs : lo.Ks), sc.data(), nb * 4, hipMemcpyHostToDevice));
    }
    HIPCHK(ctx, hipMemcpy(ctx->ws + (v ? lo.Vc : lo.Kc), raw.data(), raw.size(), hipMemcpyHostToDevice));
  }
  return MK_OK;
}

}  // extern "C"

// extern "C" entry points of libtfm.so (declared and documented in include/tfm.h).
// Host side only: argument validation, workspace planning and the launch sequence of the
// pre-norm decoder block ("Transformer 篇" (dujian.net) 5.7; "LLM 2" FFN & PreNorm).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "internal.h"
#include "tfm.h"

using namespace tfm;

namespace {

thread_local int g_last_hip = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return TFM_OK;
  g_last_hip = (int)e;
  return TFM_ERR_HIP;
}

#define TFM_TRY(expr)                 \
  do {                                \
    int _st = (expr);                 \
    if (_st != TFM_OK) return _st;    \
  } while (0)

#define TFM_HIP(expr) TFM_TRY(hip_status(expr))

// Launch trace (tfm_trace_begin / tfm_trace_end / tfm_trace_read): while it is on, the forward
// path records a HIP event on its stream after each launch, with the kernel's label, so a
// caller can time every kernel inside a real step.
struct Trace {
  std::vector<hipEvent_t> ev;      // ev[0] recorded at begin, ev[i] after launch i
  std::vector<const char *> label; // label[i] of launch i (label[0] unused)
  int n = 0;                       // events recorded so far
  bool on = false;
};
thread_local Trace g_trace;

int mark(hipStream_t s, const char *label) {
  Trace &t = g_trace;
  if (!t.on || t.n >= (int)t.ev.size()) return TFM_OK;
  t.label[t.n] = label;
  return hip_status(hipEventRecord(t.ev[t.n++], s));
}

// A launch of the forward path followed by its trace mark.
#define TFM_LAUNCH(label, expr)   \
  do {                            \
    TFM_HIP(expr);                \
    TFM_TRY(mark(s, label));      \
  } while (0)

bool valid_dt(int dt) { return dt == TFM_F32 || dt == TFM_BF16; }
size_t elt(int dt) { return dt == TFM_BF16 ? 2 : 4; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace regions of the block and model forward.
struct WsPlan {
  size_t flag, x, xn, qkv, o, u, nrm, total;
};

// The RMSNorm before the QKV and SwiGLU products is split across the product that writes the
// residual and the product that reads the norm (bf16 models with d_model within the width
// whose row partials one nrm row holds); the others run the standalone RMSNorm kernel.
bool norm_split(const tfm_config *c) {
  return c->dtype == TFM_BF16 && c->d_model <= gemm_norm_max_cols();
}

WsPlan plan_ws(const tfm_config *c, int B, int S) {
  const size_t M = (size_t)B * S, e = elt(c->dtype);
  const size_t qd = (size_t)c->n_heads * c->d_head, kvd = (size_t)c->n_kv_heads * c->d_head;
  WsPlan p;
  size_t off = 0;
  p.flag = off; off += 256;
  p.x = off; off += round256(M * c->d_model * 4);
  p.xn = off; off += round256(M * c->d_model * e);
  p.qkv = off; off += round256(M * (qd + 2 * kvd) * e);
  p.o = off; off += round256(M * qd * e);
  p.u = off; off += round256(M * c->d_ff * e);
  p.nrm = off;
  if (norm_split(c)) off += round256(M * kNormParts * 4);
  p.total = off;
  return p;
}

// Workspace regions of a decode step (B tokens).
struct DecPlan {
  size_t flag, x, xn, q, o, u, part, total;
};

DecPlan plan_decode(const tfm_config *c, int B, int cache_seq) {
  const size_t qd = (size_t)c->n_heads * c->d_head;
  DecPlan p;
  size_t off = 0;
  p.flag = off; off += 256;
  p.x = off; off += round256((size_t)B * c->d_model * 4);
  p.xn = off; off += round256((size_t)B * c->d_model * 2);
  p.q = off; off += round256((size_t)B * qd * 2);
  p.o = off; off += round256((size_t)B * qd * 2);
  p.u = off; off += round256((size_t)B * c->d_ff * 2);
  p.part = off;
  off += round256((size_t)B * c->n_heads * decode_chunks(cache_seq) * (2 + c->d_head) * 4);
  p.total = off;
  return p;
}

// What the decode path supports beyond a valid configuration.
int check_decode_config(const tfm_config *c) {
  if (c->dtype != TFM_BF16) return TFM_ERR_UNSUPPORTED;
  if ((c->d_head != 32 && c->d_head != 64 && c->d_head != 128) ||
      !decode_group_supported(c->n_heads, c->n_kv_heads))
    return TFM_ERR_UNSUPPORTED;
  return TFM_OK;
}

int check_config(const tfm_config *c, int B, int S) {
  if (!c) return TFM_ERR_NULL;
  if (!valid_dt(c->dtype)) return TFM_ERR_DTYPE;
  if (c->n_layers < 0 || c->d_model <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 ||
      c->d_head <= 0 || c->d_ff <= 0 || c->vocab <= 0 || c->max_seq_len <= 0)
    return TFM_ERR_SHAPE;
  if (c->n_heads % c->n_kv_heads != 0) return TFM_ERR_SHAPE;
  if (c->d_head % 4 != 0) return TFM_ERR_SHAPE;  // RoPE pairs, 4-wide vectors
  if (!(c->eps >= 0.f) || !std::isfinite(c->rope_theta) || !(c->rope_theta > 0.f))
    return TFM_ERR_SHAPE;
  if (B < 0 || S < 0 || S > c->max_seq_len) return TFM_ERR_SHAPE;
  if (c->attn_window < 0 || c->attn_full_every < 0) return TFM_ERR_SHAPE;
  const int kalign = c->dtype == TFM_BF16 ? 8 : 4;
  if (c->d_model % kalign != 0 || c->d_ff % kalign != 0 ||
      (c->n_heads * c->d_head) % kalign != 0)
    return TFM_ERR_SHAPE;
  if (!attention_supported(c->dtype, c->d_head) ||
      !attention_fits(c->dtype, S, (int64_t)(c->n_heads + 2 * c->n_kv_heads) * c->d_head))
    return TFM_ERR_UNSUPPORTED;
  return TFM_OK;
}

int check_layer(const tfm_layer_weights *w) {
  if (!w) return TFM_ERR_NULL;
  const void *ps[] = {w->g_attn, w->wq, w->wk, w->wv, w->wo, w->g_ffn, w->w1, w->w3, w->w2};
  for (const void *p : ps) {
    if (!p) return TFM_ERR_NULL;
    if (!aligned16(p)) return TFM_ERR_ALIGN;
  }
  return TFM_OK;
}

// Enqueue one block; arguments already validated.
// KV cache of one layer: its K block and V block (bf16, (B, Hkv, cache_seq, d_head) each).
struct LayerCache {
  void *k = nullptr, *v = nullptr;
  int seq = 0;
};

LayerCache layer_cache(const tfm_config *c, void *cache, int B, int cache_seq, int l) {
  LayerCache lc;
  if (!cache) return lc;
  const size_t blk = (size_t)B * c->n_kv_heads * cache_seq * c->d_head;
  lc.k = (uint16_t *)cache + 2 * (size_t)l * blk;
  lc.v = (uint16_t *)cache + (2 * (size_t)l + 1) * blk;
  lc.seq = cache_seq;
  return lc;
}

// norm_in: the previous block's down projection already left bf16(x * g_attn) in xn and
// its row partials in nrm (split RMSNorm). g_next: the gain of the next block's first
// RMSNorm, split into this block's down projection the same way (nullptr: not split).
// xn_ready: xn already holds RMSNorm(x; g_attn) (the embedding pass wrote it).
int enqueue_block(const tfm_config *c, const tfm_layer_weights *w, float *x,
                  const int32_t *positions, int B, int S, const float *cos_sin, uint8_t *ws,
                  const WsPlan &p, int window, hipStream_t s, const LayerCache &lc = {},
                  bool norm_in = false, const void *g_next = nullptr, bool xn_ready = false) {
  const int64_t M = (int64_t)B * S;
  const int D = c->d_model, dt = c->dtype;
  const int qd = c->n_heads * c->d_head, kvd = c->n_kv_heads * c->d_head;
  const int qkv_w = qd + 2 * kvd;
  const size_t e = elt(dt);
  void *xn = ws + p.xn;
  uint8_t *qkv = ws + p.qkv;
  void *o = ws + p.o;
  void *u = ws + p.u;
  const bool split = norm_split(c);
  float *nrm = split ? (float *)(ws + p.nrm) : nullptr;
  // the reading product's side of a split RMSNorm: 1 / rms(x) per row from the partials
  auto scale_rows = [&](GemmArgs &g) {
    g.rs_part = nrm; g.rs_parts = gemm_residual_col_tiles(D); g.rs_d = D; g.rs_eps = c->eps;
  };
  // the writing product's side: bf16(x * gain) into xn and the row partials into nrm
  auto emit_norm = [&](GemmArgs &g, const void *gain) {
    g.nrm_g = gain; g.nrm_y = xn; g.nrm_part = nrm;
  };

  if (!norm_in && !xn_ready)
    TFM_LAUNCH("rmsnorm", launch_rmsnorm(x, DT_F32, w->g_attn, dt, xn, dt, M, D, c->eps, s));

  GemmArgs g{};
  g.a = xn; g.lda = D; g.w0 = w->wq; g.w1 = w->wk; g.w2 = w->wv; g.n0 = qd; g.n1 = kvd;
  g.M = M; g.N = qkv_w; g.K = D; g.y = qkv; g.ldy = qkv_w; g.y_dt = dt;
  g.positions = positions; g.cos_sin = cos_sin; g.S = S; g.d_head = c->d_head;
  g.max_seq = c->max_seq_len;
  if (norm_in) scale_rows(g);
  TFM_LAUNCH("gemm_qkv_rope", launch_gemm(EPI_QKV_ROPE, dt, g, s));
  if (lc.k)   // prefill: rotated k and v rows into the cache slots of their positions
    TFM_LAUNCH("kv_store", launch_kv_store(qkv, qkv_w, qd, kvd, c->d_head, c->n_kv_heads, B, S,
                                           positions, lc.k, lc.v, lc.seq,
                                           (int32_t *)(ws + p.flag) + 1, s));

  TFM_LAUNCH(window > 0 ? "attention_window" : "attention",
             launch_attention(qkv, qkv_w, qkv + (size_t)qd * e, qkv + (size_t)(qd + kvd) * e,
                              qkv_w, o, qd, B, S, c->n_heads, c->n_kv_heads, c->d_head, dt,
                              window, s));

  g = GemmArgs{};
  g.a = o; g.lda = qd; g.w0 = w->wo; g.M = M; g.N = D; g.K = qd; g.y = x; g.ldy = D;
  g.y_dt = DT_F32; g.residual = x;
  if (split) emit_norm(g, w->g_ffn);
  TFM_LAUNCH("gemm_out_residual", launch_gemm(EPI_RESIDUAL, dt, g, s));

  if (!split) TFM_LAUNCH("rmsnorm", launch_rmsnorm(x, DT_F32, w->g_ffn, dt, xn, dt, M, D, c->eps, s));

  g = GemmArgs{};
  g.a = xn; g.lda = D; g.w0 = w->w1; g.w1 = w->w3; g.n0 = c->d_ff; g.M = M; g.N = c->d_ff;
  g.K = D; g.y = u; g.ldy = c->d_ff; g.y_dt = dt;
  if (split) scale_rows(g);
  TFM_LAUNCH("gemm_swiglu", launch_gemm(EPI_SWIGLU, dt, g, s));

  g = GemmArgs{};
  g.a = u; g.lda = c->d_ff; g.w0 = w->w2; g.M = M; g.N = D; g.K = c->d_ff; g.y = x; g.ldy = D;
  g.y_dt = DT_F32; g.residual = x;
  if (split && g_next) emit_norm(g, g_next);
  TFM_LAUNCH("gemm_down_residual", launch_gemm(EPI_RESIDUAL, dt, g, s));
  return TFM_OK;
}

// Attention window of layer l ("LLM 2" hybrid attention): the configured window, except every
// attn_full_every-th layer, which keeps full attention.
int layer_window(const tfm_config *c, int l) {
  const bool full = c->attn_full_every > 0 && l % c->attn_full_every == c->attn_full_every - 1;
  return full ? 0 : c->attn_window;
}

// Embedding, every block and the final RMSNorm: leaves RMSNorm(x; g_final) in the xn region
// of the workspace.
int enqueue_trunk(const tfm_config *c, const tfm_model_weights *w, const int32_t *ids,
                  const int32_t *positions, int B, int S, const float *cos_sin, uint8_t *wsb,
                  const WsPlan &p, hipStream_t s, void *kv_cache = nullptr, int cache_seq = 0) {
  const int64_t M = (int64_t)B * S;
  float *x = (float *)(wsb + p.x);
  TFM_LAUNCH("fill_flags", launch_fill_i32((int32_t *)(wsb + p.flag), 2, 0, s));   // token and position flags
  // the embedding pass also writes the first block's RMSNorm(x; g_attn) into xn
  if (c->n_layers > 0)
    TFM_LAUNCH("embed", launch_embed_rmsnorm(ids, M, w->embed, c->dtype, c->vocab, c->d_model, x,
                                             (int32_t *)(wsb + p.flag), w->layers[0].g_attn,
                                             wsb + p.xn, c->eps, s));
  else
    TFM_LAUNCH("embed", launch_embed(ids, M, w->embed, c->dtype, c->vocab, c->d_model, x,
                                     (int32_t *)(wsb + p.flag), s));
  const bool split = norm_split(c);
  for (int l = 0; l < c->n_layers; ++l) {
    const void *g_next = split && l + 1 < c->n_layers ? w->layers[l + 1].g_attn : nullptr;
    TFM_TRY(enqueue_block(c, &w->layers[l], x, positions, B, S, cos_sin, wsb, p,
                          layer_window(c, l), s, layer_cache(c, kv_cache, B, cache_seq, l),
                          split && l > 0, g_next, l == 0));
  }
  TFM_LAUNCH("rmsnorm", launch_rmsnorm(x, DT_F32, w->g_final, c->dtype, wsb + p.xn, c->dtype, M,
                                       c->d_model, c->eps, s));
  return TFM_OK;
}

// Pointers and alignment every whole-model entry point needs.
int check_model(const tfm_config *c, const tfm_model_weights *w, const int32_t *ids,
                const float *cos_sin, const void *ws) {
  if (!ids || !cos_sin || !ws || !w->embed || !w->g_final || !w->lm_head ||
      (c->n_layers > 0 && !w->layers))
    return TFM_ERR_NULL;
  if (!aligned16(cos_sin) || !aligned16(ws) || !aligned16(w->embed) || !aligned16(w->g_final) ||
      !aligned16(w->lm_head))
    return TFM_ERR_ALIGN;
  for (int l = 0; l < c->n_layers; ++l) TFM_TRY(check_layer(&w->layers[l]));
  return TFM_OK;
}

// Workspace of the fused LM-head cross-entropy: per-row partials of every column tile.
struct XentPlan {
  size_t x_max, x_sum, x_tgt, total;
  int parts;
};

XentPlan plan_xent(int64_t M, int V) {
  XentPlan p;
  p.parts = gemm_xent_parts(V);
  const size_t part_bytes = round256((size_t)M * p.parts * 4);
  p.x_max = 0;
  p.x_sum = part_bytes;
  p.x_tgt = 2 * part_bytes;
  p.total = 2 * part_bytes + round256((size_t)M * 4);
  return p;
}

int enqueue_xent(const void *x, const void *w, const int32_t *targets, float *loss, float *mean,
                 int64_t M, int V, int K, uint8_t *wsb, const XentPlan &xp, hipStream_t s) {
  GemmArgs g{};
  g.a = x; g.lda = K; g.w0 = w; g.M = M; g.N = V; g.K = K;
  g.targets = targets;
  g.x_max = (float *)(wsb + xp.x_max);
  g.x_sum = (float *)(wsb + xp.x_sum);
  g.x_tgt = (float *)(wsb + xp.x_tgt);
  TFM_LAUNCH("gemm_lm_head_xent", launch_gemm(EPI_XENT, DT_BF16, g, s));
  TFM_LAUNCH("xent_reduce", launch_xent_reduce(g.x_max, g.x_sum, g.x_tgt, targets, xp.parts, M, V,
                                               loss, mean, s));
  return TFM_OK;
}


// ---- training step: plan of the workspace and the enqueued forward / backward
struct TrainPlan {
  size_t flag, count, row_loss, xfinal, xf, logits, x_max, x_sum, x_tgt, x_lse, dlog, dlogT, xfT, wT, dx, dxb, dxb2, dxT, dh, hT, du, dac, wTl,
      da, dc, daT, dcT, actT, dout, dqkv, dqkvT, lse, dsum, rms_part, splitk;
  size_t layers, layer_bytes;
  size_t l_x, l_h1, l_qkv, l_o, l_lse, l_xm, l_h2, l_a, l_c, l_u;   // within a layer block
  int Vp;        // vocabulary padded to a multiple of 64: the K of the head's input-gradient
                 // product, which then runs the cross-stage main loop
  int64_t Mp;    // tokens padded to a multiple of 8 (K of the weight-gradient GEMMs)
  size_t total;
};

// Weight-gradient products contract over the tokens (K = B S) into small outputs, so they
// launch few tiles; they are split along K into `parts` contiguous ranges (each a multiple of
// 64, at least 512 long) so about kSplitTarget workgroups run, and the fp32 partials are
// summed in part order (deterministic).
constexpr int64_t kSplitTarget = 512;
constexpr int kSplitMax = 16;
int splitk_parts_of(int64_t tiles, int64_t K) {
  int64_t parts = (kSplitTarget + tiles - 1) / tiles;
  parts = std::min<int64_t>(parts, std::max<int64_t>(1, K / 512));
  return (int)std::min<int64_t>(parts, kSplitMax);
}
int splitk_parts(int dt, int64_t M, int N, int64_t K) {
  return splitk_parts_of(gemm_store_tiles(dt, M, N), K);
}
// the K-major product's 128 x 128 tiles: at least as many as the plain store's, so never
// more parts (the workspace sized by splitk_bytes holds them)
int splitk_parts_kmajor(int64_t M, int N, int64_t K) {
  return splitk_parts_of(((M + 127) / 128) * ((N + 127) / 128), K);
}
size_t splitk_bytes(int dt, int64_t M, int N, int64_t K) {
  const int parts = splitk_parts(dt, M, N, K);
  return parts > 1 ? (size_t)parts * M * N * 4 : 0;
}

// bf16 models take the loss through the fused LM-head cross-entropy (no logits stored) and
// recompute the logits for their gradient in the backward
bool train_fused_xent(const tfm_config *c) {
  return c->dtype == TFM_BF16 && c->d_model % 8 == 0;
}

TrainPlan plan_train(const tfm_config *c, int B, int S) {
  TrainPlan p;
  const size_t M = (size_t)B * S, e = elt(c->dtype);
  const size_t D = c->d_model, F = c->d_ff, V = c->vocab;
  const size_t qd = (size_t)c->n_heads * c->d_head, kvd = (size_t)c->n_kv_heads * c->d_head;
  const size_t W = qd + 2 * kvd;
  p.Vp = (int)((V + 63) / 64 * 64);
  p.Mp = (int64_t)((M + 7) / 8 * 8);
  const size_t Vp = p.Vp, Mp = p.Mp;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += round256(bytes); return o; };
  p.flag = take(256);
  p.count = take(4);
  p.row_loss = take(M * 4);
  p.xfinal = take(M * D * 4);
  p.xf = take(M * D * e);
  const bool fx = train_fused_xent(c);
  const size_t xparts = fx ? (size_t)gemm_xent_parts((int)V) : 0;
  p.logits = take(fx ? 4 : M * Vp * 4);
  p.x_max = take(std::max<size_t>(M * xparts * 4, 4));
  p.x_sum = take(std::max<size_t>(M * xparts * 4, 4));
  p.x_tgt = take(M * 4);
  p.x_lse = take(M * 4);
  p.dlog = take(M * Vp * e);
  p.dlogT = take(Vp * Mp * e);
  p.xfT = take(D * Mp * e);
  size_t wmax = D * Vp;
  wmax = std::max(wmax, 2 * F * D);
  wmax = std::max(wmax, D * W);
  wmax = std::max(wmax, qd * D);
  p.wT = take(wmax * e);
  // a layer's transposed weights, all made by one launch before its backward:
  // W2^T (F, D) | [W1^T | W3^T] (D, 2F) | Wo^T (qd, D) | [Wq; Wk; Wv]^T (D, W)
  p.wTl = take((3 * F * D + qd * D + D * W) * e);
  p.dx = take(M * D * 4);
  p.dxb = take(M * D * e);
  p.dxb2 = take(M * D * e);
  p.dxT = take(D * Mp * e);
  p.dh = take(M * D * 4);
  p.hT = take(D * Mp * e);
  p.du = take(M * F * 4);
  p.da = take(M * F * e);
  p.dac = take(M * 2 * F * e);
  p.dc = take(M * F * e);
  p.daT = take(F * Mp * e);
  p.dcT = take(F * Mp * e);
  p.actT = take(std::max(F, qd) * Mp * e);
  p.dout = take(M * qd * e);
  p.dqkv = take(M * W * e);
  p.dqkvT = take(W * Mp * e);
  p.lse = take(M * c->n_heads * 4);
  p.dsum = take(M * c->n_heads * 4);
  p.rms_part = take((size_t)rms_back_parts((int64_t)M) * D * 4);
  {   // split-K partials of the largest weight-gradient product
    const int dt = c->dtype == TFM_BF16 ? DT_BF16 : DT_F32;
    const int64_t K = (int64_t)Mp;
    size_t sk = splitk_bytes(dt, (int64_t)V, (int)D, K);
    sk = std::max(sk, splitk_bytes(dt, (int64_t)D, (int)F, K));
    sk = std::max(sk, splitk_bytes(dt, (int64_t)F, (int)D, K));
    sk = std::max(sk, splitk_bytes(dt, (int64_t)D, (int)qd, K));
    sk = std::max(sk, splitk_bytes(dt, (int64_t)qd, (int)D, K));
    sk = std::max(sk, splitk_bytes(dt, (int64_t)kvd, (int)D, K));
    p.splitk = take(std::max<size_t>(sk, 4));
  }
  size_t lo = 0;
  auto ltake = [&](size_t bytes) { const size_t o = lo; lo += round256(bytes); return o; };
  p.l_x = ltake(M * D * 4);
  p.l_h1 = ltake(M * D * e);
  p.l_qkv = ltake(M * W * e);
  p.l_o = ltake(M * qd * e);
  p.l_lse = ltake(M * c->n_heads * 4);
  p.l_xm = ltake(M * D * 4);
  p.l_h2 = ltake(M * D * e);
  p.l_a = ltake(M * F * e);
  p.l_c = ltake(M * F * e);
  p.l_u = ltake(M * F * e);
  p.layer_bytes = lo;
  p.layers = off;
  off += lo * (size_t)c->n_layers;
  p.total = off;
  return p;
}

int check_train_config(const tfm_config *c) {
  if (c->d_model > 2048) return TFM_ERR_UNSUPPORTED;   // RMSNorm backward keeps a row in registers
  if (!attention_backward_supported(c->d_head)) return TFM_ERR_UNSUPPORTED;
  return TFM_OK;
}

// y = a w^T on the forward GEMM kernels; a (M, K) row stride lda, w (N, K) rows of K.
int gemm(int epi, int dt, const void *a, int64_t lda, const void *w, int64_t M, int N, int K,
         void *y, int64_t ldy, int y_dt, const float *residual, hipStream_t s) {
  GemmArgs g{};
  g.a = a; g.lda = lda; g.w0 = w; g.M = M; g.N = N; g.K = K; g.y = y; g.ldy = ldy; g.y_dt = y_dt;
  g.residual = residual;
  return hip_status(launch_gemm(epi, dt, g, s));
}

// Weight gradient y (M, N) fp32 = a w^T over K = tokens, split along K (splitk_parts).
int gemm_wgrad(int dt, const void *a, int64_t lda, const void *w, int64_t M, int N, int K,
               float *y, int64_t ldy, float *part, hipStream_t s) {
  const int parts = splitk_parts(dt, M, N, K);
  if (parts <= 1) return gemm(EPI_STORE, dt, a, lda, w, M, N, K, y, ldy, DT_F32, nullptr, s);
  const int ks = ((K + parts - 1) / parts + 63) / 64 * 64;
  const int n = (K + ks - 1) / ks;
  GemmArgs g{};
  g.a = a; g.lda = lda; g.w0 = w; g.M = M; g.N = N; g.K = K;
  g.y = part; g.ldy = N; g.y_dt = DT_F32;
  g.kparts = n; g.kpart = ks; g.ypart = M * N;
  TFM_HIP(launch_gemm(EPI_STORE, dt, g, s));
  return hip_status(launch_sum_parts(part, n, M, N, y, ldy, s));
}

// The same product with both operands as the forward keeps them (bf16, tokens as rows):
// y (M, N) = sum over t < K of a[t lda + m] b[t ldb + n], on the K-major product, so no
// activation is transposed. Returns TFM_ERR_UNSUPPORTED where that product does not take the
// operands (the caller then transposes them).
int gemm_wgrad_rows(const void *a, int64_t lda, const void *b, int64_t ldb, int64_t M, int N,
                    int K, float *y, int64_t ldy, float *part, hipStream_t s) {
  if (!gemm_kmajor_ok(a, lda, b, ldb, M, N, K)) return TFM_ERR_UNSUPPORTED;
  const int parts = splitk_parts_kmajor(M, N, K);
  GemmArgs g{};
  g.a = a; g.lda = lda; g.w0 = b; g.ldw = ldb; g.M = M; g.N = N; g.K = K; g.y_dt = DT_F32;
  if (parts <= 1) {
    g.y = y; g.ldy = ldy;
    return hip_status(launch_gemm_kmajor(g, s));
  }
  const int ks = ((K + parts - 1) / parts + 63) / 64 * 64;
  const int n = (K + ks - 1) / ks;
  g.y = part; g.ldy = N;
  g.kparts = n; g.kpart = ks; g.ypart = M * N;
  TFM_HIP(launch_gemm_kmajor(g, s));
  return hip_status(launch_sum_parts(part, n, M, N, y, ldy, s));
}
}  // namespace

extern "C" {

const char *tfm_status_string(int status) {
  switch (status) {
    case TFM_OK: return "ok";
    case TFM_ERR_NULL: return "required pointer is NULL";
    case TFM_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case TFM_ERR_DTYPE: return "unknown or unsupported dtype";
    case TFM_ERR_WORKSPACE: return "workspace too small";
    case TFM_ERR_ALIGN: return "pointer or stride misaligned";
    case TFM_ERR_UNSUPPORTED: return "unsupported configuration";
    case TFM_ERR_HIP: return "HIP launch or copy failed";
    case TFM_ERR_TOKEN: return "token id outside the vocabulary";
    case TFM_ERR_POSITION: return "position outside the KV cache or the RoPE table";
  }
  return "unknown status";
}

int tfm_last_hip_error(void) { return g_last_hip; }

const char *tfm_version(void) { return "tfm 0.1 gfx950"; }

int tfm_mfma_rate(int64_t iters, int blocks, float *sink, void *stream) {
  if (!sink) return TFM_ERR_NULL;
  if (iters <= 0 || blocks <= 0) return TFM_ERR_SHAPE;
  return hip_status(launch_mfma_rate(iters, blocks, sink, (hipStream_t)stream));
}

int tfm_rope_table_init(float *cos_sin, int max_seq, int d_head, double theta, void *stream) {
  if (!cos_sin) return TFM_ERR_NULL;
  if (!aligned16(cos_sin)) return TFM_ERR_ALIGN;
  if (max_seq <= 0 || d_head <= 0 || d_head % 2 != 0 || !(theta > 0.0) || !std::isfinite(theta))
    return TFM_ERR_SHAPE;
  return hip_status(launch_rope_table(cos_sin, max_seq, d_head, theta, (hipStream_t)stream));
}

int tfm_embed(const int32_t *ids, int64_t n, const void *table, int table_dt, int vocab, int d,
              float *x, int32_t *err_flag, void *stream) {
  if (!valid_dt(table_dt)) return TFM_ERR_DTYPE;
  if (n < 0 || vocab <= 0 || d <= 0 || d % 4 != 0) return TFM_ERR_SHAPE;
  if (n == 0) return TFM_OK;
  if (!ids || !table || !x) return TFM_ERR_NULL;
  if (!aligned16(table) || !aligned16(x)) return TFM_ERR_ALIGN;
  return hip_status(launch_embed(ids, n, table, table_dt, vocab, d, x, err_flag,
                                 (hipStream_t)stream));
}

int tfm_rmsnorm(const void *x, int x_dt, const void *g, int g_dt, void *y, int y_dt,
                int64_t rows, int d, float eps, void *stream) {
  if (!valid_dt(x_dt) || !valid_dt(g_dt) || !valid_dt(y_dt)) return TFM_ERR_DTYPE;
  if (rows < 0 || d <= 0 || d % 4 != 0 || !(eps >= 0.f)) return TFM_ERR_SHAPE;
  if (rows == 0) return TFM_OK;
  if (!x || !g || !y) return TFM_ERR_NULL;
  if (!aligned16(x) || !aligned16(g) || !aligned16(y)) return TFM_ERR_ALIGN;
  if (x == y) return TFM_ERR_SHAPE;
  return hip_status(launch_rmsnorm(x, x_dt, g, g_dt, y, y_dt, rows, d, eps, (hipStream_t)stream));
}

int tfm_rope(void *x, int x_dt, int64_t row_stride, const int32_t *positions, int B, int S,
             int H, int d_head, const float *cos_sin, int max_seq, void *stream) {
  if (!valid_dt(x_dt)) return TFM_ERR_DTYPE;
  if (B < 0 || S < 0 || H < 0 || d_head <= 0 || d_head % 4 != 0 || max_seq <= 0 ||
      row_stride < (int64_t)H * d_head)
    return TFM_ERR_SHAPE;
  if ((int64_t)B * S * H == 0) return TFM_OK;
  if (!x || !cos_sin) return TFM_ERR_NULL;
  if (row_stride % 4 != 0 || !aligned16(cos_sin) || ((uintptr_t)x & 7u) != 0) return TFM_ERR_ALIGN;
  if (!positions && S > max_seq) return TFM_ERR_SHAPE;
  return hip_status(launch_rope(x, x_dt, row_stride, positions, B, S, H, d_head, cos_sin, max_seq,
                                (hipStream_t)stream));
}

int tfm_linear(const void *x, const void *w, int dt, const float *residual, void *y, int y_dt,
               int64_t M, int N, int K, int64_t ldy, void *stream) {
  if (!valid_dt(dt) || !valid_dt(y_dt)) return TFM_ERR_DTYPE;
  if (residual && y_dt != TFM_F32) return TFM_ERR_DTYPE;
  if (M < 0 || N <= 0 || K <= 0 || ldy < N) return TFM_ERR_SHAPE;
  if (K % (dt == TFM_BF16 ? 8 : 4) != 0) return TFM_ERR_SHAPE;
  if (M == 0) return TFM_OK;
  if (!x || !w || !y) return TFM_ERR_NULL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (residual && !aligned16(residual)))
    return TFM_ERR_ALIGN;
  GemmArgs g{};
  g.a = x; g.lda = K; g.w0 = w; g.M = M; g.N = N; g.K = K; g.y = y; g.ldy = ldy; g.y_dt = y_dt;
  g.residual = residual;
  return hip_status(launch_gemm(residual ? EPI_RESIDUAL : EPI_STORE, dt, g, (hipStream_t)stream));
}

int tfm_qkv_rope(const void *xn, const void *wq, const void *wk, const void *wv, void *qkv,
                 const int32_t *positions, int B, int S, int d, int Hq, int Hkv, int d_head,
                 const float *cos_sin, int max_seq, int dt, void *stream) {
  if (!valid_dt(dt)) return TFM_ERR_DTYPE;
  const int kalign = dt == TFM_BF16 ? 8 : 4;
  if (B < 0 || S < 0 || d <= 0 || Hq <= 0 || Hkv <= 0 || d_head <= 0 || d_head % 4 != 0 ||
      d % kalign != 0 || max_seq <= 0)
    return TFM_ERR_SHAPE;
  if ((int64_t)B * S == 0) return TFM_OK;
  if (!xn || !wq || !wk || !wv || !qkv || !cos_sin) return TFM_ERR_NULL;
  if (!aligned16(xn) || !aligned16(wq) || !aligned16(wk) || !aligned16(wv) || !aligned16(qkv) ||
      !aligned16(cos_sin))
    return TFM_ERR_ALIGN;
  if (!positions && S > max_seq) return TFM_ERR_SHAPE;
  const int qd = Hq * d_head, kvd = Hkv * d_head;
  GemmArgs g{};
  g.a = xn; g.lda = d; g.w0 = wq; g.w1 = wk; g.w2 = wv; g.n0 = qd; g.n1 = kvd;
  g.M = (int64_t)B * S; g.N = qd + 2 * kvd; g.K = d; g.y = qkv; g.ldy = qd + 2 * kvd; g.y_dt = dt;
  g.positions = positions; g.cos_sin = cos_sin; g.S = S; g.d_head = d_head; g.max_seq = max_seq;
  return hip_status(launch_gemm(EPI_QKV_ROPE, dt, g, (hipStream_t)stream));
}

int tfm_causal_attention(const void *q, int64_t q_stride, const void *k, const void *v,
                         int64_t kv_stride, void *o, int64_t o_stride, int B, int S, int Hq,
                         int Hkv, int d_head, int dt, void *stream) {
  return tfm_sliding_window_attention(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv,
                                      d_head, 0, dt, stream);
}

int tfm_sliding_window_attention(const void *q, int64_t q_stride, const void *k, const void *v,
                                 int64_t kv_stride, void *o, int64_t o_stride, int B, int S,
                                 int Hq, int Hkv, int d_head, int window, int dt, void *stream) {
  if (window < 0) return TFM_ERR_SHAPE;
  if (!valid_dt(dt)) return TFM_ERR_DTYPE;
  if (B < 0 || S < 0 || Hq <= 0 || Hkv <= 0 || d_head <= 0 || Hq % Hkv != 0) return TFM_ERR_SHAPE;
  if (q_stride < (int64_t)Hq * d_head || o_stride < (int64_t)Hq * d_head ||
      kv_stride < (int64_t)Hkv * d_head)
    return TFM_ERR_SHAPE;
  if (!attention_supported(dt, d_head) || !attention_fits(dt, S, kv_stride))
    return TFM_ERR_UNSUPPORTED;
  if ((int64_t)B * S == 0) return TFM_OK;
  if (!q || !k || !v || !o) return TFM_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || q_stride % 8 != 0 ||
      kv_stride % 8 != 0 || o_stride % 8 != 0)
    return TFM_ERR_ALIGN;
  return hip_status(launch_attention(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv,
                                     d_head, dt, window, (hipStream_t)stream));
}

size_t tfm_swiglu_workspace_bytes(int64_t rows, int d_ff, int dt) {
  if (rows < 0 || d_ff < 0 || !valid_dt(dt)) return 0;
  return round256((size_t)rows * d_ff * elt(dt));
}

int tfm_swiglu_ffn(const void *xn, const void *w1, const void *w3, const void *w2,
                   const float *residual, float *out, int64_t rows, int d, int d_ff, int dt,
                   void *ws, size_t ws_bytes, void *stream) {
  if (!valid_dt(dt)) return TFM_ERR_DTYPE;
  const int kalign = dt == TFM_BF16 ? 8 : 4;
  if (rows < 0 || d <= 0 || d_ff <= 0 || d % kalign != 0 || d_ff % kalign != 0)
    return TFM_ERR_SHAPE;
  if (rows == 0) return TFM_OK;
  if (!xn || !w1 || !w3 || !w2 || !out || !ws) return TFM_ERR_NULL;
  if (ws_bytes < tfm_swiglu_workspace_bytes(rows, d_ff, dt)) return TFM_ERR_WORKSPACE;
  if (!aligned16(xn) || !aligned16(w1) || !aligned16(w3) || !aligned16(w2) || !aligned16(out) ||
      !aligned16(ws) || (residual && !aligned16(residual)))
    return TFM_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  GemmArgs g{};
  g.a = xn; g.lda = d; g.w0 = w1; g.w1 = w3; g.n0 = d_ff; g.M = rows; g.N = d_ff; g.K = d;
  g.y = ws; g.ldy = d_ff; g.y_dt = dt;
  TFM_HIP(launch_gemm(EPI_SWIGLU, dt, g, s));
  g = GemmArgs{};
  g.a = ws; g.lda = d_ff; g.w0 = w2; g.M = rows; g.N = d; g.K = d_ff; g.y = out; g.ldy = d;
  g.y_dt = DT_F32; g.residual = residual;
  return hip_status(launch_gemm(residual ? EPI_RESIDUAL : EPI_STORE, dt, g, s));
}

size_t tfm_workspace_bytes(const tfm_config *cfg, int B, int S) {
  if (check_config(cfg, B, S) != TFM_OK) return 0;
  return plan_ws(cfg, B, S).total;
}

int tfm_block_forward(const tfm_config *cfg, const tfm_layer_weights *w, float *x,
                      const int32_t *positions, int B, int S, const float *cos_sin, void *ws,
                      size_t ws_bytes, void *stream) {
  TFM_TRY(check_config(cfg, B, S));
  TFM_TRY(check_layer(w));
  if ((int64_t)B * S == 0) return TFM_OK;
  if (!x || !cos_sin || !ws) return TFM_ERR_NULL;
  if (!aligned16(x) || !aligned16(cos_sin) || !aligned16(ws)) return TFM_ERR_ALIGN;
  const WsPlan p = plan_ws(cfg, B, S);
  if (ws_bytes < p.total) return TFM_ERR_WORKSPACE;
  return enqueue_block(cfg, w, x, positions, B, S, cos_sin, (uint8_t *)ws, p, cfg->attn_window,
                       (hipStream_t)stream);
}

int tfm_model_forward(const tfm_config *cfg, const tfm_model_weights *w, const int32_t *ids,
                      const int32_t *positions, void *logits, int logits_dt, int64_t ld_logits,
                      int B, int S, const float *cos_sin, void *ws, size_t ws_bytes,
                      void *stream) {
  TFM_TRY(check_config(cfg, B, S));
  if (!valid_dt(logits_dt)) return TFM_ERR_DTYPE;
  if (!w) return TFM_ERR_NULL;
  if (ld_logits < cfg->vocab) return TFM_ERR_SHAPE;
  if ((int64_t)B * S == 0) return TFM_OK;
  if (!logits) return TFM_ERR_NULL;
  if (!aligned16(logits)) return TFM_ERR_ALIGN;
  TFM_TRY(check_model(cfg, w, ids, cos_sin, ws));
  const WsPlan p = plan_ws(cfg, B, S);
  if (ws_bytes < p.total) return TFM_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  uint8_t *wsb = (uint8_t *)ws;
  TFM_TRY(enqueue_trunk(cfg, w, ids, positions, B, S, cos_sin, wsb, p, s));
  GemmArgs g{};
  g.a = wsb + p.xn; g.lda = cfg->d_model; g.w0 = w->lm_head; g.M = (int64_t)B * S;
  g.N = cfg->vocab; g.K = cfg->d_model; g.y = logits; g.ldy = ld_logits; g.y_dt = logits_dt;
  TFM_LAUNCH("gemm_lm_head", launch_gemm(EPI_STORE, cfg->dtype, g, s));
  return TFM_OK;
}

size_t tfm_xent_workspace_bytes(int64_t M, int V) {
  if (M < 0 || V <= 0) return 0;
  return plan_xent(M, V).total;
}

int tfm_lm_head_xent(const void *x, const void *w, const int32_t *targets, float *loss,
                     float *mean, int64_t M, int V, int K, void *ws, size_t ws_bytes,
                     void *stream) {
  if (M < 0 || V <= 0 || K <= 0) return TFM_ERR_SHAPE;
  if (K % 8 != 0) return TFM_ERR_SHAPE;
  if (M == 0) return TFM_OK;
  if (!x || !w || !targets || !loss || !ws) return TFM_ERR_NULL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(ws)) return TFM_ERR_ALIGN;
  const XentPlan xp = plan_xent(M, V);
  if (ws_bytes < xp.total) return TFM_ERR_WORKSPACE;
  return enqueue_xent(x, w, targets, loss, mean, M, V, K, (uint8_t *)ws, xp,
                      (hipStream_t)stream);
}

size_t tfm_loss_workspace_bytes(const tfm_config *cfg, int B, int S) {
  if (check_config(cfg, B, S) != TFM_OK) return 0;
  return plan_ws(cfg, B, S).total + plan_xent((int64_t)B * S, cfg->vocab).total;
}

int tfm_model_loss(const tfm_config *cfg, const tfm_model_weights *w, const int32_t *ids,
                   const int32_t *positions, const int32_t *targets, float *loss, float *mean,
                   int B, int S, const float *cos_sin, void *ws, size_t ws_bytes, void *stream) {
  TFM_TRY(check_config(cfg, B, S));
  if (cfg->dtype != TFM_BF16) return TFM_ERR_UNSUPPORTED;
  if (!w) return TFM_ERR_NULL;
  if ((int64_t)B * S == 0) return TFM_OK;
  if (!targets || !loss) return TFM_ERR_NULL;
  TFM_TRY(check_model(cfg, w, ids, cos_sin, ws));
  const WsPlan p = plan_ws(cfg, B, S);
  const int64_t M = (int64_t)B * S;
  const XentPlan xp = plan_xent(M, cfg->vocab);
  if (ws_bytes < p.total + xp.total) return TFM_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  uint8_t *wsb = (uint8_t *)ws;
  TFM_TRY(enqueue_trunk(cfg, w, ids, positions, B, S, cos_sin, wsb, p, s));
  return enqueue_xent(wsb + p.xn, w->lm_head, targets, loss, mean, M, cfg->vocab,
                      cfg->d_model, wsb + p.total, xp, s);
}

int tfm_check_device_flags(const void *ws, void *stream) {
  if (!ws) return TFM_ERR_NULL;
  TFM_HIP(hipStreamSynchronize((hipStream_t)stream));
  int32_t flag[2] = {0, 0};
  TFM_HIP(hipMemcpy(flag, ws, sizeof(flag), hipMemcpyDeviceToHost));
  return flag[0] ? TFM_ERR_TOKEN : flag[1] ? TFM_ERR_POSITION : TFM_OK;
}

// ---- KV-cache incremental decoding

size_t tfm_kv_cache_bytes(const tfm_config *cfg, int B, int cache_seq) {
  if (!cfg || B < 0 || cache_seq < 0 || cfg->n_layers < 0 || cfg->n_kv_heads <= 0 ||
      cfg->d_head <= 0)
    return 0;
  return 2 * (size_t)cfg->n_layers * B * cfg->n_kv_heads * cache_seq * cfg->d_head * 2;
}

int tfm_model_prefill(const tfm_config *cfg, const tfm_model_weights *w, const int32_t *ids,
                      const int32_t *positions, void *logits, int logits_dt, int64_t ld_logits,
                      int B, int S, const float *cos_sin, void *kv_cache, int cache_seq,
                      void *ws, size_t ws_bytes, void *stream) {
  TFM_TRY(check_config(cfg, B, S));
  TFM_TRY(check_decode_config(cfg));
  if (cache_seq <= 0) return TFM_ERR_SHAPE;
  if (logits && !valid_dt(logits_dt)) return TFM_ERR_DTYPE;
  if (!w) return TFM_ERR_NULL;
  if (logits && ld_logits < cfg->vocab) return TFM_ERR_SHAPE;
  if ((int64_t)B * S == 0) return TFM_OK;
  if (!kv_cache) return TFM_ERR_NULL;
  if (!aligned16(kv_cache) || (logits && !aligned16(logits))) return TFM_ERR_ALIGN;
  TFM_TRY(check_model(cfg, w, ids, cos_sin, ws));
  const WsPlan p = plan_ws(cfg, B, S);
  if (ws_bytes < p.total) return TFM_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  uint8_t *wsb = (uint8_t *)ws;
  TFM_TRY(enqueue_trunk(cfg, w, ids, positions, B, S, cos_sin, wsb, p, s, kv_cache, cache_seq));
  if (!logits) return TFM_OK;
  GemmArgs g{};
  g.a = wsb + p.xn; g.lda = cfg->d_model; g.w0 = w->lm_head; g.M = (int64_t)B * S;
  g.N = cfg->vocab; g.K = cfg->d_model; g.y = logits; g.ldy = ld_logits; g.y_dt = logits_dt;
  TFM_LAUNCH("gemm_lm_head", launch_gemm(EPI_STORE, cfg->dtype, g, s));
  return TFM_OK;
}

size_t tfm_decode_workspace_bytes(const tfm_config *cfg, int B, int cache_seq) {
  if (check_config(cfg, B, 1) != TFM_OK || check_decode_config(cfg) != TFM_OK || cache_seq <= 0 ||
      cache_seq > decode_max_cache())
    return 0;
  return plan_decode(cfg, B, cache_seq).total;
}

int tfm_model_decode(const tfm_config *cfg, const tfm_model_weights *w, const int32_t *ids,
                     const int32_t *positions, void *logits, int logits_dt, int64_t ld_logits,
                     int B, const float *cos_sin, void *kv_cache, int cache_seq, void *ws,
                     size_t ws_bytes, void *stream) {
  TFM_TRY(check_config(cfg, B, 1));
  TFM_TRY(check_decode_config(cfg));
  if (cache_seq <= 0) return TFM_ERR_SHAPE;
  if (cache_seq > decode_max_cache()) return TFM_ERR_UNSUPPORTED;
  if (!valid_dt(logits_dt)) return TFM_ERR_DTYPE;
  if (!w) return TFM_ERR_NULL;
  if (ld_logits < cfg->vocab) return TFM_ERR_SHAPE;
  if (B == 0) return TFM_OK;
  if (!positions || !kv_cache || !logits) return TFM_ERR_NULL;
  if (!aligned16(kv_cache) || !aligned16(logits)) return TFM_ERR_ALIGN;
  TFM_TRY(check_model(cfg, w, ids, cos_sin, ws));
  const DecPlan p = plan_decode(cfg, B, cache_seq);
  if (ws_bytes < p.total) return TFM_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  uint8_t *wsb = (uint8_t *)ws;
  const int D = cfg->d_model, F = cfg->d_ff, V = cfg->vocab;
  const int qd = cfg->n_heads * cfg->d_head, kvd = cfg->n_kv_heads * cfg->d_head;
  float *x = (float *)(wsb + p.x);
  void *xn = wsb + p.xn, *q = wsb + p.q, *o = wsb + p.o, *u = wsb + p.u;
  int32_t *flags = (int32_t *)(wsb + p.flag);
  TFM_HIP(launch_fill_i32(flags, 2, 0, s));
  TFM_HIP(launch_embed(ids, B, w->embed, TFM_BF16, V, D, x, flags, s));
  for (int l = 0; l < cfg->n_layers; ++l) {
    const tfm_layer_weights *lw = &w->layers[l];
    const LayerCache lc = layer_cache(cfg, kv_cache, B, cache_seq, l);
    DecodeGemmArgs g{};   // RMSNorm(x; g_attn) fused into the projection
    g.norm_x = x; g.norm_g = lw->g_attn; g.eps = cfg->eps; g.ldx = D; g.w0 = lw->wq; g.w1 = lw->wk; g.w2 = lw->wv; g.n0 = qd; g.n1 = kvd;
    g.M = B; g.N = qd + 2 * kvd; g.K = D; g.y = q; g.ldy = qd; g.y_dt = DT_BF16;
    g.positions = positions; g.cos_sin = cos_sin; g.d_head = cfg->d_head;
    g.max_seq = cfg->max_seq_len; g.k_cache = lc.k; g.v_cache = lc.v; g.cache_seq = cache_seq;
    g.n_kv_heads = cfg->n_kv_heads; g.pos_flag = flags + 1;
    TFM_HIP(launch_decode_gemm(EPI_QKV_CACHE, g, s));
    TFM_HIP(launch_decode_attention(q, qd, lc.k, lc.v, positions, B, cfg->n_heads,
                                    cfg->n_kv_heads, cfg->d_head, cache_seq,
                                    layer_window(cfg, l), (float *)(wsb + p.part), o, qd, s));
    g = DecodeGemmArgs{};
    g.x = o; g.ldx = qd; g.w0 = lw->wo; g.M = B; g.N = D; g.K = qd; g.y = x; g.ldy = D;
    g.y_dt = DT_F32;
    TFM_HIP(launch_decode_gemm(EPI_RESIDUAL, g, s));
    g = DecodeGemmArgs{};   // RMSNorm(x; g_ffn) fused into the up projection
    g.norm_x = x; g.norm_g = lw->g_ffn; g.eps = cfg->eps; g.ldx = D; g.w0 = lw->w1; g.w1 = lw->w3; g.n0 = F; g.M = B; g.N = F; g.K = D;
    g.y = u; g.ldy = F; g.y_dt = DT_BF16;
    TFM_HIP(launch_decode_gemm(EPI_SWIGLU, g, s));
    g = DecodeGemmArgs{};
    g.x = u; g.ldx = F; g.w0 = lw->w2; g.M = B; g.N = D; g.K = F; g.y = x; g.ldy = D;
    g.y_dt = DT_F32;
    TFM_HIP(launch_decode_gemm(EPI_RESIDUAL, g, s));
  }
  DecodeGemmArgs g{};   // RMSNorm(x; g_final) fused into the LM head
  g.norm_x = x; g.norm_g = w->g_final; g.eps = cfg->eps; g.ldx = D; g.w0 = w->lm_head; g.M = B; g.N = V; g.K = D; g.y = logits;
  g.ldy = ld_logits; g.y_dt = logits_dt;
  TFM_HIP(launch_decode_gemm(EPI_STORE, g, s));
  return TFM_OK;
}

size_t tfm_decode_attention_workspace_bytes(int B, int Hq, int d_head, int cache_seq) {
  if (B < 0 || Hq <= 0 || d_head <= 0 || cache_seq <= 0) return 0;
  return round256((size_t)B * Hq * decode_chunks(cache_seq) * (2 + d_head) * 4);
}

namespace {
// Checks shared by the decode attention entry points (everything but the workspace).
int check_decode_attention(const void *q, int64_t q_stride, const void *k_cache,
                           const void *v_cache, const int32_t *positions, const void *o,
                           int64_t o_stride, int B, int Hq, int Hkv, int d_head, int cache_seq,
                           int window) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || cache_seq <= 0 || window < 0)
    return TFM_ERR_SHAPE;
  if (q_stride < (int64_t)Hq * d_head || o_stride < (int64_t)Hq * d_head) return TFM_ERR_SHAPE;
  if ((d_head != 32 && d_head != 64 && d_head != 128) || !decode_group_supported(Hq, Hkv) ||
      cache_seq > decode_max_cache())
    return TFM_ERR_UNSUPPORTED;
  if (B == 0) return TFM_OK;
  if (!q || !k_cache || !v_cache || !positions || !o) return TFM_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      q_stride % 8 != 0 || o_stride % 8 != 0)
    return TFM_ERR_ALIGN;
  return TFM_OK;
}
}  // namespace

int tfm_decode_attention(const void *q, int64_t q_stride, const void *k_cache,
                         const void *v_cache, const int32_t *positions, void *o,
                         int64_t o_stride, int B, int Hq, int Hkv, int d_head, int cache_seq,
                         int window, void *ws, size_t ws_bytes, void *stream) {
  TFM_TRY(check_decode_attention(q, q_stride, k_cache, v_cache, positions, o, o_stride, B, Hq,
                                 Hkv, d_head, cache_seq, window));
  if (B == 0) return TFM_OK;
  if (!ws) return TFM_ERR_NULL;
  if (!aligned16(ws)) return TFM_ERR_ALIGN;
  if (ws_bytes < tfm_decode_attention_workspace_bytes(B, Hq, d_head, cache_seq))
    return TFM_ERR_WORKSPACE;
  return hip_status(launch_decode_attention(q, q_stride, k_cache, v_cache, positions, B, Hq,
                                            Hkv, d_head, cache_seq, window, (float *)ws, o,
                                            o_stride, (hipStream_t)stream));
}

size_t tfm_decode_attention_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int tfm_decode_attention_noalloc(const void *q, int64_t q_stride, const void *k_cache,
                                 const void *v_cache, const int32_t *positions, void *o,
                                 int64_t o_stride, int B, int Hq, int Hkv, int d_head,
                                 int cache_seq, int window, void *stream) {
  TFM_TRY(check_decode_attention(q, q_stride, k_cache, v_cache, positions, o, o_stride, B, Hq,
                                 Hkv, d_head, cache_seq, window));
  if (B == 0) return TFM_OK;
  if (tfm_decode_attention_workspace_bytes(B, Hq, d_head, cache_seq) > kNoAllocScratchBytes)
    return TFM_ERR_WORKSPACE;
  float *part = nullptr;
  TFM_HIP(noalloc_scratch((hipStream_t)stream, &part));
  return hip_status(launch_decode_attention(q, q_stride, k_cache, v_cache, positions, B, Hq,
                                            Hkv, d_head, cache_seq, window, part, o, o_stride,
                                            (hipStream_t)stream));
}


// ---- training step

size_t tfm_train_workspace_bytes(const tfm_config *cfg, int B, int S) {
  if (check_config(cfg, B, S) != TFM_OK || check_train_config(cfg) != TFM_OK) return 0;
  return plan_train(cfg, B, S).total;
}

int tfm_model_backward(const tfm_config *cfg, const tfm_model_weights *w, const int32_t *ids,
                       const int32_t *positions, const int32_t *targets, float *loss_mean,
                       const tfm_model_grads *gr, int B, int S, const float *cos_sin, void *ws,
                       size_t ws_bytes, void *stream) {
  TFM_TRY(check_config(cfg, B, S));
  TFM_TRY(check_train_config(cfg));
  if (!w || !gr) return TFM_ERR_NULL;
  if ((int64_t)B * S == 0) return TFM_OK;
  if (!targets || !loss_mean) return TFM_ERR_NULL;
  TFM_TRY(check_model(cfg, w, ids, cos_sin, ws));
  const bool tied = w->lm_head == w->embed;
  if (!gr->embed || !gr->g_final || (cfg->n_layers > 0 && !gr->layers)) return TFM_ERR_NULL;
  if (!tied && !gr->lm_head) return TFM_ERR_NULL;
  if (tied && gr->lm_head && gr->lm_head != gr->embed) return TFM_ERR_SHAPE;
  const float *gps[] = {gr->embed, gr->g_final, tied ? gr->embed : gr->lm_head};
  for (const float *q : gps)
    if (!aligned16(q)) return TFM_ERR_ALIGN;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const tfm_layer_grads *lg = &gr->layers[l];
    const float *ps[] = {lg->g_attn, lg->wq, lg->wk, lg->wv, lg->wo, lg->g_ffn, lg->w1, lg->w3, lg->w2};
    for (const float *q : ps) {
      if (!q) return TFM_ERR_NULL;
      if (!aligned16(q)) return TFM_ERR_ALIGN;
    }
  }
  const TrainPlan p = plan_train(cfg, B, S);
  if (ws_bytes < p.total) return TFM_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  uint8_t *wb = (uint8_t *)ws;
  const int dt = cfg->dtype;
  const size_t e = elt(dt);
  const int64_t M = (int64_t)B * S, Mp = p.Mp;
  const int D = cfg->d_model, F = cfg->d_ff, V = cfg->vocab, Vp = p.Vp, NL = cfg->n_layers;
  const int Hq = cfg->n_heads, Hkv = cfg->n_kv_heads, dh = cfg->d_head;
  const int qd = Hq * dh, kvd = Hkv * dh, W = qd + 2 * kvd;
  const float eps = cfg->eps;
  auto LA = [&](int l, size_t off) { return wb + p.layers + (size_t)l * p.layer_bytes + off; };
  auto X = [&](int l) { return l < NL ? (float *)LA(l, p.l_x) : (float *)(wb + p.xfinal); };
  int32_t *flags = (int32_t *)(wb + p.flag);
  void *xf = wb + p.xf, *dlog = wb + p.dlog, *dlogT = wb + p.dlogT, *xfT = wb + p.xfT;
  void *wT = wb + p.wT, *dxb = wb + p.dxb, *dxb2 = wb + p.dxb2, *dxT = wb + p.dxT;
  void *hT = wb + p.hT;
  void *dac = wb + p.dac, *dacF = wb + p.dac + (size_t)F * e;
  void *da = wb + p.da, *dc = wb + p.dc, *daT = wb + p.daT, *dcT = wb + p.dcT;
  void *actT = wb + p.actT, *dout = wb + p.dout, *dqkv = wb + p.dqkv, *dqkvT = wb + p.dqkvT;
  float *logits = (float *)(wb + p.logits), *dx = (float *)(wb + p.dx);
  float *dhp = (float *)(wb + p.dh), *du = (float *)(wb + p.du);
  float *rpart = (float *)(wb + p.rms_part);
  float *skp = (float *)(wb + p.splitk);
  // bf16 weight gradients read the stored activations K-major (tokens as rows); the others
  // transpose them first
  auto kmok = [&](const void *a, int64_t lda, const void *b, int64_t ldb, int64_t m, int n) {
    return dt == DT_BF16 && gemm_kmajor_ok(a, lda, b, ldb, m, n, M);
  };

  // ---- forward, keeping each layer's activations ("Transformer 篇" 5.7)
  TFM_HIP(launch_fill_i32(flags, 2, 0, s));
  TFM_HIP(launch_embed(ids, M, w->embed, dt, V, D, X(0), flags, s));
  for (int l = 0; l < NL; ++l) {
    const tfm_layer_weights *lw = &w->layers[l];
    float *x = X(l), *xm = (float *)LA(l, p.l_xm);
    uint8_t *qkv = LA(l, p.l_qkv);
    void *h1 = LA(l, p.l_h1), *o = LA(l, p.l_o), *h2 = LA(l, p.l_h2);
    void *a = LA(l, p.l_a), *c = LA(l, p.l_c), *u = LA(l, p.l_u);
    TFM_HIP(launch_rmsnorm(x, DT_F32, lw->g_attn, dt, h1, dt, M, D, eps, s));
    GemmArgs g{};
    g.a = h1; g.lda = D; g.w0 = lw->wq; g.w1 = lw->wk; g.w2 = lw->wv; g.n0 = qd; g.n1 = kvd;
    g.M = M; g.N = W; g.K = D; g.y = qkv; g.ldy = W; g.y_dt = dt;
    g.positions = positions; g.cos_sin = cos_sin; g.S = S; g.d_head = dh;
    g.max_seq = cfg->max_seq_len;
    TFM_HIP(launch_gemm(EPI_QKV_ROPE, dt, g, s));
    TFM_HIP(launch_attention(qkv, W, qkv + (size_t)qd * e, qkv + (size_t)(qd + kvd) * e, W, o, qd,
                             B, S, Hq, Hkv, dh, dt, layer_window(cfg, l), s,
                             (float *)LA(l, p.l_lse)));
    TFM_TRY(gemm(EPI_RESIDUAL, dt, o, qd, lw->wo, M, D, qd, xm, D, DT_F32, x, s));
    TFM_HIP(launch_rmsnorm(xm, DT_F32, lw->g_ffn, dt, h2, dt, M, D, eps, s));
    if (dt == DT_BF16) {   // one product: gate and up rows interleaved, u, a and c written
      GemmArgs gs{};
      gs.a = h2; gs.lda = D; gs.w0 = lw->w1; gs.w1 = lw->w3; gs.n0 = F; gs.M = M; gs.N = F;
      gs.K = D; gs.y = u; gs.ldy = F; gs.y_dt = dt; gs.keep_a = a; gs.keep_c = c;
      TFM_HIP(launch_gemm(EPI_SWIGLU, dt, gs, s));
    } else {
      TFM_TRY(gemm(EPI_STORE, dt, h2, D, lw->w1, M, F, D, a, F, dt, nullptr, s));
      TFM_TRY(gemm(EPI_STORE, dt, h2, D, lw->w3, M, F, D, c, F, dt, nullptr, s));
      TFM_HIP(launch_swiglu_fwd(a, c, u, dt, M * F, s));
    }
    TFM_TRY(gemm(EPI_RESIDUAL, dt, u, F, lw->w2, M, D, F, X(l + 1), D, DT_F32, xm, s));
  }
  TFM_HIP(launch_rmsnorm(X(NL), DT_F32, w->g_final, dt, xf, dt, M, D, eps, s));

  // ---- loss and its gradient with respect to the logits ("LLM 2" Optimize / Loss)
  int32_t *count = (int32_t *)(wb + p.count);
  float *row_loss = (float *)(wb + p.row_loss);
  if (train_fused_xent(cfg)) {
    // per-tile row maxima / sums of exp and the target logits, combined into each row's
    // log-sum-exp and loss; the gradient product then recomputes the logits tile by tile
    GemmArgs gx{};
    gx.a = xf; gx.lda = D; gx.w0 = w->lm_head; gx.M = M; gx.N = V; gx.K = D;
    gx.targets = targets;
    gx.x_max = (float *)(wb + p.x_max);
    gx.x_sum = (float *)(wb + p.x_sum);
    gx.x_tgt = (float *)(wb + p.x_tgt);
    TFM_HIP(launch_gemm(EPI_XENT, dt, gx, s));
    TFM_HIP(launch_count_targets(targets, M, V, count, s));
    float *x_lse = (float *)(wb + p.x_lse);
    TFM_HIP(launch_xent_reduce(gx.x_max, gx.x_sum, gx.x_tgt, targets, gemm_xent_parts(V), M, V,
                               row_loss, nullptr, s, x_lse, true));
    TFM_HIP(launch_mean_rows(row_loss, M, count, loss_mean, s));
    GemmArgs gg{};
    gg.a = xf; gg.lda = D; gg.w0 = w->lm_head; gg.M = M; gg.N = V; gg.n0 = Vp; gg.K = D;
    gg.y = dlog; gg.ldy = Vp; gg.y_dt = DT_BF16;
    gg.targets = targets; gg.xg_lse = x_lse; gg.xg_count = count;
    TFM_HIP(launch_gemm(EPI_XENT_GRAD, dt, gg, s));
  } else {
    TFM_TRY(gemm(EPI_STORE, dt, xf, D, w->lm_head, M, V, D, logits, Vp, DT_F32, nullptr, s));
    TFM_HIP(launch_ce_backward(logits, Vp, targets, M, V, dlog, dt, Vp, row_loss, count,
                               loss_mean, s));
  }

  // ---- LM head and final RMSNorm
  TFM_HIP(launch_transpose(w->lm_head, dt, D, wT, dt, Vp, Vp, V, D, s));
  TFM_TRY(gemm(EPI_STORE, dt, dlog, Vp, wT, M, D, Vp, dhp, D, DT_F32, nullptr, s));
  float *g_lm = tied ? gr->embed : gr->lm_head;
  if (kmok(dlog, Vp, xf, D, V, D)) {
    TFM_TRY(gemm_wgrad_rows(dlog, Vp, xf, D, V, D, (int)M, g_lm, D, skp, s));
  } else {
    // all Vp columns (the cross-entropy backward zeroes [V, Vp)), so the transpose takes the
    // 16-byte path; rows [V, Vp) of dlogT are zeros the weight-gradient product never reads
    TFM_HIP(launch_transpose(dlog, dt, Vp, dlogT, dt, Mp, Mp, M, Vp, s));
    TFM_HIP(launch_transpose(xf, dt, D, xfT, dt, Mp, Mp, M, D, s));
    TFM_TRY(gemm_wgrad(dt, dlogT, Mp, xfT, V, D, (int)Mp, g_lm, D, skp, s));
  }
  TFM_HIP(launch_fill_f32(dx, M * D, 0.f, s));
  // bf16: the norm backward also leaves the bf16 copy of dx the next products read
  void *dxc = dt == DT_BF16 ? dxb : nullptr;
  TFM_HIP(launch_rms_backward(X(NL), w->g_final, dt, dhp, dx, dxc, gr->g_final, 0, rpart, M, D, eps,
                              s));

  // ---- blocks, last to first; dx holds the gradient of the block's output
  for (int l = NL - 1; l >= 0; --l) {
    const tfm_layer_weights *lw = &w->layers[l];
    const tfm_layer_grads *lg = &gr->layers[l];
    float *x = X(l), *xm = (float *)LA(l, p.l_xm);
    uint8_t *qkv = LA(l, p.l_qkv);
    void *h1 = LA(l, p.l_h1), *o = LA(l, p.l_o), *h2 = LA(l, p.l_h2);
    void *a = LA(l, p.l_a), *c = LA(l, p.l_c), *u = LA(l, p.l_u);
    const uint8_t *dk = (const uint8_t *)dqkv + (size_t)qd * e, *dv = dk + (size_t)kvd * e;
    // bf16: the layer's seven weight gradients run as one grouped launch once its input
    // gradients are done (the gradient of the block output into the FFN stays in dxb, the one
    // into the attention sublayer goes to dxb2)
    const bool grouped = kmok(dxb, D, u, F, D, F) && kmok(dac, 2 * F, h2, D, F, D) &&
                         kmok(dacF, 2 * F, h2, D, F, D) && kmok(dxb2, D, o, qd, D, qd) &&
                         kmok(dqkv, W, h1, D, qd, D) && kmok(dk, W, h1, D, kvd, D) &&
                         kmok(dv, W, h1, D, kvd, D);
    WgradGroup wg{};
    wg.K = (int)M;
    auto job = [&](const void *ja, int64_t jlda, const void *jb, int64_t jldb, float *jy, int jm,
                   int jn) { wg.job[wg.njobs++] = WgradJob{ja, jb, jy, jlda, jldb, jn, jm, jn}; };
    uint8_t *wT2 = wb + p.wTl, *wT13 = wT2 + (size_t)F * D * e;
    uint8_t *wTo = wT13 + (size_t)2 * F * D * e, *wTqkv = wTo + (size_t)qd * D * e;
    if (grouped) {
      const TransposeJob tj[7] = {
          {lw->w2, wT2, F, D, D, F},
          {lw->w1, wT13, D, 2 * F, F, D},
          {lw->w3, wT13 + (size_t)F * e, D, 2 * F, F, D},
          {lw->wo, wTo, qd, D, D, qd},
          {lw->wq, wTqkv, D, W, qd, D},
          {lw->wk, wTqkv + (size_t)qd * e, D, W, kvd, D},
          {lw->wv, wTqkv + (size_t)(qd + kvd) * e, D, W, kvd, D}};
      TFM_HIP(launch_transpose_multi(tj, 7, s));
    }
    // SwiGLU FFN: out = xm + u W2^T, u = SiLU(a) c, a = h2 W1^T, c = h2 W3^T
    if (!dxc) TFM_HIP(launch_convert(dx, DT_F32, dxb, dt, M * D, s));
    if (grouped) {
      // du never leaves the registers: the product's epilogue applies the SwiGLU backward and
      // writes da | dc side by side (rows of 2 F), so one product over K = 2 F against
      // [W1^T | W3^T] gives the input gradient
      GemmArgs gb{};
      gb.a = dxb; gb.lda = D; gb.w0 = wT2; gb.M = M; gb.N = F; gb.K = D;
      gb.y = dac; gb.ldy = 2 * (int64_t)F; gb.y_dt = dt; gb.keep_a = a; gb.keep_c = c;
      TFM_HIP(launch_gemm(EPI_SWIGLU_BACK, dt, gb, s));
      job(dxb, D, u, F, lg->w2, D, F);
      TFM_TRY(gemm(EPI_STORE, dt, dac, 2 * F, wT13, M, D, 2 * F, dhp, D, DT_F32, nullptr, s));
      job(dac, 2 * F, h2, D, lg->w1, F, D);
      job(dacF, 2 * F, h2, D, lg->w3, F, D);
    } else {
      TFM_HIP(launch_transpose(lw->w2, dt, F, wT, dt, D, D, D, F, s));
      TFM_TRY(gemm(EPI_STORE, dt, dxb, D, wT, M, F, D, du, F, DT_F32, nullptr, s));
      if (kmok(dxb, D, u, F, D, F)) {
        TFM_TRY(gemm_wgrad_rows(dxb, D, u, F, D, F, (int)M, lg->w2, F, skp, s));
      } else {
        TFM_HIP(launch_transpose(dxb, dt, D, dxT, dt, Mp, Mp, M, D, s));
        TFM_HIP(launch_transpose(u, dt, F, actT, dt, Mp, Mp, M, F, s));
        TFM_TRY(gemm_wgrad(dt, dxT, Mp, actT, D, F, (int)Mp, lg->w2, F, skp, s));
      }
      TFM_HIP(launch_swiglu_backward(a, c, du, da, dc, dt, M * F, s));
      TFM_HIP(launch_transpose(lw->w1, dt, D, wT, dt, F, F, F, D, s));
      TFM_TRY(gemm(EPI_STORE, dt, da, F, wT, M, D, F, dhp, D, DT_F32, nullptr, s));
      TFM_HIP(launch_transpose(lw->w3, dt, D, wT, dt, F, F, F, D, s));
      TFM_TRY(gemm(EPI_RESIDUAL, dt, dc, F, wT, M, D, F, dhp, D, DT_F32, dhp, s));
      if (kmok(da, F, h2, D, F, D) && kmok(dc, F, h2, D, F, D)) {
        TFM_TRY(gemm_wgrad_rows(da, F, h2, D, F, D, (int)M, lg->w1, D, skp, s));
        TFM_TRY(gemm_wgrad_rows(dc, F, h2, D, F, D, (int)M, lg->w3, D, skp, s));
      } else {
        TFM_HIP(launch_transpose(da, dt, F, daT, dt, Mp, Mp, M, F, s));
        TFM_HIP(launch_transpose(dc, dt, F, dcT, dt, Mp, Mp, M, F, s));
        TFM_HIP(launch_transpose(h2, dt, D, hT, dt, Mp, Mp, M, D, s));
        TFM_TRY(gemm_wgrad(dt, daT, Mp, hT, F, D, (int)Mp, lg->w1, D, skp, s));
        TFM_TRY(gemm_wgrad(dt, dcT, Mp, hT, F, D, (int)Mp, lg->w3, D, skp, s));
      }
    }
    void *dxo = grouped ? dxb2 : dxb;   // bf16 gradient into the attention sublayer
    TFM_HIP(launch_rms_backward(xm, lw->g_ffn, dt, dhp, dx, dxc ? dxo : nullptr, lg->g_ffn, 0,
                                rpart, M, D, eps, s));
    // attention output projection: xm = x + o Wo^T
    if (!dxc) TFM_HIP(launch_convert(dx, DT_F32, dxo, dt, M * D, s));
    if (!grouped) TFM_HIP(launch_transpose(lw->wo, dt, qd, wTo, dt, D, D, D, qd, s));
    TFM_TRY(gemm(EPI_STORE, dt, dxo, D, wTo, M, qd, D, dout, qd, dt, nullptr, s));
    if (grouped) {
      job(dxo, D, o, qd, lg->wo, D, qd);
    } else if (kmok(dxb, D, o, qd, D, qd)) {
      TFM_TRY(gemm_wgrad_rows(dxb, D, o, qd, D, qd, (int)M, lg->wo, qd, skp, s));
    } else {
      TFM_HIP(launch_transpose(dxb, dt, D, dxT, dt, Mp, Mp, M, D, s));
      TFM_HIP(launch_transpose(o, dt, qd, actT, dt, Mp, Mp, M, qd, s));
      TFM_TRY(gemm_wgrad(dt, dxT, Mp, actT, D, qd, (int)Mp, lg->wo, qd, skp, s));
    }
    // attention, and back through the rotations of q and k (applied as dq, dk are stored)
    TFM_HIP(launch_attention_backward(qkv, W, o, qd, dout, qd, dqkv, B, S, Hq, Hkv, dh, dt,
                                      layer_window(cfg, l), (const float *)LA(l, p.l_lse),
                                      (float *)(wb + p.dsum), positions, cos_sin,
                                      cfg->max_seq_len, s));
    // q, k, v projections: one GEMM against [Wq; Wk; Wv]^T for the input gradient
    if (!grouped) {
      TFM_HIP(launch_transpose(lw->wq, dt, D, wTqkv, dt, W, qd, qd, D, s));
      TFM_HIP(launch_transpose(lw->wk, dt, D, wTqkv + (size_t)qd * e, dt, W, kvd, kvd, D, s));
      TFM_HIP(launch_transpose(lw->wv, dt, D, wTqkv + (size_t)(qd + kvd) * e, dt, W, kvd, kvd, D,
                               s));
    }
    TFM_TRY(gemm(EPI_STORE, dt, dqkv, W, wTqkv, M, D, W, dhp, D, DT_F32, nullptr, s));
    if (grouped) {
      job(dqkv, W, h1, D, lg->wq, qd, D);
      job(dk, W, h1, D, lg->wk, kvd, D);
      job(dv, W, h1, D, lg->wv, kvd, D);
      TFM_HIP(launch_gemm_wgrad_group(wg, s));
    } else if (kmok(dqkv, W, h1, D, qd, D) && kmok(dk, W, h1, D, kvd, D) &&
               kmok(dv, W, h1, D, kvd, D)) {
      TFM_TRY(gemm_wgrad_rows(dqkv, W, h1, D, qd, D, (int)M, lg->wq, D, skp, s));
      TFM_TRY(gemm_wgrad_rows(dk, W, h1, D, kvd, D, (int)M, lg->wk, D, skp, s));
      TFM_TRY(gemm_wgrad_rows(dv, W, h1, D, kvd, D, (int)M, lg->wv, D, skp, s));
    } else {
      TFM_HIP(launch_transpose(dqkv, dt, W, dqkvT, dt, Mp, Mp, M, W, s));
      TFM_HIP(launch_transpose(h1, dt, D, hT, dt, Mp, Mp, M, D, s));
      TFM_TRY(gemm_wgrad(dt, dqkvT, Mp, hT, qd, D, (int)Mp, lg->wq, D, skp, s));
      TFM_TRY(gemm_wgrad(dt, (uint8_t *)dqkvT + (size_t)qd * Mp * e, Mp, hT, kvd, D, (int)Mp,
                         lg->wk, D, skp, s));
      TFM_TRY(gemm_wgrad(dt, (uint8_t *)dqkvT + (size_t)(qd + kvd) * Mp * e, Mp, hT, kvd, D,
                         (int)Mp, lg->wv, D, skp, s));
    }
    TFM_HIP(launch_rms_backward(x, lw->g_attn, dt, dhp, dx, dxc, lg->g_attn, 0, rpart, M, D, eps,
                                s));
  }
  // ---- embedding rows (a tied head's gradient is already in gr->embed)
  if (!tied) TFM_HIP(launch_fill_f32(gr->embed, (int64_t)V * D, 0.f, s));
  TFM_HIP(launch_embed_backward(ids, M, V, D, dx, gr->embed, s));
  return TFM_OK;
}

size_t tfm_clip_workspace_bytes(int n_tensors) {
  if (n_tensors < 0) return 0;
  return round256((size_t)(n_tensors > 0 ? n_tensors : 1) * sumsq_parts() * 8);
}

int tfm_grad_clip_coef(const float *const *grads, const int64_t *sizes, int n_tensors,
                       float max_norm, float *coef, float *norm, void *ws, size_t ws_bytes,
                       void *stream) {
  if (n_tensors < 0 || !(max_norm > 0.f)) return TFM_ERR_SHAPE;
  if (!coef || !ws || (n_tensors > 0 && (!grads || !sizes))) return TFM_ERR_NULL;
  for (int i = 0; i < n_tensors; ++i) {
    if (sizes[i] < 0) return TFM_ERR_SHAPE;
    if (sizes[i] > 0 && !grads[i]) return TFM_ERR_NULL;
  }
  if (ws_bytes < tfm_clip_workspace_bytes(n_tensors)) return TFM_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  double *part = (double *)ws;
  const int np = sumsq_parts();
  TFM_HIP(launch_sumsq_multi(grads, sizes, n_tensors, part, s));
  TFM_HIP(launch_clip_coef(part, n_tensors * np, max_norm, coef, norm, s));
  return TFM_OK;
}

int tfm_adamw_step(float *param, void *param_bf16, const float *grad, float *m, float *v,
                   int64_t n, float lr, float beta1, float beta2, float eps, float weight_decay,
                   int step, const float *coef, void *stream) {
  if (n < 0 || step < 1 || !(lr >= 0.f) || !(beta1 >= 0.f && beta1 < 1.f) ||
      !(beta2 >= 0.f && beta2 < 1.f) || !(eps >= 0.f) || !(weight_decay >= 0.f))
    return TFM_ERR_SHAPE;
  if (n == 0) return TFM_OK;
  if (!param || !grad || !m || !v) return TFM_ERR_NULL;
  const float c1 = (float)(1.0 - std::pow((double)beta1, step));
  const float c2 = (float)(1.0 - std::pow((double)beta2, step));
  return hip_status(launch_adamw(param, param_bf16, grad, m, v, n, lr, beta1, beta2, eps,
                                 weight_decay, c1, c2, coef, (hipStream_t)stream));
}

int tfm_adamw_step_multi(float *const *params, void *const *params_bf16,
                         const float *const *grads, float *const *m, float *const *v,
                         const int64_t *sizes, int n_tensors, float lr, float beta1, float beta2,
                         float eps, float weight_decay, int step, const float *coef,
                         void *stream) {
  if (n_tensors < 0 || step < 1 || !(lr >= 0.f) || !(beta1 >= 0.f && beta1 < 1.f) ||
      !(beta2 >= 0.f && beta2 < 1.f) || !(eps >= 0.f) || !(weight_decay >= 0.f))
    return TFM_ERR_SHAPE;
  if (n_tensors == 0) return TFM_OK;
  if (!params || !grads || !m || !v || !sizes) return TFM_ERR_NULL;
  for (int i = 0; i < n_tensors; ++i) {
    if (sizes[i] < 0) return TFM_ERR_SHAPE;
    if (sizes[i] > 0 && (!params[i] || !grads[i] || !m[i] || !v[i])) return TFM_ERR_NULL;
  }
  const float c1 = (float)(1.0 - std::pow((double)beta1, step));
  const float c2 = (float)(1.0 - std::pow((double)beta2, step));
  return hip_status(launch_adamw_multi(params, params_bf16, grads, m, v, sizes, n_tensors, lr,
                                       beta1, beta2, eps, weight_decay, c1, c2, coef,
                                       (hipStream_t)stream));
}

}  // extern "C"


// ---- launch trace

int tfm_trace_begin(int capacity, void *stream) {
  if (capacity <= 0 || capacity > (1 << 20)) return TFM_ERR_SHAPE;
  tfm_trace_free();
  Trace &t = g_trace;
  t.ev.assign((size_t)capacity + 1, nullptr);
  t.label.assign((size_t)capacity + 1, nullptr);
  for (auto &e : t.ev) {
    const hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      e = nullptr;
      tfm_trace_free();
      return hip_status(r);
    }
  }
  t.n = 0;
  t.on = true;
  return mark((hipStream_t)stream, "begin");
}

int tfm_trace_end(int *n_launches) {
  Trace &t = g_trace;
  t.on = false;
  if (n_launches) *n_launches = t.n > 0 ? t.n - 1 : 0;
  return TFM_OK;
}

int tfm_trace_read(float *ms, const char **labels, int n) {
  Trace &t = g_trace;
  if (t.on) return TFM_ERR_SHAPE;
  if (n < 0 || n > t.n - 1) return TFM_ERR_SHAPE;
  if (n > 0 && (!ms || !labels)) return TFM_ERR_NULL;
  if (t.n > 0) TFM_HIP(hipEventSynchronize(t.ev[t.n - 1]));
  for (int i = 0; i < n; ++i) {
    TFM_HIP(hipEventElapsedTime(&ms[i], t.ev[i], t.ev[i + 1]));
    labels[i] = t.label[i + 1];
  }
  return TFM_OK;
}

void tfm_trace_free(void) {
  Trace &t = g_trace;
  for (auto e : t.ev)
    if (e) (void)hipEventDestroy(e);
  t.ev.clear();
  t.label.clear();
  t.n = 0;
  t.on = false;
}

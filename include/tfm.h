/* tfm — forward pass of a pre-norm decoder-only Transformer on AMD MI355X (gfx950).
 *
 * C ABI of libtfm.so. Every compute step runs in hand-written HIP kernels on the caller's
 * stream. The library allocates no device memory and keeps no pointer after a call
 * returns; the caller owns every buffer and keeps it alive until the stream has drained.
 *
 * Sources, by page title and section:
 *  [T1] "从零实现一个完整的 LLM（CS336）——Transformer 篇" (dujian.net): 5.2 Embedding,
 *       5.3 Linear and SwiGLU, 5.4 Attention, 5.5 RoPE, 5.6 RMSNorm, 5.7 assembly.
 *  [T2] "LLM 2: Transformer 原理与实现" (juejin.cn): RMSNorm, SwiGLU FFN, RoPE, GQA/MQA.
 *  [T3] "从零实现一个完整的LLM（CS336）——Transformer篇" (fengye404.top): 7 RoPE, 8 Attention.
 *
 * Common conventions
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *  - Device pointers are marked [dev]; host pointers [host]. All pointers to device data
 *    must be 16-byte aligned unless stated otherwise (TFM_ERR_ALIGN).
 *  - dtype codes: TFM_F32 (IEEE float) and TFM_BF16 (bfloat16, stored as 16-bit words).
 *  - Weight matrices are (out_features, in_features), row-major: y = x W^T  [T1 5.3].
 *  - Activations are (rows, features), row-major; for sequence data rows are (b, s) with
 *    s fastest. The residual stream is float32 for both dtypes.
 *  - Every argument check (null, shape, dtype, alignment, workspace size) runs on the host
 *    before anything is enqueued; on failure nothing is launched and a negative status is
 *    returned. TFM_ERR_HIP means a launch failed; tfm_last_hip_error() gives the code.
 *  - All calls are asynchronous with respect to the host.
 */
#ifndef TFM_H
#define TFM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { TFM_F32 = 0, TFM_BF16 = 1 } tfm_dtype;

typedef enum {
  TFM_OK = 0,
  TFM_ERR_NULL = -1,        /* a required pointer is NULL */
  TFM_ERR_SHAPE = -2,       /* sizes inconsistent or out of range */
  TFM_ERR_DTYPE = -3,       /* unknown dtype or unsupported dtype combination */
  TFM_ERR_WORKSPACE = -4,   /* workspace smaller than the *_workspace_bytes() figure */
  TFM_ERR_ALIGN = -5,       /* pointer or stride not aligned as required */
  TFM_ERR_UNSUPPORTED = -6, /* valid request the library does not implement (e.g. d_head) */
  TFM_ERR_HIP = -7,         /* a HIP launch or copy failed */
  TFM_ERR_TOKEN = -8,       /* a token id was outside [0, vocab) (device-side check) */
  TFM_ERR_POSITION = -9     /* a decode / prefill position was outside the KV cache or the
                               RoPE table (device-side check) */
} tfm_status;

/* Model hyper-parameters. n_heads * d_head need not equal d_model; n_heads % n_kv_heads
 * must be 0 (contiguous query-head groups share a KV head  [T2 GQA]). */
typedef struct {
  int n_layers, d_model, n_heads, n_kv_heads, d_head, d_ff, vocab, max_seq_len;
  float eps;        /* RMSNorm epsilon, inside the square root  [T1 5.6] */
  float rope_theta; /* RoPE base  [T1 5.5] */
  int dtype;        /* tfm_dtype of weights, GEMM operands and activations */
  /* Sliding-window and hybrid attention  [T2 sliding window and hybrid attention]:
   * attn_window > 0 limits each query to its attn_window most recent keys (itself
   * included); 0 = full causal attention. With attn_full_every > 0, layers l with
   * l % attn_full_every == attn_full_every - 1 keep full attention (tfm_model_forward,
   * tfm_model_loss); tfm_block_forward applies attn_window as given. Both >= 0. */
  int attn_window;
  int attn_full_every;
} tfm_config;

/* [dev] pointers of one block's weights, all of the model dtype.
 * g_*: (d_model); wq: (n_heads*d_head, d_model); wk, wv: (n_kv_heads*d_head, d_model);
 * wo: (d_model, n_heads*d_head); w1 (gate), w3 (up): (d_ff, d_model); w2: (d_model, d_ff). */
typedef struct {
  const void *g_attn, *wq, *wk, *wv, *wo, *g_ffn, *w1, *w3, *w2;
} tfm_layer_weights;

/* embed: [dev] (vocab, d_model); layers: [host] array of n_layers; g_final: [dev] (d_model);
 * lm_head: [dev] (vocab, d_model), may equal embed (tied weights). */
typedef struct {
  const void *embed;
  const tfm_layer_weights *layers;
  const void *g_final;
  const void *lm_head;
} tfm_model_weights;

const char *tfm_status_string(int status);
/* hipError_t behind the last TFM_ERR_HIP returned on this thread (0 if none). */
int tfm_last_hip_error(void);
/* Library version string. */
const char *tfm_version(void);

/* Matrix-core rate probe, a measurement helper beside the decoder path: `blocks` workgroups of
 * 4 waves each run `iters` rounds of 8 independent bf16 16x16x32 matrix-core products
 * (2 * 16 * 16 * 32 flops each) on pseudo-random operands held in registers, so
 * flops = blocks * 4 * iters * 8 * 16384; timing the launch gives the rate the chip sustains
 * under random bf16 data (below the published dense peak, which assumes the top clock).
 * sink: [dev] float32, blocks * 4 checksums (caller-owned). Errors: TFM_ERR_NULL, TFM_ERR_SHAPE
 * (iters or blocks <= 0), TFM_ERR_HIP. Asynchronous on `stream`. */
int tfm_mfma_rate(int64_t iters, int blocks, float *sink, void *stream);

/* RoPE table  [T1 5.5; T2 RoPE]: for p in [0, max_seq) and pair i in [0, d_head/2),
 * angle = p * theta^(-2i/d_head) formed in double precision;
 * cos_sin[(p*(d_head/2) + i)*2 + 0] = cos(angle), [... + 1] = sin(angle), stored as float.
 * cos_sin: [dev] max_seq*d_head floats. d_head must be even and > 0. */
int tfm_rope_table_init(float *cos_sin, int max_seq, int d_head, double theta, void *stream);

/* Token embedding  [T1 5.2]: x[r, :] = table[ids[r], :] widened to float32.
 * ids: [dev] int32 (n); table: [dev] (vocab, d) of table_dt; x: [dev] float32 (n, d).
 * An id outside [0, vocab) writes a NaN row and sets *err_flag = 1 ([dev] int32, may be
 * NULL); the caller clears the flag. d % 4 == 0. */
int tfm_embed(const int32_t *ids, int64_t n, const void *table, int table_dt, int vocab, int d,
              float *x, int32_t *err_flag, void *stream);

/* RMSNorm  [T1 5.6; T2 RMSNorm]: y = x / sqrt(mean(x^2) + eps) * g per row of d elements.
 * Sum of squares, scaling and gain are float32; one rounding to y_dt at the store.
 * x: [dev] (rows, d) of x_dt; g: [dev] (d) of g_dt; y: [dev] (rows, d) of y_dt; y may not
 * alias x. d % 4 == 0, rows >= 0 (0 enqueues nothing). */
int tfm_rmsnorm(const void *x, int x_dt, const void *g, int g_dt, void *y, int y_dt,
                int64_t rows, int d, float eps, void *stream);

/* RoPE in place  [T1 5.5; T2 RoPE; T3 7]: x viewed as (B, S, H, d_head) with consecutive
 * tokens `row_stride` elements apart and head h at element offset h*d_head of a row.
 * Adjacent pairs (2i, 2i+1) turn counter-clockwise by pos * theta^(-2i/d_head), using the
 * table from tfm_rope_table_init (max_seq rows). positions: [dev] int32 (B, S) or NULL for
 * 0..S-1 in every sequence; a position outside [0, max_seq) yields NaN for that token.
 * x_dt is TFM_F32 or TFM_BF16; row_stride % 4 == 0, d_head % 4 == 0. */
int tfm_rope(void *x, int x_dt, int64_t row_stride, const int32_t *positions, int B, int S,
             int H, int d_head, const float *cos_sin, int max_seq, void *stream);

/* Linear  [T1 5.3]: y[m, n] = sum_k x[m, k] w[n, k] (+ residual[m, n]).
 * x: [dev] (M, K) of dt, row stride K; w: [dev] (N, K) of dt; y: [dev] (M, ldy) of y_dt.
 * residual: [dev] float32 (M, ldy) or NULL; when given, y_dt must be TFM_F32 and y may
 * equal residual (in-place accumulate). fp32 accumulation. K % 8 == 0 (bf16) or
 * K % 4 == 0 (f32); ldy >= N. ldy need not be a multiple of anything (odd vocab sizes). */
int tfm_linear(const void *x, const void *w, int dt, const float *residual, void *y, int y_dt,
               int64_t M, int N, int K, int64_t ldy, void *stream);

/* Fused QKV projection with RoPE on q and k  [T1 5.4 Q, K, V and 5.5 RoPE; T2 RoPE]:
 * qkv[r, :] = [xn_r W_Q^T | xn_r W_K^T | xn_r W_V^T], then the q and k heads rotate as in
 * tfm_rope (adjacent pairs, position positions[r] or r % S); v is not rotated. The rotation
 * is applied to the fp32 accumulators before the single rounding to dt.
 * xn: [dev] (B*S, d) of dt; wq: [dev] (Hq*d_head, d); wk, wv: [dev] (Hkv*d_head, d);
 * qkv: [dev] (B*S, (Hq + 2 Hkv) d_head) of dt; cos_sin: table of max_seq rows.
 * d % 8 == 0 (bf16) or % 4 (f32); d_head % 4 == 0. */
int tfm_qkv_rope(const void *xn, const void *wq, const void *wk, const void *wv, void *qkv,
                 const int32_t *positions, int B, int S, int d, int Hq, int Hkv, int d_head,
                 const float *cos_sin, int max_seq, int dt, void *stream);

/* Causal multi-head attention  [T1 5.4; T3 8; T2 GQA]:
 * o[b,s,h,:] = sum_{t<=s} softmax_t(q[b,s,h,:] . k[b,t,g,:] / sqrt(d_head)) v[b,t,g,:]
 * with g = h / (Hq/Hkv). Masking follows token order within a sequence (not positions).
 * q: [dev] rows of q_stride elements, head h at offset h*d_head; k, v: rows of kv_stride
 * elements with Hkv heads; o: [dev] rows of o_stride elements, Hq heads. All of dtype dt.
 * Softmax state is float32; for bf16 the probabilities are rounded to bf16 before the PV
 * product. bf16 supports d_head in {32, 64, 128}; f32 supports d_head in {16, 32, 64, 128}.
 * Strides % 8 == 0. bf16 addresses one sequence's keys with 32-bit byte offsets:
 * (S + 64) * kv_stride * 2 must stay below 2^31, else TFM_ERR_UNSUPPORTED. */
int tfm_causal_attention(const void *q, int64_t q_stride, const void *k, const void *v,
                         int64_t kv_stride, void *o, int64_t o_stride, int B, int S, int Hq,
                         int Hkv, int d_head, int dt, void *stream);

/* Sliding-window causal attention  [T2 sliding window and hybrid attention]: as
 * tfm_causal_attention, but query s attends only to the keys max(0, s - window + 1) .. s.
 * window >= S (or 0) is plain causal attention; window < 0 is TFM_ERR_SHAPE. Key tiles wholly
 * outside a query tile's band are never read. */
int tfm_sliding_window_attention(const void *q, int64_t q_stride, const void *k, const void *v,
                                 int64_t kv_stride, void *o, int64_t o_stride, int B, int S,
                                 int Hq, int Hkv, int d_head, int window, int dt, void *stream);

/* SwiGLU FFN  [T1 5.3; T2 SwiGLU FFN]:
 * out = (residual +) W2 ( SiLU(xn W1^T) * (xn W3^T) ), W1 the gate, W3 the up branch.
 * xn: [dev] (rows, d) of dt; w1, w3: [dev] (d_ff, d); w2: [dev] (d, d_ff); residual: [dev]
 * float32 (rows, d) or NULL (may equal out); out: [dev] float32 (rows, d).
 * ws: [dev] workspace of at least tfm_swiglu_workspace_bytes(rows, d_ff, dt) bytes. */
size_t tfm_swiglu_workspace_bytes(int64_t rows, int d_ff, int dt);
int tfm_swiglu_ffn(const void *xn, const void *w1, const void *w3, const void *w2,
                   const float *residual, float *out, int64_t rows, int d, int d_ff, int dt,
                   void *ws, size_t ws_bytes, void *stream);

/* Workspace of tfm_block_forward / tfm_model_forward for B sequences of S tokens. */
size_t tfm_workspace_bytes(const tfm_config *cfg, int B, int S);

/* One pre-norm block  [T1 5.7; T2 FFN & PreNorm] on the float32 residual x (B*S, d_model),
 * in place:  x <- x + W_O attn(RoPE(RMSNorm(x) W_{Q,K,V}^T));  x <- x + SwiGLU(RMSNorm(x)).
 * positions: [dev] int32 (B, S) or NULL; cos_sin: table of cfg->max_seq_len rows.
 * bf16 models with d_model <= 768 split the RMSNorm [T1 5.6] between two products, since its
 * per-row factor commutes with a linear map: RMSNorm(x) W^T = (1/rms(x)) ((x * g) W^T). The
 * product that writes x also writes bf16(x * g) and each row's partial sums of squares; the
 * product that reads it scales its fp32 output rows by 1/rms(x). The bf16 rounding then falls
 * on x * g instead of on x * g / rms(x) (the same relative size). The block's first RMSNorm,
 * and every RMSNorm of the other models, run as the standalone kernel. */
int tfm_block_forward(const tfm_config *cfg, const tfm_layer_weights *w, float *x,
                      const int32_t *positions, int B, int S, const float *cos_sin, void *ws,
                      size_t ws_bytes, void *stream);

/* Whole forward  [T1 5.7]: x = embed[ids]; n_layers blocks; RMSNorm(g_final); logits =
 * x_f lm_head^T for every position, no softmax. bf16 models with d_model <= 768 split each
 * block's RMSNorms as tfm_block_forward does, the first one of block l > 0 into block l-1's
 * down projection; the first block's and the final RMSNorm run standalone.
 * ids: [dev] int32 (B, S); logits: [dev]
 * (B*S, ld_logits) of logits_dt, ld_logits >= vocab (any value; odd is allowed).
 * An out-of-range id is reported by tfm_check_device_flags (NaN logits for that row). */
int tfm_model_forward(const tfm_config *cfg, const tfm_model_weights *w, const int32_t *ids,
                      const int32_t *positions, void *logits, int logits_dt, int64_t ld_logits,
                      int B, int S, const float *cos_sin, void *ws, size_t ws_bytes,
                      void *stream);

/* Fused LM head and next-token cross-entropy  [T2 Optimize / Loss; T3 12 training]:
 * for each row r, loss[r] = log(sum_j exp(z_rj - max_r)) + max_r - z_r,t with z = x w^T and
 * t = targets[r]. The logits are formed tile by tile in float32 and reduced in registers to
 * per-row log-sum-exp partials; they are never written. x: [dev] bf16 (M, K); w: [dev] bf16
 * (V, K); targets: [dev] int32 (M), a negative target means no prediction for that row
 * (loss 0, left out of the mean), a target >= V gives loss NaN; loss: [dev] float32 (M);
 * mean: [dev] one float32 (mean over rows with a target, 0 if none) or NULL.
 * ws: [dev] workspace of at least tfm_xent_workspace_bytes(M, V) bytes. K % 8 == 0; bf16
 * only. The result is deterministic (fixed reduction order). */
size_t tfm_xent_workspace_bytes(int64_t M, int V);
int tfm_lm_head_xent(const void *x, const void *w, const int32_t *targets, float *loss,
                     float *mean, int64_t M, int V, int K, void *ws, size_t ws_bytes,
                     void *stream);

/* Whole forward ending in the fused cross-entropy instead of logits  [T1 5.7; T2 Optimize /
 * Loss]: the trunk of tfm_model_forward, then tfm_lm_head_xent on RMSNorm(x; g_final).
 * For next-token training targets[b, s] = ids[b, s + 1] and -1 at s = S - 1. bf16 models only
 * (TFM_ERR_UNSUPPORTED otherwise). ws: at least tfm_loss_workspace_bytes(cfg, B, S) bytes;
 * out-of-range ids are reported by tfm_check_device_flags as for the forward. */
size_t tfm_loss_workspace_bytes(const tfm_config *cfg, int B, int S);
int tfm_model_loss(const tfm_config *cfg, const tfm_model_weights *w, const int32_t *ids,
                   const int32_t *positions, const int32_t *targets, float *loss, float *mean,
                   int B, int S, const float *cos_sin, void *ws, size_t ws_bytes, void *stream);

/* ---- KV-cache incremental decoding  [T4 6.1 KV cache: keep every step's keys and values,
 * compute only the new token's q, k, v, append, then attend; T2 GQA/MQA: generation reads the
 * cache every step, which grouped heads shrink; T2 RoPE: with a cache, positions are the
 * tokens' real places in the context]. bf16 models with d_head in {32, 64, 128}, at most 8
 * query heads per kv head and cache_seq <= 131072 for decoding (TFM_ERR_UNSUPPORTED
 * otherwise).
 *
 * Cache: a caller-owned device buffer of tfm_kv_cache_bytes(cfg, B, cache_seq) bytes, 16-byte
 * aligned: per layer l a K block at element 2 l blk and a V block at (2 l + 1) blk,
 * blk = B * n_kv_heads * cache_seq * d_head, each laid out (B, n_kv_heads, cache_seq, d_head)
 * bf16. Slot t of sequence b holds the rotated key / the value of its token at position t. */
size_t tfm_kv_cache_bytes(const tfm_config *cfg, int B, int cache_seq);

/* Prefill: tfm_model_forward over (B, S) tokens that also stores every layer's rotated k and
 * v in the cache slots of the tokens' positions (positions[b, s], default s). logits may be
 * NULL (fill the cache only). Workspace as tfm_model_forward. A position outside
 * [0, cache_seq) stores nothing and makes tfm_check_device_flags return TFM_ERR_POSITION. */
int tfm_model_prefill(const tfm_config *cfg, const tfm_model_weights *w, const int32_t *ids,
                      const int32_t *positions, void *logits, int logits_dt, int64_t ld_logits,
                      int B, int S, const float *cos_sin, void *kv_cache, int cache_seq,
                      void *ws, size_t ws_bytes, void *stream);

/* Decode step: one new token ids[b] per sequence at position positions[b] ([dev] int32 (B),
 * required; sequences may sit at different positions). In every layer q and k rotate at that
 * position, k and v go to cache slot positions[b], and the token attends to slots
 * 0 .. positions[b] (the last attn_window of them on windowed layers). logits: [dev]
 * (B, ld_logits) of logits_dt. A position outside [0, min(cache_seq, max_seq_len)) gives a
 * NaN row, writes no slot and makes tfm_check_device_flags return TFM_ERR_POSITION.
 * ws: at least tfm_decode_workspace_bytes(cfg, B, cache_seq) bytes. */
size_t tfm_decode_workspace_bytes(const tfm_config *cfg, int B, int cache_seq);
int tfm_model_decode(const tfm_config *cfg, const tfm_model_weights *w, const int32_t *ids,
                     const int32_t *positions, void *logits, int logits_dt, int64_t ld_logits,
                     int B, const float *cos_sin, void *kv_cache, int cache_seq, void *ws,
                     size_t ws_bytes, void *stream);

/* Decode attention alone: o[b, h, :] = softmax over the cache slots t of sequence b,
 * 0 .. positions[b] (the last `window` of them when window > 0), of q[b, h] . k[b, g, t] /
 * sqrt(d_head), applied to v[b, g, t], with g = h / (Hq / Hkv). q: [dev] (B, q_stride) bf16;
 * k_cache, v_cache: [dev] (B, Hkv, cache_seq, d_head) bf16; o: [dev] (B, o_stride) bf16;
 * positions: [dev] int32 (B); a position outside [0, cache_seq) gives a NaN row. Strides
 * % 8 == 0. ws: tfm_decode_attention_workspace_bytes(B, Hq, d_head, cache_seq) bytes. */
size_t tfm_decode_attention_workspace_bytes(int B, int Hq, int d_head, int cache_seq);
int tfm_decode_attention(const void *q, int64_t q_stride, const void *k_cache,
                         const void *v_cache, const int32_t *positions, void *o,
                         int64_t o_stride, int B, int Hq, int Hkv, int d_head, int cache_seq,
                         int window, void *ws, size_t ws_bytes, void *stream);

/* Decode attention for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): tfm_decode_attention with
 * the same arguments, kernels and results, but its split records live in a static device
 * array of tfm_decode_attention_noalloc_max_bytes() bytes (4 MiB) that each GPU holds until the
 * process ends, instead of a caller workspace. Allocates nothing: no hipMalloc, no hipFree. The
 * first call on a device looks up the array's address on the device of `stream` (once per
 * device). A call whose records would exceed the array, i.e. whose
 * tfm_decode_attention_workspace_bytes(B, Hq, d_head, cache_seq) is larger, returns
 * TFM_ERR_WORKSPACE before any launch. Every call on one GPU uses the same array, so calls that
 * overlap on one GPU (on different streams, or from different threads) race; calls on one
 * stream are ordered. Nothing in the array needs to start at zero: each call writes every
 * record it reads. */
size_t tfm_decode_attention_noalloc_max_bytes(void);
int tfm_decode_attention_noalloc(const void *q, int64_t q_stride, const void *k_cache,
                                 const void *v_cache, const int32_t *positions, void *o,
                                 int64_t o_stride, int B, int Hq, int Hkv, int d_head,
                                 int cache_seq, int window, void *stream);

/* ---- Training step  [T2 Optimize: Loss, Optimizer - AdamW, Gradient Clip; T3 12 training
 * loop: loss, backward, clip, step]. fp32 gradients; fp32 master weights and moments. */
typedef struct {
  float *g_attn, *wq, *wk, *wv, *wo, *g_ffn, *w1, *w3, *w2;
} tfm_layer_grads;

typedef struct {
  float *embed;
  const tfm_layer_grads *layers; /* host array of n_layers */
  float *g_final, *lm_head;      /* lm_head: NULL or == embed when the head is tied */
} tfm_model_grads;

/* Workspace of tfm_model_backward: every layer's forward activations, the logits and their
 * gradient, transposed operands and activation gradients (0 if the configuration is not
 * supported for training). */
size_t tfm_train_workspace_bytes(const tfm_config *cfg, int B, int S);

/* Training forward and backward: loss_mean ([dev] 1 float) = mean next-token cross-entropy over
 * the rows with 0 <= targets[r] < vocab ([dev] int32 (B, S); others are ignored), and the
 * gradient of that mean with respect to every parameter written to the fp32 buffers of grads
 * (shapes of the weights; overwritten). A tied head (w->lm_head == w->embed) adds its gradient
 * into grads->embed. The forward keeps bf16 (or fp32) activations; the backward's products run
 * on the forward's GEMM kernels with transposed operands. d_model <= 2048, d_head in
 * {16 (fp32 only), 32, 64, 128}; TFM_ERR_UNSUPPORTED otherwise. All pointers 16-byte aligned.
 * The token flag (tfm_check_device_flags) works as for the forward. */
int tfm_model_backward(const tfm_config *cfg, const tfm_model_weights *w, const int32_t *ids,
                       const int32_t *positions, const int32_t *targets, float *loss_mean,
                       const tfm_model_grads *grads, int B, int S, const float *cos_sin,
                       void *ws, size_t ws_bytes, void *stream);

/* Global-norm clipping coefficient  [T2 Gradient Clip]: norm = sqrt(sum over the n tensors of
 * sum g^2); coef[0] = max_norm / (norm + 1e-6) when norm > max_norm, else 1; norm[0] (nullable)
 * = norm. grads, sizes: host arrays of n device pointers (fp32) and element counts; coef, norm:
 * [dev] 1 float. ws: tfm_clip_workspace_bytes(n) bytes. Sums in fp64 in a fixed order. */
size_t tfm_clip_workspace_bytes(int n_tensors);
int tfm_grad_clip_coef(const float *const *grads, const int64_t *sizes, int n_tensors,
                       float max_norm, float *coef, float *norm, void *ws, size_t ws_bytes,
                       void *stream);

/* One AdamW step  [T2 Optimizer - AdamW] on n parameters, in place: g = grad * coef[0] (coef
 * nullable: 1); m = b1 m + (1 - b1) g; v = b2 v + (1 - b2) g^2; param = param - lr
 * (m / (1 - b1^step)) / (sqrt(v / (1 - b2^step)) + eps) - lr weight_decay param (decay on the
 * value before the step). param, grad, m, v: [dev] fp32; param_bf16 (nullable): [dev] bf16
 * copy written with the new value. step >= 1; m, v zero before step 1. */
int tfm_adamw_step(float *param, void *param_bf16, const float *grad, float *m, float *v,
                   int64_t n, float lr, float beta1, float beta2, float eps, float weight_decay,
                   int step, const float *coef, void *stream);

/* tfm_adamw_step on n_tensors tensors in a few launches (up to 32 tensors each), with the
 * same per-element arithmetic, so the results equal n_tensors single calls bit for bit.
 * params, grads, m, v, sizes: host arrays of n_tensors entries (device pointers, element
 * counts); params_bf16: host array (nullable; entries nullable) of bf16 copies. A tensor of
 * size 0 is skipped (its pointers may be NULL). */
int tfm_adamw_step_multi(float *const *params, void *const *params_bf16,
                         const float *const *grads, float *const *m, float *const *v,
                         const int64_t *sizes, int n_tensors, float lr, float beta1, float beta2,
                         float eps, float weight_decay, int step, const float *coef,
                         void *stream);

/* ---- Launch trace (measurement): while a trace is on for the calling thread, every kernel
 * launch of tfm_block_forward, tfm_model_forward, tfm_model_loss and tfm_model_prefill records
 * a HIP event on the call's stream right after it, labelled with the kernel's step
 * ("embed", "rmsnorm", "gemm_qkv_rope", "attention", "attention_window", "gemm_out_residual",
 * "gemm_swiglu", "gemm_down_residual", "gemm_lm_head", "gemm_lm_head_xent", "xent_reduce",
 * "kv_store", "fill_flags"), so each launch's time inside a real step is the elapsed time
 * between consecutive events (the launch plus any gap before it). Launches beyond `capacity`
 * are not recorded. The library creates the events (no device memory) and keeps them until
 * tfm_trace_free or the next tfm_trace_begin.
 * tfm_trace_begin: starts a trace of up to `capacity` launches and records the first event on
 *   `stream`; TFM_ERR_SHAPE for capacity outside [1, 2^20].
 * tfm_trace_end: stops recording; *n_launches (nullable) = launches recorded.
 * tfm_trace_read: after tfm_trace_end, waits for the last event and writes, for launch i < n,
 *   ms[i] = its time in milliseconds and labels[i] = its label (static strings); n at most the
 *   launches recorded (TFM_ERR_SHAPE otherwise, or while the trace is on). */
int tfm_trace_begin(int capacity, void *stream);
int tfm_trace_end(int *n_launches);
int tfm_trace_read(float *ms, const char **labels, int n);
void tfm_trace_free(void);

/* Waits for `stream`, then returns TFM_ERR_TOKEN if the last whole-model call that used this
 * workspace saw an out-of-range token id, TFM_ERR_POSITION if it saw a position outside the
 * KV cache or the RoPE table (prefill / decode), else TFM_OK. */
int tfm_check_device_flags(const void *ws, void *stream);

#ifdef __cplusplus
}
#endif
#endif

/* Plain fp64 CPU oracle for the forward pass of a pre-norm decoder-only Transformer
 * (RMSNorm, RoPE, causal multi-head attention with grouped KV heads, SwiGLU, LM head).
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the benchmark's
 * CPU-baseline leg may load this library. The HIP library never calls it and shares no
 * source, header, table or helper with it.
 *
 * Conventions
 *  - Inputs that are model weights arrive as float32 (for bf16 models, already rounded to
 *    bf16 values); every computation and every result is double precision.
 *  - Weight matrices are (out_features, in_features), row-major: y = x W^T.
 *  - Activations are (rows, features) row-major, rows = batch * seq ordered (b, s).
 *  - Every output element is computed by one thread, summing in natural index order, so
 *    results do not depend on the number of OpenMP threads.
 *
 * Sources, by page title and section:
 *  [T1] "从零实现一个完整的 LLM（CS336）——Transformer 篇" (dujian.net): 5.3 Linear and
 *       SwiGLU, 5.4 Attention, 5.5 RoPE, 5.6 RMSNorm, 5.7 model assembly.
 *  [T2] "LLM 2: Transformer 原理与实现" (juejin.cn): RMSNorm, SwiGLU FFN, RoPE, GQA.
 *  [T3] "从零实现一个完整的LLM（CS336）——Transformer篇" (fengye404.top): 6 RMSNorm,
 *       7 RoPE, 8 Attention, 9 SwiGLU, 10 model assembly, 12 training (loss, checks).
 *  [T2 Optimize / Loss]: next-token cross-entropy in the logsumexp form.
 *
 * Parity pins: every function below is pinned by a CPU test against page values, closed
 * forms, invariants or brute force, except oracle_model at the real workload sizes, whose
 * full-size values are "parity unpinned" beyond the invariants (the pages print no logits).
 */
#ifndef TFM_ORACLE_H
#define TFM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int n_layers, d_model, n_heads, n_kv_heads, d_head, d_ff, vocab;
  double eps, theta;
  /* [T2 sliding window and hybrid attention]: window > 0 limits every query to its `window`
   * most recent keys (itself included); with full_every > 0, layers l with
   * l % full_every == full_every - 1 keep full causal attention. oracle_block uses `window`
   * as given. */
  int window, full_every;
} oracle_cfg;

typedef struct {
  const float *g_attn, *wq, *wk, *wv, *wo, *g_ffn, *w1, *w3, *w2;
} oracle_layer;

/* x[r, :] = E[ids[r], :]  [T1 5.2 Embedding]. Returns -1 if an id is outside [0, vocab). */
int oracle_embedding(const int32_t *ids, int64_t n, const float *E, int vocab, int d, double *x);

/* y = x / sqrt(mean(x^2) + eps) * g, per row  [T1 5.6; T2 RMSNorm]. */
void oracle_rmsnorm(const double *x, int64_t rows, int d, const double *g, double eps, double *y);

/* y = x W^T with W (n_out, n_in)  [T1 5.3 Linear]. */
void oracle_linear(const double *x, int64_t rows, int n_in, const float *W, int n_out, double *y);

/* In-place RoPE on x viewed as (B, S, H, dh) with rows of `row_stride` doubles: adjacent
 * pairs (2i, 2i+1) rotate counter-clockwise by p * theta^(-2i/dh)  [T1 5.5; T2 RoPE;
 * T3 7]. p = pos[b*S + s] when pos is given, else s. */
void oracle_rope(double *x, int B, int S, int H, int dh, int64_t row_stride,
                 const int32_t *pos, double theta);

/* Row-wise softmax over n entries, max-subtracted two-pass form  [T1 5.4; T3 8]. */
void oracle_softmax(const double *s, int64_t rows, int n, double *p);

/* Causal attention per (b, head): o_s = sum_{t<=s} softmax_t(q_s . k_t / sqrt(dh)) v_t.
 * q: rows of q_stride doubles, head j at columns [j*dh, (j+1)*dh); k, v: rows of kv_stride
 * doubles with Hkv heads. Query head j reads KV head j / (Hq/Hkv)  [T1 5.4; T2 GQA].
 * o: (B*S, Hq*dh). probs (nullable): (B, Hq, S, S) with zeros above the diagonal. */
void oracle_attention(const double *q, int64_t q_stride, const double *k, const double *v,
                      int64_t kv_stride, int B, int S, int Hq, int Hkv, int dh, double *o,
                      double *probs);

/* Sliding-window causal attention  [T2 sliding window]: as oracle_attention, but query s sees
 * the keys t with max(0, s - window + 1) <= t <= s; window <= 0 means no limit. probs has zeros
 * outside the band. */
void oracle_attention_window(const double *q, int64_t q_stride, const double *k, const double *v,
                             int64_t kv_stride, int B, int S, int Hq, int Hkv, int dh, int window,
                             double *o, double *probs);

/* The rows of oracle_attention_window listed in `rows` (row = b*S + s), every head; o is
 * (n_rows, Hq*dh). Same definition, for sampled checks at sizes where all rows would be slow. */
void oracle_attention_rows(const double *q, int64_t q_stride, const double *k, const double *v,
                           int64_t kv_stride, int B, int S, int Hq, int Hkv, int dh, int window,
                           const int64_t *rows, int64_t n_rows, double *o);

/* SiLU(u) = u * sigmoid(u)  [T1 5.3; T2 SiLU]. */
double oracle_silu(double u);

/* out = (SiLU(h W1^T) * (h W3^T)) W2^T; W1 gate, W3 up, W2 down  [T1 5.3; T2 SwiGLU].
 * u (nullable): the (rows, d_ff) gated hidden before W2. */
void oracle_swiglu(const double *h, int64_t rows, int d, int d_ff, const float *w1,
                   const float *w3, const float *w2, double *out, double *u);

/* One pre-norm block on the residual x (B*S, D), in place  [T1 5.7; T2 FFN & PreNorm]:
 * x <- x + W_O attn(rope(RMSNorm(x) W_{Q,K,V}^T)); x <- x + SwiGLU(RMSNorm(x)). */
void oracle_block(const oracle_cfg *c, const oracle_layer *w, double *x, const int32_t *pos,
                  int B, int S);

/* Whole forward  [T1 5.7]: x = E[ids]; blocks; x_f = RMSNorm(x; g_final); logits = x_f W_lm^T.
 * x_final (nullable): (B*S, D). logits (nullable): (n_rows, vocab) for the rows listed in
 * `rows` (row r = b*S + s), or for all B*S rows when rows is NULL. Returns -1 on a bad id. */
int oracle_model(const oracle_cfg *c, const float *embed, const oracle_layer *layers,
                 const float *g_final, const float *lm_head, const int32_t *ids,
                 const int32_t *pos, int B, int S, double *x_final, const int64_t *rows,
                 int64_t n_rows, double *logits);

/* Next-token cross-entropy  [T2 Optimize / Loss; T3 12 training]: per row r with target
 * t = targets[r] in [0, V): loss[r] = log(sum_j exp(logits[r, j] - max_r)) + max_r
 * - logits[r, t], the max-subtracted logsumexp form. Rows with a negative target are
 * ignored: loss[r] = 0 and they are left out of the mean. Returns the mean over the counted
 * rows (0 when none), or NAN if a target is >= V. */
double oracle_cross_entropy(const double *logits, int64_t rows, int V, const int32_t *targets,
                            double *loss);

/* Threads the OpenMP runtime will use for the loops above. */
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

/* ---- training step (oracle_train.c)  [T2 Optimize: Loss, AdamW; T3 12 training]. All
 * parameters and gradients in double. lm_head may equal embed (tied); then the gradient
 * buffers must be tied the same way and receive the sum. */
typedef struct {
  double *g_attn, *wq, *wk, *wv, *wo, *g_ffn, *w1, *w3, *w2;
} oracle_layer_d;

typedef struct {
  double *embed;
  oracle_layer_d *layers;
  double *g_final, *lm_head;
} oracle_params_d;

/* Mean next-token cross-entropy over rows with 0 <= targets[r] < vocab (0 if none) and its
 * gradient with respect to every parameter, ADDED into the buffers of g (zero them first).
 * Returns the loss, or NaN if an id is outside the vocabulary. */
double oracle_model_grads(const oracle_cfg *c, const oracle_params_d *p, const int32_t *ids,
                          const int32_t *pos, const int32_t *targets, int B, int S,
                          const oracle_params_d *g);

/* One AdamW step in place on n parameters; t is the 1-based step count. */
void oracle_adamw(double *theta, const double *grad, double *m, double *v, int64_t n, double lr,
                  double b1, double b2, double eps, double wd, int t);

#ifdef __cplusplus
}
#endif
#endif

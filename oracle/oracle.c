/* Plain fp64 CPU oracle (test infrastructure only; see oracle.h for the conventions and
 * the page citations [T1], [T2], [T3]). Written for readability, not speed: every step is
 * the definition on the pages, one loop per formula. */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads the following parallel loops use (timing of the baseline at several counts). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* [T1 5.2 Embedding]: a table lookup, row id of E. */
int oracle_embedding(const int32_t *ids, int64_t n, const float *E, int vocab, int d, double *x) {
  for (int64_t r = 0; r < n; ++r)
    if (ids[r] < 0 || ids[r] >= vocab) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    const float *e = E + (int64_t)ids[r] * d;
    for (int j = 0; j < d; ++j) x[r * d + j] = (double)e[j];
  }
  return 0;
}

/* [T1 5.6 RMSNorm; T2 RMSNorm]: RMS(a) = sqrt(mean_i a_i^2 + eps), y_i = a_i / RMS(a) * g_i.
 * eps sits inside the square root. */
void oracle_rmsnorm(const double *x, int64_t rows, int d, const double *g, double eps, double *y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const double *a = x + r * d;
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += a[i] * a[i];
    double rms = sqrt(ss / d + eps);
    for (int i = 0; i < d; ++i) y[r * d + i] = a[i] / rms * g[i];
  }
}

/* [T1 5.3 Linear]: no bias; output o of row r is the dot product of x_r with row o of W. */
void oracle_linear(const double *x, int64_t rows, int n_in, const float *W, int n_out, double *y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const double *xr = x + r * n_in;
    for (int o = 0; o < n_out; ++o) {
      const float *w = W + (int64_t)o * n_in;
      double acc = 0.0;
      for (int i = 0; i < n_in; ++i) acc += xr[i] * (double)w[i];
      y[r * n_out + o] = acc;
    }
  }
}

/* [T1 5.5 RoPE; T2 RoPE; T3 7 RoPE]: pair i of a head holds components (2i, 2i+1) and turns
 * by the angle p * omega_i, omega_i = theta^(-2i/dh) (i from 0; the pages' f_k with k from 1
 * is the same sequence). The rotation is counter-clockwise:
 *   (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a).
 * Angles and their cos/sin are formed in double precision. */
void oracle_rope(double *x, int B, int S, int H, int dh, int64_t row_stride,
                 const int32_t *pos, double theta) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)B * S; ++r) {
    int s = (int)(r % S);
    double p = pos ? (double)pos[r] : (double)s;
    for (int h = 0; h < H; ++h) {
      double *v = x + r * row_stride + (int64_t)h * dh;
      for (int i = 0; i < dh / 2; ++i) {
        double omega = pow(theta, -2.0 * i / dh);
        double a = p * omega;
        double c = cos(a), sn = sin(a);
        double x0 = v[2 * i], x1 = v[2 * i + 1];
        v[2 * i] = x0 * c - x1 * sn;
        v[2 * i + 1] = x0 * sn + x1 * c;
      }
    }
  }
}

/* [T1 5.4; T3 8]: subtract the row maximum, exponentiate, divide by the sum. */
void oracle_softmax(const double *s, int64_t rows, int n, double *p) {
  for (int64_t r = 0; r < rows; ++r) {
    const double *a = s + r * n;
    double m = a[0];
    for (int j = 1; j < n; ++j) if (a[j] > m) m = a[j];
    double sum = 0.0;
    for (int j = 0; j < n; ++j) sum += exp(a[j] - m);
    for (int j = 0; j < n; ++j) p[r * n + j] = exp(a[j] - m) / sum;
  }
}

/* [T1 5.4 Attention; T3 8]: scores q.k / sqrt(dh) over the visible keys t <= s (the causal
 * mask gives the others weight exactly 0), a max-subtracted softmax over them, then the
 * probability-weighted sum of the value rows. [T2 GQA]: a contiguous group of Hq/Hkv query
 * heads shares one KV head. One query row of one head; sc is scratch of >= s+1 doubles. */
static void attend_one(const double *q, int64_t q_stride, const double *k, const double *v,
                       int64_t kv_stride, int S, int Hq, int Hkv, int dh, int b, int h, int s,
                       int window, double *os, double *prow, double *sc) {
  const int g = h / (Hq / Hkv);
  const double scale = 1.0 / sqrt((double)dh);
  const double *qs = q + ((int64_t)b * S + s) * q_stride + (int64_t)h * dh;
  /* [T2 sliding window]: with a window W > 0 the query sees only the W most recent keys */
  const int t0 = (window > 0 && s - window + 1 > 0) ? s - window + 1 : 0;
  double m = -INFINITY;
  for (int t = t0; t <= s; ++t) {
    const double *kt = k + ((int64_t)b * S + t) * kv_stride + (int64_t)g * dh;
    double dot = 0.0;
    for (int e = 0; e < dh; ++e) dot += qs[e] * kt[e];
    sc[t] = dot * scale;
    if (sc[t] > m) m = sc[t];
  }
  double sum = 0.0;
  for (int t = t0; t <= s; ++t) sum += exp(sc[t] - m);
  for (int e = 0; e < dh; ++e) os[e] = 0.0;
  for (int t = t0; t <= s; ++t) {
    double pt = exp(sc[t] - m) / sum;
    if (prow) prow[t] = pt;
    const double *vt = v + ((int64_t)b * S + t) * kv_stride + (int64_t)g * dh;
    for (int e = 0; e < dh; ++e) os[e] += pt * vt[e];
  }
  if (prow) {
    for (int t = 0; t < t0; ++t) prow[t] = 0.0;
    for (int t = s + 1; t < S; ++t) prow[t] = 0.0;
  }
}

void oracle_attention_window(const double *q, int64_t q_stride, const double *k, const double *v,
                             int64_t kv_stride, int B, int S, int Hq, int Hkv, int dh, int window,
                             double *o, double *probs) {
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hq; ++h) {
      double *sc = (double *)malloc(sizeof(double) * (size_t)S);
      for (int s = 0; s < S; ++s)
        attend_one(q, q_stride, k, v, kv_stride, S, Hq, Hkv, dh, b, h, s, window,
                   o + ((int64_t)b * S + s) * ((int64_t)Hq * dh) + (int64_t)h * dh,
                   probs ? probs + (((int64_t)b * Hq + h) * S + s) * S : NULL, sc);
      free(sc);
    }
}

void oracle_attention(const double *q, int64_t q_stride, const double *k, const double *v,
                      int64_t kv_stride, int B, int S, int Hq, int Hkv, int dh, double *o,
                      double *probs) {
  oracle_attention_window(q, q_stride, k, v, kv_stride, B, S, Hq, Hkv, dh, 0, o, probs);
}

void oracle_attention_rows(const double *q, int64_t q_stride, const double *k, const double *v,
                           int64_t kv_stride, int B, int S, int Hq, int Hkv, int dh, int window,
                           const int64_t *rows, int64_t n_rows, double *o) {
  (void)B;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t i = 0; i < n_rows; ++i)
    for (int h = 0; h < Hq; ++h) {
      const int b = (int)(rows[i] / S), s = (int)(rows[i] % S);
      double *sc = (double *)malloc(sizeof(double) * (size_t)S);
      attend_one(q, q_stride, k, v, kv_stride, S, Hq, Hkv, dh, b, h, s, window,
                 o + i * ((int64_t)Hq * dh) + (int64_t)h * dh, NULL, sc);
      free(sc);
    }
}

/* [T1 5.3; T2 SiLU]: SiLU(u) = u * sigmoid(u), sigmoid(u) = 1 / (1 + e^-u). */
double oracle_silu(double u) { return u / (1.0 + exp(-u)); }

/* [T1 5.3 SwiGLU; T2 SwiGLU FFN]: W1 x through SiLU is the gate, W3 x the content branch;
 * their elementwise product goes through W2. */
void oracle_swiglu(const double *h, int64_t rows, int d, int d_ff, const float *w1,
                   const float *w3, const float *w2, double *out, double *u) {
  double *a = (double *)malloc(sizeof(double) * (size_t)(rows * d_ff));
  double *c = (double *)malloc(sizeof(double) * (size_t)(rows * d_ff));
  oracle_linear(h, rows, d, w1, d_ff, a);
  oracle_linear(h, rows, d, w3, d_ff, c);
  for (int64_t i = 0; i < rows * d_ff; ++i) a[i] = oracle_silu(a[i]) * c[i];
  if (u) memcpy(u, a, sizeof(double) * (size_t)(rows * d_ff));
  oracle_linear(a, rows, d_ff, w2, d, out);
  free(a);
  free(c);
}

static void widen(const float *src, int n, double *dst) {
  for (int i = 0; i < n; ++i) dst[i] = (double)src[i];
}

/* [T1 5.7 TransformerBlock; T2 FFN & PreNorm]: pre-norm residual block,
 *   z = x + MHA(RMSNorm(x)),   y = z + SwiGLU(RMSNorm(z)).
 * MHA [T1 5.5]: q, k, v projections, head split (head j = columns j*dh..), RoPE on q and k
 * only, causal attention per head, head merge, output projection. */
void oracle_block(const oracle_cfg *c, const oracle_layer *w, double *x, const int32_t *pos,
                  int B, int S) {
  const int64_t M = (int64_t)B * S;
  const int D = c->d_model, qd = c->n_heads * c->d_head, kvd = c->n_kv_heads * c->d_head;
  double *g = (double *)malloc(sizeof(double) * (size_t)D);
  double *h = (double *)malloc(sizeof(double) * (size_t)(M * D));
  double *q = (double *)malloc(sizeof(double) * (size_t)(M * qd));
  double *k = (double *)malloc(sizeof(double) * (size_t)(M * kvd));
  double *v = (double *)malloc(sizeof(double) * (size_t)(M * kvd));
  double *o = (double *)malloc(sizeof(double) * (size_t)(M * qd));
  double *y = (double *)malloc(sizeof(double) * (size_t)(M * D));

  widen(w->g_attn, D, g);
  oracle_rmsnorm(x, M, D, g, c->eps, h);
  oracle_linear(h, M, D, w->wq, qd, q);
  oracle_linear(h, M, D, w->wk, kvd, k);
  oracle_linear(h, M, D, w->wv, kvd, v);
  oracle_rope(q, B, S, c->n_heads, c->d_head, qd, pos, c->theta);
  oracle_rope(k, B, S, c->n_kv_heads, c->d_head, kvd, pos, c->theta);
  oracle_attention_window(q, qd, k, v, kvd, B, S, c->n_heads, c->n_kv_heads, c->d_head, c->window,
                          o, NULL);
  oracle_linear(o, M, qd, w->wo, D, y);
  for (int64_t i = 0; i < M * D; ++i) x[i] += y[i];

  widen(w->g_ffn, D, g);
  oracle_rmsnorm(x, M, D, g, c->eps, h);
  oracle_swiglu(h, M, D, c->d_ff, w->w1, w->w3, w->w2, y, NULL);
  for (int64_t i = 0; i < M * D; ++i) x[i] += y[i];

  free(g); free(h); free(q); free(k); free(v); free(o); free(y);
}

/* [T1 5.7 TransformerLM]: embedding, the blocks in order, final RMSNorm, LM head. */
int oracle_model(const oracle_cfg *c, const float *embed, const oracle_layer *layers,
                 const float *g_final, const float *lm_head, const int32_t *ids,
                 const int32_t *pos, int B, int S, double *x_final, const int64_t *rows,
                 int64_t n_rows, double *logits) {
  const int64_t M = (int64_t)B * S;
  const int D = c->d_model;
  double *x = (double *)malloc(sizeof(double) * (size_t)(M * D));
  if (oracle_embedding(ids, M, embed, c->vocab, D, x) != 0) { free(x); return -1; }
  for (int l = 0; l < c->n_layers; ++l) {
    /* [T2 hybrid attention]: windowed layers, except every full_every-th layer */
    oracle_cfg cl = *c;
    const int full = c->full_every > 0 && l % c->full_every == c->full_every - 1;
    cl.window = full ? 0 : c->window;
    oracle_block(&cl, &layers[l], x, pos, B, S);
  }

  double *g = (double *)malloc(sizeof(double) * (size_t)D);
  double *xf = (double *)malloc(sizeof(double) * (size_t)(M * D));
  widen(g_final, D, g);
  oracle_rmsnorm(x, M, D, g, c->eps, xf);
  if (x_final) memcpy(x_final, xf, sizeof(double) * (size_t)(M * D));
  if (logits) {
    if (rows == NULL) {
      oracle_linear(xf, M, D, lm_head, c->vocab, logits);
    } else {
      double *sel = (double *)malloc(sizeof(double) * (size_t)(n_rows * D));
      for (int64_t i = 0; i < n_rows; ++i) memcpy(sel + i * D, xf + rows[i] * D, sizeof(double) * D);
      oracle_linear(sel, n_rows, D, lm_head, c->vocab, logits);
      free(sel);
    }
  }
  free(g); free(xf); free(x);
  return 0;
}

/* [T2 Optimize / Loss; T3 12]: the logsumexp form of -log softmax(logits_r)[t_r]. */
double oracle_cross_entropy(const double *logits, int64_t rows, int V, const int32_t *targets,
                            double *loss) {
  for (int64_t r = 0; r < rows; ++r)
    if (targets[r] >= V) return NAN;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    if (targets[r] < 0) {
      loss[r] = 0.0;
      continue;
    }
    const double *a = logits + r * (int64_t)V;
    double m = a[0];
    for (int j = 1; j < V; ++j) if (a[j] > m) m = a[j];
    double sum = 0.0;
    for (int j = 0; j < V; ++j) sum += exp(a[j] - m);
    loss[r] = log(sum) + m - a[targets[r]];
  }
  double total = 0.0;
  int64_t counted = 0;
  for (int64_t r = 0; r < rows; ++r)
    if (targets[r] >= 0) {
      total += loss[r];
      ++counted;
    }
  return counted ? total / (double)counted : 0.0;
}

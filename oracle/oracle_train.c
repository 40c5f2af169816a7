/* Plain fp64 CPU oracle of one training step's arithmetic: the gradients of the mean
 * next-token cross-entropy with respect to every parameter of the model, and the AdamW
 * update. Test infrastructure only, like oracle.c (see oracle.h).
 *
 * The gradients are the chain rule applied to the forward of oracle.c, written out step by
 * step in reverse order, with every parameter in double precision:
 *   [T2 Optimize / Loss]      loss = mean over rows with a target of logsumexp(z) - z[target]
 *   [T1 5.7; T3 10]           z = RMSNorm(x_L; g_f) W_lm^T, x_{l+1} = block(x_l), x_0 = E[ids]
 *   [T1 5.3-5.6; T2]          block: pre-norm attention (RoPE on q, k; causal softmax; grouped
 *                             KV heads) and pre-norm SwiGLU FFN, each added to the residual.
 * Nothing is blocked, fused or reordered; the attention keeps its full probability matrix. */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double *dalloc(size_t n) { return (double *)calloc(n ? n : 1, sizeof(double)); }

/* y = x W^T, W (n_out, n_in) in double. */
static void lin(const double *x, int64_t rows, int n_in, const double *W, int n_out, double *y) {
  for (int64_t r = 0; r < rows; ++r)
    for (int o = 0; o < n_out; ++o) {
      double acc = 0.0;
      for (int i = 0; i < n_in; ++i) acc += x[r * n_in + i] * W[(int64_t)o * n_in + i];
      y[r * n_out + o] = acc;
    }
}

/* Backward of y = x W^T: dx += dy W (if dx), dW += dy^T x. */
static void lin_back(const double *x, const double *dy, int64_t rows, int n_in, const double *W,
                     int n_out, double *dx, double *dW) {
  for (int64_t r = 0; r < rows; ++r)
    for (int o = 0; o < n_out; ++o) {
      const double g = dy[r * n_out + o];
      for (int i = 0; i < n_in; ++i) {
        if (dx) dx[r * n_in + i] += g * W[(int64_t)o * n_in + i];
        dW[(int64_t)o * n_in + i] += g * x[r * n_in + i];
      }
    }
}

/* RMSNorm forward; keeps 1/rms per row. */
static void rms_fwd(const double *x, int64_t rows, int d, const double *g, double eps, double *y,
                    double *rinv) {
  for (int64_t r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += x[r * d + i] * x[r * d + i];
    const double ri = 1.0 / sqrt(ss / d + eps);
    rinv[r] = ri;
    for (int i = 0; i < d; ++i) y[r * d + i] = x[r * d + i] * ri * g[i];
  }
}

/* Backward of y_i = x_i r g_i, r = (mean(x^2) + eps)^(-1/2):
 * dr/dx_j = -r^3 x_j / d, so dx_j += r g_j dy_j - x_j r^3 / d * sum_i dy_i g_i x_i;
 * dg_i += dy_i x_i r. */
static void rms_back(const double *x, const double *dy, int64_t rows, int d, const double *g,
                     const double *rinv, double *dx, double *dg) {
  for (int64_t r = 0; r < rows; ++r) {
    const double ri = rinv[r];
    double dot = 0.0;
    for (int i = 0; i < d; ++i) dot += dy[r * d + i] * g[i] * x[r * d + i];
    for (int j = 0; j < d; ++j) {
      dx[r * d + j] += ri * g[j] * dy[r * d + j] - x[r * d + j] * ri * ri * ri / d * dot;
      dg[j] += dy[r * d + j] * x[r * d + j] * ri;
    }
  }
}

/* Rotation of every head of rows (B*S, H*dh) by +angle (dir = 1) or -angle (dir = -1):
 * the backward of a rotation is the rotation by the opposite angle. */
static void rope_dir(double *x, int B, int S, int H, int dh, const int32_t *pos, double theta,
                     int dir) {
  for (int64_t r = 0; r < (int64_t)B * S; ++r) {
    const double p = pos ? (double)pos[r] : (double)(r % S);
    for (int h = 0; h < H; ++h) {
      double *v = x + r * (int64_t)H * dh + (int64_t)h * dh;
      for (int i = 0; i < dh / 2; ++i) {
        const double a = p * pow(theta, -2.0 * i / dh);
        const double c = cos(a), s = dir * sin(a);
        const double x0 = v[2 * i], x1 = v[2 * i + 1];
        v[2 * i] = x0 * c - x1 * s;
        v[2 * i + 1] = x0 * s + x1 * c;
      }
    }
  }
}

static double silu(double a) { return a / (1.0 + exp(-a)); }
static double silu_grad(double a) {   /* d/da a sigma(a) = sigma(a) (1 + a (1 - sigma(a))) */
  const double sg = 1.0 / (1.0 + exp(-a));
  return sg * (1.0 + a * (1.0 - sg));
}

typedef struct {   /* saved forward values of one layer */
  double *x, *h1, *r1, *q, *k, *v, *P, *o, *xm, *h2, *r2, *a, *c, *u;
} saved_layer;

double oracle_model_grads(const oracle_cfg *c, const oracle_params_d *p, const int32_t *ids,
                          const int32_t *pos, const int32_t *targets, int B, int S,
                          const oracle_params_d *g) {
  const int64_t M = (int64_t)B * S;
  const int D = c->d_model, F = c->d_ff, V = c->vocab, L = c->n_layers;
  const int Hq = c->n_heads, Hkv = c->n_kv_heads, dh = c->d_head, G = Hq / Hkv;
  const int qd = Hq * dh, kvd = Hkv * dh;
  const double scale = 1.0 / sqrt((double)dh);

  /* ---- forward, keeping what the backward needs */
  saved_layer *sv = (saved_layer *)calloc(L > 0 ? L : 1, sizeof(saved_layer));
  double *x = dalloc(M * D);
  for (int64_t r = 0; r < M; ++r) {
    if (ids[r] < 0 || ids[r] >= V) { free(x); free(sv); return NAN; }
    for (int j = 0; j < D; ++j) x[r * D + j] = p->embed[(int64_t)ids[r] * D + j];
  }
  for (int l = 0; l < L; ++l) {
    const oracle_layer_d *w = &p->layers[l];
    saved_layer *s = &sv[l];
    const int full = c->full_every > 0 && l % c->full_every == c->full_every - 1;
    const int window = full ? 0 : c->window;
    s->x = dalloc(M * D); memcpy(s->x, x, sizeof(double) * M * D);
    s->h1 = dalloc(M * D); s->r1 = dalloc(M);
    rms_fwd(x, M, D, w->g_attn, c->eps, s->h1, s->r1);
    s->q = dalloc(M * qd); s->k = dalloc(M * kvd); s->v = dalloc(M * kvd);
    lin(s->h1, M, D, w->wq, qd, s->q);
    lin(s->h1, M, D, w->wk, kvd, s->k);
    lin(s->h1, M, D, w->wv, kvd, s->v);
    rope_dir(s->q, B, S, Hq, dh, pos, c->theta, 1);
    rope_dir(s->k, B, S, Hkv, dh, pos, c->theta, 1);
    /* probabilities P[b][h][i][j] over the visible keys, zero elsewhere */
    s->P = dalloc((size_t)B * Hq * S * S);
    s->o = dalloc(M * qd);
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < Hq; ++h) {
        const int gk = h / G;
        for (int i = 0; i < S; ++i) {
          double *pr = s->P + (((int64_t)b * Hq + h) * S + i) * S;
          const int j0 = window > 0 && i - window + 1 > 0 ? i - window + 1 : 0;
          double mx = -INFINITY;
          for (int j = j0; j <= i; ++j) {
            double d = 0.0;
            for (int e = 0; e < dh; ++e)
              d += s->q[((int64_t)b * S + i) * qd + h * dh + e] *
                   s->k[((int64_t)b * S + j) * kvd + gk * dh + e];
            pr[j] = d * scale;
            if (pr[j] > mx) mx = pr[j];
          }
          double sum = 0.0;
          for (int j = j0; j <= i; ++j) { pr[j] = exp(pr[j] - mx); sum += pr[j]; }
          for (int j = j0; j <= i; ++j) pr[j] /= sum;
          for (int e = 0; e < dh; ++e) {
            double acc = 0.0;
            for (int j = j0; j <= i; ++j) acc += pr[j] * s->v[((int64_t)b * S + j) * kvd + gk * dh + e];
            s->o[((int64_t)b * S + i) * qd + h * dh + e] = acc;
          }
        }
      }
    double *t = dalloc(M * D);
    lin(s->o, M, qd, w->wo, D, t);
    for (int64_t i = 0; i < M * D; ++i) x[i] += t[i];
    free(t);
    s->xm = dalloc(M * D); memcpy(s->xm, x, sizeof(double) * M * D);
    s->h2 = dalloc(M * D); s->r2 = dalloc(M);
    rms_fwd(x, M, D, w->g_ffn, c->eps, s->h2, s->r2);
    s->a = dalloc(M * F); s->c = dalloc(M * F); s->u = dalloc(M * F);
    lin(s->h2, M, D, w->w1, F, s->a);
    lin(s->h2, M, D, w->w3, F, s->c);
    for (int64_t i = 0; i < M * F; ++i) s->u[i] = silu(s->a[i]) * s->c[i];
    t = dalloc(M * D);
    lin(s->u, M, F, w->w2, D, t);
    for (int64_t i = 0; i < M * D; ++i) x[i] += t[i];
    free(t);
  }
  double *xf = dalloc(M * D), *rf = dalloc(M);
  rms_fwd(x, M, D, p->g_final, c->eps, xf, rf);
  double *z = dalloc(M * V);
  lin(xf, M, D, p->lm_head, V, z);

  /* ---- loss and d loss / d logits: (softmax - onehot) / N for rows with a target */
  int64_t n_valid = 0;
  for (int64_t r = 0; r < M; ++r) n_valid += targets[r] >= 0 && targets[r] < V;
  double loss = 0.0;
  double *dz = dalloc(M * V);
  for (int64_t r = 0; r < M; ++r) {
    const int t = targets[r];
    if (t < 0 || t >= V) continue;
    const double *zr = z + r * V;
    double mx = zr[0];
    for (int j = 1; j < V; ++j) if (zr[j] > mx) mx = zr[j];
    double se = 0.0;
    for (int j = 0; j < V; ++j) se += exp(zr[j] - mx);
    loss += log(se) + mx - zr[t];
    for (int j = 0; j < V; ++j) dz[r * V + j] = exp(zr[j] - mx) / se / (double)n_valid;
    dz[r * V + t] -= 1.0 / (double)n_valid;
  }
  loss = n_valid ? loss / (double)n_valid : 0.0;

  /* ---- backward */
  double *dxf = dalloc(M * D);
  lin_back(xf, dz, M, D, p->lm_head, V, dxf, g->lm_head);
  double *dx = dalloc(M * D);
  rms_back(x, dxf, M, D, p->g_final, rf, dx, g->g_final);
  for (int l = L - 1; l >= 0; --l) {
    const oracle_layer_d *w = &p->layers[l];
    const oracle_layer_d *gw = &g->layers[l];
    saved_layer *s = &sv[l];
    /* FFN: x_{l+1} = xm + u W2^T, u = silu(a) * c, a = h2 W1^T, c = h2 W3^T */
    double *du = dalloc(M * F);
    lin_back(s->u, dx, M, F, w->w2, D, du, gw->w2);
    double *da = dalloc(M * F), *dc = dalloc(M * F);
    for (int64_t i = 0; i < M * F; ++i) {
      da[i] = du[i] * s->c[i] * silu_grad(s->a[i]);
      dc[i] = du[i] * silu(s->a[i]);
    }
    double *dh2 = dalloc(M * D);
    lin_back(s->h2, da, M, D, w->w1, F, dh2, gw->w1);
    lin_back(s->h2, dc, M, D, w->w3, F, dh2, gw->w3);
    rms_back(s->xm, dh2, M, D, w->g_ffn, s->r2, dx, gw->g_ffn);   /* dx is now d xm */
    /* attention: xm = x + o Wo^T */
    double *dout = dalloc(M * qd);
    lin_back(s->o, dx, M, qd, w->wo, D, dout, gw->wo);
    double *dq = dalloc(M * qd), *dk = dalloc(M * kvd), *dv = dalloc(M * kvd);
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < Hq; ++h) {
        const int gk = h / G;
        for (int i = 0; i < S; ++i) {
          const double *pr = s->P + (((int64_t)b * Hq + h) * S + i) * S;
          const double *doi = dout + ((int64_t)b * S + i) * qd + h * dh;
          /* dP_ij = do_i . v_j; dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik) */
          double *dP = dalloc(S);
          double rs = 0.0;
          for (int j = 0; j <= i; ++j) {
            if (pr[j] == 0.0) continue;
            double d = 0.0;
            for (int e = 0; e < dh; ++e) d += doi[e] * s->v[((int64_t)b * S + j) * kvd + gk * dh + e];
            dP[j] = d;
            rs += pr[j] * d;
          }
          for (int j = 0; j <= i; ++j) {
            if (pr[j] == 0.0) continue;
            const double ds = pr[j] * (dP[j] - rs) * scale;
            for (int e = 0; e < dh; ++e) {
              dq[((int64_t)b * S + i) * qd + h * dh + e] += ds * s->k[((int64_t)b * S + j) * kvd + gk * dh + e];
              dk[((int64_t)b * S + j) * kvd + gk * dh + e] += ds * s->q[((int64_t)b * S + i) * qd + h * dh + e];
              dv[((int64_t)b * S + j) * kvd + gk * dh + e] += pr[j] * doi[e];
            }
          }
          free(dP);
        }
      }
    rope_dir(dq, B, S, Hq, dh, pos, c->theta, -1);   /* back through the rotations */
    rope_dir(dk, B, S, Hkv, dh, pos, c->theta, -1);
    double *dh1 = dalloc(M * D);
    lin_back(s->h1, dq, M, D, w->wq, qd, dh1, gw->wq);
    lin_back(s->h1, dk, M, D, w->wk, kvd, dh1, gw->wk);
    lin_back(s->h1, dv, M, D, w->wv, kvd, dh1, gw->wv);
    rms_back(s->x, dh1, M, D, w->g_attn, s->r1, dx, gw->g_attn);   /* dx is now d x_l */
    free(du); free(da); free(dc); free(dh2); free(dout); free(dq); free(dk); free(dv); free(dh1);
  }
  for (int64_t r = 0; r < M; ++r)
    for (int j = 0; j < D; ++j) g->embed[(int64_t)ids[r] * D + j] += dx[r * D + j];

  for (int l = 0; l < L; ++l) {
    saved_layer *s = &sv[l];
    free(s->x); free(s->h1); free(s->r1); free(s->q); free(s->k); free(s->v); free(s->P);
    free(s->o); free(s->xm); free(s->h2); free(s->r2); free(s->a); free(s->c); free(s->u);
  }
  free(sv); free(x); free(xf); free(rf); free(z); free(dz); free(dxf); free(dx);
  return loss;
}

/* [T2 Optimizer - AdamW]: m = b1 m + (1 - b1) g; v = b2 v + (1 - b2) g^2;
 * theta <- theta - lr m_hat / (sqrt(v_hat) + eps) - lr wd theta_prev, with the bias
 * corrections m_hat = m / (1 - b1^t), v_hat = v / (1 - b2^t) and the decay taken on the
 * parameter before this step. */
void oracle_adamw(double *theta, const double *grad, double *m, double *v, int64_t n, double lr,
                  double b1, double b2, double eps, double wd, int t) {
  const double c1 = 1.0 - pow(b1, t), c2 = 1.0 - pow(b2, t);
  for (int64_t i = 0; i < n; ++i) {
    m[i] = b1 * m[i] + (1.0 - b1) * grad[i];
    v[i] = b2 * v[i] + (1.0 - b2) * grad[i] * grad[i];
    const double mh = m[i] / c1, vh = v[i] / c2;
    theta[i] = theta[i] - lr * mh / (sqrt(vh) + eps) - lr * wd * theta[i];
  }
}

// Host-side launch interface between the C ABI layer (api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tfm {

enum DType { DT_F32 = 0, DT_BF16 = 1 };

// ---- elementwise / normalisation kernels (elementwise.hip)
hipError_t launch_rope_table(float *cos_sin, int max_seq, int d_head, double theta,
                             hipStream_t s);
hipError_t launch_embed(const int32_t *ids, int64_t n, const void *table, int table_dt,
                        int vocab, int d, float *x, int32_t *err_flag, hipStream_t s);
// embedding into x and y = RMSNorm(x; g) in one pass; table, g and y of dtype dt
hipError_t launch_embed_rmsnorm(const int32_t *ids, int64_t n, const void *table, int dt,
                                int vocab, int d, float *x, int32_t *err_flag, const void *g,
                                void *y, float eps, hipStream_t s);
// matrix-core rate probe: blocks x 4 waves x iters x 8 MFMAs of 16x16x32; sink: blocks x 4
hipError_t launch_mfma_rate(int64_t iters, int blocks, float *sink, hipStream_t s);
hipError_t launch_rmsnorm(const void *x, int x_dt, const void *g, int g_dt, void *y, int y_dt,
                          int64_t rows, int d, float eps, hipStream_t s);
hipError_t launch_rope(void *x, int x_dt, int64_t row_stride, const int32_t *positions, int B,
                       int S, int H, int d_head, const float *cos_sin, int max_seq,
                       hipStream_t s);
hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s);
// Next-token cross-entropy from the LM-head tile partials: loss[m] = max_m + log(sum_m) -
// tgt[m] with max_m, sum_m combined over the T column tiles in a fixed order; negative
// targets give 0, targets >= V give NaN. mean (optional) = mean over rows with target >= 0.
// lse (M), when not null, receives each row's log-sum-exp; with oob_zero a target >= V gives
// a zero loss (the training convention) instead of NaN.
hipError_t launch_xent_reduce(const float *x_max, const float *x_sum, const float *x_tgt,
                              const int32_t *targets, int T, int64_t M, int V, float *loss,
                              float *mean, hipStream_t s, float *lse = nullptr,
                              bool oob_zero = false);

// ---- GEMM family (gemm.hip): y = a w^T with a fused epilogue.
enum GemmEpi {
  EPI_STORE = 0,     // y = acc (y_dt)
  EPI_RESIDUAL = 1,  // y = residual + acc (float32)
  EPI_QKV_ROPE = 2,  // weight rows from wq | wk | wv; RoPE on the q and k columns
  EPI_SWIGLU = 3,    // gate rows from w1, up rows from w3; y = SiLU(gate) * up
  EPI_XENT = 4,      // no y: per row and column tile, max and sum of exp of the tile's
                     // logits, plus the logit of the row's target column (bf16 only)
  EPI_QKV_CACHE = 5, // decode only: q -> y with RoPE; k (RoPE) and v -> KV cache slot
  EPI_XENT_GRAD = 6, // bf16 only: the logits recomputed and turned into the cross-entropy
                     // gradient y = (exp(z - lse[m]) - [n == t_m]) / count for rows with a
                     // target in [0, N), 0 elsewhere; columns [N, n0) are stored as zeros
  EPI_SWIGLU_BACK = 7// bf16 only: acc is du, the gradient of u = SiLU(a) c; with the forward's a
                     // and c in keep_a / keep_c ((M, N), row stride N) it stores
                     // da = du c s (1 + a (1 - s)), s = sigmoid(a), at y[m ldy + n] and
                     // dc = du a s at y[m ldy + N + n] (ldy >= 2 N; N, ldy multiples of 4)
};

struct GemmArgs {
  const void *a;           // (M, K) activations of dt, row stride lda
  int64_t lda;
  const void *w0, *w1, *w2;// weight row sources (see GemmEpi)
  int n0, n1;              // QKV: rows of wq and of wk (= rows of wv); SwiGLU: d_ff
  int64_t M;
  int N;                   // output columns (QKV: n0 + 2 n1; SwiGLU: d_ff)
  int K;
  int64_t ldw;             // row stride of the weight rows in elements (0: K)
  // split K (EPI_STORE): part q = blockIdx.y of kparts > 1 multiplies k in
  // [q kpart, (q + 1) kpart) and stores at y + q ypart elements
  int kparts, kpart;
  int64_t ypart;
  void *y;
  int64_t ldy;
  int y_dt;
  const float *residual;   // EPI_RESIDUAL
  const int32_t *positions;// EPI_QKV_ROPE: (M) or NULL -> row % S
  const float *cos_sin;
  int S, d_head, max_seq;
  // EPI_XENT: targets (M); partials x_max / x_sum laid out [tile_n][M]; x_tgt (M)
  const int32_t *targets;
  float *x_max, *x_sum, *x_tgt;
  // RMSNorm split across two products ("Transformer 篇" 5.6: RMSNorm(x) W^T =
  // (1/rms(x)) ((x * g) W^T), the per-row factor commutes with the product).
  // EPI_RESIDUAL with nrm_y (bf16 only): besides x it writes nrm_y = bf16(x * nrm_g) (row
  // stride ldy) and the sum of squares of the tile's columns of x, row m, column tile t, into
  // nrm_part[kNormParts m + t] (at most kNormParts column tiles: N <= gemm_norm_max_cols()).
  const void *nrm_g;
  void *nrm_y;
  float *nrm_part;
  // EPI_QKV_ROPE / EPI_SWIGLU with rs_part (bf16 only): the activations a are bf16(x * g);
  // every output row m is scaled by 1 / sqrt(sum_{t < rs_parts} rs_part[kNormParts m + t] / rs_d
  // + rs_eps)
  // in fp32 before the rest of the epilogue.
  const float *rs_part;
  int rs_parts, rs_d;
  float rs_eps;
  // EPI_SWIGLU (bf16): also keep the gate and up values (bf16, same layout as y) for the
  // backward, when not null
  void *keep_a, *keep_c;
  // EPI_XENT_GRAD: each row's log-sum-exp (M) and the number of rows with a target (one int);
  // the targets come in `targets`
  const float *xg_lse;
  const int32_t *xg_count;
};

constexpr int kNormParts = 16;  // column tiles whose row partials one row of nrm_part holds
// Column tiles of the bf16 residual product over N columns, and the largest N whose row
// partials fit in nrm_part.
int gemm_residual_col_tiles(int N);
int gemm_norm_max_cols();

// Column tiles (partials per row) of the EPI_XENT GEMM for N = vocab columns.
int gemm_xent_parts(int N);

hipError_t launch_gemm(int epi, int dt, const GemmArgs &g, hipStream_t s);
// y (M, N) = sum over k of a[k lda + m] w0[k ldw + n] (bf16, both operands K-major: the
// weight-gradient products over tokens read the row-major activations as they are), fp32 or
// bf16 output, split K like launch_gemm (kparts / kpart / ypart). g.ldw must be set.
hipError_t launch_gemm_kmajor(const GemmArgs &g, hipStream_t s);
// whether launch_gemm_kmajor takes these operands (alignment, strides, 32-bit offsets)
bool gemm_kmajor_ok(const void *a, int64_t lda, const void *w, int64_t ldw, int64_t M, int N,
                    int64_t K);
// Up to kWgradJobs K-major products over the same K in one launch, unsplit, fp32 output:
// job j writes y[m ldy + n] = sum over k < K of a[k lda + m] b[k ldb + n], m < M, n < N.
// Every job must pass gemm_kmajor_ok; start[] is filled by the launcher.
constexpr int kWgradJobs = 8;
struct WgradJob {
  const void *a, *b;
  float *y;
  int64_t lda, ldb, ldy;
  int M, N;
};
struct WgradGroup {
  WgradJob job[kWgradJobs];
  int start[kWgradJobs + 1];
  int njobs, K;
};
hipError_t launch_gemm_wgrad_group(const WgradGroup &grp, hipStream_t s);
// Workgroups of a plain-store GEMM of M x N outputs.
int64_t gemm_store_tiles(int dt, int64_t M, int N);

// ---- attention (attention.hip)
// window > 0: query s sees keys s - window + 1 .. s only (window >= S or 0: full causal).
// lse (nullable): (B*S, Hq) fp32, each query row's logsumexp of its scaled scores.
hipError_t launch_attention(const void *q, int64_t q_stride, const void *k, const void *v,
                            int64_t kv_stride, void *o, int64_t o_stride, int B, int S, int Hq,
                            int Hkv, int d_head, int dt, int window, hipStream_t s,
                            float *lse = nullptr);
bool attention_supported(int dt, int d_head);
// Compute units of the current device (cached per device), for work orders over rounds of
// one workgroup per CU.
int compute_units();
// ---- incremental decoding (decode.hip), bf16 only
struct DecodeGemmArgs {
  const void *x;            // (M, K) activations, row stride ldx
  int64_t ldx;
  const void *w0, *w1, *w2; // weight rows: plain w0; QKV wq | wk | wv; SwiGLU w1 (gate), w3 (up)
  int n0, n1;               // QKV: rows of wq and of wk; SwiGLU: d_ff
  int M, N, K;
  void *y;                  // STORE: (M, ldy) y_dt; RESIDUAL: fp32 in place; SwiGLU: u bf16;
  int64_t ldy;              // QKV: rotated q (M, ldy) bf16
  int y_dt;
  const int32_t *positions; // QKV: position (= cache slot) of row m's token
  const float *cos_sin;
  int d_head, max_seq;
  void *k_cache, *v_cache;  // QKV: this layer's (B, Hkv, cache_seq, d_head) blocks
  int cache_seq, n_kv_heads;
  int32_t *pos_flag;        // set to 1 when a position is outside [0, min(cache_seq, max_seq))
  // Optional fused RMSNorm: when norm_x is set, the activations are RMSNorm(norm_x; norm_g)
  // (fp32 rows of K elements, row stride ldx; gain bf16), rounded to bf16, and x is unused.
  const float *norm_x;
  const void *norm_g;
  float eps;
};
hipError_t launch_decode_gemm(int epi, const DecodeGemmArgs &g, hipStream_t s);
// Partial records per (sequence, query head): decode_chunks(cache_seq), each 2 + d_head floats.
int decode_chunks(int cache_seq);
int decode_max_cache();   // largest cache_seq the chunk merge supports
bool decode_group_supported(int Hq, int Hkv);
// o[b, h] = attention of q[b, h] over cache slots of sequence b up to positions[b] (the last
// `window` of them when window > 0); part: B * Hq * decode_chunks * (2 + d_head) floats.
hipError_t launch_decode_attention(const void *q, int64_t q_stride, const void *k_cache,
                                   const void *v_cache, const int32_t *positions, int B, int Hq,
                                   int Hkv, int d_head, int cache_seq, int window, float *part,
                                   void *o, int64_t o_stride, hipStream_t s);
// Size of the static device scratch of the allocation-free decode attention entry point, and
// its device address on the GPU that runs `stream` (looked up once per device with
// hipGetSymbolAddress, never allocated).
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
hipError_t noalloc_scratch(hipStream_t stream, float **ptr);
// Copies the k and v columns of B*S qkv rows into the cache slots positions[r] (or r % S).
hipError_t launch_kv_store(const void *qkv, int64_t ld, int qd, int kvd, int d_head, int Hkv,
                           int B, int S, const int32_t *positions, void *k_cache, void *v_cache,
                           int cache_seq, int32_t *pos_flag, hipStream_t s);

// ---- training step (backward.hip)
// dst[c, r] = src[r, c] for an R x C source (row strides lds, ldd), converting the dtype;
// source rows in [R_valid, R) read as zero.
hipError_t launch_transpose(const void *src, int src_dt, int64_t lds, void *dst, int dst_dt,
                            int64_t ldd, int64_t R, int64_t R_valid, int C, hipStream_t s);
hipError_t launch_convert(const void *src, int src_dt, void *dst, int dst_dt, int64_t n,
                          hipStream_t s);
// Up to kTransposeJobs bf16 transposes dst[c ldd + r] = src[r lds + c] (r < R, c < C) in one
// launch; a job whose strides, sizes or pointers do not allow 16-byte accesses (or one past
// the limit) gets a launch of its own.
constexpr int kTransposeJobs = 8;
struct TransposeJob {
  const void *src;
  void *dst;
  int64_t lds, ldd, R, C;
};
hipError_t launch_transpose_multi(const TransposeJob *jobs, int n, hipStream_t s);
hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t s);
// dz = d mean-loss / d z for fp32 logits z (M, ldz), written (M, ldd) with zero padding past
// V; row_loss (M); count = rows with a target in [0, V); mean = mean loss over them.
hipError_t launch_ce_backward(const float *z, int64_t ldz, const int32_t *targets, int64_t M,
                              int V, void *dz, int dz_dt, int64_t ldd, float *row_loss,
                              int32_t *count, float *mean, hipStream_t s);
// count[0] = rows with a target in [0, V); mean[0] = sum of row_loss / count[0] (fp64, fixed
// order; 0 without targets)
hipError_t launch_count_targets(const int32_t *targets, int64_t M, int V, int32_t *count,
                                hipStream_t s);
hipError_t launch_mean_rows(const float *row_loss, int64_t M, const int32_t *count, float *mean,
                            hipStream_t s);
// dx += RMSNorm backward of rows x with gain g (d <= 2048); dg = (or +=) gain gradient.
// dg_part: rms_back_parts(rows) * d floats of scratch.
int rms_back_parts(int64_t rows);
hipError_t launch_rms_backward(const float *x, const void *g, int g_dt, const float *dy, float *dx,
                               void *dx_bf16, float *dg, int accumulate_dg, float *dg_part,
                               int64_t rows, int d, float eps, hipStream_t s);
hipError_t launch_swiglu_fwd(const void *a, const void *c, void *u, int dt, int64_t n,
                             hipStream_t s);
hipError_t launch_swiglu_backward(const void *a, const void *c, const float *du, void *da,
                                  void *dc, int dt, int64_t n, hipStream_t s);
hipError_t launch_rope_inverse(void *x, int dt, int64_t row_stride, const int32_t *positions,
                               int64_t rows, int S, int H, int d_head, const float *cos_sin,
                               int max_seq, hipStream_t s);
bool attention_backward_supported(int d_head);
// dq, dk, dv into the q | k | v columns of dqkv (same layout as qkv); lse: (B*S, Hq) row
// logsumexp kept by the forward (launch_attention's lse); dsum: (B*S, Hq) fp32 scratch.
// With cos_sin, dq and dk are then rotated back by their rows' positions (the backward of
// the forward's RoPE; positions NULL -> row % S; a position outside [0, max_seq) is left
// unrotated).
hipError_t launch_attention_backward(const void *qkv, int64_t ld, const void *o, int64_t ldo,
                                     const void *dout, int64_t lddo, void *dqkv, int B, int S,
                                     int Hq, int Hkv, int d_head, int dt, int window,
                                     const float *lse, float *dsum, const int32_t *positions,
                                     const float *cos_sin, int max_seq, hipStream_t s);
// The bf16 path of launch_attention_backward (attn_back.hip): d_head 32, 64 or 128; the
// rotation is applied to the gradients before they are stored.
hipError_t launch_attention_backward_bf16(const void *qkv, int64_t ld, const void *o,
                                          int64_t ldo, const void *dout, int64_t lddo,
                                          void *dqkv, int B, int S, int Hq, int Hkv, int d_head,
                                          int window, const float *lse, float *dsum,
                                          const int32_t *positions, const float *cos_sin,
                                          int max_seq, hipStream_t s);
// The sum-of-squares partials of `count` tensors (host arrays of device pointers and sizes),
// tensor t at part + t * sumsq_parts(), in launches of up to 32 tensors.
hipError_t launch_sumsq_multi(const float *const *g, const int64_t *n, int count, double *part,
                              hipStream_t s);
// AdamW over `count` tensors (host arrays; pb nullable, or entries nullable), batched.
hipError_t launch_adamw_multi(float *const *p, void *const *pb, const float *const *g,
                              float *const *m, float *const *v, const int64_t *n, int count,
                              float lr, float b1, float b2, float eps, float wd, float c1,
                              float c2, const float *coef, hipStream_t s);
// y[m, n] = sum over p < parts of part[p][m, n] (part: parts x M x N fp32, summed in order p).
hipError_t launch_sum_parts(const float *part, int parts, int64_t M, int N, float *y,
                            int64_t ldy, hipStream_t s);
hipError_t launch_embed_backward(const int32_t *ids, int64_t n, int vocab, int d, const float *dx,
                                 float *dE, hipStream_t s);
int sumsq_parts();
hipError_t launch_sumsq(const float *g, int64_t n, double *part, hipStream_t s);
hipError_t launch_clip_coef(const double *part, int nparts, float max_norm, float *coef,
                            float *norm, hipStream_t s);
hipError_t launch_adamw(float *p, void *pb, const float *g, float *m, float *v, int64_t n,
                        float lr, float b1, float b2, float eps, float wd, float c1, float c2,
                        const float *coef, hipStream_t s);

// Whether one sequence's keys fit the bf16 kernel's 32-bit buffer offsets.
bool attention_fits(int dt, int S, int64_t kv_stride);

}  // namespace tfm

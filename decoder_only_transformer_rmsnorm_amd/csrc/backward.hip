// Backward pass and optimizer kernels of one training step ("LLM 2: Transformer 原理与实现",
// Optimize: Loss, AdamW, Gradient Clip; the chain rule through the forward of
// "Transformer 篇" (dujian.net) 5.3-5.7).
//
// The matrix products of the backward run on the forward's GEMM kernels (y = a w^T): with
// W (out, in) and a forward y = x W^T, the input gradient is dy W = dy (W^T)^T and the
// weight gradient is dy^T x = (dy^T) (x^T)^T, so the weights and the activations are first
// transposed by transpose_kernel. Everything else is here:
//  * ce_back_kernel: d loss / d logits = (softmax(z) - onehot(target)) / N per row with a
//    target, plus each row's loss (logsumexp form);
//  * rms_back_kernel: RMSNorm backward, dx += r g dy - x r^3 / d (dy . g x), with the gain
//    gradient summed per workgroup and the partials summed in a fixed order;
//  * swiglu_fwd_kernel / swiglu_back_kernel: u = SiLU(a) c and (da, dc);
//  * rope_inv_kernel: the backward of a rotation is the rotation by the opposite angle;
//  * attention backward of fp32 models, flash style in fp32 vector arithmetic: with each query
//    row's logsumexp kept by the forward, attn_dq_kernel accumulates
//    dq = sum_j P (dP - D) k / sqrt(dh) with D = rowsum(do * o); attn_dkdv_kernel accumulates
//    dk and dv per key over the queries (and query heads of a group) that see it. The score
//    matrix is never stored. bf16 models use the matrix-core kernels of attn_back.hip.
//  * embed_back_kernel: scatter-add of the input gradient into the embedding rows;
//  * sumsq / clip_coef / adamw: the global-norm clipping coefficient and the AdamW update.
#include <cmath>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace tfm {
namespace {

inline unsigned nblk(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

template <typename T> __device__ __forceinline__ float ld1(const T *p);
template <> __device__ __forceinline__ float ld1<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float ld1<bf16_t>(const bf16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void st1(float *p, float v) { *p = v; }
__device__ __forceinline__ void st1(bf16_t *p, float v) { *p = f32_to_bf16(v); }

// ---- transpose (with conversion): dst[c, r] = src[r, c]
// Source rows in [R_valid, R) read as zero (zero padding of the destination's rows).
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void transpose_kernel(const TI *__restrict__ src, int64_t lds,
                                                        TO *__restrict__ dst, int64_t ldd,
                                                        int64_t R, int64_t R_valid, int C) {
  __shared__ float tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i;
    const int c = c0 + tx;
    tile[i][tx] = r < R_valid && c < C ? ld1(src + r * lds + c) : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i;
    const int64_t r = r0 + tx;
    if (c < C && r < R) st1(dst + (int64_t)c * ldd + r, tile[tx][i]);
  }
}

// bf16 -> bf16 transpose with 16-byte global accesses (every dimension and stride a multiple
// of 8 elements): a 64 x 64 tile, each thread reads 8 consecutive elements of a source row
// (two rows per thread) into LDS (pitch 66 elements, so the 8 threads that later read one
// column segment hit distinct banks) and writes 8 consecutive elements of a destination row.
__device__ __forceinline__ void transpose_bf16_tile(const uint16_t *__restrict__ src, int64_t lds,
                                                    uint16_t *__restrict__ dst, int64_t ldd,
                                                    int64_t R, int64_t R_valid, int C,
                                                    int64_t r0, int c0) {
  constexpr int P = 66;
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * P];
  const int tid = threadIdx.x, g8 = tid & 7, row = tid >> 3;
#pragma unroll
  for (int ps = 0; ps < 2; ++ps) {
    const int i = row + 32 * ps;
    const int64_t r = r0 + i;
    const int c = c0 + 8 * g8;
    uint4 v = {0u, 0u, 0u, 0u};
    if (r < R_valid && c < C) v = *(const uint4 *)(src + r * lds + c);
    uint32_t *t = (uint32_t *)(tile + i * P + 8 * g8);
    t[0] = v.x; t[1] = v.y; t[2] = v.z; t[3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int ps = 0; ps < 2; ++ps) {
    const int oc = row + 32 * ps;
    const int c = c0 + oc;
    const int64_t r = r0 + 8 * g8;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (uint32_t)tile[(8 * g8 + 2 * k) * P + oc] |
             ((uint32_t)tile[(8 * g8 + 2 * k + 1) * P + oc] << 16);
    if (c < C && r < R) *(uint4 *)(dst + (int64_t)c * ldd + r) = uint4{w[0], w[1], w[2], w[3]};
  }
}

__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t *__restrict__ src,
                                                             int64_t lds,
                                                             uint16_t *__restrict__ dst,
                                                             int64_t ldd, int64_t R,
                                                             int64_t R_valid, int C) {
  transpose_bf16_tile(src, lds, dst, ldd, R, R_valid, C, (int64_t)blockIdx.y * 64,
                      blockIdx.x * 64);
}

// Several bf16 transposes in one launch (a layer's weights before its backward): workgroups
// [start[j], start[j + 1]) take the 64 x 64 tiles of job j, row-major over its tile grid.
struct TransposeBatch {
  TransposeJob job[kTransposeJobs];
  int start[kTransposeJobs + 1];
  int n;
};
__global__ __launch_bounds__(256) void transpose_bf16_multi_kernel(TransposeBatch b) {
  const int bid = blockIdx.x;
  int j = 0;
#pragma unroll
  for (int i = 1; i < kTransposeJobs; ++i)
    if (i < b.n && bid >= b.start[i]) j = i;
  const TransposeJob &t = b.job[j];
  const int tc = (t.C + 63) / 64, in = bid - b.start[j];
  transpose_bf16_tile((const uint16_t *)t.src, t.lds, (uint16_t *)t.dst, t.ldd, t.R, t.R, t.C,
                      (int64_t)(in / tc) * 64, (in % tc) * 64);
}

template <typename TI, typename TO>
__global__ void convert_kernel(const TI *__restrict__ src, TO *__restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) st1(dst + i, ld1(src + i));
}

__global__ void fill_f32_kernel(float *p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---- cross-entropy ("LLM 2" Optimize / Loss)
__global__ __launch_bounds__(1024) void count_targets_kernel(const int32_t *t, int64_t M, int V,
                                                             int32_t *count) {
  __shared__ int part[1024];
  int c = 0;
  for (int64_t i = threadIdx.x; i < M; i += 1024) c += t[i] >= 0 && t[i] < V;
  part[threadIdx.x] = c;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) count[0] = part[0];
}

__device__ __forceinline__ float block_max(float v, float *red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ __forceinline__ float block_sum(float v, float *red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < nw; ++i) r += red[i];
  return r;
}

// one workgroup per row: dz[j] = (exp(z_j - lse) - [j == t]) / N for j < V, 0 in [V, ldd).
// Rows are read 16 bytes per lane when the row stride allows it, in two passes: the first
// forms each thread's sum of exp against its own reference maximum (moved only when a value
// exceeds it by more than 8 in log2 units, so the sum is rescaled rarely and stays below 2^8
// per term), the threads' (reference, sum) pairs are combined against the row maximum, and
// the second pass writes the gradient. Exponentials use the hardware exp2 (about 1 ulp, far
// below the bf16 rounding of the stored gradient), the loss itself logf.
template <typename TO>
__global__ __launch_bounds__(256) void ce_back_kernel(const float *__restrict__ z, int64_t ldz,
                                                      const int32_t *__restrict__ targets, int V,
                                                      const int32_t *__restrict__ n_valid,
                                                      TO *__restrict__ dz, int64_t ldd,
                                                      float *__restrict__ row_loss) {
  __shared__ float red[4];
  constexpr float kLog2e = 1.4426950408889634f;
  const int64_t m = blockIdx.x;
  const float *zr = z + m * ldz;
  TO *dr = dz + m * ldd;
  const int t = targets[m];
  const int tid = threadIdx.x;
  if (t < 0 || t >= V) {
    for (int64_t j = tid; j < ldd; j += 256) st1(dr + j, 0.f);
    if (tid == 0) row_loss[m] = 0.f;
    return;
  }
  // 16-byte groups [0, nv) when rows start 16-byte aligned, scalar columns [4 nv, V) after
  const int nv = (ldz & 3) == 0 ? V >> 2 : 0;
  float ref = -__builtin_inff(), sum = 0.f;   // this thread's reference (log2 units) and sum
  auto add = [&](float zv) {
    const float y = zv * kLog2e;
    if (y > ref + 8.f) {   // rare after the first values: move the reference up to y
      sum *= __builtin_amdgcn_exp2f(ref - y);   // 0 while ref is still -inf
      ref = y;
    }
    sum += __builtin_amdgcn_exp2f(y - ref);
  };
  for (int j = tid; j < nv; j += 256) {
    const f32x4_t v = *(const f32x4_t *)(zr + 4 * j);
    add(v[0]); add(v[1]); add(v[2]); add(v[3]);
  }
  for (int j = 4 * nv + tid; j < V; j += 256) add(zr[j]);
  const float mref = block_max(ref, red);   // the row maximum is within 8 of it
  float se = ref == -__builtin_inff() ? 0.f : sum * __builtin_amdgcn_exp2f(ref - mref);
  se = block_sum(se, red);
  const float lc = mref + log2f(se);        // log-sum-exp in log2 units
  const float lse = lc * 0.6931471805599453f;
  const float inv_n = 1.0f / (float)n_valid[0];
  // vector stores need 4 consecutive outputs 4-aligned in the output row as well
  const int nvo = ((ldd & 3) == 0) ? nv : 0;
  for (int j = tid; j < nvo; j += 256) {
    const f32x4_t v = *(const f32x4_t *)(zr + 4 * j);
    f32x4_t d;
#pragma unroll
    for (int x = 0; x < 4; ++x)
      d[x] = (__builtin_amdgcn_exp2f(__builtin_fmaf(v[x], kLog2e, -lc)) -
              (4 * j + x == t ? 1.f : 0.f)) * inv_n;
    store4(dr + 4 * j, d);
  }
  for (int64_t j = 4 * (int64_t)nvo + tid; j < ldd; j += 256) {
    float d = 0.f;
    if (j < V)
      d = (__builtin_amdgcn_exp2f(__builtin_fmaf(zr[j], kLog2e, -lc)) - (j == t ? 1.f : 0.f)) *
          inv_n;
    st1(dr + j, d);
  }
  if (tid == 0) row_loss[m] = lse - zr[t];
}

// mean of the row losses over the counted rows (fp64, fixed order)
__global__ __launch_bounds__(1024) void mean_rows_kernel(const float *row_loss, int64_t M,
                                                         const int32_t *n_valid, float *mean) {
  __shared__ double part[1024];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < M; i += 1024) s += (double)row_loss[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) mean[0] = n_valid[0] > 0 ? (float)(part[0] / n_valid[0]) : 0.f;
}

// ---- RMSNorm backward ("Transformer 篇" 5.6): one wave per row, 4 waves x kRows rows per
// workgroup; lane holds the 4-column groups lane + 64 i.
constexpr int kRmsRows = 4;   // rows per wave
template <int VPT, typename TG>
__global__ __launch_bounds__(256) void rms_back_kernel(const float *__restrict__ x,
                                                       const TG *__restrict__ g,
                                                       const float *__restrict__ dy,
                                                       float *__restrict__ dx,
                                                       bf16_t *__restrict__ dxb,
                                                       float *__restrict__ dg_part, int64_t rows,
                                                       int d, float eps) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ng = d >> 2;
  f32x4_t gacc[VPT], gv[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    gacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int gi = lane + 64 * i;
    gv[i] = gi < ng ? load4(g + 4 * gi) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int k = 0; k < kRmsRows; ++k) {
    const int64_t r = ((int64_t)blockIdx.x * 4 + w) * kRmsRows + k;
    if (r >= rows) break;
    f32x4_t xv[VPT], dv[VPT], ov[VPT];
    float ss = 0.f, dot = 0.f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {   // x, dy and the dx being accumulated, all issued first
      const int gi = lane + 64 * i;
      if (gi < ng) {
        xv[i] = load4(x + r * d + 4 * gi);
        dv[i] = load4(dy + r * d + 4 * gi);
        ov[i] = load4(dx + r * d + 4 * gi);
      } else {
        xv[i] = dv[i] = ov[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const f32x4_t t = dv[i] * gv[i] * xv[i];
      ss += xv[i][0] * xv[i][0] + xv[i][1] * xv[i][1] + xv[i][2] * xv[i][2] + xv[i][3] * xv[i][3];
      dot += t[0] + t[1] + t[2] + t[3];
    }
    ss = wave_sum(ss);
    dot = wave_sum(dot);
    const float ri = rsqrtf(ss / (float)d + eps);
    const float c3 = ri * ri * ri / (float)d * dot;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int gi = lane + 64 * i;
      if (gi < ng) {
        const f32x4_t nv = ov[i] + ri * gv[i] * dv[i] - xv[i] * c3;
        store4(dx + r * d + 4 * gi, nv);
        if (dxb) store4(dxb + r * d + 4 * gi, nv);   // the bf16 operand of the next products
        gacc[i] += dv[i] * xv[i] * ri;
      }
    }
  }
  // gain gradient: the 4 waves' sums meet in LDS, one partial row per workgroup
  __shared__ __attribute__((aligned(16))) float red[4][2048];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int gi = lane + 64 * i;
    if (gi < ng) *(f32x4_t *)&red[w][4 * gi] = gacc[i];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += 256)
    dg_part[(int64_t)blockIdx.x * d + c] = red[0][c] + red[1][c] + red[2][c] + red[3][c];
}

// out[c] (=|+=) sum over parts: a workgroup takes 64 columns (lane = column, so each load is
// 256 contiguous bytes); its 16 waves take parts w, w + 16, ... in order and their sums meet
// in LDS in wave order, so the result does not depend on scheduling.
constexpr int kColsumWaves = 16;
__global__ __launch_bounds__(64 * kColsumWaves) void colsum_kernel(const float *__restrict__ part,
                                                                   int nparts, int d,
                                                                   float *__restrict__ out,
                                                                   int accumulate) {
  __shared__ float red[kColsumWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  const int cc = c < d ? c : d - 1;
  float s = 0.f;
#pragma unroll 4
  for (int i = w; i < nparts; i += kColsumWaves) s += part[(int64_t)i * d + cc];
  red[w][lane] = s;
  __syncthreads();
  if (w != 0 || c >= d) return;
  s = 0.f;
#pragma unroll
  for (int i = 0; i < kColsumWaves; ++i) s += red[i][lane];
  out[c] = accumulate ? out[c] + s : s;
}

// ---- SwiGLU ("Transformer 篇" 5.3): u = SiLU(a) c; da = du c SiLU'(a), dc = du SiLU(a),
// SiLU'(a) = sigma(a) (1 + a (1 - sigma(a))).
// sigma(a) = 1 / (1 + e^-a): for bf16 data with the hardware exp2 and reciprocal (about 1 ulp
// each, far below the bf16 rounding of the results), for fp32 data with the library forms.
template <typename T>
__device__ __forceinline__ float sigmoid_of(float a) {
  if constexpr (std::is_same<T, bf16_t>::value)
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * 1.4426950408889634f));
  else
    return 1.0f / (1.0f + __expf(-a));
}

// 4 consecutive elements per thread (n % 4 == 0 and 4-element aligned buffers, which the
// callers' shapes give: d_ff is a multiple of 4)
template <typename T>
__global__ void swiglu_fwd_kernel(const T *a, const T *c, T *u, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  const f32x4_t av = load4(a + i), cv = load4(c + i);
  f32x4_t r;
#pragma unroll
  for (int x = 0; x < 4; ++x) r[x] = av[x] * sigmoid_of<T>(av[x]) * cv[x];
  store4(u + i, r);
}

template <typename T>
__global__ void swiglu_back_kernel(const T *a, const T *c, const float *du, T *da, T *dc,
                                   int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  const f32x4_t av = load4(a + i), cv = load4(c + i), g = load4(du + i);
  f32x4_t ra, rc;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const float sg = sigmoid_of<T>(av[x]);
    ra[x] = g[x] * cv[x] * sg * (1.0f + av[x] * (1.0f - sg));
    rc[x] = g[x] * av[x] * sg;
  }
  store4(da + i, ra);
  store4(dc + i, rc);
}

// ---- inverse RoPE in place on H heads of rows (row stride), position p (or row % S)
template <typename T>
__global__ void rope_inv_kernel(T *x, int64_t row_stride, const int32_t *pos, int64_t rows, int S,
                                int H, int dh, const float *cs, int max_seq) {
  const int pairs = dh >> 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * H * pairs) return;
  const int i = (int)(idx % pairs);
  const int64_t rh = idx / pairs;
  const int h = (int)(rh % H);
  const int64_t r = rh / H;
  const int p = pos ? pos[r] : (int)(r % S);
  if (p < 0 || p >= max_seq) return;
  T *v = x + r * row_stride + (int64_t)h * dh + 2 * i;
  const float c = cs[((int64_t)p * pairs + i) * 2], s = cs[((int64_t)p * pairs + i) * 2 + 1];
  const float x0 = ld1(v), x1 = ld1(v + 1);
  st1(v, x0 * c + x1 * s);
  st1(v + 1, -x0 * s + x1 * c);
}

// ---- attention backward. TPR threads share one row, each owning DPT = min(dh, 32) of its
// columns; dot products are summed across them with lane shuffles.
constexpr int kAttnRows = 64;
template <int TPR>
__device__ __forceinline__ float row_dot(float v) {
  if constexpr (TPR >= 2) v += __shfl_xor(v, 1);
  if constexpr (TPR >= 4) v += __shfl_xor(v, 2);
  return v;
}

// grid (ceil(S/64), Hq, B); thread (row i of the block, part p). lse: each query row's
// logsumexp, kept by the forward attention.
template <typename T, int DH>
__global__ __launch_bounds__(kAttnRows *(DH / (DH < 32 ? DH : 32))) void attn_dq_kernel(
    const T *__restrict__ qkv, int64_t ld, const T *__restrict__ o, int64_t ldo,
    const T *__restrict__ dout, int64_t lddo, T *__restrict__ dqkv, int S, int Hq, int Hkv,
    int window, float scale, const float *__restrict__ lse_in, float *__restrict__ dsum_out) {
  constexpr int DPT = DH < 32 ? DH : 32, TPR = DH / DPT, NT = kAttnRows * TPR;
  const int qd = Hq * DH, kvd = Hkv * DH;
  const int h = blockIdx.y, b = blockIdx.z, g = h / (Hq / Hkv);
  const int tid = threadIdx.x, row = tid / TPR, part = tid % TPR;
  const int i = blockIdx.x * kAttnRows + row;
  const bool live = i < S;
  const int ic = live ? i : S - 1;
  const int64_t rq = (int64_t)b * S + ic;
  float qv[DPT], dov[DPT], dq[DPT];
  float dsum = 0.f;
#pragma unroll
  for (int e = 0; e < DPT; ++e) {
    const int c = part * DPT + e;
    qv[e] = ld1(qkv + rq * ld + (int64_t)h * DH + c);
    dov[e] = ld1(dout + rq * lddo + (int64_t)h * DH + c);
    dsum += dov[e] * ld1(o + rq * ldo + (int64_t)h * DH + c);
    dq[e] = 0.f;
  }
  dsum = row_dot<TPR>(dsum);
  const float lse = lse_in[rq * Hq + h];
  __shared__ __attribute__((aligned(16))) float ks[kAttnRows][DH];
  __shared__ __attribute__((aligned(16))) float vs[kAttnRows][DH];
  const int i0 = blockIdx.x * kAttnRows;
  const int ilast = min(i0 + kAttnRows, S) - 1;
  const int jlo = window > 0 ? max(0, i0 - window + 1) : 0;
  const int jlo_row = window > 0 ? max(0, i - window + 1) : 0;
  // dq = sum_j P_ij (dP_ij - D_i) k_j scale, P_ij = exp(q_i . k_j scale - lse_i)
  for (int j0 = jlo - jlo % kAttnRows; j0 <= ilast; j0 += kAttnRows) {
    __syncthreads();
    for (int idx = tid; idx < kAttnRows * DH; idx += NT) {
      const int jj = idx / DH, c = idx % DH, j = j0 + jj;
      const int64_t rk = ((int64_t)b * S + (j < S ? j : 0)) * ld + (int64_t)g * DH + c;
      ks[jj][c] = j < S ? ld1(qkv + rk + qd) : 0.f;
      vs[jj][c] = j < S ? ld1(qkv + rk + qd + kvd) : 0.f;
    }
    __syncthreads();
    for (int jj = 0; jj < kAttnRows; ++jj) {
      const int j = j0 + jj;
      const f32x4_t *k4 = (const f32x4_t *)&ks[jj][part * DPT];
      const f32x4_t *v4 = (const f32x4_t *)&vs[jj][part * DPT];
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e4 = 0; e4 < DPT / 4; ++e4) {
        const f32x4_t kk = k4[e4], vv = v4[e4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          s += qv[4 * e4 + x] * kk[x];
          dp += dov[4 * e4 + x] * vv[x];
        }
      }
      s = row_dot<TPR>(s) * scale;
      dp = row_dot<TPR>(dp);
      if (j <= i && j >= jlo_row) {
        const float ds = expf(s - lse) * (dp - dsum) * scale;
#pragma unroll
        for (int e4 = 0; e4 < DPT / 4; ++e4) {
          const f32x4_t kk = k4[e4];
#pragma unroll
          for (int x = 0; x < 4; ++x) dq[4 * e4 + x] += ds * kk[x];
        }
      }
    }
  }
  if (live) {
#pragma unroll
    for (int e = 0; e < DPT; ++e) st1(dqkv + rq * ld + (int64_t)h * DH + part * DPT + e, dq[e]);
    if (part == 0) dsum_out[rq * Hq + h] = dsum;
  }
}

// grid (ceil(S/64), Hkv, B); thread (key j of the block, part p); loops over the query heads
// of the group and the queries that see key j
template <typename T, int DH>
__global__ __launch_bounds__(kAttnRows *(DH / (DH < 32 ? DH : 32))) void attn_dkdv_kernel(
    const T *__restrict__ qkv, int64_t ld, const T *__restrict__ dout, int64_t lddo,
    T *__restrict__ dqkv, int S, int Hq, int Hkv, int window, float scale,
    const float *__restrict__ lse_in, const float *__restrict__ dsum_in) {
  constexpr int DPT = DH < 32 ? DH : 32, TPR = DH / DPT, NT = kAttnRows * TPR;
  const int qd = Hq * DH, kvd = Hkv * DH, G = Hq / Hkv;
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, row = tid / TPR, part = tid % TPR;
  const int j = blockIdx.x * kAttnRows + row;
  const bool live = j < S;
  const int64_t rk = (int64_t)b * S + (live ? j : S - 1);
  float kv[DPT], vv[DPT], dk[DPT], dv[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) {
    const int c = part * DPT + e;
    kv[e] = ld1(qkv + rk * ld + qd + (int64_t)g * DH + c);
    vv[e] = ld1(qkv + rk * ld + qd + kvd + (int64_t)g * DH + c);
    dk[e] = dv[e] = 0.f;
  }
  __shared__ __attribute__((aligned(16))) float qs[kAttnRows][DH];
  __shared__ __attribute__((aligned(16))) float ds_[kAttnRows][DH];
  __shared__ float ls[kAttnRows], dsm[kAttnRows];
  const int j0b = blockIdx.x * kAttnRows;
  const int jlast = min(j0b + kAttnRows, S) - 1;
  // queries i with j <= i (and i - window + 1 <= j): i in [j0b, jlast + window - 1]
  const int ihi = window > 0 ? min(S - 1, jlast + window - 1) : S - 1;
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    for (int i0 = j0b; i0 <= ihi; i0 += kAttnRows) {
      __syncthreads();
      for (int idx = tid; idx < kAttnRows * DH; idx += NT) {
        const int ii = idx / DH, c = idx % DH, i = i0 + ii;
        const int64_t rq = (int64_t)b * S + (i < S ? i : 0);
        qs[ii][c] = i < S ? ld1(qkv + rq * ld + (int64_t)h * DH + c) : 0.f;
        ds_[ii][c] = i < S ? ld1(dout + rq * lddo + (int64_t)h * DH + c) : 0.f;
      }
      for (int ii = tid; ii < kAttnRows; ii += NT) {
        const int i = i0 + ii;
        ls[ii] = i < S ? lse_in[((int64_t)b * S + i) * Hq + h] : 0.f;
        dsm[ii] = i < S ? dsum_in[((int64_t)b * S + i) * Hq + h] : 0.f;
      }
      __syncthreads();
      for (int ii = 0; ii < kAttnRows; ++ii) {
        const int i = i0 + ii;
        const f32x4_t *q4 = (const f32x4_t *)&qs[ii][part * DPT];
        const f32x4_t *d4 = (const f32x4_t *)&ds_[ii][part * DPT];
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e4 = 0; e4 < DPT / 4; ++e4) {
          const f32x4_t qq = q4[e4], dd = d4[e4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            s += qq[x] * kv[4 * e4 + x];
            dp += dd[x] * vv[4 * e4 + x];
          }
        }
        s = row_dot<TPR>(s) * scale;
        dp = row_dot<TPR>(dp);
        const bool vis = i < S && j <= i && (window <= 0 || j >= i - window + 1);
        if (vis) {
          const float p = expf(s - ls[ii]);
          const float dsv = p * (dp - dsm[ii]) * scale;
#pragma unroll
          for (int e4 = 0; e4 < DPT / 4; ++e4) {
            const f32x4_t qq = q4[e4], dd = d4[e4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              dv[4 * e4 + x] += p * dd[x];
              dk[4 * e4 + x] += dsv * qq[x];
            }
          }
        }
      }
    }
  }
  if (live) {
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
      const int c = part * DPT + e;
      st1(dqkv + rk * ld + qd + (int64_t)g * DH + c, dk[e]);
      st1(dqkv + rk * ld + qd + kvd + (int64_t)g * DH + c, dv[e]);
    }
  }
}

// ---- split-K partial sums in a fixed order (4 outputs per thread; N % 4 == 0 or scalar tail)
__global__ void sum_parts_kernel(const float *__restrict__ part, int parts, int64_t M, int N,
                                 float *__restrict__ y, int64_t ldy) {
  const int64_t n4 = (N + 3) / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= M * n4) return;
  const int64_t m = idx / n4;
  const int n = (int)(idx % n4) * 4;
  const int64_t stride = M * N;
  const float *p = part + m * N + n;
  if (n + 4 <= N && (N & 3) == 0 && (ldy & 3) == 0 && ((uintptr_t)y & 15) == 0) {
    f32x4_t acc = *(const f32x4_t *)p;
    for (int q = 1; q < parts; ++q) acc += *(const f32x4_t *)(p + q * stride);
    *(f32x4_t *)(y + m * ldy + n) = acc;
  } else {
    for (int x = 0; x < 4 && n + x < N; ++x) {
      float acc = p[x];
      for (int q = 1; q < parts; ++q) acc += p[q * stride + x];
      y[m * ldy + n + x] = acc;
    }
  }
}

// ---- embedding backward: dE[ids[r]] += dx[r] (fp32 atomics: rows with the same id add in
// an unspecified order)
__global__ void embed_back_kernel(const int32_t *__restrict__ ids, int64_t n, int vocab, int d,
                                  const float *__restrict__ dx, float *__restrict__ dE) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * d) return;
  const int64_t r = idx / d;
  const int c = (int)(idx % d);
  const int id = ids[r];
  if (id < 0 || id >= vocab) return;
  atomicAdd(dE + (int64_t)id * d + c, dx[idx]);
}

// ---- gradient clipping ("LLM 2" Gradient Clip) and AdamW ("LLM 2" Optimizer)
constexpr int kSumsqBlocks = 256;   // partial sums per tensor

__device__ __forceinline__ double sq4(f32x4_t v) {
  return ((double)v[0] * v[0] + (double)v[1] * v[1]) + ((double)v[2] * v[2] + (double)v[3] * v[3]);
}

// Workgroup blk's share of sum g[i]^2 (fp64): 16-byte loads, four in flight per thread when g
// is 16-byte aligned; the partition and the order of the adds are fixed by (blk, thread).
__device__ __forceinline__ double sumsq_share(const float *__restrict__ g, int64_t n, int blk) {
  const int tid = threadIdx.x;
  const int64_t step = (int64_t)kSumsqBlocks * 256;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int64_t j0 = 0;   // first element left to the scalar loop
  if (((uintptr_t)g & 15) == 0) {
    const int64_t nv = n >> 2;
    const f32x4_t *gv = (const f32x4_t *)g;
    int64_t i = (int64_t)blk * 256 + tid;
    for (; i + 3 * step < nv; i += 4 * step) {
      const f32x4_t a = gv[i], b = gv[i + step], c = gv[i + 2 * step], d = gv[i + 3 * step];
      s0 += sq4(a);
      s1 += sq4(b);
      s2 += sq4(c);
      s3 += sq4(d);
    }
    for (; i < nv; i += step) s0 += sq4(gv[i]);
    j0 = 4 * nv;
  }
  for (int64_t j = j0 + (int64_t)blk * 256 + tid; j < n; j += step) s1 += (double)g[j] * (double)g[j];
  return (s0 + s1) + (s2 + s3);
}

__global__ __launch_bounds__(256) void sumsq_kernel(const float *__restrict__ g, int64_t n,
                                                    double *__restrict__ part) {
  __shared__ double red[256];
  red[threadIdx.x] = sumsq_share(g, n, blockIdx.x);
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void clip_coef_kernel(const double *__restrict__ part,
                                                        int nparts, float max_norm,
                                                        float *__restrict__ coef,
                                                        float *__restrict__ norm) {
  __shared__ double red[256];
  // four independent sums per thread, so four loads are in flight
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int i = threadIdx.x;
  for (; i + 768 < nparts; i += 1024) {
    s0 += part[i];
    s1 += part[i + 256];
    s2 += part[i + 512];
    s3 += part[i + 768];
  }
  for (; i < nparts; i += 256) s0 += part[i];
  red[threadIdx.x] = (s0 + s1) + (s2 + s3);
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double total = sqrt(red[0]);
    coef[0] = total > (double)max_norm ? (float)((double)max_norm / (total + 1e-6)) : 1.0f;
    if (norm) norm[0] = (float)total;
  }
}

// Tensors of one batched launch (kernel arguments, so no table in device memory).
constexpr int kBatch = 32;
struct SumsqBatch {
  const float *g[kBatch];
  int64_t n[kBatch];
};
struct AdamwBatch {
  float *p[kBatch];
  bf16_t *pb[kBatch];
  const float *g[kBatch];
  float *m[kBatch], *v[kBatch];
  int64_t n[kBatch];
  int64_t blk0[kBatch + 1];   // first block of each tensor; blk0[count] = total blocks
  bool vec[kBatch];           // 16-byte aligned p, g, m, v and 8-byte aligned pb (or none)
  int count;
};

// sumsq_kernel for tensor blockIdx.y of a batch, partials at part + blockIdx.y * kSumsqBlocks
__global__ __launch_bounds__(256) void sumsq_multi_kernel(SumsqBatch bt, double *__restrict__ part) {
  const int t = blockIdx.y;
  __shared__ double red[256];
  red[threadIdx.x] = sumsq_share(bt.g[t], bt.n[t], blockIdx.x);
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[(int64_t)t * kSumsqBlocks + blockIdx.x] = red[0];
}

__device__ __forceinline__ void adamw_elem(float *__restrict__ p, bf16_t *__restrict__ pb,
                                           const float *__restrict__ g, float *__restrict__ m,
                                           float *__restrict__ v, int64_t i, float lr, float b1,
                                           float b2, float eps, float wd, float c1, float c2,
                                           float cf) {
  const float gg = g[i] * cf;
  const float mi = b1 * m[i] + (1.0f - b1) * gg;
  const float vi = b2 * v[i] + (1.0f - b2) * gg * gg;
  m[i] = mi;
  v[i] = vi;
  const float th = p[i];
  const float nw = th - lr * (mi / c1) / (sqrtf(vi / c2) + eps) - lr * wd * th;
  p[i] = nw;
  if (pb) pb[i] = f32_to_bf16(nw);
}

__global__ void adamw_kernel(float *__restrict__ p, bf16_t *__restrict__ pb,
                             const float *__restrict__ g, float *__restrict__ m,
                             float *__restrict__ v, int64_t n, float lr, float b1, float b2,
                             float eps, float wd, float c1, float c2,
                             const float *__restrict__ coef) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  adamw_elem(p, pb, g, m, v, i, lr, b1, b2, eps, wd, c1, c2, coef ? coef[0] : 1.0f);
}

// one launch over a batch of tensors: block b belongs to the tensor t with
// blk0[t] <= b < blk0[t + 1]
__global__ __launch_bounds__(256) void adamw_multi_kernel(AdamwBatch bt, float lr, float b1,
                                                          float b2, float eps, float wd,
                                                          float c1, float c2,
                                                          const float *__restrict__ coef) {
  const int64_t b = blockIdx.x;
  int t = 0;
  while (t + 1 < bt.count && bt.blk0[t + 1] <= b) ++t;
  // 4 consecutive elements per thread, with 16-byte accesses where the tensor allows them
  const int64_t i = ((b - bt.blk0[t]) * 256 + threadIdx.x) * 4;
  const int64_t n = bt.n[t];
  if (i >= n) return;
  const float cf = coef ? coef[0] : 1.0f;
  float *p = bt.p[t], *m = bt.m[t], *v = bt.v[t];
  const float *g = bt.g[t];
  bf16_t *pb = bt.pb[t];
  if (bt.vec[t] && i + 4 <= n) {
    const f32x4_t gg = load4(g + i) * cf, m0 = load4(m + i), v0 = load4(v + i), th = load4(p + i);
    f32x4_t mi, vi, nw;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      mi[x] = b1 * m0[x] + (1.0f - b1) * gg[x];
      vi[x] = b2 * v0[x] + (1.0f - b2) * gg[x] * gg[x];
      nw[x] = th[x] - lr * (mi[x] / c1) / (sqrtf(vi[x] / c2) + eps) - lr * wd * th[x];
    }
    store4(m + i, mi);
    store4(v + i, vi);
    store4(p + i, nw);
    if (pb) store4(pb + i, nw);
  } else {
    for (int64_t j = i; j < i + 4 && j < n; ++j)
      adamw_elem(p, pb, g, m, v, j, lr, b1, b2, eps, wd, c1, c2, cf);
  }
}

template <typename T, int DH>
hipError_t run_attn_back(const void *qkv, int64_t ld, const void *o, int64_t ldo,
                         const void *dout, int64_t lddo, void *dqkv, int B, int S, int Hq,
                         int Hkv, int window, const float *lse, float *dsum, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)DH);
  const dim3 gq(nblk(S, kAttnRows), Hq, B), gk(nblk(S, kAttnRows), Hkv, B);
  constexpr int NT = kAttnRows * (DH / (DH < 32 ? DH : 32));
  attn_dq_kernel<T, DH><<<gq, NT, 0, s>>>(
      (const T *)qkv, ld, (const T *)o, ldo, (const T *)dout, lddo, (T *)dqkv, S, Hq, Hkv, window,
      scale, lse, dsum);
  attn_dkdv_kernel<T, DH><<<gk, NT, 0, s>>>(
      (const T *)qkv, ld, (const T *)dout, lddo, (T *)dqkv, S, Hq, Hkv, window, scale, lse, dsum);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_transpose(const void *src, int src_dt, int64_t lds, void *dst, int dst_dt,
                            int64_t ldd, int64_t R, int64_t R_valid, int C, hipStream_t s) {
  if (R == 0 || C == 0) return hipSuccess;
  const dim3 grid(nblk(C, 64), nblk(R, 64));
  if (grid.y > 65535) return hipErrorInvalidValue;
  const bool vec = ((lds | ldd | R | C) & 7) == 0 && (((uintptr_t)src | (uintptr_t)dst) & 15) == 0;
  if (src_dt == DT_BF16 && dst_dt == DT_BF16 && vec)
    transpose_bf16_kernel<<<grid, 256, 0, s>>>((const uint16_t *)src, lds, (uint16_t *)dst, ldd,
                                               R, R_valid, C);
  else if (src_dt == DT_BF16 && dst_dt == DT_BF16)
    transpose_kernel<bf16_t, bf16_t><<<grid, 256, 0, s>>>((const bf16_t *)src, lds, (bf16_t *)dst, ldd, R, R_valid, C);
  else if (src_dt == DT_F32 && dst_dt == DT_BF16)
    transpose_kernel<float, bf16_t><<<grid, 256, 0, s>>>((const float *)src, lds, (bf16_t *)dst, ldd, R, R_valid, C);
  else if (src_dt == DT_F32 && dst_dt == DT_F32)
    transpose_kernel<float, float><<<grid, 256, 0, s>>>((const float *)src, lds, (float *)dst, ldd, R, R_valid, C);
  else
    transpose_kernel<bf16_t, float><<<grid, 256, 0, s>>>((const bf16_t *)src, lds, (float *)dst, ldd, R, R_valid, C);
  return hipGetLastError();
}

hipError_t launch_transpose_multi(const TransposeJob *jobs, int n, hipStream_t s) {
  TransposeBatch b{};
  int64_t t = 0;
  for (int j = 0; j < n; ++j) {
    const TransposeJob &q = jobs[j];
    const bool vec = ((q.lds | q.ldd | q.R | q.C) & 7) == 0 &&
                     (((uintptr_t)q.src | (uintptr_t)q.dst) & 15) == 0;
    if (!vec || b.n == kTransposeJobs) {   // the general kernel, one launch
      const hipError_t e = launch_transpose(q.src, DT_BF16, q.lds, q.dst, DT_BF16, q.ldd, q.R, q.R,
                                            (int)q.C, s);
      if (e != hipSuccess) return e;
      continue;
    }
    b.job[b.n] = q;
    b.start[b.n++] = (int)t;
    t += ((q.R + 63) / 64) * ((q.C + 63) / 64);
    if (t > 0x7fffffff) return hipErrorInvalidValue;
  }
  if (b.n == 0 || t == 0) return hipSuccess;
  b.start[b.n] = (int)t;
  transpose_bf16_multi_kernel<<<(unsigned)t, 256, 0, s>>>(b);
  return hipGetLastError();
}

hipError_t launch_convert(const void *src, int src_dt, void *dst, int dst_dt, int64_t n,
                          hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (src_dt == DT_F32 && dst_dt == DT_BF16)
    convert_kernel<float, bf16_t><<<nblk(n, 256), 256, 0, s>>>((const float *)src, (bf16_t *)dst, n);
  else if (src_dt == DT_F32 && dst_dt == DT_F32)
    convert_kernel<float, float><<<nblk(n, 256), 256, 0, s>>>((const float *)src, (float *)dst, n);
  else if (src_dt == DT_BF16 && dst_dt == DT_F32)
    convert_kernel<bf16_t, float><<<nblk(n, 256), 256, 0, s>>>((const bf16_t *)src, (float *)dst, n);
  else
    convert_kernel<bf16_t, bf16_t><<<nblk(n, 256), 256, 0, s>>>((const bf16_t *)src, (bf16_t *)dst, n);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  fill_f32_kernel<<<nblk(n, 256), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_ce_backward(const float *z, int64_t ldz, const int32_t *targets, int64_t M,
                              int V, void *dz, int dz_dt, int64_t ldd, float *row_loss,
                              int32_t *count, float *mean, hipStream_t s) {
  if (M == 0) return hipSuccess;
  count_targets_kernel<<<1, 1024, 0, s>>>(targets, M, V, count);
  if (dz_dt == DT_BF16)
    ce_back_kernel<bf16_t><<<(unsigned)M, 256, 0, s>>>(z, ldz, targets, V, count, (bf16_t *)dz,
                                                       ldd, row_loss);
  else
    ce_back_kernel<float><<<(unsigned)M, 256, 0, s>>>(z, ldz, targets, V, count, (float *)dz, ldd,
                                                      row_loss);
  mean_rows_kernel<<<1, 1024, 0, s>>>(row_loss, M, count, mean);
  return hipGetLastError();
}

hipError_t launch_count_targets(const int32_t *targets, int64_t M, int V, int32_t *count,
                                hipStream_t s) {
  count_targets_kernel<<<1, 1024, 0, s>>>(targets, M, V, count);
  return hipGetLastError();
}

hipError_t launch_mean_rows(const float *row_loss, int64_t M, const int32_t *count, float *mean,
                            hipStream_t s) {
  mean_rows_kernel<<<1, 1024, 0, s>>>(row_loss, M, count, mean);
  return hipGetLastError();
}

int rms_back_parts(int64_t rows) { return (int)nblk(rows, 4 * kRmsRows); }

hipError_t launch_rms_backward(const float *x, const void *g, int g_dt, const float *dy, float *dx,
                               void *dx_bf16, float *dg, int accumulate_dg, float *dg_part,
                               int64_t rows, int d, float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int ng = d / 4, vpt = (ng + 63) / 64;
  const unsigned nb = (unsigned)rms_back_parts(rows);
#define TFM_RMSB(V)                                                                            \
  if (g_dt == DT_BF16)                                                                         \
    rms_back_kernel<V, bf16_t><<<nb, 256, 0, s>>>(x, (const bf16_t *)g, dy, dx,               \
                                                  (bf16_t *)dx_bf16, dg_part, rows, d, eps);    \
  else                                                                                         \
    rms_back_kernel<V, float><<<nb, 256, 0, s>>>(x, (const float *)g, dy, dx,                 \
                                                 (bf16_t *)dx_bf16, dg_part, rows, d, eps);
  switch (vpt) {
    case 1: TFM_RMSB(1) break;
    case 2: TFM_RMSB(2) break;
    case 3: TFM_RMSB(3) break;
    case 4: TFM_RMSB(4) break;
    case 5: TFM_RMSB(5) break;
    case 6: TFM_RMSB(6) break;
    case 7: TFM_RMSB(7) break;
    case 8: TFM_RMSB(8) break;
    default: return hipErrorInvalidValue;
  }
#undef TFM_RMSB
  colsum_kernel<<<nblk(d, 64), 64 * kColsumWaves, 0, s>>>(dg_part, (int)nb, d, dg, accumulate_dg);
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const void *a, const void *c, void *u, int dt, int64_t n,
                             hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (n % 4) return hipErrorInvalidValue;   // the kernel takes 4 elements per thread
  if (dt == DT_BF16)
    swiglu_fwd_kernel<bf16_t><<<nblk(n / 4, 256), 256, 0, s>>>((const bf16_t *)a, (const bf16_t *)c,
                                                           (bf16_t *)u, n);
  else
    swiglu_fwd_kernel<float><<<nblk(n / 4, 256), 256, 0, s>>>((const float *)a, (const float *)c,
                                                          (float *)u, n);
  return hipGetLastError();
}

hipError_t launch_swiglu_backward(const void *a, const void *c, const float *du, void *da,
                                  void *dc, int dt, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (n % 4) return hipErrorInvalidValue;   // the kernel takes 4 elements per thread
  if (dt == DT_BF16)
    swiglu_back_kernel<bf16_t><<<nblk(n / 4, 256), 256, 0, s>>>(
        (const bf16_t *)a, (const bf16_t *)c, du, (bf16_t *)da, (bf16_t *)dc, n);
  else
    swiglu_back_kernel<float><<<nblk(n / 4, 256), 256, 0, s>>>(
        (const float *)a, (const float *)c, du, (float *)da, (float *)dc, n);
  return hipGetLastError();
}

hipError_t launch_rope_inverse(void *x, int dt, int64_t row_stride, const int32_t *positions,
                               int64_t rows, int S, int H, int d_head, const float *cos_sin,
                               int max_seq, hipStream_t s) {
  const int64_t total = rows * H * (d_head / 2);
  if (total == 0) return hipSuccess;
  if (dt == DT_BF16)
    rope_inv_kernel<bf16_t><<<nblk(total, 256), 256, 0, s>>>((bf16_t *)x, row_stride, positions,
                                                             rows, S, H, d_head, cos_sin, max_seq);
  else
    rope_inv_kernel<float><<<nblk(total, 256), 256, 0, s>>>((float *)x, row_stride, positions,
                                                            rows, S, H, d_head, cos_sin, max_seq);
  return hipGetLastError();
}

bool attention_backward_supported(int d_head) {
  return d_head == 16 || d_head == 32 || d_head == 64 || d_head == 128;
}

hipError_t launch_attention_backward(const void *qkv, int64_t ld, const void *o, int64_t ldo,
                                     const void *dout, int64_t lddo, void *dqkv, int B, int S,
                                     int Hq, int Hkv, int d_head, int dt, int window,
                                     const float *lse, float *dsum, const int32_t *positions,
                                     const float *cos_sin, int max_seq, hipStream_t s) {
  if ((int64_t)B * S == 0) return hipSuccess;
  if (B > 65535 || Hq > 65535) return hipErrorInvalidValue;
  const int w = window > 0 && window < S ? window : 0;
  if (dt == DT_BF16)
    return launch_attention_backward_bf16(qkv, ld, o, ldo, dout, lddo, dqkv, B, S, Hq, Hkv,
                                          d_head, w, lse, dsum, positions, cos_sin, max_seq, s);
  hipError_t e = hipErrorInvalidValue;
  switch (d_head) {
    case 16: e = run_attn_back<float, 16>(qkv, ld, o, ldo, dout, lddo, dqkv, B, S, Hq, Hkv, w, lse, dsum, s); break;
    case 32: e = run_attn_back<float, 32>(qkv, ld, o, ldo, dout, lddo, dqkv, B, S, Hq, Hkv, w, lse, dsum, s); break;
    case 64: e = run_attn_back<float, 64>(qkv, ld, o, ldo, dout, lddo, dqkv, B, S, Hq, Hkv, w, lse, dsum, s); break;
    case 128: e = run_attn_back<float, 128>(qkv, ld, o, ldo, dout, lddo, dqkv, B, S, Hq, Hkv, w, lse, dsum, s); break;
  }
  if (e != hipSuccess || !cos_sin) return e;
  const int64_t qd = (int64_t)Hq * d_head;
  e = launch_rope_inverse(dqkv, dt, ld, positions, (int64_t)B * S, S, Hq, d_head, cos_sin, max_seq,
                          s);
  if (e != hipSuccess) return e;
  return launch_rope_inverse((float *)dqkv + qd, dt, ld, positions, (int64_t)B * S, S, Hkv,
                             d_head, cos_sin, max_seq, s);
}

hipError_t launch_sumsq_multi(const float *const *g, const int64_t *n, int count, double *part,
                              hipStream_t s) {
  for (int t0 = 0; t0 < count; t0 += kBatch) {
    SumsqBatch bt{};
    const int c = count - t0 < kBatch ? count - t0 : kBatch;
    for (int t = 0; t < c; ++t) {
      bt.g[t] = n[t0 + t] > 0 ? g[t0 + t] : nullptr;
      bt.n[t] = n[t0 + t];
    }
    sumsq_multi_kernel<<<dim3(kSumsqBlocks, c), 256, 0, s>>>(bt, part + (size_t)t0 * kSumsqBlocks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_adamw_multi(float *const *p, void *const *pb, const float *const *g,
                              float *const *m, float *const *v, const int64_t *n, int count,
                              float lr, float b1, float b2, float eps, float wd, float c1,
                              float c2, const float *coef, hipStream_t s) {
  int t = 0;
  while (t < count) {
    AdamwBatch bt{};
    int c = 0;
    int64_t blocks = 0;
    for (; t < count && c < kBatch; ++t) {   // empty tensors take no slot
      if (n[t] == 0) continue;
      bt.p[c] = p[t];
      bt.pb[c] = pb ? (bf16_t *)pb[t] : nullptr;
      bt.g[c] = g[t];
      bt.m[c] = m[t];
      bt.v[c] = v[t];
      bt.n[c] = n[t];
      bt.vec[c] = (((uintptr_t)p[t] | (uintptr_t)g[t] | (uintptr_t)m[t] | (uintptr_t)v[t]) & 15) == 0 &&
                  ((uintptr_t)bt.pb[c] & 7) == 0;
      bt.blk0[c] = blocks;
      blocks += nblk(n[t], 1024);
      ++c;
    }
    if (c == 0) break;
    bt.blk0[c] = blocks;
    bt.count = c;
    adamw_multi_kernel<<<(unsigned)blocks, 256, 0, s>>>(bt, lr, b1, b2, eps, wd, c1, c2, coef);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_sum_parts(const float *part, int parts, int64_t M, int N, float *y,
                            int64_t ldy, hipStream_t s) {
  const int64_t total = M * ((N + 3) / 4);
  if (total == 0) return hipSuccess;
  sum_parts_kernel<<<nblk(total, 256), 256, 0, s>>>(part, parts, M, N, y, ldy);
  return hipGetLastError();
}

hipError_t launch_embed_backward(const int32_t *ids, int64_t n, int vocab, int d, const float *dx,
                                 float *dE, hipStream_t s) {
  if (n == 0) return hipSuccess;
  embed_back_kernel<<<nblk(n * d, 256), 256, 0, s>>>(ids, n, vocab, d, dx, dE);
  return hipGetLastError();
}

int sumsq_parts() { return kSumsqBlocks; }

hipError_t launch_sumsq(const float *g, int64_t n, double *part, hipStream_t s) {
  sumsq_kernel<<<kSumsqBlocks, 256, 0, s>>>(g, n, part);
  return hipGetLastError();
}

hipError_t launch_clip_coef(const double *part, int nparts, float max_norm, float *coef,
                            float *norm, hipStream_t s) {
  clip_coef_kernel<<<1, 256, 0, s>>>(part, nparts, max_norm, coef, norm);
  return hipGetLastError();
}

hipError_t launch_adamw(float *p, void *pb, const float *g, float *m, float *v, int64_t n,
                        float lr, float b1, float b2, float eps, float wd, float c1, float c2,
                        const float *coef, hipStream_t s) {
  if (n == 0) return hipSuccess;
  adamw_kernel<<<nblk(n, 256), 256, 0, s>>>(p, (bf16_t *)pb, g, m, v, n, lr, b1, b2, eps, wd, c1,
                                            c2, coef);
  return hipGetLastError();
}

}  // namespace tfm

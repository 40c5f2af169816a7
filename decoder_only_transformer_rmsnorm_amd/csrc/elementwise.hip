// Memory-bound kernels of the decoder forward: RoPE table, embedding gather, RMSNorm,
// standalone RoPE, and a small fill kernel (used instead of hipMemsetAsync so the forward
// stays safe to capture in a HIP graph).
#include "common.h"
#include "internal.h"

namespace tfm {
namespace {

// RoPE table ("Transformer 篇" (dujian.net) 5.5; "LLM 2" RoPE): angle p * theta^(-2i/d)
// formed in double precision, cos and sin stored interleaved as float.
__global__ void rope_table_kernel(float *cs, int max_seq, int half, double theta, int d_head) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)max_seq * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  const double omega = pow(theta, -2.0 * (double)i / (double)d_head);
  const double a = (double)p * omega;
  cs[2 * idx] = (float)cos(a);
  cs[2 * idx + 1] = (float)sin(a);
}

// Embedding ("Transformer 篇" 5.2): x[r, :] = table[ids[r], :], 4 elements per thread.
template <typename T>
__global__ void embed_kernel(const int32_t *ids, int64_t n, const T *table, int vocab, int d,
                             float *x, int32_t *err) {
  const int groups = d >> 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * groups) return;
  const int64_t r = idx / groups;
  const int c = (int)(idx % groups) * 4;
  const int id = ids[r];
  f32x4_t val;
  if (id >= 0 && id < vocab) {
    val = load4(table + (int64_t)id * d + c);
  } else {
    const float nan = __builtin_nanf("");
    val = f32x4_t{nan, nan, nan, nan};
    if (err) *err = 1;
  }
  store4(x + r * d + c, val);
}

// RMSNorm ("Transformer 篇" 5.6; "LLM 2" RMSNorm): one wave per row. Each lane reads
// 4 consecutive elements per step (a wave covers 256 contiguous elements per step, so every
// load is a full, coalesced 1 KiB (fp32) or 512 B (bf16) transaction). VPT steps per lane
// are a compile-time count, so all of a row's loads are issued before the first is used and
// the row is read from HBM exactly once; rows wider than 256 * kMaxVpt take a second pass.
// Sum of squares and scaling in fp32, one rounding at the store.
constexpr int kMaxVpt = 8;

template <int VPT, typename TX, typename TG, typename TY>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const TX *__restrict__ x,
                                                      const TG *__restrict__ g,
                                                      TY *__restrict__ y, int64_t rows, int d,
                                                      float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const TX *xr = x + row * d;
  TY *yr = y + row * d;
  const int ng = d >> 2;
  f32x4_t c[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int gi = lane + 64 * i;
    // clamp the index instead of branching so every load issues back to back
    c[i] = load4(xr + 4 * (gi < ng ? gi : 0));
    if (gi >= ng) c[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i)
    ss += c[i][0] * c[i][0] + c[i][1] * c[i][1] + c[i][2] * c[i][2] + c[i][3] * c[i][3];
  for (int gi = lane + 64 * VPT; gi < ng; gi += 64) {
    const f32x4_t v = load4(xr + 4 * gi);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / (float)d + eps);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int gi = lane + 64 * i;
    if (gi < ng) store4(yr + 4 * gi, c[i] * inv * load4(g + 4 * gi));
  }
  for (int gi = lane + 64 * VPT; gi < ng; gi += 64)
    store4(yr + 4 * gi, load4(xr + 4 * gi) * inv * load4(g + 4 * gi));
}

// Embedding followed by the first block's RMSNorm ("Transformer 篇" 5.2 and 5.6) in one pass:
// one wave per token gathers its table row, writes it to the fp32 residual x and writes
// y = RMSNorm(x; g) — the same loads, sum order and rounding as embed_kernel followed by
// rmsnorm_kernel (the table values convert to fp32 exactly), without reading x back. A bad id
// gives a NaN row (and NaN y) and sets the flag.
template <int VPT, typename TT, typename TG, typename TY>
__global__ __launch_bounds__(256) void embed_rmsnorm_kernel(const int32_t *__restrict__ ids,
                                                            int64_t rows,
                                                            const TT *__restrict__ table,
                                                            int vocab, int d, float *__restrict__ x,
                                                            int32_t *err, const TG *__restrict__ g,
                                                            TY *__restrict__ y, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int id = ids[row];
  const bool ok = id >= 0 && id < vocab;
  if (!ok && lane == 0 && err) *err = 1;
  const TT *tr = table + (int64_t)(ok ? id : 0) * d;
  float *xr = x + row * d;
  TY *yr = y + row * d;
  const int ng = d >> 2;
  const float nan = __builtin_nanf("");
  const f32x4_t bad = {nan, nan, nan, nan};
  f32x4_t c[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int gi = lane + 64 * i;
    c[i] = load4(tr + 4 * (gi < ng ? gi : 0));
    if (!ok) c[i] = bad;
    if (gi >= ng) c[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int gi = lane + 64 * i;
    if (gi < ng) store4(xr + 4 * gi, c[i]);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i)
    ss += c[i][0] * c[i][0] + c[i][1] * c[i][1] + c[i][2] * c[i][2] + c[i][3] * c[i][3];
  for (int gi = lane + 64 * VPT; gi < ng; gi += 64) {
    const f32x4_t v = ok ? load4(tr + 4 * gi) : bad;
    store4(xr + 4 * gi, v);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / (float)d + eps);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int gi = lane + 64 * i;
    if (gi < ng) store4(yr + 4 * gi, c[i] * inv * load4(g + 4 * gi));
  }
  for (int gi = lane + 64 * VPT; gi < ng; gi += 64)
    store4(yr + 4 * gi, (ok ? load4(tr + 4 * gi) : bad) * inv * load4(g + 4 * gi));
}

// RoPE in place ("Transformer 篇" 5.5; "Transformer篇" (fengye404.top) 7): each thread
// rotates two adjacent pairs (4 elements) of one head of one token.
template <typename T>
__global__ void rope_kernel(T *x, int64_t row_stride, const int32_t *pos, int B, int S, int H,
                            int d_head, const float *cs, int max_seq) {
  const int gph = d_head >> 2;  // 4-element groups per head
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)B * S * H * gph;
  if (idx >= total) return;
  const int gi = (int)(idx % gph);
  const int64_t rh = idx / gph;
  const int hh = (int)(rh % H);
  const int64_t r = rh / H;  // token row b*S + s
  const int p = pos ? pos[r] : (int)(r % S);
  T *px = x + r * row_stride + (int64_t)hh * d_head + 4 * gi;
  f32x4_t v = load4(px);
  if (p >= 0 && p < max_seq) {
    const f32x4_t c = *(const f32x4_t *)(cs + ((int64_t)p * (d_head >> 1) + 2 * gi) * 2);
    const float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
    v[0] = x0 * c[0] - x1 * c[1];
    v[1] = x0 * c[1] + x1 * c[0];
    v[2] = x2 * c[2] - x3 * c[3];
    v[3] = x2 * c[3] + x3 * c[2];
  } else {
    const float nan = __builtin_nanf("");
    v = f32x4_t{nan, nan, nan, nan};
  }
  store4(px, v);
}

// Next-token cross-entropy ("LLM 2" Optimize / Loss; "Transformer篇" (fengye404.top) 12):
// combine the LM-head tile partials of one row, max_t and sum_t of exp(logit - max_t), into
// the row's log-sum-exp in a fixed order and subtract the target logit.
// A workgroup takes 64 consecutive rows (lane = row, so every load of a wave reads 256
// consecutive bytes of one partial column) and its 8 waves split the column tiles t = w, w + 8,
// ...; the waves' maxima, then their sums of exp, are combined through LDS in wave order, so
// the result is deterministic.
constexpr int kXentWaves = 8;
__global__ __launch_bounds__(64 * kXentWaves) void xent_reduce_kernel(
    const float *__restrict__ x_max, const float *__restrict__ x_sum,
    const float *__restrict__ x_tgt, const int32_t *targets, int T, int64_t M, int V,
    float *loss, float *lse, bool oob_zero) {
  __shared__ float red[kXentWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t m = (int64_t)blockIdx.x * 64 + lane;
  const int64_t mc = m < M ? m : M - 1;
  constexpr float kLog2e = 1.4426950408889634f;
  float mx = -__builtin_inff();
#pragma unroll 4
  for (int i = w; i < T; i += kXentWaves) mx = fmaxf(mx, x_max[(int64_t)i * M + mc]);
  red[w][lane] = mx;
  __syncthreads();
  mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < kXentWaves; ++i) mx = fmaxf(mx, red[i][lane]);
  __syncthreads();
  float se = 0.f;
#pragma unroll 4
  for (int i = w; i < T; i += kXentWaves)
    se += x_sum[(int64_t)i * M + mc] * exp2f((x_max[(int64_t)i * M + mc] - mx) * kLog2e);
  red[w][lane] = se;
  __syncthreads();
  if (w != 0 || m >= M) return;
  se = 0.f;
#pragma unroll
  for (int i = 0; i < kXentWaves; ++i) se += red[i][lane];
  const int t = targets[m];
  const float l = mx + logf(se);
  if (lse) lse[m] = l;
  if (t < 0 || (oob_zero && t >= V)) loss[m] = 0.f;
  else if (t >= V) loss[m] = __builtin_nanf("");
  else loss[m] = l - x_tgt[m];
}

// Mean over the rows with a target: one workgroup, strided fp64 partial sums in a fixed order
// and a fixed tree, so the result does not depend on scheduling.
constexpr int kMeanThreads = 1024;
__global__ __launch_bounds__(kMeanThreads) void mean_loss_kernel(const float *loss,
                                                                 const int32_t *targets,
                                                                 int64_t M, float *mean) {
  __shared__ double ps[kMeanThreads];
  __shared__ int64_t pc[kMeanThreads];
  const int tid = threadIdx.x;
  double acc = 0.0;
  int64_t cnt = 0;
  for (int64_t m = tid; m < M; m += kMeanThreads)
    if (targets[m] >= 0) {
      acc += (double)loss[m];
      ++cnt;
    }
  ps[tid] = acc;
  pc[tid] = cnt;
  __syncthreads();
  for (int w = kMeanThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      ps[tid] += ps[tid + w];
      pc[tid] += pc[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) mean[0] = pc[0] ? (float)(ps[0] / (double)pc[0]) : 0.f;
}

__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

inline unsigned blocks_for(int64_t n, int t) { return (unsigned)((n + t - 1) / t); }

template <int VPT, typename TX, typename TG, typename TY>
hipError_t rms4(const void *x, const void *g, void *y, int64_t rows, int d, float eps,
                hipStream_t s) {
  rmsnorm_kernel<VPT, TX, TG, TY><<<blocks_for(rows, 4), 256, 0, s>>>(
      (const TX *)x, (const TG *)g, (TY *)y, rows, d, eps);
  return hipGetLastError();
}

template <typename TX, typename TG, typename TY>
hipError_t rms3(const void *x, const void *g, void *y, int64_t rows, int d, float eps,
                hipStream_t s) {
  switch ((d + 255) / 256) {   // float4 steps per lane
    case 1: return rms4<1, TX, TG, TY>(x, g, y, rows, d, eps, s);
    case 2: return rms4<2, TX, TG, TY>(x, g, y, rows, d, eps, s);
    case 3: return rms4<3, TX, TG, TY>(x, g, y, rows, d, eps, s);
    case 4: return rms4<4, TX, TG, TY>(x, g, y, rows, d, eps, s);
    case 5: return rms4<5, TX, TG, TY>(x, g, y, rows, d, eps, s);
    case 6: return rms4<6, TX, TG, TY>(x, g, y, rows, d, eps, s);
    case 7: return rms4<7, TX, TG, TY>(x, g, y, rows, d, eps, s);
    default: return rms4<kMaxVpt, TX, TG, TY>(x, g, y, rows, d, eps, s);
  }
}

template <typename TX, typename TG>
hipError_t rms2(const void *x, const void *g, void *y, int y_dt, int64_t rows, int d, float eps,
                hipStream_t s) {
  return y_dt == DT_BF16 ? rms3<TX, TG, bf16_t>(x, g, y, rows, d, eps, s)
                         : rms3<TX, TG, float>(x, g, y, rows, d, eps, s);
}

template <typename TX>
hipError_t rms1(const void *x, const void *g, int g_dt, void *y, int y_dt, int64_t rows, int d,
                float eps, hipStream_t s) {
  return g_dt == DT_BF16 ? rms2<TX, bf16_t>(x, g, y, y_dt, rows, d, eps, s)
                         : rms2<TX, float>(x, g, y, y_dt, rows, d, eps, s);
}

template <int VPT, typename T>
hipError_t er4(const int32_t *ids, int64_t rows, const void *table, int vocab, int d, float *x,
               int32_t *err, const void *g, void *y, float eps, hipStream_t s) {
  embed_rmsnorm_kernel<VPT, T, T, T><<<blocks_for(rows, 4), 256, 0, s>>>(
      ids, rows, (const T *)table, vocab, d, x, err, (const T *)g, (T *)y, eps);
  return hipGetLastError();
}

template <typename T>
hipError_t er3(const int32_t *ids, int64_t rows, const void *table, int vocab, int d, float *x,
               int32_t *err, const void *g, void *y, float eps, hipStream_t s) {
  switch ((d + 255) / 256) {   // float4 steps per lane, as for rmsnorm_kernel
    case 1: return er4<1, T>(ids, rows, table, vocab, d, x, err, g, y, eps, s);
    case 2: return er4<2, T>(ids, rows, table, vocab, d, x, err, g, y, eps, s);
    case 3: return er4<3, T>(ids, rows, table, vocab, d, x, err, g, y, eps, s);
    case 4: return er4<4, T>(ids, rows, table, vocab, d, x, err, g, y, eps, s);
    case 5: return er4<5, T>(ids, rows, table, vocab, d, x, err, g, y, eps, s);
    case 6: return er4<6, T>(ids, rows, table, vocab, d, x, err, g, y, eps, s);
    case 7: return er4<7, T>(ids, rows, table, vocab, d, x, err, g, y, eps, s);
    default: return er4<kMaxVpt, T>(ids, rows, table, vocab, d, x, err, g, y, eps, s);
  }
}

// Matrix-core rate probe (a measurement of the sustained bf16 MFMA rate, the second
// denominator beside the published peak): each wave runs `iters` rounds of 8 independent
// v_mfma_f32_16x16x32_bf16 on operands held in registers, filled with pseudo-random bf16
// values in +-[1, 2) (the chip sustains less with random than with constant operands), and
// writes a checksum so that no product can be dropped.
__global__ __launch_bounds__(256) void mfma_rate_kernel(int64_t iters, float *sink) {
  uint32_t x = 0x9e3779b9u * (uint32_t)(blockIdx.x * 256 + threadIdx.x + 1);
  u32x4_t a[2], b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x ^= x << 13; x ^= x >> 17; x ^= x << 5;
      a[i][j] = (x & 0x807f807fu) | 0x3f803f80u;
      x ^= x << 13; x ^= x >> 17; x ^= x << 5;
      b[i][j] = (x & 0x807f807fu) | 0x3f803f80u;
    }
  // 8 independent accumulators, written out one by one so that each stays in its registers
  const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, a[0]), a1 = __builtin_bit_cast(bf16x8_t, a[1]);
  const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, b[0]), b1 = __builtin_bit_cast(bf16x8_t, b[1]);
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  f32x4_t c0 = z, c1 = z, c2 = z, c3 = z, c4 = z, c5 = z, c6 = z, c7 = z;
  // the products are written as instructions with each accumulator read and written in place
  // (left to itself the compiler moves the accumulators between registers every round, and
  // those moves, not the products, then set the rate)
#define TFM_MFMA(C, A, B) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(C) : "v"(A), "v"(B))
  for (int64_t it = 0; it < iters; ++it) {
    TFM_MFMA(c0, a0, b0); TFM_MFMA(c1, a1, b0); TFM_MFMA(c2, a0, b1); TFM_MFMA(c3, a1, b1);
    TFM_MFMA(c4, a0, b0); TFM_MFMA(c5, a1, b0); TFM_MFMA(c6, a0, b1); TFM_MFMA(c7, a1, b1);
  }
#undef TFM_MFMA
  // the vector ALU reads the last products only after they have left the matrix core
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  const f32x4_t t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
  float s = t[0] + t[1] + t[2] + t[3];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace

hipError_t launch_mfma_rate(int64_t iters, int blocks, float *sink, hipStream_t s) {
  if (blocks <= 0 || iters <= 0) return hipSuccess;
  mfma_rate_kernel<<<blocks, 256, 0, s>>>(iters, sink);
  return hipGetLastError();
}

hipError_t launch_rope_table(float *cos_sin, int max_seq, int d_head, double theta,
                             hipStream_t s) {
  const int64_t n = (int64_t)max_seq * (d_head / 2);
  if (n == 0) return hipSuccess;
  rope_table_kernel<<<blocks_for(n, 256), 256, 0, s>>>(cos_sin, max_seq, d_head / 2, theta,
                                                       d_head);
  return hipGetLastError();
}

hipError_t launch_embed(const int32_t *ids, int64_t n, const void *table, int table_dt,
                        int vocab, int d, float *x, int32_t *err_flag, hipStream_t s) {
  const int64_t total = n * (d / 4);
  if (total == 0) return hipSuccess;
  if (table_dt == DT_BF16)
    embed_kernel<bf16_t><<<blocks_for(total, 256), 256, 0, s>>>(ids, n, (const bf16_t *)table,
                                                                vocab, d, x, err_flag);
  else
    embed_kernel<float><<<blocks_for(total, 256), 256, 0, s>>>(ids, n, (const float *)table,
                                                               vocab, d, x, err_flag);
  return hipGetLastError();
}

hipError_t launch_embed_rmsnorm(const int32_t *ids, int64_t n, const void *table, int dt,
                                int vocab, int d, float *x, int32_t *err_flag, const void *g,
                                void *y, float eps, hipStream_t s) {
  if (n == 0) return hipSuccess;
  return dt == DT_BF16 ? er3<bf16_t>(ids, n, table, vocab, d, x, err_flag, g, y, eps, s)
                       : er3<float>(ids, n, table, vocab, d, x, err_flag, g, y, eps, s);
}

hipError_t launch_rmsnorm(const void *x, int x_dt, const void *g, int g_dt, void *y, int y_dt,
                          int64_t rows, int d, float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  return x_dt == DT_BF16 ? rms1<bf16_t>(x, g, g_dt, y, y_dt, rows, d, eps, s)
                         : rms1<float>(x, g, g_dt, y, y_dt, rows, d, eps, s);
}

hipError_t launch_rope(void *x, int x_dt, int64_t row_stride, const int32_t *positions, int B,
                       int S, int H, int d_head, const float *cos_sin, int max_seq,
                       hipStream_t s) {
  const int64_t total = (int64_t)B * S * H * (d_head / 4);
  if (total == 0) return hipSuccess;
  if (x_dt == DT_BF16)
    rope_kernel<bf16_t><<<blocks_for(total, 256), 256, 0, s>>>(
        (bf16_t *)x, row_stride, positions, B, S, H, d_head, cos_sin, max_seq);
  else
    rope_kernel<float><<<blocks_for(total, 256), 256, 0, s>>>(
        (float *)x, row_stride, positions, B, S, H, d_head, cos_sin, max_seq);
  return hipGetLastError();
}

hipError_t launch_xent_reduce(const float *x_max, const float *x_sum, const float *x_tgt,
                              const int32_t *targets, int T, int64_t M, int V, float *loss,
                              float *mean, hipStream_t s, float *lse, bool oob_zero) {
  if (M == 0) return hipSuccess;
  xent_reduce_kernel<<<blocks_for(M, 64), 64 * kXentWaves, 0, s>>>(x_max, x_sum, x_tgt, targets,
                                                                   T, M, V, loss, lse, oob_zero);
  if (mean) mean_loss_kernel<<<1, kMeanThreads, 0, s>>>(loss, targets, M, mean);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  fill_i32_kernel<<<blocks_for(n, 256), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace tfm

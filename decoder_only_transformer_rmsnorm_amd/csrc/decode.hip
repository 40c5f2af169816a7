// Incremental decoding with a KV cache ("LLMs-from-scratch" (deepseek.csdn.net) 6.1: the key
// and value of every earlier step are kept and only the new token's q, k, v are computed;
// "LLM 2" GQA/MQA: generation is bound by reading the cache, which grouped heads shrink).
//
// KV cache layout (bf16): per layer a K block and a V block, each (B, Hkv, cache_seq, d_head),
// so one head's keys are a contiguous run of d_head-element rows and slot t holds the token at
// position t. Layer l's K block starts at element 2 l blk, its V block at (2 l + 1) blk,
// blk = B Hkv cache_seq d_head.
//
// Kernels:
//  * dgemm_kernel: y = x W^T for few rows (one new token per sequence). Every weight row is
//    read once and used by all rows of x, so the kernel streams the weights from HBM. A
//    workgroup owns 16 output columns (SwiGLU: 16 hidden units = 16 gate + 16 up rows) and 16
//    rows of x; its 4 waves split K and each runs v_mfma_f32_16x16x32_bf16 with the weight
//    rows as the A operand (lane l: row l % 16, k chunk l / 16), so a lane's accumulator holds
//    4 consecutive output columns of one row m = l % 16. The 4 partial sums meet in LDS.
//    Epilogues: store (logits), residual add, SiLU(gate) * up, and q / k / v with RoPE where
//    k and v go straight to the cache slot of the token's position.
//  * dec_attn_kernel: one workgroup per (sequence, kv head, chunk of 128 cached keys); all
//    query heads of the group share each K / V row read (grouped-query attention). Scores and
//    softmax in fp32 (log2 domain); the partial (max, sum, unnormalised output) of each chunk
//    goes to the workspace and dec_combine_kernel merges the chunks in chunk order.
//  * kv_store_kernel: after a prefill block's QKV projection, copies the rotated k and v rows
//    into the cache slots of their positions.
#include <cmath>

#include "common.h"
#include "internal.h"

namespace tfm {
namespace {

constexpr int kDecKeys = 128;   // cached keys (and threads) per attention workgroup
constexpr int kDecMaxGroup = 8; // query heads per kv head supported by the decode kernel
constexpr int kMaxChunks = 1024; // chunks per sequence the merge holds (cache_seq <= 131072)
constexpr float kLog2e = 1.4426950408889634f;

inline unsigned grid1(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

__device__ __forceinline__ u32x4_t ld16(const bf16_t *p) { return *(const u32x4_t *)p; }

// Rotates the adjacent pairs (n, n+1), (n+2, n+3) of a q or k head by the angles of position
// pos ("Transformer 篇" 5.5; "LLM 2" RoPE); n is the column within the head.
__device__ __forceinline__ f32x4_t rope4(f32x4_t v, const float *cos_sin, int pos, int d_head,
                                         int n) {
  const f32x4_t cs = *(const f32x4_t *)(cos_sin + ((int64_t)pos * (d_head >> 1) + (n >> 1)) * 2);
  const float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
  return f32x4_t{x0 * cs[0] - x1 * cs[1], x0 * cs[1] + x1 * cs[0], x2 * cs[2] - x3 * cs[3],
                 x2 * cs[3] + x3 * cs[2]};
}

template <int EPI>
__global__ __launch_bounds__(256) void dgemm_kernel(DecodeGemmArgs g) {
  constexpr int NA = EPI == EPI_SWIGLU ? 2 : 1;   // weight row sets (gate, up)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, kc = lane >> 4;
  const int nb0 = blockIdx.x * 16;     // first output column (SwiGLU: hidden unit)
  const int m0 = blockIdx.y * 16;

  // A operand rows: output column nb0 + r16 of each weight row set
  const bf16_t *wrow[NA];
  bool wok[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const int n = nb0 + r16;
    if constexpr (EPI == EPI_SWIGLU) {
      wok[a] = n < g.n0;
      wrow[a] = (const bf16_t *)(a == 0 ? g.w0 : g.w1) + (int64_t)(wok[a] ? n : 0) * g.K;
    } else if constexpr (EPI == EPI_QKV_CACHE) {
      wok[a] = n < g.N;
      const int nn = wok[a] ? n : 0;
      wrow[a] = nn < g.n0 ? (const bf16_t *)g.w0 + (int64_t)nn * g.K
              : nn < g.n0 + g.n1 ? (const bf16_t *)g.w1 + (int64_t)(nn - g.n0) * g.K
                                 : (const bf16_t *)g.w2 + (int64_t)(nn - g.n0 - g.n1) * g.K;
    } else {
      wok[a] = n < g.N;
      wrow[a] = (const bf16_t *)g.w0 + (int64_t)(wok[a] ? n : 0) * g.K;
    }
  }
  const int mr = m0 + r16;
  const bool xok = mr < g.M;
  const bf16_t *xrow = (const bf16_t *)g.x + (int64_t)(xok ? mr : 0) * g.ldx;
  // fused RMSNorm ("Transformer 篇" 5.6): 1 / rms of each of the 16 rows, wave w takes rows
  // 4w .. 4w+3; the operand is then x * inv * g, rounded once to bf16
  __shared__ float inv_rms[16];
  const bool fuse = g.norm_x != nullptr;
  const float *nrow = fuse ? g.norm_x + (int64_t)(xok ? mr : 0) * g.ldx : nullptr;
  if (fuse) {   // 16 threads per row, each summing every 16th group of 4 columns
    const int row = threadIdx.x >> 4, part = threadIdx.x & 15;
    const int m = m0 + row;
    float ss = 0.f;
    if (m < g.M) {
      const float *xr = g.norm_x + (int64_t)m * g.ldx;
#pragma unroll 4
      for (int k = 4 * part; k < g.K; k += 64) {
        const f32x4_t v = load4(xr + k);
        ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
      }
    }
    for (int off = 8; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if (part == 0) inv_rms[row] = rsqrtf(ss / (float)g.K + g.eps);
    __syncthreads();
  }
  const float rinv = fuse ? inv_rms[r16] : 0.f;
  auto x_chunk = [&](int k) -> u32x4_t {   // 8 activations of row mr from column k
    if (!fuse) return ld16(xrow + k);
    const f32x4_t a = load4(nrow + k), b = load4(nrow + k + 4);
    const f32x4_t ga = load4((const bf16_t *)g.norm_g + k), gb = load4((const bf16_t *)g.norm_g + k + 4);
    const f32x4_t ya = a * rinv * ga, yb = b * rinv * gb;
    return u32x4_t{pack_bf16x2(ya[0], ya[1]), pack_bf16x2(ya[2], ya[3]),
                   pack_bf16x2(yb[0], yb[1]), pack_bf16x2(yb[2], yb[3])};
  };

  f32x4_t acc[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) acc[a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  const int nks = (g.K + 31) / 32;   // 32-wide k steps; wave w takes steps w, w + 4, ...
  constexpr int U = 4;               // steps whose loads are in flight together
  for (int ks0 = w; ks0 < nks; ks0 += 4 * U) {
    u32x4_t xa[U], wa[U][NA];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (ks0 + 4 * u) * 32 + kc * 8;   // K % 8 == 0: a chunk is all in or out
      const bool kok = ks0 + 4 * u < nks && k < g.K;
      xa[u] = xok && kok ? x_chunk(k) : zero;
#pragma unroll
      for (int a = 0; a < NA; ++a) wa[u][a] = wok[a] && kok ? ld16(wrow[a] + k) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int a = 0; a < NA; ++a)
        acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wa[u][a]),
                                                        __builtin_bit_cast(bf16x8_t, xa[u]),
                                                        acc[a], 0, 0, 0);
  }

  // the four waves' partial sums meet in LDS; wave 0 finishes
  __shared__ __attribute__((aligned(16))) f32x4_t red[3][NA][64];
  if (w > 0) {
#pragma unroll
    for (int a = 0; a < NA; ++a) red[w - 1][a][lane] = acc[a];
  }
  __syncthreads();
  if (w > 0) return;
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int j = 0; j < 3; ++j) acc[a] += red[j][a][lane];

  // lane holds columns n .. n+3 of row m
  const int m = m0 + r16;
  const int n = nb0 + 4 * kc;
  if (m >= g.M) return;
  if constexpr (EPI == EPI_STORE) {
    if (g.y_dt == DT_BF16) {
      bf16_t *y = (bf16_t *)g.y + (int64_t)m * g.ldy + n;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < g.N) y[r] = f32_to_bf16(acc[0][r]);
    } else {
      float *y = (float *)g.y + (int64_t)m * g.ldy + n;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < g.N) y[r] = acc[0][r];
    }
  } else if constexpr (EPI == EPI_RESIDUAL) {
    float *y = (float *)g.y + (int64_t)m * g.ldy + n;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < g.N) y[r] += acc[0][r];
  } else if constexpr (EPI == EPI_SWIGLU) {
    bf16_t *y = (bf16_t *)g.y + (int64_t)m * g.ldy + n;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < g.n0) {
        const float a = acc[0][r], b = acc[1][r];
        y[r] = f32_to_bf16(a / (1.0f + __expf(-a)) * b);
      }
  } else {   // EPI_QKV_CACHE: row m is sequence m's new token at position positions[m]
    if (n >= g.N) return;
    const int pos = g.positions[m];
    const bool ok = pos >= 0 && pos < g.cache_seq && pos < g.max_seq;
    if (!ok) g.pos_flag[0] = 1;
    f32x4_t v = acc[0];
    const int dh = g.d_head;
    if (n < g.n0) {   // q column: rotate, keep for the attention
      const float nan = __builtin_nanf("");
      v = ok ? rope4(v, g.cos_sin, pos, dh, n % dh) : f32x4_t{nan, nan, nan, nan};
      store4((bf16_t *)g.y + (int64_t)m * g.ldy + n, v);
    } else if (ok) {  // k (rotated) or v column: into the cache slot of the position
      const bool is_k = n < g.n0 + g.n1;
      const int j = n - g.n0 - (is_k ? 0 : g.n1);
      if (is_k) v = rope4(v, g.cos_sin, pos, dh, j % dh);
      const int grp = j / dh, d = j % dh;
      bf16_t *dst = (bf16_t *)(is_k ? g.k_cache : g.v_cache) +
                    (((int64_t)m * g.n_kv_heads + grp) * g.cache_seq + pos) * dh + d;
      store4(dst, v);
    }
  }
}

// ---- decode attention
// One workgroup per (sequence b, kv head grp, chunk c of 128 cached keys). Every thread first
// loads its key's K and V rows (all loads in flight together); V goes to LDS for the P.V pass.
// The chunk's partial (max, sum, unnormalised output) per query head goes to `part`;
// dec_combine_kernel merges the chunks in chunk order.
template <int DH>
__global__ __launch_bounds__(kDecKeys) void dec_attn_kernel(
    const bf16_t *__restrict__ q, int64_t q_stride, const bf16_t *__restrict__ kc,
    const bf16_t *__restrict__ vc, const int32_t *__restrict__ positions, int Hq, int Hkv,
    int cache_seq, int window, float scale_log2, float *__restrict__ part, int n_ch,
    bf16_t *__restrict__ o, int64_t o_stride) {
  constexpr int PS = 2 + DH;               // partial record: max, sum, output
  constexpr int DC = DH / 8;               // 16-byte chunks per K / V row
  constexpr int D4 = DH / 4;               // threads per value row in the P.V pass
  constexpr int TG = kDecKeys / D4;        // key groups in the P.V pass
  constexpr int NW = kDecKeys / 64;        // waves (one thread per key of the chunk)
  const int c = blockIdx.x, grp = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int pos = positions[b];
  const bool valid = pos >= 0 && pos < cache_seq;
  if (!valid) {   // no cache slot: NaN output for the group's heads
    if (c == 0)
      for (int i = tid; i < G * DH; i += kDecKeys)
        o[(int64_t)b * o_stride + (int64_t)grp * G * DH + i] = f32_to_bf16(__builtin_nanf(""));
    return;
  }
  const int n = pos + 1;
  const int t0 = window > 0 && n > window ? n - window : 0;
  const int used = (n - t0 + kDecKeys - 1) / kDecKeys;
  if (c >= used) return;
  const int ks = t0 + c * kDecKeys;
  const int cnt = min(kDecKeys, n - ks);

  __shared__ float qs[kDecMaxGroup][DH];
  __shared__ float sc[kDecMaxGroup][kDecKeys];
  __shared__ __attribute__((aligned(16))) bf16_t vs[kDecKeys][DH];
  __shared__ __attribute__((aligned(16))) float red[TG][DH];
  __shared__ float stat[kDecMaxGroup][2];
  __shared__ float wred[NW][kDecMaxGroup];

  const int64_t head = ((int64_t)b * Hkv + grp) * cache_seq;   // first row of this head
  u32x4_t kr[DC], vr[DC];
  if (tid < cnt) {
    const bf16_t *kp = kc + (head + ks + tid) * DH;
    const bf16_t *vp = vc + (head + ks + tid) * DH;
#pragma unroll
    for (int j = 0; j < DC; ++j) kr[j] = ld16(kp + 8 * j);
#pragma unroll
    for (int j = 0; j < DC; ++j) vr[j] = ld16(vp + 8 * j);
  }
  for (int i = tid; i < G * DH; i += kDecKeys) {
    const int h = i / DH, d = i % DH;
    qs[h][d] = bf16_to_f32(q[(int64_t)b * q_stride + (int64_t)(grp * G + h) * DH + d]) *
               scale_log2;
  }
  if (tid < cnt) {
#pragma unroll
    for (int j = 0; j < DC; ++j) *(u32x4_t *)&vs[tid][8 * j] = vr[j];
  }
  __syncthreads();

  // scores (log2 units): thread t takes key ks + t
  if (tid < cnt) {
    float s[kDecMaxGroup];
#pragma unroll
    for (int h = 0; h < kDecMaxGroup; ++h) s[h] = 0.f;
#pragma unroll
    for (int j = 0; j < DC; ++j) {
      float kf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = __uint_as_float(kr[j][e] << 16);
        kf[2 * e + 1] = __uint_as_float(kr[j][e] & 0xffff0000u);
      }
#pragma unroll
      for (int h = 0; h < kDecMaxGroup; ++h)
        if (h < G) {
#pragma unroll
          for (int e = 0; e < 8; ++e) s[h] = __builtin_fmaf(qs[h][8 * j + e], kf[e], s[h]);
        }
    }
#pragma unroll
    for (int h = 0; h < kDecMaxGroup; ++h)
      if (h < G) sc[h][tid] = s[h];
  }
  // per head: max over the chunk, then p = 2^(s - max) and its sum
  const int wv = tid >> 6, lane = tid & 63;
  for (int h = 0; h < G; ++h) {
    float mx = -__builtin_inff();
    __syncthreads();
    for (int t = tid; t < cnt; t += kDecKeys) mx = fmaxf(mx, sc[h][t]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) wred[wv][h] = mx;
    __syncthreads();
    mx = wred[0][h];
    for (int j = 1; j < NW; ++j) mx = fmaxf(mx, wred[j][h]);
    float sum = 0.f;
    for (int t = tid; t < cnt; t += kDecKeys) {
      const float p = exp2f(sc[h][t] - mx);
      sc[h][t] = p;
      sum += p;
    }
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    __syncthreads();
    if (lane == 0) wred[wv][h] = sum;
    __syncthreads();
    if (tid == 0) {
      stat[h][0] = mx;
      float tot = 0.f;
      for (int j = 0; j < NW; ++j) tot += wred[j][h];
      stat[h][1] = tot;
    }
  }
  __syncthreads();

  // P.V from LDS: thread (key group tg, 4 columns d4) sums over keys tg, tg + TG, ...
  const int d4 = tid % D4, tg = tid / D4;
  f32x4_t acc[kDecMaxGroup];
#pragma unroll
  for (int h = 0; h < kDecMaxGroup; ++h) acc[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int t = tg; t < cnt; t += TG) {
    const u32x2_t raw = *(const u32x2_t *)&vs[t][4 * d4];
    const f32x4_t vv = {__uint_as_float(raw[0] << 16), __uint_as_float(raw[0] & 0xffff0000u),
                        __uint_as_float(raw[1] << 16), __uint_as_float(raw[1] & 0xffff0000u)};
#pragma unroll
    for (int h = 0; h < kDecMaxGroup; ++h)
      if (h < G) acc[h] += sc[h][t] * vv;
  }
  float *rec0 = part + (((int64_t)b * Hq + grp * G) * n_ch + c) * PS;   // head h: + h n_ch PS
  for (int h = 0; h < G; ++h) {
    __syncthreads();
    *(f32x4_t *)&red[tg][4 * d4] = acc[h];
    __syncthreads();
    for (int d = tid; d < DH; d += kDecKeys) {
      float sum = 0.f;
      for (int j = 0; j < TG; ++j) sum += red[j][d];
      rec0[(int64_t)h * n_ch * PS + 2 + d] = sum;
    }
    if (tid == 0) {
      rec0[(int64_t)h * n_ch * PS + 0] = stat[h][0];
      rec0[(int64_t)h * n_ch * PS + 1] = stat[h][1];
    }
  }

}

// Merges the chunk partials of one (sequence, query head) in chunk order. (A merge by the
// last chunk workgroup would need device-scope fences, which write back the XCD's L2.)
template <int DH>
__global__ __launch_bounds__(128) void dec_combine_kernel(const float *__restrict__ part,
                                                          const int32_t *__restrict__ positions,
                                                          int Hq, int cache_seq, int window,
                                                          int n_ch, bf16_t *__restrict__ o,
                                                          int64_t o_stride) {
  constexpr int PS = 2 + DH;
  const int bh = blockIdx.x, b = bh / Hq, h = bh % Hq;
  const int pos = positions[b];
  if (pos < 0 || pos >= cache_seq) return;   // the attention kernel wrote the NaN row
  const int n = pos + 1;
  const int t0 = window > 0 && n > window ? n - window : 0;
  const int used = (n - t0 + kDecKeys - 1) / kDecKeys;
  const float *rec = part + (int64_t)bh * n_ch * PS;
  // chunk weights 2^(m_c - max) and the denominator, computed once in LDS
  __shared__ float wgt[kMaxChunks];
  __shared__ float den;
  for (int c = threadIdx.x; c < used; c += blockDim.x) wgt[c] = rec[c * PS];
  __syncthreads();
  if (threadIdx.x == 0) {
    float mx = -__builtin_inff();
    for (int c = 0; c < used; ++c) mx = fmaxf(mx, wgt[c]);
    float l = 0.f;
    for (int c = 0; c < used; ++c) {
      wgt[c] = exp2f(wgt[c] - mx);
      l += wgt[c] * rec[c * PS + 1];
    }
    den = l;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < DH; d += blockDim.x) {
    float num = 0.f;
#pragma unroll 4
    for (int c = 0; c < used; ++c) num += wgt[c] * rec[c * PS + 2 + d];
    o[(int64_t)b * o_stride + (int64_t)h * DH + d] = f32_to_bf16(num / den);
  }
}

// Prefill: the k and v columns of the qkv rows go to the cache slots of their positions.
__global__ void kv_store_kernel(const bf16_t *__restrict__ qkv, int64_t ld, int qd, int kvd,
                                int dh, int Hkv, int S, int64_t rows,
                                const int32_t *__restrict__ positions, bf16_t *__restrict__ kc,
                                bf16_t *__restrict__ vc, int cache_seq, int32_t *pos_flag) {
  const int chunks = 2 * kvd / 8;   // 16-byte chunks of k | v per row
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * chunks) return;
  const int64_t r = idx / chunks;
  const int c = (int)(idx % chunks) * 8;
  const int b = (int)(r / S), s = (int)(r % S);
  const int pos = positions ? positions[r] : s;
  if (pos < 0 || pos >= cache_seq) {
    pos_flag[0] = 1;
    return;
  }
  const bool is_k = c < kvd;
  const int j = is_k ? c : c - kvd;
  const int grp = j / dh, d = j % dh;
  bf16_t *dst = (is_k ? kc : vc) + (((int64_t)b * Hkv + grp) * cache_seq + pos) * dh + d;
  *(u32x4_t *)dst = ld16(qkv + r * ld + qd + c);
}

template <int DH>
hipError_t run_dec_attn(const void *q, int64_t q_stride, const void *kc, const void *vc,
                        const int32_t *positions, int B, int Hq, int Hkv, int cache_seq,
                        int window, float *part, void *o, int64_t o_stride,
                        hipStream_t s) {
  const int n_ch = decode_chunks(cache_seq);
  const float sl2 = kLog2e / sqrtf((float)DH);
  dec_attn_kernel<DH><<<dim3(n_ch, Hkv, B), kDecKeys, 0, s>>>(
      (const bf16_t *)q, q_stride, (const bf16_t *)kc, (const bf16_t *)vc, positions, Hq, Hkv,
      cache_seq, window, sl2, part, n_ch, (bf16_t *)o, o_stride);
  dec_combine_kernel<DH><<<B * Hq, 128, 0, s>>>(part, positions, Hq, cache_seq, window, n_ch,
                                                (bf16_t *)o, o_stride);
  return hipGetLastError();
}

}  // namespace

int decode_chunks(int cache_seq) { return (cache_seq + kDecKeys - 1) / kDecKeys; }
int decode_max_cache() { return kDecKeys * kMaxChunks; }
bool decode_group_supported(int Hq, int Hkv) { return Hq % Hkv == 0 && Hq / Hkv <= kDecMaxGroup; }

hipError_t launch_decode_gemm(int epi, const DecodeGemmArgs &g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  const int cols = epi == EPI_SWIGLU ? g.n0 : g.N;
  const dim3 grid(grid1(cols, 16), grid1(g.M, 16));
  if (grid.y > 65535) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_STORE: dgemm_kernel<EPI_STORE><<<grid, 256, 0, s>>>(g); break;
    case EPI_RESIDUAL: dgemm_kernel<EPI_RESIDUAL><<<grid, 256, 0, s>>>(g); break;
    case EPI_SWIGLU: dgemm_kernel<EPI_SWIGLU><<<grid, 256, 0, s>>>(g); break;
    case EPI_QKV_CACHE: dgemm_kernel<EPI_QKV_CACHE><<<grid, 256, 0, s>>>(g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_attention(const void *q, int64_t q_stride, const void *k_cache,
                                   const void *v_cache, const int32_t *positions, int B, int Hq,
                                   int Hkv, int d_head, int cache_seq, int window, float *part,
                                   void *o, int64_t o_stride, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (B > 65535 || Hkv > 65535) return hipErrorInvalidValue;
  switch (d_head) {
    case 32: return run_dec_attn<32>(q, q_stride, k_cache, v_cache, positions, B, Hq, Hkv,
                                     cache_seq, window, part, o, o_stride, s);
    case 64: return run_dec_attn<64>(q, q_stride, k_cache, v_cache, positions, B, Hq, Hkv,
                                     cache_seq, window, part, o, o_stride, s);
    case 128: return run_dec_attn<128>(q, q_stride, k_cache, v_cache, positions, B, Hq, Hkv,
                                       cache_seq, window, part, o, o_stride, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_kv_store(const void *qkv, int64_t ld, int qd, int kvd, int d_head, int Hkv,
                           int B, int S, const int32_t *positions, void *k_cache, void *v_cache,
                           int cache_seq, int32_t *pos_flag, hipStream_t s) {
  const int64_t rows = (int64_t)B * S;
  const int64_t total = rows * (2 * kvd / 8);
  if (total == 0) return hipSuccess;
  kv_store_kernel<<<grid1(total, 256), 256, 0, s>>>((const bf16_t *)qkv, ld, qd, kvd, d_head, Hkv,
                                                    S, rows, positions, (bf16_t *)k_cache,
                                                    (bf16_t *)v_cache, cache_seq, pos_flag);
  return hipGetLastError();
}

}  // namespace tfm

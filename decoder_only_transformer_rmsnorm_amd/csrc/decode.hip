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
//  * dec_attn_kernel: one workgroup per (split of the visible keys, kv head, sequence); its
//    waves take 64-key chunks with coalesced loads, and all query heads of the group share each
//    K / V row read (grouped-query attention). Scores and softmax in fp32 (log2 domain), online
//    over a wave's chunks; the waves merge in LDS. With one split per sequence and head (short
//    caches, or many sequences) the workgroup writes the output; otherwise each split leaves
//    a partial (max, sum, unnormalised output) and dec_combine_kernel merges them in order.
//  * kv_store_kernel: after a prefill block's QKV projection, copies the rotated k and v rows
//    into the cache slots of their positions.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "common.h"
#include "internal.h"

namespace tfm {

// Split records of the allocation-free decode attention entry point. One copy per GPU, held
// until the process ends; every call on a GPU shares it (concurrent calls on one GPU race).
// Host code never uses this name as an address: it passes the device address that
// hipGetSymbolAddress returns for the device running the call.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {

constexpr int kDecMaxGroup = 8;      // query heads per kv head supported by the decode kernel
constexpr int kDecMaxCache = 131072; // largest cache (slots per sequence) decoding supports
constexpr int kDecTargetGroups = 256;  // attention workgroups when chunks are scarce
constexpr int kDecBusyWaves = 1024;    // chunk waves that keep HBM busy without more splits
constexpr int kMaxSplits = 1024;   // split records per (sequence, head) the merge holds
constexpr float kLog2e = 1.4426950408889634f;

inline unsigned grid1(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

__device__ __forceinline__ u32x4_t ld16(const bf16_t *p) { return *(const u32x4_t *)p; }

// Rotates the adjacent pairs (n, n+1), (n+2, n+3) of a q or k head by the angles of position
// pos ("Transformer 篇" 5.5; "LLM 2" RoPE); n is the column within the head.
// cs = (cos, sin) of the two pairs' angles
__device__ __forceinline__ f32x4_t rope4(f32x4_t v, f32x4_t cs) {
  const float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
  return f32x4_t{x0 * cs[0] - x1 * cs[1], x0 * cs[1] + x1 * cs[0], x2 * cs[2] - x3 * cs[3],
                 x2 * cs[3] + x3 * cs[2]};
}

// NWV waves share the workgroup's 16 columns and split K; each wave keeps the loads of U
// 32-wide k steps in flight together
template <int EPI, int NWV, int U>
__global__ __launch_bounds__(64 * NWV) void dgemm_kernel(DecodeGemmArgs g) {
  constexpr int NA = EPI == EPI_SWIGLU ? 2 : 1;   // weight row sets (gate, up)
  constexpr int NT = 64 * NWV;
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
  const int nks = (g.K + 31) / 32;   // 32-wide k steps; wave w takes steps w, w + NWV, ...
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  u32x4_t wa[U][NA];
  auto load_w = [&](int ks0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (ks0 + NWV * u) * 32 + kc * 8;   // K % 8 == 0: a chunk is all in or out
      const bool kok = ks0 + NWV * u < nks && k < g.K;
#pragma unroll
      for (int a = 0; a < NA; ++a) wa[u][a] = wok[a] && kok ? ld16(wrow[a] + k) : zero;
    }
  };
  load_w(w);   // the first weights are in flight while the norm is computed

  // Wave 0 writes the block's outputs: the operands its epilogue reads besides the products
  // (the residual, the token's position and its rotation angles) are requested now, so their
  // latency hides behind the weight stream.
  const int m_out = m0 + r16, n_out = nb0 + 4 * kc;
  f32x4_t y_pre = {0.f, 0.f, 0.f, 0.f}, cs_pre = {0.f, 0.f, 0.f, 0.f};
  int pos_pre = 0;
  if (w == 0 && m_out < g.M) {
    if constexpr (EPI == EPI_RESIDUAL) {
      const float *yr = (const float *)g.y + (int64_t)m_out * g.ldy + n_out;
      if (n_out + 3 < g.N && (g.ldy & 3) == 0) {
        y_pre = load4(yr);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) y_pre[r] = n_out + r < g.N ? yr[r] : 0.f;
      }
    } else if constexpr (EPI == EPI_QKV_CACHE) {
      pos_pre = g.positions[m_out];
      if (n_out < g.n0 + g.n1 && pos_pre >= 0 && pos_pre < g.max_seq) {
        const int j = n_out < g.n0 ? n_out : n_out - g.n0;
        cs_pre = *(const f32x4_t *)(g.cos_sin +
                                    ((int64_t)pos_pre * (g.d_head >> 1) + ((j % g.d_head) >> 1)) * 2);
      }
    }
  }

  const bool fuse = g.norm_x != nullptr;
  const int mr = m_out;
  const bool xok = mr < g.M;
  f32x4_t acc[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) acc[a] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // (the gate and up weights of 8 steps leave no registers for a whole row: SwiGLU with 8
  // steps per wave takes the general path)
  constexpr bool kOnePass = !(NA == 2 && U > 4);
  if (kOnePass && fuse && nks <= NWV * U) {
    // fused RMSNorm ("Transformer 篇" 5.6) with the whole row in one batch of chunks: the
    // chunks of row r16 over the block's lanes (waves w, k pieces kc, steps u) cover its K
    // columns once, so the row's sum of squares is summed from them (two lane exchanges, then
    // the waves through LDS) and the row is read only once; the operand is x * inv * g,
    // rounded once to bf16
    __shared__ float ssp[NWV][16];
    const float *nrow = g.norm_x + (int64_t)(xok ? mr : 0) * g.ldx;
    f32x4_t xl[U], xh[U];
    u32x4_t gr[U];   // 8 gains (bf16) per chunk
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (w + NWV * u) * 32 + kc * 8;
      const bool kok = xok && w + NWV * u < nks && k < g.K;
      const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      xl[u] = kok ? load4(nrow + k) : z;
      xh[u] = kok ? load4(nrow + k + 4) : z;
      gr[u] = kok ? ld16((const bf16_t *)g.norm_g + k) : zero;
    }
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += xl[u][e] * xl[u][e] + xh[u][e] * xh[u][e];
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (kc == 0) ssp[w][r16] = ss;
    // LDS only: the weight loads stay in flight across this barrier
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float tot = 0.f;
#pragma unroll
    for (int v = 0; v < NWV; ++v) tot += ssp[v][r16];
    const float rinv = rsqrtf(tot / (float)g.K + g.eps);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4_t gl, gh;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        gl[2 * e] = __uint_as_float(gr[u][e] << 16);
        gl[2 * e + 1] = __uint_as_float(gr[u][e] & 0xffff0000u);
        gh[2 * e] = __uint_as_float(gr[u][e + 2] << 16);
        gh[2 * e + 1] = __uint_as_float(gr[u][e + 2] & 0xffff0000u);
      }
      const f32x4_t ya = xl[u] * rinv * gl, yb = xh[u] * rinv * gh;
      const u32x4_t xa = {pack_bf16x2(ya[0], ya[1]), pack_bf16x2(ya[2], ya[3]),
                          pack_bf16x2(yb[0], yb[1]), pack_bf16x2(yb[2], yb[3])};
#pragma unroll
      for (int a = 0; a < NA; ++a)
        acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wa[u][a]),
                                                        __builtin_bit_cast(bf16x8_t, xa),
                                                        acc[a], 0, 0, 0);
    }
  } else {
    const bf16_t *xrow = (const bf16_t *)g.x + (int64_t)(xok ? mr : 0) * g.ldx;
    // fused RMSNorm over several batches: 1 / rms of each of the 16 rows first (NT / 16
    // threads per row)
    __shared__ float inv_rms[16];
    const float *nrow = fuse ? g.norm_x + (int64_t)(xok ? mr : 0) * g.ldx : nullptr;
    if (fuse) {
      constexpr int TPR = NT / 16;
      const int row = threadIdx.x / TPR, part = threadIdx.x % TPR;
      const int m = m0 + row;
      float ss = 0.f;
      if (m < g.M) {
        const float *xr = g.norm_x + (int64_t)m * g.ldx;
#pragma unroll 8
        for (int k = 4 * part; k < g.K; k += 4 * TPR) {
          const f32x4_t v = load4(xr + k);
          ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
        }
      }
#pragma unroll
      for (int off = TPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
      if (part == 0) inv_rms[row] = rsqrtf(ss / (float)g.K + g.eps);
      // LDS only: the weight loads above stay in flight across this barrier
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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
    for (int ks0 = w; ks0 < nks; ks0 += NWV * U) {
      u32x4_t xa[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = (ks0 + NWV * u) * 32 + kc * 8;
        const bool kok = ks0 + NWV * u < nks && k < g.K;
        xa[u] = xok && kok ? x_chunk(k) : zero;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int a = 0; a < NA; ++a)
          acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wa[u][a]),
                                                          __builtin_bit_cast(bf16x8_t, xa[u]),
                                                          acc[a], 0, 0, 0);
      if (ks0 + NWV * U < nks) load_w(ks0 + NWV * U);
    }
  }

  // the waves' partial sums meet in LDS; wave 0 finishes
  if constexpr (NWV > 1) {
    __shared__ __attribute__((aligned(16))) f32x4_t red[NWV - 1][NA][64];
    if (w > 0) {
#pragma unroll
      for (int a = 0; a < NA; ++a) red[w - 1][a][lane] = acc[a];
    }
    __syncthreads();
    if (w > 0) return;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int j = 0; j < NWV - 1; ++j) acc[a] += red[j][a][lane];
  }

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
  } else if constexpr (EPI == EPI_RESIDUAL) {   // the residual was read ahead (y_pre)
    float *y = (float *)g.y + (int64_t)m * g.ldy + n;
    if (n + 3 < g.N && (g.ldy & 3) == 0) {
      store4(y, y_pre + acc[0]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < g.N) y[r] = y_pre[r] + acc[0][r];
    }
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
    const int pos = pos_pre;   // read ahead with the angles cs_pre of the lane's columns
    const bool ok = pos >= 0 && pos < g.cache_seq && pos < g.max_seq;
    if (!ok) g.pos_flag[0] = 1;
    f32x4_t v = acc[0];
    const int dh = g.d_head;
    if (n < g.n0) {   // q column: rotate, keep for the attention
      const float nan = __builtin_nanf("");
      v = ok ? rope4(v, cs_pre) : f32x4_t{nan, nan, nan, nan};
      store4((bf16_t *)g.y + (int64_t)m * g.ldy + n, v);
    } else if (ok) {  // k (rotated) or v column: into the cache slot of the position
      const bool is_k = n < g.n0 + g.n1;
      const int j = n - g.n0 - (is_k ? 0 : g.n1);
      if (is_k) v = rope4(v, cs_pre);
      const int grp = j / dh, d = j % dh;
      bf16_t *dst = (bf16_t *)(is_k ? g.k_cache : g.v_cache) +
                    (((int64_t)m * g.n_kv_heads + grp) * g.cache_seq + pos) * dh + d;
      store4(dst, v);
    }
  }
}

// Wide plain-store products (the LM head over the vocabulary): a workgroup of 4 waves owns 64
// output columns and each wave streams 16 of them over the whole K, U 32-wide k steps in
// flight. The block's activation rows (at most 16, `rows` of them held) are RMS-normalised
// once per workgroup into LDS (bf16, rows padded by 16 bytes so the 16 rows of a fragment read
// fall on distinct banks), instead of once per 16 columns. Row r is normalised by the 16
// consecutive lanes of threads 16 r .. 16 r + 15 (a DPP row), which sum its squares without
// LDS. Lanes of rows past `rows` read row rows - 1: their products are never stored.
constexpr int kWideCols = 64;
template <int U>
__global__ __launch_bounds__(256) void dgemv_wide_kernel(DecodeGemmArgs g, int rows) {
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  bf16_t *xs = (bf16_t *)dyn_lds;
  const int KP = g.K + 8;   // padded row pitch (elements)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, kc = lane >> 4;
  const int nb = blockIdx.x * kWideCols + w * 16;   // this wave's first output column
  const int m0 = blockIdx.y * 16;
  const int nks = (g.K + 31) / 32;
  const bool wok = nb + r16 < g.N;
  const bf16_t *wrow = (const bf16_t *)g.w0 + (int64_t)(wok ? nb + r16 : 0) * g.K;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  u32x4_t wa[U];
  auto load_w = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s0 + u) * 32 + kc * 8;
      wa[u] = wok && s0 + u < nks && k < g.K ? ld16(wrow + k) : zero;
    }
  };
  load_w(0);   // in flight while the activations are normalised

  // activations: thread t handles row t / 16 of the block, 4 columns of every 64
  {
    const int row = tid >> 4, part = tid & 15;
    const int m = m0 + row;
    bf16_t *dst = xs + row * KP;
    if (row >= rows) {
    } else if (g.norm_x) {
      const float *xr = g.norm_x + (int64_t)(m < g.M ? m : 0) * g.ldx;
      float ss = 0.f;
      for (int k = 4 * part; k < g.K; k += 64) {
        const f32x4_t v = m < g.M ? load4(xr + k) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
      }
      ss = group_sum<16>(ss);
      const float rinv = rsqrtf(ss / (float)g.K + g.eps);
      for (int k = 4 * part; k < g.K; k += 64) {
        const f32x4_t v = m < g.M ? load4(xr + k) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        const f32x4_t gg = load4((const bf16_t *)g.norm_g + k);
        const f32x4_t y = v * rinv * gg;
        *(u32x2_t *)(dst + k) = u32x2_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      }
    } else {
      const bf16_t *xr = (const bf16_t *)g.x + (int64_t)(m < g.M ? m : 0) * g.ldx;
      for (int k = 4 * part; k < g.K; k += 64)
        *(u32x2_t *)(dst + k) = m < g.M ? *(const u32x2_t *)(xr + k) : u32x2_t{0u, 0u};
    }
  }
  // LDS only: the weight loads stay in flight across this barrier
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const bf16_t *xrow = xs + min(r16, rows - 1) * KP + kc * 8;
  for (int s0 = 0; s0 < nks; s0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s0 + u) * 32;
      const u32x4_t xa = s0 + u < nks && k + kc * 8 < g.K ? *(const u32x4_t *)(xrow + k) : zero;
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wa[u]),
                                                   __builtin_bit_cast(bf16x8_t, xa), acc, 0, 0, 0);
    }
    if (s0 + U < nks) load_w(s0 + U);
  }
  // lane holds columns n .. n+3 of row m
  const int m = m0 + r16, n = nb + 4 * kc;
  if (m >= g.M) return;
  if (g.y_dt == DT_BF16) {
    bf16_t *y = (bf16_t *)g.y + (int64_t)m * g.ldy + n;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < g.N) y[r] = f32_to_bf16(acc[r]);
  } else {
    float *y = (float *)g.y + (int64_t)m * g.ldy + n;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < g.N) y[r] = acc[r];
  }
}

// ---- decode attention
// Workgroup = (split s, kv head grp, sequence b) with NWV waves; a wave takes 64-key chunks of
// the visible keys (chunk c covers keys t0 + 64 c ..), chunks s*cps .. (s+1)*cps - 1 of the
// split in steps of NWV. Loads are coalesced: with PPR = d_head / 8 pieces of 8 elements per
// row and RPI = 64 / PPR rows per 1 KB, load j of a chunk gives lane l piece l % PPR of key
// row RPI j + l / PPR. The lane's q piece (8 elements per head) sits in registers; the dot
// products are summed over the PPR lanes of a row, the chunk maximum over the row groups.
// Softmax is online over the wave's chunks (fp32, log2 domain); p . v accumulates per lane
// and is summed over the row groups once at the end. The waves' (max, sum, output) meet in
// LDS: with one split the workgroup writes the normalised output, otherwise a partial record
// per query head that dec_combine_kernel merges in split order.
constexpr int dec_regs(int dh, int g) { return 8 * g + dh + (dh / 8) * g + 8 * g + 24; }
constexpr int dec_waves(int dh, int g) {
  return dec_regs(dh, g) <= 128 ? 16 : dec_regs(dh, g) <= 256 ? 8 : 4;
}

template <int DH, int GM, int NWV>
__global__ __launch_bounds__(64 * NWV) void dec_attn_kernel(
    const bf16_t *__restrict__ q, int64_t q_stride, const bf16_t *__restrict__ kc,
    const bf16_t *__restrict__ vc, const int32_t *__restrict__ positions, int Hq, int Hkv,
    int cache_seq, int window, int cps, float scale_log2, float *__restrict__ part, int n_split,
    bf16_t *__restrict__ o, int64_t o_stride) {
  constexpr int PPR = DH / 8, RPI = 64 / PPR, NJ = PPR, PS = 2 + DH;
  const int split = blockIdx.x, grp = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int nwv = blockDim.x >> 6;   // waves of this launch, <= NWV
  const int pc = lane % PPR, rg = lane / PPR;
  const int64_t head = ((int64_t)b * Hkv + grp) * cache_seq;   // first row of this kv head
  // Full causal attention: the first chunk's rows do not depend on the position, so they are
  // requested before it is read (rows clamped into the cache; rows past the position are
  // masked below).
  // (Kernels with many registers per lane skip this: the early rows would spill.)
  const int c_first = split * cps + w;
  const bool pre = dec_regs(DH, GM) <= 200 && window == 0 && 64 * c_first < cache_seq;
  u32x4_t kr[NJ], vr[NJ];
  if (pre) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      kr[j] = ld16(kc + (head + min(64 * c_first + RPI * j + rg, cache_seq - 1)) * DH + 8 * pc);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      vr[j] = ld16(vc + (head + min(64 * c_first + RPI * j + rg, cache_seq - 1)) * DH + 8 * pc);
  }
  const int pos = positions[b];
  if (pos < 0 || pos >= cache_seq) {   // no cache slot: NaN output for the group's heads
    if (split == 0)
      for (int i = tid; i < G * DH; i += 64 * nwv)
        o[(int64_t)b * o_stride + (int64_t)grp * G * DH + i] = f32_to_bf16(__builtin_nanf(""));
    return;
  }
  const int n = pos + 1;
  const int t0 = window > 0 && n > window ? n - window : 0;
  const int nch = (n - t0 + 63) / 64;
  const int c_end = min((split + 1) * cps, nch);

  const u32x4_t zero = {0u, 0u, 0u, 0u};
  // this lane's q pieces (raw bf16); converted inside the loop, so the first chunk's K / V
  // loads are issued before anything waits on q
  u32x4_t qraw[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h)
    qraw[h] = h < G ? ld16(q + (int64_t)b * q_stride + (int64_t)(grp * G + h) * DH + 8 * pc) : zero;
  float m[GM], l[GM], acc[GM][8];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m[h] = -__builtin_inff();
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  for (int c = c_first; c < c_end; c += nwv) {
    const int k0 = t0 + 64 * c;
    // rows past the last visible key load that key again (no branch around the loads) and
    // are zeroed afterwards
    if (!(pre && c == c_first)) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        kr[j] = ld16(kc + (head + min(k0 + RPI * j + rg, n - 1)) * DH + 8 * pc);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        vr[j] = ld16(vc + (head + min(k0 + RPI * j + rg, n - 1)) * DH + 8 * pc);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (k0 + RPI * j + rg >= n) vr[j] = zero;
    // q is used after this chunk's loads are issued: the empty statement keeps its conversion
    // (and the wait for it) in the loop, below the loads
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < GM; ++h) asm volatile("" : "+v"(qraw[h]));
    float qf[GM][8];   // q pieces in log2 units
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[h][2 * e] = __uint_as_float(qraw[h][e] << 16) * scale_log2;
        qf[h][2 * e + 1] = __uint_as_float(qraw[h][e] & 0xffff0000u) * scale_log2;
      }
    // scores of the lane's rows, summed over the PPR lanes of each row
    float sc[NJ][GM];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      float kf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = __uint_as_float(kr[j][e] << 16);
        kf[2 * e + 1] = __uint_as_float(kr[j][e] & 0xffff0000u);
      }
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = __builtin_fmaf(qf[h][e], kf[e], d);
        d = group_sum<PPR>(d);
        sc[j][h] = k0 + RPI * j + rg < n ? d : -__builtin_inff();
      }
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      float mx = sc[0][h];
#pragma unroll
      for (int j = 1; j < NJ; ++j) mx = fmaxf(mx, sc[j][h]);
      mx = across_groups<PPR>(mx, [](float a, float b) { return fmaxf(a, b); });
      const float mn = fmaxf(m[h], mx);        // finite: the chunk has a visible key
      const float alpha = exp2f(m[h] - mn);    // 0 for the first chunk
      m[h] = mn;
      float ls = 0.f;
      float a8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a8[e] = acc[h][e] * alpha;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float p = exp2f(sc[j][h] - mn);
        ls += p;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a8[2 * e] = __builtin_fmaf(p, __uint_as_float(vr[j][e] << 16), a8[2 * e]);
          a8[2 * e + 1] = __builtin_fmaf(p, __uint_as_float(vr[j][e] & 0xffff0000u), a8[2 * e + 1]);
        }
      }
      l[h] = l[h] * alpha + ls;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = a8[e];
    }
  }
  // sums over the row groups (lanes with the same piece)
  const auto add = [](float a, float b) { return a + b; };
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    l[h] = across_groups<PPR>(l[h], add);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = across_groups<PPR>(acc[h][e], add);
  }

  __shared__ float wm[NWV][GM], wl[NWV][GM];
  __shared__ __attribute__((aligned(16))) float wo[NWV][GM][DH];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (lane == 0) {
      wm[w][h] = m[h];
      wl[w][h] = l[h];
    }
    if (rg == 0) {
      *(f32x4_t *)&wo[w][h][8 * pc] = f32x4_t{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
      *(f32x4_t *)&wo[w][h][8 * pc + 4] = f32x4_t{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
    }
  }
  __syncthreads();
  for (int i = tid; i < G * DH; i += 64 * nwv) {
    const int h = i / DH, d = i % DH;
    float M = -__builtin_inff();
    for (int v = 0; v < nwv; ++v) M = fmaxf(M, wm[v][h]);
    float L = 0.f, O = 0.f;
    if (M != -__builtin_inff()) {
      for (int v = 0; v < nwv; ++v) {
        const float f = exp2f(wm[v][h] - M);   // 0 for a wave without keys
        L += f * wl[v][h];
        O += f * wo[v][h][d];
      }
    }
    if (n_split == 1) {
      o[(int64_t)b * o_stride + (int64_t)(grp * G + h) * DH + d] = f32_to_bf16(O / L);
    } else {
      float *rec = part + (((int64_t)b * Hq + grp * G + h) * n_split + split) * PS;
      rec[2 + d] = O;
      if (d == 0) {
        rec[0] = M;
        rec[1] = L;
      }
    }
  }
}

// Merges the split records of one (sequence, query head) in split order; a split without
// visible keys holds (-inf, 0, 0). (A merge by the last workgroup would need device-scope
// fences, which write back the XCD's L2.)
template <int DH>
__global__ __launch_bounds__(128) void dec_combine_kernel(const float *__restrict__ part,
                                                          const int32_t *__restrict__ positions,
                                                          int Hq, int cache_seq, int n_split,
                                                          bf16_t *__restrict__ o,
                                                          int64_t o_stride) {
  constexpr int PS = 2 + DH;
  const int bh = blockIdx.x, b = bh / Hq, h = bh % Hq;
  const int pos = positions[b];
  if (pos < 0 || pos >= cache_seq) return;   // the attention kernel wrote the NaN row
  const float *rec = part + (int64_t)bh * n_split * PS;
  // split weights 2^(m_s - max) and the denominator, computed once in LDS
  __shared__ float wgt[kMaxSplits];
  __shared__ float den;
  for (int c = threadIdx.x; c < n_split; c += blockDim.x) wgt[c] = rec[c * PS];
  __syncthreads();
  if (threadIdx.x == 0) {
    float mx = -__builtin_inff();
    for (int c = 0; c < n_split; ++c) mx = fmaxf(mx, wgt[c]);
    float l = 0.f;
    for (int c = 0; c < n_split; ++c) {
      wgt[c] = exp2f(wgt[c] - mx);
      l += wgt[c] * rec[c * PS + 1];
    }
    den = l;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < DH; d += blockDim.x) {
    float num = 0.f;
#pragma unroll 4
    for (int c = 0; c < n_split; ++c) num += wgt[c] * rec[c * PS + 2 + d];
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

// Splits per (sequence, kv head) and waves per split: a split's waves take its 64-key chunks
// (at most NWV waves, each looping when a split has more chunks than waves).
template <int DH, int GM>
hipError_t run_dec_attn(const void *q, int64_t q_stride, const void *kc, const void *vc,
                        const int32_t *positions, int B, int Hq, int Hkv, int cache_seq,
                        int window, float *part, void *o, int64_t o_stride, hipStream_t s) {
  constexpr int NWV = dec_waves(DH, GM);
  const int span = window > 0 ? std::min(window, cache_seq) : cache_seq;
  const int chunks = (span + 63) / 64;
  const int64_t groups = (int64_t)B * Hkv;
  // Fewest splits that give every chunk a wave: a split costs the merge launch, which at the
  // d768 workload's 1001-key context outweighs what spreading the cache over more CUs gains
  // (measured: 96 workgroups 10.8 us; 768 workgroups 8.4 us + 3.7 us merge). More splits only
  // while the chunk waves are too few to keep the memory system busy.
  int n_split = (chunks + NWV - 1) / NWV;
  if (groups * chunks < kDecBusyWaves)
    n_split = (int)std::max<int64_t>(n_split, std::min<int64_t>(chunks, (kDecTargetGroups + groups - 1) / groups));
  n_split = std::min(n_split, decode_chunks(cache_seq));
  const int cps = (chunks + n_split - 1) / n_split;
  n_split = (chunks + cps - 1) / cps;
  const int waves = std::min(NWV, cps);
  const float sl2 = kLog2e / sqrtf((float)DH);
  dec_attn_kernel<DH, GM, NWV><<<dim3(n_split, Hkv, B), 64 * waves, 0, s>>>(
      (const bf16_t *)q, q_stride, (const bf16_t *)kc, (const bf16_t *)vc, positions, Hq, Hkv,
      cache_seq, window, cps, sl2, part, n_split, (bf16_t *)o, o_stride);
  if (n_split > 1)
    dec_combine_kernel<DH><<<B * Hq, 128, 0, s>>>(part, positions, Hq, cache_seq, n_split,
                                                  (bf16_t *)o, o_stride);
  return hipGetLastError();
}

template <int DH>
hipError_t run_dec_attn_g(const void *q, int64_t q_stride, const void *kc, const void *vc,
                          const int32_t *positions, int B, int Hq, int Hkv, int cache_seq,
                          int window, float *part, void *o, int64_t o_stride, hipStream_t s) {
  const int G = Hq / Hkv;
  if (G == 1)
    return run_dec_attn<DH, 1>(q, q_stride, kc, vc, positions, B, Hq, Hkv, cache_seq, window,
                               part, o, o_stride, s);
  if (G == 2)
    return run_dec_attn<DH, 2>(q, q_stride, kc, vc, positions, B, Hq, Hkv, cache_seq, window,
                               part, o, o_stride, s);
  if (G <= 4)
    return run_dec_attn<DH, 4>(q, q_stride, kc, vc, positions, B, Hq, Hkv, cache_seq, window,
                               part, o, o_stride, s);
  return run_dec_attn<DH, 8>(q, q_stride, kc, vc, positions, B, Hq, Hkv, cache_seq, window,
                             part, o, o_stride, s);
}

}  // namespace

int decode_chunks(int cache_seq) { return std::min(kMaxSplits, (cache_seq + 63) / 64); }

hipError_t noalloc_scratch(hipStream_t stream, float **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float *addr[kMaxDevices] = {};
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // the symbol's address on `dev`, looked up with that device current
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = (float *)p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}
int decode_max_cache() { return kDecMaxCache; }
bool decode_group_supported(int Hq, int Hkv) { return Hq % Hkv == 0 && Hq / Hkv <= kDecMaxGroup; }

template <int NWV, int U>
hipError_t run_dgemm(int epi, const DecodeGemmArgs &g, dim3 grid, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: dgemm_kernel<EPI_STORE, NWV, U><<<grid, 64 * NWV, 0, s>>>(g); break;
    case EPI_RESIDUAL: dgemm_kernel<EPI_RESIDUAL, NWV, U><<<grid, 64 * NWV, 0, s>>>(g); break;
    case EPI_SWIGLU: dgemm_kernel<EPI_SWIGLU, NWV, U><<<grid, 64 * NWV, 0, s>>>(g); break;
    case EPI_QKV_CACHE: dgemm_kernel<EPI_QKV_CACHE, NWV, U><<<grid, 64 * NWV, 0, s>>>(g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_gemm(int epi, const DecodeGemmArgs &g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  const int cols = epi == EPI_SWIGLU ? g.n0 : g.N;
  const dim3 grid(grid1(cols, 16), grid1(g.M, 16));
  if (grid.y > 65535) return hipErrorInvalidValue;
  // Few column blocks (the layers' projections): 8 waves split K with 4 or 8 steps each in
  // flight, so one round of loads covers K <= 2048 on the few CUs that have work. Many blocks
  // (the LM head) fill the chip anyway: 4 waves with 4 steps each keep the registers, and so
  // the occupancy, of a streaming kernel.
  if ((int64_t)grid.x * grid.y >= 1024) {
    // plain stores over many columns (the LM head): the wide kernel when the block's
    // activation rows fit in 64 KB of LDS
    const int rows = g.M < 16 ? g.M : 16;
    const size_t lds = (size_t)rows * (g.K + 8) * 2;
    if (epi == EPI_STORE && g.K % 8 == 0 && lds <= 65536) {
      const dim3 gw(grid1(g.N, kWideCols), grid1(g.M, 16));
      dgemv_wide_kernel<8><<<gw, 256, lds, s>>>(g, rows);
      return hipGetLastError();
    }
    return run_dgemm<4, 4>(epi, g, grid, s);
  }
  // 4 steps per wave when they cover K (K <= 1024): fewer registers held for steps past K
  if (g.K <= 8 * 4 * 32) return run_dgemm<8, 4>(epi, g, grid, s);
  return run_dgemm<8, 8>(epi, g, grid, s);
}

hipError_t launch_decode_attention(const void *q, int64_t q_stride, const void *k_cache,
                                   const void *v_cache, const int32_t *positions, int B, int Hq,
                                   int Hkv, int d_head, int cache_seq, int window, float *part,
                                   void *o, int64_t o_stride, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (B > 65535 || Hkv > 65535) return hipErrorInvalidValue;
  switch (d_head) {
    case 32: return run_dec_attn_g<32>(q, q_stride, k_cache, v_cache, positions, B, Hq, Hkv,
                                     cache_seq, window, part, o, o_stride, s);
    case 64: return run_dec_attn_g<64>(q, q_stride, k_cache, v_cache, positions, B, Hq, Hkv,
                                     cache_seq, window, part, o, o_stride, s);
    case 128: return run_dec_attn_g<128>(q, q_stride, k_cache, v_cache, positions, B, Hq, Hkv,
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

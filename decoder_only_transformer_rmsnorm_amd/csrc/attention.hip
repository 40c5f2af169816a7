// Causal multi-head attention with grouped KV heads, flash-style (one pass over the keys
// with an online softmax), on the CDNA4 matrix cores.
//
// What it computes ("Transformer 篇" (dujian.net) 5.4 Attention; "Transformer篇"
// (fengye404.top) 8 Attention; "LLM 2" GQA/MQA): for every (b, query head h, query s),
//   o = sum_{t <= s} softmax_t(q_s . k_t / sqrt(d_head)) v_t,  KV head g = h / (Hq / Hkv).
// Keys after s get weight exactly 0 (they are never added); masking is by token order.
//
// bf16 kernel (d_head in {32, 64, 128}):
//  * A workgroup owns 128 queries of one (b, h): 4 waves x 32 queries. K/V tiles of 64
//    keys are staged in LDS (double-buffered, next tile's global loads in flight during
//    the current tile's math) and shared by the 4 waves.
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16, K rows as the
//    A operand, Q held in registers as the B operand), so each lane holds 16 keys of ONE
//    query: the running row max needs one cross-lane exchange (lane l <-> l^32) per tile
//    and the row sum none until the end.
//  * O^T = V^T P^T: the bf16-rounded probabilities go straight from the score accumulator
//    into the B operand (no shuffle). V is written into LDS transposed, with the keys of
//    each 16-key group permuted so that the 8 keys a lane needs are contiguous.
//  * Softmax state (max, sum, rescale) is fp32; exponentials are base 2 with the
//    1/sqrt(d_head) * log2(e) factor folded into one multiply.
//  * Tiles entirely above the diagonal are never loaded; per wave, tiles past its last
//    query are skipped; only the diagonal tile is masked. Query tiles are issued
//    longest-first to even out the causal imbalance.
// f32 kernel (d_head in {16, 32, 64, 128}): one thread per query with the same online
// softmax in fp32; it exists for the small fp32 model and for tests, not for speed.
#include "common.h"
#include "internal.h"

namespace tfm {
namespace {

constexpr int kBQ = 128;   // queries per workgroup
constexpr int kBKV = 64;   // keys per tile
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

// 16-byte chunk swizzle for an LDS tile whose rows are `RB` bytes: keeps the rows that one
// 8-lane phase of a 16-byte-per-lane read touches on distinct bank groups.
template <int RB>
__device__ __forceinline__ int swz_chunk(int row, int ch) {
  if constexpr (RB >= 128) {
    return ch ^ (row & 7);
  } else {
    constexpr int rows_per_128 = 128 / RB, cpr = RB / 16;
    return ch ^ ((row / rows_per_128) & (cpr - 1));
  }
}

// Position of key t (0..63 within the tile) in a transposed V row: inside each group of
// 16 keys, keys {4c+j} for c in 0..3 map so that a lane of half h reads keys
// {8e'+4h+j : e' in 0..1, j in 0..3} as one contiguous run of 8.
__device__ __forceinline__ int vt_pos(int t) {
  const int k16 = t & 15;
  return (t & ~15) + 8 * ((k16 >> 2) & 1) + 4 * (k16 >> 3) + (k16 & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DH>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(
    const bf16_t *__restrict__ q, int64_t q_stride, const bf16_t *__restrict__ k,
    const bf16_t *__restrict__ v, int64_t kv_stride, bf16_t *__restrict__ o, int64_t o_stride,
    int B, int S, int Hq, int Hkv, int n_qt, float scale_log2) {
  constexpr int KRB = DH * 2;                 // K tile row bytes
  constexpr int KCPR = DH / 8;                // K chunks per row
  constexpr int K_LD = kBKV * KCPR / kThreads;// K chunks per thread
  constexpr int VRB = kBKV * 2;               // V^T tile row bytes (128)
  constexpr int V_UNITS = (kBKV / 2) * (DH / 8);  // (2 keys x 8 dims) units per tile
  constexpr int K_BYTES = kBKV * KRB, V_BYTES = DH * VRB;
  constexpr int STAGE = K_BYTES + V_BYTES;
  constexpr int NKB = kBKV / 32;              // 32-key score blocks per tile
  constexpr int NDB = DH / 32;                // 32-dim output blocks
  constexpr int QK_STEPS = DH / 16;           // k-steps of the score MFMA
  constexpr int PV_STEPS = kBKV / 16;         // k-steps of the PV MFMA
  constexpr int K_PER_T = K_LD > 0 ? K_LD : 1;
  constexpr int V_PER_T = (V_UNITS + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int bh_count = B * Hq;
  const int qt = n_qt - 1 - (int)(blockIdx.x / bh_count);   // longest first
  const int bh = (int)(blockIdx.x % bh_count);
  const int b = bh / Hq, hq = bh % Hq, hkv = hq / (Hq / Hkv);
  const int q0 = qt * kBQ, qw0 = q0 + wid * 32;

  const bf16_t *kbase = k + (int64_t)b * S * kv_stride + (int64_t)hkv * DH;
  const bf16_t *vbase = v + (int64_t)b * S * kv_stride + (int64_t)hkv * DH;

  // ---- Q fragments (B operand of S^T = K Q^T): query qw0 + l32, dims 16*kk + 8h .. +7
  uint4 qf[QK_STEPS];
  {
    const int qi = qw0 + l32;
    const bf16_t *qp = q + ((int64_t)b * S + (qi < S ? qi : 0)) * q_stride + (int64_t)hq * DH;
#pragma unroll
    for (int kk = 0; kk < QK_STEPS; ++kk)
      qf[kk] = qi < S ? *(const uint4 *)(qp + 16 * kk + 8 * h) : uint4{0u, 0u, 0u, 0u};
  }

  const int kv_end = min(q0 + kBQ, S);
  const int n_tiles = (kv_end + kBKV - 1) / kBKV;

  uint4 rk[K_PER_T];
  uint4 rv[V_PER_T][2];
  auto gload = [&](int j) {
    const int kv0 = j * kBKV;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / KCPR, ch = c % KCPR;
      const bool ok = (K_LD > 0 || c < kBKV * KCPR) && kv0 + row < S;
      rk[i] = ok ? *(const uint4 *)(kbase + (int64_t)(kv0 + row) * kv_stride + ch * 8)
                 : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + kThreads * i;
      const int kp = u / (DH / 8), dc = u % (DH / 8);   // key pair, 8-dim column
      const int t0 = kv0 + 2 * kp;
      const bool ok = u < V_UNITS;
      rv[i][0] = (ok && t0 < S) ? *(const uint4 *)(vbase + (int64_t)t0 * kv_stride + dc * 8)
                                : uint4{0u, 0u, 0u, 0u};
      rv[i][1] = (ok && t0 + 1 < S)
                     ? *(const uint4 *)(vbase + (int64_t)(t0 + 1) * kv_stride + dc * 8)
                     : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
    uint8_t *Ks = lds + buf * STAGE;
    uint8_t *Vt = Ks + K_BYTES;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + kThreads * i;
      if (K_LD > 0 || c < kBKV * KCPR) {
        const int row = c / KCPR, ch = c % KCPR;
        *(uint4 *)(Ks + row * KRB + (swz_chunk<KRB>(row, ch) << 4)) = rk[i];
      }
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + kThreads * i;
      if (u < V_UNITS) {
        const int kp = u / (DH / 8), dc = u % (DH / 8);
        const int col = vt_pos(2 * kp);               // even; key 2kp+1 sits at col + 1
        const uint32_t *a = (const uint32_t *)&rv[i][0];
        const uint32_t *bb = (const uint32_t *)&rv[i][1];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = dc * 8 + e;
          const uint32_t lo = (e & 1) ? (a[e >> 1] >> 16) : (a[e >> 1] & 0xffffu);
          const uint32_t hi = (e & 1) ? (bb[e >> 1] >> 16) : (bb[e >> 1] & 0xffffu);
          const int off = d * VRB + (swz_chunk<VRB>(d, col >> 3) << 4) + (col & 7) * 2;
          *(uint32_t *)(Vt + off) = lo | (hi << 16);
        }
      }
    }
  };

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_run = -__builtin_inff(), l_run = 0.f;
  const int my_q = qw0 + l32;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) gload(j + 1);
    const int kv0 = j * kBKV;
    if (kv0 <= qw0 + 31) {
      const uint8_t *Ks = lds + buf * STAGE;
      const uint8_t *Vt = Ks + K_BYTES;
      f32x16_t sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
        const int row = kb * 32 + l32;
#pragma unroll
        for (int kk = 0; kk < QK_STEPS; ++kk) {
          const uint4 a = *(const uint4 *)(Ks + row * KRB + (swz_chunk<KRB>(row, 2 * kk + h) << 4));
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, qf[kk]), sacc[kb], 0, 0, 0);
        }
      }
      // scores in log2 units; mask keys after the query on the diagonal tile
      const bool diag = kv0 + kBKV - 1 > qw0;
      float mt = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float s = sacc[kb][e] * scale_log2;
          if (diag) {
            const int key = kv0 + kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
            if (key > my_q) s = -__builtin_inff();
          }
          sacc[kb][e] = s;
          mt = fmaxf(mt, s);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
      const float m_new = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      float ls = 0.f;
      uint4 pf[PV_STEPS];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(sacc[kb][e] - m_new);
          sacc[kb][e] = p;
          ls += p;
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint32_t w[4];
#pragma unroll
          for (int x = 0; x < 4; ++x)
            w[x] = pack_bf16x2(sacc[kb][8 * half + 2 * x], sacc[kb][8 * half + 2 * x + 1]);
          pf[2 * kb + half] = uint4{w[0], w[1], w[2], w[3]};
        }
      }
      l_run = l_run * alpha + ls;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        oacc[db] *= alpha;
        const int row = db * 32 + l32;
#pragma unroll
        for (int kk = 0; kk < PV_STEPS; ++kk) {
          const uint4 a = *(const uint4 *)(Vt + row * VRB + (swz_chunk<VRB>(row, 2 * kk + h) << 4));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, pf[kk]), oacc[db], 0, 0, 0);
        }
      }
    }
    if (j + 1 < n_tiles) sstore(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (my_q < S) {
    const float inv = 1.0f / l_tot;
    bf16_t *op = o + ((int64_t)b * S + my_q) * o_stride + (int64_t)hq * DH;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t r;
#pragma unroll
        for (int x = 0; x < 4; ++x) r[x] = oacc[db][4 * g + x] * inv;
        store4(op + 32 * db + 8 * g + 4 * h, r);
      }
  }
}

template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float *__restrict__ q, int64_t q_stride,
                                                      const float *__restrict__ k,
                                                      const float *__restrict__ v, int64_t kv_stride,
                                                      float *__restrict__ o, int64_t o_stride, int B,
                                                      int S, int Hq, int Hkv, float scale) {
  const int s = blockIdx.x * 64 + threadIdx.x;
  const int hq = blockIdx.y, b = blockIdx.z;
  if (s >= S) return;
  const int hkv = hq / (Hq / Hkv);
  float qv[DH], acc[DH];
  const float *qp = q + ((int64_t)b * S + s) * q_stride + (int64_t)hq * DH;
#pragma unroll
  for (int e = 0; e < DH; ++e) { qv[e] = qp[e] * scale; acc[e] = 0.f; }
  float m = -__builtin_inff(), l = 0.f;
  for (int t = 0; t <= s; ++t) {
    const float *kp = k + ((int64_t)b * S + t) * kv_stride + (int64_t)hkv * DH;
    const float *vp = v + ((int64_t)b * S + t) * kv_stride + (int64_t)hkv * DH;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < DH; ++e) dot = fmaf(qv[e], kp[e], dot);
    const float m_new = fmaxf(m, dot);
    const float alpha = expf(m - m_new), p = expf(dot - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < DH; ++e) acc[e] = acc[e] * alpha + p * vp[e];
    m = m_new;
  }
  float *op = o + ((int64_t)b * S + s) * o_stride + (int64_t)hq * DH;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < DH; ++e) op[e] = acc[e] * inv;
}

template <int DH>
hipError_t run_bf16(const void *q, int64_t qs, const void *k, const void *v, int64_t kvs, void *o,
                    int64_t os, int B, int S, int Hq, int Hkv, hipStream_t st) {
  const int n_qt = (S + kBQ - 1) / kBQ;
  const int64_t blocks = (int64_t)n_qt * B * Hq;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const float sl2 = kLog2e / sqrtf((float)DH);
  attn_bf16_kernel<DH><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
      (const bf16_t *)q, qs, (const bf16_t *)k, (const bf16_t *)v, kvs, (bf16_t *)o, os, B, S, Hq,
      Hkv, n_qt, sl2);
  return hipGetLastError();
}

template <int DH>
hipError_t run_f32(const void *q, int64_t qs, const void *k, const void *v, int64_t kvs, void *o,
                   int64_t os, int B, int S, int Hq, int Hkv, hipStream_t st) {
  if ((int64_t)B * S * Hq == 0) return hipSuccess;
  if (B > 65535 || Hq > 65535) return hipErrorInvalidValue;
  dim3 grid((S + 63) / 64, Hq, B);
  attn_f32_kernel<DH><<<grid, dim3(64), 0, st>>>((const float *)q, qs, (const float *)k,
                                                 (const float *)v, kvs, (float *)o, os, B, S, Hq,
                                                 Hkv, 1.0f / sqrtf((float)DH));
  return hipGetLastError();
}

}  // namespace

bool attention_supported(int dt, int d_head) {
  if (dt == DT_BF16) return d_head == 32 || d_head == 64 || d_head == 128;
  return d_head == 16 || d_head == 32 || d_head == 64 || d_head == 128;
}

hipError_t launch_attention(const void *q, int64_t q_stride, const void *k, const void *v,
                            int64_t kv_stride, void *o, int64_t o_stride, int B, int S, int Hq,
                            int Hkv, int d_head, int dt, hipStream_t s) {
  if (dt == DT_BF16) {
    switch (d_head) {
      case 32: return run_bf16<32>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, s);
      case 64: return run_bf16<64>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, s);
      case 128: return run_bf16<128>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, s);
    }
  } else {
    switch (d_head) {
      case 16: return run_f32<16>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, s);
      case 32: return run_f32<32>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, s);
      case 64: return run_f32<64>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, s);
      case 128: return run_f32<128>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace tfm

// Backward of causal (and sliding-window) attention with grouped KV heads on the CDNA4
// matrix cores, flash style: the score matrix is recomputed tile by tile from q, k and each
// query row's logsumexp kept by the forward, never stored ("LLM 2: Transformer 原理与实现",
// Optimize; the chain rule through "Transformer 篇" (dujian.net) 5.4 Attention).
//
// With s = q k^T / sqrt(d), P = exp(s - lse) and D = rowsum(dO * O) per query row:
//   dP = dO V^T,  dS = P * (dP - D),  dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),  dV = P^T dO.
//
// Two kernels, each owning 128 rows (4 waves x 32) of one head and streaming the other side in
// tiles of 64 rows through LDS (plain loads staged through registers, so the next tile's
// loads overlap the current tile's math):
//  * attn_dq_mfma_kernel owns queries: S^T = K Q^T and dP^T = V dO^T (v_mfma_f32_32x32x16_bf16,
//    K and V rows as A operands, the wave's q and dO held in registers as B operands) give each
//    lane 16 keys of ONE query, so lse and D are per-lane scalars. dQ^T += K^T dS^T takes dS^T
//    straight from the accumulators as the B operand (bf16) and K^T fragments from the LDS
//    transpose read (ds_read_b64_tr_b16, four consecutive keys of one dimension per lane).
//    It also writes D for the other kernel.
//  * attn_dkdv_mfma_kernel owns keys: S = Q K^T and dP = dO V^T give each lane 16 queries of
//    ONE key; dV^T += dO^T P and dK^T += Q^T dS the same way, over the query heads of the
//    group (grouped-query attention sums their contributions to the shared k and v).
// In both, the contraction index of the second product is taken in the order the
// accumulator holds it ({4h..4h+3, 4h+8..4h+11} per 16 for lane half h), and the transpose
// read fetches the same rows, so no shuffle is needed. P and dS are rounded to bf16 for the
// second products; everything else accumulates in fp32.
#include <cmath>

#include "common.h"
#include "internal.h"

namespace tfm {
namespace {

constexpr int kRows = 128;   // rows a workgroup owns (4 waves x 32)
constexpr int kTile = 64;    // rows of a streamed tile
constexpr float kLog2eB = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(4))) short v4s_t;
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

// LDS tile of kTile rows x DH bf16: 16-byte chunk c of row r sits at chunk c ^ (r % CPR).
template <int DH>
struct BTile {
  static constexpr int RB = DH * 2, CPR = DH / 8;
  static constexpr int BYTES = kTile * RB;
  static constexpr int CH = kTile * CPR / 256;   // 16-byte chunks per thread per tile
  static_assert(CH >= 1 && CH * 256 == kTile * CPR, "tile / thread mismatch");
  __device__ static int off(int r, int c) { return r * RB + ((c ^ (r & (CPR - 1))) << 4); }
};

// A operand (32 rows x 16 k) of rows r0 .. r0+31 (lane l: row r0 + l % 32), k = dims
// 16 kk + 8 h .. +7, read as one 16-byte chunk.
template <int DH>
__device__ __forceinline__ u32x4_t frag_rows(const uint8_t *t, int r0, int kk, int lane) {
  const int r = r0 + (lane & 31), c = 2 * kk + (lane >> 5);
  return *(const u32x4_t *)(t + BTile<DH>::off(r, c));
}

// A operand of X^T for dims 32 db .. +31 and rows 16 ks .. +15 of the tile X (lane l: dim
// 32 db + l % 32; k = the rows {4h..4h+3, 4h+8..4h+11} + 16 ks, h = l / 32), from two
// transpose reads: lane (g = l / 16, i = l % 16) addresses row 16 ks + 4 (g / 2) + 8 half +
// i / 4, dims d0 + 4 (i % 4) .. +3 with d0 = 32 db + 16 (g % 2), and receives the four rows
// of dim d0 + i.
template <int DH>
__device__ __forceinline__ u32x4_t frag_tr(const uint8_t *t, int db, int ks, int lane) {
  const int g = lane >> 4, i = lane & 15;
  u32x2_t part[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int r = 16 * ks + 4 * (g >> 1) + 8 * half + (i >> 2);
    const int d = 32 * db + 16 * (g & 1) + 4 * (i & 3);
    const int byte = BTile<DH>::off(r, d >> 3) + 2 * (d & 7);
    const v4s_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t *)(t + byte));
    part[half] = __builtin_bit_cast(u32x2_t, v);
  }
  return u32x4_t{part[0][0], part[0][1], part[1][0], part[1][1]};
}

// B operand of the second product from a 32x32 accumulator pair: 16 rows of the contraction
// index per step ks (elements 8 (ks % 2) .. +7 of block ks / 2), rounded to bf16.
__device__ __forceinline__ u32x4_t pack_step(const f32x16_t &a, int half) {
  u32x4_t w;
#pragma unroll
  for (int x = 0; x < 4; ++x) w[x] = pack_bf16x2(a[8 * half + 2 * x], a[8 * half + 2 * x + 1]);
  return w;
}

__device__ __forceinline__ u32x4_t ldg16(const bf16_t *p) { return *(const u32x4_t *)p; }

// Cooperative tile load: rows row0 .. row0+63 of a (rows, ld) bf16 matrix at column col0,
// DH columns; rows at or past `rows_end` are zero. Thread t takes chunks t + 256 x.
template <int DH>
struct TileLoader {
  u32x4_t v[BTile<DH>::CH];
  __device__ void load(const bf16_t *base, int64_t ld, int64_t row0, int valid, int tid) {
    constexpr int CPR = BTile<DH>::CPR;
#pragma unroll
    for (int x = 0; x < BTile<DH>::CH; ++x) {
      const int idx = tid + 256 * x, r = idx / CPR, c = idx % CPR;
      v[x] = r < valid ? ldg16(base + (row0 + r) * ld + 8 * c) : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  __device__ void store(uint8_t *t, int tid) const {
    constexpr int CPR = BTile<DH>::CPR;
#pragma unroll
    for (int x = 0; x < BTile<DH>::CH; ++x) {
      const int idx = tid + 256 * x, r = idx / CPR, c = idx % CPR;
      *(u32x4_t *)(t + BTile<DH>::off(r, c)) = v[x];
    }
  }
};

// Work item of block `bid` in a grid of `n` blocks: rounds of `cus` blocks (one per CU when
// the grid is dispatched in order) alternate direction, so a CU's blocks of successive rounds
// take items from the long and the short end of the longest-first order.
__device__ __forceinline__ int snake_item(int bid, int n, int cus) {
  const int round = bid / cus, in_round = bid % cus;
  const int item = (round & 1) ? round * cus + (cus - 1 - in_round) : bid;
  return item < n ? item : bid;   // partial last round: keep in order
}

// The backward of RoPE: the (cos, sin) pairs of a row's position, or null without a table or
// for a position outside it (the gradient then stays unrotated) ...
template <int DH>
__device__ __forceinline__ const float *rope_row(const float *cs, int p, int max_seq) {
  return cs && p >= 0 && p < max_seq ? cs + (int64_t)p * DH : nullptr;
}
// ... and two adjacent pairs (v0, v1), (v2, v3) rotated by the opposite angles, with
// c = (cos0, sin0, cos1, sin1)
__device__ __forceinline__ f32x4_t rope_back4(f32x4_t v, const float *c) {
  const f32x4_t t = *(const f32x4_t *)c;
  return f32x4_t{v[0] * t[0] + v[1] * t[1], v[1] * t[0] - v[0] * t[1],
                 v[2] * t[2] + v[3] * t[3], v[3] * t[2] - v[2] * t[3]};
}

// ---------------------------------------------------------------- dQ (and D)
// grid ceil(S / 128) * Hq * B, query tiles longest first (the last tile sees every key)
template <int DH>
__global__ __launch_bounds__(256, DH >= 128 ? 1 : 2) void attn_dq_mfma_kernel(
    const bf16_t *__restrict__ qkv, int64_t ld, const bf16_t *__restrict__ o, int64_t ldo,
    const bf16_t *__restrict__ dout, int64_t lddo, bf16_t *__restrict__ dqkv, int S, int Hq,
    int Hkv, int window, float scale, const float *__restrict__ lse_in,
    float *__restrict__ dsum_out, int B, int cus, const int32_t *__restrict__ pos,
    const float *__restrict__ cs, int max_seq) {
  constexpr int KS = DH / 16, NDB = DH / 32;
  using TL = BTile<DH>;
  __shared__ __attribute__((aligned(16))) uint8_t kt[TL::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vt[TL::BYTES];
  const int qd = Hq * DH, kvd = Hkv * DH;
  const int nqt = (S + kRows - 1) / kRows;
  const int item = snake_item((int)blockIdx.x, (int)gridDim.x, cus);
  const int hq = (item % (Hq * B)) % Hq, b = (item % (Hq * B)) / Hq, g = hq / (Hq / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int q0 = (nqt - 1 - item / (Hq * B)) * kRows, qw0 = q0 + 32 * w;
  const int my_q = qw0 + l32;
  const bool live = my_q < S;
  const int64_t rq = (int64_t)b * S + (live ? my_q : S - 1);
  const float sl2 = scale * kLog2eB;

  // B operands: q and dO of this lane's query, dims 16 kk + 8 h .. +7; D = rowsum(dO * O)
  u32x4_t qf[KS], df[KS];
  float dpart = 0.f;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const int d0 = 16 * kk + 8 * h;
    qf[kk] = ldg16(qkv + rq * ld + (int64_t)hq * DH + d0);
    df[kk] = ldg16(dout + rq * lddo + (int64_t)hq * DH + d0);
    const u32x4_t of = ldg16(o + rq * ldo + (int64_t)hq * DH + d0);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      dpart += __uint_as_float(df[kk][x] << 16) * __uint_as_float(of[x] << 16);
      dpart += __uint_as_float(df[kk][x] & 0xffff0000u) * __uint_as_float(of[x] & 0xffff0000u);
    }
  }
  const float dsum = dpart + __shfl_xor(dpart, 32);
  if (live && h == 0) dsum_out[rq * Hq + hq] = dsum;
  const float lse2 = lse_in[rq * Hq + hq] * kLog2eB;

  f32x16_t dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[db][e] = 0.f;

  const int kv_end = min(q0 + kRows, S);
  const int n_tiles = (kv_end + kTile - 1) / kTile;
  const int j_lo = window > 0 ? max(0, q0 - window + 1) / kTile : 0;
  const bf16_t *kbase = qkv + (int64_t)b * S * ld + qd + (int64_t)g * DH;
  const bf16_t *vbase = kbase + kvd;
  TileLoader<DH> lk, lv;
  lk.load(kbase, ld, (int64_t)j_lo * kTile, S - j_lo * kTile, tid);
  lv.load(vbase, ld, (int64_t)j_lo * kTile, S - j_lo * kTile, tid);
  for (int j = j_lo; j < n_tiles; ++j) {
    __syncthreads();   // every wave is done with the previous tile
    lk.store(kt, tid);
    lv.store(vt, tid);
    __syncthreads();
    if (j + 1 < n_tiles) {
      lk.load(kbase, ld, (int64_t)(j + 1) * kTile, S - (j + 1) * kTile, tid);
      lv.load(vbase, ld, (int64_t)(j + 1) * kTile, S - (j + 1) * kTile, tid);
    }
    const int kv0 = j * kTile;
    if (kv0 > qw0 + 31) continue;                                        // keys after the wave
    if (window > 0 && kv0 + kTile - 1 < qw0 - window + 1) continue;      // keys too old
    // S^T and dP^T: lane = query, 16 keys per 32-key block
    f32x16_t sa[2], pa[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sa[kb][e] = pa[kb][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const u32x4_t ka = frag_rows<DH>(kt, 32 * kb, kk, lane);
        const u32x4_t va = frag_rows<DH>(vt, 32 * kb, kk, lane);
        sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ka),
                                                         __builtin_bit_cast(bf16x8_t, qf[kk]),
                                                         sa[kb], 0, 0, 0);
        pa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                         __builtin_bit_cast(bf16x8_t, df[kk]),
                                                         pa[kb], 0, 0, 0);
      }
    }
    // dS^T = P^T (dP^T - D), P = 2^(s sl2 - lse log2 e); invisible keys get 0
    const bool edge = kv0 + kTile - 1 > qw0 ||
                      (window > 0 && kv0 < qw0 + 31 - window + 1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kv0 + 32 * kb + 8 * (e >> 2) + 4 * h + (e & 3);
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[kb][e], sl2, -lse2));
        if (edge && (key > my_q || (window > 0 && key < my_q - window + 1))) p = 0.f;
        sa[kb][e] = p * (pa[kb][e] - dsum);
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int ks = 0; ks < kTile / 16; ++ks) {
      const u32x4_t bs = pack_step(sa[ks >> 1], ks & 1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const u32x4_t a = frag_tr<DH>(kt, db, ks, lane);
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                         __builtin_bit_cast(bf16x8_t, bs), dq[db],
                                                         0, 0, 0);
      }
    }
  }
  if (live) {
    bf16_t *op = dqkv + rq * ld + (int64_t)hq * DH;
    const int p = pos ? pos[rq] : my_q;
    const float *csr = rope_row<DH>(cs, p, max_seq);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        f32x4_t r;
#pragma unroll
        for (int x = 0; x < 4; ++x) r[x] = dq[db][4 * gq + x] * scale;
        if (csr) r = rope_back4(r, csr + 32 * db + 8 * gq + 4 * h);
        store4(op + 32 * db + 8 * gq + 4 * h, r);
      }
  }
}

// ---------------------------------------------------------------- dK, dV
// grid ceil(S / 128) * Hkv * B, key tiles longest first (the first tile is seen by every
// query); loops over the query heads of the group
template <int DH>
__global__ __launch_bounds__(256, DH >= 128 ? 1 : 2) void attn_dkdv_mfma_kernel(
    const bf16_t *__restrict__ qkv, int64_t ld, const bf16_t *__restrict__ dout, int64_t lddo,
    bf16_t *__restrict__ dqkv, int S, int Hq, int Hkv, int window, float scale,
    const float *__restrict__ lse_in, const float *__restrict__ dsum_in, int B, int cus,
    const int32_t *__restrict__ pos, const float *__restrict__ cs, int max_seq) {
  constexpr int KS = DH / 16, NDB = DH / 32;
  using TL = BTile<DH>;
  __shared__ __attribute__((aligned(16))) uint8_t qt[TL::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t ot[TL::BYTES];
  __shared__ __attribute__((aligned(16))) float ls[kTile], dsm[kTile];
  const int qd = Hq * DH, kvd = Hkv * DH, G = Hq / Hkv;
  const int item = snake_item((int)blockIdx.x, (int)gridDim.x, cus);
  const int g = (item % (Hkv * B)) % Hkv, b = (item % (Hkv * B)) / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int k0 = (item / (Hkv * B)) * kRows, kw0 = k0 + 32 * w;
  const int my_k = kw0 + l32;
  const bool live = my_k < S;
  const int64_t rk = (int64_t)b * S + (live ? my_k : S - 1);
  const float sl2 = scale * kLog2eB;

  // B operands: k and v of this lane's key, dims 16 kk + 8 h .. +7
  u32x4_t kf[KS], vf[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    kf[kk] = ldg16(qkv + rk * ld + qd + (int64_t)g * DH + 16 * kk + 8 * h);
    vf[kk] = ldg16(qkv + rk * ld + qd + kvd + (int64_t)g * DH + 16 * kk + 8 * h);
  }
  f32x16_t dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[db][e] = dv[db][e] = 0.f;

  const int k_last = min(k0 + kRows, S) - 1;
  const int i_lo = k0 / kTile;
  const int i_hi = (window > 0 ? min(S - 1, k_last + window - 1) : S - 1) / kTile;
  const int n_it = i_hi - i_lo + 1;   // query tiles per head
  const int total = G * n_it;
  TileLoader<DH> lq, lo;
  float lsv = 0.f, dsv = 0.f;
  auto fetch = [&](int it) {
    const int hh = it / n_it, i0 = (i_lo + it % n_it) * kTile;
    const int hq = g * G + hh;
    const int64_t r0 = (int64_t)b * S + i0;
    lq.load(qkv + (int64_t)hq * DH, ld, r0, S - i0, tid);
    lo.load(dout + (int64_t)hq * DH, lddo, r0, S - i0, tid);
    if (tid < kTile) {
      const bool ok = i0 + tid < S;
      lsv = ok ? lse_in[(r0 + tid) * Hq + hq] * kLog2eB : 0.f;
      dsv = ok ? dsum_in[(r0 + tid) * Hq + hq] : 0.f;
    }
  };
  fetch(0);
  for (int it = 0; it < total; ++it) {
    __syncthreads();
    lq.store(qt, tid);
    lo.store(ot, tid);
    if (tid < kTile) {
      ls[tid] = lsv;
      dsm[tid] = dsv;
    }
    __syncthreads();
    if (it + 1 < total) fetch(it + 1);
    const int i0 = (i_lo + it % n_it) * kTile;
    if (i0 + kTile - 1 < kw0) continue;                                  // queries before keys
    if (window > 0 && i0 > kw0 + 31 + window - 1) continue;              // keys too old for all
    // per 32-query block qb: S and dP (lane = key, 16 queries), then P and dS = P (dP - D)
    // (queries that do not see this key, or past S, get 0), then dV^T += dO^T P and
    // dK^T += Q^T dS over the block's 32 queries; one block at a time keeps the registers
    // of a single pair of score accumulators
    const bool edge = i0 < kw0 + 31 || (window > 0 && i0 + kTile - 1 > kw0 - 1 + window - 1) ||
                      i0 + kTile > S;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16_t sa, pa;
#pragma unroll
      for (int e = 0; e < 16; ++e) sa[e] = pa[e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const u32x4_t qa = frag_rows<DH>(qt, 32 * qb, kk, lane);
        const u32x4_t oa = frag_rows<DH>(ot, 32 * qb, kk, lane);
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, qa),
                                                     __builtin_bit_cast(bf16x8_t, kf[kk]), sa,
                                                     0, 0, 0);
        pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, oa),
                                                     __builtin_bit_cast(bf16x8_t, vf[kk]), pa,
                                                     0, 0, 0);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int qr = 32 * qb + 8 * x + 4 * h;   // first of the 4 query rows of group x
        const f32x4_t l4 = *(const f32x4_t *)&ls[qr];
        const f32x4_t d4 = *(const f32x4_t *)&dsm[qr];
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int e = 4 * x + y, qi = i0 + qr + y;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[e], sl2, -l4[y]));
          if (edge && (my_k > qi || qi >= S || (window > 0 && my_k < qi - window + 1))) p = 0.f;
          sa[e] = p;
          pa[e] = p * (pa[e] - d4[y]);
        }
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ks = 2 * qb + half;
        const u32x4_t bp = pack_step(sa, half);
        const u32x4_t bd = pack_step(pa, half);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x4_t ao = frag_tr<DH>(ot, db, ks, lane);
          const u32x4_t aq = frag_tr<DH>(qt, db, ks, lane);
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ao),
                                                           __builtin_bit_cast(bf16x8_t, bp),
                                                           dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, aq),
                                                           __builtin_bit_cast(bf16x8_t, bd),
                                                           dk[db], 0, 0, 0);
        }
      }
    }
  }
  if (live) {
    bf16_t *kp = dqkv + rk * ld + qd + (int64_t)g * DH;
    bf16_t *vp = kp + kvd;
    const int p = pos ? pos[rk] : my_k;
    const float *csr = rope_row<DH>(cs, p, max_seq);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        f32x4_t rkv, rvv;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          rkv[x] = dk[db][4 * gq + x] * scale;
          rvv[x] = dv[db][4 * gq + x];
        }
        if (csr) rkv = rope_back4(rkv, csr + 32 * db + 8 * gq + 4 * h);
        store4(kp + 32 * db + 8 * gq + 4 * h, rkv);
        store4(vp + 32 * db + 8 * gq + 4 * h, rvv);
      }
  }
}

template <int DH>
hipError_t run(const void *qkv, int64_t ld, const void *o, int64_t ldo, const void *dout,
               int64_t lddo, void *dqkv, int B, int S, int Hq, int Hkv, int window,
               const float *lse, float *dsum, const int32_t *pos, const float *cs,
               int max_seq, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)DH);
  const int64_t nb = (S + kRows - 1) / kRows;
  if (nb * Hq * B > 0x7fffffff) return hipErrorInvalidValue;
  const int cus = compute_units();
  attn_dq_mfma_kernel<DH><<<dim3((unsigned)(nb * Hq * B)), 256, 0, s>>>(
      (const bf16_t *)qkv, ld, (const bf16_t *)o, ldo, (const bf16_t *)dout, lddo,
      (bf16_t *)dqkv, S, Hq, Hkv, window, scale, lse, dsum, B, cus, pos, cs, max_seq);
  attn_dkdv_mfma_kernel<DH><<<dim3((unsigned)(nb * Hkv * B)), 256, 0, s>>>(
      (const bf16_t *)qkv, ld, (const bf16_t *)dout, lddo, (bf16_t *)dqkv, S, Hq, Hkv, window,
      scale, lse, dsum, B, cus, pos, cs, max_seq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_backward_bf16(const void *qkv, int64_t ld, const void *o,
                                          int64_t ldo, const void *dout, int64_t lddo,
                                          void *dqkv, int B, int S, int Hq, int Hkv, int d_head,
                                          int window, const float *lse, float *dsum,
                                          const int32_t *positions, const float *cos_sin,
                                          int max_seq, hipStream_t s) {
#define TFM_RUN(D)                                                                             \
  return run<D>(qkv, ld, o, ldo, dout, lddo, dqkv, B, S, Hq, Hkv, window, lse, dsum, positions, \
                cos_sin, max_seq, s);
  switch (d_head) {
    case 32: TFM_RUN(32)
    case 64: TFM_RUN(64)
    case 128: TFM_RUN(128)
  }
#undef TFM_RUN
  return hipErrorInvalidValue;
}

}  // namespace tfm

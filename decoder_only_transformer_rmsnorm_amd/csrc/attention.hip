// Causal multi-head attention with grouped KV heads, flash-style (one pass over the keys
// with an online softmax), on the CDNA4 matrix cores.
//
// What it computes ("Transformer 篇" (dujian.net) 5.4 Attention; "Transformer篇"
// (fengye404.top) 8 Attention; "LLM 2" GQA/MQA): for every (b, query head h, query s),
//   o = sum_{t <= s} softmax_t(q_s . k_t / sqrt(d_head)) v_t,  KV head g = h / (Hq / Hkv).
// Keys after s get weight exactly 0 (they are never added); masking is by token order.
//
// bf16 kernel (d_head in {32, 64, 128}):
//  * A workgroup owns 128 queries of one (b, h): 4 waves x 32 queries. K and V tiles of 64
//    keys go from HBM straight into an LDS ring (buffer_load ... lds, no staging registers),
//    several tiles ahead of the math, and are shared by the 4 waves. Key rows past S read
//    as zero (buffer bounds) and are masked.
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16, K rows as the
//    A operand, Q held in registers as the B operand), so each lane holds 16 keys of ONE
//    query: the running row max needs one cross-lane exchange (lane l <-> l^32) per tile
//    and the row sum none until the end.
//  * O^T = V^T P^T: the bf16-rounded probabilities go straight from the score accumulator
//    into the B operand (no shuffle). V stays row-major in LDS; its A-operand fragments are
//    read with the LDS transpose read ds_read_b64_tr_b16, which hands each lane four
//    consecutive keys of one head dimension. The keys of a 16-key step are taken in the
//    order the score accumulator holds them ({4h..4h+3, 4h+8..4h+11} for lane half h).
//  * Softmax state (max, sum, rescale) is fp32; exponentials are base 2 with the
//    1/sqrt(d_head) * log2(e) factor folded into one fused multiply-add. A row's reference
//    maximum only moves when a tile's scores exceed it by more than 8 in log2 units, so the
//    output is rescaled rarely (softmax does not depend on the shift).
//  * Tiles entirely above the diagonal are never loaded; per wave, tiles past its last
//    query are skipped; only the diagonal tile is masked. Query tiles are issued
//    longest-first to even out the causal imbalance.
//  * Sliding window ("LLM 2" sliding window and hybrid attention): with window W > 0 query s
//    sees keys s - W + 1 .. s. Tiles older than a workgroup's band are never loaded, a wave
//    skips tiles outside its queries' band, and tiles on the band's lower edge are masked
//    like the diagonal tile.
// f32 kernel (d_head in {16, 32, 64, 128}): one thread per query with the same online
// softmax in fp32; it exists for the small fp32 model and for tests, not for speed.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace tfm {
namespace {

constexpr int kBQ = 128;   // queries per workgroup
constexpr int kBKV = 64;   // keys per tile
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.f;   // headroom of the softmax reference maximum (log2 units)
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

template <int DH>
struct AttnTile {
  static constexpr int RB = DH * 2;              // bytes of one K or V row
  static constexpr int CPR = RB / 16;            // 16-byte chunks per row
  static constexpr int FR = 1024 / RB;           // rows one 64-lane 16-byte fill covers
  static constexpr int TILE = kBKV * RB;         // bytes of a K (or V) tile
  static constexpr int INS = TILE / 1024 / 4;    // fills per wave for K (and again for V)
  static constexpr int LOADS = 2 * INS;
  static constexpr int STAGE = 2 * TILE;
  static constexpr int NST = DH >= 128 ? 2 : 3;  // ring depth
  static constexpr int OCC = DH >= 128 ? 1 : 2;
  static_assert(INS >= 1 && INS * 4 * 1024 == TILE, "tile/fill mismatch");
  // every LDS read offset is a per-lane register plus an immediate below 2^16
  static_assert((NST - 1) * STAGE + TILE + (kBKV - 4) * RB < 65536, "LDS offset immediate");
};

// Chunk swizzles. K rows are read 16 bytes per lane (32 consecutive rows, one chunk column);
// V rows are read with the transpose read (8 rows x 4 chunks per instruction, rows 0..3 in
// the first half-wave, 4..7 in the second). Both keep one instruction on distinct banks. The
// V swizzle depends only on row bits that are fixed per lane, so a lane's V addresses differ
// by constants between key steps.
template <int DH>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (DH == 32) return ((r >> 1) ^ (r >> 2)) & 3;
  else if constexpr (DH == 64) return (r ^ (r >> 3)) & 7;
  else return r & 15;
}
template <int DH>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (DH == 32) return 0;
  else if constexpr (DH == 64) return ((r >> 1) & 1) << 2;
  else return (r & 3) << 2;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int N>
using ic = std::integral_constant<int, N>;

template <int DH>
__global__ __launch_bounds__(kThreads, AttnTile<DH>::OCC) void attn_bf16_kernel(
    const bf16_t *__restrict__ q, int64_t q_stride, const bf16_t *__restrict__ k,
    const bf16_t *__restrict__ v, int64_t kv_stride, bf16_t *__restrict__ o, int64_t o_stride,
    int B, int S, int Hq, int Hkv, int n_qt, float scale_log2, int cus, int window,
    float *__restrict__ lse) {
#if defined(__HIP_DEVICE_COMPILE__)
  using T = AttnTile<DH>;
  constexpr int RB = T::RB, CPR = T::CPR, FR = T::FR, TILE = T::TILE, INS = T::INS;
  constexpr int LOADS = T::LOADS, STAGE = T::STAGE, NST = T::NST;
  constexpr int NKB = kBKV / 32;              // 32-key score blocks per tile
  constexpr int NDB = DH / 32;                // 32-dim output blocks
  constexpr int QK_STEPS = DH / 16;           // k-steps of the score MFMA
  constexpr int PV_STEPS = kBKV / 16;         // k-steps of the PV MFMA

  __shared__ __attribute__((aligned(16))) uint8_t lds[NST * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int bh_count = B * Hq;
  // Work items in order of decreasing length (query tile n_qt-1 of every head first). Blocks
  // take them in a snake over rounds of `cus` blocks (one per CU when the grid is dispatched
  // in order): a CU's blocks of rounds 0, 1, 2 get long, shorter and short items.
  const int round = (int)(blockIdx.x / cus), in_round = (int)(blockIdx.x % cus);
  int item = (round & 1) ? round * cus + (cus - 1 - in_round) : (int)blockIdx.x;
  if (item >= (int)gridDim.x) item = (int)blockIdx.x;   // partial last round: keep in order
  const int qt = n_qt - 1 - item / bh_count;
  const int bh = item % bh_count;
  const int b = bh / Hq, hq = bh % Hq, hkv = hq / (Hq / Hkv);
  const int q0 = qt * kBQ, qw0 = q0 + wid * 32;
  const uint32_t kvsb = (uint32_t)(kv_stride * 2);   // bytes between key rows

  // K and V rows 0..S-1 of this (b, kv head); rows at or past S read as zero.
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(k + (int64_t)b * S * kv_stride + (int64_t)hkv * DH), 0,
      (int)(S * kvsb), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(v + (int64_t)b * S * kv_stride + (int64_t)hkv * DH), 0,
      (int)(S * kvsb), kRsrcWord3);

  // ---- Q fragments (B operand of S^T = K Q^T): query qw0 + l32, dims 16*kk + 8h .. +7.
  //      The empty statements make the compiler finish these loads here, so it does not wait
  //      for them (and for every fill issued after them) inside the loop.
  u32x4_t qf[QK_STEPS];
  {
    const int qi = qw0 + l32;
    const bf16_t *qp = q + ((int64_t)b * S + (qi < S ? qi : 0)) * q_stride + (int64_t)hq * DH;
#pragma unroll
    for (int kk = 0; kk < QK_STEPS; ++kk)
      qf[kk] = qi < S ? *(const u32x4_t *)(qp + 16 * kk + 8 * h) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int kk = 0; kk < QK_STEPS; ++kk) asm volatile("" : "+v"(qf[kk]));
  }

  const int kv_end = min(q0 + kBQ, S);
  const int n_tiles = (kv_end + kBKV - 1) / kBKV;
  // sliding window ("LLM 2" sliding window): query s sees keys s - window + 1 .. s
  const int j_lo = window > 0 ? max(0, q0 - window + 1) / kBKV : 0;

  // ---- fills: lane l of a fill lands at base + 16 l, i.e. row frow, chunk slot fchunk; it
  //      fetches the global chunk that the swizzle places in that slot.
  const int frow = lane / CPR, fchunk = lane % CPR;
  uint32_t k_off[INS], v_off[INS];
#pragma unroll
  for (int i = 0; i < INS; ++i) {
    const int r = (wid * INS + i) * FR + frow;
    k_off[i] = (uint32_t)r * kvsb + (uint32_t)((fchunk ^ swz_k<DH>(r)) << 4);
    v_off[i] = (uint32_t)r * kvsb + (uint32_t)((fchunk ^ swz_v<DH>(r)) << 4);
  }
  auto issue = [&](int j, auto slot) {
    uint8_t *base = lds + decltype(slot)::value * STAGE;
    const uint32_t t0 = (uint32_t)(j * kBKV) * kvsb;
#pragma unroll
    for (int i = 0; i < INS; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          k_rsrc, (lds_void_t *)(base + (wid * INS + i) * 1024), 16, t0 + k_off[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          v_rsrc, (lds_void_t *)(base + TILE + (wid * INS + i) * 1024), 16, t0 + v_off[i], 0,
          0, 0);
    }
  };
  auto wait_fills = [&](int tiles) {
    if (NST >= 3 && tiles >= 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // ---- LDS read addresses: a per-lane register plus an immediate for the slot and step.
  //      The reads are inline so the compiler does not wait for every in-flight fill before
  //      them; each is waited for explicitly before its first use.
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_u8_t *)lds;
  uint32_t k_rd[NKB][QK_STEPS];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int kk = 0; kk < QK_STEPS; ++kk) {
      const int row = kb * 32 + l32;
      k_rd[kb][kk] = lds_base + row * RB + (((2 * kk + h) ^ swz_k<DH>(row)) << 4);
    }
  // V^T fragment of dims 32 db .. +31, key step ks: lane (group g = lane / 16, i = lane % 16)
  // addresses row 16 ks + 4 (g / 2) + 8 half + i / 4, dims d0 + 4 (i % 4) with
  // d0 = 32 db + 16 (g % 2); the transpose read returns to lane i of the group the four keys
  // of dim d0 + i.
  const int tg = lane >> 4, ti = lane & 15;
  uint32_t v_rd[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int row = 4 * (tg >> 1) + (ti >> 2);          // row bits the swizzle reads
    const int chunk = ((db * 32 + 16 * (tg & 1)) >> 3) + ((ti & 3) >> 1);
    v_rd[db] = lds_base + TILE + row * RB + ((chunk ^ swz_v<DH>(row)) << 4) + 8 * (ti & 1);
  }
  auto lgkm_wait0 = [&]() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
  auto read_v = [](auto soff, uint32_t addr, u32x2_t (&f)[2 * PV_STEPS]) {
#pragma unroll
    for (int ks = 0; ks < PV_STEPS; ++ks)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                     : "=v"(f[2 * ks + half])
                     : "v"(addr), "i"(decltype(soff)::value + (16 * ks + 8 * half) * RB) : "memory");
  };

  f32x16_t oacc[NDB], lacc;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) lacc[e] = 0.f;
  // all-ones A operand: the row sums of P come out of the matrix core with the P V product
  const u32x4_t ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  float m_run = -__builtin_inff();
  const int my_q = qw0 + l32;

  auto tile = [&](int j, auto slot) {
    constexpr int SL = decltype(slot)::value;
    constexpr int SOFF = SL * STAGE;
    wait_fills(min(NST - 2, n_tiles - 1 - j));
    // every wave's fills of tile j are in LDS; every wave is done reading tile j - 1's slot
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (j + NST - 1 < n_tiles) issue(j + NST - 1, ic<(SL + NST - 1) % NST>{});
    const int kv0 = j * kBKV;
    if (kv0 > qw0 + 31) return;   // every key of the tile is after this wave's queries
    if (window > 0 && kv0 + kBKV - 1 < qw0 - window + 1) return;   // every key is too old

    // ---- S^T = K Q^T
    f32x16_t sacc[NKB];
    {
      u32x4_t kf[2][QK_STEPS];
#pragma unroll
      for (int kk = 0; kk < QK_STEPS; ++kk)
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(kf[0][kk]) : "v"(k_rd[0][kk]), "i"(SOFF) : "memory");
      lgkm_wait0();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if (kb + 1 < NKB) {
#pragma unroll
          for (int kk = 0; kk < QK_STEPS; ++kk)
            asm volatile("ds_read_b128 %0, %1 offset:%2"
                         : "=v"(kf[(kb + 1) & 1][kk]) : "v"(k_rd[kb + 1][kk]), "i"(SOFF) : "memory");
        }
#pragma unroll
        for (int kk = 0; kk < QK_STEPS; ++kk) asm volatile("" : "+v"(kf[kb & 1][kk]));
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < QK_STEPS; ++kk)
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, kf[kb & 1][kk]), __builtin_bit_cast(bf16x8_t, qf[kk]),
              sacc[kb], 0, 0, 0);
        lgkm_wait0();
      }
    }
    // V fragments of the first output block load while the softmax runs
    u32x2_t vf[2][2 * PV_STEPS];
    read_v(ic<SOFF>{}, v_rd[0], vf[0]);

    // ---- online softmax (scores stay in raw units; the scale is folded into the exponent)
    if (kv0 + kBKV - 1 > qw0) {   // diagonal tile: keys after the query get no weight
      const int lim = my_q - kv0 - 4 * h;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kb * 32 + 8 * (e >> 2) + (e & 3) > lim) sacc[kb][e] = -__builtin_inff();
    }
    if (window > 0 && kv0 < qw0 + 31 - window + 1) {   // band edge: keys older than the window
      const int lo = my_q - window + 1 - kv0 - 4 * h;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kb * 32 + 8 * (e >> 2) + (e & 3) < lo) sacc[kb][e] = -__builtin_inff();
    }
    float mt = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[kb][e]);
    {   // lanes l and l ^ 32 hold the two key halves of one query
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                       false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // The reference maximum only moves when the tile's maximum exceeds it by more than 2^8 in
    // probability (log2 units): exp2(s - ref) then stays below 256, and the result does not
    // depend on which reference is used (the same one scales the row sum), so the running
    // output is rescaled rarely instead of on almost every tile.
    const bool move = (mt - m_run) * scale_log2 > kLazyLog2;
    const float m_new = move ? fmaxf(m_run, mt) : m_run;
    // a lane that has seen no visible key yet (possible at a window's edge) keeps zero weight
    const float mc = m_new == -__builtin_inff() ? 0.f : m_new * scale_log2;
    u32x4_t pf[PV_STEPS];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4_t w;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int e = 8 * half + 2 * x;
          w[x] = pack_bf16x2(fast_exp2(__builtin_fmaf(sacc[kb][e], scale_log2, -mc)),
                             fast_exp2(__builtin_fmaf(sacc[kb][e + 1], scale_log2, -mc)));
        }
        pf[2 * kb + half] = w;
      }
    if (__any(move)) {   // some row's reference moved: rescale the running output
      const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run * scale_log2 - mc);
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      lacc[0] *= alpha;
    }
    m_run = m_new;

    // ---- O^T += V^T P^T, and the row sums (all-ones rows times P^T)
#pragma unroll
    for (int ks = 0; ks < PV_STEPS; ++ks)
      lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ones),
                                                     __builtin_bit_cast(bf16x8_t, pf[ks]), lacc,
                                                     0, 0, 0);
    lgkm_wait0();
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      if (db + 1 < NDB) read_v(ic<SOFF>{}, v_rd[db + 1], vf[(db + 1) & 1]);
#pragma unroll
      for (int x = 0; x < 2 * PV_STEPS; ++x) asm volatile("" : "+v"(vf[db & 1][x]));
#pragma unroll
      for (int ks = 0; ks < PV_STEPS; ++ks) {
        const u32x4_t a = {vf[db & 1][2 * ks][0], vf[db & 1][2 * ks][1], vf[db & 1][2 * ks + 1][0],
                           vf[db & 1][2 * ks + 1][1]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, pf[ks]), oacc[db], 0,
            0, 0);
      }
      lgkm_wait0();
    }
  };

  issue(j_lo, ic<0>{});
  if (NST > 2 && j_lo + 1 < n_tiles) issue(j_lo + 1, ic<(NST > 2 ? 1 : 0)>{});
  for (int j0 = j_lo; j0 < n_tiles; j0 += NST) {
    tile(j0, ic<0>{});
    if (j0 + 1 < n_tiles) tile(j0 + 1, ic<1 % NST>{});
    if constexpr (NST > 2)
      if (j0 + 2 < n_tiles) tile(j0 + 2, ic<2 % NST>{});
  }

  if (my_q < S) {
    // row logsumexp of the scaled scores (kept for the backward): max + log(sum)
    if (lse && h == 0)
      lse[((int64_t)b * S + my_q) * Hq + hq] = m_run * (scale_log2 / kLog2e) + logf(lacc[0]);
    const float inv = 1.0f / lacc[0];
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
#endif
}

// bf16 kernel for d_head 128, software pipelined. Its 456 registers per lane leave one wave
// per SIMD, so no other wave hides the serial chain scores -> softmax -> P V of a tile; the
// wave itself overlaps them instead. Step t computes the scores of tile t + 1 on the matrix
// core between the exponentials of tile t, then tile t's P V products with tile t + 1's mask
// and row maximum between them. K therefore runs one tile ahead of V in the LDS ring, and
// every wave runs every step of its workgroup (tiles outside a wave's queries are masked).
// Layouts, fills, swizzles and the lazy reference are those of attn_bf16_kernel.
template <int DH>
__global__ __launch_bounds__(kThreads, AttnTile<DH>::OCC) void attn_bf16_pipe_kernel(
    const bf16_t *__restrict__ q, int64_t q_stride, const bf16_t *__restrict__ k,
    const bf16_t *__restrict__ v, int64_t kv_stride, bf16_t *__restrict__ o, int64_t o_stride,
    int B, int S, int Hq, int Hkv, int n_qt, float scale_log2, int cus, int window,
    float *__restrict__ lse) {
#if defined(__HIP_DEVICE_COMPILE__)
  using T = AttnTile<DH>;
  constexpr int RB = T::RB, CPR = T::CPR, FR = T::FR, TILE = T::TILE, INS = T::INS;
  constexpr int LOADS = T::LOADS, STAGE = T::STAGE, NST = T::NST;
  constexpr int NKB = kBKV / 32;              // 32-key score blocks per tile
  constexpr int NDB = DH / 32;                // 32-dim output blocks
  constexpr int QK_STEPS = DH / 16;           // k-steps of the score MFMA
  constexpr int PV_STEPS = kBKV / 16;         // k-steps of the PV MFMA

  __shared__ __attribute__((aligned(16))) uint8_t lds[NST * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int bh_count = B * Hq;
  // Work items in order of decreasing length (query tile n_qt-1 of every head first). Blocks
  // take them in a snake over rounds of `cus` blocks (one per CU when the grid is dispatched
  // in order): a CU's blocks of rounds 0, 1, 2 get long, shorter and short items.
  const int round = (int)(blockIdx.x / cus), in_round = (int)(blockIdx.x % cus);
  int item = (round & 1) ? round * cus + (cus - 1 - in_round) : (int)blockIdx.x;
  if (item >= (int)gridDim.x) item = (int)blockIdx.x;   // partial last round: keep in order
  const int qt = n_qt - 1 - item / bh_count;
  const int bh = item % bh_count;
  const int b = bh / Hq, hq = bh % Hq, hkv = hq / (Hq / Hkv);
  const int q0 = qt * kBQ, qw0 = q0 + wid * 32;
  const uint32_t kvsb = (uint32_t)(kv_stride * 2);   // bytes between key rows

  // K and V rows 0..S-1 of this (b, kv head); rows at or past S read as zero.
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(k + (int64_t)b * S * kv_stride + (int64_t)hkv * DH), 0,
      (int)(S * kvsb), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(v + (int64_t)b * S * kv_stride + (int64_t)hkv * DH), 0,
      (int)(S * kvsb), kRsrcWord3);

  // ---- Q fragments (B operand of S^T = K Q^T): query qw0 + l32, dims 16*kk + 8h .. +7.
  //      The empty statements make the compiler finish these loads here, so it does not wait
  //      for them (and for every fill issued after them) inside the loop.
  u32x4_t qf[QK_STEPS];
  {
    const int qi = qw0 + l32;
    const bf16_t *qp = q + ((int64_t)b * S + (qi < S ? qi : 0)) * q_stride + (int64_t)hq * DH;
#pragma unroll
    for (int kk = 0; kk < QK_STEPS; ++kk)
      qf[kk] = qi < S ? *(const u32x4_t *)(qp + 16 * kk + 8 * h) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int kk = 0; kk < QK_STEPS; ++kk) asm volatile("" : "+v"(qf[kk]));
  }

  const int kv_end = min(q0 + kBQ, S);
  const int n_tiles = (kv_end + kBKV - 1) / kBKV;
  // sliding window ("LLM 2" sliding window): query s sees keys s - window + 1 .. s
  const int j_lo = window > 0 ? max(0, q0 - window + 1) / kBKV : 0;

  // ---- fills: lane l of a fill lands at base + 16 l, i.e. row frow, chunk slot fchunk; it
  //      fetches the global chunk that the swizzle places in that slot.
  const int frow = lane / CPR, fchunk = lane % CPR;
  uint32_t k_off[INS], v_off[INS];
#pragma unroll
  for (int i = 0; i < INS; ++i) {
    const int r = (wid * INS + i) * FR + frow;
    k_off[i] = (uint32_t)r * kvsb + (uint32_t)((fchunk ^ swz_k<DH>(r)) << 4);
    v_off[i] = (uint32_t)r * kvsb + (uint32_t)((fchunk ^ swz_v<DH>(r)) << 4);
  }
  // The scores of tile t + 1 are computed while the softmax of tile t runs, so K runs one tile
  // ahead of V: stage t (t = j_lo - 1 .. n_tiles - 1) holds the K rows of tile t + 1 and the
  // V rows of tile t (clamped into j_lo .. n_tiles - 1 at the two ends, where that half is not
  // read), and step t reads only stage t.
  auto issue = [&](int t, auto slot) {
    uint8_t *base = lds + decltype(slot)::value * STAGE;
    const uint32_t tk = (uint32_t)(min(t + 1, n_tiles - 1) * kBKV) * kvsb;
    const uint32_t tv = (uint32_t)(max(t, j_lo) * kBKV) * kvsb;
#pragma unroll
    for (int i = 0; i < INS; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          k_rsrc, (lds_void_t *)(base + (wid * INS + i) * 1024), 16, tk + k_off[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          v_rsrc, (lds_void_t *)(base + TILE + (wid * INS + i) * 1024), 16, tv + v_off[i], 0,
          0, 0);
    }
  };
  auto wait_fills = [&](int stages_after) {
    if (NST >= 3 && stages_after >= 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // ---- LDS read addresses: a per-lane register plus an immediate for the slot and step.
  //      The reads are inline so the compiler does not wait for every in-flight fill before
  //      them; each is waited for explicitly before its first use.
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_u8_t *)lds;
  uint32_t k_rd[NKB][QK_STEPS];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int kk = 0; kk < QK_STEPS; ++kk) {
      const int row = kb * 32 + l32;
      k_rd[kb][kk] = lds_base + row * RB + (((2 * kk + h) ^ swz_k<DH>(row)) << 4);
    }
  // V^T fragment of dims 32 db .. +31, key step ks: lane (group g = lane / 16, i = lane % 16)
  // addresses row 16 ks + 4 (g / 2) + 8 half + i / 4, dims d0 + 4 (i % 4) with
  // d0 = 32 db + 16 (g % 2); the transpose read returns to lane i of the group the four keys
  // of dim d0 + i.
  const int tg = lane >> 4, ti = lane & 15;
  uint32_t v_rd[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int row = 4 * (tg >> 1) + (ti >> 2);          // row bits the swizzle reads
    const int chunk = ((db * 32 + 16 * (tg & 1)) >> 3) + ((ti & 3) >> 1);
    v_rd[db] = lds_base + TILE + row * RB + ((chunk ^ swz_v<DH>(row)) << 4) + 8 * (ti & 1);
  }

  f32x16_t oacc[NDB], lacc;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) lacc[e] = 0.f;
  // all-ones A operand: the row sums of P come out of the matrix core with the P V product
  const u32x4_t ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  float m_run = -__builtin_inff();
  const int my_q = qw0 + l32;
  float mc = 0.f;   // m_run in the exponent's units (scale_log2 folded in)

  // ---- scores of tile t: S^T = K Q^T from the K fragments, as products into s
  auto qk_mfma = [&](f32x16_t &s, const u32x4_t &kfr, int kk) {
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kfr),
                                                __builtin_bit_cast(bf16x8_t, qf[kk]),
                                                kk == 0 ? f32x16_t{} : s, 0, 0, 0);
  };
  // ---- masks of tile t on its scores: keys after the query (diagonal tile, and every tile
  //      past the wave's queries) and, with a window, keys older than the band
  auto mask = [&](f32x16_t (&s)[NKB], int t) {
    const int kv0 = t * kBKV;
    if (kv0 + kBKV - 1 > qw0) {
      const int lim = my_q - kv0 - 4 * h;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kb * 32 + 8 * (e >> 2) + (e & 3) > lim) s[kb][e] = -__builtin_inff();
    }
    if (window > 0 && kv0 < qw0 + 31 - window + 1) {
      const int lo = my_q - window + 1 - kv0 - 4 * h;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kb * 32 + 8 * (e >> 2) + (e & 3) < lo) s[kb][e] = -__builtin_inff();
    }
  };
  // ---- the tile's row maximum against the running reference. The reference only moves when
  //      the tile's maximum exceeds it by more than 2^8 in probability (log2 units): exp2(s -
  //      ref) then stays below 256, and the result does not depend on which reference is used
  //      (the same one scales the row sum), so the running output is rescaled rarely instead
  //      of on almost every tile. Returns whether some row's reference moved.
  auto row_max = [&](const f32x16_t (&s)[NKB], float &alpha) -> bool {
    float mt0 = s[0][0], mt1 = s[NKB - 1][1];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        mt0 = fmaxf(mt0, s[kb][e]);
        mt1 = fmaxf(mt1, s[kb][e + 1]);
      }
    float mt = fmaxf(mt0, mt1);
    {   // lanes l and l ^ 32 hold the two key halves of one query
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                       false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const bool move = (mt - m_run) * scale_log2 > kLazyLog2;
    const float m_new = move ? fmaxf(m_run, mt) : m_run;
    // a lane that has seen no visible key yet (possible at a window's edge) keeps zero weight
    const float mc_new = m_new == -__builtin_inff() ? 0.f : m_new * scale_log2;
    alpha = m_new == m_run ? 1.f : fast_exp2(m_run * scale_log2 - mc_new);
    m_run = m_new;
    mc = mc_new;
    return __any(move);
  };
  auto rescale = [&](float alpha) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    lacc[0] *= alpha;
  };
  // ---- exponentials of 8 keys per lane (chunk c = key block c / 2, half c % 2) of the scores
  //      in s, packed to bf16 into pf[c], and their row sums on the matrix core
  auto expo = [&](const f32x16_t (&s)[NKB], int c, u32x4_t (&pf)[PV_STEPS]) {
    const int kb = c >> 1, half = c & 1;
    u32x4_t w;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int e = 8 * half + 2 * x;
      w[x] = pack_bf16x2(fast_exp2(__builtin_fmaf(s[kb][e], scale_log2, -mc)),
                         fast_exp2(__builtin_fmaf(s[kb][e + 1], scale_log2, -mc)));
    }
    pf[c] = w;
    lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ones),
                                                   __builtin_bit_cast(bf16x8_t, w), lacc, 0, 0, 0);
  };
  constexpr int KR = NKB * QK_STEPS;   // K fragment reads of a tile
  constexpr int PER = QK_STEPS / 2;    // score products per exponential chunk
  static_assert(PER >= 1 && 2 * PER == QK_STEPS, "chunking");

  // Step j. On entry sc holds tile j's masked scores and mc its reference; the step issues
  // tile j + 1's K reads, then tile j's exponentials with tile j + 1's score products
  // (into sn) between them, then tile j's P V products with tile j + 1's mask and row maximum
  // between them; a moved reference rescales the output after tile j's products.
  auto body = [&](int j, auto soff, f32x16_t (&sc)[NKB], f32x16_t (&sn)[NKB]) {
    constexpr int SOFF = decltype(soff)::value;
    u32x4_t kf[NKB][QK_STEPS];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int kk = 0; kk < QK_STEPS; ++kk) ds_read16<SOFF>(kf[kb][kk], k_rd[kb][kk]);
    u32x4_t pf[PV_STEPS];
    u32x2_t vf[NDB][2 * PV_STEPS];
    // key block 0 of tile j (chunks 0, 1) with the products of key block 0 of tile j + 1
    if constexpr (KR / 2 <= 15) asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(KR / 2) : "memory");
    else asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int kk = 0; kk < QK_STEPS; ++kk) asm volatile("" : "+v"(kf[0][kk]));
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int x = 0; x < PER; ++x) qk_mfma(sn[0], kf[0][c * PER + x], c * PER + x);
      expo(sc, c, pf);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 20 / (PER + 1), 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 20 - PER * (20 / (PER + 1)), 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // key block 1 likewise; tile j's V fragments go out first
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int kk = 0; kk < QK_STEPS; ++kk) asm volatile("" : "+v"(kf[NKB - 1][kk]));
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ks = 0; ks < PV_STEPS; ++ks)
#pragma unroll
        for (int half = 0; half < 2; ++half)
          asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                       : "=v"(vf[db][2 * ks + half])
                       : "v"(v_rd[db]), "i"(SOFF + (16 * ks + 8 * half) * RB) : "memory");
#pragma unroll
    for (int c = 2; c < 4; ++c) {
#pragma unroll
      for (int x = 0; x < PER; ++x) qk_mfma(sn[NKB - 1], kf[NKB - 1][(c - 2) * PER + x], (c - 2) * PER + x);
      expo(sc, c, pf);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 20 / (PER + 1), 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 20 - PER * (20 / (PER + 1)), 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // tile j + 1's masks (a branch taken on few tiles), then tile j's P V products with tile
    // j + 1's row maximum between them
    mask(sn, j + 1);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int x = 0; x < 2 * PV_STEPS; ++x) asm volatile("" : "+v"(vf[db][x]));
#pragma unroll
    for (int ks = 0; ks < PV_STEPS; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const u32x4_t a = {vf[db][2 * ks][0], vf[db][2 * ks][1], vf[db][2 * ks + 1][0],
                           vf[db][2 * ks + 1][1]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, pf[ks]), oacc[db],
            0, 0, 0);
      }
    float alpha;
    const bool moved = row_max(sn, alpha);
    if (moved) rescale(alpha);
  };

  // stages j_lo - 1 .. j_lo + NST - 3 go out first; the first step (stage j_lo - 1) computes
  // tile j_lo's scores, mask and reference, and sends stage j_lo + NST - 2
  f32x16_t sa[NKB], sb[NKB];
  issue(j_lo - 1, ic<0>{});
  if constexpr (NST > 2) issue(j_lo, ic<1>{});   // j_lo <= n_tiles - 1 always
  wait_fills(NST - 2);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (j_lo + NST - 2 < n_tiles) issue(j_lo + NST - 2, ic<(NST - 1) % NST>{});
  {
    u32x4_t kf[NKB][QK_STEPS];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int kk = 0; kk < QK_STEPS; ++kk) ds_read16<0>(kf[kb][kk], k_rd[kb][kk]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int kk = 0; kk < QK_STEPS; ++kk) {
        asm volatile("" : "+v"(kf[kb][kk]));
        qk_mfma(sa[kb], kf[kb][kk], kk);
      }
    mask(sa, j_lo);
    float alpha;
    row_max(sa, alpha);   // the output is still zero: nothing to rescale
  }
  // Step j reads stage j from slot (j - j_lo + 1) % NST. Every wave runs every step of the
  // workgroup: on a tile outside a wave's queries (after its last query or, with a window,
  // before its band) the masks give every key zero weight, and the last step's scores (of
  // the clamped tile, past every query) are all masked. This keeps the loop to one path.
  auto step = [&](int j, auto slot, f32x16_t (&sc)[NKB], f32x16_t (&sn)[NKB]) {
    constexpr int SL = decltype(slot)::value;
    wait_fills(min(NST - 2, n_tiles - 1 - j));
    // every wave's fills of stage j are in LDS; every wave is done reading stage j - 1's slot
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (j + NST - 1 < n_tiles) issue(j + NST - 1, ic<(SL + NST - 1) % NST>{});
    body(j, ic<SL * STAGE>{}, sc, sn);
  };
  // unrolled over lcm(NST, 2) steps so the score buffers alternate without copies
  constexpr int PERIOD = NST > 2 ? 6 : 2;
  static_assert(NST == 2 || NST == 3, "ring depth");
  for (int j0 = j_lo; j0 < n_tiles; j0 += PERIOD) {
    step(j0, ic<1 % NST>{}, sa, sb);
    if (j0 + 1 >= n_tiles) break;
    step(j0 + 1, ic<2 % NST>{}, sb, sa);
    if constexpr (NST > 2) {
      if (j0 + 2 >= n_tiles) break;
      step(j0 + 2, ic<0>{}, sa, sb);
      if (j0 + 3 >= n_tiles) break;
      step(j0 + 3, ic<1>{}, sb, sa);
      if (j0 + 4 >= n_tiles) break;
      step(j0 + 4, ic<2>{}, sa, sb);
      if (j0 + 5 >= n_tiles) break;
      step(j0 + 5, ic<0>{}, sb, sa);
    }
  }
  if (my_q < S) {
    // row logsumexp of the scaled scores (kept for the backward): max + log(sum)
    if (lse && h == 0)
      lse[((int64_t)b * S + my_q) * Hq + hq] = m_run * (scale_log2 / kLog2e) + logf(lacc[0]);
    const float inv = 1.0f / lacc[0];
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
#endif
}

template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float *__restrict__ q, int64_t q_stride,
                                                      const float *__restrict__ k,
                                                      const float *__restrict__ v, int64_t kv_stride,
                                                      float *__restrict__ o, int64_t o_stride, int B,
                                                      int S, int Hq, int Hkv, float scale,
                                                      int window, float *__restrict__ lse) {
  const int s = blockIdx.x * 64 + threadIdx.x;
  const int hq = blockIdx.y, b = blockIdx.z;
  if (s >= S) return;
  const int hkv = hq / (Hq / Hkv);
  float qv[DH], acc[DH];
  const float *qp = q + ((int64_t)b * S + s) * q_stride + (int64_t)hq * DH;
#pragma unroll
  for (int e = 0; e < DH; ++e) { qv[e] = qp[e] * scale; acc[e] = 0.f; }
  float m = -__builtin_inff(), l = 0.f;
  for (int t = window > 0 ? max(0, s - window + 1) : 0; t <= s; ++t) {
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
  if (lse) lse[((int64_t)b * S + s) * Hq + hq] = m + logf(l);
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < DH; ++e) op[e] = acc[e] * inv;
}

template <int DH>
hipError_t run_bf16(const void *q, int64_t qs, const void *k, const void *v, int64_t kvs, void *o,
                    int64_t os, int B, int S, int Hq, int Hkv, int window, float *lse,
                    hipStream_t st) {
  const int n_qt = (S + kBQ - 1) / kBQ;
  const int64_t blocks = (int64_t)n_qt * B * Hq;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff || !attention_fits(DT_BF16, S, kvs)) return hipErrorInvalidValue;
  const float sl2 = kLog2e / sqrtf((float)DH);
  if constexpr (DH >= 128)
    attn_bf16_pipe_kernel<DH><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        (const bf16_t *)q, qs, (const bf16_t *)k, (const bf16_t *)v, kvs, (bf16_t *)o, os, B, S,
        Hq, Hkv, n_qt, sl2, compute_units(), window, lse);
  else
    attn_bf16_kernel<DH><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        (const bf16_t *)q, qs, (const bf16_t *)k, (const bf16_t *)v, kvs, (bf16_t *)o, os, B, S,
        Hq, Hkv, n_qt, sl2, compute_units(), window, lse);
  return hipGetLastError();
}

template <int DH>
hipError_t run_f32(const void *q, int64_t qs, const void *k, const void *v, int64_t kvs, void *o,
                   int64_t os, int B, int S, int Hq, int Hkv, int window, float *lse,
                   hipStream_t st) {
  if ((int64_t)B * S * Hq == 0) return hipSuccess;
  if (B > 65535 || Hq > 65535) return hipErrorInvalidValue;
  dim3 grid((S + 63) / 64, Hq, B);
  attn_f32_kernel<DH><<<grid, dim3(64), 0, st>>>((const float *)q, qs, (const float *)k,
                                                 (const float *)v, kvs, (float *)o, os, B, S, Hq,
                                                 Hkv, 1.0f / sqrtf((float)DH), window, lse);
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device (cached per device).
int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

bool attention_fits(int dt, int S, int64_t kv_stride) {
  return dt != DT_BF16 || ((int64_t)S + kBKV) * kv_stride * 2 < ((int64_t)1 << 31);
}

bool attention_supported(int dt, int d_head) {
  if (dt == DT_BF16) return d_head == 32 || d_head == 64 || d_head == 128;
  return d_head == 16 || d_head == 32 || d_head == 64 || d_head == 128;
}

hipError_t launch_attention(const void *q, int64_t q_stride, const void *k, const void *v,
                            int64_t kv_stride, void *o, int64_t o_stride, int B, int S, int Hq,
                            int Hkv, int d_head, int dt, int window, hipStream_t s, float *lse) {
  const int w = window > 0 && window < S ? window : 0;   // a window of S or more is no limit
  if (dt == DT_BF16) {
    switch (d_head) {
      case 32: return run_bf16<32>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, w, lse, s);
      case 64: return run_bf16<64>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, w, lse, s);
      case 128: return run_bf16<128>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, w, lse, s);
    }
  } else {
    switch (d_head) {
      case 16: return run_f32<16>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, w, lse, s);
      case 32: return run_f32<32>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, w, lse, s);
      case 64: return run_f32<64>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, w, lse, s);
      case 128: return run_f32<128>(q, q_stride, k, v, kv_stride, o, o_stride, B, S, Hq, Hkv, w, lse, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace tfm

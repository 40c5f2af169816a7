// GEMM family y[m, n] = sum_k a[m, k] w[n, k] on the CDNA4 matrix cores, with fused
// epilogues for the decoder block ("Transformer 篇" (dujian.net) 5.3 Linear: y = x W^T,
// no bias).
//
// Common to both kernels:
//  * A workgroup computes a BM x BN output tile; its waves split it in a grid, each wave
//    owning a sub-tile of MS x MS matrix-core blocks accumulated in fp32.
//  * The WEIGHT rows are the MFMA "A" operand and the activation rows the "B" operand, so
//    each lane's accumulator holds 4 consecutive output columns n of one row m. That makes
//    the RoPE pairs (2i, 2i+1) and the gate/up pairs of SwiGLU lane-local and lets every
//    lane store 4 contiguous outputs.
//  * K stages are kept in LDS as 16-byte chunks whose position is XOR-swizzled by the row,
//    so the rows one fragment read touches fall on distinct banks.
//  * Epilogues: plain store (LM head; bf16 or f32, any row stride, odd N; streaming stores,
//    since nothing on the path re-reads the logits), residual add into
//    the fp32 stream (out and down projections), RoPE on the q/k columns of the fused QKV
//    projection ("Transformer 篇" 5.5; "LLM 2" RoPE) and SiLU(gate) * up for the SwiGLU up
//    projection ("Transformer 篇" 5.3; "LLM 2" SwiGLU FFN). For SwiGLU the weight tile
//    interleaves 32 rows of W1 with the matching 32 rows of W3, so a wave's gate and up
//    accumulator blocks hold the same hidden units.
//
// bf16 kernel (the model's GEMMs): tiles up to 256 x 256, 4 or 8 waves, matrix-core blocks
// of 32 x 32 x 16 or 16 x 16 x 32 (the latter moves less data through the register file
// per flop, which is what counts once the chip runs at its power limit). Global data goes
// straight into LDS with buffer_load_dwordx4 ... lds (no staging registers): each wave
// instruction fills 1 KB of tile rows (lane l lands at base + 16 l) and each lane fetches
// the global chunk that the swizzle assigns to its LDS slot; the k offset of a stage rides
// in the scalar offset, so a fill costs no vector arithmetic. Buffer resources cover
// exactly the rows a tile may read, so rows past M or N (and K chunks past K) read as zero
// without branches. A ring of 2-6 stages runs ahead of the MFMAs, refilled between them.
// Main loops: the cross-stage pipeline (the products whose K is a multiple of 64) reads the
// fragments of the next 32-deep k step while the MFMAs of the current one run, across the
// stage barrier too, with two waves per SIMD; the classic loop (ragged K, split K) reads a
// stage's first fragments after its barrier; the 8-wave ping-pong variant (SwiGLU with ragged
// K) splits the waves into two groups half a step apart, so one group's LDS reads and fills
// overlap the other's MFMAs on every SIMD. Tiles are assigned
// to XCDs in contiguous runs (workgroup b runs on XCD b % 8) and ordered in groups of 8
// tile-rows, so the workgroups an XCD runs at once share activation and weight row-blocks
// in its L2.
// f32 kernel (the small fp32 model): the same tile logic with register-staged loads and
// v_mfma_f32_32x32x2_f32.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace tfm {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;  // bytes of one tile row per K stage
constexpr int kChunks = 8;      // 16-byte chunks per tile row and stage
constexpr int kGroupM = 8;      // tile-rows per ordering group
constexpr int kXentBM = 192, kXentBN = 128;   // tile of the fused LM-head cross-entropy
constexpr int kResidualBN = 192;              // BN of the bf16 residual product
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kOOB = 0x80000000u;        // offset beyond any num_records used here

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

__device__ __forceinline__ int swz(int row) { return row & 7; }


template <int N>
using ic2 = std::integral_constant<int, N>;

// f(integral_constant<int, I>) for I = B .. E - 1, each index a constant expression
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(ic2<B>{});
    static_for<B + 1, E>(f);
  }
}

// Buffer resources exist only for the device target; the host pass sees the kernels'
// signatures (to emit launch stubs) but not their bodies.
#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, kRsrcWord3);
}
#endif

// Workgroup id -> (tile row, tile column): contiguous runs per XCD, grouped order.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int T = tiles_m * tiles_n;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = T >> 3, extra = T & 7;
  const int logical = xcd * per + min(xcd, extra) + local;
  const int group = logical / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(kGroupM, tiles_m - first_m);
  const int in = logical - group * kGroupM * tiles_n;
  tm = first_m + in % gm;
  tn = in / gm;
}

// Weight rows: pointer to virtual row n and the number of rows of that source from n on.
// Row stride of the weight rows (a weight-gradient product over part of K keeps the full rows).
__device__ __forceinline__ int64_t wstride(const GemmArgs &g) { return g.ldw > 0 ? g.ldw : g.K; }

// The arguments of K part blockIdx.y of a split product: operands advanced to the part's first
// k (the weight rows keep their full stride), K cut to the part, output advanced to its slab.
template <typename T, bool KMAJ = false>
__device__ __forceinline__ GemmArgs k_part(const GemmArgs &g0) {
  GemmArgs g = g0;
  if (g0.kparts > 1) {
    const int64_t k0 = (int64_t)blockIdx.y * g0.kpart;
    g.ldw = wstride(g0);
    // K-major operands (row k of both is one k): the part starts k0 rows in
    g.a = (const T *)g0.a + (KMAJ ? k0 * g0.lda : k0);
    g.w0 = (const T *)g0.w0 + (KMAJ ? k0 * g.ldw : k0);
    g.K = (int)min((int64_t)g0.kpart, (int64_t)g0.K - k0);
    g.y = (uint8_t *)g0.y + (size_t)blockIdx.y * g0.ypart * (g0.y_dt == DT_F32 ? 4 : 2);
  }
  return g;
}

template <int EPI, typename T>
__device__ __forceinline__ const T *weight_rows(const GemmArgs &g, int n, int &rows_left) {
  if constexpr (EPI == EPI_SWIGLU) {
    // virtual rows come in 64-row groups: 32 gate rows (W1) then the same 32 up rows (W3)
    const int j = ((n >> 6) << 5) | (n & 31);
    rows_left = min(g.n0 - j, 32 - (n & 31));
    const T *base = (const T *)(((n >> 5) & 1) ? g.w1 : g.w0);
    return base + (int64_t)(rows_left > 0 ? j : 0) * wstride(g);
  } else if constexpr (EPI == EPI_QKV_ROPE) {
    if (n < g.n0) {
      rows_left = g.n0 - n;
      return (const T *)g.w0 + (int64_t)n * wstride(g);
    }
    if (n < g.n0 + g.n1) {
      rows_left = g.n0 + g.n1 - n;
      return (const T *)g.w1 + (int64_t)(n - g.n0) * wstride(g);
    }
    rows_left = g.N - n;
    return (const T *)g.w2 + (int64_t)(rows_left > 0 ? n - g.n0 - g.n1 : 0) * wstride(g);
  } else {
    rows_left = g.N - n;
    return (const T *)g.w0 + (int64_t)(rows_left > 0 ? n : 0) * wstride(g);
  }
}

__device__ __forceinline__ void store_out(const GemmArgs &g, int64_t m, int n, f32x4_t v,
                                          int ncols) {
  const int64_t off = m * g.ldy + n;
  const bool vec = ((g.ldy & 3) == 0) && (n + 3 < ncols);
  if (g.y_dt == DT_BF16) {
    bf16_t *y = (bf16_t *)g.y;
    if (vec) {
      store4(y + off, v);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < ncols) y[off + r] = f32_to_bf16(v[r]);
    }
  } else {
    float *y = (float *)g.y;
    if (vec) {
      store4(y + off, v);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < ncols) y[off + r] = v[r];
    }
  }
}

// Epilogue of one wave: lane holds acc[bn][bm][4q + r] for
//   n = nw + bn*32 + 8q + 4h + r,   m = mw + bm*32 + (lane & 31).
template <int EPI, int NBM, int NBN>
__device__ __forceinline__ void epilogue(const GemmArgs &g, f32x16_t (&acc)[NBN][NBM], int64_t mw,
                                         int nw, int lane) {
  const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int bm = 0; bm < NBM; ++bm) {
    const int64_t m = mw + bm * 32 + l32;
    if (m >= g.M) continue;
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int t = 0; t < NBN / 2; ++t) {
        const int jbase = (nw + 64 * t) / 2;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = jbase + 8 * q + 4 * h;
          if (j >= g.n0) continue;
          f32x4_t u;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = acc[2 * t][bm][4 * q + r], b = acc[2 * t + 1][bm][4 * q + r];
            u[r] = a / (1.0f + __expf(-a)) * b;
          }
          store_out(g, m, j, u, g.n0);
        }
      }
    } else {
      int pos = 0;
      if constexpr (EPI == EPI_QKV_ROPE) pos = g.positions ? g.positions[m] : (int)(m % g.S);
#pragma unroll
      for (int bn = 0; bn < NBN; ++bn) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nw + bn * 32 + 8 * q + 4 * h;
          if (n >= g.N) continue;
          f32x4_t v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[bn][bm][4 * q + r];
          if constexpr (EPI == EPI_RESIDUAL) {
            const float *res = g.residual + m * g.ldy + n;
            if (((g.ldy & 3) == 0) && n + 3 < g.N) {
              v += load4(res);
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (n + r < g.N) v[r] += res[r];
            }
          } else if constexpr (EPI == EPI_QKV_ROPE) {
            if (n < g.n0 + g.n1) {  // q and k columns rotate; v columns pass through
              if (pos >= 0 && pos < g.max_seq) {
                const int i0 = (n % g.d_head) >> 1;
                const f32x4_t cs =
                    *(const f32x4_t *)(g.cos_sin + ((int64_t)pos * (g.d_head >> 1) + i0) * 2);
                const float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
                v[0] = x0 * cs[0] - x1 * cs[1];
                v[1] = x0 * cs[1] + x1 * cs[0];
                v[2] = x2 * cs[2] - x3 * cs[3];
                v[3] = x2 * cs[3] + x3 * cs[2];
              } else {
                const float nan = __builtin_nanf("");
                v = f32x4_t{nan, nan, nan, nan};
              }
            }
          }
          store_out(g, m, n, v, g.N);
        }
      }
    }
  }
}

// 1 / rms(x) of each of a lane's NBM rows (rows m0 + wm WM + MS bm + l32) from the producer's
// per-column-tile sums of squares, added in tile order (deterministic); four partials are
// loaded per step while the previous four are added. Rows past M read row M - 1 (their
// outputs are never stored).
template <int NBM, int MS, int WM>
__device__ __forceinline__ void split_norm_scales(const GemmArgs &g, int64_t m0, int wm, int l32,
                                                  float (&rsv)[NBM]) {
  constexpr int NV = kNormParts / 4;
  const float *rowp[NBM];
  float ss[NBM];
  f32x4_t cur[NBM], nxt[NBM];
#pragma unroll
  for (int bm = 0; bm < NBM; ++bm) {
    const int64_t m = m0 + wm * WM + bm * MS + l32;
    rowp[bm] = g.rs_part + (m < g.M ? m : g.M - 1) * kNormParts;
    cur[bm] = *(const f32x4_t *)rowp[bm];
    ss[bm] = 0.f;
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const bool more = v + 1 < NV && 4 * (v + 1) < g.rs_parts;
    if (more) {
#pragma unroll
      for (int bm = 0; bm < NBM; ++bm) nxt[bm] = *(const f32x4_t *)(rowp[bm] + 4 * (v + 1));
    }
#pragma unroll
    for (int bm = 0; bm < NBM; ++bm)
#pragma unroll
      for (int t = 0; t < 4; ++t) ss[bm] += 4 * v + t < g.rs_parts ? cur[bm][t] : 0.f;
    if (!more) break;
#pragma unroll
    for (int bm = 0; bm < NBM; ++bm) cur[bm] = nxt[bm];
  }
#pragma unroll
  for (int bm = 0; bm < NBM; ++bm) rsv[bm] = rsqrtf(ss[bm] / (float)g.rs_d + g.rs_eps);
}

// Epilogue of the SwiGLU product's 16 x 16 blocks, written from registers. Block (bn, bm) of
// the lane holds rows m = m0 + wm WM + 16 bm + l32 and virtual weight rows n0 + wn WN + 16 bn
// + 4 h .. + 3; in every 64-row group of virtual rows, gate block gb and up block gb + 2 hold
// the same hidden units, and the output column is the hidden unit. Rows are first scaled by
// 1 / rms(x) when the RMSNorm is split across the products.
template <int NBM, int NBN, int WM, int WN, typename Acc>
__device__ __forceinline__ void swiglu_direct_epilogue(const GemmArgs &g, Acc (&acc)[NBN][NBM],
                                                       int64_t m0, int n0, int wm, int wn, int h,
                                                       int l32) {
  const int ncols = g.n0;   // d_ff
  const bool vec = (g.ldy & 3) == 0;
  float rsv[NBM];
#pragma unroll
  for (int bm = 0; bm < NBM; ++bm) rsv[bm] = 1.f;
  if (g.rs_part) split_norm_scales<NBM, 16, WM>(g, m0, wm, l32, rsv);
  bf16_t *y = (bf16_t *)g.y;
#pragma unroll
  for (int bm = 0; bm < NBM; ++bm) {
    const int64_t m = m0 + wm * WM + bm * 16 + l32;
    if (m >= g.M) continue;
#pragma unroll
    for (int bn = 0; bn < NBN / 2; ++bn) {
      const int gb = 4 * (bn >> 1) + (bn & 1), ub = gb + 2;
      const int col = (n0 + wn * WN) / 2 + bn * 16 + 4 * h;
      float v[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        // SiLU(a) b = a b / (1 + 2^(-a log2 e)) with the hardware exp2 and reciprocal (about 1
        // ulp each, far inside the bf16 rounding that follows); a very negative a gives
        // 2^(+big) = inf, a reciprocal of 0 and SiLU = -0
        const float a = acc[gb][bm][x] * rsv[bm], b = acc[ub][bm][x] * rsv[bm];
        v[x] = a * b * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * 1.4426950408889634f));
      }
      bf16_t *p = y + m * g.ldy + col;
      if (vec && col + 3 < ncols) {
        *(u32x2_t *)p = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x)
          if (col + x < ncols) p[x] = f32_to_bf16(v[x]);
      }
      if (g.keep_a) {   // training: the gate and up values the backward reads
        bf16_t *pa = (bf16_t *)g.keep_a + m * g.ldy + col, *pc = (bf16_t *)g.keep_c + m * g.ldy + col;
        float a[4], c[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          a[x] = acc[gb][bm][x] * rsv[bm];
          c[x] = acc[ub][bm][x] * rsv[bm];
        }
        if (vec && col + 3 < ncols) {
          *(u32x2_t *)pa = u32x2_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
          *(u32x2_t *)pc = u32x2_t{pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])};
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x)
            if (col + x < ncols) {
              pa[x] = f32_to_bf16(a[x]);
              pc[x] = f32_to_bf16(c[x]);
            }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ bf16 kernel
constexpr int kLdsBytes = 160 * 1024;   // gfx950 LDS per workgroup

// Chunk swizzle of a tile row of RB bytes (RB/16 chunks), chosen by measuring ds_read_b128
// throughput for the fragment reads of both matrix-core blocks (16 rows x 4 chunks and
// 32 rows x 2 chunks per instruction): this mask keeps both at the LDS port's full rate
// (~200 B/clk per CU) for 64- and 128-byte rows, where e.g. row ^ (row >> 3) halves it for
// 16-row reads of 128-byte rows (2-way bank conflicts). The fills swizzle a weight row by its
// row within the weight part of the tile and the reads by its row within the whole tile (BM
// further on), so the mask must repeat with a period that divides BM: it repeats every 32.
template <int RB>
__device__ __forceinline__ int swz_rb(int row) {
  return ((row >> 1) ^ (row >> 2)) & (RB / 16 - 1);
}

// Epilogue staging: output rows of `rb` bytes, 16-byte chunks XOR-swizzled by the row so
// that the 32 rows written by one store instruction spread over the banks. The XOR stays
// inside an aligned block of p chunks, p the largest power of two dividing the row's chunk
// count, so it permutes the chunks of a row even when that count is not a power of two.
__device__ __forceinline__ int stage_off(int r, int byte, int rb) {
  const int cpr = rb >> 4;
  const int p = cpr & -cpr;
  const int c = byte >> 4;
  return r * rb + ((c ^ (r & (p - 1) & 31)) << 4) + (byte & 15);
}

template <int BM, int BN, int BK, int NST, int NW>
struct BfTile {
  static constexpr int RB = BK * 2;                   // bytes per tile row per stage
  static constexpr int FILL_ROWS = 1024 / RB;         // rows one 64-lane 16-byte fill covers
  static constexpr int A_INS = BM / (NW * FILL_ROWS); // fills per wave per stage
  static constexpr int B_INS = BN / (NW * FILL_ROWS);
  static constexpr int LOADS = A_INS + B_INS;
  static constexpr int STAGE = (BM + BN) * RB;
  static constexpr int RING = NST * STAGE;
  static_assert(A_INS * NW * FILL_ROWS == BM && B_INS * NW * FILL_ROWS == BN,
                "tile/fill mismatch");
  static_assert(RING <= kLdsBytes, "LDS ring too large");
  static_assert(NST >= 2 && NST <= 6 && (NST - 2) * LOADS <= 63, "vmcnt range");
};

// EARLY: issue all fills of the refilled stage right after the barrier (one burst) instead of
// spreading them between the MFMAs of the step. WGM x WGN waves share the tile (each owns a
// (BM/WGM) x (BN/WGN) sub-tile); with 8 waves two of them share each SIMD.
// PP (ping-pong, 8 waves): the two waves of a SIMD belong to different wave groups (rows
// 0..BM/2 and BM/2..BM of the tile) that run half a step apart. While one group multiplies
// out of registers, the other reads its next fragments from LDS and issues its fills, so
// the matrix cores of every SIMD alternate between the two waves instead of idling while
// both wait on memory.
// MS: matrix-core block, 32 (v_mfma_f32_32x32x16_bf16) or 16 (v_mfma_f32_16x16x32_bf16). The
// 16x16 form moves less accumulator and operand data through the register file per flop,
// which pays under the chip's power limit.
// XS (cross-stage pipeline): the KM-deep k steps run as one flat sequence and the fragments of
// step s + 1 are read while the MFMAs of step s run, also across a stage boundary, so no wave
// waits on LDS at the start of a stage (see the main loop).
// KMAJ (the weight-gradient products, K = tokens): both operands are K-major, element (m, k)
// of the activations at a[k lda + m] and (n, k) of the weights at w0[k ldw + n], as the
// row-major activations of the forward are read when the sum runs over tokens. A stage then
// holds BK rows of k, each BM (or BN) contiguous elements, and every MFMA fragment (8
// consecutive k of one row m) comes from two LDS transpose reads (ds_read_b64_tr_b16: each
// lane of a 16-lane group reads 4 elements of one k row, and lane i receives the 4 k values
// of column i). No operand is ever transposed in memory.
template <int BM, int BN, int BK, int NST, int EPI, int OCC = 1, bool EARLY = false, int WGM = 2,
          int WGN = 2, bool PP = false, int MS = 32, bool XS = false, bool KMAJ = false>
__device__ __forceinline__ void gemm_bf16_tile(const GemmArgs &g, int tm, int tn) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NT = 64 * WGM * WGN;
  using T = BfTile<BM, BN, BK, NST, WGM * WGN>;
  constexpr int RB = T::RB, FR = T::FILL_ROWS, A_INS = T::A_INS, B_INS = T::B_INS;
  static_assert(MS == 32 || MS == 16, "matrix-core block");
  constexpr int KM = MS == 32 ? 16 : 32;           // k per MFMA
  constexpr int LOADS = T::LOADS, STAGE = T::STAGE, KK = BK / KM;
  constexpr int AE = MS * MS / 64;                 // accumulator elements per lane and block
  constexpr int WM = BM / WGM, WN = BN / WGN;      // wave sub-tile
  constexpr int NBM = WM / MS, NBN = WN / MS;      // MS x MS blocks per wave
  static_assert(NBM * MS * WGM == BM && NBN * MS * WGN == BN, "wave grid does not tile");
  static_assert(EPI != EPI_SWIGLU || MS == 32 || WN % 64 == 0,
                "16x16 SwiGLU pairs gate/up blocks inside 64-row groups");
  static_assert(WGM % 2 == 0, "the two-pass epilogue splits the waves along M");
  constexpr int OUT_COLS = EPI == EPI_SWIGLU ? BN / 2 : (EPI == EPI_XENT ? 0 : BN);
  constexpr int LDS = T::RING > BM * OUT_COLS * 2 ? T::RING : BM * OUT_COLS * 2;
  static_assert(EPI != EPI_XENT || 2 * BM * WGN * 4 <= LDS, "cross-entropy row buffers");
  static_assert(LDS * OCC <= kLdsBytes, "LDS does not allow the requested occupancy");
  static_assert(EPI != EPI_SWIGLU || (NBN % 2) == 0, "SwiGLU needs gate/up block pairs");
  using acc_t = std::conditional_t<MS == 32, f32x16_t, f32x4_t>;
  static_assert(!KMAJ || (!XS && !PP && MS == 32 && BK == 64 && BM == 128 && BN == 128 &&
                          EPI == EPI_STORE),
                "K-major operands: 128 x 128 tiles of 32 x 32 blocks, classic loop, plain store");

  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  // ping-pong: waves w and w + 4 share a SIMD and sit in different groups (wm)
  const int wm = PP ? wid / WGN : wid % WGM, wn = PP ? wid % WGN : wid / WGM;
  // lane -> (row of the block it reads / m of its outputs, k chunk it reads / n group it holds)
  const int h = lane / MS, l32 = lane % MS;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const int K = g.K;
  const int frow = lane / (RB / 16), fchunk = lane % (RB / 16);  // lane's slot in a fill

  // cross-entropy gradient: each of the lane's rows' exponent offset (log2 units: log-sum-exp
  // plus log2 of the counted rows) and target (-1 for a row without one in [0, N)), read
  // before the main loop so that their latency is hidden
  constexpr int XR = EPI == EPI_XENT_GRAD ? NBM : 1;
  float xl[XR], xinv = 0.f;
  int xt[XR];
  if constexpr (EPI == EPI_XENT_GRAD) {
    const int cnt = max(g.xg_count[0], 1);
    xinv = 1.0f / (float)cnt;
    const float l2c = __builtin_amdgcn_logf((float)cnt);   // log2
#pragma unroll
    for (int bm = 0; bm < NBM; ++bm) {
      const int64_t m = m0 + wm * WM + bm * MS + l32;
      const int64_t mc = m < g.M ? m : g.M - 1;
      const int t = g.targets[mc];
      xt[bm] = t >= 0 && t < g.N ? t : -1;
      xl[bm] = __builtin_fmaf(g.xg_lse[mc], 1.4426950408889634f, l2c);
      asm volatile("" : "+v"(xl[bm]), "+v"(xt[bm]));
    }
  }

  // Activation rows m0 .. m0+BM-1: one resource; rows past M read as zero.
  // K-major: the resource starts at column m0 and ends with the operand's last element
  // (column M - 1 of row K - 1), so rows past K read as zero and nothing past the operand is
  // read; columns past M inside earlier rows only feed outputs that are never stored.
  const __amdgpu_buffer_rsrc_t a_rsrc =
      KMAJ ? make_rsrc((const bf16_t *)g.a + m0, ((int64_t)(g.K - 1) * g.lda + g.M - m0) * 2)
           : make_rsrc((const bf16_t *)g.a + m0 * g.lda, min((int64_t)BM, g.M - m0) * g.lda * 2);
  // K-major fills: a 1 KB fill covers 4 k rows of 128 elements; lane l lands in row l / 16,
  // 16-byte slot l % 16, which holds chunk (l % 16) ^ 4 (row % 4) of the row (the swizzle
  // the transpose reads need).
  const int krow = lane >> 4, kslot = lane & 15;
  uint32_t a_off[A_INS];
  int a_k[A_INS];
#pragma unroll
  for (int i = 0; i < A_INS; ++i) {
    if constexpr (KMAJ) {
      const int r = (wid * A_INS + i) * 4 + krow;
      a_k[i] = 0;
      a_off[i] = (uint32_t)(r * g.lda * 2 + ((kslot ^ (4 * krow)) << 4));
    } else {
      const int r = (wid * A_INS + i) * FR + frow;
      a_k[i] = (fchunk ^ swz_rb<RB>(r)) * 8;
      a_off[i] = (uint32_t)(r * g.lda * 2 + a_k[i] * 2);
    }
  }
  // Weight rows: one resource per fill group (a group never straddles two sources).
  __amdgpu_buffer_rsrc_t b_rsrc[B_INS];
  uint32_t b_off[B_INS];
  int b_k[B_INS];
#pragma unroll
  for (int i = 0; i < B_INS; ++i) {
    if constexpr (KMAJ) {
      const int r = (wid * B_INS + i) * 4 + krow;
      b_rsrc[i] = make_rsrc((const bf16_t *)g.w0 + n0, ((int64_t)(g.K - 1) * g.ldw + g.N - n0) * 2);
      b_k[i] = 0;
      b_off[i] = (uint32_t)(r * g.ldw * 2 + ((kslot ^ (4 * krow)) << 4));
    } else {
      const int r0 = (wid * B_INS + i) * FR;
      int rows_left;
      const bf16_t *src = weight_rows<EPI, bf16_t>(g, n0 + r0, rows_left);
      b_rsrc[i] = make_rsrc(src, (int64_t)min(rows_left, FR) * wstride(g) * 2);
      b_k[i] = (fchunk ^ swz_rb<RB>(r0 + frow)) * 8;
      b_off[i] = (uint32_t)(frow * wstride(g) * 2 + b_k[i] * 2);
    }
  }

  // Residual epilogue: the fp32 residual tile is read into registers before the main loop,
  // in the chunk order of the coalesced output stores, so its HBM latency hides behind the
  // matrix work instead of stalling each store of the epilogue. These loads are older than
  // every fill, so the first stage's wait also covers them. Chunks a vector load cannot take
  // (ragged tile edge, row stride not a multiple of 4) are read again in the epilogue.
  constexpr bool kRes = EPI == EPI_RESIDUAL;
  constexpr int RES_CPR = BN * 4 / 16;                    // 16-byte chunks per fp32 tile row
  constexpr int RES_LDS = T::RING > BM * BN * 2 ? T::RING : BM * BN * 2;
  constexpr int RES_PASSES = BM * BN * 4 > RES_LDS ? 2 : 1;
  constexpr int RES_IT = (BM / RES_PASSES) * RES_CPR / NT; // chunks per thread and pass
  static_assert(!kRes || RES_IT * NT == (BM / RES_PASSES) * RES_CPR, "residual chunk split");
  f32x4_t resv[kRes ? RES_PASSES * RES_IT : 1];
  // fused RMSNorm: the gain of each chunk's 4 columns (bf16), read with the residual
  uint2 gnv[kRes ? RES_PASSES * RES_IT : 1];
  if constexpr (kRes) {
    const bool rvec = (g.ldy & 3) == 0;
    const bool fuse = g.nrm_y != nullptr;
#pragma unroll
    for (int j = 0; j < RES_PASSES * RES_IT; ++j) {
      const int idx = tid + (j % RES_IT) * NT;
      const int64_t m = m0 + (j / RES_IT) * (BM / RES_PASSES) + idx / RES_CPR;
      const int n = n0 + (idx % RES_CPR) * 4;
      resv[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      gnv[j] = uint2{0u, 0u};
      if (rvec && m < g.M && n + 4 <= g.N) resv[j] = *(const f32x4_t *)(g.residual + m * g.ldy + n);
      if (fuse && n + 4 <= g.N) gnv[j] = *(const uint2 *)((const bf16_t *)g.nrm_g + n);
    }
  }

  const int nk = (K + BK - 1) / BK;
  // The k offset of a stage travels in the scalar offset of the load, so a fill costs no
  // vector arithmetic. Only a ragged last stage (K % BK != 0) switches each lane to its
  // precomputed tail offset: out of range (reads zero) where its chunk lies past K.
  const int tail_kt = K % BK != 0 && !KMAJ ? nk - 1 : -1;
  uint32_t a_toff[A_INS], b_toff[B_INS];
#pragma unroll
  for (int i = 0; i < A_INS; ++i) a_toff[i] = (nk - 1) * BK + a_k[i] >= K ? kOOB : a_off[i];
#pragma unroll
  for (int i = 0; i < B_INS; ++i) b_toff[i] = (nk - 1) * BK + b_k[i] >= K ? kOOB : b_off[i];
  // Fill number `idx` (A fills first, then B fills) of stage `kt`.
  // the stage's k offset in bytes: along the row, or (K-major) whole rows
  const uint32_t kstep_a = KMAJ ? (uint32_t)(BK * g.lda * 2) : (uint32_t)(BK * 2);
  const uint32_t kstep_b = KMAJ ? (uint32_t)(BK * wstride(g) * 2) : (uint32_t)(BK * 2);
  auto issue_one = [&](int kt, int idx) {
    uint8_t *base = lds + (kt % NST) * STAGE;
    if (idx < A_INS) {
      const uint32_t off = kt == tail_kt ? a_toff[idx] : a_off[idx];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          a_rsrc, (lds_void_t *)(base + (wid * A_INS + idx) * FR * RB), 16, off, kt * kstep_a,
          0, 0);
    } else {
      const int i = idx - A_INS;
      const uint32_t off = kt == tail_kt ? b_toff[i] : b_off[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          b_rsrc[i], (lds_void_t *)(base + (BM + (wid * B_INS + i) * FR) * RB), 16, off,
          kt * kstep_b, 0, 0);
    }
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int idx = 0; idx < LOADS; ++idx) issue_one(kt, idx);
  };
  // Wait until at most `stages` stages of this wave's fills are still in flight.
  auto wait_fills = [&](int stages) {
    if (NST >= 6 && stages >= 4) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * LOADS) : "memory");
    else if (NST >= 5 && stages >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * LOADS) : "memory");
    else if (NST >= 4 && stages >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LOADS) : "memory");
    else if (NST >= 3 && stages >= 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  acc_t acc[NBN][NBM];
#pragma unroll
  for (int bn = 0; bn < NBN; ++bn)
#pragma unroll
    for (int bm = 0; bm < NBM; ++bm)
#pragma unroll
      for (int e = 0; e < AE; ++e) acc[bn][bm][e] = 0.f;

  // Fragment reads are issued as inline ds_read_b128: the compiler's wait insertion cannot
  // tell which LDS bytes an in-flight buffer->LDS fill writes, and would otherwise wait for
  // every outstanding fill (all prefetched stages) before the first read of a stage. The
  // fills of the stage being read are already complete (wait_fills + barrier); the reads
  // are waited for explicitly (wait_frags) before the MFMAs that use them.
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_u8_t *)lds;
  // K-major fragment of 32 rows (block j of the operand tile) for k rows 16 kk .. +15: lane
  // (group q = lane / 16, i = lane % 16) addresses k row 16 kk + 8 (q / 2) + 4 t + i / 4 and
  // columns 32 j + 16 (q % 2) + 4 (i % 4) .. +3 (read t = 0, 1), so it receives k values
  // 8 (q / 2) + 4 t .. +3 of column 32 j + 16 (q % 2) + i: lane l holds row l % 32 and k
  // 8 (l / 32) .. +7, the MFMA operand layout. Per lane and block: one base address.
  uint32_t kmA[KMAJ ? NBM : 1], kmB[KMAJ ? NBN : 1];
  if constexpr (KMAJ) {
    const int q = lane >> 4, i = lane & 15;
    const int rowl = 8 * (q >> 1) + (i >> 2);   // row within the 16-row k step (t = 0)
    auto col_off = [&](int j) {
      const int chunk = 4 * j + 2 * (q & 1) + ((i & 3) >> 1);
      return (uint32_t)(((chunk ^ (4 * (i >> 2))) << 4) + 8 * (i & 1));
    };
#pragma unroll
    for (int bm = 0; bm < NBM; ++bm)
      kmA[bm] = lds_base + rowl * (BM * 2) + col_off(wm * NBM + bm);
#pragma unroll
    for (int bn = 0; bn < NBN; ++bn)
      kmB[bn] = lds_base + BK * BM * 2 + rowl * (BN * 2) + col_off(wn * NBN + bn);
  }
  auto read_km = [](uint32_t addr, auto imm_c, u32x4_t &f) {
    constexpr int IMM = decltype(imm_c)::value;
    u32x2_t lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(addr), "i"(IMM) : "memory");
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                 : "=v"(hi) : "v"(addr), "i"(IMM + 4 * BM * 2) : "memory");
    f = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  };
  auto read_frags = [&](int stage, int kk, u32x4_t (&fa)[NBM], u32x4_t (&fb)[NBN]) {
    const uint32_t st = lds_base + stage * STAGE;
    if constexpr (KMAJ) {
      static_assert(BM == BN, "one row pitch for both K-major operands");
      const uint32_t so = stage * STAGE;
      // kk is a compile-time value in the unrolled loop; the immediate needs it as one
      static_for<0, KK>([&](auto kc) {
        if (kc.value == kk) {
#pragma unroll
          for (int bm = 0; bm < NBM; ++bm)
            read_km(kmA[bm] + so, ic2<decltype(kc)::value * 16 * BM * 2>{}, fa[bm]);
#pragma unroll
          for (int bn = 0; bn < NBN; ++bn)
            read_km(kmB[bn] + so, ic2<decltype(kc)::value * 16 * BN * 2>{}, fb[bn]);
        }
      });
      (void)st;
      return;
    }
#pragma unroll
    for (int bm = 0; bm < NBM; ++bm) {
      const int row = wm * WM + bm * MS + l32;
      const uint32_t addr = st + row * RB + ((((KM / 8) * kk + h) ^ swz_rb<RB>(row)) << 4);
      asm volatile("ds_read_b128 %0, %1" : "=v"(fa[bm]) : "v"(addr) : "memory");
    }
#pragma unroll
    for (int bn = 0; bn < NBN; ++bn) {
      const int row = BM + wn * WN + bn * MS + l32;
      const uint32_t addr = st + row * RB + ((((KM / 8) * kk + h) ^ swz_rb<RB>(row)) << 4);
      asm volatile("ds_read_b128 %0, %1" : "=v"(fb[bn]) : "v"(addr) : "memory");
    }
  };
  // Wait until at most `pending` fragment reads are in flight; the empty statements tie the
  // fragments to the wait so no MFMA that reads them is scheduled above it.
  auto wait_frags = [&](auto pending, u32x4_t (&fa)[NBM], u32x4_t (&fb)[NBN]) {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(decltype(pending)::value));
#pragma unroll
    for (int bm = 0; bm < NBM; ++bm) asm volatile("" : "+v"(fa[bm]));
#pragma unroll
    for (int bn = 0; bn < NBN; ++bn) asm volatile("" : "+v"(fb[bn]));
  };
  // MFMAs of one k step; fills of the refilled stage are slotted in between them (at most
  // one fill per `gap` MFMAs) so the address FIFO drains while the matrix cores work.
  constexpr int MF = NBN * NBM;
  constexpr int PER_STEP = (LOADS + KK - 1) / KK;
  constexpr int GAP = MF / PER_STEP > 0 ? MF / PER_STEP : 1;
  auto mfma_step = [&](const u32x4_t (&fa)[NBM], const u32x4_t (&fb)[NBN], int fill_kt, int fill0) {
#pragma unroll
    for (int bn = 0; bn < NBN; ++bn)
#pragma unroll
      for (int bm = 0; bm < NBM; ++bm) {
        const int i = bn * NBM + bm;
        if constexpr (MS == 32)
          acc[bn][bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, fb[bn]), __builtin_bit_cast(bf16x8_t, fa[bm]),
              acc[bn][bm], 0, 0, 0);
        else
          acc[bn][bm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, fb[bn]), __builtin_bit_cast(bf16x8_t, fa[bm]),
              acc[bn][bm], 0, 0, 0);
        if (fill_kt >= 0 && i % GAP == GAP - 1) {
          const int idx = fill0 + i / GAP;
          if (i / GAP < PER_STEP && idx < LOADS) issue_one(fill_kt, idx);
        }
      }
  };

  // Pipeline: fills run NST-1 stages ahead. Each iteration waits for its stage, meets the
  // other waves at the barrier (after which the stage consumed one iteration earlier is
  // free and gets refilled, interleaved with this stage's MFMAs), then multiplies, reading
  // the next k step's fragments while the current step's MFMAs run.
  constexpr int NRD = (KMAJ ? 2 : 1) * (NBM + NBN);   // LDS reads of one k step's fragments
  static_assert(XS || NRD <= 15, "fragment reads exceed the lgkmcnt range");
  if constexpr (XS) {
    // Cross-stage pipeline (one wave per SIMD, K a multiple of BK, two 32-deep k slices per
    // stage). Slice step s multiplies fragments read during step s - 1 while it reads those
    // of step s + 1, one fragment between every few MFMAs. Before the second slice of a stage
    // each wave waits for its own fills of the next stage and meets the others at the
    // barrier: after it the next stage is complete in LDS (its first fragments are read
    // during this slice) and every wave has finished reading the current stage (its last
    // fragments are in registers), so the current stage's slot is refilled at once with the
    // stage NST ahead, the fills spread between this slice's MFMAs. Fragment reads never wait
    // on a barrier.
    static_assert(!PP && MS == 16 && KK == 2, "cross-stage pipeline layout");
    constexpr int NR = NBM + NBN;                        // fragment reads per slice
    constexpr int MFN = NBN * NBM;                       // MFMAs per slice
    constexpr int RG = (3 * MFN / 4) / NR > 0 ? (3 * MFN / 4) / NR : 1;   // MFMAs per read
    constexpr int FG = MFN / LOADS > 0 ? MFN / LOADS : 1;                 // MFMAs per fill
    // Per-lane LDS read addresses within a stage slot. The chunk swizzle depends on row bits
    // 1..4 only, and bit 4 of a block's rows is the parity of its 16-row block index, so one
    // base per (parity, k slice) serves every block; the block's row offset is the read's
    // immediate and the slot's offset is added once per slice.
    uint32_t ra[2][KK], rb[2][KK];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int rowa = wm * WM + q * MS + l32, rowb = BM + wn * WN + q * MS + l32;
        ra[q][kk] = lds_base + (rowa - q * MS) * RB + ((((KM / 8) * kk + h) ^ swz_rb<RB>(rowa)) << 4);
        rb[q][kk] = lds_base + (rowb - q * MS) * RB + ((((KM / 8) * kk + h) ^ swz_rb<RB>(rowb)) << 4);
      }
    u32x4_t fa[2][NBM], fb[2][NBN];
    // fragment R (activation block R, then weight block R - NBM) into buffer BU
    auto rd = [&](const uint32_t (&ba)[2], const uint32_t (&bb)[2], auto r_, auto buf_) {
      constexpr int R = decltype(r_)::value, BU = decltype(buf_)::value;
      if constexpr (R < NBM)
        ds_read16<R * MS * RB>(fa[BU][R], ba[R & 1]);
      else
        ds_read16<(R - NBM) * MS * RB>(fb[BU][R - NBM], bb[(R - NBM) & 1]);
    };
    // fill J of a stage into `slot`; koff past the last stage puts every lane out of range
    // (zeros land in a slot nobody reads again)
    auto fill_one = [&](uint32_t koff, int slot, auto j_) {
      constexpr int J = decltype(j_)::value;
      uint8_t *base = lds + slot * STAGE;
      if constexpr (J < A_INS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            a_rsrc, (lds_void_t *)(base + (wid * A_INS + J) * FR * RB), 16, a_off[J], koff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            b_rsrc[J - A_INS], (lds_void_t *)(base + (BM + (wid * B_INS + J - A_INS) * FR) * RB),
            16, b_off[J - A_INS], koff, 0, 0);
    };
    // slice KS of stage st; NEXT: read the fragments of the following slice during it
    auto slice = [&](int st, auto ks_, auto next_) {
      constexpr int KS = decltype(ks_)::value, C = KS, N = KS ^ 1;
      constexpr bool NEXT = decltype(next_)::value;
      constexpr bool LAST = KS == KK - 1;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int bm = 0; bm < NBM; ++bm) asm volatile("" : "+v"(fa[C][bm]));
#pragma unroll
      for (int bn = 0; bn < NBN; ++bn) asm volatile("" : "+v"(fb[C][bn]));
      uint32_t koff = kOOB;
      int slot = 0;
      if constexpr (LAST && NEXT) {
        wait_fills(min(NST - 2, nk - 2 - st));
        asm volatile("s_barrier" ::: "memory");
        koff = st + NST < nk ? (uint32_t)((st + NST) * BK * 2) : kOOB;
        slot = st % NST;
      }
      // read bases of the following slice: same stage, next k slice; or next stage, slice 0
      constexpr int NKS = LAST ? 0 : KS + 1;
      const uint32_t soff = (uint32_t)(((LAST ? st + 1 : st) % NST) * STAGE);
      uint32_t ba[2], bb[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        ba[q] = ra[q][NKS] + soff;
        bb[q] = rb[q][NKS] + soff;
      }
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, MFN>([&](auto i_) {
        constexpr int I = decltype(i_)::value;
        constexpr int BN_ = I / NBM, BM_ = I % NBM;
        acc[BN_][BM_] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, fb[C][BN_]), __builtin_bit_cast(bf16x8_t, fa[C][BM_]),
            acc[BN_][BM_], 0, 0, 0);
        if constexpr (NEXT && I % RG == 0 && I / RG < NR) {
          rd(ba, bb, ic2<I / RG>{}, ic2<N>{});
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (LAST && NEXT && I % FG == FG / 2 && I / FG < LOADS) {
          fill_one(koff, slot, ic2<I / FG>{});
          __builtin_amdgcn_sched_barrier(0);
        }
      });
      if constexpr (NEXT) {   // reads the MFMAs ran out before
        static_for<(MFN + RG - 1) / RG, NR>([&](auto r) { rd(ba, bb, r, ic2<N>{}); });
      }
      if constexpr (LAST && NEXT) {   // fills the MFMAs ran out before
        static_for<(MFN - FG / 2 + FG - 1) / FG, LOADS>([&](auto j) { fill_one(koff, slot, j); });
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int s0 = 0; s0 < NST && s0 < nk; ++s0)
      static_for<0, LOADS>([&](auto j) { fill_one((uint32_t)(s0 * BK * 2), s0, j); });
    wait_fills(min(NST - 1, nk - 1));
    asm volatile("s_barrier" ::: "memory");
    {
      uint32_t ba[2] = {ra[0][0], ra[1][0]}, bb[2] = {rb[0][0], rb[1][0]};
      static_for<0, NR>([&](auto r) { rd(ba, bb, r, ic2<0>{}); });
    }
    using T_ = std::true_type;
    using F_ = std::false_type;
    for (int st = 0; st + 1 < nk; ++st) {
      slice(st, ic2<0>{}, T_{});
      slice(st, ic2<1>{}, T_{});
    }
    slice(nk - 1, ic2<0>{}, T_{});
    slice(nk - 1, ic2<1>{}, F_{});
  } else if constexpr (PP) {
    // Phases alternate memory / matrix work; group 1 runs one phase behind group 0, and
    // every phase ends at a barrier of all 8 waves. Fills run D = NST-1 stages ahead: the
    // memory phase of step kt reads all of stage kt's fragments into registers and issues
    // this wave's fills of stage kt + D into the slot of stage kt - 1, which both groups
    // finished reading before the previous barrier. Before the barrier that ends phase
    // 2kt+1 every wave has its fills of stage kt + 1 complete, so both groups' later reads
    // of that stage see all of it.
    static_assert(WGM == 2 && WGM * WGN == 8 && NST >= 3, "ping-pong layout");
    static_assert(KK * (NBM + NBN) <= 15, "fragment reads exceed the lgkmcnt range");
    constexpr int D = NST - 1;
    const int grp = wm;
    for (int s = 0; s < D && s < nk; ++s) issue(s);
    wait_fills(min(D - 1, nk - 1));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (grp == 1) asm volatile("s_barrier" ::: "memory");
    u32x4_t fa[KK][NBM], fb[KK][NBN];
    for (int kt = 0; kt < nk; ++kt) {
      // ---- memory phase
      const int stage = kt % NST;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) read_frags(stage, kk, fa[kk], fb[kk]);
      if (kt + D < nk) issue(kt + D);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int bm = 0; bm < NBM; ++bm) asm volatile("" : "+v"(fa[kk][bm]));
#pragma unroll
        for (int bn = 0; bn < NBN; ++bn) asm volatile("" : "+v"(fb[kk][bn]));
      }
      if (grp == 1) wait_fills(min(D - 1, nk - 2 - kt));
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      // ---- matrix phase
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) mfma_step(fa[kk], fb[kk], -1, 0);
      if (grp == 0) wait_fills(min(D - 1, nk - 2 - kt));
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    if (grp == 0) asm volatile("s_barrier" ::: "memory");
  } else {
  for (int s = 0; s < NST - 1 && s < nk; ++s) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    wait_fills(min(NST - 2, nk - 1 - kt));
    // every wave's fills of stage kt are in LDS, and every wave's reads of the stage that
    // is refilled next have completed
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    int fill_kt = kt + NST - 1 < nk ? kt + NST - 1 : -1;
    if constexpr (EARLY) {
      if (fill_kt >= 0) issue(fill_kt);
      fill_kt = -1;
    }
    const int stage = kt % NST;
    u32x4_t fa[2][NBM], fb[2][NBN];
    read_frags(stage, 0, fa[0], fb[0]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + 1 < KK) {
        read_frags(stage, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
        wait_frags(std::integral_constant<int, NRD>{}, fa[kk & 1], fb[kk & 1]);
      } else {
        wait_frags(std::integral_constant<int, 0>{}, fa[kk & 1], fb[kk & 1]);
      }
      // keep each step's MFMAs between its wait and the next step's reads: sunk below the
      // next wait they would stall on reads they do not need
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(fa[kk & 1], fb[kk & 1], fill_kt, kk * PER_STEP);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  }
  // 16 x 16 blocks of the SwiGLU product leave the accumulators straight to global memory (each
  // lane holds 4 consecutive hidden units of one row), without staging the tile in LDS. The
  // large plain-store output (the logits) must leave in whole 128-byte lines: written from
  // registers in 32-byte row pieces it took 1.4x as long (measured), so it and the QKV
  // product stage through LDS.
  if constexpr (MS == 16 && EPI == EPI_SWIGLU) {
    swiglu_direct_epilogue<NBM, NBN, WM, WN>(g, acc, m0, n0, wm, wn, h, l32);
    return;
  }
  __syncthreads();  // every wave is done with the ring: reuse it to stage the output

  if constexpr (EPI == EPI_XENT) {
    // ---- cross-entropy partials ("LLM 2" Optimize / Loss: logsumexp with the max taken
    //      out). Lane holds row m = m0 + wm*WM + bm*MS + l32 and the columns
    //      n = n0 + wn*WN + bn*32 + 8q + 4h + r (32x32 blocks) or n0 + wn*WN + bn*16 + 4h + r
    //      (16x16 blocks). Per row: max over the lane's columns, over the lanes that hold the
    //      row's other columns (permlane swaps: the two lane halves, and for 16x16 blocks the
    //      four 16-lane rows), then over the WGN waves along N (LDS); the same for the sum of
    //      exp(logit - max). The logits stay in registers. Column bounds are only checked in
    //      the last column tile.
    constexpr float kLog2e = 1.4426950408889634f;
    float *red = (float *)lds;   // [BM][WGN]
    const int nw0 = n0 + wn * WN;
    const bool full = n0 + BN <= g.N;
    auto col_of = [&](int bn, int e) {   // column of element e of block bn, within the wave
      return MS == 32 ? bn * 32 + 8 * (e >> 2) + 4 * h + (e & 3) : bn * 16 + 4 * h + e;
    };
    auto col_ok = [&](int bn, int e) { return full || nw0 + col_of(bn, e) < g.N; };
    // the same op over the lanes holding the row's columns
    auto lanes_op = [&](float v, auto op) {
      if constexpr (MS == 16) {
        const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                          false, false);
        v = op(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
      }
      const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                        false, false);
      return op(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    };
    float rmax[NBM];
#pragma unroll
    for (int bm = 0; bm < NBM; ++bm) {
      const int rt = wm * WM + bm * MS + l32;
      float mx = -__builtin_inff();
#pragma unroll
      for (int bn = 0; bn < NBN; ++bn)
#pragma unroll
        for (int e = 0; e < AE; ++e)
          if (col_ok(bn, e)) mx = fmaxf(mx, acc[bn][bm][e]);
      mx = lanes_op(mx, [](float x, float y) { return fmaxf(x, y); });
      if (h == 0) red[rt * WGN + wn] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int bm = 0; bm < NBM; ++bm) {
      const int rt = wm * WM + bm * MS + l32;
      float mx = -__builtin_inff();
#pragma unroll
      for (int w = 0; w < WGN; ++w) mx = fmaxf(mx, red[rt * WGN + w]);
      rmax[bm] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int bm = 0; bm < NBM; ++bm) {
      const int rt = wm * WM + bm * MS + l32;
      const int64_t m = m0 + rt;
      const float mc = rmax[bm] * kLog2e;
      float se = 0.f;
#pragma unroll
      for (int bn = 0; bn < NBN; ++bn)
#pragma unroll
        for (int e = 0; e < AE; ++e)
          if (col_ok(bn, e)) se += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[bn][bm][e], kLog2e, -mc));
      se = lanes_op(se, [](float x, float y) { return x + y; });
      if (h == 0) red[rt * WGN + wn] = se;
      // the row's target logit, if its column is one of this wave's (rare: one column tile)
      const int tr = (m < g.M ? g.targets[m] : -1) - nw0;
      const int th = MS == 32 ? (tr >> 2) & 1 : (tr & 15) >> 2;   // lane group holding it
      const bool mine = tr >= 0 && tr < WN && th == h;
      if (__any(mine)) {
        float tv = 0.f;
#pragma unroll
        for (int bn = 0; bn < NBN; ++bn)
#pragma unroll
          for (int e = 0; e < AE; ++e)
            if (tr == col_of(bn, e)) tv = acc[bn][bm][e];
        if (mine) g.x_tgt[m] = tv;
      }
    }
    __syncthreads();
    if (wn == 0 && h == 0) {
#pragma unroll
      for (int bm = 0; bm < NBM; ++bm) {
        const int rt = wm * WM + bm * MS + l32;
        const int64_t m = m0 + rt;
        if (m >= g.M) continue;
        float se = 0.f;
#pragma unroll
        for (int w = 0; w < WGN; ++w) se += red[rt * WGN + w];
        g.x_max[(int64_t)tn * g.M + m] = rmax[bm];
        g.x_sum[(int64_t)tn * g.M + m] = se;
      }
    }
    return;
  }

  // ---- epilogue: final values -> LDS (output dtype, row-major tile) -> coalesced rows.
  //      Lane holds acc[bn][bm][4q + r] for m = m0 + wm*WM + bm*MS + l32 and
  //      n = n0 + wn*WN + bn*MS + 8q + 4h + r (MS = 32, q < 4) or + 4h + r (MS = 16).
  // the SwiGLU backward stages du in fp32 and writes bf16 da, dc from the coalesced pass
  const bool out_bf16 = EPI == EPI_RESIDUAL || EPI == EPI_SWIGLU_BACK ? false : g.y_dt == DT_BF16;
  const int ob = out_bf16 ? 2 : 4;
  const int rb = OUT_COLS * ob;
  const int passes = kRes ? RES_PASSES : (BM * rb > LDS ? 2 : 1);
  static_assert(!kRes || RES_LDS == LDS, "residual pass split");
  const int prow = BM / passes;
  const int ncols = EPI == EPI_SWIGLU || EPI == EPI_XENT_GRAD ? g.n0 : g.N;
  const int nout0 = EPI == EPI_SWIGLU ? n0 / 2 : n0;
  const bool vec_ok = ((g.ldy * ob) & 15) == 0;
#pragma unroll
  for (int p = 0; p < passes; ++p) {
    if (passes == 1 || (2 * wm) / WGM == p) {
      // RoPE: the (cos, sin) pairs of a row block are all loaded before any is used, and the
      // next block's while this one is rotated, so the table reads cost one latency instead
      // of one per output group. Indices are clamped into the table; a position outside it
      // turns the rotated values into NaN below.
      constexpr int NQ = EPI == EPI_QKV_ROPE ? NBN * (AE / 4) : 1;
      f32x4_t csr[2][NQ];
      bool pok[2] = {true, true};
      // The integer divisions are taken once per lane, not per row block: a column group's
      // offset in a position's (cos, sin) row is the same for every row (its column within the
      // head; columns come in groups of 4 and d_head is even, so it is the pair index times 2),
      // and without a positions array the rows of block bm are tokens MS bm further on, i.e.
      // the first block's position stepped with wrap-around at S. Rows fit in 32 bits here
      // (M * row width < 2^31 elements).
      int cso[NQ];
      int pbase = 0;
      if constexpr (EPI == EPI_QKV_ROPE) {
        const int dmask = g.d_head - 1;
        const bool pow2 = (g.d_head & dmask) == 0;
#pragma unroll
        for (int bn = 0; bn < NBN; ++bn)
#pragma unroll
          for (int q = 0; q < AE / 4; ++q) {
            const int n = n0 + wn * WN + bn * MS + (MS == 32 ? 8 * q + 4 * h : 4 * h);
            cso[bn * (AE / 4) + q] = pow2 ? (n & dmask) : n % g.d_head;
          }
        if (!g.positions) pbase = (int)(m0 + wm * WM + l32) % g.S;
      }
      auto load_cs = [&](int bm, f32x4_t (&c)[NQ], bool &ok) {
        int pos;
        if (g.positions) {
          const int64_t m = m0 + wm * WM + bm * MS + l32;
          pos = g.positions[m < g.M ? m : g.M - 1];
        } else {
          pos = pbase + bm * MS;
          while (pos >= g.S) pos -= g.S;
        }
        ok = pos >= 0 && pos < g.max_seq;
        const float *row = g.cos_sin + (int64_t)(ok ? pos : 0) * g.d_head;
#pragma unroll
        for (int i = 0; i < NQ; ++i) c[i] = *(const f32x4_t *)(row + cso[i]);
      };
      // a tile of v columns only (a third of the tiles) rotates nothing: no table reads
      const bool tile_rope = EPI == EPI_QKV_ROPE && n0 < g.n0 + g.n1;
      if constexpr (EPI == EPI_QKV_ROPE)
        if (tile_rope) load_cs(0, csr[0], pok[0]);
      // RMSNorm split across the products: each of the lane's rows gets 1 / rms(x) from the
      // producer's per-tile sums of squares (summed in tile order), all read up front
      float rsv[NBM];
#pragma unroll
      for (int bm = 0; bm < NBM; ++bm) rsv[bm] = 1.f;
      if constexpr (EPI == EPI_QKV_ROPE || EPI == EPI_SWIGLU) {
        if (g.rs_part) split_norm_scales<NBM, MS, WM>(g, m0, wm, l32, rsv);
      }
      const bool xfull = n0 + BN <= g.N;   // cross-entropy gradient: no padded column here
#pragma unroll
      for (int bm = 0; bm < NBM; ++bm) {
        const int r = wm * WM + bm * MS + l32 - p * prow;
        if constexpr (EPI == EPI_QKV_ROPE)
          if (tile_rope && bm + 1 < NBM) load_cs(bm + 1, csr[(bm + 1) & 1], pok[(bm + 1) & 1]);
#pragma unroll
        for (int bn = 0; bn < (EPI == EPI_SWIGLU ? NBN / 2 : NBN); ++bn) {
#pragma unroll
          for (int q = 0; q < AE / 4; ++q) {
            f32x4_t v;
            int col;
            const int nq = MS == 32 ? 8 * q + 4 * h : 4 * h;   // n of the lane's 4 values
            if constexpr (EPI == EPI_SWIGLU) {
              // virtual weight rows come in 64-row groups, 32 gate rows then their 32 up
              // rows; gate block gb pairs with up block ub of the same hidden units
              const int gb = MS == 32 ? 2 * bn : 4 * (bn >> 1) + (bn & 1);
              const int ub = MS == 32 ? 2 * bn + 1 : gb + 2;
              col = wn * WN / 2 + bn * MS + nq;
              // SiLU(a) b = a b / (1 + 2^(-a log2 e)) with the hardware exp2 and reciprocal
              // (about 1 ulp each, far inside the bf16 rounding that follows); a very negative
              // a gives 2^(+big) = inf, a reciprocal of 0 and SiLU = -0
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                const float a = acc[gb][bm][4 * q + x] * rsv[bm], b = acc[ub][bm][4 * q + x] * rsv[bm];
                v[x] = a * b *
                       __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * 1.4426950408889634f));
              }
            } else {
              col = wn * WN + bn * MS + nq;
#pragma unroll
              for (int x = 0; x < 4; ++x) v[x] = acc[bn][bm][4 * q + x] * rsv[bm];
              if constexpr (EPI == EPI_QKV_ROPE) {
                const int n = n0 + col;
                if (n < g.n0 + g.n1) {  // q and k columns rotate; v columns pass through
                  if (pok[bm & 1]) {
                    const f32x4_t cs = csr[bm & 1][bn * (AE / 4) + q];
                    const float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
                    v[0] = x0 * cs[0] - x1 * cs[1];
                    v[1] = x0 * cs[1] + x1 * cs[0];
                    v[2] = x2 * cs[2] - x3 * cs[3];
                    v[3] = x2 * cs[3] + x3 * cs[2];
                  } else {
                    const float nan = __builtin_nanf("");
                    v = f32x4_t{nan, nan, nan, nan};
                  }
                }
              }
              if constexpr (EPI == EPI_XENT_GRAD) {
                // (softmax(z) - onehot(t)) / count as 2^(z log2 e - xl) with the row's offset
                // xl (log2 units) = lse log2 e + log2 count; the hardware exp2 (about 1 ulp) is
                // far inside the bf16 rounding of the stored gradient. Rows without a target
                // and padded columns store 0.
                const int n = n0 + col;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                  const float e =
                      __builtin_amdgcn_exp2f(__builtin_fmaf(v[x], 1.4426950408889634f, -xl[bm]));
                  v[x] = xt[bm] >= 0 ? e : 0.f;
                }
                const int tc = xt[bm] - n;
                if ((unsigned)tc < 4u) {
#pragma unroll
                  for (int x = 0; x < 4; ++x)
                    if (x == tc) v[x] -= xinv;
                }
                if (!xfull) {
#pragma unroll
                  for (int x = 0; x < 4; ++x)
                    if (n + x >= g.N) v[x] = 0.f;
                }
              }
            }
            // bf16: rows with bit 3 set keep the two 8-byte halves of their chunks swapped,
            // so the 16 rows of one 8-byte store cover distinct banks (rows r and r ^ 8 would
            // otherwise share them); the reading pass swaps them back
            uint8_t *dst = lds + (stage_off(r, col * ob, rb) ^ (out_bf16 ? (r & 8) : 0));
            if (out_bf16) {
              uint2 u;
              u.x = pack_bf16x2(v[0], v[1]);
              u.y = pack_bf16x2(v[2], v[3]);
              *(uint2 *)dst = u;
            } else {
              *(f32x4_t *)dst = v;
            }
          }
        }
      }
    }
    __syncthreads();
    // coalesced stores: consecutive threads take consecutive 16-byte chunks of a row
    const int cpr = rb >> 4, epc = 16 / ob;
    if constexpr (EPI == EPI_SWIGLU_BACK) {
      // SwiGLU backward: a thread takes 16-byte chunks (4 du values) of the staged rows, reads
      // the forward's gate a and up c of those hidden units (8 bytes each, all loads issued
      // before any is used) and writes da = du c s (1 + a (1 - s)), dc = du a s, s =
      // sigmoid(a), side by side in one row of y (dc N columns after da). N is a multiple
      // of 4, so a chunk is whole or past N.
      constexpr int CPR = BN / 4;
      constexpr int SB_PASSES = BM * BN * 4 > LDS ? 2 : 1;
      constexpr int SB_ROWS = BM / SB_PASSES, IT = SB_ROWS * CPR / NT;
      static_assert(IT * NT == SB_ROWS * CPR, "SwiGLU backward chunk split");
      constexpr int IB = 4;   // chunks whose loads are in flight together
      static_assert(IT % IB == 0, "SwiGLU backward batches");
      const bf16_t *ka = (const bf16_t *)g.keep_a, *kc = (const bf16_t *)g.keep_c;
#pragma unroll
      for (int i0 = 0; i0 < IT; i0 += IB) {
        f32x4_t dv[IB];
        u32x2_t av[IB], cv[IB];
#pragma unroll
        for (int i = 0; i < IB; ++i) {
          const int idx = tid + (i0 + i) * NT, r = idx / CPR, cc = idx % CPR;
          const int64_t m = m0 + p * SB_ROWS + r;
          const int n = n0 + 4 * cc;
          const int64_t ko = m < g.M && n < g.N ? m * g.N + n : 0;
          av[i] = *(const u32x2_t *)(ka + ko);
          cv[i] = *(const u32x2_t *)(kc + ko);
          dv[i] = *(const f32x4_t *)(lds + stage_off(r, cc * 16, rb));
        }
#pragma unroll
        for (int i = 0; i < IB; ++i) {
          const int idx = tid + (i0 + i) * NT, r = idx / CPR, cc = idx % CPR;
          const int64_t m = m0 + p * SB_ROWS + r;
          const int n = n0 + 4 * cc;
          if (m >= g.M || n >= g.N) continue;
          float da[4], dc[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const uint32_t aw = av[i][x >> 1], cw = cv[i][x >> 1];
            const float a = __uint_as_float((x & 1) ? (aw & 0xffff0000u) : (aw << 16));
            const float c = __uint_as_float((x & 1) ? (cw & 0xffff0000u) : (cw << 16));
            // sigmoid with the hardware exp2 and reciprocal (about 1 ulp each, inside the
            // bf16 rounding that follows)
            const float sg =
                __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * 1.4426950408889634f));
            da[x] = dv[i][x] * c * sg * (1.0f + a * (1.0f - sg));
            dc[x] = dv[i][x] * a * sg;
          }
          bf16_t *pa = (bf16_t *)g.y + m * g.ldy + n;
          *(u32x2_t *)pa = u32x2_t{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3])};
          *(u32x2_t *)(pa + g.N) =
              u32x2_t{pack_bf16x2(dc[0], dc[1]), pack_bf16x2(dc[2], dc[3])};
        }
      }
    } else if constexpr (kRes) {
      // a fresh copy of the thread id: without it the compiler keeps every chunk's address
      // from the prefetch alive through the main loop (and spills)
      int tid_e = tid;
      asm volatile("" : "+v"(tid_e));
      const bool fuse = g.nrm_y != nullptr;
      // fused RMSNorm: each chunk's sum of squares, [row][chunk] after this pass's staged rows
      constexpr int PSQ_LD = RES_CPR + 1;
      static_assert(!kRes || (BM / RES_PASSES) * (BN * 4 + PSQ_LD * 4) <= LDS,
                    "fused RMSNorm partials do not fit");
      float *psq = (float *)(lds + prow * rb);
#pragma unroll
      for (int i = 0; i < RES_IT; ++i) {
        const int idx = tid_e + i * NT;
        const int r = idx / RES_CPR, c = idx % RES_CPR;
        const int64_t m = m0 + p * prow + r;
        const int n = n0 + c * 4;
        float sq = 0.f;
        if (m < g.M && n < g.N) {
          const f32x4_t v = *(const f32x4_t *)(lds + stage_off(r, c * 16, rb));
          const int64_t off = m * g.ldy + n;
          float *y = (float *)g.y + off;
          if (vec_ok && n + 4 <= g.N) {
            const f32x4_t xv = v + resv[p * RES_IT + i];
            *(f32x4_t *)y = xv;
            if (fuse) {
              const uint2 gg = gnv[p * RES_IT + i];
              sq = xv[0] * xv[0] + xv[1] * xv[1] + xv[2] * xv[2] + xv[3] * xv[3];
              uint2 hv;
              hv.x = pack_bf16x2(xv[0] * __uint_as_float(gg.x << 16),
                                 xv[1] * __uint_as_float(gg.x & 0xffff0000u));
              hv.y = pack_bf16x2(xv[2] * __uint_as_float(gg.y << 16),
                                 xv[3] * __uint_as_float(gg.y & 0xffff0000u));
              *(uint2 *)((bf16_t *)g.nrm_y + off) = hv;
            }
          } else {
            const float *res = g.residual + off;
            for (int x = 0; x < 4 && n + x < g.N; ++x) {
              const float xv = v[x] + res[x];
              y[x] = xv;
              if (fuse) {
                sq += xv * xv;
                ((bf16_t *)g.nrm_y)[off + x] =
                    f32_to_bf16(xv * bf16_to_f32(((const bf16_t *)g.nrm_g)[n + x]));
              }
            }
          }
        }
        if (fuse) psq[r * PSQ_LD + c] = sq;
      }
      if (fuse) {
        // each row's sum over the tile's columns: TPR consecutive lanes per row each sum a
        // run of chunks in order, then the runs are added pairwise across the lanes (a fixed
        // order, so the partial is deterministic)
        __syncthreads();
        constexpr int PROW = BM / RES_PASSES, TPR = NT / PROW;
        if constexpr (TPR >= 1 && TPR <= 4 && (TPR & (TPR - 1)) == 0 && TPR * PROW == NT &&
                      RES_CPR % TPR == 0) {
          constexpr int RUN = RES_CPR / TPR;
          const int r = tid / TPR, part = tid % TPR;
          float ss = 0.f;
#pragma unroll
          for (int c = 0; c < RUN; ++c) ss += psq[r * PSQ_LD + part * RUN + c];
#pragma unroll
          for (int o = 1; o < TPR; o <<= 1) ss += __shfl_xor(ss, o);
          const int64_t m = m0 + p * prow + r;
          if (part == 0 && m < g.M) g.nrm_part[m * kNormParts + tn] = ss;
        } else if (tid < prow) {
          const int64_t m = m0 + p * prow + tid;
          float ss = 0.f;
          for (int c = 0; c < RES_CPR; ++c) ss += psq[tid * PSQ_LD + c];
          if (m < g.M) g.nrm_part[m * kNormParts + tn] = ss;
        }
      }
    } else {
    for (int idx = tid; idx < prow * cpr; idx += NT) {
      const int r = idx / cpr, c = idx - r * cpr;
      const int64_t m = m0 + p * prow + r;
      const int n = nout0 + c * epc;
      if (m >= g.M || n >= ncols) continue;
      uint4 raw = *(const uint4 *)(lds + stage_off(r, c * 16, rb));
      if (out_bf16 && (r & 8)) raw = uint4{raw.z, raw.w, raw.x, raw.y};
      const int64_t off = m * g.ldy + n;
      if (out_bf16) {
        bf16_t *y = (bf16_t *)g.y + off;
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
        if (vec_ok && n + 8 <= ncols) {
          if constexpr (EPI == EPI_STORE || EPI == EPI_XENT_GRAD)   // streamed out
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, raw), (u32x4_t *)y);
          else
            *(uint4 *)y = raw;
        } else if (n + 8 <= ncols && (off & 1) == 0) {
          // row stride not a multiple of 8 elements: 4-byte stores on an even element
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            if constexpr (EPI == EPI_STORE || EPI == EPI_XENT_GRAD)
              __builtin_nontemporal_store(w4[x], (uint32_t *)y + x);
            else
              ((uint32_t *)y)[x] = w4[x];
          }
        } else if (n + 8 <= ncols) {
          // odd element offset: one 2-byte store, three 4-byte stores, one 2-byte store
          y[0] = (bf16_t)(w4[0] & 0xffffu);
#pragma unroll
          for (int x = 0; x < 3; ++x)
            *(uint32_t *)(y + 1 + 2 * x) = (w4[x] >> 16) | (w4[x + 1] << 16);
          y[7] = (bf16_t)(w4[3] >> 16);
        } else {
          for (int x = 0; x < 8 && n + x < ncols; ++x)
            y[x] = (bf16_t)((x & 1) ? (w4[x >> 1] >> 16) : (w4[x >> 1] & 0xffffu));
        }
      } else {
        float *y = (float *)g.y + off;
        f32x4_t v = __builtin_bit_cast(f32x4_t, raw);
        if (vec_ok && n + 4 <= ncols) {
          if constexpr (EPI == EPI_STORE || EPI == EPI_XENT_GRAD)
            __builtin_nontemporal_store(v, (f32x4_t *)y);
          else
            *(f32x4_t *)y = v;
        } else {
          for (int x = 0; x < 4 && n + x < ncols; ++x) y[x] = v[x];
        }
      }
    }
    }
    if (p + 1 < passes) __syncthreads();
  }

#endif
}

template <int BM, int BN, int BK, int NST, int EPI, int OCC = 1, bool EARLY = false, int WGM = 2,
          int WGN = 2, bool PP = false, int MS = 32, bool XS = false, bool KMAJ = false>
__global__ __launch_bounds__(64 * WGM * WGN, OCC) void gemm_bf16_kernel(GemmArgs g0, int tiles_m,
                                                                        int tiles_n) {
  const GemmArgs g = k_part<bf16_t, KMAJ>(g0);
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  gemm_bf16_tile<BM, BN, BK, NST, EPI, OCC, EARLY, WGM, WGN, PP, MS, XS, KMAJ>(g, tm, tn);
}

// Several weight-gradient products over the same tokens in one launch, one 128 x 128 tile of
// one product per workgroup and the whole token range per tile (no split, no partial sums):
// a layer's products together launch enough tiles to fill the chip. Workgroup ids map to a
// contiguous run of the concatenated tiles per XCD; inside a product the tiles go in the
// grouped order of tile_coords.
__global__ __launch_bounds__(256, 2) void gemm_wgrad_group_kernel(WgradGroup grp) {
  const int T = grp.start[grp.njobs];
  const int bid = blockIdx.x, xcd = bid & 7, local = bid >> 3;
  const int per = T >> 3, extra = T & 7;
  const int logical = xcd * per + min(xcd, extra) + local;
  GemmArgs g{};
  int t0 = 0, tiles_m = 1;
#pragma unroll
  for (int j = 0; j < kWgradJobs; ++j) {
    if (j < grp.njobs && logical >= grp.start[j]) {
      const WgradJob &jb = grp.job[j];
      g.a = jb.a; g.lda = jb.lda; g.w0 = jb.b; g.ldw = jb.ldb; g.M = jb.M; g.N = jb.N;
      g.y = jb.y; g.ldy = jb.ldy;
      t0 = grp.start[j];
      tiles_m = (jb.M + 127) / 128;
    }
  }
  g.K = grp.K;
  g.y_dt = DT_F32;
  const int tiles_n = (g.N + 127) / 128;
  const int in = logical - t0;
  const int group = in / (kGroupM * tiles_n), first_m = group * kGroupM;
  const int gm = min(kGroupM, tiles_m - first_m), r = in - group * kGroupM * tiles_n;
  gemm_bf16_tile<128, 128, 64, 2, EPI_STORE, 2, true, 2, 2, false, 32, false, true>(
      g, first_m + r % gm, r / gm);
}

// ------------------------------------------------------------------ f32 kernel

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_f32_kernel(GemmArgs g0, int tiles_m,
                                                               int tiles_n) {
  const GemmArgs g = k_part<float>(g0);
  constexpr int CE = 4;                              // floats per 16-byte chunk
  constexpr int BKE = kRowBytes / 4;                 // K elements per stage
  constexpr int A_LD = BM * kChunks / kThreads;
  constexpr int W_LD = BN * kChunks / kThreads;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int NBM = WM / 32, NBN = WN / 32;
  constexpr int STAGE = (BM + BN) * kRowBytes;

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid & 1, wn = wid >> 1;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;

  const float *a_src[A_LD];
  bool a_ok[A_LD];
  int a_lds[A_LD], a_k[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int c = tid + kThreads * i, row = c >> 3, ch = c & 7;
    const int64_t m = m0 + row;
    a_ok[i] = m < g.M;
    a_src[i] = (const float *)g.a + (a_ok[i] ? m : 0) * g.lda + ch * CE;
    a_k[i] = ch * CE;
    a_lds[i] = row * kRowBytes + ((ch ^ swz(row)) << 4);
  }
  const float *w_src[W_LD];
  bool w_ok[W_LD];
  int w_lds[W_LD], w_k[W_LD];
#pragma unroll
  for (int i = 0; i < W_LD; ++i) {
    const int c = tid + kThreads * i, row = c >> 3, ch = c & 7;
    int rows_left;
    w_src[i] = weight_rows<EPI, float>(g, n0 + row, rows_left) + ch * CE;
    w_ok[i] = rows_left > 0;
    w_k[i] = ch * CE;
    w_lds[i] = BM * kRowBytes + row * kRowBytes + ((ch ^ swz(row)) << 4);
  }

  const int nk = (g.K + BKE - 1) / BKE;
  f32x4_t ra[A_LD], rw[W_LD];
  auto gload = [&](int kt) {
    const int kb = kt * BKE;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      f32x4_t v = {0.f, 0.f, 0.f, 0.f};
      if (a_ok[i] && kb + a_k[i] < g.K) v = *(const f32x4_t *)(a_src[i] + kb);
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < W_LD; ++i) {
      f32x4_t v = {0.f, 0.f, 0.f, 0.f};
      if (w_ok[i] && kb + w_k[i] < g.K) v = *(const f32x4_t *)(w_src[i] + kb);
      rw[i] = v;
    }
  };
  auto sstore = [&](int buf) {
    uint8_t *base = lds + buf * STAGE;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *(f32x4_t *)(base + a_lds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < W_LD; ++i) *(f32x4_t *)(base + w_lds[i]) = rw[i];
  };

  f32x16_t acc[NBN][NBM];
#pragma unroll
  for (int bn = 0; bn < NBN; ++bn)
#pragma unroll
    for (int bm = 0; bm < NBM; ++bm)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bn][bm][e] = 0.f;

  const int h = lane >> 5, l32 = lane & 31;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t *As = lds + buf * STAGE;
    const uint8_t *Ws = As + BM * kRowBytes;
#pragma unroll
    for (int kg = 0; kg < kChunks / 2; ++kg) {
      f32x4_t fb[NBM], fa[NBN];
#pragma unroll
      for (int bm = 0; bm < NBM; ++bm) {
        const int row = wm * WM + bm * 32 + l32;
        fb[bm] = *(const f32x4_t *)(As + row * kRowBytes + (((2 * kg + h) ^ swz(row)) << 4));
      }
#pragma unroll
      for (int bn = 0; bn < NBN; ++bn) {
        const int row = wn * WN + bn * 32 + l32;
        fa[bn] = *(const f32x4_t *)(Ws + row * kRowBytes + (((2 * kg + h) ^ swz(row)) << 4));
      }
#pragma unroll
      for (int bn = 0; bn < NBN; ++bn)
#pragma unroll
        for (int bm = 0; bm < NBM; ++bm)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[bn][bm] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[bn][e], fb[bm][e], acc[bn][bm],
                                                               0, 0, 0);
    }
    asm volatile("" ::: "memory");  // keep the next stage's LDS stores after this stage's MFMAs
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }
  epilogue<EPI, NBM, NBN>(g, acc, m0 + wm * WM, n0 + wn * WN, lane);
}

template <int BM, int BN, int EPI>
void grid_for(const GemmArgs &g, int64_t &tm, int64_t &tn) {
  tm = (g.M + BM - 1) / BM;
  tn = EPI == EPI_SWIGLU ? (g.n0 + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN;
}

template <int BM, int BN, int BK, int NST, int EPI, int OCC = 1, bool EARLY = false, int WGM = 2,
          int WGN = 2, bool PP = false, int MS = 32, bool XS = false, bool KMAJ = false>
hipError_t run_bf16(const GemmArgs &g, hipStream_t s) {
  int64_t tm, tn;
  grid_for<BM, BN, EPI>(g, tm, tn);
  if (tm * tn == 0) return hipSuccess;
  if (tm * tn > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, NST, EPI, OCC, EARLY, WGM, WGN, PP, MS, XS, KMAJ>),
                     dim3((unsigned)(tm * tn), g.kparts > 1 ? g.kparts : 1), dim3(64 * WGM * WGN), 0,
                     s, g, (int)tm, (int)tn);
  return hipGetLastError();
}

template <int BM, int BN, int EPI>
hipError_t run_f32(const GemmArgs &g, hipStream_t s) {
  int64_t tm, tn;
  grid_for<BM, BN, EPI>(g, tm, tn);
  if (tm * tn == 0) return hipSuccess;
  if (tm * tn > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, EPI>), dim3((unsigned)(tm * tn), g.kparts > 1 ? g.kparts : 1), dim3(kThreads), 0,
                     s, g, (int)tm, (int)tn);
  return hipGetLastError();
}

hipError_t dispatch_bf16(int epi, const GemmArgs &g, hipStream_t s) {
  switch (epi) {
    // Tile shapes chosen per epilogue by sweeps on the decoder's GEMM shapes with random
    // operands of the real scale.
    // The choices are checked by the whole forward, same box, variants alternated: the chip
    // runs the step at its power limit, so a kernel that is faster alone can make the step
    // slower (the LM head on the 256 x 256 ping-pong kernel: 650 against 693 us alone, but
    // 3.39 against 3.28 ms per forward step; 128 x 96 residual and 128 x 192 QKV tiles of 4
    // waves: 6-12 % faster alone, 3.452 against 3.435 ms per step). QKV + RoPE on the
    // 192 x 128 16x16 tiles of the plain store: 3.24 against 3.38 ms per step (QKV 47 against
    // 54 us); residual products on those tiles: 3.62 ms, SwiGLU on them: no gain. Residual
    // products on 16x16 blocks of the same 128 x 192 tiles: 3.179 against 3.197 ms.
    // The cross-stage pipeline (K a multiple of 64, not split), same-box A/B over three
    // alternating rounds of the d768 step: LM head 582 against 597 us, SwiGLU (8 waves, plain
    // order instead of ping-pong) 57.6 against 60.6, down / out projections 38.0 / 24.8
    // against 39.3 / 25.3; step 2.795 against 2.868 ms. With one wave per SIMD (256 x 256 and
    // 256 x 288 tiles, one workgroup per CU) the same loop was slower (LM head 747-829 us):
    // nothing covers a wave's memory stalls there.
    case EPI_STORE:
      // narrow outputs (the backward's input-gradient products, N = d_model): 128 x 96 tiles
      // launch twice the workgroups of 192 x 128 ones, two per CU at M = 8192, N = 768
      // (alone: 28 against 40 us at K = 2048, 696 against 799 us at K = 50304)
      if (g.K % 64 == 0 && g.kparts <= 1 && g.N <= 1024)
        return run_bf16<128, 96, 64, 2, EPI_STORE, 2, false, 2, 2, false, 16, true>(g, s);
      if (g.K % 64 == 0 && g.kparts <= 1)
        return run_bf16<192, 128, 64, 2, EPI_STORE, 2, false, 2, 2, false, 16, true>(g, s);
      return run_bf16<192, 128, 64, 2, EPI_STORE, 2, true, 2, 2, false, 16>(g, s);
    case EPI_RESIDUAL:
      if (g.K % 64 == 0 && g.kparts <= 1)
        return run_bf16<128, kResidualBN, 64, 4, EPI_RESIDUAL, 1, false, 4, 2, false, 16, true>(g, s);
      return run_bf16<128, kResidualBN, 64, 4, EPI_RESIDUAL, 1, true, 4, 2, false, 16>(g, s);
    case EPI_QKV_ROPE:
      if (g.K % 64 == 0 && g.kparts <= 1)
        return run_bf16<192, 128, 64, 2, EPI_QKV_ROPE, 2, false, 2, 2, false, 16, true>(g, s);
      return run_bf16<192, 128, 64, 2, EPI_QKV_ROPE, 2, true, 2, 2, false, 16>(g, s);
    case EPI_SWIGLU:
      if (g.K % 64 == 0 && g.kparts <= 1)
        return run_bf16<256, 256, 64, 2, EPI_SWIGLU, 1, false, 2, 4, false, 16, true>(g, s);
      return run_bf16<256, 256, 32, 4, EPI_SWIGLU, 1, false, 2, 4, true, 16>(g, s);
    case EPI_XENT:
      if (g.K % 64 == 0 && g.kparts <= 1)
        return run_bf16<kXentBM, kXentBN, 64, 2, EPI_XENT, 2, false, 2, 2, false, 16, true>(g, s);
      return run_bf16<kXentBM, kXentBN, 64, 2, EPI_XENT, 2, true>(g, s);
    case EPI_SWIGLU_BACK:
      if (g.y_dt != DT_BF16 || !g.keep_a || !g.keep_c || g.ldy < 2 * (int64_t)g.N ||
          g.N % 4 != 0 || g.ldy % 4 != 0)
        return hipErrorInvalidValue;
      if (g.K % 64 == 0 && g.kparts <= 1)
        return run_bf16<192, 128, 64, 2, EPI_SWIGLU_BACK, 2, false, 2, 2, false, 16, true>(g, s);
      return run_bf16<192, 128, 64, 2, EPI_SWIGLU_BACK, 2, true, 2, 2, false, 16>(g, s);
    case EPI_XENT_GRAD:
      // the padded columns [N, n0) must lie inside the last column tile
      if (g.n0 < g.N || g.n0 > (g.N + 127) / 128 * 128 || g.y_dt != DT_BF16)
        return hipErrorInvalidValue;
      if (g.K % 64 == 0 && g.kparts <= 1)
        return run_bf16<192, 128, 64, 2, EPI_XENT_GRAD, 2, false, 2, 2, false, 16, true>(g, s);
      return run_bf16<192, 128, 64, 2, EPI_XENT_GRAD, 2, true, 2, 2, false, 16>(g, s);
  }
  return hipErrorInvalidValue;
}

hipError_t dispatch_f32(int epi, const GemmArgs &g, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return run_f32<128, 128, EPI_STORE>(g, s);
    case EPI_RESIDUAL: return run_f32<128, 128, EPI_RESIDUAL>(g, s);
    case EPI_QKV_ROPE: return run_f32<128, 128, EPI_QKV_ROPE>(g, s);
    case EPI_SWIGLU: return run_f32<128, 128, EPI_SWIGLU>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int gemm_xent_parts(int N) { return (N + kXentBN - 1) / kXentBN; }

int gemm_residual_col_tiles(int N) { return (N + kResidualBN - 1) / kResidualBN; }
int gemm_norm_max_cols() { return kNormParts * kResidualBN; }

int64_t gemm_store_tiles(int dt, int64_t M, int N) {
  // the plain-store tile shapes of dispatch_bf16 / dispatch_f32
  const int64_t bm = dt == DT_BF16 ? 192 : 128, bn = 128;
  return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

hipError_t launch_gemm(int epi, int dt, const GemmArgs &g, hipStream_t s) {
  if (g.M == 0) return hipSuccess;
  return dt == DT_BF16 ? dispatch_bf16(epi, g, s) : dispatch_f32(epi, g, s);
}

bool gemm_kmajor_ok(const void *a, int64_t lda, const void *w, int64_t ldw, int64_t M, int N,
                    int64_t K) {
  // 16-byte chunks of every row; every offset of a part (k rows x row stride) in 32 bits
  return ((uintptr_t)a & 15) == 0 && ((uintptr_t)w & 15) == 0 && lda % 8 == 0 && ldw % 8 == 0 &&
         lda >= M && ldw >= N && K * std::max(lda, ldw) * 2 < ((int64_t)1 << 31);
}

hipError_t launch_gemm_wgrad_group(const WgradGroup &grp, hipStream_t s) {
  if (grp.njobs < 1 || grp.njobs > kWgradJobs || grp.K < 1) return hipErrorInvalidValue;
  int64_t t = 0;
  WgradGroup q = grp;
  for (int j = 0; j < grp.njobs; ++j) {
    const WgradJob &jb = grp.job[j];
    if (jb.M < 1 || jb.N < 1 || !jb.y ||
        !gemm_kmajor_ok(jb.a, jb.lda, jb.b, jb.ldb, jb.M, jb.N, grp.K))
      return hipErrorInvalidValue;
    q.start[j] = (int)t;
    t += (int64_t)((jb.M + 127) / 128) * ((jb.N + 127) / 128);
    if (t > 0x7fffffff) return hipErrorInvalidValue;
  }
  q.start[grp.njobs] = (int)t;
  hipLaunchKernelGGL(gemm_wgrad_group_kernel, dim3((unsigned)t), dim3(256), 0, s, q);
  return hipGetLastError();
}

hipError_t launch_gemm_kmajor(const GemmArgs &g, hipStream_t s) {

  if (g.M == 0) return hipSuccess;
  if (g.ldw <= 0) return hipErrorInvalidValue;
  return run_bf16<128, 128, 64, 2, EPI_STORE, 2, true, 2, 2, false, 32, false, true>(g, s);
}

}  // namespace tfm

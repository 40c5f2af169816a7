// GEMM family y[m, n] = sum_k a[m, k] w[n, k] on the CDNA4 matrix cores, with fused
// epilogues for the decoder block ("Transformer 篇" (dujian.net) 5.3 Linear: y = x W^T,
// no bias).
//
// Design (gfx950, wave64):
//  * 256 threads = 4 waves in a 2 x 2 grid; each wave owns a (BN/2) x (BM/2) sub-tile
//    made of 32 x 32 MFMA blocks. bf16 uses v_mfma_f32_32x32x16_bf16; f32 uses four
//    v_mfma_f32_32x32x2_f32 per 8-wide k group. Accumulation is fp32 in both cases.
//  * The WEIGHT rows are the MFMA "A" operand and the activation rows the "B" operand, so
//    the 32x32 accumulator puts 4 consecutive output columns n (same row m) in each lane.
//    That makes the RoPE pairs (2i, 2i+1) and the gate/up pairs of SwiGLU lane-local and
//    lets every lane store 4 contiguous outputs.
//  * Each K stage is 128 bytes per tile row (64 bf16 or 32 f32), staged through LDS in
//    16-byte chunks whose position is XOR-swizzled by the row so that the 32 rows read by
//    one MFMA fragment hit distinct banks. Two LDS buffers; the next stage's global loads
//    are in flight in registers while the current stage is multiplied; one barrier per
//    stage.
//  * Epilogues: plain store (LM head; bf16 or f32, any row stride, odd N), residual add
//    into the fp32 stream (out and down projections), RoPE on the q/k columns of the fused
//    QKV projection ("Transformer 篇" 5.5; "LLM 2" RoPE), and SiLU(gate) * up for the
//    SwiGLU up projection ("Transformer 篇" 5.3; "LLM 2" SwiGLU FFN). For SwiGLU the weight
//    tile interleaves 32 rows of W1 and the matching 32 rows of W3, so the two 32-column
//    accumulator blocks of a wave hold gate and up of the same hidden units.
#include "common.h"
#include "internal.h"

namespace tfm {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;  // bytes of one tile row per K stage
constexpr int kChunks = 8;      // 16-byte chunks per tile row and stage

__device__ __forceinline__ int swz(int row) { return row & 7; }

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  __device__ __forceinline__ static void step(const uint4 &a, const uint4 &b, f32x16_t &c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  __device__ __forceinline__ static void step(const uint4 &a, const uint4 &b, f32x16_t &c) {
    f32x4_t av = __builtin_bit_cast(f32x4_t, a), bv = __builtin_bit_cast(f32x4_t, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bv[e], c, 0, 0, 0);
  }
};

// Base pointer of weight row n (virtual row for SwiGLU) and whether it exists.
template <int EPI, typename T>
__device__ __forceinline__ const T *weight_row(const GemmArgs &g, int n, bool &ok) {
  if constexpr (EPI == EPI_SWIGLU) {
    // virtual rows come in 64-row groups: 32 gate rows (W1) then the same 32 up rows (W3)
    const int j = ((n >> 6) << 5) | (n & 31);
    ok = j < g.n0;
    const T *base = (const T *)(((n >> 5) & 1) ? g.w1 : g.w0);
    return base + (int64_t)(ok ? j : 0) * g.K;
  } else if constexpr (EPI == EPI_QKV_ROPE) {
    ok = n < g.N;
    if (!ok) return (const T *)g.w0;
    if (n < g.n0) return (const T *)g.w0 + (int64_t)n * g.K;
    if (n < g.n0 + g.n1) return (const T *)g.w1 + (int64_t)(n - g.n0) * g.K;
    return (const T *)g.w2 + (int64_t)(n - g.n0 - g.n1) * g.K;
  } else {
    ok = n < g.N;
    return (const T *)g.w0 + (int64_t)(ok ? n : 0) * g.K;
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

template <typename T, int BM, int BN, int EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmArgs g, int tiles_m) {
  constexpr int CE = 16 / (int)sizeof(T);            // elements per 16-byte chunk
  constexpr int BKE = kRowBytes / (int)sizeof(T);    // K elements per stage
  constexpr int A_LD = BM * kChunks / kThreads;      // A chunks loaded per thread
  constexpr int W_LD = BN * kChunks / kThreads;      // W chunks loaded per thread
  constexpr int WM = BM / 2, WN = BN / 2;            // wave sub-tile
  constexpr int NBM = WM / 32, NBN = WN / 32;        // 32x32 blocks per wave
  constexpr int STAGE = (BM + BN) * kRowBytes;
  static_assert(A_LD >= 1 && W_LD >= 1 && NBM >= 1 && NBN >= 1, "tile too small");
  static_assert(EPI != EPI_SWIGLU || (NBN % 2) == 0, "SwiGLU needs gate/up block pairs");

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid & 1, wn = wid >> 1;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;

  const T *a_src[A_LD];
  bool a_ok[A_LD];
  int a_lds[A_LD], a_k[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int c = tid + kThreads * i, row = c >> 3, ch = c & 7;
    const int64_t m = m0 + row;
    a_ok[i] = m < g.M;
    a_src[i] = (const T *)g.a + (a_ok[i] ? m : 0) * g.lda + ch * CE;
    a_k[i] = ch * CE;
    a_lds[i] = row * kRowBytes + ((ch ^ swz(row)) << 4);
  }
  const T *w_src[W_LD];
  bool w_ok[W_LD];
  int w_lds[W_LD], w_k[W_LD];
#pragma unroll
  for (int i = 0; i < W_LD; ++i) {
    const int c = tid + kThreads * i, row = c >> 3, ch = c & 7;
    w_src[i] = weight_row<EPI, T>(g, n0 + row, w_ok[i]) + ch * CE;
    w_k[i] = ch * CE;
    w_lds[i] = BM * kRowBytes + row * kRowBytes + ((ch ^ swz(row)) << 4);
  }

  const int nk = (g.K + BKE - 1) / BKE;
  uint4 ra[A_LD], rw[W_LD];
  const uint4 zero = {0u, 0u, 0u, 0u};
  auto gload = [&](int kt) {
    const int kb = kt * BKE;
#pragma unroll
    for (int i = 0; i < A_LD; ++i)
      ra[i] = (a_ok[i] && kb + a_k[i] < g.K) ? *(const uint4 *)(a_src[i] + kb) : zero;
#pragma unroll
    for (int i = 0; i < W_LD; ++i)
      rw[i] = (w_ok[i] && kb + w_k[i] < g.K) ? *(const uint4 *)(w_src[i] + kb) : zero;
  };
  auto sstore = [&](int buf) {
    uint8_t *base = lds + buf * STAGE;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *(uint4 *)(base + a_lds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < W_LD; ++i) *(uint4 *)(base + w_lds[i]) = rw[i];
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
      uint4 fb[NBM], fa[NBN];
#pragma unroll
      for (int bm = 0; bm < NBM; ++bm) {
        const int row = wm * WM + bm * 32 + l32;
        fb[bm] = *(const uint4 *)(As + row * kRowBytes + (((2 * kg + h) ^ swz(row)) << 4));
      }
#pragma unroll
      for (int bn = 0; bn < NBN; ++bn) {
        const int row = wn * WN + bn * 32 + l32;
        fa[bn] = *(const uint4 *)(Ws + row * kRowBytes + (((2 * kg + h) ^ swz(row)) << 4));
      }
#pragma unroll
      for (int bn = 0; bn < NBN; ++bn)
#pragma unroll
        for (int bm = 0; bm < NBM; ++bm) Mfma<T>::step(fa[bn], fb[bm], acc[bn][bm]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds acc[bn][bm][4g + r] for
  //      n = n0 + wn*WN + bn*32 + 8g + 4h + r,  m = m0 + wm*WM + bm*32 + l32
#pragma unroll
  for (int bm = 0; bm < NBM; ++bm) {
    const int64_t m = m0 + wm * WM + bm * 32 + l32;
    if (m >= g.M) continue;
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int t = 0; t < NBN / 2; ++t) {
        const int jbase = (n0 + wn * WN + 64 * t) / 2;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int j = jbase + 8 * gq + 4 * h;
          if (j >= g.n0) continue;
          f32x4_t u;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = acc[2 * t][bm][4 * gq + r], b = acc[2 * t + 1][bm][4 * gq + r];
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
        for (int gq = 0; gq < 4; ++gq) {
          const int n = n0 + wn * WN + bn * 32 + 8 * gq + 4 * h;
          if (n >= g.N) continue;
          f32x4_t v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[bn][bm][4 * gq + r];
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
                v = f32x4_t{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                            __builtin_nanf("")};
              }
            }
          }
          store_out(g, m, n, v, g.N);
        }
      }
    }
  }
}

template <typename T, int BM, int BN, int EPI>
hipError_t run(const GemmArgs &g, hipStream_t s) {
  const int tiles_m = (int)((g.M + BM - 1) / BM);
  const int tiles_n = EPI == EPI_SWIGLU ? (g.n0 + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  if (tiles == 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  gemm_kernel<T, BM, BN, EPI><<<dim3((unsigned)tiles), dim3(kThreads), 0, s>>>(g, tiles_m);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(int epi, const GemmArgs &g, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return run<T, 128, 128, EPI_STORE>(g, s);
    case EPI_RESIDUAL: return run<T, 128, 128, EPI_RESIDUAL>(g, s);
    case EPI_QKV_ROPE: return run<T, 128, 128, EPI_QKV_ROPE>(g, s);
    case EPI_SWIGLU: return run<T, 128, 128, EPI_SWIGLU>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int epi, int dt, const GemmArgs &g, hipStream_t s) {
  if (g.M == 0) return hipSuccess;
  return dt == DT_BF16 ? dispatch<bf16_t>(epi, g, s) : dispatch<float>(epi, g, s);
}

}  // namespace tfm

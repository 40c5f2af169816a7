// Device-side helpers shared by the tfm kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tfm {

typedef uint16_t bf16_t;  // bfloat16 storage word

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA bf16 operand
typedef __attribute__((ext_vector_type(16))) float f32x16_t;   // 32x32 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;   // buffer load/store data
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round-to-nearest-even float -> bfloat16 (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}

// Two floats -> two round-to-nearest-even bfloat16 in one word (lo in bits 0..15); one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) float f2;
  typedef __attribute__((ext_vector_type(2))) __bf16 b2;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, b2));
}

// 16-byte LDS read at addr + IMM, issued as written: the compiler's own wait insertion cannot
// tell which LDS bytes an in-flight buffer->LDS fill writes, so fragment reads are inline and
// waited for explicitly (s_waitcnt lgkmcnt) before first use.
template <int IMM>
__device__ __forceinline__ void ds_read16(u32x4_t &dst, uint32_t addr) {
  static_assert(IMM >= 0 && IMM < 65536, "LDS offset immediate");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(IMM) : "memory");
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  static constexpr int bytes = 4;
  __device__ __forceinline__ static float load(const float *p) { return *p; }
  __device__ __forceinline__ static void store(float *p, float v) { *p = v; }
};
template <> struct Elt<bf16_t> {
  static constexpr int bytes = 2;
  __device__ __forceinline__ static float load(const bf16_t *p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(bf16_t *p, float v) { *p = f32_to_bf16(v); }
};

// Load 4 consecutive elements as floats (16-byte or 8-byte aligned vector load).
__device__ __forceinline__ f32x4_t load4(const float *p) { return *(const f32x4_t *)p; }
__device__ __forceinline__ f32x4_t load4(const bf16_t *p) {
  uint2 u = *(const uint2 *)p;
  f32x4_t r;
  r[0] = __uint_as_float(u.x << 16);
  r[1] = __uint_as_float(u.x & 0xffff0000u);
  r[2] = __uint_as_float(u.y << 16);
  r[3] = __uint_as_float(u.y & 0xffff0000u);
  return r;
}
__device__ __forceinline__ void store4(float *p, f32x4_t v) { *(f32x4_t *)p = v; }
__device__ __forceinline__ void store4(bf16_t *p, f32x4_t v) {
  uint2 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  *(uint2 *)p = u;
}

// Lane exchanges without LDS: DPP moves inside 16-lane rows (quad permutations, the half-row
// mirror, row rotations) and the row / half swaps of v_permlane16/32_swap.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// sum over each group of P consecutive lanes (P = 4, 8 or 16), in every lane of the group
template <int P>
__device__ __forceinline__ float group_sum(float d) {
  d += dpp<0xB1>(d);                              // quad_perm [1,0,3,2]: lane ^ 1
  d += dpp<0x4E>(d);                              // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (P >= 8) d += dpp<0x141>(d);      // half-row mirror: the other quad of 8
  if constexpr (P >= 16) d += dpp<0x128>(d);     // row rotate by 8: the other half row
  return d;
}
// op over the lanes with the same lane % P (P = 4, 8 or 16), in every lane
template <int P, typename Op>
__device__ __forceinline__ float across_groups(float v, Op op) {
  if constexpr (P <= 4) v = op(v, dpp<0x124>(v));   // row rotate by 4
  if constexpr (P <= 8) v = op(v, dpp<0x128>(v));   // row rotate by 8
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// sum over the 64 lanes of the wave, in every lane (DPP and permlane swaps, no LDS)
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  return across_groups<16>(v, [](float a, float b) { return a + b; });
}

}  // namespace tfm

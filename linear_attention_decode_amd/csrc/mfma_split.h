// Split-BF16 matrix-core helpers for fp32 operands on gfx950: an fp32 value x is carried as
// two BF16 terms hi = bf16(x) (round to nearest even) and lo = bf16(x - hi); a product of
// two such operands takes three v_mfma_f32_16x16x32_bf16 (hi*hi + hi*lo + lo*hi, ~16
// significant bits, fp32 range), a product with an exact BF16 operand takes two.
//
// MFMA operand layout (16x16x32): lane l holds row (l % 16) of A and column (l % 16) of B,
// 8 consecutive k from 8 (l / 16); the accumulator of lane l holds rows 4 (l / 16) + r,
// r = 0..3, column l % 16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {
namespace mfma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

struct Frag {
  u32x4_t hi, lo;                      // 8 BF16 each
};

__device__ __forceinline__ unsigned pk_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// x = hi + lo, hi = bf16(x) (round to nearest even), lo = bf16(x - hi)
__device__ __forceinline__ Frag split8(const float (&x)[8]) {
  Frag f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const unsigned h = pk_bf16(x[2 * e], x[2 * e + 1]);
    f.hi[e] = h;
    f.lo[e] = pk_bf16(x[2 * e] - __builtin_bit_cast(float, h << 16),
                      x[2 * e + 1] - __builtin_bit_cast(float, h & 0xffff0000u));
  }
  return f;
}

// acc += a b over 32 k: lo*hi + hi*lo + hi*hi
__device__ __forceinline__ f32x4_t mma3(const Frag& a, const Frag& b, f32x4_t acc) {
  const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, a.hi), al = __builtin_bit_cast(bf16x8_t, a.lo);
  const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, b.hi), bl = __builtin_bit_cast(bf16x8_t, b.lo);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
  return acc;
}

// Fragment f of an operand array: [f][hi, lo][64 lanes] x 16 bytes.
__device__ __forceinline__ void store_frag(u32x4_t* base, int f, int lane, const Frag& v) {
  base[(2 * f) * 64 + lane] = v.hi;
  base[(2 * f + 1) * 64 + lane] = v.lo;
}
__device__ __forceinline__ Frag load_frag(const u32x4_t* base, int f, int lane) {
  return Frag{base[(2 * f) * 64 + lane], base[(2 * f + 1) * 64 + lane]};
}

__device__ __forceinline__ void lds_load8(const float* p, float (&x)[8]) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
}

// acc += a b over 32 k, a split, b exact BF16: lo*b + hi*b
__device__ __forceinline__ f32x4_t mma2(const Frag& a, const u32x4_t& b, f32x4_t acc) {
  const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, a.hi), al = __builtin_bit_cast(bf16x8_t, a.lo);
  const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, b);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bb, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bb, acc, 0, 0, 0);
  return acc;
}


// 4-value operands of v_mfma_f32_16x16x16_bf16 (lane l: row / column l % 16, k = 4 (l / 16)
// .. + 3; the accumulator's rows 4 (l / 16) + r are exactly the k of a B operand).
typedef short s16x4_t __attribute__((ext_vector_type(4)));
struct Frag4 {
  s16x4_t hi, lo;
};
__device__ __forceinline__ Frag4 split4(const f32x4_t x) {
  Frag4 f;
  const unsigned h0 = pk_bf16(x[0], x[1]), h1 = pk_bf16(x[2], x[3]);
  const unsigned l0 = pk_bf16(x[0] - __builtin_bit_cast(float, h0 << 16), x[1] - __builtin_bit_cast(float, h0 & 0xffff0000u));
  const unsigned l1 = pk_bf16(x[2] - __builtin_bit_cast(float, h1 << 16), x[3] - __builtin_bit_cast(float, h1 & 0xffff0000u));
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  f.hi = __builtin_bit_cast(s16x4_t, u32x2_t{h0, h1});
  f.lo = __builtin_bit_cast(s16x4_t, u32x2_t{l0, l1});
  return f;
}
// acc += a b over 16 k: lo*hi + hi*lo + hi*hi
__device__ __forceinline__ f32x4_t mma3_16(const Frag4& a, const Frag4& b, f32x4_t acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b.hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.lo, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.hi, acc, 0, 0, 0);
  return acc;
}

}  // namespace mfma
}  // namespace kda

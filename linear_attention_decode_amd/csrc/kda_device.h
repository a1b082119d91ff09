// Device helpers shared by the gfx950 kernels of the KDA library.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kda {

constexpr int kWave = 64;

// Sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sum over lanes that share (lane % width); every lane receives its group's total.
template <int kWidth>
__device__ __forceinline__ float wave_sum_strided(float v) {
#pragma unroll
  for (int o = 32; o >= kWidth; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Logistic function in the overflow-free form 1/(1+e^|z|), mirrored by sign, with the
// precise (library) exp; the fast-approximate exp differs in the last bit (the
// sigmoid trap of "Thirty tiny kernels per layer", section on bit-exactness).
__device__ __forceinline__ float sigmoid_f(float z) {
  const float y = 1.0f / (1.0f + expf(fabsf(z)));
  return z >= 0.0f ? 1.0f - y : y;
}

__device__ __forceinline__ float silu_f(float y) { return y * sigmoid_f(y); }

__device__ __forceinline__ float softplus_f(float z) {
  return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
}

// 16 bytes with a non-temporal hint: weights are streamed once per token.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

}  // namespace kda

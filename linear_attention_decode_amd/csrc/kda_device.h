// Device helpers shared by the gfx950 kernels of the KDA library.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kda {

constexpr int kWave = 64;

// ---- cross-lane sums with DPP (VALU-rate lane permutes inside 16-lane rows) ----
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xb1;        // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4e;        // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i inside each group of 8
constexpr int kDppRor8 = 0x128;       // lane i <- lane (i+8) mod 16 inside each row of 16

// Sum over aligned groups of n lanes (n in 1, 2, 4, 8, 16); every lane of a group gets it.
__device__ __forceinline__ float group_sum(float v, int n) {
  if (n >= 2) v += dpp_mov<kDppXor1>(v);
  if (n >= 4) v += dpp_mov<kDppXor2>(v);
  if (n >= 8) v += dpp_mov<kDppHalfMirror>(v);
  if (n >= 16) v += dpp_mov<kDppRor8>(v);
  return v;
}
__device__ __forceinline__ float sum8(float v) {
  v += dpp_mov<kDppXor1>(v);
  v += dpp_mov<kDppXor2>(v);
  return v + dpp_mov<kDppHalfMirror>(v);
}
__device__ __forceinline__ float sum16(float v) { v = sum8(v); return v + dpp_mov<kDppRor8>(v); }

// Sum over the 64 lanes of a wave; every lane receives the total (wave-uniform).
__device__ __forceinline__ float wave_sum(float v) {
  const int b = __float_as_int(sum16(v));
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
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

// Weight packing kernels: fp32 -> F32 / BF16 / Q8_0 device layouts, and the canonical
// view of a Q8_0 matrix.  Q8_0 is the block format of the antirez/ds4 PR #964 commit that
// requantises KDA's projections: 32 consecutive values of a row share one fp16 scale.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

__global__ void pack_copy_f32(const float* __restrict__ src, float* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// Round to nearest even; NaN stays a quiet NaN.
__global__ void pack_bf16(const float* __restrict__ src, uint16_t* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t b = __float_as_uint(src[i]);
  uint16_t r;
  if ((b & 0x7fffffffu) > 0x7f800000u) {
    r = (uint16_t)((b >> 16) | 0x40u);
  } else {
    r = (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
  }
  dst[i] = r;
}

// One thread per block of 32: amax, d = amax/127 (fp32, round to nearest), d16 = fp16
// round-to-nearest-even of d, q = clamp(round-half-away(x / d16), -127, 127) with a
// correctly rounded fp32 division; q = 0 everywhere when d16 == 0.  Stored as q + 128.
__global__ void pack_q8_0(const float* __restrict__ src, int64_t rows, int64_t cols,
                          uint8_t* __restrict__ qs, __half* __restrict__ dplane) {
  const int64_t nb_row = cols / 32;
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= rows * nb_row) return;
  const int64_t r = b / nb_row, j = b - r * nb_row;
  const float* x = src + r * cols + j * 32;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = x[i];
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const float d = __fdiv_rn(amax, 127.0f);
  const __half h = __float2half_rn(d);
  const float dq = __half2float(h);
  uint8_t* q = qs + r * cols + j * 32;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float t = 0.0f;
    if (dq != 0.0f) {
      t = roundf(__fdiv_rn(v[i], dq));
      t = fminf(fmaxf(t, -127.0f), 127.0f);
    }
    q[i] = (uint8_t)((int)t + 128);
  }
  dplane[b] = h;
}

// MXFP4 (OCP Microscaling format v1.0), one thread per block of 32: s = floor(log2 amax) - 2
// clamped to [-127, 127], X = 2^s; each element the E2M1 value nearest to x / X (ties to
// the even mantissa bit), clamped to 6: with a = |x / X| the grid index is the count of
// the thresholds 0.25 < a, 0.75 <= a, 1.25 < a, 1.75 <= a, 2.5 < a, 3.5 <= a, 5 < a that
// hold (the midpoints of the grid 0, .5, 1, 1.5, 2, 3, 4, 6; at a midpoint the index with
// mantissa bit 0 wins).  Code = sign << 3 | index (no sign on 0); codes 2 i, 2 i + 1 of a
// block share byte i (low nibble first); the scale byte is s + 127.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t idx = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                       (a >= 3.5f) + (a > 5.0f);
  return ((v < 0.0f && idx > 0) ? 8u : 0u) | idx;
}

__global__ void pack_mxfp4(const float* __restrict__ src, int64_t rows, int64_t cols,
                           uint8_t* __restrict__ codes, uint8_t* __restrict__ eplane) {
  const int64_t nb_row = cols / 32;
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= rows * nb_row) return;
  const int64_t r = b / nb_row, j = b - r * nb_row;
  const float* x = src + r * cols + j * 32;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = x[i];
    amax = fmaxf(amax, fabsf(v[i]));
  }
  int s = -127;
  if (amax > 0.0f) s = min(max(__builtin_amdgcn_frexp_expf(amax) - 1 - 2, -127), 127);
  uint8_t* q = codes + r * (cols / 2) + j * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t lo = e2m1_code(__builtin_amdgcn_ldexpf(v[2 * i], -s));
    const uint32_t hi = e2m1_code(__builtin_amdgcn_ldexpf(v[2 * i + 1], -s));
    q[i] = (uint8_t)(lo | (hi << 4));
  }
  eplane[b] = (uint8_t)(s + 127);
}

__global__ void unpack_q8_0(const uint8_t* __restrict__ qs, const __half* __restrict__ dplane,
                            int64_t rows, int64_t cols, uint16_t* __restrict__ d16,
                            int8_t* __restrict__ qo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = rows * cols;
  if (i < n) qo[i] = (int8_t)((int)qs[i] - 128);
  if (i < n / 32) d16[i] = __half_as_ushort(dplane[i]);
}

// MXFP4 -> Q8_0, exactly: twice an element's E2M1 value is an integer in -12..12 (the
// int8 code) and half the block's E8M0 scale, 2^(e - 128), is an fp16 power of two for
// e - 128 in [-24, 15]; a block whose codes are all +-0 takes scale 0 whatever its e.  A
// nonzero block outside that range sets *bad (the matrix then cannot be held as Q8_0).
// One thread per code byte (two elements), and per scale block.
__global__ void mx4_to_q8(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ eplane,
                          int64_t rows, int64_t cols, uint8_t* __restrict__ qs,
                          __half* __restrict__ dplane, int* __restrict__ bad) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = rows * cols;
  if (i < n / 2) {
    const uint32_t b = codes[i];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t c = (b >> (4 * h)) & 15u, k = c & 7u;
      // doubled magnitudes of grid indices 0..7: 0 1 2 3 4 6 8 12
      const int mag = (int)(((k < 4 ? 0x03020100u : 0x0C080604u) >> (8 * (k & 3))) & 0xffu);
      qs[2 * i + h] = (uint8_t)(128 + ((c & 8u) ? -mag : mag));
    }
  }
  if (i < n / 32) {
    const uint4 blk = *reinterpret_cast<const uint4*>(codes + 16 * i);   // the block's 32 codes
    const bool zero = ((blk.x | blk.y | blk.z | blk.w) & 0x77777777u) == 0u;
    const int e = (int)eplane[i] - 128;
    if (!zero && (e < -24 || e > 15)) atomicOr(bad, 1);
    dplane[i] = __float2half(zero ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, e));
  }
}

static inline int grid_for(int64_t n, int t) { return (int)((n + t - 1) / t); }

// Q8_0 [rows][cols] -> Q8_0 [rows * rep][cols] with every row repeated rep times in place
// (output row r is input row r / rep): bytes and scales copied, one thread per byte.
__global__ void q8_repeat_rows(const uint8_t* __restrict__ qs, const __half* __restrict__ dplane,
                               int64_t rows, int64_t cols, int rep, uint8_t* __restrict__ qo,
                               __half* __restrict__ dout) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = rows * rep * cols;
  if (i < n) {
    const int64_t r = i / cols, c = i - r * cols;
    qo[i] = qs[(r / rep) * cols + c];
  }
  if (i < n / 32) {
    const int64_t r = i / (cols / 32), b = i - r * (cols / 32);
    dout[i] = dplane[(r / rep) * (cols / 32) + b];
  }
}

// out[l][h * rep + i] = in[l][h] for l < layers, h < heads, i < rep
__global__ void f32_repeat(const float* __restrict__ in, int64_t n_in, int rep,
                           float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_in * rep) out[i] = in[i / rep];
}

hipError_t launch_q8_repeat_rows(const void* q8, int64_t rows, int64_t cols, int rep, void* out,
                                 hipStream_t s) {
  const uint8_t* q = static_cast<const uint8_t*>(q8);
  uint8_t* o = static_cast<uint8_t*>(out);
  q8_repeat_rows<<<grid_for(rows * rep * cols, 256), 256, 0, s>>>(
      q, reinterpret_cast<const __half*>(q + q8_scale_offset(rows, cols)), rows, cols, rep, o,
      reinterpret_cast<__half*>(o + q8_scale_offset(rows * rep, cols)));
  return hipGetLastError();
}

hipError_t launch_f32_repeat(const float* in, int64_t n, int rep, float* out, hipStream_t s) {
  f32_repeat<<<grid_for(n * rep, 256), 256, 0, s>>>(in, n, rep, out);
  return hipGetLastError();
}

hipError_t launch_mx4_to_q8(const void* mx4, int64_t rows, int64_t cols, void* q8, int* bad,
                            hipStream_t s) {
  const uint8_t* c = static_cast<const uint8_t*>(mx4);
  uint8_t* q = static_cast<uint8_t*>(q8);
  mx4_to_q8<<<grid_for(rows * cols / 2, 256), 256, 0, s>>>(
      c, c + mx4_scale_offset(rows, cols), rows, cols, q,
      reinterpret_cast<__half*>(q + q8_scale_offset(rows, cols)), bad);
  return hipGetLastError();
}

hipError_t launch_pack(int wt, const float* src, int64_t rows, int64_t cols, void* dst,
                       hipStream_t s) {
  const int64_t n = rows * cols;
  if (wt == kF32) {
    pack_copy_f32<<<grid_for(n, 256), 256, 0, s>>>(src, static_cast<float*>(dst), n);
  } else if (wt == kBF16) {
    pack_bf16<<<grid_for(n, 256), 256, 0, s>>>(src, static_cast<uint16_t*>(dst), n);
  } else if (wt == kMX4) {
    uint8_t* q = static_cast<uint8_t*>(dst);
    pack_mxfp4<<<grid_for(n / 32, 128), 128, 0, s>>>(src, rows, cols, q, q + mx4_scale_offset(rows, cols));
  } else {
    uint8_t* q = static_cast<uint8_t*>(dst);
    __half* d = reinterpret_cast<__half*>(q + q8_scale_offset(rows, cols));
    pack_q8_0<<<grid_for(n / 32, 128), 128, 0, s>>>(src, rows, cols, q, d);
  }
  return hipGetLastError();
}

hipError_t launch_unpack_q8(const void* packed, int64_t rows, int64_t cols, uint16_t* d16,
                            int8_t* qs, hipStream_t s) {
  const uint8_t* q = static_cast<const uint8_t*>(packed);
  const __half* d = reinterpret_cast<const __half*>(q + q8_scale_offset(rows, cols));
  unpack_q8_0<<<grid_for(rows * cols, 256), 256, 0, s>>>(q, d, rows, cols, d16, qs);
  return hipGetLastError();
}

}  // namespace kda

// Dense GEMM on gfx950 matrix cores for the chunked prefill:
//   C[m][coff + n] = sum_k A[m][k] * B[n][k]          (A: [M][lda], B rows: [N][K])
// B is BF16 (the packed projection weights), possibly several matrices stacked along n
// (a segment table, like the decode GEMV).  A is BF16, or FP32 split into two BF16 terms
// a = hi + lo (hi = a with the low 16 bits cleared, lo = bf16(a - hi)) so that products
// keep ~16 significant bits: C = A_hi B + A_lo B, both on MFMA with fp32 accumulation.
//
// Tile 128 x 128 x 64 per block of 4 waves (2 x 2 waves of 64 x 64), v_mfma_f32_16x16x32_bf16
// with the gfx950 operand layout: lane l holds row (l % 16) of A and column (l % 16) of B,
// k = 8 (l / 16) .. 8 (l / 16) + 7; the 4 accumulators of lane l are rows 4 (l / 16) + r,
// column l % 16.  LDS rows are padded by 16 bytes.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsRow = kBK + 8;   // bf16 elements per LDS row (16-byte pad)

__device__ __forceinline__ uint32_t pack_bf16x2(uint16_t lo, uint16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// fp32 -> (hi, lo) bf16 bit patterns with a = hi + lo + O(2^-17 |a|)
__device__ __forceinline__ void split_bf16(float a, uint16_t& hi, uint16_t& lo) {
  const uint32_t b = __float_as_uint(a);
  hi = (uint16_t)(b >> 16);
  const float r = a - __uint_as_float(b & 0xffff0000u);
  const uint32_t rb = __float_as_uint(r);
  lo = (uint16_t)((rb + 0x7fffu + ((rb >> 16) & 1u)) >> 16);
}

template <bool SPLIT>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Al[SPLIT ? kBM * kLdsRow : 8];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLdsRow];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;

  // B row pointers of the rows this thread loads (4 chunks of 8 bf16 per thread per step)
  const uint16_t* brow[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = tid + 256 * u;
    const int r = q >> 3;
    const int n = n0 + r;
    brow[u] = nullptr;
    if (n < P.N) {
      int first = P.seg_first[0];
      const uint16_t* base = P.seg_b[0];
#pragma unroll
      for (int i = 1; i < kMaxSegs; ++i)
        if (i < P.nseg && n >= P.seg_first[i]) { first = P.seg_first[i]; base = P.seg_b[i]; }
      brow[u] = base + (size_t)(n - first) * P.K;
    }
  }

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < P.K; k0 += kBK) {
    // ---- global -> LDS ----
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = tid + 256 * u;
      const int r = q >> 3, c8 = (q & 7) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (brow[u]) v = *reinterpret_cast<const uint4*>(brow[u] + k0 + c8);
      *reinterpret_cast<uint4*>(Bs + r * kLdsRow + c8) = v;
    }
    if constexpr (!SPLIT) {
      const uint16_t* A = static_cast<const uint16_t*>(P.A);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = tid + 256 * u;
        const int r = q >> 3, c8 = (q & 7) * 8;
        const int m = m0 + r;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (m < P.M) v = *reinterpret_cast<const uint4*>(A + (size_t)m * P.lda + k0 + c8);
        *reinterpret_cast<uint4*>(As + r * kLdsRow + c8) = v;
      }
    } else {
      const float* A = static_cast<const float*>(P.A);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = tid + 256 * u;
        const int r = q >> 4, c4 = (q & 15) * 4;
        const int m = m0 + r;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (m < P.M) v = *reinterpret_cast<const float4*>(A + (size_t)m * P.lda + k0 + c4);
        uint16_t h0, h1, h2, h3, l0, l1, l2, l3;
        split_bf16(v.x, h0, l0); split_bf16(v.y, h1, l1);
        split_bf16(v.z, h2, l2); split_bf16(v.w, h3, l3);
        *reinterpret_cast<uint2*>(As + r * kLdsRow + c4) = make_uint2(pack_bf16x2(h0, h1), pack_bf16x2(h2, h3));
        *reinterpret_cast<uint2*>(Al + r * kLdsRow + c4) = make_uint2(pack_bf16x2(l0, l1), pack_bf16x2(l2, l3));
      }
    }
    __syncthreads();
    // ---- MFMA ----
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      const int kc = kk + 8 * (lane >> 4);
      bf16x8_t bfr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = wn * 64 + j * 16 + (lane & 15);
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + n * kLdsRow + kc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wm * 64 + i * 16 + (lane & 15);
        const bf16x8_t afr = *reinterpret_cast<const bf16x8_t*>(As + m * kLdsRow + kc);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[j], acc[i][j], 0, 0, 0);
        if constexpr (SPLIT) {
          const bf16x8_t alr = *reinterpret_cast<const bf16x8_t*>(Al + m * kLdsRow + kc);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alr, bfr[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // ---- store ----
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + j * 16 + (lane & 15);
      if (col >= P.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
        if (row < P.M) P.C[(size_t)row * P.ldc + P.coff + col] = acc[i][j][r];
      }
    }
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  dim3 grid((p.N + kBN - 1) / kBN, (p.M + kBM - 1) / kBM);
  if (p.split_a)
    gemm_kernel<true><<<grid, 256, 0, s>>>(p);
  else
    gemm_kernel<false><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace kda

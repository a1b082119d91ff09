// Fused multi-matrix GEMV for gfx950: several packed weight matrices that read the same
// input are streamed by one launch, the grid split per matrix (each block works on rows
// of one matrix, so the weight format branch is uniform per block).  Used for
// [W_q; W_k; W_v; F_a; G_a; W_beta] on the layer input, and for W_o on the gated norm.
//
// Block = 4 waves of 64 lanes; a wave owns kGemvRowsPerWave rows; lanes split the input
// dimension in 16-byte chunks so every weight load is one 128-bit coalesced read.  The
// input columns (up to NC of them per pass) sit in LDS as fp32; products accumulate in
// fp32 and each row's partial sums are reduced across the wave by butterfly shuffles.
//
// Q8_0 rows hold q + 128 as bytes (one v_cvt_f32_ubyte per weight); the bias is removed
// once per 16-value chunk with a precomputed chunk sum of the input:
//   sum_j (u_j - 128) x_j = sum_j u_j x_j - 128 * sum_j x_j.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int WT>
struct WFmt;
template <>
struct WFmt<kF32> { static constexpr int kElems = 4; static constexpr int kBytes = 4; };
template <>
struct WFmt<kBF16> { static constexpr int kElems = 8; static constexpr int kBytes = 2; };
template <>
struct WFmt<kQ8> { static constexpr int kElems = 16; static constexpr int kBytes = 1; };

// Dot of one 16-byte weight chunk with 16/8/4 LDS inputs (Q8_0: biased, un-scaled).
template <int WT>
__device__ __forceinline__ float chunk_dot(const uint4 w, const float* __restrict__ x) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  float s = 0.0f;
  if constexpr (WT == kF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s += __uint_as_float(wd[i]) * x[i];
  } else if constexpr (WT == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s += bf16_lo(wd[i]) * x[2 * i];
      s += bf16_hi(wd[i]) * x[2 * i + 1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s += (float)(wd[i] & 0xffu) * x[4 * i];
      s += (float)((wd[i] >> 8) & 0xffu) * x[4 * i + 1];
      s += (float)((wd[i] >> 16) & 0xffu) * x[4 * i + 2];
      s += (float)(wd[i] >> 24) * x[4 * i + 3];
    }
  }
  return s;
}

int gemv_cols_per_pass(int N) { return N >= 8 ? 8 : (N >= 4 ? 4 : (N >= 2 ? 2 : 1)); }

size_t gemv_smem_bytes(int wt, int nc, int K, int H) {
  size_t f = (size_t)nc * K;                       // inputs
  if (wt == kQ8) f += (size_t)nc * (K / 16);      // chunk sums
  f += (size_t)nc * (H > 0 ? H : 1) + 64;          // per-column / per-head scales
  return f * sizeof(float);
}

template <int WT, int NC, int PRO>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(const GemvParams P) {
  extern __shared__ float smem[];
  constexpr int EL = WFmt<WT>::kElems;
  constexpr int U = (WT == kQ8) ? 2 : 4;          // chunks per lane per row in flight
  const int K = P.K;
  const int nchunk = K / EL;
  float* xs = smem;                                // [NC][K]
  float* xsum = xs + NC * K;                       // [NC][K/16] (Q8_0)
  float* scal = xsum + (WT == kQ8 ? NC * (K / 16) : 0);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;
  // constant indices only, so the segment table stays in scalar registers
  GemvSeg sg = P.seg[0];
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i)
    if (i < P.nseg && tile >= P.seg[i].first_tile) sg = P.seg[i];
  const int row_base = (tile - sg.first_tile) * kGemvRowsPerBlock + wave * kGemvRowsPerWave;

  for (int c0 = 0; c0 < P.N; c0 += NC) {
    const int nc = min(NC, P.N - c0);
    // ---------------- prologue: the NC input columns into LDS ----------------
    if constexpr (PRO == kProX) {
      if (P.prenorm) {
        for (int n = wave; n < nc; n += 4) {
          const float* xr = P.x + (size_t)(c0 + n) * P.x_stride;
          float a = 0.0f;
          for (int k = lane; k < K; k += 64) a += xr[k] * xr[k];
          a = wave_sum(a);
          if (lane == 0) scal[n] = 1.0f / sqrtf(a / (float)K + P.eps);
        }
        __syncthreads();
      }
      for (int i = tid; i < NC * K; i += kGemvThreads) {
        const int n = i / K, k = i - n * K;
        float v = 0.0f;
        if (n < nc) {
          v = P.x[(size_t)(c0 + n) * P.x_stride + k];
          if (P.prenorm) v *= scal[n];
        }
        xs[i] = v;
      }
    } else {
      // gated RMSNorm per head over dv, from partial sums of squares
      const int H = P.H;
      for (int i = tid; i < nc * H; i += kGemvThreads) {
        const int n = i / H, h = i - n * H;
        const float* sp = P.ss + ((size_t)(c0 + n) * H + h) * P.ncb;
        float a = 0.0f;
        for (int j = 0; j < P.ncb; ++j) a += sp[j];
        scal[i] = 1.0f / sqrtf(a / (float)P.dv + P.eps);
      }
      __syncthreads();
      for (int i = tid; i < NC * K; i += kGemvThreads) {
        const int n = i / K, k = i - n * K;
        float v = 0.0f;
        if (n < nc) {
          const size_t g = (size_t)(c0 + n) * K + k;
          const int h = k / P.dv;
          const float w = P.onw ? P.onw[k - h * P.dv] : 1.0f;
          v = P.o[g] * scal[n * H + h] * w * P.gate[g];
        }
        xs[i] = v;
      }
    }
    __syncthreads();
    if constexpr (WT == kQ8) {
      for (int i = tid; i < NC * (K / 16); i += kGemvThreads) {
        const float* xp = xs + (size_t)i * 16;
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) a += xp[j];
        xsum[i] = a;
      }
      __syncthreads();
    }

    // ---------------- weight stream ----------------
    float acc[kGemvRowsPerWave][NC];
#pragma unroll
    for (int r = 0; r < kGemvRowsPerWave; ++r)
#pragma unroll
      for (int n = 0; n < NC; ++n) acc[r][n] = 0.0f;

    for (int cb = 0; cb < nchunk; cb += 64 * U) {
      uint4 wv[kGemvRowsPerWave][U];
      float dsc[kGemvRowsPerWave][U];
#pragma unroll
      for (int r = 0; r < kGemvRowsPerWave; ++r) {
        const int row = row_base + r;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = cb + u * 64 + lane;
          wv[r][u] = make_uint4(0, 0, 0, 0);
          dsc[r][u] = 0.0f;
          if (row < sg.rows && c < nchunk) {
            const uint8_t* base = sg.m.w + ((size_t)row * K + (size_t)c * EL) * WFmt<WT>::kBytes;
            wv[r][u] = load_stream16(base);
            if constexpr (WT == kQ8) dsc[r][u] = __half2float(sg.m.d[(size_t)row * (K / 32) + (c >> 1)]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < kGemvRowsPerWave; ++r) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = cb + u * 64 + lane;
          if (c < nchunk) {
#pragma unroll
            for (int n = 0; n < NC; ++n) {
              const float d = chunk_dot<WT>(wv[r][u], xs + n * K + c * EL);
              if constexpr (WT == kQ8)
                acc[r][n] += dsc[r][u] * (d - 128.0f * xsum[n * (K / 16) + c]);
              else
                acc[r][n] += d;
            }
          }
        }
      }
    }

    // ---------------- reduce + epilogue ----------------
#pragma unroll
    for (int r = 0; r < kGemvRowsPerWave; ++r) {
#pragma unroll
      for (int n = 0; n < NC; ++n) acc[r][n] = wave_sum(acc[r][n]);
      const int row = row_base + r;
      if (row < sg.rows && lane < nc) {
        float v = acc[r][0];
#pragma unroll
        for (int n = 1; n < NC; ++n)
          if (lane == n) v = acc[r][n];
        const int n = c0 + lane;
        if (sg.conv_chan >= 0) {
          // causal conv over (window, this token), SiLU, window roll (one owner per channel)
          const int c = sg.conv_chan + row;
          const float4 w = *reinterpret_cast<const float4*>(P.conv_w + (size_t)c * 4);
          float* z = P.win + (size_t)n * 3 * P.C + c;
          const float z0 = z[0], z1 = z[P.C], z2 = z[2 * P.C];
          const float y = w.x * z0 + w.y * z1 + w.z * z2 + w.w * v;
          z[0] = z1;
          z[P.C] = z2;
          z[2 * P.C] = v;
          v = silu_f(y);
        }
        const size_t o = (size_t)n * P.out_stride + sg.out_off + row;
        if (P.resid) v += P.resid[o];
        P.out[o] = v;
      }
    }
    __syncthreads();
  }
}

template <int WT, int PRO>
static hipError_t launch_nc(const GemvParams& p, int grid, hipStream_t s) {
  const int nc = gemv_cols_per_pass(p.N);
  const size_t smem = gemv_smem_bytes(WT, nc, p.K, PRO == kProGatedNorm ? p.H : 1);
  switch (nc) {
    case 1: gemv_kernel<WT, 1, PRO><<<grid, kGemvThreads, smem, s>>>(p); break;
    case 2: gemv_kernel<WT, 2, PRO><<<grid, kGemvThreads, smem, s>>>(p); break;
    case 4: gemv_kernel<WT, 4, PRO><<<grid, kGemvThreads, smem, s>>>(p); break;
    default: gemv_kernel<WT, 8, PRO><<<grid, kGemvThreads, smem, s>>>(p); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemv(int wt, int prologue, const GemvParams& p, int grid, hipStream_t s) {
  if (prologue == kProX) {
    if (wt == kF32) return launch_nc<kF32, kProX>(p, grid, s);
    if (wt == kBF16) return launch_nc<kBF16, kProX>(p, grid, s);
    return launch_nc<kQ8, kProX>(p, grid, s);
  }
  if (wt == kF32) return launch_nc<kF32, kProGatedNorm>(p, grid, s);
  if (wt == kBF16) return launch_nc<kBF16, kProGatedNorm>(p, grid, s);
  return launch_nc<kQ8, kProGatedNorm>(p, grid, s);
}

template <int WT, int PRO>
static hipError_t set_attr_all(int big) {
  hipError_t e;
  e = hipFuncSetAttribute((const void*)gemv_kernel<WT, 1, PRO>, hipFuncAttributeMaxDynamicSharedMemorySize, big);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)gemv_kernel<WT, 2, PRO>, hipFuncAttributeMaxDynamicSharedMemorySize, big);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)gemv_kernel<WT, 4, PRO>, hipFuncAttributeMaxDynamicSharedMemorySize, big);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)gemv_kernel<WT, 8, PRO>, hipFuncAttributeMaxDynamicSharedMemorySize, big);
}

// Allow the largest dynamic LDS a block may have on this device (the input columns of a
// pass can exceed the default 64 KB).
hipError_t gemv_prepare_attributes() {
  int dev = 0, big = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&big, hipDeviceAttributeMaxSharedMemoryPerBlock, dev)) != hipSuccess) return e;
  if ((e = set_attr_all<kF32, kProX>(big)) != hipSuccess) return e;
  if ((e = set_attr_all<kBF16, kProX>(big)) != hipSuccess) return e;
  if ((e = set_attr_all<kQ8, kProX>(big)) != hipSuccess) return e;
  if ((e = set_attr_all<kF32, kProGatedNorm>(big)) != hipSuccess) return e;
  if ((e = set_attr_all<kBF16, kProGatedNorm>(big)) != hipSuccess) return e;
  return set_attr_all<kQ8, kProGatedNorm>(big);
}

}  // namespace kda

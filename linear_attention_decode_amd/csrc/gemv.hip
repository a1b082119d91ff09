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
template <>
struct WFmt<kMX4> { static constexpr int kElems = 32; static constexpr int kBytes = 1; };

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

// Input float4s a thread loads per column without a loop (K <= 4096); larger K adds a
// strided tail loop.
constexpr int kXVec = 4;

// LDS is static and sized by the template (a kernel with dynamic LDS measured about twice
// as slow on gfx950 for the same code): KMAX = 2048 takes up to 8 columns a pass, the
// 8192 variant one column a pass.
template <int WT, int NC, int PRO, int KMAX>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(const GemvParams P) {
  __shared__ float xs[NC * KMAX];                              // [NC][K]
  __shared__ float xsum[WT == kQ8 ? NC * (KMAX / 16) : 1];     // [NC][K/16] (Q8_0)
  __shared__ float scal[NC * kGemvMaxHeads];                   // per-column / per-head scales
  __shared__ float red[4 * NC];                                // [4][NC]
  constexpr int EL = WFmt<WT>::kElems;
  // 16-byte chunks per lane per row kept in flight: a 2048-wide row in one pass
  constexpr int U = (WT == kMX4) ? 1 : (WT == kQ8) ? 2 : (WT == kBF16 ? 4 : 8);
  constexpr int RPW = kGemvRowsPerWave;
  const int K = P.K;
  const int K4 = K / 4;
  const int nchunk = K / EL;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;
  // constant indices only, so the segment table stays in scalar registers
  GemvSeg sg = P.seg[0];
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i)
    if (i < P.nseg && tile >= P.seg[i].first_tile) sg = P.seg[i];
  const int row_base = (tile - sg.first_tile) * kGemvRowsPerBlock + wave * RPW;

  uint4 wv[RPW][U];
  float dsc[RPW][U];
  auto load_weights = [&](int cb) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int row = row_base + r;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = cb + u * 64 + lane;
        wv[r][u] = make_uint4(0, 0, 0, 0);
        dsc[r][u] = 0.0f;
        if (row < sg.rows && c < nchunk) {
          wv[r][u] = load_stream16(sg.m.w + ((size_t)row * nchunk + c) * 16);
          if constexpr (WT == kQ8) dsc[r][u] = __half2float(sg.m.d[(size_t)row * (K / 32) + (c >> 1)]);
          // MXFP4: the block scale 2^(e - 127), halved for the doubled element values
          if constexpr (WT == kMX4) dsc[r][u] = __builtin_amdgcn_ldexpf(1.0f, (int)sg.m.e[(size_t)row * (K / 32) + c] - 128);
        }
      }
    }
  };
  // The weight stream does not depend on the input: start it before the prologue.
  load_weights(0);
  // Epilogue operands of the first column pass (conv taps and window, or the residual),
  // also independent of the dot products.
  float4 ep_w[RPW];
  float ep_z[RPW][3], ep_r[RPW];
  auto load_epilogue = [&](int c0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int row = row_base + r, n = c0 + lane;
      ep_w[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      ep_z[r][0] = ep_z[r][1] = ep_z[r][2] = ep_r[r] = 0.0f;
      if (row < sg.rows && lane < NC && n < P.N) {
        if (sg.conv_chan >= 0) {
          const int c = sg.conv_chan + row;
          ep_w[r] = *reinterpret_cast<const float4*>(P.conv_w + (size_t)c * 4);
          const float* z = P.win + (size_t)n * 3 * P.C + c;
          ep_z[r][0] = z[0];
          ep_z[r][1] = z[P.C];
          ep_z[r][2] = z[2 * P.C];
        }
        if (P.resid) ep_r[r] = P.resid[(size_t)n * P.out_stride + sg.out_off + row];
      }
    }
  };
  load_epilogue(0);

  for (int c0 = 0; c0 < P.N; c0 += NC) {
    const int nc = min(NC, P.N - c0);
    // ---------------- prologue: the NC input columns into LDS ----------------
    if constexpr (PRO == kProX) {
      float4 xv[NC][kXVec];
#pragma unroll
      for (int n = 0; n < NC; ++n)
#pragma unroll
        for (int m = 0; m < kXVec; ++m) {
          const int i4 = tid + m * kGemvThreads;
          xv[n][m] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (n < nc && i4 < K4)
            xv[n][m] = *reinterpret_cast<const float4*>(P.x + (size_t)(c0 + n) * P.x_stride + 4 * i4);
        }
      float ssq[NC];
#pragma unroll
      for (int n = 0; n < NC; ++n) {
        ssq[n] = 0.0f;
#pragma unroll
        for (int m = 0; m < kXVec; ++m) {
          const int i4 = tid + m * kGemvThreads;
          if (i4 < K4) {
            const float4 v = xv[n][m];
            ssq[n] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
            *reinterpret_cast<float4*>(xs + n * K + 4 * i4) = v;
          }
        }
        for (int i4 = tid + kXVec * kGemvThreads; i4 < K4; i4 += kGemvThreads) {
          float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
          if (n < nc) v = *reinterpret_cast<const float4*>(P.x + (size_t)(c0 + n) * P.x_stride + 4 * i4);
          ssq[n] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
          *reinterpret_cast<float4*>(xs + n * K + 4 * i4) = v;
        }
      }
      if (P.prenorm) {
#pragma unroll
        for (int n = 0; n < NC; ++n) {
          const float a = wave_sum(ssq[n]);
          if (lane == 0) red[wave * NC + n] = a;
        }
        __syncthreads();
        if (tid < NC) {
          const float a = red[tid] + red[NC + tid] + red[2 * NC + tid] + red[3 * NC + tid];
          scal[tid] = 1.0f / sqrtf(a / (float)K + P.eps);
        }
        __syncthreads();
#pragma unroll
        for (int n = 0; n < NC; ++n) {
          const float sc = scal[n];
          for (int i4 = tid; i4 < K4; i4 += kGemvThreads) {
            float4* p = reinterpret_cast<float4*>(xs + n * K + 4 * i4);
            float4 v = *p;
            v.x *= sc; v.y *= sc; v.z *= sc; v.w *= sc;
            *p = v;
          }
        }
      }
    } else {
      // gated RMSNorm per head over dv, from partial sums of squares
      const int H = P.H;
      float4 ov[NC][kXVec], gv[NC][kXVec];
#pragma unroll
      for (int n = 0; n < NC; ++n)
#pragma unroll
        for (int m = 0; m < kXVec; ++m) {
          const int i4 = tid + m * kGemvThreads;
          ov[n][m] = make_float4(0.f, 0.f, 0.f, 0.f);
          gv[n][m] = ov[n][m];
          if (n < nc && i4 < K4) {
            const size_t g = (size_t)(c0 + n) * K + 4 * i4;
            ov[n][m] = *reinterpret_cast<const float4*>(P.o + g);
            gv[n][m] = *reinterpret_cast<const float4*>(P.gate + g);
          }
        }
      if (tid < nc * H) {
        const int n = tid / H, h = tid - n * H;
        const float* sp = P.ss + ((size_t)(c0 + n) * H + h) * P.ncb;
        scal[tid] = 1.0f / sqrtf(sum_partials(sp, P.ncb) / (float)P.dv + P.eps);
      }
      __syncthreads();
#pragma unroll
      for (int n = 0; n < NC; ++n) {
#pragma unroll
        for (int m = 0; m < kXVec; ++m) {
          const int i4 = tid + m * kGemvThreads;
          if (i4 < K4) {
            const int k = 4 * i4, h = k / P.dv;
            const float sc = n < nc ? scal[n * H + h] : 0.0f;
            float4 w = make_float4(1.f, 1.f, 1.f, 1.f);
            if (P.onw) w = *reinterpret_cast<const float4*>(P.onw + (k - h * P.dv));
            const float4 o = ov[n][m], g = gv[n][m];
            *reinterpret_cast<float4*>(xs + n * K + k) =
                make_float4(o.x * sc * w.x * g.x, o.y * sc * w.y * g.y, o.z * sc * w.z * g.z, o.w * sc * w.w * g.w);
          }
        }
        for (int i4 = tid + kXVec * kGemvThreads; i4 < K4; i4 += kGemvThreads) {
          const int k = 4 * i4, h = k / P.dv;
          float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
          if (n < nc) {
            const size_t g = (size_t)(c0 + n) * K + k;
            const float sc = scal[n * H + h];
            float4 w = make_float4(1.f, 1.f, 1.f, 1.f);
            if (P.onw) w = *reinterpret_cast<const float4*>(P.onw + (k - h * P.dv));
            const float4 o = *reinterpret_cast<const float4*>(P.o + g);
            const float4 gg = *reinterpret_cast<const float4*>(P.gate + g);
            v = make_float4(o.x * sc * w.x * gg.x, o.y * sc * w.y * gg.y, o.z * sc * w.z * gg.z, o.w * sc * w.w * gg.w);
          }
          *reinterpret_cast<float4*>(xs + n * K + k) = v;
        }
      }
    }
    __syncthreads();
    if constexpr (WT == kQ8) {
      for (int i = tid; i < NC * (K / 16); i += kGemvThreads) {
        const float4* xp = reinterpret_cast<const float4*>(xs + (size_t)i * 16);
        const float4 a = xp[0], b = xp[1], c = xp[2], d = xp[3];
        xsum[i] = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w)) +
                  ((c.x + c.y) + (c.z + c.w)) + ((d.x + d.y) + (d.z + d.w));
      }
      __syncthreads();
    }

    // ---------------- weight stream ----------------
    float acc[RPW][NC];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int n = 0; n < NC; ++n) acc[r][n] = 0.0f;

    if (c0 > 0) load_epilogue(c0);
    for (int cb = 0; cb < nchunk; cb += 64 * U) {
      if (c0 > 0 || cb > 0) load_weights(cb);
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = cb + u * 64 + lane;
          if (c < nchunk) {
#pragma unroll
            for (int n = 0; n < NC; ++n) {
              if constexpr (WT == kMX4) {
                acc[r][n] = fmaf(dsc[r][u], mx4_chunk_dot2(wv[r][u], xs + n * K + c * EL), acc[r][n]);
              } else {
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
    }

    // ---------------- reduce + epilogue ----------------
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
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
          const float4 w = ep_w[r];
          float* z = P.win + (size_t)n * 3 * P.C + c;
          const float y = conv4_f(w, ep_z[r][0], ep_z[r][1], ep_z[r][2], v);
          if (!P.active || P.active[n]) {
            z[0] = ep_z[r][1];
            z[P.C] = ep_z[r][2];
            z[2 * P.C] = v;
          }
          v = silu_f(y);
        }
        const size_t o = (size_t)n * P.out_stride + sg.out_off + row;
        if (P.resid) v += ep_r[r];
        P.out[o] = v;
      }
    }
    __syncthreads();
  }
}

template <int WT, int PRO>
static hipError_t launch_nc(const GemvParams& p, int grid, hipStream_t s) {
  if (p.K > kGemvKSmall) {
    gemv_kernel<WT, 1, PRO, kGemvKMax><<<grid, kGemvThreads, 0, s>>>(p);
    return hipGetLastError();
  }
  switch (gemv_cols_per_pass(p.N)) {
    case 1: gemv_kernel<WT, 1, PRO, kGemvKSmall><<<grid, kGemvThreads, 0, s>>>(p); break;
    case 2: gemv_kernel<WT, 2, PRO, kGemvKSmall><<<grid, kGemvThreads, 0, s>>>(p); break;
    case 4: gemv_kernel<WT, 4, PRO, kGemvKSmall><<<grid, kGemvThreads, 0, s>>>(p); break;
    default: gemv_kernel<WT, 8, PRO, kGemvKSmall><<<grid, kGemvThreads, 0, s>>>(p); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemv(int wt, int prologue, const GemvParams& p, int grid, hipStream_t s) {
  if (prologue == kProX) {
    if (wt == kF32) return launch_nc<kF32, kProX>(p, grid, s);
    if (wt == kBF16) return launch_nc<kBF16, kProX>(p, grid, s);
    if (wt == kMX4) return launch_nc<kMX4, kProX>(p, grid, s);
    return launch_nc<kQ8, kProX>(p, grid, s);
  }
  if (wt == kF32) return launch_nc<kF32, kProGatedNorm>(p, grid, s);
  if (wt == kBF16) return launch_nc<kBF16, kProGatedNorm>(p, grid, s);
  if (wt == kMX4) return launch_nc<kMX4, kProGatedNorm>(p, grid, s);
  return launch_nc<kQ8, kProGatedNorm>(p, grid, s);
}

}  // namespace kda

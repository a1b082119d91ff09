// Chunked prefill of one KDA layer on gfx950, the parts around the chunked delta rule
// (chunk.hip): the sequence pass (causal conv + SiLU, L2 norms of q and k, the forget gate
// as a per-channel log2 decay, the output gate and beta), the final conv window, and the
// per-head gated RMSNorm ahead of the output projection.  The projections themselves are
// GEMMs (gemm.hip).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------------------
// Sequence pass: one block per token.
// ---------------------------------------------------------------------------------------
template <int DK>
__global__ __launch_bounds__(256) void prefill_seq_kernel(const PrefillParams P) {
  __shared__ float s_a[kPrefillMaxChannels];     // [C] conv outputs, then [2H] inverse norms
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.y, t = blockIdx.x;
  const int H = P.H, dv = P.dv, C = P.C, K = H * DK, V = H * dv, L = P.L;
  const size_t n = (size_t)b * L + t;
  const float* prow = P.P + n * P.proj_stride;
  float* s_inv = s_a + C;

  // causal depthwise conv over the last three projections (window for t < 3) + SiLU
  for (int c = tid; c < C; c += 256) {
    float pj[4];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int tt = t - 3 + j;
      pj[j] = tt >= 0 ? P.P[((size_t)b * L + tt) * P.proj_stride + c]
                      : P.win[((size_t)b * 3 + (3 + tt)) * C + c];
    }
    pj[3] = prow[c];
    const float4 w = *reinterpret_cast<const float4*>(P.conv_w + (size_t)c * 4);
    s_a[c] = silu_f(w.x * pj[0] + w.y * pj[1] + w.z * pj[2] + w.w * pj[3]);
  }
  __syncthreads();
  for (int vi = wave; vi < 2 * H; vi += 4) {
    const float* src = s_a + vi * DK;
    float a = 0.0f;
    for (int i = lane; i < DK; i += 64) a += src[i] * src[i];
    a = wave_sum(a);
    if (lane == 0) s_inv[vi] = 1.0f / sqrtf(a + P.l2_eps);
  }
  __syncthreads();
  for (int c = tid; c < C; c += 256) {
    if (c < K) {
      const int h = c / DK, i = c - h * DK;
      P.q[(((size_t)b * H + h) * L + t) * DK + i] = s_a[c] * s_inv[h] * P.q_scale;
    } else if (c < 2 * K) {
      const int h = (c - K) / DK, i = c - K - h * DK;
      P.k[(((size_t)b * H + h) * L + t) * DK + i] = s_a[c] * s_inv[H + h];
    } else {
      const int h = (c - 2 * K) / dv, j = c - 2 * K - h * dv;
      P.v[(((size_t)b * H + h) * L + t) * dv + j] = s_a[c];
    }
  }
  // forget gate as a log2 decay; output gate; beta
  const float* fg = P.FG + n * (size_t)(K + V);
  for (int c = tid; c < K; c += 256) {
    const int h = c / DK, i = c - h * DK;
    const float f = fg[c] + P.dt_bias[c];
    const float g = -expf(P.a_log[h]) * softplus_f(f);
    P.g2[(((size_t)b * H + h) * L + t) * DK + i] = g * kLog2e;
  }
  for (int j = tid; j < V; j += 256) P.gate[n * V + j] = sigmoid_f(fg[K + j]);
  if (tid < H) P.beta[((size_t)b * H + tid) * L + t] = sigmoid_f(prow[C + P.rank_f + P.rank_g + tid]);
}

// Final conv window: last three of (window, p_0 .. p_{L-1}).
__global__ void prefill_window_kernel(const PrefillParams P) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int b = blockIdx.y;
  if (c >= P.C) return;
  float z[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int idx = P.L + j;          // position in (w0, w1, w2, p_0, ...)
    z[j] = idx < 3 ? P.win[((size_t)b * 3 + idx) * P.C + c]
                   : P.P[((size_t)b * P.L + (idx - 3)) * P.proj_stride + c];
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) P.win_out[((size_t)b * 3 + j) * P.C + c] = z[j];
}

// ---------------------------------------------------------------------------------------
// Gated RMSNorm per (token, head), in place on o: one wave per (token, head).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gated_norm_kernel(const PrefillParams P, int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (token, head)
  if (r >= rows) return;
  const int dv = P.dv;
  float* o = P.o + r * dv;
  const float* g = P.gate + r * dv;
  float v[4];
  float a = 0.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int j = lane + 64 * m;
    v[m] = j < dv ? o[j] : 0.0f;
    a += v[m] * v[m];
  }
  a = wave_sum(a);
  const float sc = 1.0f / sqrtf(a / (float)dv + P.norm_eps);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int j = lane + 64 * m;
    if (j < dv) o[j] = v[m] * sc * (P.onw ? P.onw[j] : 1.0f) * g[j];
  }
}

// ---------------------------------------------------------------------------------------
hipError_t launch_prefill_seq(const PrefillParams& p, hipStream_t s) {
  dim3 grid(p.L, p.B);
  if (p.dk == 128)
    prefill_seq_kernel<128><<<grid, 256, 0, s>>>(p);
  else
    prefill_seq_kernel<64><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_prefill_window(const PrefillParams& p, hipStream_t s) {
  dim3 grid((p.C + 255) / 256, p.B);
  prefill_window_kernel<<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_gated_norm(const PrefillParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.L * p.H;
  gated_norm_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(p, rows);
  return hipGetLastError();
}

}  // namespace kda

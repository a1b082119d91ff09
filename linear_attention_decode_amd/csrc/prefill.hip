// Chunked prefill of one KDA layer on gfx950: the sequence pass (conv + SiLU + L2 norms +
// gates), the intra-chunk WY/UT kernel and the inter-chunk state carry, and the per-head
// gated RMSNorm ahead of the output projection.  The projections themselves are GEMMs
// (gemm.hip).
//
// The chunked delta rule is the chunk_kda form of torad-labs/llama.cpp PR #84 (the commit
// that moves KDA's prefill onto the chunked pipeline): per chunk of C tokens and per head,
// with G the inclusive sum of each key channel's log-decay along the chunk (so every
// exponent below is <= 0),
//   L[t][s] = beta_t sum_i k_t[i] k_s[i] exp(G_t[i] - G_s[i])   (s < t)
//   A[t][s] = sum_i q_t[i] k_s[i] exp(G_t[i] - G_s[i])           (s <= t)
//   (I + L) W = beta exp(G) k,   (I + L) U = beta v              (forward substitution)
// and across chunks, with S the fp32 state at the chunk start ([dk][dv], row = key
// channel):
//   D = U - W S
//   O_t = (q_t exp(G_t)) S + sum_{s<=t} A[t][s] D_s
//   S <- diag(exp(G_last)) S + (k exp(G_last - G))^T D
// Exponents are kept in log2 units and evaluated pairwise (exp2 of G_t - G_s <= 0), so no
// factor can overflow whatever the decay.
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
// Intra-chunk: one block per (chunk, head, sequence).
// ---------------------------------------------------------------------------------------
template <int DK>
__global__ __launch_bounds__(256) void chunk_intra_kernel(const PrefillParams P) {
  constexpr int CS = kChunk;
  constexpr int TP = CS + 1;                     // padded row of the channel-major tiles
  __shared__ float kT[DK * TP], qT[DK * TP], gT[DK * TP];
  __shared__ float s_beta[CS];
  __shared__ float Lm[CS * TP];
  __shared__ float Xu[CS * DK];

  const int tid = threadIdx.x;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int H = P.H, L = P.L, dv = P.dv;
  const int t0 = c * CS;
  const int nt = min(CS, L - t0);
  const size_t bh = (size_t)b * H + h;
  const size_t chunk = bh * P.nch + c;

  for (int e = tid; e < CS * DK; e += 256) {
    const int t = e / DK, i = e - t * DK;
    float kv = 0.f, qv = 0.f, gv = 0.f;
    if (t < nt) {
      const size_t g = (bh * L + t0 + t) * DK + i;
      kv = P.k[g]; qv = P.q[g]; gv = P.g2[g];
    }
    kT[i * TP + t] = kv; qT[i * TP + t] = qv; gT[i * TP + t] = gv;
  }
  if (tid < CS) s_beta[tid] = tid < nt ? P.beta[bh * L + t0 + tid] : 0.0f;
  __syncthreads();
  // inclusive cumulative log2-decay per key channel
  if (tid < DK) {
    float a = 0.0f;
    for (int t = 0; t < CS; ++t) {
      a += gT[tid * TP + t];
      gT[tid * TP + t] = a;
    }
  }
  __syncthreads();

  // L and A (causal: s <= t only): thread (t = tid % 64, s in a group of 16); a group
  // entirely above the diagonal skips its channel loop
  {
    const int t = tid & (CS - 1), sg = tid / CS;
    float accL[16], accA[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) { accL[j] = 0.f; accA[j] = 0.f; }
    if (sg * 16 <= t) {
      for (int i = 0; i < DK; ++i) {
        const float kt = kT[i * TP + t], qt = qT[i * TP + t], gt = gT[i * TP + t];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int s = sg * 16 + j;
          const float e = exp2f(fminf(gt - gT[i * TP + s], 0.0f));
          const float ks = kT[i * TP + s] * e;
          accL[j] += kt * ks;
          accA[j] += qt * ks;
        }
      }
    }
    float* Ag = P.A + chunk * CS * CS;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int s = sg * 16 + j;
      Lm[t * TP + s] = s < t ? s_beta[t] * accL[j] : 0.0f;
      Ag[t * CS + s] = s <= t ? accA[j] : 0.0f;
    }
  }
  __syncthreads();

  // decay-scaled q and k, and the per-channel decay over the whole chunk
  for (int e = tid; e < CS * DK; e += 256) {
    const int t = e / DK, i = e - t * DK;
    const float gl = gT[i * TP + nt - 1], gt = gT[i * TP + t];
    float qv = 0.f, kv = 0.f;
    if (t < nt) {
      qv = qT[i * TP + t] * exp2f(gt);
      kv = kT[i * TP + t] * exp2f(fminf(gl - gt, 0.0f));
    }
    P.Qt[chunk * CS * DK + e] = qv;
    P.Kt[chunk * CS * DK + e] = kv;
  }
  if (tid < DK) P.dec[chunk * DK + tid] = exp2f(gT[tid * TP + nt - 1]);
  __syncthreads();

  // forward substitution (I + L) X = R, row by row, one right-hand-side column per thread,
  // both right-hand sides at once: threads [0, DK) solve R = beta exp(G) k -> W with X in the
  // (no longer needed) q tile, threads [DK, 2 DK) solve R = beta v -> U with X in Xu.
  {
    const int pass = tid / DK, col = tid - pass * DK;
    if (pass < 2) {
      float* X = pass == 0 ? qT : Xu;                // [CS][DK]
      const float* vsrc = P.v + (bh * L + t0) * dv + col;
      for (int t = 0; t < CS; ++t) {
        float acc = 0.0f;
        if (t < nt) acc = pass == 0 ? s_beta[t] * exp2f(gT[col * TP + t]) * kT[col * TP + t]
                                    : s_beta[t] * vsrc[(size_t)t * dv];
        for (int s = 0; s < t; ++s) acc -= Lm[t * TP + s] * X[s * DK + col];
        X[t * DK + col] = acc;
      }
      float* dst = (pass == 0 ? P.W : P.U) + chunk * CS * DK + col;
      for (int t = 0; t < CS; ++t) dst[(size_t)t * DK] = X[t * DK + col];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Inter-chunk state carry: one block per (32 value columns, head, sequence), sequential
// over the chunks of the sequence; the fp32 state tile stays in LDS.
// ---------------------------------------------------------------------------------------
template <int DK>
__global__ __launch_bounds__(256) void chunk_inter_kernel(const PrefillParams P) {
  constexpr int CS = kChunk, NJ = kInterCols;
  constexpr int RP = DK + 1;                    // padded row of W / Qt tiles
  __shared__ float sS[DK * NJ];
  __shared__ float sW[CS * RP];
  __shared__ float sQ[CS * RP];
  __shared__ float sK[CS * DK];
  __shared__ float sA[CS * CS];
  __shared__ float sD[CS * NJ];
  __shared__ float sDec[DK];

  const int tid = threadIdx.x;
  const int cb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int H = P.H, L = P.L, dv = P.dv;
  const int j0 = cb * NJ;
  const size_t bh = (size_t)b * H + h;
  float* Sg = P.S + bh * DK * dv;

  for (int e = tid; e < DK * NJ; e += 256) {
    const int i = e / NJ, j = e - i * NJ;
    sS[e] = Sg[(size_t)i * dv + j0 + j];
  }
  // output / D mapping: row t = tid / 4, columns 8 (tid % 4) .. +7
  const int tr = tid >> 2, jc = (tid & 3) * 8;
  // state-update mapping: row i, SPT consecutive columns per thread
  constexpr int SPT = DK * NJ / 256;
  const int ir = tid / (NJ / SPT), js = (tid % (NJ / SPT)) * SPT;

  for (int c = 0; c < P.nch; ++c) {
    const size_t chunk = bh * P.nch + c;
    const int t0 = c * CS;
    const int nt = min(CS, L - t0);
    __syncthreads();
    for (int e = tid; e < CS * DK; e += 256) {
      const int t = e / DK, i = e - t * DK;
      sW[t * RP + i] = P.W[chunk * CS * DK + e];
      sQ[t * RP + i] = P.Qt[chunk * CS * DK + e];
      sK[e] = P.Kt[chunk * CS * DK + e];
    }
    for (int e = tid; e < CS * CS; e += 256) sA[e] = P.A[chunk * CS * CS + e];
    if (tid < DK) sDec[tid] = P.dec[chunk * DK + tid];
    float u[8];
    const float* Ug = P.U + chunk * CS * dv + (size_t)tr * dv + j0 + jc;
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = Ug[j];
    __syncthreads();
    // D = U - W S
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = u[j];
    for (int i = 0; i < DK; ++i) {
      const float w = sW[tr * RP + i];
      const float4 s0 = *reinterpret_cast<const float4*>(sS + i * NJ + jc);
      const float4 s1 = *reinterpret_cast<const float4*>(sS + i * NJ + jc + 4);
      acc[0] -= w * s0.x; acc[1] -= w * s0.y; acc[2] -= w * s0.z; acc[3] -= w * s0.w;
      acc[4] -= w * s1.x; acc[5] -= w * s1.y; acc[6] -= w * s1.z; acc[7] -= w * s1.w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) sD[tr * NJ + jc + j] = acc[j];
    __syncthreads();
    // O = (q exp(G)) S + A D
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    for (int i = 0; i < DK; ++i) {
      const float q = sQ[tr * RP + i];
      const float4 s0 = *reinterpret_cast<const float4*>(sS + i * NJ + jc);
      const float4 s1 = *reinterpret_cast<const float4*>(sS + i * NJ + jc + 4);
      acc[0] += q * s0.x; acc[1] += q * s0.y; acc[2] += q * s0.z; acc[3] += q * s0.w;
      acc[4] += q * s1.x; acc[5] += q * s1.y; acc[6] += q * s1.z; acc[7] += q * s1.w;
    }
    for (int s = 0; s <= tr; ++s) {
      const float a = sA[tr * CS + s];
      const float4 d0 = *reinterpret_cast<const float4*>(sD + s * NJ + jc);
      const float4 d1 = *reinterpret_cast<const float4*>(sD + s * NJ + jc + 4);
      acc[0] += a * d0.x; acc[1] += a * d0.y; acc[2] += a * d0.z; acc[3] += a * d0.w;
      acc[4] += a * d1.x; acc[5] += a * d1.y; acc[6] += a * d1.z; acc[7] += a * d1.w;
    }
    if (tr < nt) {
      float* og = P.o + ((size_t)b * L + t0 + tr) * (size_t)(H * dv) + h * dv + j0 + jc;
#pragma unroll
      for (int j = 0; j < 8; ++j) og[j] = acc[j];
    }
    __syncthreads();
    // S <- diag(dec) S + Kt^T D
    float sacc[SPT];
    const float dk_ = sDec[ir];
#pragma unroll
    for (int j = 0; j < SPT; ++j) sacc[j] = dk_ * sS[ir * NJ + js + j];
    for (int t = 0; t < CS; ++t) {
      const float kv = sK[t * DK + ir];
#pragma unroll
      for (int j4 = 0; j4 < SPT / 4; ++j4) {
        const float4 d = *reinterpret_cast<const float4*>(sD + t * NJ + js + 4 * j4);
        sacc[4 * j4 + 0] += kv * d.x; sacc[4 * j4 + 1] += kv * d.y;
        sacc[4 * j4 + 2] += kv * d.z; sacc[4 * j4 + 3] += kv * d.w;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SPT; ++j) sS[ir * NJ + js + j] = sacc[j];
  }
  __syncthreads();
  for (int e = tid; e < DK * NJ; e += 256) {
    const int i = e / NJ, j = e - i * NJ;
    Sg[(size_t)i * dv + j0 + j] = sS[e];
  }
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

hipError_t launch_chunk_intra(const PrefillParams& p, hipStream_t s) {
  dim3 grid(p.nch, p.H, p.B);
  if (p.dk == 128)
    chunk_intra_kernel<128><<<grid, 256, 0, s>>>(p);
  else
    chunk_intra_kernel<64><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_chunk_inter(const PrefillParams& p, hipStream_t s) {
  dim3 grid(p.dv / kInterCols, p.H, p.B);
  if (p.dk == 128)
    chunk_inter_kernel<128><<<grid, 256, 0, s>>>(p);
  else
    chunk_inter_kernel<64><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_gated_norm(const PrefillParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.L * p.H;
  gated_norm_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(p, rows);
  return hipGetLastError();
}

}  // namespace kda

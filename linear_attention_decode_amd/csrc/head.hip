// Per-head kernel of the KDA step for gfx950: conv (verify / commit), L2-normalised q and
// k, the softplus forget gate and sigmoid beta, the low-rank up-projections F_b and G_b,
// the gated delta rule and the read-out o = S^T q.
//
// Steps as listed under "Where the time goes" in "Thirty tiny kernels per layer"
// (frederic.ai) and written as its pure decode step; the forget gate is the workload's
// alpha = exp(-exp(A_log[h]) softplus(F_b F_a u + dt_bias)), one A_log per head as in the
// KDA recurrence-kernel commit of antirez/ds4 PR #964.
//
// Layout.  A block owns one (sequence b, head h, 32 value columns).  Its 256 threads hold
// the state tile S[0:dk][j0:j0+32] in registers: thread (row group rg, column quad cq)
// keeps rows rg*RPT .. rg*RPT+RPT-1 of columns j0+4cq .. j0+4cq+3 as float4s, so every
// state load and store is a 128-bit access and a wave touches 8 full 128-byte row
// segments.  Value columns are independent in the delta rule, so blocks never talk to
// each other; every block recomputes the head's q, k and alpha (dk values each).
// The state is read once and written once per call; in verify mode (several tokens,
// state read-only) it stays in registers across the tokens.
//
// Per token (column j, rows i of the tile):
//   S'_ij = alpha_i S_ij ;  e_j = sum_i S'_ij k_i ;  delta_j = beta (v_j - e_j)
//   S_ij = S'_ij + k_i delta_j ;  o_j = sum_i S_ij q_i
// The two column sums reduce over lanes of a wave (butterfly over the row-group bits)
// and then over the 4 waves through LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// One row of a packed matrix dotted with an LDS vector, by a single thread.
__device__ __forceinline__ float row_dot(const PackedMat m, int wt, int row, int K,
                                         const float* __restrict__ x) {
  float acc = 0.0f;
  if (wt == kF32) {
    const float4* w = reinterpret_cast<const float4*>(m.w) + (size_t)row * (K / 4);
    for (int i = 0; i < K / 4; ++i) {
      const float4 v = w[i];
      acc += v.x * x[4 * i] + v.y * x[4 * i + 1] + v.z * x[4 * i + 2] + v.w * x[4 * i + 3];
    }
  } else if (wt == kBF16) {
    const uint4* w = reinterpret_cast<const uint4*>(m.w + (size_t)row * K * 2);
    for (int i = 0; i < K / 8; ++i) {
      const uint4 v = w[i];
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc += bf16_lo(d[j]) * x[8 * i + 2 * j] + bf16_hi(d[j]) * x[8 * i + 2 * j + 1];
    }
  } else {
    const uint4* w = reinterpret_cast<const uint4*>(m.w + (size_t)row * K);
    const __half* ds = m.d + (size_t)row * (K / 32);
    for (int blk = 0; blk < K / 32; ++blk) {
      float s = 0.0f;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint4 v = w[2 * blk + hh];
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
        const float* xp = x + blk * 32 + hh * 16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s += ((float)(d[j] & 0xffu) - 128.0f) * xp[4 * j];
          s += ((float)((d[j] >> 8) & 0xffu) - 128.0f) * xp[4 * j + 1];
          s += ((float)((d[j] >> 16) & 0xffu) - 128.0f) * xp[4 * j + 2];
          s += ((float)(d[j] >> 24) - 128.0f) * xp[4 * j + 3];
        }
      }
      acc += __half2float(ds[blk]) * s;
    }
  }
  return acc;
}

constexpr int kMaxRank = 256;

template <int DK>
__global__ __launch_bounds__(kHeadThreads) void head_kernel(const HeadParams P) {
  constexpr int CB = kHeadCols;
  constexpr int QPR = CB / 4;                 // column quads per row
  constexpr int RG = kHeadThreads / QPR;      // row groups
  constexpr int RPT = DK / RG;                // rows per thread
  static_assert(RPT >= 1 && RPT * RG == DK, "tile shape");
  constexpr int NCH = 2 * DK + CB;            // conv channels a block needs

  __shared__ float s_qk[2 * DK];
  __shared__ float s_v[CB];
  __shared__ float s_alpha[DK];
  __shared__ float s_gate[CB];
  __shared__ float s_lr[2 * kMaxRank];
  __shared__ float s_red[2][4][CB];
  __shared__ float s_misc[4];

  const int cb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cq = tid % QPR, rg = tid / QPR;
  const int H = P.H, dv = P.dv, C = P.C, K = H * DK;
  const int j0 = cb * CB;
  const int ncb = dv / CB;

  int ntok = P.T;
  if (P.ntok) ntok = min(max(P.ntok[b], 1), P.T);

  float* Sb = P.S + ((size_t)b * H + h) * DK * dv;
  float4 st[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    st[i] = *reinterpret_cast<const float4*>(Sb + (size_t)(rg * RPT + i) * dv + j0 + 4 * cq);

  // conv channels of this thread: q (h*DK + i), k (K + h*DK + i), v (2K + h*dv + j0 + j)
  int chan[2];
  float z[2][3], cw[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int ci = tid + m * kHeadThreads;
    chan[m] = -1;
    if (ci < NCH) {
      chan[m] = ci < DK ? h * DK + ci : (ci < 2 * DK ? K + h * DK + (ci - DK) : 2 * K + h * dv + j0 + (ci - 2 * DK));
      if (P.conv_in_head) {
        const float* zw = P.win + (size_t)b * 3 * C + chan[m];
        z[m][0] = zw[0];
        z[m][1] = zw[C];
        z[m][2] = zw[2 * C];
        const float4 w = *reinterpret_cast<const float4*>(P.conv_w + (size_t)chan[m] * 4);
        cw[m][0] = w.x; cw[m][1] = w.y; cw[m][2] = w.z; cw[m][3] = w.w;
      }
    }
  }

  const float a_h = expf(P.a_log[h]);
  const int rl = P.rank_f + P.rank_g;

  for (int t = 0; t < ntok; ++t) {
    const int n = b * P.T + t;
    const float* prow = P.proj + (size_t)n * P.proj_stride;
    // ---- q, k, v channel values (post conv + SiLU) ----
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int ci = tid + m * kHeadThreads;
      if (ci < NCH) {
        float a = prow[chan[m]];
        if (P.conv_in_head) {
          const float y = cw[m][0] * z[m][0] + cw[m][1] * z[m][1] + cw[m][2] * z[m][2] + cw[m][3] * a;
          z[m][0] = z[m][1];
          z[m][1] = z[m][2];
          z[m][2] = a;
          a = silu_f(y);
        }
        if (ci < 2 * DK) s_qk[ci] = a; else s_v[ci - 2 * DK] = a;
      }
    }
    for (int i = tid; i < rl; i += kHeadThreads) s_lr[i] = prow[C + i];
    if (tid == 0) s_misc[2] = sigmoid_f(prow[C + rl + h]);
    __syncthreads();
    // ---- L2 norms of q (wave 0) and k (wave 1) ----
    if (wave < 2) {
      const float* src = s_qk + wave * DK;
      float a = 0.0f;
      for (int i = lane; i < DK; i += 64) a += src[i] * src[i];
      a = wave_sum(a);
      if (lane == 0) s_misc[wave] = 1.0f / sqrtf(a + P.l2_eps);
    }
    // ---- forget gate (alpha, one per key channel) and output gate (this block's columns)
    if (tid < DK) {
      const float f = row_dot(P.fb, P.wt, h * DK + tid, P.rank_f, s_lr) + P.dt_bias[h * DK + tid];
      s_alpha[tid] = expf(-a_h * softplus_f(f));
    } else if (tid < DK + CB) {
      const int j = tid - DK;
      const float g = row_dot(P.gb, P.wt, h * dv + j0 + j, P.rank_g, s_lr + P.rank_f);
      s_gate[j] = sigmoid_f(g);
    }
    __syncthreads();
    const float inv_q = s_misc[0] * P.q_scale, inv_k = s_misc[1], beta = s_misc[2];

    // ---- delta rule on the register tile ----
    float e0 = 0.f, e1 = 0.f, e2 = 0.f, e3 = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg * RPT + i;
      const float al = s_alpha[r], kk = s_qk[DK + r] * inv_k;
      st[i].x *= al; st[i].y *= al; st[i].z *= al; st[i].w *= al;
      e0 += st[i].x * kk; e1 += st[i].y * kk; e2 += st[i].z * kk; e3 += st[i].w * kk;
    }
    e0 = wave_sum_strided<QPR>(e0); e1 = wave_sum_strided<QPR>(e1);
    e2 = wave_sum_strided<QPR>(e2); e3 = wave_sum_strided<QPR>(e3);
    if (lane < QPR) {
      s_red[0][wave][4 * cq + 0] = e0; s_red[0][wave][4 * cq + 1] = e1;
      s_red[0][wave][4 * cq + 2] = e2; s_red[0][wave][4 * cq + 3] = e3;
    }
    __syncthreads();
    float dl[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = 4 * cq + c;
      const float e = s_red[0][0][j] + s_red[0][1][j] + s_red[0][2][j] + s_red[0][3][j];
      dl[c] = beta * (s_v[j] - e);
    }
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg * RPT + i;
      const float kk = s_qk[DK + r] * inv_k, qq = s_qk[r] * inv_q;
      st[i].x += kk * dl[0]; st[i].y += kk * dl[1]; st[i].z += kk * dl[2]; st[i].w += kk * dl[3];
      o0 += st[i].x * qq; o1 += st[i].y * qq; o2 += st[i].z * qq; o3 += st[i].w * qq;
    }
    o0 = wave_sum_strided<QPR>(o0); o1 = wave_sum_strided<QPR>(o1);
    o2 = wave_sum_strided<QPR>(o2); o3 = wave_sum_strided<QPR>(o3);
    if (lane < QPR) {
      s_red[1][wave][4 * cq + 0] = o0; s_red[1][wave][4 * cq + 1] = o1;
      s_red[1][wave][4 * cq + 2] = o2; s_red[1][wave][4 * cq + 3] = o3;
    }
    __syncthreads();
    if (P.write_out && wave == 0) {
      float oj = 0.0f;
      if (lane < CB) {
        oj = s_red[1][0][lane] + s_red[1][1][lane] + s_red[1][2][lane] + s_red[1][3][lane];
        const size_t g = (size_t)n * H * dv + h * dv + j0 + lane;
        P.o[g] = oj;
        P.gate[g] = s_gate[lane];
      }
      const float sq = wave_sum(oj * oj);
      if (lane == 0) P.ss[((size_t)n * H + h) * ncb + cb] = sq;
    }
    __syncthreads();
  }

  if (P.write_state) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *reinterpret_cast<float4*>(Sb + (size_t)(rg * RPT + i) * dv + j0 + 4 * cq) = st[i];
  }
}

hipError_t launch_head(const HeadParams& p, hipStream_t s) {
  dim3 grid(p.dv / kHeadCols, p.H, p.B);
  if (p.dk == 128)
    head_kernel<128><<<grid, kHeadThreads, 0, s>>>(p);
  else
    head_kernel<64><<<grid, kHeadThreads, 0, s>>>(p);
  return hipGetLastError();
}

__global__ void window_commit_kernel(const float* __restrict__ plog, int stride,
                                     float* __restrict__ win, int T, int C,
                                     const int* __restrict__ ntok) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int b = blockIdx.y;
  if (c >= C) return;
  const int a = min(max(ntok[b], 1), T);
  float* z = win + (size_t)b * 3 * C + c;
  float seq[3 + 8];
  seq[0] = z[0];
  seq[1] = z[C];
  seq[2] = z[2 * C];
  for (int t = 0; t < a; ++t) seq[3 + t] = plog[(size_t)(b * T + t) * stride + c];
  z[0] = seq[a];
  z[C] = seq[a + 1];
  z[2 * C] = seq[a + 2];
}

hipError_t launch_window_commit(const float* plog, int proj_stride, float* win, int B, int T,
                                int C, const int* ntok, hipStream_t s) {
  dim3 grid((C + 255) / 256, B);
  window_commit_kernel<<<grid, 256, 0, s>>>(plog, proj_stride, win, T, C, ntok);
  return hipGetLastError();
}

}  // namespace kda

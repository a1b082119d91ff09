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

template <int WT>
struct HFmt;
template <>
struct HFmt<kF32> { static constexpr int kElems = 4; static constexpr int kBytes = 4; };
template <>
struct HFmt<kBF16> { static constexpr int kElems = 8; static constexpr int kBytes = 2; };
template <>
struct HFmt<kQ8> { static constexpr int kElems = 16; static constexpr int kBytes = 1; };

// Dot of one 16-byte chunk of a packed row with LDS inputs (Q8_0: q = byte - 128, unscaled).
template <int WT>
__device__ __forceinline__ float hchunk_dot(const uint4 w, const float* __restrict__ x) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
  float s = 0.0f;
  if constexpr (WT == kF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s += __uint_as_float(d[i]) * x[i];
  } else if constexpr (WT == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s += bf16_lo(d[i]) * x[2 * i] + bf16_hi(d[i]) * x[2 * i + 1];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s += ((float)(d[i] & 0xffu) - 128.0f) * x[4 * i];
      s += ((float)((d[i] >> 8) & 0xffu) - 128.0f) * x[4 * i + 1];
      s += ((float)((d[i] >> 16) & 0xffu) - 128.0f) * x[4 * i + 2];
      s += ((float)(d[i] >> 24) - 128.0f) * x[4 * i + 3];
    }
  }
  return s;
}

constexpr int kMaxRank = 256;
constexpr int kMaxLrLoads = 10;   // 16-byte chunks of F_b / G_b rows per thread

template <int DK, int WT>
__global__ __launch_bounds__(kHeadThreads) void head_kernel(const HeadParams P) {
  constexpr int CB = kHeadCols;
  constexpr int QPR = CB / 4;                 // column quads per row
  constexpr int RG = kHeadThreads / QPR;      // row groups
  constexpr int RPT = DK / RG;                // rows per thread
  static_assert(RPT >= 1 && RPT * RG == DK, "tile shape");
  constexpr int NCH = 2 * DK + CB;            // conv channels a block needs
  constexpr int EL = HFmt<WT>::kElems;
  constexpr int BY = HFmt<WT>::kBytes;

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
  const int rl = P.rank_f + P.rank_g;

  int ntok = P.T;
  if (P.ntok) ntok = min(max(P.ntok[b], 1), P.T);

  // ---- everything that does not depend on the token is requested first ----
  float* Sb = P.S + ((size_t)b * H + h) * DK * dv;
  float4 st[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    st[i] = *reinterpret_cast<const float4*>(Sb + (size_t)(rg * RPT + i) * dv + j0 + 4 * cq);

  // F_b rows h*DK .. h*DK+DK-1 (forget gate) then G_b rows of this block's columns, as
  // (row, 16-byte chunk) items spread over the block; a row's chunks sit in adjacent lanes.
  const int cpr = P.rank_f * BY / 16;         // chunks per row (rank_f == rank_g checked)
  const int items = (DK + CB) * cpr;
  const int nld = (items + kHeadThreads - 1) / kHeadThreads;
  uint4 lw[kMaxLrLoads];
  float lsc[kMaxLrLoads], lbias[kMaxLrLoads];
#pragma unroll
  for (int m = 0; m < kMaxLrLoads; ++m) {
    lw[m] = make_uint4(0, 0, 0, 0);
    lsc[m] = 0.0f;
    lbias[m] = 0.0f;
    const int it = tid + m * kHeadThreads;
    if (m < nld && it < items) {
      const int rloc = it / cpr, c = it - rloc * cpr;
      const PackedMat& M = rloc < DK ? P.fb : P.gb;
      const int rank = rloc < DK ? P.rank_f : P.rank_g;
      const int row = rloc < DK ? h * DK + rloc : h * dv + j0 + (rloc - DK);
      lw[m] = *reinterpret_cast<const uint4*>(M.w + ((size_t)row * rank + (size_t)c * EL) * BY);
      if constexpr (WT == kQ8) lsc[m] = __half2float(M.d[(size_t)row * (rank / 32) + (c >> 1)]);
      if (rloc < DK && c == 0) lbias[m] = P.dt_bias[h * DK + rloc];
    }
  }

  // conv channels of this thread: q (h*DK + i), k (K + h*DK + i), v (2K + h*dv + j0 + j)
  int chan[2];
  float z[2][3], cw[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int ci = tid + m * kHeadThreads;
    chan[m] = -1;
    z[m][0] = z[m][1] = z[m][2] = 0.0f;
    cw[m][0] = cw[m][1] = cw[m][2] = cw[m][3] = 0.0f;
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
  const float a_log_h = P.a_log[h];

  // token inputs (q, k, v channel values, low-rank activations, beta logit), loaded one
  // token ahead so the first token's loads travel with the state and weight loads
  float av[2], lrv[2], blog = 0.0f;
  auto load_token = [&](int t) {
    const float* prow = P.proj + (size_t)(b * P.T + t) * P.proj_stride;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int i = tid + m * kHeadThreads;
      av[m] = i < NCH ? prow[chan[m]] : 0.0f;
      lrv[m] = i < rl ? prow[C + i] : 0.0f;
    }
    if (tid == 0) blog = prow[C + rl + h];
  };
  load_token(0);

  for (int t = 0; t < ntok; ++t) {
    const int n = b * P.T + t;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int ci = tid + m * kHeadThreads;
      if (ci < NCH) {
        float a = av[m];
        if (P.conv_in_head) {
          const float y = cw[m][0] * z[m][0] + cw[m][1] * z[m][1] + cw[m][2] * z[m][2] + cw[m][3] * a;
          z[m][0] = z[m][1];
          z[m][1] = z[m][2];
          z[m][2] = a;
          a = silu_f(y);
        }
        if (ci < 2 * DK) s_qk[ci] = a; else s_v[ci - 2 * DK] = a;
      }
      const int i = tid + m * kHeadThreads;
      if (i < rl) s_lr[i] = lrv[m];
    }
    if (tid == 0) s_misc[2] = sigmoid_f(blog);
    if (t + 1 < ntok) load_token(t + 1);
    __syncthreads();
    const float a_h = expf(a_log_h);
    // ---- L2 norms of q (wave 0) and k (wave 1) ----
    if (wave < 2) {
      const float* src = s_qk + wave * DK;
      float a = 0.0f;
      for (int i = lane; i < DK; i += 64) a += src[i] * src[i];
      a = wave_sum(a);
      if (lane == 0) s_misc[wave] = 1.0f / sqrtf(a + P.l2_eps);
    }
    // ---- forget gate alpha (per key channel) and output gate (this block's columns) ----
#pragma unroll
    for (int m = 0; m < kMaxLrLoads; ++m) {
      if (m < nld) {
        const int it = tid + m * kHeadThreads;
        float part = 0.0f;
        int rloc = 0, c = 0;
        if (it < items) {
          rloc = it / cpr;
          c = it - rloc * cpr;
          const float* xv = rloc < DK ? s_lr + c * EL : s_lr + P.rank_f + c * EL;
          part = hchunk_dot<WT>(lw[m], xv);
          if constexpr (WT == kQ8) part *= lsc[m];
        }
        for (int o = 1; o < cpr; o <<= 1) part += __shfl_xor(part, o, kWave);
        if (it < items && c == 0) {
          if (rloc < DK) {
            s_alpha[rloc] = expf(-a_h * softplus_f(part + lbias[m]));
          } else {
            s_gate[rloc - DK] = sigmoid_f(part);
          }
        }
      }
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

template <int DK>
static void launch_dk(const HeadParams& p, dim3 grid, hipStream_t s) {
  if (p.wt == kF32)
    head_kernel<DK, kF32><<<grid, kHeadThreads, 0, s>>>(p);
  else if (p.wt == kBF16)
    head_kernel<DK, kBF16><<<grid, kHeadThreads, 0, s>>>(p);
  else
    head_kernel<DK, kQ8><<<grid, kHeadThreads, 0, s>>>(p);
}

// Loads of F_b / G_b chunks a thread holds: (dk + 32 rows) x rank*bytes/16 chunks / 256.
bool head_supported(int dk, int wt, int rank_f, int rank_g) {
  const int by = wt == kF32 ? 4 : (wt == kBF16 ? 2 : 1);
  if (rank_f != rank_g) return false;
  const int cpr = rank_f * by / 16;
  if (cpr < 1 || cpr > 64 || (cpr & (cpr - 1))) return false;
  const int items = (dk + kHeadCols) * cpr;
  return (items + kHeadThreads - 1) / kHeadThreads <= kMaxLrLoads;
}

hipError_t launch_head(const HeadParams& p, hipStream_t s) {
  dim3 grid(p.dv / kHeadCols, p.H, p.B);
  if (p.dk == 128)
    launch_dk<128>(p, grid, s);
  else
    launch_dk<64>(p, grid, s);
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

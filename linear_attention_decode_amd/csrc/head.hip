// Per-head kernels of the KDA step for gfx950: the forget / output gates (low-rank
// up-projections F_b and G_b) and the gated delta rule with its conv (verify / commit),
// L2-normalised q and k and read-out o = S^T q.
//
// Steps as listed under "Where the time goes" in "Thirty tiny kernels per layer"
// (frederic.ai) and written as its pure decode step; the forget gate is the workload's
// alpha = exp(-exp(A_log[h]) softplus(F_b F_a u + dt_bias)), one A_log per head as in the
// KDA recurrence-kernel commit of antirez/ds4 PR #964.
//
// Per token (column j, key rows i of the head):
//   S'_ij = alpha_i S_ij ;  e_j = sum_i S'_ij k_i ;  delta_j = beta (v_j - e_j)
//   S_ij = S'_ij + k_i delta_j ;  o_j = sum_i S_ij q_i
// Value columns are independent, so each wave owns 32 of them with the whole key
// dimension in registers and needs no other wave; the state is read once and written
// once per call (verify keeps it in registers across its tokens and writes nothing).
#include <type_traits>
#include <utility>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int WT>
struct HFmt;
template <>
struct HFmt<kF32> { static constexpr int kElems = 4; static constexpr int kBytes = 4; };
template <>
struct HFmt<kBF16> { static constexpr int kElems = 8; static constexpr int kBytes = 2; };
template <>
struct HFmt<kQ8> { static constexpr int kElems = 16; static constexpr int kBytes = 1; };
template <>
struct HFmt<kMX4> { static constexpr int kElems = 32; static constexpr int kBytes = 1; };

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

// ---------------------------------------------------------------------------------------
// Gates: alpha from f = F_b f_lr + dt_bias per key channel (per head for the scalar gate)
// and gate = sigmoid(G_b g_lr) per value channel, for N tokens.  Rows of F_b (then G_b) are
// split into 16-byte chunks; a row's CPR chunks sit in adjacent lanes and reduce by DPP.
// The forget-gate forms:
//   KDA      alpha = exp(-exp(A_log[h]) softplus(f))              (per key channel)
//   safe     alpha = exp(lb sigmoid(-f a[h])), a[h] as given      (per key channel)
//   scalar   alpha = exp(-exp(A_log[h]) softplus(f_h))            (per head, on all channels)
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float forget_alpha_f(int gate, float f, float ah, float lb) {
  if (gate == kGateSafe) return expf(lb * sigmoid_f(-f * ah));
  return expf(-expf(ah) * softplus_f(f));
}

constexpr int kGateThreads = 256;
constexpr int kMaxRank = 256;
constexpr int kGateCols = 16;    // columns staged per round (a multiple of every CPR)

template <int WT, int CPR>
__global__ __launch_bounds__(kGateThreads) void gates_kernel(const GatesParams P) {
  constexpr int EL = HFmt<WT>::kElems;
  __shared__ __align__(16) float s_lr[kGateCols][2 * kMaxRank];
  const int tid = threadIdx.x;
  // forget rows (one per key channel, or one per head for the scalar gate), then gate rows
  const bool scalar = P.gate == kGateScalar;
  const int FR = scalar ? P.K / P.dk : P.K;
  const int rows = FR + P.V, ostride = P.K + P.V;
  const int it = blockIdx.x * kGateThreads + tid;
  const int row = it / CPR, c = it - row * CPR;
  const bool valid = row < rows;
  const bool f = row < FR;
  const int rank = P.rank;
  uint4 w = make_uint4(0, 0, 0, 0);
  float sc = 1.0f, bias = 0.0f, ah = 0.0f;
  if (valid) {
    const PackedMat M = f ? P.fb : P.gb;
    const int r = f ? row : row - FR;
    w = *reinterpret_cast<const uint4*>(M.w + ((size_t)r * (rank / EL) + c) * 16);
    if constexpr (WT == kQ8) sc = __half2float(M.d[(size_t)r * (rank / 32) + (c >> 1)]);
    if constexpr (WT == kMX4) sc = __builtin_amdgcn_ldexpf(1.0f, (int)M.e[(size_t)r * (rank / 32) + c] - 128);
    if (f) {
      bias = P.dt_bias[row];
      ah = P.a_log[scalar ? row : row / P.dk];
    }
  }
  // kGateCols columns' low-rank inputs per round (the rounds are spread over blockIdx.y),
  // staged with independent loads; within a round, the CPR lanes of a row's group each
  // finish one of CPR consecutive columns
  for (int n0 = blockIdx.y * kGateCols; n0 < P.N; n0 += gridDim.y * kGateCols) {
    const int nc = min(kGateCols, P.N - n0);
    {
      // all loads first (a fixed, unrolled count per thread, indices clamped so no load
      // sits behind a branch), then the LDS stores
      constexpr int kStage = kGateCols * 2 * kMaxRank / 4 / kGateThreads;
      const int per4 = 2 * rank / 4, total4 = nc * per4;
      f32x4 v[kStage];
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int i = min(tid + u * kGateThreads, total4 - 1);
        const int nn = i / per4, k4 = i - nn * per4;
        v[u] = *reinterpret_cast<const f32x4*>(P.proj + (size_t)(n0 + nn) * P.proj_stride + P.C + 4 * k4);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the loads together, ahead of the stores
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int i = tid + u * kGateThreads;
        if (i < total4) {
          const int nn = i / per4, k4 = i - nn * per4;
          *reinterpret_cast<f32x4*>(&s_lr[nn][4 * k4]) = v[u];
        }
      }
    }
    __syncthreads();
    for (int nb = 0; nb < nc; nb += CPR) {
      float mine = 0.0f;
#pragma unroll
      for (int g = 0; g < CPR; ++g) {
        const int nn = nb + g;
        float part = 0.0f;
        if (valid && nn < nc) {
          if constexpr (WT == kMX4)
            part = sc * mx4_chunk_dot2(w, (f ? s_lr[nn] : s_lr[nn] + rank) + c * EL);
          else
            part = hchunk_dot<WT>(w, (f ? s_lr[nn] : s_lr[nn] + rank) + c * EL);
          if constexpr (WT == kQ8) part *= sc;
        }
        part = group_sum(part, CPR);
        if (c == g) mine = part;
      }
      const int nn = nb + c;
      if (valid && nn < nc) {
        float* orow = P.out + (size_t)(n0 + nn) * ostride;
        if (!f) {
          orow[P.K + row - FR] = sigmoid_f(mine);
        } else {
          const float a = forget_alpha_f(P.gate, mine + bias, ah, P.gate_lb);
          if (scalar)
            for (int i = 0; i < P.dk; ++i) orow[row * P.dk + i] = a;
          else
            orow[row] = a;
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// The same gates for N > 1 token columns on the int8 matrix cores, from F_b and G_b in
// gate-tile order (per tile of 16 rows: [2 halves][rank/32 blocks][16 rows][16 bytes] of
// signed q, scales [tile][rank/32][16]).  A block takes 4 tiles (one per wave) and 8 token
// columns.  It first turns each column's f_lr and g_lr into three signed 7-bit planes per
// 32-element block under the block's own power-of-two scale (x s = x0 + x1/128 + x2/16384
// + r, |r| <= 2^-15, every product exact in int32).  Then, per column, A row 4 i + p holds
// plane p of block i on lane group i and B the tile's bytes, so accumulator lane (n, g) has
// block g's plane dots for row n; each block's scales are applied there and the four lane
// groups summed.  Lane group g finishes columns g and 4 + g of its row.
// ---------------------------------------------------------------------------------------
typedef int i32x4g __attribute__((ext_vector_type(4)));
constexpr int kGmCols = 8;       // token columns per block

// The steps of the matrix-core gates, shared with the head kernel's own gates, each with
// contraction off so that both places round alike (the gates are then bit for bit the same
// whichever kernel computes them).
// Element u of a 32-element block held by a half-wave: its three planes and the block's
// inverse scale.
struct GmPlanes {
  int8_t q0, q1, q2;
  float inv;
};
__device__ __forceinline__ GmPlanes gm_quantise(float u) {
#pragma clang fp contract(off)
  constexpr float M = 12582912.0f;
  float ss = sum16(u * u);
  ss += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(ss), 0x401F));   // lane ^ 16
  const int ex = (__builtin_amdgcn_frexp_expf(ss) + 1) >> 1;
  const float sc = __builtin_amdgcn_ldexpf(1.0f, 6 - ex);
  const float t0 = fmaf(u, sc, M), q0 = t0 - M, r0 = fmaf(u, sc, -q0);
  const float t1 = fmaf(r0, 128.0f, M), q1 = t1 - M, r1 = fmaf(r0, 128.0f, -q1);
  const float t2 = fmaf(r1, 128.0f, M);
  return {(int8_t)__float_as_uint(t0), (int8_t)__float_as_uint(t1), (int8_t)__float_as_uint(t2),
          __builtin_amdgcn_ldexpf(1.0f, ex - 6)};
}
// One (tile, column) MFMA result: block g's plane dots in lane group g, weighed by the
// block's weight scale dsc and inverse input scale gi (live: g < blocks), summed over the
// four groups (every group ends with the total).
__device__ __forceinline__ float gm_row(const i32x4g c, float dsc, float gi, bool live) {
#pragma clang fp contract(off)
  const float v = fmaf((float)(c[1] * 128 + c[2]), 1.0f / 16384.0f, (float)c[0]);
  float y = live ? dsc * gi * v : 0.0f;
  y += __shfl_xor(y, 16);
  y += __shfl_xor(y, 32);
  return y;
}
__device__ __forceinline__ float gm_alpha(float ah, float x) {
#pragma clang fp contract(off)
  return expf(-expf(ah) * softplus_f(x));
}
__device__ __forceinline__ float gm_gate(float x) {
#pragma clang fp contract(off)
  return sigmoid_f(x);
}

template <int CPR>
__global__ __launch_bounds__(256) void gates_mfma_kernel(const GatesParams P) {
  constexpr int NB = CPR / 2, rank = CPR * 16;     // Q8_0 blocks per row, rank
  __shared__ __align__(16) int8_t gpl[kGmCols][4][256];   // [column][plane][f | g]; plane 3 = 0
  __shared__ float ginv[kGmCols][8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.y * kGmCols, nc = min(kGmCols, P.N - n0);
  // this wave's weight tile, scales, bias and A_log are requested first: they do not depend
  // on the columns, so their latency overlaps the columns' load and quantisation below
  const int ftiles = P.K / 16, tau = blockIdx.x * 4 + wave;
  const bool live = tau < (P.K + P.V) / 16;
  const bool f = tau < ftiles;
  const int tl = f ? tau : tau - ftiles;
  const int m = lane & 15, g = lane >> 4;
  i32x4g bw0 = {0, 0, 0, 0}, bw1 = {0, 0, 0, 0};
  float dsc = 0.0f;
  if (live && g < NB) {
    const int8_t* bp = (f ? P.fbw : P.gbw) + (size_t)tl * 16 * rank + (g * 16 + m) * 16;
    bw0 = *reinterpret_cast<const i32x4g*>(bp);
    bw1 = *reinterpret_cast<const i32x4g*>(bp + NB * 256);
    const uint16_t* dp = (f ? P.fbd : P.gbd) + ((size_t)tl * NB + g) * 16 + m;
    dsc = __half2float(__ushort_as_half(*dp));
  }
  const int row = 16 * tau + m;              // alpha rows, then gate rows
  float bias = 0.0f, ah = 0.0f;
  if (live && f) {
    bias = P.dt_bias[row];
    ah = P.a_log[row / P.dk];
  }
  {
    // thread t: column t / 32, element t % 32 of each 32-element block (a half-wave a block)
    const int cn = tid >> 5, j = tid & 31;
#pragma unroll
    for (int blk = 0; blk < 2 * NB; ++blk) {
      const float u = cn < nc ? P.proj[(size_t)(n0 + cn) * P.proj_stride + P.C + 32 * blk + j] : 0.0f;
      const GmPlanes q = gm_quantise(u);
      const int e = 32 * blk + j;
      gpl[cn][0][e] = q.q0;
      gpl[cn][1][e] = q.q1;
      gpl[cn][2][e] = q.q2;
      gpl[cn][3][e] = 0;
      if (j == 0) ginv[cn][blk] = q.inv;
    }
    // the rest of the zero plane (lane groups past the last block read it)
    for (int e = 2 * rank + j; e < 256; e += 32) gpl[cn][3][e] = 0;
  }
  __syncthreads();
  if (!live) return;
  const int8_t* abase = &gpl[0][(m >> 2) == g && g < NB ? (m & 3) : 3][(f ? 0 : rank) + 32 * g];
  const i32x4g zero = {0, 0, 0, 0};
  float res[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    float ys[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cn = 4 * r + q;
      const int8_t* pa = abase + cn * 4 * 256;
      i32x4g c = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<const i32x4g*>(pa), bw0, zero, 0, 0, 0);
      c = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<const i32x4g*>(pa + 16), bw1, c, 0, 0, 0);
      ys[q] = gm_row(c, dsc, ginv[cn][(f ? 0 : NB) + min(g, NB - 1)], g < NB);
    }
    res[r] = g == 0 ? ys[0] : g == 1 ? ys[1] : g == 2 ? ys[2] : ys[3];
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int cn = 4 * r + g;
    if (cn < nc)
      P.out[(size_t)(n0 + cn) * (P.K + P.V) + row] = f ? gm_alpha(ah, res[r] + bias) : gm_gate(res[r]);
  }
}

template <int WT>
static void launch_gates_wt(const GatesParams& p, hipStream_t s) {
  const int cpr = p.rank / HFmt<WT>::kElems;
  const int items = ((p.gate == kGateScalar ? p.K / p.dk : p.K) + p.V) * cpr;
  const dim3 grid((items + kGateThreads - 1) / kGateThreads,
                  std::min(8, (p.N + kGateCols - 1) / kGateCols));
  switch (cpr) {
    case 1: gates_kernel<WT, 1><<<grid, kGateThreads, 0, s>>>(p); break;
    case 2: gates_kernel<WT, 2><<<grid, kGateThreads, 0, s>>>(p); break;
    case 4: gates_kernel<WT, 4><<<grid, kGateThreads, 0, s>>>(p); break;
    case 8: gates_kernel<WT, 8><<<grid, kGateThreads, 0, s>>>(p); break;
    default: gates_kernel<WT, 16><<<grid, kGateThreads, 0, s>>>(p); break;
  }
}

hipError_t launch_gates(const GatesParams& p, hipStream_t s) {
  const int nbq = p.rank / 32;
  if (p.fbw && p.gate == kGateKda && p.wt == kQ8 && (p.rank == 32 || p.rank == 64 || p.rank == 128) &&
      p.K % 16 == 0 && p.V % 16 == 0) {
    const dim3 grid(((p.K + p.V) / 16 + 3) / 4, (p.N + kGmCols - 1) / kGmCols);
    if (nbq == 1) gates_mfma_kernel<2><<<grid, 256, 0, s>>>(p);
    else if (nbq == 2) gates_mfma_kernel<4><<<grid, 256, 0, s>>>(p);
    else gates_mfma_kernel<8><<<grid, 256, 0, s>>>(p);
    return hipGetLastError();
  }
  if (p.wt == kF32)
    launch_gates_wt<kF32>(p, s);
  else if (p.wt == kBF16)
    launch_gates_wt<kBF16>(p, s);
  else if (p.wt == kMX4)
    launch_gates_wt<kMX4>(p, s);
  else
    launch_gates_wt<kQ8>(p, s);
  return hipGetLastError();
}

bool head_supported(int dk, int wt, int rank_f, int rank_g) {
  (void)dk;
  const int el = wt == kF32 ? 4 : (wt == kBF16 ? 8 : (wt == kMX4 ? 32 : 16));
  if (rank_f != rank_g || rank_f > kMaxRank || rank_f % el) return false;
  const int cpr = rank_f / el;
  return cpr >= 1 && cpr <= 16 && (cpr & (cpr - 1)) == 0;
}

// ---------------------------------------------------------------------------------------
// Delta rule: one wave per (CW value columns, head, sequence).  Lane (rg = lane % RG,
// cq = lane / RG, RG = 256 / CW row groups) holds state rows rg*RPT .. rg*RPT + RPT - 1 of
// columns 4cq .. 4cq + 3 of the wave's CW as float4s; column sums reduce over the row
// groups (low lane bits) with DPP, the L2 norms over the same row groups.  No LDS, no
// barrier.  Tokens of a sequence (verify, commit) run in order, the next token's inputs
// requested while the current one is computed.
// ---------------------------------------------------------------------------------------
template <int RG>
__device__ __forceinline__ float rowsum(float v) {
  if constexpr (RG == 8) return sum8(v);
  else return sum16(v);
}

// f(integral_constant<U>) for U = FIRST, FIRST + 1, ... while U < n (at most LAST - 1),
// each call nested inside the test of the one before
template <int U, int LAST, typename F>
__device__ __forceinline__ void unroll_nested(int n, F& f) {
  if constexpr (U < LAST) {
    if (U < n) {
      f(std::integral_constant<int, U>{});
      unroll_nested<U + 1, LAST>(n, f);
    }
  }
}

// token steps unrolled per round of the head kernel's token loop (even: the two input sets
// alternate), enough for a verify with a folded commit (at most 8 + 8 tokens) in one round
constexpr int kHeadUnroll = 16;

// Fused decode gates (one token, no replay): each head wave computes the gates it needs
// from the token's f_lr, g_lr itself instead of reading them from a gates launch: alpha of
// all DK forget rows of its head (lane l takes rows l, l + 64, ... whole, so no reduction;
// the scalar form: the head's one row, a chunk a lane) and sigmoid of its CW output-gate
// rows (four lanes a row).  Every chunk is requested first thing in the kernel, ahead of the
// state; f_lr | g_lr are staged in LDS and read as broadcasts.  (Measured against a variant
// with whole-wave coalesced loads transposed through LDS: the staging cost more than the
// coalescing saved.)  Row-major F_b, G_b; a model's own gate-tile-order copy takes the
// matrix-core form below.
constexpr int kFgGateChunks = 4;    // chunks of a gate row a lane (four lanes a row)

// chunk c of row r: its 16 bytes and the raw bits of its scale (fp16 for Q8_0, the E8M0
// exponent for MXFP4; converted where used, so a load is not waited for early); wb, sb are
// the matrix's data and scale planes
template <int GT>
__device__ __forceinline__ void fg_chunk(const uint8_t* wb, const void* sb, int r, int c, int rank,
                                         uint4& w, uint32_t& sc) {
  constexpr int EL = HFmt<GT>::kElems;
  w = *reinterpret_cast<const uint4*>(wb + ((size_t)r * (rank / EL) + c) * 16);
  if constexpr (GT == kQ8)
    sc = static_cast<const uint16_t*>(sb)[(size_t)r * (rank / 32) + (c >> 1)];
  else if constexpr (GT == kMX4)
    sc = static_cast<const uint8_t*>(sb)[(size_t)r * (rank / 32) + c];
  else
    sc = 0;
}

template <int GT>
__device__ __forceinline__ float fg_dot(uint4 w, uint32_t sc, const float* __restrict__ x) {
  if constexpr (GT == kMX4) {
    return __builtin_amdgcn_ldexpf(1.0f, (int)sc - 128) * mx4_chunk_dot2(w, x);
  } else if constexpr (GT == kQ8) {
    return __half2float(__ushort_as_half((unsigned short)sc)) * hchunk_dot<kQ8>(w, x);
  } else {
    return hchunk_dot<GT>(w, x);
  }
}

// alpha of the head's DK forget rows into s_al, sigmoid of the wave's CW output-gate rows
// into s_gt.  start() requests every input (the first RC chunks of each forget row, the gate
// chunks, f_lr | g_lr, bias, A_log); finish() waits for them and computes (requesting any
// further chunks of long rows as it goes).  n is the token's column, cb the wave's column
// block.
template <int GT, int DK, int CW>
struct FusedGates {
  static constexpr int EL = HFmt<GT>::kElems;
  static constexpr int RL = DK / 64;            // forget rows a lane
  // forget-row chunks in flight a row: all 16 of a 128-rank BF16 row; 8 for the byte formats
  // (the scales take registers too)
  static constexpr int RC = (GT == kBF16 || GT == kF32) ? 16 : 8;
  static_assert(CW == 16, "four lanes a gate row");
  int cpr, rank, h;
  bool scalar;
  float ah;
  float bias[RL];
  float4 lv[2];
  const uint8_t* fwp;
  const void* fsp;
  uint4 fw[RL][RC];
  uint32_t fs[RL][RC];
  uint4 gw[kFgGateChunks];
  uint32_t gs[kFgGateChunks];

  __device__ __forceinline__ void issue_rows(int c0) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < RL; ++i)
#pragma unroll
      for (int c = 0; c < RC; ++c)   // (clamped, not branched: no wait where paths join)
        fg_chunk<GT>(fwp, fsp, h * DK + lane + 64 * i, min(c0 + c, cpr - 1), rank, fw[i][c], fs[i][c]);
  }

  __device__ __forceinline__ void start(const HeadParams& P, int n, int h_, int cb) {
    const int lane = threadIdx.x & 63;
    h = h_;
    rank = P.rank_f;
    cpr = rank / EL;
    scalar = P.gate_form == kGateScalar;
    fwp = P.fb.w;
    fsp = GT == kMX4 ? static_cast<const void*>(P.fb.e) : static_cast<const void*>(P.fb.d);
    const uint8_t* gwp = P.gb.w;
    const void* gsp = GT == kMX4 ? static_cast<const void*>(P.gb.e) : static_cast<const void*>(P.gb.d);
    if (scalar)
      fg_chunk<GT>(fwp, fsp, h, min(lane, cpr - 1), rank, fw[0][0], fs[0][0]);
    else
      issue_rows(0);
    const int grow = h * P.dv + cb * CW + (lane >> 2);
#pragma unroll
    for (int k = 0; k < kFgGateChunks; ++k)
      fg_chunk<GT>(gwp, gsp, grow, min((lane & 3) + 4 * k, cpr - 1), rank, gw[k], gs[k]);
    const float* lr = P.proj + (size_t)n * P.proj_stride + P.C;
#pragma unroll
    for (int k = 0; k < 2; ++k)     // 2 rank floats: at most 128 float4s
      lv[k] = *reinterpret_cast<const float4*>(lr + 4 * min(lane + 64 * k, rank / 2 - 1));
#pragma unroll
    for (int i = 0; i < RL; ++i) bias[i] = P.dt_bias[scalar ? h : h * DK + lane + 64 * i];
    ah = P.a_log[h];
  }

  __device__ __forceinline__ void finish(const HeadParams& P, float* s_gl, float* s_al, float* s_gt) {
    const int lane = threadIdx.x & 63;
    // (lanes past the vector store its last float4 again: the same value)
#pragma unroll
    for (int k = 0; k < 2; ++k)
      *reinterpret_cast<float4*>(s_gl + 4 * min(lane + 64 * k, rank / 2 - 1)) = lv[k];
    __syncthreads();
    if (scalar) {
      float f = lane < cpr ? fg_dot<GT>(fw[0][0], fs[0][0], s_gl + lane * EL) : 0.0f;
      f = group_sum(f, 16);                     // cpr <= 16: lanes 0..15 hold the row
      f = __shfl(f, 0);
      const float a = forget_alpha_f(kGateKda, f + bias[0], ah, P.gate_lb);
#pragma unroll
      for (int i = 0; i < RL; ++i) s_al[lane + 64 * i] = a;
    } else {
      float f[RL];
#pragma unroll
      for (int i = 0; i < RL; ++i) f[i] = 0.0f;
      for (int c0 = 0;;) {
#pragma unroll
        for (int i = 0; i < RL; ++i)
#pragma unroll
          for (int c = 0; c < RC; ++c)
            if (c0 + c < cpr) f[i] += fg_dot<GT>(fw[i][c], fs[i][c], s_gl + (c0 + c) * EL);
        c0 += RC;
        if (c0 >= cpr) break;
        issue_rows(c0);
      }
#pragma unroll
      for (int i = 0; i < RL; ++i)
        s_al[lane + 64 * i] = forget_alpha_f(P.gate_form, f[i] + bias[i], ah, P.gate_lb);
    }
    float g = 0.0f;
#pragma unroll
    for (int k = 0; k < kFgGateChunks; ++k) {
      const int c = (lane & 3) + 4 * k;
      if (c < cpr) g += fg_dot<GT>(gw[k], gs[k], s_gl + rank + c * EL);
    }
    g = group_sum(g, 4);
    if ((lane & 3) == 0) s_gt[lane >> 2] = sigmoid_f(g);
    __syncthreads();
  }
};
struct FusedNone {};

// Gates of this call's tokens on the int8 matrix cores, inside the head kernel, for a model
// with its own gate-tile-order copy (KDA form, rank = 16 CPR in {32, 64, 128}): the same
// arithmetic, in the same order, as gates_mfma_kernel (so the gates are bit for bit those
// of the separate launch).  The wave's 8 forget tiles (the head's DK rows) and its gate tile
// are requested at kernel entry; each of the call's T tokens (at most kFmMaxTok: one-token
// steps only, since at verify's 4 tokens the per-token serial chain below cost more than the
// separate launch) is
// quantised into three 7-bit planes per 32-element block in LDS, then per (token, tile) two
// MFMAs give each lane group a block's plane dots, which the block scales weigh and the
// four groups sum.  alpha goes to s_al[t][row], gate to s_gt[t][column], and (ag_out set) to
// the rows that a later replay of these tokens reads.
constexpr int kGateMfma = 200;   // head_kernel GT = kGateMfma + CPR
constexpr int kFmMaxTok = 1;

template <int CPR, int DK, int CW>
struct FusedGatesMfma {
  static constexpr int NB = CPR / 2, rank = CPR * 16;
  static constexpr int FT = DK / 16;             // forget tiles of the head
  static constexpr int RL = DK / 64;             // forget rows a lane in the last pass
  static constexpr int NP = 2 * rank / 64;       // 64-element passes over f_lr | g_lr
  i32x4g bw[FT + 1][2];
  uint32_t bd[FT + 1];
  float dtb[RL];
  float ah;
  float u[kFmMaxTok][NP];                         // f_lr | g_lr of the tokens, lane's elements

  // n0, T: this call's tokens (columns of proj)
  __device__ __forceinline__ void start(const HeadParams& P, int h, int cb, int n0, int T) {
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    // (token index clamped, not branched on: no wait where paths would join)
#pragma unroll
    for (int t = 0; t < kFmMaxTok; ++t) {
      const float* lr = P.proj + (size_t)(n0 + min(t, T - 1)) * P.proj_stride + P.C;
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) u[t][pp] = lr[64 * pp + lane];
    }
    const int gc = min(g, NB - 1);               // groups past the last block: any valid
#pragma unroll                                   // bytes (their A operand is the zero plane)
    for (int tt = 0; tt <= FT; ++tt) {
      const bool f = tt < FT;
      const int tl = f ? h * FT + tt : (h * P.dv + cb * CW) >> 4;
      const int8_t* bp = (f ? P.fbw : P.gbw) + (size_t)tl * 16 * rank + (gc * 16 + m) * 16;
      bw[tt][0] = *reinterpret_cast<const i32x4g*>(bp);
      bw[tt][1] = *reinterpret_cast<const i32x4g*>(bp + NB * 256);
      bd[tt] = (f ? P.fbd : P.gbd)[((size_t)tl * NB + gc) * 16 + m];
    }
#pragma unroll
    for (int i = 0; i < RL; ++i) dtb[i] = P.dt_bias[h * DK + lane + 64 * i];
    ah = P.a_log[h];
  }

  // tokens n0 .. n0 + T - 1 (columns of proj / alpha_gate)
  __device__ __forceinline__ void finish(const HeadParams& P, int n0, int T, int h, int cb,
                                         int8_t (*gpl)[4][256], float (*ginv)[8],
                                         float (*s_al)[DK], float (*s_gt)[CW]) {
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    // quantise: element e = 64 p + lane of f_lr | g_lr, block e / 32 on a half-wave
#pragma unroll
    for (int t = 0; t < kFmMaxTok; ++t) {
      if (t >= T) break;
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const int e = 64 * pp + lane, blk = e >> 5, jj = e & 31;
        const GmPlanes q = gm_quantise(this->u[t][pp]);
        gpl[t][0][e] = q.q0;
        gpl[t][1][e] = q.q1;
        gpl[t][2][e] = q.q2;
        if (jj == 0) ginv[t][blk] = q.inv;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) gpl[t][3][64 * k + lane] = 0;
    }
    __syncthreads();
    // per (token, tile): the raw row dots, stored by lane group 0
    const int8_t* abase0 = &gpl[0][(m >> 2) == g && g < NB ? (m & 3) : 3][32 * g];
    const i32x4g zero = {0, 0, 0, 0};
    for (int t = 0; t < T; ++t) {
      const int8_t* abase = abase0 + (size_t)t * 4 * 256;
#pragma unroll
      for (int tt = 0; tt <= FT; ++tt) {
        const bool f = tt < FT;
        const int8_t* pa = abase + (f ? 0 : rank);
        i32x4g c = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<const i32x4g*>(pa), bw[tt][0], zero, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<const i32x4g*>(pa + 16), bw[tt][1], c, 0, 0, 0);
        const float dsc = __half2float(__ushort_as_half((unsigned short)bd[tt]));
        const float y = gm_row(c, dsc, ginv[t][(f ? 0 : NB) + min(g, NB - 1)], g < NB);
        if (g == 0) {
          if (f) s_al[t][16 * tt + m] = y;
          else s_gt[t][m] = y;
        }
      }
    }
    __syncthreads();
    // the forms, a row (or column) a lane
    const size_t agw = (size_t)(P.H * DK + P.H * P.dv);
    for (int t = 0; t < T; ++t) {
      float* agr = P.ag_out + (size_t)(n0 + t) * agw;
#pragma unroll
      for (int i = 0; i < RL; ++i) {
        const int r = lane + 64 * i;
        const float a = gm_alpha(ah, s_al[t][r] + dtb[i]);
        s_al[t][r] = a;
        if (P.ag_out && cb == 0) agr[h * DK + r] = a;
      }
      if (lane < CW) {
        const float gt = gm_gate(s_gt[t][lane]);
        s_gt[t][lane] = gt;
        if (P.ag_out) agr[P.H * DK + h * P.dv + cb * CW + lane] = gt;
      }
    }
    __syncthreads();
  }
};

template <int DK, int CW, int GT>
__global__ __launch_bounds__(64) void head_kernel(const HeadParams P) {
  constexpr int RG = 256 / CW;
  constexpr int RPT = DK / RG;
  // block id = cb * (H B) + h * B + b: the dv / CW waves of one (sequence, head), which
  // read the same q, k and alpha rows (and with fused gates the same F_b rows), are H B
  // apart, so on one XCD (blocks go round-robin over the 8) whenever H B is a multiple of
  // 8, and those rows come from its L2
  const int hb = (int)blockIdx.x % (P.H * P.B);
  const int cb = (int)blockIdx.x / (P.H * P.B), h = hb / P.B, b = hb - h * P.B;
  const int lane = threadIdx.x;
  const int rg = lane % RG, cq = lane / RG;
  const int H = P.H, dv = P.dv, C = P.C, K = H * DK;
  const int j = cb * CW + cq * 4;             // this lane's first value column in the head
  const int r0 = rg * RPT;                     // this lane's first key row
  const int nparts = dv / CW;
  const int rl = P.rank_f + P.rank_g;
  constexpr bool kMf = GT >= kGateMfma;           // gates of this call's tokens on MFMA
  std::conditional_t<(GT >= kGateMfma), FusedGatesMfma<(kMf ? GT - kGateMfma : 8), DK, CW>,
                     std::conditional_t<(GT >= 0), FusedGates<(GT >= 0 && !kMf ? GT : kF32), DK, CW>,
                                        FusedNone>> fg;
  __shared__ __align__(16) float s_mal[kMf ? kFmMaxTok : 1][kMf ? DK : 1];
  __shared__ __align__(16) float s_mgt[kMf ? kFmMaxTok : 1][kMf ? CW : 1];
  if constexpr (kMf) fg.start(P, h, cb, b * P.T, P.T);
  else if constexpr (GT >= 0) fg.start(P, b, h, cb);

  float* Sb = P.S + ((size_t)b * H + h) * DK * dv + j;
  float4 st[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    st[i] = *reinterpret_cast<const float4*>(Sb + (size_t)(r0 + i) * dv);

  const int cq0 = h * DK + r0, ck0 = K + h * DK + r0, cv0 = 2 * K + h * dv + j;

  // token inputs (q, k rows and v columns of this lane; alpha rows; gate columns; beta),
  // requested two tokens ahead of their use
  struct Tok {
    float qv[RPT], kv[RPT], al[RPT], v4[4];
    float4 gate;
    float braw;
  };
  // One sequence of tokens: first (a commit folded into this verify) the previous verify's
  // accepted tokens from its log, state only, after which the state is written back; then
  // this call's tokens
  const int a_pre = P.pre_ntok ? min(max(P.pre_ntok[b], 1), P.pre_T) : 0;
  const int a_cur = P.ntok ? min(max(P.ntok[b], 1), P.T) : P.T;
  const int total = a_pre + a_cur;
  auto load_tok = [&](int u, Tok& x) __attribute__((always_inline)) {
    const bool pre = u < a_pre;
    const int n = pre ? b * P.pre_T + u : b * P.T + (u - a_pre);
    const float* prow = (pre ? P.pre_proj : P.proj) + (size_t)n * P.proj_stride;
    const float* sact = pre ? P.pre_act : P.act;
    const float* arow = sact ? sact + (size_t)n * C : prow;   // activated q | k | v
    const float* ag = (pre ? P.pre_ag : P.alpha_gate) + (size_t)n * (K + H * dv);
#pragma unroll
    for (int i = 0; i < RPT; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(arow + cq0 + i);
      const float4 k4 = *reinterpret_cast<const float4*>(arow + ck0 + i);
      x.qv[i] = a.x; x.qv[i + 1] = a.y; x.qv[i + 2] = a.z; x.qv[i + 3] = a.w;
      x.kv[i] = k4.x; x.kv[i + 1] = k4.y; x.kv[i + 2] = k4.z; x.kv[i + 3] = k4.w;
      if constexpr (GT < 0 || kMf) {
        const float4 g4 = kMf && !pre ? *reinterpret_cast<const float4*>(&s_mal[u - a_pre][r0 + i])
                                      : *reinterpret_cast<const float4*>(ag + h * DK + r0 + i);
        x.al[i] = g4.x; x.al[i + 1] = g4.y; x.al[i + 2] = g4.z; x.al[i + 3] = g4.w;
      }
    }
    const float4 a = *reinterpret_cast<const float4*>(arow + cv0);
    x.v4[0] = a.x; x.v4[1] = a.y; x.v4[2] = a.z; x.v4[3] = a.w;
    if constexpr (GT < 0 || kMf)
      x.gate = kMf && !pre ? *reinterpret_cast<const float4*>(&s_mgt[u - a_pre][cq * 4])
                           : *reinterpret_cast<const float4*>(ag + K + h * dv + j);
    x.braw = prow[C + rl + h];
  };
  // token u of the sequence from the inputs in x: state update, outputs (this call's
  // tokens), and the state written back after the last replayed token.  Every
  // multiply-add is an explicit fma, so each unrolled copy rounds the same way (a token's
  // results do not depend on its position in the launch: a folded commit gives the bits
  // of a separate replay)
  auto process = [&](const Tok& x, int u) __attribute__((always_inline)) {
    const bool outp = u >= a_pre && P.write_out;
    const int n = b * P.T + (u - a_pre);
    {
      const float (&qv)[RPT] = x.qv;
      const float (&kv)[RPT] = x.kv;
      const float (&al)[RPT] = x.al;
      const float (&v4)[4] = x.v4;
      const float4 gate = x.gate;
      const float beta = sigmoid_f(x.braw);
      // L2 norms over the head's DK rows: local rows, then the row groups
      float aq = 0.0f, ak = 0.0f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) { aq = __builtin_fmaf(qv[i], qv[i], aq); ak = __builtin_fmaf(kv[i], kv[i], ak); }
      const float inv_q = P.q_scale / sqrtf(rowsum<RG>(aq) + P.l2_eps);
      const float inv_k = 1.0f / sqrtf(rowsum<RG>(ak) + P.l2_eps);

      float e0 = 0.f, e1 = 0.f, e2 = 0.f, e3 = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float a = al[i], kk = kv[i] * inv_k;
        st[i].x *= a; st[i].y *= a; st[i].z *= a; st[i].w *= a;
        e0 = __builtin_fmaf(st[i].x, kk, e0); e1 = __builtin_fmaf(st[i].y, kk, e1);
        e2 = __builtin_fmaf(st[i].z, kk, e2); e3 = __builtin_fmaf(st[i].w, kk, e3);
      }
      e0 = rowsum<RG>(e0); e1 = rowsum<RG>(e1); e2 = rowsum<RG>(e2); e3 = rowsum<RG>(e3);
      const float d0 = beta * (v4[0] - e0), d1 = beta * (v4[1] - e1);
      const float d2 = beta * (v4[2] - e2), d3 = beta * (v4[3] - e3);
      float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float kk = kv[i] * inv_k, qq = qv[i] * inv_q;
        st[i].x = __builtin_fmaf(kk, d0, st[i].x); st[i].y = __builtin_fmaf(kk, d1, st[i].y);
        st[i].z = __builtin_fmaf(kk, d2, st[i].z); st[i].w = __builtin_fmaf(kk, d3, st[i].w);
        o0 = __builtin_fmaf(st[i].x, qq, o0); o1 = __builtin_fmaf(st[i].y, qq, o1);
        o2 = __builtin_fmaf(st[i].z, qq, o2); o3 = __builtin_fmaf(st[i].w, qq, o3);
      }
      if (outp) {
        o0 = rowsum<RG>(o0); o1 = rowsum<RG>(o1); o2 = rowsum<RG>(o2); o3 = rowsum<RG>(o3);
        if (rg == 0) {
          const size_t g = (size_t)n * H * dv + h * dv + j;
          *reinterpret_cast<float4*>(P.o + g) = make_float4(o0, o1, o2, o3);
          *reinterpret_cast<float4*>(P.gate + g) = gate;
        }
        // o^2 over the wave's columns: each row of 16 lanes holds 16 / RG column quads
        float q2 = __builtin_fmaf(o3, o3, __builtin_fmaf(o2, o2, __builtin_fmaf(o1, o1, o0 * o0)));
        if constexpr (RG == 8) q2 += dpp_mov<kDppRor8>(q2);
        const int qb = __float_as_int(q2);
        const float tot = (__int_as_float(__builtin_amdgcn_readlane(qb, 0)) + __int_as_float(__builtin_amdgcn_readlane(qb, 16))) +
                          (__int_as_float(__builtin_amdgcn_readlane(qb, 32)) + __int_as_float(__builtin_amdgcn_readlane(qb, 48)));
        if (lane == 0) P.ss[((size_t)n * H + h) * nparts + cb] = tot;
      }
    }
    if (u + 1 == a_pre) {
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        *reinterpret_cast<float4*>(Sb + (size_t)(r0 + i) * dv) = st[i];
    }
  };
  // two input sets in flight, used in turn; the token loop is unrolled into rounds of
  // nested steps (step u runs only after steps 0 .. u-1), so the compiler sees exactly
  // which loads are still outstanding at each use and waits for one set while the other's
  // are in flight; past the last token the loads repeat it
  Tok x0, x1;
  if constexpr (kMf) {
    __shared__ __align__(16) int8_t s_gpl[kFmMaxTok][4][256];
    __shared__ float s_ginv[kFmMaxTok][8];
    fg.finish(P, b * P.T, a_cur, h, cb, s_gpl, s_ginv, s_mal, s_mgt);
  }
  if constexpr (GT >= 0 && !kMf) {
    // fused decode gates: the sequence's one token, its gates computed here
    __shared__ __align__(16) float s_gl[2 * kMaxRank];
    __shared__ __align__(16) float s_al[DK];
    __shared__ __align__(16) float s_gt[CW];
    load_tok(0, x0);
    fg.finish(P, s_gl, s_al, s_gt);
#pragma unroll
    for (int i = 0; i < RPT; ++i) x0.al[i] = s_al[r0 + i];
    x0.gate = *reinterpret_cast<const float4*>(s_gt + cq * 4);
    process(x0, 0);
  } else {
    load_tok(0, x0);
    load_tok(min(1, total - 1), x1);
    for (int base = 0; base < total; base += kHeadUnroll) {
      auto step = [&](auto uc) __attribute__((always_inline)) {
        constexpr int k = decltype(uc)::value;
        const int u = base + k;
        if constexpr ((k & 1) == 0) {
          process(x0, u);
          load_tok(min(u + 2, total - 1), x0);
        } else {
          process(x1, u);
          load_tok(min(u + 2, total - 1), x1);
        }
      };
      unroll_nested<0, kHeadUnroll>(total - base, step);
    }
  }
  if (P.write_state && (!P.active || P.active[b])) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *reinterpret_cast<float4*>(Sb + (size_t)(r0 + i) * dv) = st[i];
  }

  // commit: the window becomes the last 3 of (window, p_0 .. p_{a-1}) per (sequence,
  // channel), a = the accepted tokens; every wave of the grid takes a strided share (the
  // replay above reads the logged activations, never the window)
  if (P.win_commit) {
    const int nwave = gridDim.x;
    const int wid = blockIdx.x;
    for (int i = wid * 64 + lane; i < C * P.B; i += nwave * 64) {
      const int sb = i / C, c = i - sb * C;
      const int a = P.ntok ? min(max(P.ntok[sb], 1), P.T) : P.T;
      float* z = P.win_commit + (size_t)sb * 3 * C + c;
      // row j of the new window is element a + j of (window rows 0..2, p_0 .. p_{a-1})
      float nz[3];
#pragma unroll
      for (int j = 0; j < 3; ++j)
        nz[j] = a + j < 3 ? z[(size_t)(a + j) * C]
                          : P.proj[(size_t)(sb * P.T + a + j - 3) * P.proj_stride + c];
      z[0] = nz[0];
      z[C] = nz[1];
      z[2 * C] = nz[2];
    }
  }
}

template <int GT>
static void launch_head_gt(const HeadParams& p, const dim3 grid, hipStream_t s) {
  if (p.dk == 128)
    head_kernel<128, kHeadCols, GT><<<grid, 64, 0, s>>>(p);
  else
    head_kernel<64, kHeadCols, GT><<<grid, 64, 0, s>>>(p);
}

hipError_t launch_head(const HeadParams& p, hipStream_t s) {
  if (p.fuse_gates == 1 && (p.T != 1 || p.pre_ntok)) return hipErrorInvalidValue;
  const dim3 grid((p.dv / kHeadCols) * p.H * p.B);
  if (p.fuse_gates == 2) {
    const int cpr = p.rank_f / 16;
    if (p.dk != 128 || p.T > kFmMaxTok || p.gate_form != kGateKda || !p.fbw || p.rank_g != p.rank_f ||
        (cpr != 2 && cpr != 4 && cpr != 8))
      return hipErrorInvalidValue;
    if (cpr == 2) head_kernel<128, kHeadCols, kGateMfma + 2><<<grid, 64, 0, s>>>(p);
    else if (cpr == 4) head_kernel<128, kHeadCols, kGateMfma + 4><<<grid, 64, 0, s>>>(p);
    else head_kernel<128, kHeadCols, kGateMfma + 8><<<grid, 64, 0, s>>>(p);
    return hipGetLastError();
  }
  if (!p.fuse_gates) launch_head_gt<-1>(p, grid, s);
  else if (p.wt == kF32) launch_head_gt<kF32>(p, grid, s);
  else if (p.wt == kBF16) launch_head_gt<kBF16>(p, grid, s);
  else if (p.wt == kMX4) launch_head_gt<kMX4>(p, grid, s);
  else launch_head_gt<kQ8>(p, grid, s);
  return hipGetLastError();
}

// Conv + SiLU over a sequence's T tokens, one thread per (channel, sequence); the window is
// read, not rolled (verify leaves the state as committed), except for the roll by a
// previous verify's accepted tokens when a commit is folded in.
__global__ void conv_seq_kernel(const float* __restrict__ plog, int stride, float* __restrict__ win,
                                const float* __restrict__ conv_w, float* __restrict__ act, int T,
                                int C, const float* __restrict__ pre_plog,
                                const int* __restrict__ pre_ntok, int pre_T) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int b = blockIdx.y;
  if (c >= C) return;
  float* z = win + (size_t)b * 3 * C + c;
  float z0, z1, z2;
  if (pre_ntok) {
    const int a = min(max(pre_ntok[b], 1), pre_T);
    const float* pp = pre_plog + (size_t)b * pre_T * stride + c;
    z0 = a < 3 ? z[(size_t)a * C] : pp[(size_t)(a - 3) * stride];
    z1 = a < 2 ? z[(size_t)(a + 1) * C] : pp[(size_t)(a - 2) * stride];
    z2 = pp[(size_t)(a - 1) * stride];
    z[0] = z0;
    z[C] = z1;
    z[2 * C] = z2;
  } else {
    z0 = z[0];
    z1 = z[C];
    z2 = z[2 * C];
  }
  const float4 w = *reinterpret_cast<const float4*>(conv_w + (size_t)c * 4);
  // tokens in groups of 8, each group's projections requested together
  for (int t0 = 0; t0 < T; t0 += 8) {
    float p[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) p[t] = plog[(size_t)(b * T + min(t0 + t, T - 1)) * stride + c];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t0 + t < T) {
        const float y = conv4_f(w, z0, z1, z2, p[t]);
        z0 = z1;
        z1 = z2;
        z2 = p[t];
        act[(size_t)(b * T + t0 + t) * C + c] = silu_f(y);
      }
    }
  }
}

hipError_t launch_conv_seq(const float* plog, int proj_stride, float* win, const float* conv_w,
                           float* act, int B, int T, int C, const float* pre_plog,
                           const int* pre_ntok, int pre_T, hipStream_t s) {
  dim3 grid((C + 255) / 256, B);
  conv_seq_kernel<<<grid, 256, 0, s>>>(plog, proj_stride, win, conv_w, act, T, C, pre_plog,
                                       pre_ntok, pre_T);
  return hipGetLastError();
}

}  // namespace kda

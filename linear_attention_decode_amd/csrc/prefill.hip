// Chunked prefill of one KDA layer on gfx950, between the input and output projection
// GEMMs (gemm.hip): per (chunk, head) the causal conv + SiLU, L2 norms, gates and the WY/UT
// preparation; the sequential scan over chunks that carries the fp32 state; the gated
// RMSNorm; the final conv window.
//
// The chunked form is the chunk_kda pipeline of torad-labs/llama.cpp PR #84 (per chunk of
// C tokens and per head, G = the inclusive sum of each key channel's log-decay along the
// chunk, so every exponent below is <= 0 unless stated):
//   L[t][s] = beta_t sum_i k_t[i] k_s[i] 2^(G_t[i] - G_s[i])   (s < t)
//   A[t][s] = sum_i q_t[i] k_s[i] 2^(G_t[i] - G_s[i])           (s <= t)
//   W = (I + L)^-1 (beta 2^G k),   U = (I + L)^-1 (beta v)
//   D = U - W S,  O_t = (q_t 2^G_t) S + sum_{s<=t} A[t][s] D_s,
//   S <- diag(2^G_last) S + (k 2^(G_last - G))^T D
// with S the [dk][dv] state at the chunk start (row = key channel) and G in log2 units.
//
// Every product runs on v_mfma_f32_16x16x32_bf16 with both fp32 operands split into two
// BF16 terms, x = hi + lo (hi = bf16(x), lo = bf16(x - hi)), and three products
// hi*hi + hi*lo + lo*hi accumulated in fp32: ~16 significant bits per product, the fp32
// range, no overflow.
//
// Pairwise decays as matrix products: for the rows t of 16-row block I and any s <= t,
//   2^(G_t - G_s) = 2^(G_t - R_I) 2^(R_I - G_s),   R_I = G at the last row of block I-1
// (0 for I = 0).  For s in an earlier block both factors are <= 1.  For s inside block I
// the second factor is >= 1 and at most 2^rho_I, rho_I = max_i (R_I[i] - G_last-of-I[i]);
// when rho_I > 64 the diagonal 16x16 block is computed pairwise instead, so no factor
// ever exceeds 2^64.
//
// MFMA operand layout (16x16x32): lane l holds row (l % 16) of A and column (l % 16) of B,
// 8 consecutive k from 8 (l / 16); the accumulator of lane l holds rows 4 (l / 16) + r,
// r = 0..3, column l % 16.  Products whose k dimension comes out of an accumulator use the
// permuted k order  k(p, q, e) = 32 p + 4 q + e (e < 4),  32 p + 16 + 4 q + e - 4 (e >= 4),
// q = l / 16: then the 8 k values of lane l are accumulator entries 0..3 of row tiles 2p
// and 2p+1 in the same lane, and a GEMM result feeds the next GEMM without leaving the
// registers.  The preparation kernel writes W, q 2^G, (k 2^(G_last - G))^T and A in that
// order (W negated), U in accumulator order, so the scan reads each fragment with one
// 16-byte load per lane.
#include "kda_device.h"
#include "kda_internal.h"
#include "mfma_split.h"

namespace kda {
namespace {

using namespace mfma;

constexpr int CS = kChunk;             // tokens per chunk
constexpr int NB = CS / 16;            // 16-row blocks per chunk
constexpr float kFactorMax = 64.0f;    // largest log2 factor of the factored diagonal blocks
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Hardware-approximate special functions (v_exp_f32, v_log_f32, v_rcp_f32, ~1 ulp each):
// this path's products carry ~16 significant bits, so the precise library forms buy
// nothing here and cost ~5x the instructions.
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float fsigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + fexp(-z)); }
__device__ __forceinline__ float fsilu(float y) { return y * fsigmoid(y); }
__device__ __forceinline__ float fsoftplus(float z) {
  return fmaxf(z, 0.0f) + __builtin_amdgcn_logf(1.0f + fexp(-fabsf(z))) * kLn2;
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS carve-up of the preparation kernel (floats).
template <int DK>
struct PrepLds {
  static constexpr int RS = DK + 4;    // row stride of the q, k and G tiles [CS][RS]
  static constexpr int AS = CS + 4;    // row stride of A, L, T [CS][AS]
  static constexpr int Q = 0;
  static constexpr int A = Q + CS * RS;
  static constexpr int K = A + CS * AS;
  static constexpr int G = K + CS * RS;
  static constexpr int L = G + CS * RS;
  static constexpr int T = L + CS * AS;
  static constexpr int BETA = T + CS * AS;
  static constexpr int FLAG = BETA + CS;
  static constexpr int INV = FLAG + NB;   // inverse L2 norms of the q rows, then of the k rows
  static constexpr int TOTAL = INV + 2 * CS;
  static constexpr int FL = L;         // f_lr rows [CS][rank + 4] over L and T, before either
  static constexpr int FL_FLOATS = 2 * CS * AS;
  static_assert(TOTAL * 4 <= 160 * 1024, "LDS");
};

// Barrier for LDS traffic only: global loads stay in flight across it (the compiler waits
// for them where their values are used).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// ---------------------------------------------------------------------------------------
// Preparation: one block of 8 waves per (chunk, head, sequence), two per SIMD (the phases
// are chains of dependent steps, which a second wave on the SIMD overlaps); RF = rank of the forget
// gate's low-rank projection.
// ---------------------------------------------------------------------------------------
template <int DK, int RF>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void chunk_prep_kernel(const PrefillParams P) {
  using Lds = PrepLds<DK>;
  constexpr int RS = Lds::RS, AS = Lds::AS, KS = DK / 32;
  constexpr int FS = RF + 4;           // row stride of the staged f_lr rows
  constexpr int NW = 8, NT = 64 * NW;  // waves and threads of the block
  constexpr int NCT = DK / 16;         // 16-channel tiles (gate GEMM; value tiles of U)
  constexpr int NTW = (NCT + NW - 1) / NW;   // of them per wave: tile wave + NW n
  static_assert(CS * FS <= Lds::FL_FLOATS, "f_lr staging");
  __shared__ __attribute__((aligned(16))) float sm[Lds::TOTAL];
  float* sQ = sm + Lds::Q;
  float* sA = sm + Lds::A;
  float* sK = sm + Lds::K;
  float* sG = sm + Lds::G;
  float* sL = sm + Lds::L;
  float* sT = sm + Lds::T;
  float* sBeta = sm + Lds::BETA;
  float* sFlag = sm + Lds::FLAG;
  float* sInv = sm + Lds::INV;
  float* sFL = sm + Lds::FL;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, r16 = lane & 15;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = P.L;
  const int t0 = c * CS, nt = min(CS, L - t0);
  const size_t bh = (size_t)b * P.H + h;
  const size_t chunk = bh * P.nch + c;
  u32x4_t* Wf = static_cast<u32x4_t*>(P.Wf) + chunk * (4 * KS * 2 * 64);
  u32x4_t* Qf = static_cast<u32x4_t*>(P.Qf) + chunk * (4 * KS * 2 * 64);
  u32x4_t* Kf = static_cast<u32x4_t*>(P.Kf) + chunk * ((DK / 16) * 2 * 2 * 64);
  u32x4_t* Af = static_cast<u32x4_t*>(P.Af) + chunk * (4 * 2 * 2 * 64);
  f32x4_t* Uf = reinterpret_cast<f32x4_t*>(P.Uf) + chunk * ((DK / 16) * 4 * 64);

  const size_t row0 = (size_t)b * L + t0;         // first token row of the chunk
  // conv input of channel ch at chunk row tau (>= -3): the projections, or before the
  // sequence start the carried window; rows past the end read the last row
  auto conv_src = [&](int tau, int ch) -> const float* {
    const int tc = min(tau, nt - 1);
    return t0 + tc >= 0 ? P.P + (size_t)((int64_t)row0 + tc) * P.proj_stride + ch
                        : P.win + ((size_t)b * 3 + 3 + t0 + tc) * P.C + ch;
  };

  // ---- f_lr rows (staged in LDS for the gate GEMM) and this wave's F_b fragments, issued
  //      ahead of the conv loads ----
  constexpr int NFL = CS * RF / 4 / NT;
  static_assert(CS * RF / 4 % NT == 0, "f_lr rows");
  f32x4_t fl[NFL];
#pragma unroll
  for (int u = 0; u < NFL; ++u) {
    const int e = tid + NT * u;
    const int t = min(e / (RF / 4), nt - 1), c4 = e % (RF / 4);
    fl[u] = *reinterpret_cast<const f32x4_t*>(P.P + (row0 + t) * P.proj_stride + P.C + 4 * c4);
  }
  u32x4_t fbf[NTW][RF / 32];
#pragma unroll
  for (int n = 0; n < NTW; ++n)
#pragma unroll
    for (int ks = 0; ks < RF / 32; ++ks) {
      const int i = 16 * min(wave + NW * n, NCT - 1) + r16;   // past the head: a copy, unused
      // (the scalar gate has one F_b row per head: every channel of the head reads it)
      const size_t frow = P.gate == kGateScalar ? (size_t)h : (size_t)h * DK + i;
      fbf[n][ks] = *reinterpret_cast<const u32x4_t*>(P.Fb + frow * RF + 32 * ks + 8 * q4);
    }
  // ---- causal conv + SiLU of the chunk's q and k channels: an item is 4 channels x 8 rows
  //      (11 input rows); rows past the sequence end are zero ----
  {
    constexpr int NG = DK / 4;
    constexpr int ITEMS = 2 * 8 * NG;
    constexpr int NIT = (ITEMS + NT - 1) / NT;
    static_assert(ITEMS % NT == 0 || ITEMS < NT, "conv items");
    // all input rows and weights first (one round trip), then the conv of each item
    f32x4_t xin[NIT][11], w[NIT][4];
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
      const int it = min(tid + NT * u, ITEMS - 1);   // past the items: a copy of the last
      const int c4 = it % NG, rg = (it / NG) % 8, mat = it / (8 * NG);
      const int ch = mat * P.H * DK + h * DK + 4 * c4;
#pragma unroll
      for (int k = 0; k < 11; ++k) xin[u][k] = *reinterpret_cast<const f32x4_t*>(conv_src(8 * rg - 3 + k, ch));
#pragma unroll
      for (int e = 0; e < 4; ++e) w[u][e] = *reinterpret_cast<const f32x4_t*>(P.conv_w + (size_t)(ch + e) * 4);
    }
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
      const int it = tid + NT * u;
      if (it >= ITEMS) continue;
      const int c4 = it % NG, rg = (it / NG) % 8, mat = it / (8 * NG);
      float* dst = (mat ? sK : sQ) + 4 * c4;
#pragma unroll
      for (int o = 0; o < 8; ++o) {
        const int t = 8 * rg + o;
        f32x4_t y;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          y[e] = fsilu(w[u][e][0] * xin[u][o][e] + w[u][e][1] * xin[u][o + 1][e] +
                        w[u][e][2] * xin[u][o + 2][e] + w[u][e][3] * xin[u][o + 3][e]);
        *reinterpret_cast<f32x4_t*>(dst + t * RS) = t < nt ? y : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    if (tid < CS)
      sBeta[tid] = tid < nt ? fsigmoid(P.P[(row0 + tid) * P.proj_stride + P.C + P.rank_f + P.rank_g + h])
                            : 0.0f;
    if (tid < NB) sFlag[tid] = 0.0f;
  }
#pragma unroll
  for (int u = 0; u < NFL; ++u) {
    const int e = tid + NT * u;
    *reinterpret_cast<f32x4_t*>(sFL + (e / (RF / 4)) * FS + 4 * (e % (RF / 4))) = fl[u];
  }
  lds_barrier();
  // ---- forget gate: f = F_b f_lr on the matrix cores (f_lr fp32 split, F_b exact BF16),
  //      then the per-channel log2 decay: -exp(a_log) softplus(f + dt_bias) log2(e) (KDA,
  //      and the scalar gate with one f per head), lb sigmoid(-(f + dt_bias) a) log2(e)
  //      (the lower-bounded gate, a = a_log as given) ----
  {
    f32x4_t acc[4][NTW];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int n = 0; n < NTW; ++n) acc[mt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < RF / 32; ++ks) {
      Frag fa[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        float x[8];
        lds_load8(sFL + (16 * mt + r16) * FS + 32 * ks + 8 * q4, x);
        fa[mt] = split8(x);
      }
#pragma unroll
      for (int n = 0; n < NTW; ++n)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][n] = mma2(fa[mt], fbf[n][ks], acc[mt][n]);
    }
    const bool safe = P.gate == kGateSafe;
    const float ea = safe ? P.a_log[h] : fexp(P.a_log[h]);
#pragma unroll
    for (int n = 0; n < NTW; ++n) {
      if (wave + NW * n >= NCT) continue;
      const int i = 16 * (wave + NW * n) + r16;
      const float bias = P.dt_bias[P.gate == kGateScalar ? h : h * DK + i];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * mt + 4 * q4 + r;
          const float z = acc[mt][n][r] + bias;
          const float lg = safe ? P.gate_lb * fsigmoid(-z * ea) : -ea * fsoftplus(z);
          sG[t * RS + i] = t < nt ? lg * kLog2e : 0.0f;
        }
    }
  }
  // ---- inverse L2 norms of the q and k rows (q also takes the 1/sqrt(d_k) scale) ----
  if (tid < 2 * CS) {
    const int row = tid & (CS - 1), mat = tid / CS;
    const float* src = (mat ? sK : sQ) + row * RS;
    float a = 0.0f;
#pragma unroll 8
    for (int i = 0; i < DK; i += 4) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(src + i);
      a += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    sInv[tid] = (1.0f / sqrtf(a + P.l2_eps)) * (mat ? 1.0f : P.q_scale);
  }
  lds_barrier();

  // ---- normalised q and k rows; inclusive prefix sums of the log2-decays per channel and
  //      the decay range of each 16-row block ----
#pragma unroll
  for (int u = 0; u < 2 * CS * DK / 4 / NT; ++u) {
    const int e = tid + NT * u;
    const int c4 = e % (DK / 4), row = (e / (DK / 4)) % CS, mat = e / (CS * DK / 4);
    f32x4_t* v = reinterpret_cast<f32x4_t*>((mat ? sK : sQ) + row * RS + 4 * c4);
    *v = *v * sInv[mat * CS + row];
  }
  if (tid < DK) {
    float a = 0.0f, prev = 0.0f;
#pragma unroll
    for (int I = 0; I < NB; ++I) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        a += sG[(16 * I + u) * RS + tid];
        sG[(16 * I + u) * RS + tid] = a;
      }
      if (prev - a > kFactorMax) sFlag[I] = 1.0f;
      prev = a;
    }
    P.dec[chunk * DK + tid] = ex2(a);
  }
  lds_barrier();

  // ---- q 2^G in operand order (row tile wave & 3, key steps of half wave >> 2) ----
  {
    const int t = 16 * (wave & 3) + r16;
#pragma unroll
    for (int pp = 0; pp < KS / 2; ++pp) {
      const int p = (wave >> 2) * (KS / 2) + pp;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 32 * p + (e < 4 ? 4 * q4 + e : 16 + 4 * q4 + e - 4);
        x[e] = sQ[t * RS + i] * ex2(sG[t * RS + i]);
      }
      store_frag(Qf, (wave & 3) * KS + p, lane, split8(x));
    }
  }

  // ---- A and L together as transposed products, for row block I and key blocks
  //      J in [j0, j1]:  X^T[s][t] = sum_i (k_s 2^(R_I - G_s))[i] (x_t 2^(G_t - R_I))[i],
  //      x = q for A and k for L; the two share every decay factor.  Waves 0-5: (I 3,
  //      J 0-1), (I 3, J 2-3), (I 2, J 0-1), (I 2, J 2), (I 1, J 0-1), (I 0, J 0).  The wave
  //      that ends a row block at its diagonal also writes the zero blocks above it ----
  if (wave < 6) {
    {
      const int I = wave < 2 ? 3 : (wave < 4 ? 2 : 5 - wave);
      const int j0 = (wave == 1 || wave == 3) ? 2 : 0;
      const int j1 = (wave == 0 || wave == 2 || wave == 4) ? 1 : I;
      const bool fac = sFlag[I] == 0.0f;                  // factored diagonal block
      const int t = 16 * I + r16;
      f32x4_t accA[3], accL[3];
#pragma unroll
      for (int n = 0; n < 3; ++n) { accA[n] = f32x4_t{0.f, 0.f, 0.f, 0.f}; accL[n] = accA[n]; }
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int c0 = 32 * kk + 8 * q4;
        float xq[8], xk[8], g[8], rr[8];
        lds_load8(sQ + t * RS + c0, xq);
        lds_load8(sK + t * RS + c0, xk);
        lds_load8(sG + t * RS + c0, g);
        if (I > 0) {
          lds_load8(sG + (16 * I - 1) * RS + c0, rr);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) rr[e] = 0.0f;
        }
        float bq[8], bk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = ex2(g[e] - rr[e]);
          bq[e] = xq[e] * f;
          bk[e] = xk[e] * f;
        }
        const Frag fq = split8(bq), fk = split8(bk);
#pragma unroll
        for (int n = 0; n < 3; ++n) {
          const int J = j0 + n;
          if (J > j1 || (J == I && !fac)) continue;
          const int s = 16 * J + r16;
          float kv[8], gs[8], av[8];
          lds_load8(sK + s * RS + c0, kv);
          lds_load8(sG + s * RS + c0, gs);
#pragma unroll
          for (int e = 0; e < 8; ++e) av[e] = kv[e] * ex2(rr[e] - gs[e]);
          const Frag fa = split8(av);
          accA[n] = mma3(fa, fq, accA[n]);
          accL[n] = mma3(fa, fk, accL[n]);
        }
      }
      // acc[n], lane: X[t][s] for s = 16 (j0 + n) + 4 q4 + r
      const float bt = sBeta[t];
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        const int J = j0 + n;
        if (J > j1) continue;
        const bool live = J < I || fac;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 16 * J + 4 * q4 + r;
          sA[t * AS + s] = live && s <= t ? accA[n][r] : 0.0f;
          sL[t * AS + s] = live && s < t ? bt * accL[n][r] : 0.0f;
        }
      }
      if (j1 == I) {
        for (int s = 16 * (I + 1) + 4 * q4; s < CS; s += 16)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sA[t * AS + s + r] = 0.0f;
            sL[t * AS + s + r] = 0.0f;
          }
      }
    }
  }
  lds_barrier();

  // ---- diagonal blocks whose decay range is too wide to factor: pairwise ----
#pragma unroll 1
  for (int I = 0; I < NB; ++I) {
    if (sFlag[I] == 0.0f) continue;
    const int t = 16 * I + ((tid >> 4) & 15), s = 16 * I + (tid & 15);
    if (tid < 256 && s <= t) {
      float aa = 0.0f, al = 0.0f;
      for (int i = 0; i < DK; ++i) {
        const float ks = sK[s * RS + i] * ex2(sG[t * RS + i] - sG[s * RS + i]);
        aa += sQ[t * RS + i] * ks;
        al += sK[t * RS + i] * ks;
      }
      sA[t * AS + s] = aa;
      sL[t * AS + s] = s < t ? sBeta[t] * al : 0.0f;
    }
  }
  lds_barrier();

  // ---- conv inputs of U's right-hand side beta silu(conv(v)): for value tile
  //      nj = wave + 8 n and token step kk, lane (r16, q4) needs channel 16 nj + r16 at
  //      tokens 32 kk + 8 q4 .. + 7, i.e. 11 input rows; issued here, used after the inverse ----
  float vin[NTW][2][11];
  f32x4_t vw[NTW];
  {
    const int chv = 2 * P.H * DK + h * DK;
#pragma unroll
    for (int n = 0; n < NTW; ++n) {
      const int ch = chv + 16 * min(wave + NW * n, NCT - 1) + r16;   // past the head: unused
      vw[n] = *reinterpret_cast<const f32x4_t*>(P.conv_w + (size_t)ch * 4);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int k = 0; k < 11; ++k) vin[n][kk][k] = *conv_src(32 * kk + 8 * q4 - 3 + k, ch);
    }
  }
  // ---- A in operand order (row tile wave & 3, key step wave >> 2) ----
  {
    const int t = 16 * (wave & 3) + r16;
    {
      const int p = wave >> 2;
      float x[8];
      const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(sA + t * AS + 32 * p + 4 * q4);
      const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(sA + t * AS + 32 * p + 16 + 4 * q4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { x[e] = a0[e]; x[4 + e] = a1[e]; }
      store_frag(Af, (wave & 3) * 2 + p, lane, split8(x));
    }
  }
  // ---- diagonal blocks of T = (I + L)^-1 (forward substitution per column); zeros above ----
  if (tid < 64) {
    const int I = tid >> 4, j = tid & 15;
    const float* Lr = sL + (16 * I) * AS + 16 * I;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float a = r == j ? 1.0f : 0.0f;
#pragma unroll
      for (int u = 0; u < r; ++u) a -= Lr[r * AS + u] * x[u];
      x[r] = a;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sT[(16 * I + r) * AS + 16 * I + j] = x[r];
  } else {
    for (int e = tid - 64; e < 6 * 256; e += NT - 64) {
      const int tile = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      const int I = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
      const int J = tile < 3 ? 1 + tile : (tile < 5 ? tile - 1 : 3);
      sT[(16 * I + r) * AS + 16 * J + cc] = 0.0f;
    }
  }
  // ---- (k 2^(G_last - G))^T in operand order ----
  {
    const float* gl = sG + (CS - 1) * RS;
    for (int f = wave; f < (DK / 16) * 2; f += NW) {
      const int mt = f >> 1, p = f & 1;
      const int i = 16 * mt + r16;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = 32 * p + (e < 4 ? 4 * q4 + e : 16 + 4 * q4 + e - 4);
        x[e] = sK[t * RS + i] * ex2(gl[i] - sG[t * RS + i]);
      }
      store_frag(Kf, f, lane, split8(x));
    }
  }
  lds_barrier();

  // ---- off-diagonal blocks of T, one block diagonal at a time, on the matrix cores:
  //      T_IJ = -T_II sum_{K=J}^{I-1} L_IK T_KJ, wave J takes block (J + d, J); the first
  //      product's accumulator is the second product's B operand as it stands ----
#pragma unroll 1
  for (int d = 1; d < NB; ++d) {
    if (wave < NB - d) {
      const int J = wave, I = J + d;
      f32x4_t m = {0.f, 0.f, 0.f, 0.f};
      for (int K = J; K < I; ++K) {
        const f32x4_t la = *reinterpret_cast<const f32x4_t*>(sL + (16 * I + r16) * AS + 16 * K + 4 * q4);
        f32x4_t tb;
#pragma unroll
        for (int e = 0; e < 4; ++e) tb[e] = sT[(16 * K + 4 * q4 + e) * AS + 16 * J + r16];
        m = mma3_16(split4(la), split4(tb), m);
      }
      const f32x4_t ta = *reinterpret_cast<const f32x4_t*>(sT + (16 * I + r16) * AS + 16 * I + 4 * q4);
      const f32x4_t t = mma3_16(split4(ta), split4(m), f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) sT[(16 * I + 4 * q4 + r) * AS + 16 * J + r16] = -t[r];
    }
    lds_barrier();
  }

  // ---- T row fragments (t tile nt, s step kk; T is zero above the diagonal) ----
  Frag tf[NB][2];
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (kk > n / 2) continue;
      float x[8];
      lds_load8(sT + (16 * n + r16) * AS + 32 * kk + 8 * q4, x);
      tf[n][kk] = split8(x);
    }
  // ---- W^T = (beta 2^G k)^T T^T: wave w takes key tiles 2 kp, 2 kp + 1 (kp = w % KS) for
  //      the token tiles n with n % GS = w / KS (interleaved, so that with T lower
  //      triangular every wave runs the same products): -W in operand order ----
  {
    constexpr int GS = NW / KS, NPW = NB / GS;
    static_assert(NW % KS == 0 && NB % GS == 0, "W split");
    const int kp = wave % KS, g0 = wave / KS;
    f32x4_t acc[2][NPW];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int q = 0; q < NPW; ++q) acc[m][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int i = 16 * (2 * kp + m) + r16;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int s = 32 * kk + 8 * q4 + e;
          x[e] = sBeta[s] * sK[s * RS + i] * ex2(sG[s * RS + i]);
        }
        const Frag fa = split8(x);
#pragma unroll
        for (int n = 0; n < NB; ++n)
          if (n % GS == g0 && kk <= n / 2) acc[m][n / GS] = mma3(fa, tf[n][kk], acc[m][n / GS]);
      }
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      if (n % GS != g0) continue;
      float x[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) { x[r] = -acc[0][n / GS][r]; x[4 + r] = -acc[1][n / GS][r]; }
      store_frag(Wf, n * KS + kp, lane, split8(x));
    }
  }
  // ---- U = T (beta v) for value tiles w + 8 n, in accumulator order ----
#pragma unroll
  for (int n = 0; n < NTW; ++n) {
    const int nj = wave + NW * n;
    if (nj >= NCT) continue;
    Frag fv[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float* xi = vin[n][kk] + e;
        x[e] = sBeta[32 * kk + 8 * q4 + e] *
               fsilu(vw[n][0] * xi[0] + vw[n][1] * xi[1] + vw[n][2] * xi[2] + vw[n][3] * xi[3]);
      }
      fv[kk] = split8(x);
    }
#pragma unroll
    for (int mt = 0; mt < NB; ++mt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        if (kk <= mt / 2) acc = mma3(tf[mt][kk], fv[kk], acc);
      Uf[(nj * 4 + mt) * 64 + lane] = acc;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Scan over the chunks of one (sequence, head): a block of four waves; waves 0 and 1 own 32
// value columns (16 each) and keep those state columns in MFMA accumulators for the whole
// sequence, waves 2 and 3 only stream each chunk's operands into LDS.  A chunk's operands
// come in four segments, shared by both computing waves:
//   0: -W              D = -W S
//   1: q 2^G           O = (q 2^G) S
//   2: A | U | dec     D += U, O += A D (then stored), S <- diag(dec) S
//   3: Kt^T            S += Kt^T D
// The segments go round five LDS slots (the whole LDS) by direct global->LDS loads issued
// four segments ahead of their use: the scan is bound by these loads (~120 KB per block and
// chunk), not by its products.  Only the loading waves issue loads, so a wait for "at most
// the loads of the three later segments outstanding" (vector memory operations retire in
// order) means the segment about to be read has landed, and the computing waves' output
// stores count against no such wait.  One barrier per segment hands the segment to the
// computing waves and the slot they have finished with back to the loaders.
// ---------------------------------------------------------------------------------------
template <int D>
struct ScanSeg {
  static constexpr int KS = D / 32, MTI = D / 16, NJ = D / 16;
  static constexpr int FW = 4 * KS * 2 * 64;        // 16-byte entries of -W (and of q 2^G)
  static constexpr int FK = MTI * 2 * 2 * 64;       // Kt^T
  static constexpr int FA = 4 * 2 * 2 * 64;         // A
  static constexpr int FU = 2 * 4 * 64;             // U, the block's two value tiles
  static constexpr int FD = D / 4;                  // dec
  static constexpr int S2 = FA + FU + FD;
  static constexpr int SLOT = FW > FK ? (FW > S2 ? FW : S2) : (FK > S2 ? FK : S2);
  static constexpr int NSLOT = 5;
  // loads per loading wave (= per lane) of each segment
  static constexpr int NLD[4] = {FW / 128, FW / 128, FA / 128 + FU / 128 + 1, FK / 128};
  static_assert(FW % 128 == 0 && FK % 128 == 0 && FA % 128 == 0 && FU % 128 == 0 && FD <= 128,
                "segment pieces are whole rounds of 128 loads");
  static_assert(NSLOT * SLOT * 16 <= 160 * 1024, "LDS");
  static_assert(NLD[0] + NLD[1] + NLD[2] + NLD[3] - 1 < 64, "vmcnt");
};

struct ScanSrc {
  const u32x4_t *W, *Q, *K, *A, *U, *D;
};

// One 16-byte load per active lane straight into LDS: the lanes of the wave fill
// consecutive entries from lds_wave_base.  Issued as inline assembly so that the compiler
// does not track it: the explicit waits below carry the ordering (nothing else in these
// kernels uses m0).
__device__ __forceinline__ void dma16(const u32x4_t* src, u32x4_t* lds_wave_base) {
  const unsigned lds = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "m0");
}

// Segment SEG of chunk c into slot, by the two loading waves (lt = thread 0..127 among
// them, lw = loading wave 0 or 1).
template <int D, int SEG>
__device__ __forceinline__ void scan_issue(const ScanSrc& g, size_t c, u32x4_t* slot, int lt,
                                           int lane, int lw) {
  using Sg = ScanSeg<D>;
  if constexpr (SEG == 0 || SEG == 1) {
    const u32x4_t* src = (SEG == 0 ? g.W : g.Q) + c * Sg::FW + lt;
#pragma unroll
    for (int u = 0; u < Sg::FW / 128; ++u) dma16(src + 128 * u, slot + 128 * u + 64 * lw);
  } else if constexpr (SEG == 2) {
    const u32x4_t* sa = g.A + c * Sg::FA + lt;
#pragma unroll
    for (int u = 0; u < Sg::FA / 128; ++u) dma16(sa + 128 * u, slot + 128 * u + 64 * lw);
    const u32x4_t* su = g.U + c * (Sg::NJ * 4 * 64) + lt;
#pragma unroll
    for (int u = 0; u < Sg::FU / 128; ++u) dma16(su + 128 * u, slot + Sg::FA + 128 * u + 64 * lw);
    if (lane < Sg::FD / 2)
      dma16(g.D + c * Sg::FD + lw * (Sg::FD / 2) + lane, slot + Sg::FA + Sg::FU + lw * (Sg::FD / 2));
  } else {
    const u32x4_t* src = g.K + c * Sg::FK + lt;
#pragma unroll
    for (int u = 0; u < Sg::FK / 128; ++u) dma16(src + 128 * u, slot + 128 * u + 64 * lw);
  }
}

// wait until at most N vector memory operations of this wave are outstanding and all of
// its LDS operations are done
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" : : : "memory"); }
// the computing waves' barrier: their LDS reads of the segment just used have returned
__device__ __forceinline__ void lds_done_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// acc[mt] += sum_p F(mt, p) B[p] for the four token tiles mt, fragment mt * KS + p of the
// slot; the fragments of step p + 1 are read while step p runs on the matrix cores.
template <int KS>
__device__ __forceinline__ void row_tiles_times(const u32x4_t* slot, const Frag (&B)[KS],
                                                f32x4_t (&acc)[4], int lane) {
  Frag cur[4], nxt[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) cur[mt] = load_frag(slot, mt * KS, lane);
#pragma unroll
  for (int p = 0; p < KS; ++p) {
    if (p + 1 < KS) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) nxt[mt] = load_frag(slot, mt * KS + p + 1, lane);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = mma3(cur[mt], B[p], acc[mt]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) cur[mt] = nxt[mt];
  }
}

// S[mt] += sum_p F(mt, p) B[p] for the MTI key tiles, fragment mt * 2 + p of the slot, two
// key tiles per step, the next step's fragments read ahead.
template <int MTI>
__device__ __forceinline__ void key_tiles_times(const u32x4_t* slot, const Frag (&B)[2],
                                                f32x4_t (&S)[MTI], int lane) {
  Frag cur[4], nxt[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) cur[i] = load_frag(slot, i, lane);
#pragma unroll
  for (int m2 = 0; m2 < MTI / 2; ++m2) {
    if (m2 + 1 < MTI / 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) nxt[i] = load_frag(slot, 4 * (m2 + 1) + i, lane);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) S[2 * m2 + (i >> 1)] = mma3(cur[i], B[i & 1], S[2 * m2 + (i >> 1)]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
  }
}

template <int D>
__global__ __launch_bounds__(256) void chunk_scan_kernel(const PrefillParams P) {
  using Sg = ScanSeg<D>;
  constexpr int KS = Sg::KS, MTI = Sg::MTI, NJ2 = Sg::NJ / 2;
  constexpr int N0 = Sg::NLD[0], N1 = Sg::NLD[1], N2 = Sg::NLD[2], N3 = Sg::NLD[3];
  __shared__ u32x4_t slots[Sg::NSLOT * Sg::SLOT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, r16 = lane & 15;
  // the blocks of one (sequence, head) on one XCD (blocks go round-robin over 8)
  const int ng = P.B * P.H, id = blockIdx.x;
  int g, nj2;
  if ((ng & 7) == 0) {
    const int sl = id >> 3;
    nj2 = sl % NJ2;
    g = (sl / NJ2) * 8 + (id & 7);
  } else {
    g = id / NJ2;
    nj2 = id % NJ2;
  }
  const int b = g / P.H, h = g - b * P.H;
  const int nch = P.nch;
  const size_t gc = (size_t)g * nch;
  // global segment gs = 4 c + s sits in slot gs % 5
  auto slot_of = [&](int gs) { return slots + (gs % Sg::NSLOT) * Sg::SLOT; };

  if (wave >= 2) {
    // ---- loading waves: segment 4 c + s + 4 (chunk c + 1, segment s) is issued into the
    // slot of segment 4 c + s - 1 once the barrier before segment 4 c + s has passed ----
    const int lt = tid - 128, lw = wave - 2;
    ScanSrc src;
    src.W = static_cast<const u32x4_t*>(P.Wf) + gc * Sg::FW;
    src.Q = static_cast<const u32x4_t*>(P.Qf) + gc * Sg::FW;
    src.K = static_cast<const u32x4_t*>(P.Kf) + gc * Sg::FK;
    src.A = static_cast<const u32x4_t*>(P.Af) + gc * Sg::FA;
    src.U = reinterpret_cast<const u32x4_t*>(P.Uf) + gc * (Sg::NJ * 4 * 64) + nj2 * Sg::FU;
    src.D = reinterpret_cast<const u32x4_t*>(P.dec) + gc * Sg::FD;
    scan_issue<D, 0>(src, 0, slot_of(0), lt, lane, lw);
    scan_issue<D, 1>(src, 0, slot_of(1), lt, lane, lw);
    scan_issue<D, 2>(src, 0, slot_of(2), lt, lane, lw);
    scan_issue<D, 3>(src, 0, slot_of(3), lt, lane, lw);
#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
      const bool more = c + 1 < nch;
      const int g0 = 4 * c;
      // each wait leaves in flight only the loads of the segments issued after the one
      // about to be read (in the last chunk: those of its own later segments)
      wait_vm_lgkm0<N1 + N2 + N3>();
      block_barrier();
      if (more) scan_issue<D, 0>(src, c + 1, slot_of(g0 + 4), lt, lane, lw);
      if (more) wait_vm_lgkm0<N2 + N3 + N0>();
      else wait_vm_lgkm0<N2 + N3>();
      block_barrier();
      if (more) scan_issue<D, 1>(src, c + 1, slot_of(g0 + 5), lt, lane, lw);
      if (more) wait_vm_lgkm0<N3 + N0 + N1>();
      else wait_vm_lgkm0<N3>();
      block_barrier();
      if (more) scan_issue<D, 2>(src, c + 1, slot_of(g0 + 6), lt, lane, lw);
      if (more) wait_vm_lgkm0<N0 + N1 + N2>();
      else wait_vm_lgkm0<0>();
      block_barrier();
      if (more) scan_issue<D, 3>(src, c + 1, slot_of(g0 + 7), lt, lane, lw);
    }
    return;
  }

  // ---- computing waves ----
  const int j = 16 * (2 * nj2 + wave) + r16;
  float* Sgl = P.S + (size_t)g * D * D;
  f32x4_t S[MTI];
#pragma unroll
  for (int mt = 0; mt < MTI; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[mt][r] = Sgl[(size_t)(16 * mt + 4 * q4 + r) * D + j];

  const size_t orow = (size_t)P.H * D;
  f32x4_t Dm[4], Om[4];
  Frag sf[KS], df[2];
#pragma unroll 1
  for (int c = 0; c < nch; ++c) {
    const int g0 = 4 * c;
    const u32x4_t* slot0 = slot_of(g0);
    const u32x4_t* slot1 = slot_of(g0 + 1);
    const u32x4_t* slot2 = slot_of(g0 + 2);
    const u32x4_t* slot3 = slot_of(g0 + 3);
    // ---- segment 0: D = -W S (state columns as B operands, k = key channel permuted) ----
#pragma unroll
    for (int p = 0; p < KS; ++p) {
      float x[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) { x[r] = S[2 * p][r]; x[4 + r] = S[2 * p + 1][r]; }
      sf[p] = split8(x);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) Dm[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    lds_done_barrier();
    row_tiles_times<KS>(slot0, sf, Dm, lane);
    // ---- segment 1: O = (q 2^G) S ----
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) Om[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    lds_done_barrier();
    row_tiles_times<KS>(slot1, sf, Om, lane);
    // ---- segment 2: D += U; O += A D; S <- diag(dec) S ----
    lds_done_barrier();
    {
      const f32x4_t* sU = reinterpret_cast<const f32x4_t*>(slot2 + Sg::FA) + wave * 4 * 64;
      const f32x4_t* sD = reinterpret_cast<const f32x4_t*>(slot2 + Sg::FA + Sg::FU);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) Dm[mt] += sU[mt * 64 + lane];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float x[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) { x[r] = Dm[2 * p][r]; x[4 + r] = Dm[2 * p + 1][r]; }
        df[p] = split8(x);
      }
      {
        Frag fa[6];
#pragma unroll
        for (int i = 0; i < 6; ++i) fa[i] = load_frag(slot2, i < 2 ? 2 * i : i + 2, lane);
        // (mt, p) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1): fragment mt * 2 + p
        Om[0] = mma3(fa[0], df[0], Om[0]);
        Om[1] = mma3(fa[1], df[0], Om[1]);
        Om[2] = mma3(fa[2], df[0], Om[2]);
        Om[2] = mma3(fa[3], df[1], Om[2]);
        Om[3] = mma3(fa[4], df[0], Om[3]);
        Om[3] = mma3(fa[5], df[1], Om[3]);
      }
#pragma unroll
      for (int mt = 0; mt < MTI; ++mt) S[mt] = S[mt] * sD[4 * mt + q4];
    }
    {
      const int t0 = c * CS, nt = min(CS, P.L - t0);
      float* og = P.o + ((size_t)b * P.L + t0) * orow + (size_t)h * D + j;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * mt + 4 * q4 + r;
          if (t < nt) og[(size_t)t * orow] = Om[mt][r];
        }
    }
    // ---- segment 3: S += (k 2^(G_last - G))^T D ----
    lds_done_barrier();
    key_tiles_times<MTI>(slot3, df, S, lane);
  }
#pragma unroll
  for (int mt = 0; mt < MTI; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) Sgl[(size_t)(16 * mt + 4 * q4 + r) * D + j] = S[mt][r];
}

// ---------------------------------------------------------------------------------------
// Gated RMSNorm of the chunk's outputs, one block per (chunk, head, sequence), written as
// BF16 hi/lo planes for the output projection: the output gate sigmoid(G_b g_lr) on the matrix cores (g_lr fp32 split, G_b exact
// BF16), then per token the RMS over the head's d_v values, the norm weight and the gate.
// Wave w owns value tiles w * NTW .. w * NTW + NTW - 1, all four token tiles.
// ---------------------------------------------------------------------------------------
template <int D, int RG>
__global__ __launch_bounds__(256) void chunk_gnorm_kernel(const PrefillParams P) {
  constexpr int NTW = D / 64;                       // value tiles per wave
  __shared__ float part[4][CS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, r16 = lane & 15;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t0 = c * CS, nt = min(CS, P.L - t0);
  const size_t row0 = (size_t)b * P.L + t0;
  const int V = P.H * D;

  // gate pre-activations: acc[mt][n] = sum_r g_lr[t][r] G_b[h D + j][r]
  f32x4_t acc[4][NTW];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int n = 0; n < NTW; ++n) acc[mt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // every g_lr row and G_b fragment of all RG / 32 k-steps is requested before the first
  // product (one round trip a block; a k-step at a time took one each)
  constexpr int NKS = RG / 32;
  const float* glr = P.P + P.C + P.rank_f;
  f32x4_t ga[NKS][4][2];
  u32x4_t gb[NKS][NTW];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int t = min(16 * mt + r16, nt - 1);
      const float* src = glr + (row0 + t) * P.proj_stride + 32 * ks + 8 * q4;
      ga[ks][mt][0] = *reinterpret_cast<const f32x4_t*>(src);
      ga[ks][mt][1] = *reinterpret_cast<const f32x4_t*>(src + 4);
    }
#pragma unroll
    for (int n = 0; n < NTW; ++n) {
      const int j = 16 * (wave * NTW + n) + r16;
      gb[ks][n] = *reinterpret_cast<const u32x4_t*>(P.Gb + ((size_t)h * D + j) * RG + 32 * ks + 8 * q4);
    }
  }
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    Frag fa[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) { x[e] = ga[ks][mt][0][e]; x[4 + e] = ga[ks][mt][1][e]; }
      fa[mt] = split8(x);
    }
#pragma unroll
    for (int n = 0; n < NTW; ++n)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt][n] = mma2(fa[mt], gb[ks][n], acc[mt][n]);
  }
  // o in the accumulator layout; per-token sums of squares over the head
  float ov[4][NTW][4];
  float ss[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = min(16 * mt + 4 * q4 + r, nt - 1);
      float a = 0.0f;
#pragma unroll
      for (int n = 0; n < NTW; ++n) {
        const int j = 16 * (wave * NTW + n) + r16;
        ov[mt][n][r] = P.o[(row0 + t) * V + (size_t)h * D + j];
        a += ov[mt][n][r] * ov[mt][n][r];
      }
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) a += __shfl_xor(a, m, 64);
      ss[mt][r] = a;
    }
  if (r16 == 0) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[wave][16 * mt + 4 * q4 + r] = ss[mt][r];
  }
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * mt + 4 * q4 + r;
      if (t >= nt) continue;
      const float tot = part[0][t] + part[1][t] + part[2][t] + part[3][t];
      const float sc = 1.0f / sqrtf(tot / (float)D + P.norm_eps);
#pragma unroll
      for (int n = 0; n < NTW; ++n) {
        const int j = 16 * (wave * NTW + n) + r16;
        const float w = P.onw ? P.onw[j] : 1.0f;
        const float g = fsigmoid(acc[mt][n][r]);
        const float y = ov[mt][n][r] * sc * w * g;
        const __bf16 yh = (__bf16)y;
        const size_t at = (row0 + t) * V + (size_t)h * D + j;
        P.on_hi[at] = __builtin_bit_cast(uint16_t, yh);
        P.on_lo[at] = __builtin_bit_cast(uint16_t, (__bf16)(y - (float)yh));
      }
    }
}

// ---------------------------------------------------------------------------------------
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

}  // namespace

hipError_t launch_chunk_prep(const PrefillParams& p, hipStream_t s) {
  dim3 grid(p.nch, p.H, p.B);
  if (p.dk == 128 && p.rank_f == 128)
    chunk_prep_kernel<128, 128><<<grid, 512, 0, s>>>(p);
  else if (p.dk == 128 && p.rank_f == 64)
    chunk_prep_kernel<128, 64><<<grid, 512, 0, s>>>(p);
  else if (p.dk == 64 && p.rank_f == 128)
    chunk_prep_kernel<64, 128><<<grid, 512, 0, s>>>(p);
  else if (p.dk == 64 && p.rank_f == 64)
    chunk_prep_kernel<64, 64><<<grid, 512, 0, s>>>(p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_chunk_scan(const PrefillParams& p, hipStream_t s) {
  const int blocks = p.B * p.H * (p.dk / 32);
  if (p.dk == 128)
    chunk_scan_kernel<128><<<blocks, 256, 0, s>>>(p);
  else
    chunk_scan_kernel<64><<<blocks, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_chunk_gnorm(const PrefillParams& p, hipStream_t s) {
  dim3 grid(p.nch, p.H, p.B);
  if (p.rank_g != 64 && p.rank_g != 128) return hipErrorInvalidValue;
  if (p.dk == 128 && p.rank_g == 128)
    chunk_gnorm_kernel<128, 128><<<grid, 256, 0, s>>>(p);
  else if (p.dk == 128)
    chunk_gnorm_kernel<128, 64><<<grid, 256, 0, s>>>(p);
  else if (p.rank_g == 128)
    chunk_gnorm_kernel<64, 128><<<grid, 256, 0, s>>>(p);
  else
    chunk_gnorm_kernel<64, 64><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_prefill_window(const PrefillParams& p, hipStream_t s) {
  dim3 grid((p.C + 255) / 256, p.B);
  prefill_window_kernel<<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace kda

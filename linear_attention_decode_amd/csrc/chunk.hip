// Chunked delta rule on gfx950 matrix cores: the per-chunk WY/UT preparation and the
// sequential scan over chunks that carries the fp32 state.
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

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int CS = kChunk;             // tokens per chunk
constexpr int NB = CS / 16;            // 16-row blocks per chunk
constexpr float kFactorMax = 64.0f;    // largest log2 factor of the factored diagonal blocks

struct Frag {
  u32x4_t hi, lo;                      // 8 BF16 each
};

__device__ __forceinline__ unsigned pk_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// x = hi + lo, hi = bf16(x) (round to nearest even), lo = bf16(x - hi)
__device__ __forceinline__ Frag split8(const float (&x)[8]) {
  Frag f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const unsigned h = pk_bf16(x[2 * e], x[2 * e + 1]);
    f.hi[e] = h;
    f.lo[e] = pk_bf16(x[2 * e] - __builtin_bit_cast(float, h << 16),
                      x[2 * e + 1] - __builtin_bit_cast(float, h & 0xffff0000u));
  }
  return f;
}

// acc += a b over 32 k: lo*hi + hi*lo + hi*hi
__device__ __forceinline__ f32x4_t mma3(const Frag& a, const Frag& b, f32x4_t acc) {
  const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, a.hi), al = __builtin_bit_cast(bf16x8_t, a.lo);
  const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, b.hi), bl = __builtin_bit_cast(bf16x8_t, b.lo);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
  return acc;
}

// Fragment f of an operand array: [f][hi, lo][64 lanes] x 16 bytes.
__device__ __forceinline__ void store_frag(u32x4_t* base, int f, int lane, const Frag& v) {
  base[(2 * f) * 64 + lane] = v.hi;
  base[(2 * f + 1) * 64 + lane] = v.lo;
}
__device__ __forceinline__ Frag load_frag(const u32x4_t* base, int f, int lane) {
  return Frag{base[(2 * f) * 64 + lane], base[(2 * f + 1) * 64 + lane]};
}

__device__ __forceinline__ void lds_load8(const float* p, float (&x)[8]) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS carve-up of the preparation kernel (floats).
template <int DK>
struct PrepLds {
  static constexpr int RS = DK + 4;    // row stride of the q, k and G tiles [CS][RS]
  static constexpr int AS = CS + 4;    // row stride of A, L, T [CS][AS] and of beta v^T [DK][AS]
  static constexpr int Q = 0;
  static constexpr int A = Q + CS * RS;
  static constexpr int K = A + CS * AS;
  static constexpr int G = K + CS * RS;
  static constexpr int L = G + CS * RS;
  static constexpr int T = L + CS * AS;
  static constexpr int BETA = T + CS * AS;
  static constexpr int FLAG = BETA + CS;
  static constexpr int TOTAL = FLAG + NB;
  static constexpr int VT = Q;         // beta v^T, over q and A once both are dead
  static constexpr int M = VT + DK * AS;   // three 16x16 scratch tiles of the inverse
  static_assert(M + 3 * 256 <= K, "v^T and the scratch tiles overlap k");
  static_assert(TOTAL * 4 <= 160 * 1024, "LDS");
};

// ---------------------------------------------------------------------------------------
// Preparation: one block of 4 waves per (chunk, head, sequence).
// ---------------------------------------------------------------------------------------
template <int DK>
__global__ __launch_bounds__(256) void chunk_prep_kernel(const PrefillParams P) {
  using Lds = PrepLds<DK>;
  constexpr int RS = Lds::RS, AS = Lds::AS, KS = DK / 32;
  __shared__ __attribute__((aligned(16))) float sm[Lds::TOTAL];
  float* sQ = sm + Lds::Q;
  float* sA = sm + Lds::A;
  float* sK = sm + Lds::K;
  float* sG = sm + Lds::G;
  float* sL = sm + Lds::L;
  float* sT = sm + Lds::T;
  float* sBeta = sm + Lds::BETA;
  float* sFlag = sm + Lds::FLAG;
  float* sVT = sm + Lds::VT;
  float* sM = sm + Lds::M;

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

  // ---- q, k and log2-decay rows of the chunk (rows past the sequence end are zero) ----
  {
    const size_t g0 = (bh * L + t0) * DK;
    const f32x4_t* gq = reinterpret_cast<const f32x4_t*>(P.q + g0);
    const f32x4_t* gk = reinterpret_cast<const f32x4_t*>(P.k + g0);
    const f32x4_t* gg = reinterpret_cast<const f32x4_t*>(P.g2 + g0);
    for (int e = tid; e < CS * DK / 4; e += 256) {
      const int t = e / (DK / 4), c4 = (e % (DK / 4)) * 4;
      f32x4_t vq = {0.f, 0.f, 0.f, 0.f}, vk = vq, vg = vq;
      if (t < nt) { vq = gq[e]; vk = gk[e]; vg = gg[e]; }
      *reinterpret_cast<f32x4_t*>(sQ + t * RS + c4) = vq;
      *reinterpret_cast<f32x4_t*>(sK + t * RS + c4) = vk;
      *reinterpret_cast<f32x4_t*>(sG + t * RS + c4) = vg;
    }
    if (tid < CS) sBeta[tid] = tid < nt ? P.beta[bh * L + t0 + tid] : 0.0f;
    if (tid < NB) sFlag[tid] = 0.0f;
  }
  __syncthreads();

  // ---- inclusive prefix sums of the log2-decays per channel; decay range per block ----
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
  __syncthreads();

  // ---- q 2^G in operand order (row tile = wave) ----
  {
    const int t = 16 * wave + r16;
#pragma unroll
    for (int p = 0; p < KS; ++p) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 32 * p + (e < 4 ? 4 * q4 + e : 16 + 4 * q4 + e - 4);
        x[e] = sQ[t * RS + i] * ex2(sG[t * RS + i]);
      }
      store_frag(Qf, wave * KS + p, lane, split8(x));
    }
  }

  // ---- A (waves 0, 1) and L (waves 2, 3) as transposed products, row blocks {0,3} / {1,2}:
  //      X^T[s][t] = sum_i (k_s 2^(R_I - G_s))[i] (x_t 2^(G_t - R_I))[i] ----
  {
    const bool isA = wave < 2;
    const float* sX = isA ? sQ : sK;
    float* sOut = isA ? sA : sL;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      const int I = (wave & 1) ? 1 + pass : 3 * pass;
      const bool fac = sFlag[I] == 0.0f;                  // factored diagonal block
      const int t = 16 * I + r16;
      f32x4_t acc[NB];
#pragma unroll
      for (int J = 0; J < NB; ++J) acc[J] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int c0 = 32 * kk + 8 * q4;
        float x[8], g[8], rr[8];
        lds_load8(sX + t * RS + c0, x);
        lds_load8(sG + t * RS + c0, g);
        if (I > 0) {
          lds_load8(sG + (16 * I - 1) * RS + c0, rr);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) rr[e] = 0.0f;
        }
        float bv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = x[e] * ex2(g[e] - rr[e]);
        const Frag fb = split8(bv);
#pragma unroll
        for (int J = 0; J < NB; ++J) {
          if (J > I || (J == I && !fac)) continue;
          const int s = 16 * J + r16;
          float kv[8], gs[8], av[8];
          lds_load8(sK + s * RS + c0, kv);
          lds_load8(sG + s * RS + c0, gs);
#pragma unroll
          for (int e = 0; e < 8; ++e) av[e] = kv[e] * ex2(rr[e] - gs[e]);
          acc[J] = mma3(split8(av), fb, acc[J]);
        }
      }
      // acc[J], lane: X[t][s] for s = 16 J + 4 q4 + r
      const float bt = sBeta[t];
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        const bool live = J < I || (J == I && fac);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 16 * J + 4 * q4 + r;
          const float v = live ? acc[J][r] : 0.0f;
          sOut[t * AS + s] = isA ? (s <= t ? v : 0.0f) : (s < t ? bt * v : 0.0f);
        }
      }
    }
  }
  __syncthreads();

  // ---- diagonal blocks whose decay range is too wide to factor: pairwise ----
#pragma unroll 1
  for (int I = 0; I < NB; ++I) {
    if (sFlag[I] == 0.0f) continue;
    const int t = 16 * I + (tid >> 4), s = 16 * I + (tid & 15);
    if (s <= t) {
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
  __syncthreads();

  // ---- A in operand order (row tile = wave) ----
  {
    const int t = 16 * wave + r16;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float x[8];
      const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(sA + t * AS + 32 * p + 4 * q4);
      const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(sA + t * AS + 32 * p + 16 + 4 * q4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { x[e] = a0[e]; x[4 + e] = a1[e]; }
      store_frag(Af, wave * 2 + p, lane, split8(x));
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
    for (int e = tid - 64; e < 6 * 256; e += 192) {
      const int tile = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      const int I = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
      const int J = tile < 3 ? 1 + tile : (tile < 5 ? tile - 1 : 3);
      sT[(16 * I + r) * AS + 16 * J + cc] = 0.0f;
    }
  }
  // ---- (k 2^(G_last - G))^T in operand order ----
  {
    const float* gl = sG + (CS - 1) * RS;
    for (int f = wave; f < (DK / 16) * 2; f += 4) {
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
  __syncthreads();

  // ---- beta v^T over the dead q and A tiles: lane = token, 4 value columns per load ----
  {
    const float* gv = P.v + (bh * L + t0) * DK;
    const int t = lane;
    const float bt = sBeta[t];
    for (int j4 = wave; j4 < DK / 4; j4 += 4) {
      f32x4_t v = {0.f, 0.f, 0.f, 0.f};
      if (t < nt) v = *reinterpret_cast<const f32x4_t*>(gv + (size_t)t * DK + 4 * j4);
#pragma unroll
      for (int u = 0; u < 4; ++u) sVT[(4 * j4 + u) * AS + t] = bt * v[u];
    }
  }
  // ---- off-diagonal blocks of T, one block diagonal at a time:
  //      T_IJ = -T_II sum_{K=J}^{I-1} L_IK T_KJ ----
#pragma unroll 1
  for (int d = 1; d < NB; ++d) {
    const int ntile = NB - d;
    for (int e = tid; e < ntile * 256; e += 256) {
      const int J = e >> 8, I = J + d, r = (e >> 4) & 15, cc = e & 15;
      float a = 0.0f;
      for (int K = J; K < I; ++K) {
        const float* Lr = sL + (16 * I + r) * AS + 16 * K;
        const float* Tc = sT + (16 * K) * AS + 16 * J + cc;
#pragma unroll
        for (int u = 0; u < 16; ++u) a += Lr[u] * Tc[u * AS];
      }
      sM[e] = a;
    }
    __syncthreads();
    for (int e = tid; e < ntile * 256; e += 256) {
      const int J = e >> 8, I = J + d, r = (e >> 4) & 15, cc = e & 15;
      const float* Tr = sT + (16 * I + r) * AS + 16 * I;
      const float* Mc = sM + (J << 8) + cc;
      float a = 0.0f;
      for (int u = 0; u <= r; ++u) a += Tr[u] * Mc[u * 16];
      sT[(16 * I + r) * AS + 16 * J + cc] = -a;
    }
    __syncthreads();
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
  // ---- W^T = (beta 2^G k)^T T^T for key tiles 2w, 2w+1: -W in operand order ----
  if (wave < KS) {
    f32x4_t acc[2][NB];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int i = 16 * (2 * wave + m) + r16;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int s = 32 * kk + 8 * q4 + e;
          x[e] = sBeta[s] * sK[s * RS + i] * ex2(sG[s * RS + i]);
        }
        const Frag fa = split8(x);
#pragma unroll
        for (int n = 0; n < NB; ++n)
          if (kk <= n / 2) acc[m][n] = mma3(fa, tf[n][kk], acc[m][n]);
      }
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      float x[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) { x[r] = -acc[0][n][r]; x[4 + r] = -acc[1][n][r]; }
      store_frag(Wf, n * KS + wave, lane, split8(x));
    }
  }
  // ---- U = T (beta v) for value tiles w, w + 4, in accumulator order ----
  for (int nj = wave; nj < DK / 16; nj += 4) {
    Frag fv[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float x[8];
      lds_load8(sVT + (16 * nj + r16) * AS + 32 * kk + 8 * q4, x);
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
// Scan over the chunks of one (sequence, head) for 16 value columns: one wave, the state
// columns in MFMA accumulators for the whole sequence.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void chunk_scan_kernel(const PrefillParams P) {
  constexpr int KS = D / 32, MTI = D / 16, NJ = D / 16;
  const int lane = threadIdx.x, q4 = lane >> 4, r16 = lane & 15;
  // the value tiles of one (sequence, head) on one XCD (blocks go round-robin over 8)
  const int ng = P.B * P.H, id = blockIdx.x;
  int g, nj;
  if ((ng & 7) == 0) {
    const int slot = id >> 3;
    nj = slot % NJ;
    g = (slot / NJ) * 8 + (id & 7);
  } else {
    g = id / NJ;
    nj = id % NJ;
  }
  const int b = g / P.H, h = g - b * P.H;
  const int j = 16 * nj + r16;
  float* Sg = P.S + (size_t)g * D * D;

  f32x4_t S[MTI];
#pragma unroll
  for (int mt = 0; mt < MTI; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[mt][r] = Sg[(size_t)(16 * mt + 4 * q4 + r) * D + j];

  const size_t orow = (size_t)P.H * D;
#pragma unroll 1
  for (int c = 0; c < P.nch; ++c) {
    const size_t chunk = (size_t)g * P.nch + c;
    const u32x4_t* Wf = static_cast<const u32x4_t*>(P.Wf) + chunk * (4 * KS * 2 * 64);
    const u32x4_t* Qf = static_cast<const u32x4_t*>(P.Qf) + chunk * (4 * KS * 2 * 64);
    const u32x4_t* Kf = static_cast<const u32x4_t*>(P.Kf) + chunk * (MTI * 2 * 2 * 64);
    const u32x4_t* Af = static_cast<const u32x4_t*>(P.Af) + chunk * (4 * 2 * 2 * 64);
    const f32x4_t* Uf = reinterpret_cast<const f32x4_t*>(P.Uf) + chunk * (NJ * 4 * 64) + nj * 4 * 64;
    const f32x4_t* dec4 = reinterpret_cast<const f32x4_t*>(P.dec + chunk * D);
    const int t0 = c * CS, nt = min(CS, P.L - t0);

    // state columns as B operands: k = key channel in the permuted order
    Frag sf[KS];
#pragma unroll
    for (int p = 0; p < KS; ++p) {
      float x[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) { x[r] = S[2 * p][r]; x[4 + r] = S[2 * p + 1][r]; }
      sf[p] = split8(x);
    }
    // D = U - W S and O = (q 2^G) S
    f32x4_t Dm[4], Om[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Dm[mt] = Uf[mt * 64 + lane];
      Om[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int p = 0; p < KS; ++p)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        Dm[mt] = mma3(load_frag(Wf, mt * KS + p, lane), sf[p], Dm[mt]);
        Om[mt] = mma3(load_frag(Qf, mt * KS + p, lane), sf[p], Om[mt]);
      }
    // D as B operands: k = token in the permuted order
    Frag df[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float x[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) { x[r] = Dm[2 * p][r]; x[4 + r] = Dm[2 * p + 1][r]; }
      df[p] = split8(x);
    }
    // O += A D (A is zero above the diagonal: token tiles 0, 1 need only s < 32)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        if (p <= mt / 2) Om[mt] = mma3(load_frag(Af, mt * 2 + p, lane), df[p], Om[mt]);
    // S <- diag(2^G_last) S + (k 2^(G_last - G))^T D
#pragma unroll
    for (int mt = 0; mt < MTI; ++mt) {
      const f32x4_t dd = dec4[4 * mt + q4];
      S[mt] = S[mt] * dd;
#pragma unroll
      for (int p = 0; p < 2; ++p) S[mt] = mma3(load_frag(Kf, mt * 2 + p, lane), df[p], S[mt]);
    }
    float* og = P.o + ((size_t)b * P.L + t0) * orow + (size_t)h * D + j;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * mt + 4 * q4 + r;
        if (t < nt) og[(size_t)t * orow] = Om[mt][r];
      }
  }
#pragma unroll
  for (int mt = 0; mt < MTI; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) Sg[(size_t)(16 * mt + 4 * q4 + r) * D + j] = S[mt][r];
}

}  // namespace

hipError_t launch_chunk_prep(const PrefillParams& p, hipStream_t s) {
  dim3 grid(p.nch, p.H, p.B);
  if (p.dk == 128)
    chunk_prep_kernel<128><<<grid, 256, 0, s>>>(p);
  else
    chunk_prep_kernel<64><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_chunk_scan(const PrefillParams& p, hipStream_t s) {
  const int blocks = p.B * p.H * (p.dk / 16);
  if (p.dk == 128)
    chunk_scan_kernel<128><<<blocks, 64, 0, s>>>(p);
  else
    chunk_scan_kernel<64><<<blocks, 64, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace kda

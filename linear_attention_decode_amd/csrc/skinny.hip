// Q8_0 weights times a few columns on the matrix cores of gfx950: the projections of verify
// (B sequences x T tokens) and of batched decode, where the vector GEMV would stream the
// weights once per 8 columns at two VALU instructions per weight and column.
//
// Two launches per product:
//   skinny_prep   one block per input column: the GEMV's prologue (RMSNorm of x, or the
//                 gated RMSNorm of the heads), a power-of-two column scale keeping the values
//                 well inside fp16 range, and the split x = hi + lo into two fp16 values, both
//                 written in the B-operand layout of v_mfma_f32_16x16x32_f16, plus each
//                 32-element block's sum of hi + lo;
//   skinny_gemm   one block per 16 weight rows, four waves splitting K.  A lane turns 8
//                 weight bytes u = q + 128 into the fp16 values 1024 + u with two byte
//                 permutes per 4 bytes (1152 + q exactly), so one MFMA pair per 32-wide Q8_0
//                 block gives sum (1152 + q) x; the block's scale and the bias 1152 * sum x
//                 are applied to the MFMA output before it joins the fp32 sum.  The waves'
//                 partial sums meet in LDS, then the GEMV's epilogues (conv + SiLU + window
//                 roll, residual) run unchanged.
// The result differs from the fp32 GEMV only by rounding: x is carried to ~22 bits by the
// hi/lo pair, the weight values are exact, and the MFMA accumulates in fp32.
// BF16 weights (BF = true) go to v_mfma_f32_16x16x32_bf16 as they are, against x split into
// two BF16 terms (hi = bf16(x), lo = bf16(x - hi): ~16 significant bits, as in the prefill
// GEMMs); no scales or bias, the MFMAs accumulate over the whole K range.  MXFP4 weights
// (FP4 = true) take the same path after gfx950's scaled FP4 -> BF16 conversion
// (v_cvt_scalef32_pk_bf16_fp4, two codes a byte, low nibble first, times the block's E8M0
// scale), which is exact: every E2M1 value times a power of two is a BF16 value.
#include <type_traits>

#include "kda_device.h"
#include "skinny.h"

namespace kda {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8s __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2s __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kSkThreads = 256;
constexpr int kSkRows = 16;        // weight rows per block

size_t skinny_scratch_bytes(int N, int K) {
  const size_t NT = (size_t)(N + 15) / 16, KB = (size_t)K / 32;
  return align_up(KB * NT * 64 * 16, 256) * 2 + align_up(KB * NT * 16 * 4, 256) +
         align_up(NT * 16 * 4, 256);
}

bool skinny_supported(int wt, int N, int K) {
  // Q8_0 from 9 columns (the vector GEMV streams its bytes fast enough below), BF16 from 5
  // (its vector GEMV pays an unpack and N FMAs a weight: 49 us for the D = 2048 projections
  // at 8 columns against 12 here; at 2 columns the GEMV's 14 us beat the prep + GEMM pair),
  // MXFP4 from 2 (its vector GEMV's code decoding: 36 us at 2 columns, 79 at 4)
  return ((wt == kQ8 && N > 8 && (K == 2048 || K == 4096)) || (wt == kBF16 && N > 4 && K == 2048) ||
          (wt == kMX4 && N > 1 && K == 2048)) &&
         N <= 64;
}

bool skinny_mma_supported(int N, int K) { return N >= 1 && N <= 64 && (K == 1024 || K == 2048); }

struct SkScratch {
  uint4* fh;        // [K/32][NT][64] fp16 x 8: hi parts, B-operand layout
  uint4* fl;        // same, lo parts
  float* xsum;      // [K/32][NT * 16] sum of (hi + lo) over each 32-element block
  float* cscale;    // [NT * 16] 2^-e: the factor the column was multiplied by, inverted
};

static SkScratch carve(void* scratch, int N, int K) {
  const size_t NT = (size_t)(N + 15) / 16, KB = (size_t)K / 32;
  char* p = static_cast<char*>(scratch);
  SkScratch s;
  s.fh = reinterpret_cast<uint4*>(p);
  p += align_up(KB * NT * 64 * 16, 256);
  s.fl = reinterpret_cast<uint4*>(p);
  p += align_up(KB * NT * 64 * 16, 256);
  s.xsum = reinterpret_cast<float*>(p);
  p += align_up(KB * NT * 16 * 4, 256);
  s.cscale = reinterpret_cast<float*>(p);
  return s;
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 a, _Float16 b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// fp32 -> BF16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------------------------------------
// skinny_prep: column n of the (prologue-applied) input -> fp16 hi/lo fragments.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// KG = ceil(K / 2048) groups of 8 consecutive elements per thread (all loaded in one
// pass; groups past K are empty).
template <int PRO, int KG, bool BF>
__global__ __launch_bounds__(kSkThreads) void skinny_prep_kernel(const GemvParams P, int NT,
                                                                 SkScratch S) {
  __shared__ float red[2][4];
  __shared__ float scal[kGemvMaxHeads];
  const int n = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = P.K;
  const bool live = n < P.N;   // block-uniform
  if (PRO == kProGatedNorm && live) {
    if (tid < P.H) {
      const float* sp = P.ss + ((size_t)n * P.H + tid) * P.ncb;
      scal[tid] = 1.0f / sqrtf(sum_partials(sp, P.ncb) / (float)P.dv + P.eps);
    }
    __syncthreads();
  }
  // this thread's values: groups g8 = tid + 256 q, elements 8 g8 .. + 7
  float v[KG][8];
#pragma unroll
  for (int q = 0; q < KG; ++q) {
    const int k0 = 8 * (tid + kSkThreads * q);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (live && k0 < K) {
        if constexpr (PRO == kProX) {
          x = *reinterpret_cast<const float4*>(P.x + (size_t)n * P.x_stride + k0 + 4 * h2);
        } else {
          const int k = k0 + 4 * h2, hh = k / P.dv;
          const size_t g = (size_t)n * K + k;
          const float4 o = *reinterpret_cast<const float4*>(P.o + g);
          const float4 gt = *reinterpret_cast<const float4*>(P.gate + g);
          float4 w = make_float4(1.f, 1.f, 1.f, 1.f);
          if (P.onw) w = *reinterpret_cast<const float4*>(P.onw + (k - hh * P.dv));
          const float sc = scal[hh];
          x = make_float4(o.x * sc * w.x * gt.x, o.y * sc * w.y * gt.y, o.z * sc * w.z * gt.z,
                          o.w * sc * w.w * gt.w);
        }
      }
      v[q][4 * h2] = x.x; v[q][4 * h2 + 1] = x.y; v[q][4 * h2 + 2] = x.z; v[q][4 * h2 + 3] = x.w;
    }
  }
  // one reduction round: sum of squares (RMSNorm of x) and max |value|
  float ssq = 0.0f, amax = 0.0f;
#pragma unroll
  for (int q = 0; q < KG; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ssq += v[q][e] * v[q][e];
      amax = fmaxf(amax, fabsf(v[q][e]));
    }
  ssq = wave_sum(ssq);
  amax = wave_max(amax);
  if (lane == 0) { red[0][wave] = ssq; red[1][wave] = amax; }
  __syncthreads();
  float sc = 1.0f;
  if (PRO == kProX && P.prenorm)
    sc = 1.0f / sqrtf((red[0][0] + red[0][1] + red[0][2] + red[0][3]) / (float)K + P.eps);
  amax = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3])) * sc;
  // power-of-two column scale: max |x| lands in [1024, 2048)
  int e = 0;
  if (amax > 0.0f) frexpf(amax, &e);           // amax in [2^(e-1), 2^e)
  const float up = ldexpf(1.0f, 11 - e) * sc;
  if (tid == 0) S.cscale[n] = live && amax > 0.0f ? ldexpf(1.0f, e - 11) : 0.0f;
  const int ct = n >> 4, nl = n & 15;
#pragma unroll
  for (int q = 0; q < KG; ++q) {
    const int k0 = 8 * (tid + kSkThreads * q), kb = k0 >> 5, g = (k0 >> 3) & 3;
    if (k0 >= K) break;
    const size_t fi = ((size_t)kb * NT + ct) * 64 + nl + 16 * g;
    float s = 0.0f;
    if constexpr (BF) {
      uint32_t hb[8], lb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = v[q][j] * up;
        hb[j] = bf16_bits(x);
        lb[j] = bf16_bits(x - __uint_as_float(hb[j] << 16));
      }
      S.fh[fi] = make_uint4(hb[0] | hb[1] << 16, hb[2] | hb[3] << 16, hb[4] | hb[5] << 16, hb[6] | hb[7] << 16);
      S.fl[fi] = make_uint4(lb[0] | lb[1] << 16, lb[2] | lb[3] << 16, lb[4] | lb[5] << 16, lb[6] | lb[7] << 16);
    } else {
      _Float16 hi[8], lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = v[q][j] * up;
        hi[j] = (_Float16)x;
        const float hv = (float)hi[j];
        lo[j] = (_Float16)(x - hv);
        s += hv + (float)lo[j];
      }
      S.fh[fi] = make_uint4(pack_h2(hi[0], hi[1]), pack_h2(hi[2], hi[3]), pack_h2(hi[4], hi[5]), pack_h2(hi[6], hi[7]));
      S.fl[fi] = make_uint4(pack_h2(lo[0], lo[1]), pack_h2(lo[2], lo[3]), pack_h2(lo[4], lo[5]), pack_h2(lo[6], lo[7]));
    }
    // the four threads of a k block are consecutive lanes
    s = group_sum(s, 4);
    if (g == 0) S.xsum[(size_t)kb * NT * 16 + n] = s;
  }
}

// ------------------------------------------------------------------------------------
// skinny_gemm: out[n][out_off + row] = sum_k W[row][k] x[n][k] (+ epilogue)
// ------------------------------------------------------------------------------------
struct SkSeg {
  PackedMat m;
  int rows = 0, first_tile = 0, out_off = 0, conv_chan = -1;
};
struct SkParams {
  SkSeg seg[kMaxSegs];
  int nseg = 0, K = 0, N = 0;
  SkScratch S;
  float* out = nullptr;
  int out_stride = 0;
  const float* resid = nullptr;
  const float* conv_w = nullptr;
  float* win = nullptr;
  int C = 0;
  float* act = nullptr;
  int T = 0;
  const int* active = nullptr;
  const float* pre_proj = nullptr;
  const int* pre_ntok = nullptr;
  int pre_T = 0;
};

// 8 weight bytes u -> 8 fp16 values 1024 + u (byte permutes against 0x64 high bytes)
__device__ __forceinline__ f16x8 bytes_to_f16(const uint2 w) {
  const uint32_t k64 = 0x64646464u;
  uint32_t r[4];
  r[0] = __builtin_amdgcn_perm(k64, w.x, 0x04010400u);
  r[1] = __builtin_amdgcn_perm(k64, w.x, 0x04030402u);
  r[2] = __builtin_amdgcn_perm(k64, w.y, 0x04010400u);
  r[3] = __builtin_amdgcn_perm(k64, w.y, 0x04030402u);
  return __builtin_bit_cast(f16x8, r);
}

// NT column tiles of 16; KB4 = K / 128 k blocks per wave; RT row tiles of 16 per block
// (each wave's B fragments serve all of them).
// MMA: the Q8_0 matrices are in the matrix-core order of the one-launch decode (persist.h:
// per 16-row tile, 16-byte chunks c = ((w * 2U + t) * 2 + h) * 64 + r + 16 g holding row r,
// bytes 16 h .. + 15 of block 4 (4 t + w) + g as signed q; the tile's scales at
// ((w * 64 + r + 16 g) * 2U + t)), U = K / 1024.
// 8 MXFP4 codes (4 bytes, low nibble first) times 2^(e - 127) as 8 BF16 values
__device__ __forceinline__ bf16x8s fp4x8_to_bf16(uint32_t codes, uint32_t e) {
  const float sc = __builtin_amdgcn_ldexpf(1.0f, (int)e - 127);
  const bf16x2s p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0);
  const bf16x2s p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1);
  const bf16x2s p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2);
  const bf16x2s p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3);
  return bf16x8s{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <int NT, int KB4, bool MMA, int RT, bool BF, bool FP4 = false>
__global__ __launch_bounds__(kSkThreads, 2) void skinny_gemm_kernel(const SkParams P) {
  constexpr int KB = 4 * KB4;
  constexpr int PD = 4;                          // k blocks of B fragments in flight
  constexpr int ROWS = kSkRows * RT;             // weight rows per block
  __shared__ float part[4][RT][NT][64][4];       // per-wave partial outputs
  __shared__ float s_row[ROWS][NT * 16];         // verify conv: the block's rows, all columns
  __shared__ __half s_sc[KB][ROWS];              // [k block][row] Q8_0 scales
  __shared__ __align__(16) float s_xs[KB][NT * 16];   // [k block][column] block sums
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int K = KB * 32;
  // segment of this block
  SkSeg sg = P.seg[0];
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i)
    if (i < P.nseg && (int)blockIdx.x >= P.seg[i].first_tile) sg = P.seg[i];
  const int row0 = ((int)blockIdx.x - sg.first_tile) * ROWS;
  const int nrows = min(ROWS, sg.rows - row0);
  // a row tile past the segment's last repeats the first (its rows are not stored)
  auto tile_of = [&](int rt) { return 16 * rt < nrows ? rt : 0; };

  // scales [k block][row] and block sums: loaded first (ahead of the weights in the
  // in-order load counter), stored to LDS after the weight requests are out
  // scales: row r's KB halves are contiguous; 8 per 16-byte load
  constexpr int kScPer = KB * kSkRows / 8;       // 16-byte loads per row tile
  constexpr int kScLoadsN = (kScPer * RT + kSkThreads - 1) / kSkThreads;
  constexpr int kScLoads = BF ? 0 : kScLoadsN;   // (BF16: no scales, no block sums)
  u32x4 sv[kScLoadsN];
#pragma unroll
  for (int u = 0; u < kScLoads; ++u) {
    const int i = min(tid + u * kSkThreads, kScPer * RT - 1);
    const int rt = tile_of(i / kScPer), ii = i % kScPer;
    if constexpr (MMA) {
      sv[u] = *reinterpret_cast<const u32x4*>(sg.m.d + (size_t)(row0 + 16 * rt) * KB + 8 * ii);
    } else {
      const int r = min(16 * rt + ii / (KB / 8), nrows - 1), c8 = ii % (KB / 8);
      sv[u] = *reinterpret_cast<const u32x4*>(sg.m.d + (size_t)(row0 + r) * KB + 8 * c8);
    }
  }
  constexpr int kXsLoadsN = (KB * NT * 4 + kSkThreads - 1) / kSkThreads;
  constexpr int kXsLoads = BF ? 0 : kXsLoadsN;
  f32x4v xv[kXsLoadsN];
#pragma unroll
  for (int u = 0; u < kXsLoads; ++u) {
    const int i = min(tid + u * kSkThreads, KB * NT * 4 - 1);
    xv[u] = reinterpret_cast<const f32x4v*>(P.S.xsum)[i];
  }
  __builtin_amdgcn_sched_barrier(0);
  // A operand: lane holds row (lane & 15) of each row tile, bytes 8 (lane >> 4) .. + 7 of
  // each k block (BF16: elements 8 (lane >> 4) .. + 7, 16 bytes); the wave's whole K range
  // is requested up front
  const int ag = lane >> 4;
  const int kb0 = wave * KB4;
  // (MXFP4: 4 bytes of codes, elements 8 (lane >> 4) .. + 7, and the block's scale byte)
  std::conditional_t<BF, std::conditional_t<FP4, uint32_t, uint4>, uint2> a[RT][KB4];
  uint32_t ae[FP4 ? RT : 1][FP4 ? KB4 : 1];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int tr = tile_of(rt);
    const int ar = min(16 * tr + (lane & 15), nrows - 1);
    const uint8_t* wrow = FP4 ? sg.m.w + (size_t)(row0 + ar) * (K / 2) + 4 * ag
                              : sg.m.w + (size_t)(row0 + ar) * K * (BF ? 2 : 1) + (BF ? 16 : 8) * ag;
#pragma unroll
    for (int j = 0; j < KB4; ++j) {
      if constexpr (FP4) {
        a[rt][j] = *reinterpret_cast<const uint32_t*>(wrow + (size_t)(kb0 + j) * 16);
        ae[rt][j] = sg.m.e[(size_t)(row0 + ar) * KB + kb0 + j];
      } else if constexpr (BF) {
        a[rt][j] = *reinterpret_cast<const uint4*>(wrow + (size_t)(kb0 + j) * 64);
      } else if constexpr (MMA) {
        constexpr int U2 = KB4 / 4;              // 2U
        const int kb = kb0 + j, g = kb & 3, w = (kb >> 2) & 3, t = kb >> 4;
        const uint8_t* cp = sg.m.w + (size_t)(row0 + 16 * tr) * K +
                            ((size_t)(((w * U2 + t) * 2 + (ag >> 1)) * 64 + (lane & 15) + 16 * g)) * 16 +
                            8 * (ag & 1);
        const u32x2 v = *reinterpret_cast<const u32x2*>(cp);
        a[rt][j] = make_uint2(v.x ^ 0x80808080u, v.y ^ 0x80808080u);   // q -> q + 128
      } else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(wrow + (size_t)(kb0 + j) * 32);
        a[rt][j] = make_uint2(v.x, v.y);
      }
    }
  }
  // B operand: a ring of PD k blocks of hi/lo fragments ahead of the MFMAs
  const u32x4* fh = reinterpret_cast<const u32x4*>(P.S.fh) + lane;
  const u32x4* fl = reinterpret_cast<const u32x4*>(P.S.fl) + lane;
  u32x4 bh[PD][NT], bl[PD][NT];
  auto load_b = [&](int j, int slot) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const size_t fi = ((size_t)(kb0 + j) * NT + t) * 64;
      bh[slot][t] = fh[fi];
      bl[slot][t] = fl[fi];
    }
  };
#pragma unroll
  for (int j = 0; j < PD && j < KB4; ++j) load_b(j, j);
  __builtin_amdgcn_sched_barrier(0);
  {
#pragma unroll
    for (int u = 0; u < kScLoads; ++u) {
      const int i = tid + u * kSkThreads;
      if (i < kScPer * RT) {
        const int rt = i / kScPer, ii = i % kScPer;
        const uint32_t w[4] = {sv[u][0], sv[u][1], sv[u][2], sv[u][3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const unsigned short bits = (unsigned short)((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
          int r, kb;
          if constexpr (MMA) {
            constexpr int U2 = KB4 / 4;
            const int q = 8 * ii + e, t = q % U2, L = (q / U2) & 63, wv = q / (U2 * 64);
            r = L & 15;
            kb = 4 * (4 * t + wv) + (L >> 4);
          } else {
            r = ii / (KB / 8);
            kb = 8 * (ii % (KB / 8)) + e;
          }
          r += 16 * rt;
          s_sc[kb][r] = r < nrows ? __ushort_as_half(bits) : __float2half(0.0f);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kXsLoads; ++u) {
      const int i = tid + u * kSkThreads;
      if (i < KB * NT * 4) reinterpret_cast<f32x4v*>(&s_xs[0][0])[i] = xv[u];
    }
  }
  __syncthreads();

  f32x4v acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[rt][t] = f32x4v{0.f, 0.f, 0.f, 0.f};
  const int og = lane >> 4, oc = lane & 15;      // output rows 4 og .. + 3, column oc (+ 16 t)
#pragma unroll
  for (int j = 0; j < KB4; ++j) {
    const int kb = kb0 + j, slot = j % PD;
    if constexpr (BF) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        bf16x8s av;
        if constexpr (FP4) av = fp4x8_to_bf16(a[rt][j], ae[rt][j]);
        else av = __builtin_bit_cast(bf16x8s, a[rt][j]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8s, bh[slot][t]),
                                                               acc[rt][t], 0, 0, 0);
          acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8s, bl[slot][t]),
                                                               acc[rt][t], 0, 0, 0);
        }
      }
      if (j + PD < KB4) load_b(j + PD, slot);
    } else {
      f32x4v o[RT][NT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const f16x8 av = bytes_to_f16(a[rt][j]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          o[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(f16x8, bh[slot][t]),
                                                            f32x4v{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          o[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(f16x8, bl[slot][t]),
                                                            o[rt][t], 0, 0, 0);
        }
      }
      if (j + PD < KB4) load_b(j + PD, slot);
      float bias[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) bias[t] = 1152.0f * s_xs[kb][t * 16 + oc];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const uint2 sc2 = *reinterpret_cast<const uint2*>(&s_sc[kb][16 * rt + 4 * og]);
        const float d0 = __half2float(__ushort_as_half((unsigned short)(sc2.x & 0xffffu)));
        const float d1 = __half2float(__ushort_as_half((unsigned short)(sc2.x >> 16)));
        const float d2 = __half2float(__ushort_as_half((unsigned short)(sc2.y & 0xffffu)));
        const float d3 = __half2float(__ushort_as_half((unsigned short)(sc2.y >> 16)));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[rt][t][0] += d0 * (o[rt][t][0] - bias[t]);
          acc[rt][t][1] += d1 * (o[rt][t][1] - bias[t]);
          acc[rt][t][2] += d2 * (o[rt][t][2] - bias[t]);
          acc[rt][t][3] += d3 * (o[rt][t][3] - bias[t]);
        }
      }
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wave][rt][t][lane][i] = acc[rt][t][i];
  __syncthreads();
  // sum the four waves' partials and run the epilogue: thread -> (rt, t, lane, i)
  for (int e = tid; e < RT * NT * 64 * 4; e += kSkThreads) {
    const int rt = e / (NT * 256), t = (e / 256) % NT, l = (e >> 2) & 63, i = e & 3;
    const int row = 16 * rt + 4 * (l >> 4) + i, n = t * 16 + (l & 15);
    if (row >= nrows || n >= P.N) continue;
    float v = (part[0][rt][t][l][i] + part[1][rt][t][l][i]) + (part[2][rt][t][l][i] + part[3][rt][t][l][i]);
    v *= P.S.cscale[n];
    const int grow = row0 + row;
    if (sg.conv_chan >= 0 && P.act) {
      s_row[row][n] = v;           // raw projection (logged); the conv runs below
    } else if (sg.conv_chan >= 0) {
      // causal conv over (window, this token), SiLU, window roll (one owner per channel)
      const int c = sg.conv_chan + grow;
      const float4 w = *reinterpret_cast<const float4*>(P.conv_w + (size_t)c * 4);
      float* z = P.win + (size_t)n * 3 * P.C + c;
      const float z0 = z[0], z1 = z[P.C], z2 = z[2 * P.C];
      const float y = conv4_f(w, z0, z1, z2, v);
      if (!P.active || P.active[n]) {
        z[0] = z1;
        z[P.C] = z2;
        z[2 * P.C] = v;
      }
      v = silu_f(y);
    }
    const size_t o = (size_t)n * P.out_stride + sg.out_off + grow;
    if (P.resid) v += P.resid[o];
    P.out[o] = v;
  }
  if (sg.conv_chan >= 0 && P.act) {
    // verify: each (row, sequence) runs the causal conv + SiLU over the sequence's window
    // and its T tokens in order; the window is read, not rolled (the commit rolls it), but
    // a commit folded into this verify first moves it on by the previous verify's accepted
    // tokens, from that verify's logged projections, and writes it back
    __syncthreads();
    const int nb = P.N / P.T;
    for (int e = tid; e < nrows * nb; e += kSkThreads) {
      const int row = e / nb, b = e - row * nb;
      const int c = sg.conv_chan + row0 + row;
      const float4 w = *reinterpret_cast<const float4*>(P.conv_w + (size_t)c * 4);
      float* z = P.win + (size_t)b * 3 * P.C + c;
      float z0, z1, z2;
      if (P.pre_ntok) {
        const int a = min(max(P.pre_ntok[b], 1), P.pre_T);
        const float* pp = P.pre_proj + (size_t)b * P.pre_T * P.out_stride + sg.out_off + row0 + row;
        z0 = a < 3 ? z[(size_t)a * P.C] : pp[(size_t)(a - 3) * P.out_stride];
        z1 = a < 2 ? z[(size_t)(a + 1) * P.C] : pp[(size_t)(a - 2) * P.out_stride];
        z2 = pp[(size_t)(a - 1) * P.out_stride];
        z[0] = z0;
        z[P.C] = z1;
        z[2 * P.C] = z2;
      } else {
        z0 = z[0];
        z1 = z[P.C];
        z2 = z[2 * P.C];
      }
      for (int t = 0; t < P.T; ++t) {
        const float pv = s_row[row][b * P.T + t];
        const float y = conv4_f(w, z0, z1, z2, pv);
        z0 = z1;
        z1 = z2;
        z2 = pv;
        P.act[(size_t)(b * P.T + t) * P.C + c] = silu_f(y);
      }
    }
  }
}

hipError_t launch_skinny(int prologue, const GemvParams& g, void* scratch, hipStream_t s) {
  const int NT = (g.N + 15) / 16;
  SkParams p;
  p.nseg = g.nseg;
  // two 16-row tiles per block (each B fragment used twice) when that still leaves at
  // least 192 blocks and the operands fit the registers (up to 32 columns, K = 2048)
  int rows32 = 0;
  for (int i = 0; i < g.nseg; ++i) rows32 += (g.seg[i].rows + 31) / 32;
  const int RT = (g.wt == kQ8 && rows32 >= 192 && NT <= 2 && g.K == 2048) ? 2 : 1;
  int tiles = 0;
  for (int i = 0; i < g.nseg; ++i) {
    p.seg[i].m = g.seg[i].m;
    p.seg[i].rows = g.seg[i].rows;
    p.seg[i].first_tile = tiles;
    p.seg[i].out_off = g.seg[i].out_off;
    p.seg[i].conv_chan = g.seg[i].conv_chan;
    tiles += (g.seg[i].rows + kSkRows * RT - 1) / (kSkRows * RT);
  }
  p.K = g.K;
  p.N = g.N;
  p.S = carve(scratch, g.N, g.K);
  p.out = g.out;
  p.out_stride = g.out_stride;
  p.resid = g.resid;
  p.conv_w = g.conv_w;
  p.win = g.win;
  p.C = g.C;
  p.act = g.act;
  p.T = g.T;
  p.active = g.active;
  p.pre_proj = g.pre_proj;
  p.pre_ntok = g.pre_ntok;
  p.pre_T = g.pre_T;
  const int KG = g.K > 2048 ? 2 : 1;             // 8-element groups a thread (K <= 4096)
  const bool bf = g.wt == kBF16 || g.wt == kMX4, fp4 = g.wt == kMX4;
#define KDA_SK_PREP(pro, kg, b) \
  if ((prologue == kProX) == (pro == kProX) && KG == kg && bf == b) \
    skinny_prep_kernel<pro, kg, b><<<NT * 16, kSkThreads, 0, s>>>(g, NT, p.S);
  KDA_SK_PREP(kProX, 1, false) KDA_SK_PREP(kProX, 2, false)
  KDA_SK_PREP(kProGatedNorm, 1, false) KDA_SK_PREP(kProGatedNorm, 2, false)
  KDA_SK_PREP(kProX, 1, true) KDA_SK_PREP(kProX, 2, true)
  KDA_SK_PREP(kProGatedNorm, 1, true) KDA_SK_PREP(kProGatedNorm, 2, true)
#undef KDA_SK_PREP
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int KB4 = g.K / 128;
#define KDA_SK_CASE(nt, kb4, mm, rt) \
  if (!bf && NT == nt && KB4 == kb4 && (g.mma != 0) == mm && RT == rt) \
    skinny_gemm_kernel<nt, kb4, mm, rt, false><<<tiles, kSkThreads, 0, s>>>(p);
#define KDA_SK_BF(nt, kb4) \
  if (bf && !fp4 && NT == nt && KB4 == kb4 && RT == 1) \
    skinny_gemm_kernel<nt, kb4, false, 1, true><<<tiles, kSkThreads, 0, s>>>(p); \
  if (fp4 && NT == nt && KB4 == kb4 && RT == 1) \
    skinny_gemm_kernel<nt, kb4, false, 1, true, true><<<tiles, kSkThreads, 0, s>>>(p);
  KDA_SK_CASE(1, 8, false, 1) KDA_SK_CASE(2, 8, false, 1) KDA_SK_CASE(3, 8, false, 1) KDA_SK_CASE(4, 8, false, 1)
  KDA_SK_CASE(1, 16, false, 1) KDA_SK_CASE(2, 16, false, 1) KDA_SK_CASE(3, 16, false, 1) KDA_SK_CASE(4, 16, false, 1)
  KDA_SK_CASE(1, 32, false, 1) KDA_SK_CASE(2, 32, false, 1) KDA_SK_CASE(3, 32, false, 1) KDA_SK_CASE(4, 32, false, 1)
  KDA_SK_CASE(1, 8, true, 1) KDA_SK_CASE(2, 8, true, 1) KDA_SK_CASE(3, 8, true, 1) KDA_SK_CASE(4, 8, true, 1)
  KDA_SK_CASE(1, 16, true, 1) KDA_SK_CASE(2, 16, true, 1) KDA_SK_CASE(3, 16, true, 1) KDA_SK_CASE(4, 16, true, 1)
  KDA_SK_CASE(1, 16, false, 2) KDA_SK_CASE(2, 16, false, 2) KDA_SK_CASE(1, 16, true, 2) KDA_SK_CASE(2, 16, true, 2)
  KDA_SK_BF(1, 16) KDA_SK_BF(2, 16) KDA_SK_BF(3, 16) KDA_SK_BF(4, 16)
#undef KDA_SK_BF
#undef KDA_SK_CASE
  return hipGetLastError();
}

}  // namespace kda

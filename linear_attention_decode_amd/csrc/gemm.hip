// Dense GEMM on gfx950 matrix cores for the chunked prefill's projections:
//   C[m][coff + n] = sum_k A[m][k] B[n][k]      (A: BF16 [M][lda], B rows: BF16 [N][K])
// B may be several matrices stacked along n (a segment table).  An fp32 operand is passed
// as two BF16 planes A = A_hi + A_lo (hi = bf16(a), lo = bf16(a - hi)); the k loop then
// runs over both planes against the same B, i.e. C = A_hi B^T + A_lo B^T, every product
// exact in fp32 accumulation.
//
// Block tile 256 x 256 x 64, 8 waves as 4 (m) x 2 (n), each 64 x 128 = 4 x 8 tiles of
// v_mfma_f32_16x16x32_bf16 (lane l: row l % 16 of A and of B^T, k = 8 (l / 16) .. + 7;
// accumulator rows 4 (l / 16) + r, column l % 16).  Operand tiles stream through a
// two-stage LDS ring filled by direct global->LDS loads one k-step ahead; a tile row is
// eight 16-byte chunks stored with chunk c of row r at position c ^ (r & 7), so the
// fragment reads of 8 consecutive rows hit distinct banks.  Tiles are visited in groups of
// 8 row tiles, each XCD taking a contiguous run, so the blocks running together on one XCD
// share their A and B tiles in its L2.  C is written with non-temporal stores (it is read
// back from HBM by the next kernel, not from the caches).  The tile shape, ring depth and
// store kind were chosen by timing the two prefill projection shapes.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 64, NST = 2;
constexpr int CPR = BK / 8;              // 16-byte chunks per tile row
constexpr int TCH = BM * CPR;           // 16-byte chunks per operand tile (2048)
constexpr int LPT = TCH / 512;          // chunk loads per thread per operand per k-step
constexpr int GROUP_M = 8;

// One 16-byte load per lane straight into LDS (the lanes of the wave fill consecutive
// entries from lds_wave_base).  Inline assembly, so the compiler does not track it; the
// explicit waits below order it.  Nothing else in this kernel uses m0.
__device__ __forceinline__ void dma16(const void* src, u32x4_t* lds_wave_base) {
  const unsigned lds = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

__global__ __launch_bounds__(512) void gemm_kernel(const GemmParams P) {
  __shared__ u32x4_t ring[NST][2 * TCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;           // 4 x 2 waves of 64 x 128

  // tile order: XCD-contiguous runs, groups of GROUP_M row tiles
  const int tiles_m = (P.M + BM - 1) / BM, tiles_n = (P.N + BN - 1) / BN;
  const int nblk = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((nblk & 7) == 0) t = (t & 7) * (nblk >> 3) + (t >> 3);
  const int per_group = GROUP_M * tiles_n;
  const int g = t / per_group, first_m = g * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int pid_m = first_m + (t % per_group) % gsize;
  const int pid_n = (t % per_group) / gsize;
  const int m0 = pid_m * BM, n0 = pid_n * BN;

  // per thread: LPT chunks of the A tile and LPT of the B tile per k-step
  const uint16_t* pa[LPT];
  const uint16_t* pa2[LPT];
  const uint16_t* pb[LPT];
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    const int e = tid + 512 * u;
    const int r = e / CPR, c = (e % CPR) ^ (r & 7);
    const int am = min(m0 + r, P.M - 1);
    pa[u] = P.A + (size_t)am * P.lda + 8 * c;
    pa2[u] = P.A2 ? P.A2 + (size_t)am * P.lda + 8 * c : pa[u];
    const int n = min(n0 + r, P.N - 1);
    int first = P.seg_first[0];
    const uint16_t* base = P.seg_b[0];
#pragma unroll
    for (int i = 1; i < kMaxSegs; ++i)
      if (i < P.nseg && n >= P.seg_first[i]) { first = P.seg_first[i]; base = P.seg_b[i]; }
    pb[u] = base + (size_t)(n - first) * P.K + 8 * c;
  }
  const int nk = P.K / BK;
  const int NK = P.A2 ? 2 * nk : nk;
  auto issue = [&](int kt) {
    const int st = kt % NST;
    const bool second = kt >= nk;
    const int k0 = (second ? kt - nk : kt) * BK;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      u32x4_t* wa = &ring[st][64 * (wave + 8 * u)];
      dma16((second ? pa2[u] : pa[u]) + k0, wa);
      dma16(pb[u] + k0, wa + TCH);
    }
  };

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  issue(0);
  // fragment rows: 64 wm + 16 i + r16 (A), 128 wn + 16 j + r16 (B); k chunk 4 ks + q4 of the
  // row sits at position (4 ks + q4) ^ (row & 7) = (4 ks + q4) ^ (r16 & 7)
  const int a_row = ((64 * wm + r16) * CPR), b_row = TCH + ((128 * wn + r16) * CPR);
  const int sw = r16 & 7;

#pragma unroll 1
  for (int kt = 0; kt < NK; ++kt) {
    // tile kt has landed (no later tile is in flight yet); every wave is done with the
    // other slot, which the next tile's loads then fill
    wait_vm_barrier<0>();
    if (kt + 1 < NK) issue(kt + 1);
    const u32x4_t* st = ring[kt % NST];
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int ch = (4 * ks + q4) ^ sw;
      u32x4_t af[4], bf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = st[a_row + 16 * i * CPR + ch];
#pragma unroll
      for (int j = 0; j < 8; ++j) bf[j] = st[b_row + 16 * j * CPR + ch];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[i]),
                                                              __builtin_bit_cast(bf16x8_t, bf[j]),
                                                              acc[i][j], 0, 0, 0);
    }
  }

#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int col = n0 + 128 * wn + 16 * j + r16;
    if (col >= P.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 64 * wm + 16 * i + 4 * q4 + r;
        if (row < P.M) __builtin_nontemporal_store(acc[i][j][r], P.C + (size_t)row * P.ldc + P.coff + col);
      }
  }
}

// fp32 -> two BF16 planes hi = bf16(x), lo = bf16(x - hi), 4 values per thread
__global__ void split_planes_kernel(const float* __restrict__ x, uint16_t* __restrict__ hi,
                                    uint16_t* __restrict__ lo, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const f32x4_t v = reinterpret_cast<const f32x4_t*>(x)[i];
  uint16_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 bh = (__bf16)v[e];
    const float r = v[e] - (float)bh;
    const __bf16 bl = (__bf16)r;
    h[e] = __builtin_bit_cast(uint16_t, bh);
    l[e] = __builtin_bit_cast(uint16_t, bl);
  }
  reinterpret_cast<uint2*>(hi)[i] = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
  reinterpret_cast<uint2*>(lo)[i] = make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  if (p.K % BK || p.lda % 8 || p.M < 1 || p.N < 1) return hipErrorInvalidValue;
  const int blocks = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  gemm_kernel<<<blocks, 512, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_split_planes(const float* x, uint16_t* hi, uint16_t* lo, int64_t n, hipStream_t s) {
  if (n % 4) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  split_planes_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(x, hi, lo, n4);
  return hipGetLastError();
}

}  // namespace kda

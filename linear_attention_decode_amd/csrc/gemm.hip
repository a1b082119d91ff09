// Dense GEMM on gfx950 matrix cores for the chunked prefill's projections:
//   C[m][coff + n] = sum_k A[m][k] B[n][k]      (A: BF16 [M][lda], B rows: BF16 [N][K])
// B may be several matrices stacked along n (a segment table).  An fp32 operand is passed
// as two BF16 planes A = A_hi + A_lo (hi = bf16(a), lo = bf16(a - hi)); the k loop then
// runs over both planes against the same B, i.e. C = A_hi B^T + A_lo B^T, every product
// exact in fp32 accumulation.
//
// Block tile 256 x 256 x 32, 8 waves as 2 (m) x 4 (n), each 128 x 64 = 8 x 4 tiles of
// v_mfma_f32_16x16x32_bf16 (lane l: row l % 16 of A and of B^T, k = 8 (l / 16) .. + 7;
// accumulator rows 4 (l / 16) + r, column l % 16).  Operand tiles stream through a
// four-stage LDS ring filled by direct global->LDS loads three k-steps ahead; a tile row
// is four 16-byte chunks stored with chunk c of row r at position c ^ ((r >> 1) & 3), so
// the fragment reads of 8 consecutive rows hit distinct banks.  Tiles are visited in
// groups of 8 row tiles, each XCD taking a contiguous run, so the blocks running together
// on one XCD share their A and B tiles in its L2.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 32, NST = 4;
constexpr int TCH = BM * BK / 8;        // 16-byte chunks per operand tile (1024)
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
  const int wm = wave >> 2, wn = wave & 3;

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

  // per thread: two chunks of the A tile and two of the B tile per k-step
  const uint16_t* pa[2];
  const uint16_t* pa2[2];
  const uint16_t* pb[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + 512 * u;
    const int r = e >> 2, c = (e & 3) ^ ((r >> 1) & 3);
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
    for (int u = 0; u < 2; ++u) {
      u32x4_t* wa = &ring[st][64 * (wave + 8 * u)];
      dma16((second ? pa2[u] : pa[u]) + k0, wa);
      dma16(pb[u] + k0, wa + TCH);
    }
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int kt = 0; kt < NST - 1; ++kt)
    if (kt < NK) issue(kt);

  // fragment positions: row r (r16 = r % 16) and chunk q4 -> (r << 2) | (q4 ^ ((r16 >> 1) & 3))
  const int sw = q4 ^ ((r16 >> 1) & 3);
  const int a_off = ((128 * wm + r16) << 2) | sw;
  const int b_off = TCH + (((64 * wn + r16) << 2) | sw);

#pragma unroll 1
  for (int kt = 0; kt < NK; ++kt) {
    // tile kt has landed once at most the later tiles' loads are outstanding
    const int later = min(NK - 1 - kt, NST - 2);
    if (later >= 2) wait_vm_barrier<8>();
    else if (later == 1) wait_vm_barrier<4>();
    else wait_vm_barrier<0>();
    if (kt + NST - 1 < NK) issue(kt + NST - 1);
    const u32x4_t* st = ring[kt % NST];
    u32x4_t af[8], bf[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) af[i] = st[a_off + 64 * i];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = st[b_off + 64 * j];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[i]),
                                                            __builtin_bit_cast(bf16x8_t, bf[j]),
                                                            acc[i][j], 0, 0, 0);
  }

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + 64 * wn + 16 * j + r16;
    if (col >= P.N) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 128 * wm + 16 * i + 4 * q4 + r;
        if (row < P.M) P.C[(size_t)row * P.ldc + P.coff + col] = acc[i][j][r];
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

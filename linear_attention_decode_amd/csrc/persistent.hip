// One-launch decode step for gfx950: every layer of the stack for one token (batch 1) in a
// single launch of one block per CU (a plain launch by default; cooperative on request).
//
// Per layer the blocks run three phases of the KDA step ("Where the time goes", "Thirty
// tiny kernels per layer", frederic.ai), each on blocks of its own:
//   P  projection blocks: RMSNorm(x) and their rows of the fused input projections
//      [W_q; W_k; W_v; F_a; G_a; W_beta], with the causal conv + SiLU + window roll applied
//      by the owner of each q/k/v channel;
//   H  two blocks per head, each owning half of its value columns: the low-rank forget gate
//      alpha and its output-gate columns (F_b, G_b on the matrix cores), then the gated
//      delta rule (one wave per 16 value columns, state in registers), posting the gated
//      outputs and partial sums of o^2;
//   O  output blocks, 32 rows each: the heads' RMSNorm scales from those partials, the
//      output projection of the normalised heads and the residual.
// Every block streams its slice of its matrices, and it requests the next layer's slice
// soon after it has used the current one, so the weights of layer l + 1 are in flight
// while layer l's later phases run.  All dots run on the int8 matrix cores: the weights
// come from copies rearranged at model creation so that each load is 1 KB of consecutive
// signed Q8_0 bytes in B-operand order, and the input vector enters as three 7-bit planes
// under a power-of-two scale (exact products, integer accumulation, the Q8_0 scales applied
// per block afterwards).
//
// Blocks hand activations to each other as 64-bit words (tag << 32 | fp32 bits) written
// and read with agent-scope relaxed atomics (coherent across the XCDs' L2s); the tag names
// the token and layer.  The head blocks poll their input words directly from the start of
// the layer.  The head blocks post a flag word when they are done; the output blocks and
// the next layer's projection blocks watch those flags -- one wave, a short sleep between
// polls -- and poll their data words (the heads' outputs, and x, which lands 1.5-2 us later)
// once the first head block has flagged, so that polling stays far below the weight stream
// and a fresh word's fetch is also its detection (a flag posted with its words costs a
// second fetch of a fresh line).  A consumer always checks the tag of every data word it uses.  Every wait is
// bounded: on a timeout the block records an error word and every block leaves the kernel.
#include "kda_device.h"
#include "persist.h"

#define KDA_GLOBAL __attribute__((address_space(1)))
#define KDA_CONST __attribute__((address_space(4)))

// Phase timestamps for profiling builds (-DKDA_TRACE): thread 0 of every block records the
// 100 MHz real-time counter at up to 8 points of each layer in LDS, and the block copies
// them to a device table when it leaves; kda_trace_read copies the table out.  Product
// builds compile none of it.
#ifdef KDA_TRACE
constexpr int kTraceLayers = 64, kTraceSlots = 8;
#define KDA_STAMP(l, k) \
  do { if (threadIdx.x == 0 && (l) < kTraceLayers) sm.stamps[(l)][(k)] = __builtin_amdgcn_s_memrealtime(); } while (0)
#else
#define KDA_STAMP(l, k) do { } while (0)
#endif

namespace kda {

constexpr int kPT = 256;         // threads per block
constexpr int kHD = 128;         // d_k = d_v of the one-launch path
constexpr int kHSplit = 2;       // head blocks per head
constexpr int kPTiles = 3;       // 16-row tiles of a projection block (48 q/k/v rows)
constexpr int kOTiles = 2;       // 16-row tiles of an output band (32 rows)
constexpr int kHCols = kHD / kHSplit;   // value columns of one head block (16 per wave)

using GLayer = const KDA_CONST PersistLayer;

template <class T>
__device__ __forceinline__ const KDA_GLOBAL T* gp(const T* p) { return (const KDA_GLOBAL T*)p; }
template <class T>
__device__ __forceinline__ KDA_GLOBAL T* gpw(T* p) { return (KDA_GLOBAL T*)p; }

typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 gload4(const float* p) {
  const f32x4 v = *(const KDA_GLOBAL f32x4*)p;
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void gstore4(float* p, const float4 v) {
  *(KDA_GLOBAL f32x4*)p = f32x4{v.x, v.y, v.z, v.w};
}

// 16 weight bytes, streamed once per token.
__device__ __forceinline__ uint4 wload(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load((const KDA_GLOBAL u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Raw fp16 bits of a Q8_0 scale (converted when used, so the load is not waited on).
__device__ __forceinline__ uint32_t sload(const __half* p) { return *(const KDA_GLOBAL uint16_t*)p; }
__device__ __forceinline__ float h2f(uint32_t bits) {
  return __half2float(__ushort_as_half((unsigned short)bits));
}

__device__ __forceinline__ uint64_t tagged(uint32_t tag, float v) {
  return ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
}
__device__ __forceinline__ void put(uint64_t* p, uint32_t tag, float v) {
  __hip_atomic_store(gpw(p), tagged(tag, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t peek(const uint64_t* p) {
  return __hip_atomic_load(const_cast<KDA_GLOBAL uint64_t*>(gp(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int err_set(const PersistParams& P) {
  return __hip_atomic_load(gpw(P.err), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Records a failed wait: the device word every block checks, and the host-mapped word the
// host checks before it launches another step on this model.
__device__ __forceinline__ void err_raise(const PersistParams& P) {
  __hip_atomic_store(gpw(P.err), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (P.err_host) __hip_atomic_store(P.err_host, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left free): every vector memory access issued so
// far has completed.  Used before a store whose completion later waits must not include:
// the wait counter retires in order, so a load issued before a store can otherwise only be
// waited for together with that store.
__device__ __forceinline__ void retire_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Poll bookkeeping: every 32 polls look at the error word and the wall clock; give up after
// P.timeout wall-clock ticks (tens of milliseconds, against microseconds expected).
struct Spin {
  uint64_t t0;
  int n = 0;
  __device__ Spin() : t0(wall_clock64()) {}
  // true when the wait must stop (another block failed, or this one timed out)
  __device__ bool stop(const PersistParams& P) {
    if ((++n & 31) != 0) return false;
    if (err_set(P)) return true;
    if (wall_clock64() - t0 > P.timeout) {
      err_raise(P);
      return true;
    }
    return false;
  }
};

// The critical path's transcendentals on the hardware's base-2 exp and log, reciprocal and
// reciprocal square root (about 1 ulp each, against the 1e-3 the step is held to); the
// correctly rounded library forms cost 20-60 instructions each.
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ __forceinline__ float ln_hw(float x) { return __builtin_amdgcn_logf(x) * 0.693147180559945309f; }
__device__ __forceinline__ float rsq_hw(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float sigmoid_hw(float z) { return __builtin_amdgcn_rcpf(1.0f + exp_hw(-z)); }
__device__ __forceinline__ float softplus_hw(float z) { return fmaxf(z, 0.0f) + ln_hw(1.0f + exp_hw(-fabsf(z))); }

enum FlagPhase { kFlagH = 1 };

// Wall-clock ticks (100 MHz) a block holds its next-layer prefetch back after its phase, so
// that the burst does not queue ahead of the polls its consumers issue meanwhile (timed:
// 0.5-1 us of hold was 4 % faster per token than none; the weights are needed ~7 us later).
#ifndef KDA_PREFETCH_DELAY
#define KDA_PREFETCH_DELAY 75
#endif
__device__ __forceinline__ void hold_prefetch() {
  const uint64_t t0 = wall_clock64();
  while (wall_clock64() - t0 < KDA_PREFETCH_DELAY) __builtin_amdgcn_s_sleep(8);
}

__device__ __forceinline__ uint64_t* flag_slot(const PersistParams& P, int phase, int i) {
  return P.flags + (size_t)phase * kMaxPersistBlocks + i;
}

// One wave, every lane active: poll the tag word *f of each lane (lanes may share a word)
// until some lane sees `tag`, for at most `rounds` rounds (>= 1).  Three loads stay in flight, issued
// ~0.16 us apart (a third of a round trip to the memory side), so a posted tag is seen about
// one spacing after it lands rather than up to a whole round trip later.  Written as one asm
// loop so that every check waits for its own load only (vmcnt 2; the counter retires in
// order).  Returns true when seen: up to two loads may then still be in flight into a, b, c,
// which the caller keeps live (keep_live) until a later wait has retired them.  Returns false
// after the rounds with nothing in flight.
__device__ __forceinline__ bool poll_tag3(const uint32_t* f, uint32_t tag, int rounds, uint32_t& a,
                                          uint32_t& b, uint32_t& c) {
  uint32_t found, cnt;
  asm volatile(
      "global_load_dword %0, %5, off sc1\n\t"
      "s_sleep 6\n\t"
      "global_load_dword %1, %5, off sc1\n\t"
      "s_sleep 6\n\t"
      "global_load_dword %2, %5, off sc1\n\t"
      "s_mov_b32 %4, %7\n\t"
      "s_mov_b32 %3, 1\n"
      "1:\n\t"
      "s_waitcnt vmcnt(2)\n\t"
      "v_cmp_eq_u32 vcc, %6, %0\n\t"
      "s_cbranch_vccnz 2f\n\t"
      "global_load_dword %0, %5, off sc1\n\t"
      "s_sleep 6\n\t"
      "s_waitcnt vmcnt(2)\n\t"
      "v_cmp_eq_u32 vcc, %6, %1\n\t"
      "s_cbranch_vccnz 2f\n\t"
      "global_load_dword %1, %5, off sc1\n\t"
      "s_sleep 6\n\t"
      "s_waitcnt vmcnt(2)\n\t"
      "v_cmp_eq_u32 vcc, %6, %2\n\t"
      "s_cbranch_vccnz 2f\n\t"
      "global_load_dword %2, %5, off sc1\n\t"
      "s_sleep 6\n\t"
      "s_sub_u32 %4, %4, 1\n\t"
      "s_cmp_eq_u32 %4, 0\n\t"
      "s_cbranch_scc0 1b\n\t"
      "s_waitcnt vmcnt(0)\n\t"
      "s_mov_b32 %3, 0\n"
      "2:"
      : "=&v"(a), "=&v"(b), "=&v"(c), "=&s"(found), "=&s"(cnt)
      : "v"(f), "s"(tag), "s"(rounds)
      : "vcc", "scc", "memory");
  return found != 0;
}

// Ends the live range of poll registers whose loads a later wait has retired.
__device__ __forceinline__ void keep_live(const uint32_t (&r)[3]) {
  asm volatile("" : : "v"(r[0]), "v"(r[1]), "v"(r[2]) : "memory");
}

// Wave 0 watches flags [0, n) of `phase` (n <= 64) until one carries `tag`; the caller's
// block_any then holds the other waves.  pend[] holds wave 0's poll registers (see
// poll_tag3).  The wait is bounded by the wall clock: on a timeout the error word is recorded
// and 1 is returned.
__device__ int wave0_wait_flags(const PersistParams& P, int phase, int n, uint32_t tag,
                                uint32_t (&pend)[3]) {
  int bad = 0;
  // every earlier load (a prefetch long landed) is retired first, in every wave: a wait for
  // one of them after the polls would also wait for the polls still in flight
  retire_vmem();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const uint32_t* f = reinterpret_cast<const uint32_t*>(flag_slot(P, phase, lane < n ? lane : 0)) + 1;
    const uint64_t t0 = wall_clock64();
    // (the error word is read only after a round of polls that found nothing, when no poll
    // is in flight: a load issued among them would make the code after the wait retire the
    // polls still in flight)
    while (!poll_tag3(f, tag, P.poll_rounds, pend[0], pend[1], pend[2])) {
      if (err_set(P)) {
        bad = 1;
        break;
      }
      if (wall_clock64() - t0 > P.timeout) {
        err_raise(P);
        bad = 1;
        break;
      }
    }
  }
  return bad;
}


// ---- matrix-core dots of the projections ----
// A block's projection rows meet the input vector on v_mfma_i32_16x16x64_i8.  The input is
// cut into runs of 128 elements (run rho = elements [128 rho, 128 rho + 128), one head of
// the output projection's input); wave w owns runs rho = 4 t + w and holds, in lane j,
// elements 128 rho + j and 128 rho + 64 + j of each (value 2 t + half).  Each run is split
// into three signed 7-bit planes under a power-of-two scale (below), so that every product
// with a Q8_0 weight byte is exact in the integer accumulator.  In one pair of MFMAs per run
// lane group g (lanes 16 g .. 16 g + 15) carries Q8_0 block 4 rho + g (32 bytes, 16 per
// MFMA) of row (lane & 15) in the B operand, and A row 4 i + p holds plane p of block i on
// lane group i only, so accumulator row 4 g + p is plane p of block g alone and the block's
// scale is applied afterwards (accumulator lane (n, g) holds rows 4 g .. 4 g + 3 of column
// n).  Rows 4 g + 3 read a zero plane.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int run_elem(int k, int wave, int lane) {
  return 512 * (k >> 1) + 128 * wave + 64 * (k & 1) + lane;
}

// This wave's NV tagged words of the runs it owns (NV = 2 per run) from buf into v[].  Every
// load is issued at once; each round re-issues the loads of the words not yet tagged, so a
// round costs one memory trip however many words are missing.  Returns false on a failed
// wait (the values are then meaningless).
template <int NV>
__device__ bool poll_runs(const uint64_t* buf, uint32_t tag, float (&v)[NV], const PersistParams& P) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t* p = buf + run_elem(0, wave, lane);
  uint64_t w[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) w[k] = peek(p + 512 * (k >> 1) + 64 * (k & 1));
  Spin sp;
  bool ok = true;
  while (true) {
    bool all = true;
#pragma unroll
    for (int k = 0; k < NV; ++k) all &= (uint32_t)(w[k] >> 32) == tag;
    if (all) break;
    if (sp.stop(P)) { ok = false; break; }
#pragma unroll
    for (int k = 0; k < NV; ++k)
      if ((uint32_t)(w[k] >> 32) != tag) w[k] = peek(p + 512 * (k >> 1) + 64 * (k & 1));
  }
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] = __uint_as_float((uint32_t)w[k]);
  return ok;
}

// The wave's runs as planes.  With s = 2^(6 - e), e the smallest exponent with
// sqrt(ssw) < 2^e (ssw = the wave's sum of squares, so every |x| < 2^e), x s = x0 + x1 / 128
// + x2 / 16384 + r with integers |x0|, |x1|, |x2| <= 64 and |r| <= 2^-15: an error of at
// most 2^-20 of the 2-norm of the wave's 4 D / 1024 runs.  Every step is exact in fp32
// except the three roundings to integers, done by adding 1.5 * 2^23 (which leaves the
// integer in the low mantissa bits, whose low byte is its two's complement).  Plane p goes to
// LDS bytes planes[p * D + element]; returns 1 / s.  Only this wave reads these bytes again.
template <int NV, int D>
__device__ __forceinline__ float quantize_runs(const float (&v)[NV], float ssw, int8_t* planes) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr float M = 12582912.0f;
  const int e = (__builtin_amdgcn_frexp_expf(ssw) + 1) >> 1;
  const float s = __builtin_amdgcn_ldexpf(1.0f, 6 - e);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const float x = v[k];
    const int i = run_elem(k, wave, lane);
    const float t0 = fmaf(x, s, M), q0 = t0 - M, r0 = fmaf(x, s, -q0);
    const float t1 = fmaf(r0, 128.0f, M), q1 = t1 - M, r1 = fmaf(r0, 128.0f, -q1);
    const float t2 = fmaf(r1, 128.0f, M);
    planes[i] = (int8_t)__float_as_uint(t0);
    planes[D + i] = (int8_t)__float_as_uint(t1);
    planes[2 * D + i] = (int8_t)__float_as_uint(t2);
  }
  return __builtin_amdgcn_ldexpf(1.0f, e - 6);
}

// The A operands of the wave's runs (see above): lane (m, g) reads plane m & 3 of block
// 4 rho + g when m >> 2 == g, else the zero plane 3.
template <int NT, int D>
__device__ __forceinline__ void run_operands(const int8_t* planes, i32x4 (&a)[NT][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int8_t* base = planes + ((m >> 2) == g ? (m & 3) : 3) * D + 128 * wave + 32 * g;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h) a[t][h] = *reinterpret_cast<const i32x4*>(base + 512 * t + 16 * h);
}

// Partial dots of the first ntiles (block-uniform) row tiles over the wave's runs: lane
// (n, g) returns, in y[tile], inv_s times the sum over runs t of the Q8_0 scale of block
// 4 (4 t + wave) + g of row 16 tile + n times that block's dot.
template <int NT, int NTILE>
__device__ __forceinline__ void mfma_tiles(const i32x4 (&a)[NT][2], const i32x4 (&w)[NTILE][NT][2],
                                           const uint32_t (&d)[NTILE][NT], float inv_s, int ntiles,
                                           float (&y)[NTILE]) {
  // every pair gets its own accumulator, so the MFMAs issue back to back before the first
  // epilogue waits for a result
  const i32x4 zero = {0, 0, 0, 0};
  i32x4 c[NTILE][NT];
#pragma unroll
  for (int tile = 0; tile < NTILE; ++tile)
    if (tile < ntiles) {
#pragma unroll
      for (int t = 0; t < NT; ++t) c[tile][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t][0], w[tile][t][0], zero, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < NT; ++t) c[tile][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t][1], w[tile][t][1], c[tile][t], 0, 0, 0);
    }
#pragma unroll
  for (int tile = 0; tile < NTILE; ++tile) {
    float acc = 0.0f;
    if (tile < ntiles) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const i32x4 r = c[tile][t];
        const float v = fmaf((float)(r[1] * 128 + r[2]), 1.0f / 16384.0f, (float)r[0]);
        acc = fmaf(h2f(d[tile][t]), v, acc);
      }
    }
    y[tile] = acc * inv_s;
  }
}

// The projection weights of a block's rows [p0, p1) (p0 a multiple of 16, at most kPTiles
// tiles of 16) of layer L in the operand layout above, read from the matrix-core order (every load
// is 1 KB of consecutive bytes): the wave's runs of row p0 + 16 tile + (lane & 15) and the
// scales of the lane's blocks.  Thread t < p1 - p0 also holds the conv taps and window of
// row p0 + t (q/k/v channels).
template <int U>
struct ProjRegs {
  i32x4 w[kPTiles][2 * U][2];   // [tile][run t][half]: 16 weight bytes (signed q)
  uint32_t d[kPTiles][2 * U];    // fp16 bits of the scale of block 4 (4 t + wave) + (lane >> 4)
  float4 cw;
  float z0, z1, z2;        // conv window, oldest first
};

// 16 weight bytes, streamed once per token.
__device__ __forceinline__ i32x4 wload_i(const int8_t* p) {
  return __builtin_nontemporal_load((const KDA_GLOBAL i32x4*)p);
}

// Tile `tile` (16 rows) of a matrix in the matrix-core order: this lane's 2 x 2U chunks and
// its 2U scales.
template <int U>
__device__ __forceinline__ void load_tile(const int8_t* w, const uint16_t* d, int tile,
                                          i32x4 (&rw)[2 * U][2], uint32_t (&rd)[2 * U]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int8_t* wb = w + ((size_t)(tile * 4 + wave) * (4 * U) * 64 + lane) * 16;
#pragma unroll
  for (int t = 0; t < 2 * U; ++t) {
    rw[t][0] = wload_i(wb + (2 * t) * 1024);
    rw[t][1] = wload_i(wb + (2 * t + 1) * 1024);
  }
  const uint16_t* db = d + ((size_t)(tile * 4 + wave) * 64 + lane) * (2 * U);
  if constexpr (U == 1) {
    const uint32_t v = *(const KDA_GLOBAL uint32_t*)db;
    rd[0] = v & 0xffffu;
    rd[1] = v >> 16;
  } else {
#pragma unroll
    for (int q = 0; q < U / 2; ++q) {
      const u32x2 v = *(const KDA_GLOBAL u32x2*)(db + 4 * q);
      rd[4 * q] = v[0] & 0xffffu;
      rd[4 * q + 1] = v[0] >> 16;
      rd[4 * q + 2] = v[1] & 0xffffu;
      rd[4 * q + 3] = v[1] >> 16;
    }
  }
}

template <int U>
__device__ __forceinline__ void issue_proj(const PersistParams& P, GLayer& L, const float* win,
                                           int p0, int p1, ProjRegs<U>& R) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int tile = 0; tile < kPTiles; ++tile) {
#pragma unroll
    for (int t = 0; t < 2 * U; ++t) {
      R.w[tile][t][0] = R.w[tile][t][1] = i32x4{0, 0, 0, 0};
      R.d[tile][t] = 0;
    }
    if (p0 + 16 * tile < p1) load_tile<U>(L.pw, L.pd, p0 / 16 + tile, R.w[tile], R.d[tile]);
  }
  const int myrow = p0 + tid;
  R.cw = make_float4(0.f, 0.f, 0.f, 0.f);
  R.z0 = R.z1 = R.z2 = 0.0f;
  if (myrow < p1 && myrow < P.C) {
    R.cw = gload4(L.conv_w + (size_t)myrow * 4);
    R.z0 = *gp(win + myrow);
    R.z1 = *gp(win + P.C + myrow);
    R.z2 = *gp(win + 2 * P.C + myrow);
  }
}

// The output-projection weights of band ob (rows [32 ob, 32 ob + 32)), as for ProjRegs (the
// input is the V = D head outputs).
template <int U>
struct OutRegs {
  i32x4 w[kOTiles][2 * U][2];
  uint32_t d[kOTiles][2 * U];
};

template <int U>
__device__ __forceinline__ void issue_out(GLayer& L, int ob, OutRegs<U>& R) {
#pragma unroll
  for (int tile = 0; tile < kOTiles; ++tile) load_tile<U>(L.ow, L.od, kOTiles * ob + tile, R.w[tile], R.d[tile]);
}

// A head block owns value columns [half * kHCols, + kHCols) of head h.  Its registers: wave
// w's state tile (rows 8 (lane & 15) .. + 8, columns half * kHCols + 16 w + 4 (lane >> 4)
// .. + 4) and the B operands of its three gate tiles (below): F_b rows 16 w and 16 (w + 4) of
// the head (alpha), G_b rows half * kHCols + 16 w of the head (output gate).
template <int CPR>   // CPR = rank / 16
struct HeadRegs {
  float4 st[8];
  i32x4 bw[3][2];          // [tile][half]: the lane's 16 bytes of Q8_0 block lane >> 4 of row lane & 15
  uint32_t bd[3];          // fp16 bits of that block's scale
  float dtb;               // dt_bias of the alpha row this lane finishes (lane groups 0 and 1)
  float4 onw;
  float ea;                // A_log[h], exponentiated when used
};

// The gate tiles in the order gate_order_kernel writes them: tile tau of a matrix is 16 rank
// bytes, lane (n, g) reads chunk (half, g, n) when g < rank / 32 (zero otherwise).
template <int CPR>
__device__ __forceinline__ void load_gate_tile(const int8_t* w, const uint16_t* d, int tau,
                                               i32x4 (&rw)[2], uint32_t& rd) {
  constexpr int NB = CPR / 2, rank = CPR * 16;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  rw[0] = rw[1] = i32x4{0, 0, 0, 0};
  rd = 0;
  if (g < NB) {
    const int8_t* b = w + (size_t)tau * 16 * rank + (g * 16 + n) * 16;
    rw[0] = wload_i(b);
    rw[1] = wload_i(b + NB * 256);
    rd = *(const KDA_GLOBAL uint16_t*)(d + ((size_t)tau * NB + g) * 16 + n);
  }
}

template <int CPR>
__device__ __forceinline__ void issue_head(const PersistParams& P, GLayer& L, const float* Sl,
                                           int h, int half, HeadRegs<CPR>& R) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = half * kHCols + wave * 16 + (lane >> 4) * 4, r0 = (lane & 15) * 8;
  const float* Sb = Sl + (size_t)h * kHD * kHD + j;
#pragma unroll
  for (int i = 0; i < 8; ++i) R.st[i] = gload4(Sb + (size_t)(r0 + i) * kHD);
  constexpr int kTilesPerHead = kHD / 16;
  load_gate_tile<CPR>(L.fbw, L.fbd, h * kTilesPerHead + wave, R.bw[0], R.bd[0]);
  load_gate_tile<CPR>(L.fbw, L.fbd, h * kTilesPerHead + wave + 4, R.bw[1], R.bd[1]);
  load_gate_tile<CPR>(L.gbw, L.gbd, h * kTilesPerHead + half * (kHCols / 16) + wave, R.bw[2], R.bd[2]);
  const int g = lane >> 4;
  R.dtb = g < 2 ? *gp(L.dt_bias + h * kHD + 16 * (wave + 4 * g) + (lane & 15)) : 0.0f;
  R.onw = make_float4(1.f, 1.f, 1.f, 1.f);
  if (L.o_norm_w) R.onw = gload4(L.o_norm_w + j);
  R.ea = *gp(L.a_log + h);
}

// LDS of one block.
struct Smem {
  alignas(16) int8_t planes[4 * 2048];  // [4][D] input planes of the matrix-core dots; [3] = 0
  alignas(16) float part[48 * 16];      // [row][wave * 4 + g] partial dots of the block's rows
  float red[8];
  float xres[32];          // an output block's residual rows
  alignas(16) float s_in[1024];  // head block: q | k | v | f_lr | g_lr | beta
  alignas(16) float s_al[kHD];     // head block: alpha rows
  alignas(16) float s_gt[kHCols];  // head block: output-gate columns
  alignas(16) int8_t gpl[4 * 256];   // head block: planes of [f_lr | g_lr]; [3] = 0
  float ginv[8];                     // head block: 1 / scale of each 32-element block of them
  alignas(16) int any[2][4];       // block_any: per-wave votes, two alternating sets
#ifdef KDA_TRACE
  uint64_t stamps[kTraceLayers][kTraceSlots];
#endif
};

// Block-wide OR of pred (every thread of the block calls it): each wave's vote goes to LDS,
// one barrier, every thread reads the four votes.  Consecutive calls of a block use the two
// vote sets alternately (`set`), since no wave can be more than one call ahead of another.
// Unlike __syncthreads_or (which reads the block size from memory) it issues no global load, which would make it wait for every load
// still in flight.
__device__ __forceinline__ bool block_any(Smem& sm, int set, int pred) {
  const bool any = __builtin_amdgcn_ballot_w64(pred != 0) != 0;
  if ((threadIdx.x & 63) == 0) sm.any[set][threadIdx.x >> 6] = any;
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
  const int4 v = *reinterpret_cast<const int4*>(sm.any[set]);
  // the same value in every lane: said so, so that the branches on it (and the layer loops
  // they leave) stay scalar
  return __builtin_amdgcn_readfirstlane(v.x | v.y | v.z | v.w) != 0;
}

// Static roles of block b: [0, kHSplit H) heads, then P.o_blocks output bands of 32 rows,
// then the projection blocks: q/k/v rows 48 per block to the first q_blocks, then the
// low-rank and beta rows one tile of 16 per block, so that the rows the head blocks need
// first (their gates) are finished early; blocks past them have no rows.
struct Roles {
  int p0, p1;              // this block's projection rows
  int ob, or0;             // output band index and its first row
};

__device__ __forceinline__ Roles make_roles(const PersistParams& P) {
  Roles R;
  const int b = blockIdx.x - P.o_first_block - P.o_blocks;
  const int C = P.C;
  if (b < 0) {
    R.p0 = R.p1 = 0;
  } else if (b < P.q_blocks) {
    R.p0 = min(C, b * 16 * kPTiles);
    R.p1 = min(C, R.p0 + 16 * kPTiles);
  } else {
    R.p0 = min(P.proj_rows, C + (b - P.q_blocks) * 16);
    R.p1 = min(P.proj_rows, R.p0 + 16);
  }
  R.ob = (int)blockIdx.x - P.o_first_block;
  R.or0 = R.ob * 16 * kOTiles;
  return R;
}

// P phase of layer l (projection blocks): wait for x_l, RMSNorm, this block's projection
// rows, conv epilogue; the next layer's slice is requested as soon as this one is used.
// Returns false on a failed wait.
template <int U>
__device__ __forceinline__ bool phase_p(const PersistParams& P, Smem& sm, const Roles& R, int l,
                                        uint32_t tag, ProjRegs<U>& pr) {
  constexpr int D = 1024 * U, NV = 4 * U, NT = 2 * U;
  GLayer* Lt = (GLayer*)P.layers;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int C = P.C;
  float* win = P.win + (size_t)l * 3 * C;
  float v[NV];
  int bad = 0;
  KDA_STAMP(l, 0);
  if (l == 0) {
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = *gp(P.x_in + run_elem(k, wave, lane));
  } else {
    // x_l: once the first head block of layer l - 1 has flagged (the O blocks post x 1.5-2 us
    // later), poll the tagged words of the wave's runs: already polling when the fresh words
    // land, the fetch that brings them is also their detection
    uint32_t pend[3] = {0u, 0u, 0u};
    if (block_any(sm, 0, wave0_wait_flags(P, kFlagH, kHSplit * P.H, tag - 1u, pend))) return false;
    KDA_STAMP(l, 1);
    bad = !poll_runs<NV>(P.xbuf + (size_t)((l - 1) & 1) * D, tag - 1u, v, P);
    keep_live(pend);
    KDA_STAMP(l, 2);
  }
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < NV; ++k) ss = fmaf(v[k], v[k], ss);
  ss = wave_sum(ss);
  if (lane == 0) sm.red[wave] = ss;
  const float inv_s = quantize_runs<NV, D>(v, ss, sm.planes);
  KDA_STAMP(l, 6);
  i32x4 a[NT][2];
  run_operands<NT, D>(sm.planes, a);
  KDA_STAMP(l, 7);
  const int rows = R.p1 - R.p0, ntiles = (rows + 15) >> 4;
  float y[kPTiles];
  mfma_tiles<NT, kPTiles>(a, pr.w, pr.d, inv_s, ntiles, y);
#pragma unroll
  for (int tile = 0; tile < kPTiles; ++tile)
    if (tile < ntiles) sm.part[(16 * tile + (lane & 15)) * 16 + 4 * wave + (lane >> 4)] = y[tile];
  KDA_STAMP(l, 3);
  if (block_any(sm, 1, bad)) return false;
  KDA_STAMP(l, 4);
  // thread t finishes row p0 + t: RMSNorm scale, conv + SiLU + window roll for q/k/v channels
  if (tid < rows) {
    const int row = R.p0 + tid;
    const float4* q = reinterpret_cast<const float4*>(sm.part + 16 * tid);
    const float4 s0 = q[0], s1 = q[1], s2 = q[2], s3 = q[3];
    const float sum = ((s0.x + s0.y) + (s0.z + s0.w)) + ((s1.x + s1.y) + (s1.z + s1.w)) +
                      ((s2.x + s2.y) + (s2.z + s2.w)) + ((s3.x + s3.y) + (s3.z + s3.w));
    const float sc = rsq_hw((sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3]) / (float)D + P.eps);
    const float pre = sum * sc;
    float o = pre;
    if (row < C) {
      const float cv = pr.cw.x * pr.z0 + pr.cw.y * pr.z1 + pr.cw.z * pr.z2 + pr.cw.w * pre;
      o = cv * sigmoid_hw(cv);
    }
    put(P.pbuf + row, tag, o);
    // off the critical path: roll the conv window
    if (row < C) {
      float* z = win + row;
      *gpw(z) = pr.z1;
      *gpw(z + C) = pr.z2;
      *gpw(z + 2 * C) = pre;
    }
  }
  KDA_STAMP(l, 5);
  if (l + 1 < P.n_layers) {
    hold_prefetch();
    issue_proj<U>(P, Lt[l + 1], win + 3 * C, R.p0, R.p1, pr);
  }
  return true;
}

// H phase of layer l for head block b = half * H + h: gates, delta rule on its value columns,
// the gated outputs before the head's RMSNorm and per-wave partial sums of o^2 (the output
// blocks finish the norm, since it spans both blocks of the head).
template <int CPR>
__device__ __forceinline__ bool phase_h(const PersistParams& P, Smem& sm, int l, uint32_t tag,
                                        HeadRegs<CPR>& hr) {
  GLayer* Lt = (GLayer*)P.layers;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int dk = kHD, dv = kHD, rank = CPR * 16;
  const int H = P.H, C = P.C, K = H * dk;
  const int h = blockIdx.x % H, half = blockIdx.x / H;
  float* Sl = P.S + (size_t)l * H * dk * dv;
  // the head's inputs are polled word by word from the start of the layer (32 blocks of
  // ~4.6 KB a round, no flag first: the low-rank rows land early)
  // inputs: q [dk] | k [dk] | v [kHCols] | f_lr [rank] | g_lr [rank] | beta  (<= 3 per thread)
  constexpr int n_in = 2 * dk + kHCols + 2 * rank + 1;
  static_assert(n_in <= 3 * kPT, "head inputs");
  // every input is requested at once; the low-rank rows and beta (finished first by their
  // projection blocks) are waited for before the gates, q / k / v after them
  constexpr int i_lr = 2 * dk + kHCols;          // first low-rank input
  KDA_STAMP(l, 0);
  uint64_t w[3];
  const uint64_t* src[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int i = min(tid + k * kPT, n_in - 1);
    int r;
    if (i < dk) r = h * dk + i;
    else if (i < 2 * dk) r = K + h * dk + (i - dk);
    else if (i < 2 * dk + kHCols) r = 2 * K + h * dv + half * kHCols + (i - 2 * dk);
    else if (i < 2 * dk + kHCols + 2 * rank) r = C + (i - 2 * dk - kHCols);
    else r = C + 2 * rank + h;
    src[k] = P.pbuf + r;
    w[k] = peek(src[k]);
  }
  // wait until the slots selected by `lr` (low-rank ones, or the others) carry the tag;
  // every round re-reads all three slots, so its loads go out together
  auto wait_slots = [&](bool lr) {
    Spin sp;
    while (true) {
      bool all = true;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int i = tid + k * kPT;
        const bool want = i < n_in && ((i >= i_lr) == lr);
        all &= !want || (uint32_t)(w[k] >> 32) == tag;
      }
      if (all) return true;
      if (sp.stop(P)) return false;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const uint64_t r = peek(src[k]);
        w[k] = (uint32_t)(w[k] >> 32) == tag ? w[k] : r;
      }
    }
  };
  {
    const int bad = !wait_slots(true);
    KDA_STAMP(l, 1);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int i = tid + k * kPT;
      if (i >= i_lr && i < n_in) sm.s_in[i] = __uint_as_float((uint32_t)w[k]);
    }
    // element e = i - i_lr of [f_lr | g_lr] is in this thread's slot 1 or 2, and each block of
    // 32 of them (the Q8_0 blocks of F_b and G_b rows) fills half a wave, which turns it into
    // three signed 7-bit planes under the block's own power-of-two scale (as the projection
    // inputs, with a block in place of a wave's runs)
    static_assert(i_lr % 64 == 0 && (2 * rank) % 64 == 0, "whole waves per low-rank block pair");
    {
      const int e1 = tid + kPT - i_lr, e2 = e1 + kPT;
      const bool in1 = e1 >= 0 && e1 < 2 * rank, in2 = e2 >= 0 && e2 < 2 * rank;  // wave-uniform
      if (in1 || in2) {
        const int e = in1 ? e1 : e2;
        const float u = __uint_as_float((uint32_t)(in1 ? w[1] : w[2]));
        float ss = sum16(u * u);
        ss += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(ss), 0x401F));  // lane ^ 16
        constexpr float M = 12582912.0f;
        const int ex = (__builtin_amdgcn_frexp_expf(ss) + 1) >> 1;
        const float sc = __builtin_amdgcn_ldexpf(1.0f, 6 - ex);
        const float t0 = fmaf(u, sc, M), q0 = t0 - M, r0 = fmaf(u, sc, -q0);
        const float t1 = fmaf(r0, 128.0f, M), q1 = t1 - M, r1 = fmaf(r0, 128.0f, -q1);
        const float t2 = fmaf(r1, 128.0f, M);
        sm.gpl[e] = (int8_t)__float_as_uint(t0);
        sm.gpl[256 + e] = (int8_t)__float_as_uint(t1);
        sm.gpl[512 + e] = (int8_t)__float_as_uint(t2);
        if ((e & 31) == 0) sm.ginv[e >> 5] = __builtin_amdgcn_ldexpf(1.0f, ex - 6);
      }
    }
    if (block_any(sm, 0, bad)) return false;
    KDA_STAMP(l, 2);
  }
  // request the q/k/v words again now: the round trip overlaps the gates below, and the
  // replies are merged only after them.  Only slots that hold q/k/v inputs are requested: a
  // load whose result is never used frees its register at once, and reusing that register
  // makes the code wait for the load.
  uint64_t again[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    again[k] = w[k];
    if (k * kPT < i_lr && tid + k * kPT < i_lr) again[k] = peek(src[k]);
  }
  const float* s_q = sm.s_in;
  const float* s_k = sm.s_in + dk;
  const float* s_v = sm.s_in + 2 * dk;
  const float beta = sigmoid_hw(sm.s_in[2 * dk + kHCols + 2 * rank]);
  // alpha = exp(-exp(A_log) softplus(F_b f_lr + dt_bias)) (KDA; the lower-bounded gate:
  // exp(lb sigmoid(-(F_b f_lr + dt_bias) A_log)), A_log as given), gate = sigmoid(G_b g_lr), on the
  // int8 matrix cores as the projections: A row 4 i + p holds plane p of block i on lane
  // group i, B the tile's Q8_0 bytes, so accumulator lane (n, g) holds block g's three plane
  // dots for row n.  Each block's two scales are applied there and the four lane groups
  // summed (the same total in every group); lane group 0 then finishes alpha row 16 w + n,
  // group 1 alpha row 16 (w + 4) + n, group 2 gate column 16 w + n.
  {
    constexpr int NB = CPR / 2;
    const int m = lane & 15, g = lane >> 4;
    const int8_t* pa = sm.gpl + ((m >> 2) == g && g < NB ? (m & 3) : 3) * 256 + 32 * g;
    const i32x4 af0 = *reinterpret_cast<const i32x4*>(pa);
    const i32x4 af1 = *reinterpret_cast<const i32x4*>(pa + 16);
    const i32x4 ag0 = *reinterpret_cast<const i32x4*>(pa + rank);
    const i32x4 ag1 = *reinterpret_cast<const i32x4*>(pa + rank + 16);
    const i32x4 zero = {0, 0, 0, 0};
    i32x4 c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(af0, hr.bw[0][0], zero, 0, 0, 0);
    i32x4 c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(af0, hr.bw[1][0], zero, 0, 0, 0);
    i32x4 c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ag0, hr.bw[2][0], zero, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(af1, hr.bw[0][1], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(af1, hr.bw[1][1], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ag1, hr.bw[2][1], c2, 0, 0, 0);
    // (lane groups past the last block have zero weights and take no scale)
    const float sf = g < NB ? sm.ginv[g] : 0.0f, sg = g < NB ? sm.ginv[NB + g] : 0.0f;
    auto planes = [](const i32x4 r) { return fmaf((float)(r[1] * 128 + r[2]), 1.0f / 16384.0f, (float)r[0]); };
    float y0 = h2f(hr.bd[0]) * sf * planes(c0);
    float y1 = h2f(hr.bd[1]) * sf * planes(c1);
    float y2 = h2f(hr.bd[2]) * sg * planes(c2);
    y0 += __shfl_xor(y0, 16);
    y1 += __shfl_xor(y1, 16);
    y2 += __shfl_xor(y2, 16);
    y0 += __shfl_xor(y0, 32);
    y1 += __shfl_xor(y1, 32);
    y2 += __shfl_xor(y2, 32);
    const float pre = g == 0 ? y0 : g == 1 ? y1 : y2;
    const float al = P.gate_safe ? exp_hw(P.gate_lb * sigmoid_hw(-(pre + hr.dtb) * hr.ea))
                                 : exp_hw(-exp_hw(hr.ea) * softplus_hw(pre + hr.dtb));
    const float gt = sigmoid_hw(pre);   // (alpha and gate in every lane: no lane branch)
    if (g < 2) sm.s_al[16 * (wave + 4 * g) + m] = al;
    else if (g == 2) sm.s_gt[16 * wave + m] = gt;
  }
  KDA_STAMP(l, 3);
  {
    // q, k, v
#pragma unroll
    for (int k = 0; k < 3; ++k)
      if (k * kPT < i_lr) w[k] = (uint32_t)(w[k] >> 32) == tag ? w[k] : again[k];
    const int bad = !wait_slots(false);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int i = tid + k * kPT;
      if (i < i_lr) sm.s_in[i] = __uint_as_float((uint32_t)w[k]);
    }
    if (block_any(sm, 1, bad)) return false;
    KDA_STAMP(l, 4);
  }
  // delta rule: lane (rg, cq) holds rows 8 rg .. + 8 of columns jl .. + 4 (block-local jl)
  const int rg = lane & 15, cq = lane >> 4;
  const int jl = wave * 16 + cq * 4, j = half * kHCols + jl, r0 = rg * 8;
  float4 qv[2], kv[2], av[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    qv[k] = reinterpret_cast<const float4*>(s_q + r0)[k];
    kv[k] = reinterpret_cast<const float4*>(s_k + r0)[k];
    av[k] = reinterpret_cast<const float4*>(sm.s_al + r0)[k];
  }
  const float4 vv = *reinterpret_cast<const float4*>(s_v + jl);
  const float4 gv = *reinterpret_cast<const float4*>(sm.s_gt + jl);
  const float* qa = reinterpret_cast<const float*>(qv);
  const float* ka = reinterpret_cast<const float*>(kv);
  const float* aa = reinterpret_cast<const float*>(av);
  float aq = 0.0f, ak = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    aq += qa[i] * qa[i];
    ak += ka[i] * ka[i];
  }
  const float inv_q = P.q_scale * rsq_hw(sum16(aq) + P.l2_eps);
  const float inv_k = rsq_hw(sum16(ak) + P.l2_eps);
  float e0 = 0.f, e1 = 0.f, e2 = 0.f, e3 = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = aa[i], kk = ka[i] * inv_k;
    float4& s = hr.st[i];
    s.x *= a; s.y *= a; s.z *= a; s.w *= a;
    e0 += s.x * kk; e1 += s.y * kk; e2 += s.z * kk; e3 += s.w * kk;
  }
  e0 = sum16(e0); e1 = sum16(e1); e2 = sum16(e2); e3 = sum16(e3);
  KDA_STAMP(l, 6);
  const float d0 = beta * (vv.x - e0), d1 = beta * (vv.y - e1);
  const float d2 = beta * (vv.z - e2), d3 = beta * (vv.w - e3);
  float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float kk = ka[i] * inv_k, qq = qa[i] * inv_q;
    float4& s = hr.st[i];
    s.x += kk * d0; s.y += kk * d1; s.z += kk * d2; s.w += kk * d3;
    o0 += s.x * qq; o1 += s.y * qq; o2 += s.z * qq; o3 += s.w * qq;
  }
  o0 = sum16(o0); o1 = sum16(o1); o2 = sum16(o2); o3 = sum16(o3);
  KDA_STAMP(l, 7);
  // gated outputs (the norm scale comes later) and this wave's partial sum of o^2
  if (rg == 0) {
    uint64_t* ob = P.obuf + h * dv + j;
    put(ob + 0, tag, o0 * hr.onw.x * gv.x);
    put(ob + 1, tag, o1 * hr.onw.y * gv.y);
    put(ob + 2, tag, o2 * hr.onw.z * gv.z);
    put(ob + 3, tag, o3 * hr.onw.w * gv.w);
  }
  const int qb = __float_as_int(o0 * o0 + o1 * o1 + o2 * o2 + o3 * o3);   // same on a row's lanes
  const float tot = (__int_as_float(__builtin_amdgcn_readlane(qb, 0)) + __int_as_float(__builtin_amdgcn_readlane(qb, 16))) +
                    (__int_as_float(__builtin_amdgcn_readlane(qb, 32)) + __int_as_float(__builtin_amdgcn_readlane(qb, 48)));
  if (lane == 0) {
    put(P.obuf + P.H * dv + (h * kHSplit + half) * 4 + wave, tag, tot);
    if (wave == 0) put(flag_slot(P, kFlagH, blockIdx.x), tag, 0.0f);
  }
  KDA_STAMP(l, 5);
  // off the critical path: write the state back, request the next layer's
  float* Sb = Sl + (size_t)h * dk * dv + j;
#pragma unroll
  for (int i = 0; i < 8; ++i) gstore4(Sb + (size_t)(r0 + i) * dv, hr.st[i]);
  if (l + 1 < P.n_layers) {
    hold_prefetch();
    issue_head<CPR>(P, Lt[l + 1], Sl + (size_t)H * dk * dv, h, half, hr);
  }
  // (the next layer's first wait is a barrier, so LDS is not rewritten while still read)
  return true;
}

// O phase of layer l: this band's output-projection rows of the normalised heads, plus the
// residual; the last layer also writes the output row.  The heads' RMSNorm scales come from
// the per-wave partial sums of o^2 that the head blocks post after their outputs; run t of
// wave w is head 4 t + w, so each wave needs the scales of its own heads only.
template <int U>
__device__ __forceinline__ bool phase_o(const PersistParams& P, Smem& sm, const Roles& R, int l,
                                        uint32_t tag, OutRegs<U>& orr) {
  constexpr int D = 1024 * U, NV = 4 * U, NT = 2 * U;
  constexpr int kParts = kHSplit * 4;                // o^2 partials per head
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // once the first head block has posted, fetch the output words of the wave's heads and
  // their partials (lane kParts t + i: partial i of head 4 t + wave)
  uint32_t pend[3] = {0u, 0u, 0u};
  KDA_STAMP(l, 0);
  if (block_any(sm, 0, wave0_wait_flags(P, kFlagH, kHSplit * P.H, tag, pend))) return false;
  KDA_STAMP(l, 1);
  const bool has = lane < kParts * NT;
  const uint64_t* src = P.obuf + D + (4 * (has ? lane / kParts : 0) + wave) * kParts + lane % kParts;
  uint64_t pw = has ? peek(src) : tagged(tag, 0.0f);
  float v[NV];
  int bad = !poll_runs<NV>(P.obuf, tag, v, P);
  {
    Spin sp;
    while (!bad && (uint32_t)(pw >> 32) != tag) {
      if (sp.stop(P)) bad = 1;
      else pw = peek(src);
    }
  }
  keep_live(pend);
  KDA_STAMP(l, 2);
  // the normalised heads (run t = head 4 t + wave), then their planes
  // lane kParts t ends up with head t's sum of squares; every lane computes a scale, lane
  // kParts t's is head t's
  const float psum = group_sum(__uint_as_float((uint32_t)pw), kParts);
  const int hsl = __float_as_int(rsq_hw(psum / (float)kHD + P.eps));
  float ss = 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float hs = __int_as_float(__builtin_amdgcn_readlane(hsl, kParts * t));
    v[2 * t] *= hs;
    v[2 * t + 1] *= hs;
    ss = fmaf(v[2 * t], v[2 * t], ss);
    ss = fmaf(v[2 * t + 1], v[2 * t + 1], ss);
  }
  const float inv_s = quantize_runs<NV, D>(v, wave_sum(ss), sm.planes);
  KDA_STAMP(l, 6);
  i32x4 a[NT][2];
  run_operands<NT, D>(sm.planes, a);
  KDA_STAMP(l, 7);
  float y[kOTiles];
  mfma_tiles<NT, kOTiles>(a, orr.w, orr.d, inv_s, kOTiles, y);
#pragma unroll
  for (int tile = 0; tile < kOTiles; ++tile)
    sm.part[(16 * tile + (lane & 15)) * 16 + 4 * wave + (lane >> 4)] = y[tile];
  KDA_STAMP(l, 3);
  if (block_any(sm, 1, bad)) return false;
  KDA_STAMP(l, 4);
  if (tid < 16 * kOTiles) {
    const int row = R.or0 + tid;
    const float4* q = reinterpret_cast<const float4*>(sm.part + 16 * tid);
    const float4 s0 = q[0], s1 = q[1], s2 = q[2], s3 = q[3];
    const float sum = ((s0.x + s0.y) + (s0.z + s0.w)) + ((s1.x + s1.y) + (s1.z + s1.w)) +
                      ((s2.x + s2.y) + (s2.z + s2.w)) + ((s3.x + s3.y) + (s3.z + s3.w));
    const float xn = sm.xres[tid] + sum;
    sm.xres[tid] = xn;     // the band's residual rows of the next layer
    put(P.xbuf + (size_t)(l & 1) * D + row, tag, xn);
    if (l + 1 == P.n_layers) *gpw(P.y_out + row) = xn;
  }
  KDA_STAMP(l, 5);
  return true;
}

// The layer loop of one role: ROLE 0 projection block, 1 head block, 2 output band.  Each
// role keeps only its own prefetch registers live.  Prefetches are issued right after a phase
// that is followed by a long wait, never just before a poll on the critical path (a poll's
// load completes only after the loads issued before it).
template <int U, int CPR, int ROLE>
__device__ __forceinline__ void run_role(const PersistParams& P, Smem& sm, int err0) {
  GLayer* Lt = (GLayer*)P.layers;
  const Roles R = make_roles(P);
  const uint32_t tag0 = P.epoch * (uint32_t)P.n_layers;
  const int tid = threadIdx.x;
  if constexpr (ROLE == 1) {
    sm.gpl[3 * 256 + tid] = 0;   // the zero plane of the gate inputs
    HeadRegs<CPR> hr;
    issue_head<CPR>(P, Lt[0], P.S, blockIdx.x % P.H, blockIdx.x / P.H, hr);
    if (__builtin_amdgcn_readfirstlane(err0)) return;
    for (int l = 0; l < P.n_layers; ++l)
      if (!phase_h<CPR>(P, sm, l, tag0 + (uint32_t)l + 1u, hr)) return;
    return;
  }
  // the zero plane of the wave's runs (no other wave reads them)
#pragma unroll
  for (int k = 0; k < 4 * U; ++k) sm.planes[3 * 1024 * U + run_elem(k, tid >> 6, tid & 63)] = 0;
  if constexpr (ROLE == 2) {
    OutRegs<U> orr;
    issue_out<U>(Lt[0], R.ob, orr);
    if (__builtin_amdgcn_readfirstlane(err0)) return;
    if (tid < 16 * kOTiles) sm.xres[tid] = *gp(P.x_in + R.or0 + tid);
    for (int l = 0; l < P.n_layers; ++l) {
      if (!phase_o<U>(P, sm, R, l, tag0 + (uint32_t)l + 1u, orr)) return;
      if (l + 1 < P.n_layers) {
        hold_prefetch();
        // (the layer index is uniform; said so, so that its table entry is a scalar load)
        issue_out<U>(Lt[__builtin_amdgcn_readfirstlane(l + 1)], R.ob, orr);
      }
    }
  } else {
    // a block left without projection rows has nothing to do: no phase waits for it, and
    // it must not fall layers behind while it reads the residual stream
    if (R.p1 <= R.p0) return;
    ProjRegs<U> pr;
    issue_proj<U>(P, Lt[0], P.win, R.p0, R.p1, pr);
    if (__builtin_amdgcn_readfirstlane(err0)) return;
    for (int l = 0; l < P.n_layers; ++l)
      if (!phase_p<U>(P, sm, R, l, tag0 + (uint32_t)l + 1u, pr)) return;
  }
}

// U = D / 1024 (16-byte chunks per lane per row), CPR = rank / 16
#ifdef KDA_TRACE
__device__ uint64_t g_trace[kMaxPersistBlocks * kTraceLayers * kTraceSlots];
#endif

template <int U, int CPR>
__global__ __launch_bounds__(kPT, 1) void decode_persistent_kernel(const PersistParams P) {
  __shared__ Smem sm;
  const int b = blockIdx.x;
#ifdef KDA_TRACE
  for (int i = threadIdx.x; i < kTraceLayers * kTraceSlots; i += kPT) (&sm.stamps[0][0])[i] = 0;
  __syncthreads();
#endif
  // a model whose earlier step failed a wait keeps its error word until the host resets it:
  // every block then leaves before it touches the state, the window or the output (the
  // word is requested first and looked at after the block's first weight requests)
  const int err0 = err_set(P);
  if (b < kHSplit * P.H) run_role<U, CPR, 1>(P, sm, err0);
  else if (b >= P.o_first_block && b < P.o_first_block + P.o_blocks) run_role<U, CPR, 2>(P, sm, err0);
  else run_role<U, CPR, 0>(P, sm, err0);
#ifdef KDA_TRACE
  __syncthreads();
  for (int i = threadIdx.x; i < kTraceLayers * kTraceSlots; i += kPT)
    g_trace[(size_t)b * kTraceLayers * kTraceSlots + i] = (&sm.stamps[0][0])[i];
#endif
}

// One thread per 16-byte chunk of the matrix-core order (persist.h): chunk
// c = (((tile * 4 + wave) * 2U + t) * 2 + h) * 64 + lane holds row 16 tile + (lane & 15),
// columns 128 (4 t + wave) + 32 (lane >> 4) + 16 h .. + 16, flipped from q + 128 to q; the
// h = 0 chunk also places the scale of that row's block 16 t + 4 wave + (lane >> 4).
template <int U>
__global__ void mma_order_kernel(const MmaSource src, int rows, int8_t* __restrict__ w,
                                 uint16_t* __restrict__ d, int64_t nchunks) {
  constexpr int D = 1024 * U;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nchunks) return;
  const int lane = (int)(c % 64);
  int64_t r = c / 64;
  const int h = (int)(r % 2);
  r /= 2;
  const int t = (int)(r % (2 * U));
  r /= 2 * U;
  const int wave = (int)(r % 4);
  const int64_t tile = r / 4;
  const int64_t row = tile * 16 + (lane & 15);
  const int col = 128 * (4 * t + wave) + 32 * (lane >> 4) + 16 * h;
  u32x4 out = {0u, 0u, 0u, 0u};
  uint16_t sc = 0;
  if (row < rows) {
    int seg = 0;
    for (int i = 1; i < src.nseg; ++i)
      if (row >= src.first[i]) seg = i;
    const int64_t rr = row - src.first[seg];
    out = *reinterpret_cast<const u32x4*>(src.w[seg] + rr * D + col) ^ 0x80808080u;
    sc = __half_as_ushort(src.d[seg][rr * (D / 32) + col / 32]);
  }
  *reinterpret_cast<u32x4*>(w + c * 16) = out;
  if (h == 0) d[((tile * 4 + wave) * 64 + lane) * (2 * U) + t] = sc;
}

hipError_t launch_mma_order(const MmaSource& src, int rows, int D, int8_t* w, uint16_t* d,
                            hipStream_t s) {
  if ((D != 1024 && D != 2048) || rows < 1 || src.nseg < 1 || src.nseg > 6) return hipErrorInvalidValue;
  const int64_t n = (int64_t)((rows + 15) / 16) * D;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (D == 1024) mma_order_kernel<1><<<blocks, 256, 0, s>>>(src, rows, w, d, n);
  else mma_order_kernel<2><<<blocks, 256, 0, s>>>(src, rows, w, d, n);
  return hipGetLastError();
}

// One thread per 16-byte chunk of the gate order (persist.h): chunk
// c = ((tile * 2 + h) * NB + g) * 16 + n holds row 16 tile + n, bytes [32 g + 16 h, + 16),
// flipped from q + 128 to q; the h = 0 chunk also places that block's scale.
__global__ void gate_order_kernel(const uint8_t* __restrict__ src_w, const __half* __restrict__ src_d,
                                  int rank, int8_t* __restrict__ w, uint16_t* __restrict__ d,
                                  int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nchunks) return;
  const int nb = rank / 32;
  const int n = (int)(c % 16);
  int64_t r = c / 16;
  const int g = (int)(r % nb);
  r /= nb;
  const int h = (int)(r % 2);
  const int64_t tile = r / 2;
  const int64_t row = tile * 16 + n;
  const u32x4 v = *reinterpret_cast<const u32x4*>(src_w + row * rank + 32 * g + 16 * h);
  *reinterpret_cast<u32x4*>(w + c * 16) = v ^ 0x80808080u;
  if (h == 0) d[(tile * nb + g) * 16 + n] = __half_as_ushort(src_d[row * nb + g]);
}

hipError_t launch_gate_order(const uint8_t* w_src, const __half* d_src, int rows, int rank,
                             int8_t* w, uint16_t* d, hipStream_t s) {
  if ((rank != 32 && rank != 64 && rank != 128) || rows < 16 || rows % 16 != 0) return hipErrorInvalidValue;
  const int64_t n = (int64_t)rows * rank / 16;
  gate_order_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(w_src, d_src, rank, w, d, n);
  return hipGetLastError();
}

hipError_t launch_persistent(const PersistParams& p, int blocks, bool cooperative, hipStream_t s) {
  void* args[] = {const_cast<PersistParams*>(&p)};
  const void* fn = nullptr;
#define KDA_PERSIST_CASE(u, cpr) \
  if (p.D == 1024 * (u) && p.rank == 16 * (cpr)) fn = (const void*)decode_persistent_kernel<u, cpr>;
  KDA_PERSIST_CASE(1, 2) KDA_PERSIST_CASE(1, 4) KDA_PERSIST_CASE(1, 8)
  KDA_PERSIST_CASE(2, 2) KDA_PERSIST_CASE(2, 4) KDA_PERSIST_CASE(2, 8)
#undef KDA_PERSIST_CASE
  if (!fn) return hipErrorInvalidValue;
  // a plain launch of one block per CU is co-resident on a GPU this stream has to itself
  // (kernels of one stream run in order); on a shared GPU a block that cannot start leaves
  // the others to their bounded waits, and the step is reported.  The cooperative launch
  // guarantees co-residency but costs ~17 us more per step.
  if (cooperative) return hipLaunchCooperativeKernel(fn, dim3(blocks), dim3(kPT), args, 0, s);
  return hipLaunchKernel(fn, dim3(blocks), dim3(kPT), args, 0, s);
}

#ifdef KDA_TRACE
}  // namespace kda
// Copies the phase timestamps of the last one-launch step ([blocks][64 layers][8 points]
// of 100 MHz counter values, 0 where a block recorded nothing).  Profiling builds only.
extern "C" int kda_trace_read(void* host, size_t bytes) {
  const size_t n = sizeof(kda::g_trace) < bytes ? sizeof(kda::g_trace) : bytes;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(kda::g_trace), n, 0, hipMemcpyDeviceToHost) == hipSuccess ? 0 : 6;
}
namespace kda {
#endif

int persistent_max_blocks() {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_persistent_kernel<2, 8>, kPT, 0) != hipSuccess) return 0;
  return cus * (per > 0 ? 1 : 0);
}

}  // namespace kda

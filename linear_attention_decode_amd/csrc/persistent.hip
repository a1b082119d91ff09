// One-launch decode step for gfx950: every layer of the stack for one token (batch 1) in a
// single cooperative launch of one block per CU.
//
// Per layer the blocks run three phases of the KDA step ("Where the time goes", "Thirty
// tiny kernels per layer", frederic.ai):
//   P  every block: RMSNorm(x) and its slice of the fused input projections
//      [W_q; W_k; W_v; F_a; G_a; W_beta], with the causal conv + SiLU + window roll applied
//      by the owner of each q/k/v channel;
//   H  two blocks per head, each owning half of its value columns: the low-rank forget gate
//      alpha and its output-gate columns (all four waves), then the gated delta rule (one
//      wave per 16 value columns, state in registers), posting the gated outputs and
//      partial sums of o^2;
//   O  a band of blocks: the heads' RMSNorm scales from those partials, the output
//      projection of the normalised heads and the residual.
// Every block streams a slice of every matrix, and it requests the next slice as soon as it
// has used the current one, so the weights of layer l + 1 are in flight while layer l's
// later phases run.  The weight loads go through global-address-space pointers (no flat
// accesses) with wave-uniform row addresses, so a wave issues all of its rows back to back.
//
// Blocks hand activations to each other as 64-bit words (tag << 32 | fp32 bits) written
// and read with agent-scope relaxed atomics (coherent across the XCDs' L2s); the tag names
// the token and layer.  Each producer block also posts a flag word: the projection blocks
// when they start a layer (their consumers, the few head blocks, then poll their input
// words directly), the head and output blocks when they are done (their many consumers
// watch the flags -- one wave, a short sleep between polls -- and fetch the data words once
// the first producer has posted, so that polling stays far below the weight stream).  A
// consumer always checks the tag of every data word it uses.  Every wait is bounded: on a
// timeout the block records an error word and every block leaves the kernel.
#include "kda_device.h"
#include "persist.h"

#define KDA_GLOBAL __attribute__((address_space(1)))
#define KDA_CONST __attribute__((address_space(4)))

namespace kda {

constexpr int kPT = 256;         // threads per block
constexpr int kPRows = 8;        // max projection rows per wave
constexpr int kORows = 4;        // max output-projection rows per wave
constexpr int kHD = 128;         // d_k = d_v of the one-launch path
constexpr int kHSplit = 2;       // head blocks per head
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
      __hip_atomic_store(gpw(P.err), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return true;
    }
    return false;
  }
};

enum FlagPhase { kFlagP = 0, kFlagH = 1, kFlagO = 2 };

__device__ __forceinline__ uint64_t* flag_slot(const PersistParams& P, int phase, int i) {
  return P.flags + (size_t)phase * kMaxPersistBlocks + i;
}

// One wave: wait until at least `need` of flags [0, n) of `phase` carry `tag` (n <= 4 * 64).
// Every flag is loaded at once; only the ones not yet set are polled again.
__device__ bool wave_wait_flags(const PersistParams& P, int phase, int n, uint32_t tag, int need) {
  const int lane = threadIdx.x & 63;
  Spin sp;
  bool ok[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) ok[k] = false;
  while (true) {
    uint64_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (!ok[k] && lane + 64 * k < n) w[k] = peek(flag_slot(P, phase, lane + 64 * k));
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!ok[k] && lane + 64 * k < n) ok[k] = (uint32_t)(w[k] >> 32) == tag;
      cnt += __popcll(__ballot(ok[k]));
    }
    if (cnt >= need) return true;
    if (sp.stop(P)) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Whole block: wave 0 watches the producer flags, the other waves wait at the barrier.
__device__ bool block_wait_flags(const PersistParams& P, int phase, int n, uint32_t tag, int need) {
  int bad = 0;
  if (threadIdx.x < 64) bad = !wave_wait_flags(P, phase, n, tag, need);
  return __syncthreads_or(bad) == 0;
}

// This thread's tagged words p[0], p[stride], ..., p[(n - 1) stride] (n <= N) into w[]:
// every load is issued at once, then each round re-issues the loads of all words not yet
// tagged, so a round costs one memory trip however many words are missing.  Returns false
// on a failed wait.
template <int N>
__device__ bool poll_words(const uint64_t* p, int stride, uint32_t tag, uint64_t (&w)[N], int n,
                           const PersistParams& P) {
#pragma unroll
  for (int k = 0; k < N; ++k) w[k] = k < n ? peek(p + (size_t)k * stride) : tagged(tag, 0.0f);
  Spin sp;
  while (true) {
    bool all = true;
#pragma unroll
    for (int k = 0; k < N; ++k) all &= (uint32_t)(w[k] >> 32) == tag;
    if (all) return true;
    if (sp.stop(P)) return false;
#pragma unroll
    for (int k = 0; k < N; ++k)
      if ((uint32_t)(w[k] >> 32) != tag) w[k] = peek(p + (size_t)k * stride);
  }
}

// Block-wide fetch of NPT * kPT tagged words into dst[] (LDS), with the sums of every 16
// consecutive words into dsum[] and each thread's sum of squares in ss.  Thread t takes words
// t, t + kPT, ...; every load is issued before the first tag is checked, and only words not
// yet tagged are polled again.  The 16 lanes t & ~15 .. hold one 16-word chunk.  Ends with a
// barrier; returns block-uniform false on a failed wait.
template <int NPT>
__device__ bool fetch_vec(const uint64_t* buf, uint32_t tag, float* dst, float* dsum, float& ss,
                          const PersistParams& P) {
  const int tid = threadIdx.x;
  uint64_t w[NPT];
  const int bad = !poll_words<NPT>(buf + tid, kPT, tag, w, NPT, P);
  ss = 0.0f;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const float v = __uint_as_float((uint32_t)w[k]);
    const int i = tid + k * kPT;
    dst[i] = v;
    ss += v * v;
    const float cs = sum16(v);
    if ((tid & 15) == 0) dsum[i >> 4] = cs;
  }
  return __syncthreads_or(bad) == 0;
}

// Dot of one 16-byte Q8_0 chunk with 16 inputs held in registers.
__device__ __forceinline__ float q8_dot16(const uint4 w, const float4 (&x)[4]) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += (float)(d[i] & 0xffu) * x[i].x;
    s += (float)((d[i] >> 8) & 0xffu) * x[i].y;
    s += (float)((d[i] >> 16) & 0xffu) * x[i].z;
    s += (float)(d[i] >> 24) * x[i].w;
  }
  return s;
}

// Wave-wide dots of up to NR rows (the first n, n wave-uniform) whose chunks this lane holds
// (chunk u * 64 + lane of each row) with the LDS vector xs (chunk sums in xsum).  The lane's
// 16-element slices of xs are read once, as aligned float4s, for all rows.
// With HSCALE, the 16-element chunk c of xs is scaled by hs[c / 8] (one head = 128 elements).
template <int U, int NR, bool HSCALE = false>
__device__ __forceinline__ void dot_rows(const uint4 (&w)[NR][U], const uint32_t (&d)[NR][U],
                                         int n, const float* xs, const float* xsum,
                                         const float* hs, float (&acc)[NR]) {
  const int lane = threadIdx.x & 63;
  float4 xv[U][4];
  float xc[U], cs[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = u * 64 + lane;
    const float4* p = reinterpret_cast<const float4*>(xs + c * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) xv[u][k] = p[k];
    xc[u] = xsum[c];
    cs[u] = HSCALE ? hs[c >> 3] : 1.0f;
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    float a = 0.0f;
    if (r < n) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float t = h2f(d[r][u]) * (q8_dot16(w[r][u], xv[u]) - 128.0f * xc[u]);
        a += HSCALE ? t * cs[u] : t;
      }
      a = wave_sum(a);
    }
    acc[r] = a;
  }
}

// The projection weights of one wave's rows [r0, r1) of layer L (r0, r1 wave-uniform).
template <int U>
struct ProjRegs {
  uint4 w[kPRows][U];
  uint32_t d[kPRows][U];
  float4 cw;               // lane r: conv taps of row r0 + r (q/k/v channels)
  float z0, z1, z2;        // lane r: its conv window, oldest first
};

template <int U>
__device__ __forceinline__ void issue_proj(const PersistParams& P, GLayer& L, const float* win,
                                           int r0, int r1, ProjRegs<U>& R) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < kPRows; ++r) {
    const int row = r0 + r;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      R.w[r][u] = make_uint4(0, 0, 0, 0);
      R.d[r][u] = 0;
    }
    if (row < r1) {
      int first = 0, seg = 0;
#pragma unroll
      for (int i = 1; i < 6; ++i)
        if (row >= P.seg_first[i]) { first = P.seg_first[i]; seg = i; }
      const uint8_t* wr = L.seg[seg].w + (size_t)(row - first) * P.D;
      const __half* dr = L.seg[seg].d + (size_t)(row - first) * (P.D / 32);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = u * 64 + lane;
        R.w[r][u] = wload(wr + (size_t)c * 16);
        R.d[r][u] = sload(dr + (c >> 1));
      }
    }
  }
  const int myrow = r0 + lane;
  R.cw = make_float4(0.f, 0.f, 0.f, 0.f);
  R.z0 = R.z1 = R.z2 = 0.0f;
  if (lane < kPRows && myrow < r1 && myrow < P.C) {
    R.cw = gload4(L.conv_w + (size_t)myrow * 4);
    R.z0 = *gp(win + myrow);
    R.z1 = *gp(win + P.C + myrow);
    R.z2 = *gp(win + 2 * P.C + myrow);
  }
}

// The output-projection weights of one wave's rows [r0, r0 + n).
template <int U>
struct OutRegs {
  uint4 w[kORows][U];
  uint32_t d[kORows][U];
};

template <int U>
__device__ __forceinline__ void issue_out(const PersistParams& P, GLayer& L, int r0, int n,
                                          OutRegs<U>& R) {
  const int lane = threadIdx.x & 63;
  const int KO = P.H * P.dv;
#pragma unroll
  for (int r = 0; r < kORows; ++r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      R.w[r][u] = make_uint4(0, 0, 0, 0);
      R.d[r][u] = 0;
    }
    if (r < n) {
      const uint8_t* wr = L.wo.w + (size_t)(r0 + r) * KO;
      const __half* dr = L.wo.d + (size_t)(r0 + r) * (KO / 32);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = u * 64 + lane;
        R.w[r][u] = wload(wr + (size_t)c * 16);
        R.d[r][u] = sload(dr + (c >> 1));
      }
    }
  }
}

// A head block owns value columns [half * kHCols, + kHCols) of head h.  Its registers: wave
// w's state tile (rows 8 (lane & 15) .. + 8, columns half * kHCols + 16 w + 4 (lane >> 4)
// .. + 4) and the block's gate-weight chunks: item i of thread t is chunk (i * kPT + t) of
// the [kHD alpha rows | kHCols gate rows] x rank slice (the first CPR / 2 items of every
// thread are alpha rows).
template <int CPR>   // 16-byte chunks per low-rank row: CPR = rank / 16
struct HeadRegs {
  static constexpr int kItems = ((kHD + kHCols) * CPR + kPT - 1) / kPT;
  float4 st[8];
  uint4 gw[kItems];
  uint32_t gd[kItems];
  float dtb[kItems];
  float4 onw;
  float ea;                // A_log[h], exponentiated when used
};

template <int CPR>
__device__ __forceinline__ void issue_head(const PersistParams& P, GLayer& L, const float* Sl,
                                           int h, int half, HeadRegs<CPR>& R) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int rank = CPR * 16;
  const int j = half * kHCols + wave * 16 + (lane >> 4) * 4, r0 = (lane & 15) * 8;
  const float* Sb = Sl + (size_t)h * kHD * kHD + j;
#pragma unroll
  for (int i = 0; i < 8; ++i) R.st[i] = gload4(Sb + (size_t)(r0 + i) * kHD);
  const int c = tid % CPR;
#pragma unroll
  for (int i = 0; i < HeadRegs<CPR>::kItems; ++i) {
    const int it = i * kPT + tid;
    const int row = it / CPR;                        // [0, kHD): alpha, then gate columns
    const bool f = i < CPR / 2;
    R.gw[i] = make_uint4(0, 0, 0, 0);
    R.gd[i] = 0;
    R.dtb[i] = 0.0f;
    if (it < (kHD + kHCols) * CPR) {
      const uint8_t* mw = f ? L.fb.w : L.gb.w;
      const __half* md = f ? L.fb.d : L.gb.d;
      const int r = f ? h * kHD + row : h * kHD + half * kHCols + (row - kHD);
      R.gw[i] = wload(mw + (size_t)r * rank + (size_t)c * 16);
      R.gd[i] = sload(md + (size_t)r * (rank / 32) + (c >> 1));
      if (f) R.dtb[i] = *gp(L.dt_bias + r);
    }
  }
  R.onw = make_float4(1.f, 1.f, 1.f, 1.f);
  if (L.o_norm_w) R.onw = gload4(L.o_norm_w + j);
  R.ea = *gp(L.a_log + h);
}

// LDS of one block.
struct Smem {
  alignas(16) float xs[4096];          // x, then (O blocks) the normalised heads
  float xsum[256];         // 16-element chunk sums of xs
  float red[8];
  float xres[4 * kORows];  // this O block's residual rows
  alignas(16) float s_in[1024];  // head block: q | k | v | f_lr | g_lr | beta
  alignas(16) float s_al[kHD];     // head block: alpha rows
  alignas(16) float s_gt[kHCols];  // head block: output-gate columns
  float s_hs[64];                  // O blocks: per-head RMSNorm scales
};

// Static roles of block b: its projection rows, and whether it runs a head or an
// output-projection band.
struct Roles {
  int wr0, wr1;            // this wave's projection rows (wave-uniform)
  int ob, or0, owr0, orw;  // O band index, block's first row, wave's first row, rows/wave
};

__device__ __forceinline__ Roles make_roles(const PersistParams& P, int wave) {
  Roles R;
  // projection rows go to blocks [kHSplit H, nb) (head blocks keep their loads for the
  // state): q/k/v rows 32 per block to the first q_blocks, then the low-rank and beta rows
  // spread thin over the rest, so that the rows the head blocks need first (their gates)
  // are finished early
  const int b = blockIdx.x - kHSplit * P.H, nb = gridDim.x - kHSplit * P.H;
  const int C = P.C, nl = nb - P.q_blocks;
  const int rl = (P.proj_rows - C + nl - 1) / nl;
  int p0, p1, rp;
  if (b < 0) {
    p0 = p1 = rp = 0;
  } else if (b < P.q_blocks) {
    rp = 32;
    p0 = min(C, b * 32);
    p1 = min(C, p0 + 32);
  } else {
    rp = rl;
    p0 = min(P.proj_rows, C + (b - P.q_blocks) * rl);
    p1 = min(P.proj_rows, p0 + rl);
  }
  const int rpw = (rp + 3) / 4;
  R.wr0 = min(p1, p0 + wave * rpw);
  R.wr1 = min(p1, R.wr0 + rpw);
  const int ro = P.D / P.o_blocks;
  R.ob = (int)blockIdx.x - P.o_first_block;
  R.orw = ro / 4;
  R.or0 = R.ob * ro;
  R.owr0 = R.or0 + wave * R.orw;
  return R;
}

// P phase of layer l (blocks [H, nb)): wait for x_l, RMSNorm, this block's projection rows,
// conv epilogue; the next layer's slice is requested as soon as this one is used.
// Returns false on a failed wait.
template <int U, bool OBLK>
__device__ __forceinline__ bool phase_p(const PersistParams& P, Smem& sm, const Roles& R, int l,
                                        uint32_t tag, ProjRegs<U>& pr, OutRegs<U>* orr) {
  GLayer* Lt = (GLayer*)P.layers;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = P.D, C = P.C;
  float* win = P.win + (size_t)l * 3 * C;
  float ss = 0.0f;
  if (l == 0) {
    for (int i = tid; i < D; i += kPT) {
      const float v = *gp(P.x_in + i);
      sm.xs[i] = v;
      ss += v * v;
      const float cs = sum16(v);
      if ((tid & 15) == 0) sm.xsum[i >> 4] = cs;
    }
    __syncthreads();
  } else {
    // x_l: once the first O block of layer l - 1 has posted (they finish together), fetch
    // the tagged words of x
    if (!block_wait_flags(P, kFlagO, P.o_blocks, tag - 1u, 1)) return false;
    if (!fetch_vec<4 * U>(P.xbuf + (size_t)((l - 1) & 1) * D, tag - 1u, sm.xs, sm.xsum, ss, P)) return false;
  }
  ss = wave_sum(ss);
  if (lane == 0) sm.red[wave] = ss;
  if (OBLK && tid < 4 * R.orw) sm.xres[tid] = sm.xs[R.or0 + tid];
  // the flag says "this layer's projections are under way": the head blocks start polling
  // their input words (flags are hints; every data word carries its own tag).  The
  // prefetched weights have landed by now; retiring them first keeps the dots below from
  // waiting for the flag store.
  retire_vmem();
  if (tid == 0) put(flag_slot(P, kFlagP, blockIdx.x - kHSplit * P.H), tag, 0.0f);
  __syncthreads();
  const float sc = 1.0f / sqrtf((sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3]) / (float)D + P.eps);
  float accs[kPRows];
  // an output block requests this layer's W_o rows now: they land during the dots, and the
  // wait for the head blocks later has no loads queued ahead of its polls
  if (OBLK) issue_out<U>(P, Lt[l], R.owr0, R.orw, *orr);
  dot_rows<U, kPRows>(pr.w, pr.d, R.wr1 - R.wr0, sm.xs, sm.xsum, nullptr, accs);
  // lane r finishes row wr0 + r: conv + SiLU + window roll for q/k/v channels
  float v = 0.0f;
#pragma unroll
  for (int r = 0; r < kPRows; ++r)
    if (lane == r) v = accs[r] * sc;
  const int row = R.wr0 + lane;
  const bool mine = lane < kPRows && row < R.wr1;
  const float pre = v;
  if (mine) {
    if (row < C) v = silu_f(pr.cw.x * pr.z0 + pr.cw.y * pr.z1 + pr.cw.z * pr.z2 + pr.cw.w * v);
    put(P.pbuf + row, tag, v);
  }
  // off the critical path: roll the conv window, request the next layer's slice
  if (mine && row < C) {
    float* z = win + row;
    *gpw(z) = pr.z1;
    *gpw(z + C) = pr.z2;
    *gpw(z + 2 * C) = pre;
  }
  if (l + 1 < P.n_layers) issue_proj<U>(P, Lt[l + 1], win + 3 * C, R.wr0, R.wr1, pr);
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
  // ~2 KB a round, no flag first: the low-rank rows land early)
  // inputs: q [dk] | k [dk] | v [kHCols] | f_lr [rank] | g_lr [rank] | beta  (<= 3 per thread)
  constexpr int n_in = 2 * dk + kHCols + 2 * rank + 1;
  static_assert(n_in <= 3 * kPT, "head inputs");
  // every input is requested at once; the low-rank rows and beta (finished first by their
  // projection blocks) are waited for before the gates, q / k / v after them
  constexpr int i_lr = 2 * dk + kHCols;          // first low-rank input
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
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int i = tid + k * kPT;
      if (i >= i_lr && i < n_in) sm.s_in[i] = __uint_as_float((uint32_t)w[k]);
    }
    if (__syncthreads_or(bad)) return false;
  }
  const float* s_q = sm.s_in;
  const float* s_k = sm.s_in + dk;
  const float* s_v = sm.s_in + 2 * dk;
  const float* s_fl = sm.s_in + 2 * dk + kHCols;
  const float* s_gl = s_fl + rank;
  const float beta = sigmoid_f(sm.s_in[2 * dk + kHCols + 2 * rank]);
  // alpha = exp(-exp(A_log) softplus(F_b f_lr + dt_bias)), gate = sigmoid(G_b g_lr).
  // Thread t's items all sit in chunk c = t % CPR of their rows, so it needs one 16-element
  // slice of f_lr and one of g_lr.  After the group sums, lane c of each group finishes
  // item c: one transcendental per lane.
  {
    constexpr int NI = HeadRegs<CPR>::kItems;
    const int c = tid % CPR;
    float4 xf[4], xg[4];
    float sf = 0.0f, sg = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      xf[k] = reinterpret_cast<const float4*>(s_fl + c * 16)[k];
      xg[k] = reinterpret_cast<const float4*>(s_gl + c * 16)[k];
      sf += (xf[k].x + xf[k].y) + (xf[k].z + xf[k].w);
      sg += (xg[k].x + xg[k].y) + (xg[k].z + xg[k].w);
    }
    float mine = 0.0f, bias = 0.0f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float part = i < CPR / 2 ? q8_dot16(hr.gw[i], xf) - 128.0f * sf : q8_dot16(hr.gw[i], xg) - 128.0f * sg;
      part = group_sum(h2f(hr.gd[i]) * part, CPR);
      if (c == i) { mine = part; bias = hr.dtb[i]; }
    }
    const int it = c * kPT + tid, grow = it / CPR;
    if (c < NI && it < (kHD + kHCols) * CPR) {
      if (grow < dk) sm.s_al[grow] = expf(-expf(hr.ea) * softplus_f(mine + bias));
      else sm.s_gt[grow - dk] = sigmoid_f(mine);
    }
  }
  {
    // q, k, v
    const int bad = !wait_slots(false);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int i = tid + k * kPT;
      if (i < i_lr) sm.s_in[i] = __uint_as_float((uint32_t)w[k]);
    }
    if (__syncthreads_or(bad)) return false;
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
  const float inv_q = P.q_scale / sqrtf(sum16(aq) + P.l2_eps);
  const float inv_k = 1.0f / sqrtf(sum16(ak) + P.l2_eps);
  float e0 = 0.f, e1 = 0.f, e2 = 0.f, e3 = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = aa[i], kk = ka[i] * inv_k;
    float4& s = hr.st[i];
    s.x *= a; s.y *= a; s.z *= a; s.w *= a;
    e0 += s.x * kk; e1 += s.y * kk; e2 += s.z * kk; e3 += s.w * kk;
  }
  e0 = sum16(e0); e1 = sum16(e1); e2 = sum16(e2); e3 = sum16(e3);
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
  // off the critical path: write the state back, request the next layer's
  float* Sb = Sl + (size_t)h * dk * dv + j;
#pragma unroll
  for (int i = 0; i < 8; ++i) gstore4(Sb + (size_t)(r0 + i) * dv, hr.st[i]);
  if (l + 1 < P.n_layers) issue_head<CPR>(P, Lt[l + 1], Sl + (size_t)H * dk * dv, h, half, hr);
  // (the next layer's first wait is a barrier, so LDS is not rewritten while still read)
  return true;
}

// O phase of layer l: this band's output-projection rows of the normalised heads, plus the
// residual; the last layer also writes the output row.  The heads' RMSNorm scales come from
// the per-wave partial sums of o^2 that the head blocks post after their outputs.
template <int U>
__device__ __forceinline__ bool phase_o(const PersistParams& P, Smem& sm, const Roles& R, int l,
                                        uint32_t tag, OutRegs<U>& orr) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int D = P.D, H = P.H, V = H * kHD;
  constexpr int kParts = kHSplit * 4;                // o^2 partials per head
  // once the first head block has posted, fetch the output words
  if (!block_wait_flags(P, kFlagH, kHSplit * H, tag, 1)) return false;
  {
    const uint64_t* src = P.obuf + V + tid;
    const bool has = tid < H * kParts;
    uint64_t w = has ? peek(src) : tagged(tag, 0.0f);
    float ssd;
    bool ok = fetch_vec<4 * U>(P.obuf, tag, sm.xs, sm.xsum, ssd, P);   // ends with a barrier
    int bad = !ok;
    Spin sp;
    while (!bad && (uint32_t)(w >> 32) != tag) {
      if (sp.stop(P)) bad = 1;
      else w = peek(src);
    }
    float v = __uint_as_float((uint32_t)w);
    // the kParts partials of a head sit on consecutive lanes
    v = group_sum(v, kParts);
    if (has && tid % kParts == 0) sm.s_hs[tid / kParts] = 1.0f / sqrtf(v / (float)kHD + P.eps);
    if (__syncthreads_or(bad)) return false;
  }
  float accs[kORows];
  dot_rows<U, kORows, true>(orr.w, orr.d, R.orw, sm.xs, sm.xsum, sm.s_hs, accs);
  float v = 0.0f;
#pragma unroll
  for (int r = 0; r < kORows; ++r)
    if (lane == r) v = accs[r];
  if (lane < R.orw) {
    const int row = R.owr0 + lane;
    const float xn = sm.xres[row - R.or0] + v;
    put(P.xbuf + (size_t)(l & 1) * D + row, tag, xn);
    if (l + 1 == P.n_layers) *gpw(P.y_out + row) = xn;
  }
  __syncthreads();
  if (tid == 0) put(flag_slot(P, kFlagO, R.ob), tag, 0.0f);
  return true;
}

// The layer loop of one role: ROLE 0 projection only, 1 head block, 2 projection + output
// band.  Each role keeps only its own prefetch registers live.  Prefetches are issued right
// after a phase that is followed by a long wait, never just before a poll on the critical
// path (a poll's load completes only after the loads issued before it).
template <int U, int CPR, int ROLE>
__device__ __forceinline__ void run_role(const PersistParams& P, Smem& sm) {
  GLayer* Lt = (GLayer*)P.layers;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const Roles R = make_roles(P, wave);
  const uint32_t tag0 = P.epoch * (uint32_t)P.n_layers;
  if constexpr (ROLE == 1) {
    HeadRegs<CPR> hr;
    issue_head<CPR>(P, Lt[0], P.S, blockIdx.x % P.H, blockIdx.x / P.H, hr);
    for (int l = 0; l < P.n_layers; ++l)
      if (!phase_h<CPR>(P, sm, l, tag0 + (uint32_t)l + 1u, hr)) return;
  } else {
    ProjRegs<U> pr;
    issue_proj<U>(P, Lt[0], P.win, R.wr0, R.wr1, pr);
    if constexpr (ROLE == 2) {
      OutRegs<U> orr;
      for (int l = 0; l < P.n_layers; ++l) {
        const uint32_t tag = tag0 + (uint32_t)l + 1u;
        if (!phase_p<U, true>(P, sm, R, l, tag, pr, &orr)) return;
        if (!phase_o<U>(P, sm, R, l, tag, orr)) return;
      }
    } else {
      // a block left without projection rows has nothing to do: no phase waits for it, and
      // it must not fall layers behind while it reads the residual stream
      if (__syncthreads_or(R.wr1 > R.wr0) == 0) return;
      for (int l = 0; l < P.n_layers; ++l)
        if (!phase_p<U, false>(P, sm, R, l, tag0 + (uint32_t)l + 1u, pr, nullptr)) return;
    }
  }
}

// U = D / 1024 (16-byte chunks per lane per row), CPR = rank / 16
template <int U, int CPR>
__global__ __launch_bounds__(kPT, 1) void decode_persistent_kernel(const PersistParams P) {
  __shared__ Smem sm;
  const int b = blockIdx.x;
  if (b < kHSplit * P.H) run_role<U, CPR, 1>(P, sm);
  else if (b >= P.o_first_block && b < P.o_first_block + P.o_blocks) run_role<U, CPR, 2>(P, sm);
  else run_role<U, CPR, 0>(P, sm);
}

hipError_t launch_persistent(const PersistParams& p, int blocks, hipStream_t s) {
  void* args[] = {const_cast<PersistParams*>(&p)};
  const void* fn = nullptr;
#define KDA_PERSIST_CASE(u, cpr) \
  if (p.D == 1024 * (u) && p.rank == 16 * (cpr)) fn = (const void*)decode_persistent_kernel<u, cpr>;
  KDA_PERSIST_CASE(1, 2) KDA_PERSIST_CASE(1, 4) KDA_PERSIST_CASE(1, 8)
  KDA_PERSIST_CASE(2, 2) KDA_PERSIST_CASE(2, 4) KDA_PERSIST_CASE(2, 8)
#undef KDA_PERSIST_CASE
  if (!fn) return hipErrorInvalidValue;
  return hipLaunchCooperativeKernel(fn, dim3(blocks), dim3(kPT), args, 0, s);
}

int persistent_max_blocks() {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_persistent_kernel<2, 8>, kPT, 0) != hipSuccess) return 0;
  return cus * (per > 0 ? 1 : 0);
}

}  // namespace kda

// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stddef.h>
#include <stdint.h>

#include "persist.h"

namespace kda {

// Causal depthwise conv of one channel over (window z0, z1, z2 oldest first, this token x)
// with taps w: one fixed chain of fused multiply-adds, so every per-layer kernel that
// computes it (decode, verify, the sequential scan) gets the same bits whatever the
// compiler would have contracted
__device__ __forceinline__ float conv4_f(const float4 w, float z0, float z1, float z2, float x) {
  return __builtin_fmaf(w.w, x, __builtin_fmaf(w.z, z2, __builtin_fmaf(w.y, z1, w.x * z0)));
}

enum WType { kF32 = 0, kBF16 = 1, kQ8 = 2, kMX4 = 3 };
enum GateForm { kGateKda = 0, kGateSafe = 1, kGateScalar = 2 };

// A packed weight matrix as the kernels see it.

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Byte offset of the Q8_0 scale plane inside a packed matrix.
inline size_t q8_scale_offset(int64_t rows, int64_t cols) {
  return align_up((size_t)rows * (size_t)cols, 256);
}

// Byte offset of the MXFP4 scale plane inside a packed matrix (after rows*cols/2 bytes of
// 4-bit codes).
inline size_t mx4_scale_offset(int64_t rows, int64_t cols) {
  return align_up((size_t)rows * (size_t)cols / 2, 256);
}

inline PackedMat packed_view(const void* base, int wt, int64_t rows, int64_t cols) {
  PackedMat m;
  m.w = static_cast<const uint8_t*>(base);
  if (wt == kQ8) m.d = reinterpret_cast<const __half*>(m.w + q8_scale_offset(rows, cols));
  if (wt == kMX4) m.e = m.w + mx4_scale_offset(rows, cols);
  return m;
}

// 16 bytes of MXFP4 codes (32 elements, code 2i in the low nibble of byte i) times 32
// inputs: sum over the elements of twice the E2M1 value times x (the caller halves the
// block scale).  gfx950's packed FP4 conversion with scale 2 turns a byte's two codes (low
// nibble into the first float) into the doubled values, exactly; the products are summed
// in the order elements 8 i + 2 k + half, the low nibbles of a word's bytes first.
__device__ __forceinline__ float mx4_chunk_dot2(const uint4 w, const float* __restrict__ x) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2v v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[i], 2.0f, 0),
                         __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[i], 2.0f, 1),
                         __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[i], 2.0f, 2),
                         __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[i], 2.0f, 3)};
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int k = 0; k < 4; ++k) s = fmaf(v[k][half], x[8 * i + 2 * k + half], s);
  }
  return s;
}

// ---------------------------------------------------------------------------------------
// Fused multi-matrix GEMV (projections and the output projection).
// ---------------------------------------------------------------------------------------
constexpr int kGemvThreads = 256;
constexpr int kGemvRowsPerWave = 2;
constexpr int kGemvRowsPerBlock = (kGemvThreads / 64) * kGemvRowsPerWave;
constexpr int kMaxSegs = 6;

enum GemvPrologue { kProX = 0, kProGatedNorm = 1 };

struct GemvSeg {
  PackedMat m;
  int rows = 0;
  int first_tile = 0;   // first block index of this matrix in the grid
  int out_off = 0;      // column offset of this matrix's rows in an output row
  int conv_chan = -1;   // >= 0: rows are conv channels from here; apply conv + SiLU + roll
};

struct GemvParams {
  GemvSeg seg[kMaxSegs];
  int nseg = 0;
  int K = 0;            // input length
  int N = 0;            // columns (sequences x tokens)
  // prologue kProX: input rows x[n][x_stride], optional RMSNorm (weight ones)
  const float* x = nullptr;
  int x_stride = 0;
  int prenorm = 0;
  float eps = 0.f;
  // prologue kProGatedNorm: n = o * rsqrt(mean_h(o^2) + eps) * o_norm_w * gate, per head
  const float* o = nullptr;
  const float* gate = nullptr;
  const float* ss = nullptr;     // [N][H][ncb] partial sums of o^2
  const float* onw = nullptr;    // [dv] or null (ones)
  int H = 0, dv = 0, ncb = 0;
  // output: out[n][out_stride] (+ resid[n][out_stride] if resid != null; may alias out)
  float* out = nullptr;
  int out_stride = 0;
  const float* resid = nullptr;
  // decode conv epilogue (T = 1, column n = sequence n)
  const float* conv_w = nullptr;  // [C][4]
  float* win = nullptr;           // [N][3][C]
  int C = 0;
  const int* active = nullptr;    // [N] or null: a column n with active[n] == 0 leaves its
                                  // window as it is (its outputs are still computed)
  // verify conv epilogue (launch_skinny only): columns n = b T + t; act[n][c] = SiLU of the
  // conv over sequence b's window and its tokens 0..t, the window left as it is
  float* act = nullptr;           // [N][C]
  int T = 0;
  // verify with a commit folded in: the window first moves on by the previous verify's
  // accepted tokens, pre_ntok[b] of them (clamped 1..pre_T), whose pre-conv projections
  // are rows b pre_T + t of pre_proj ([B pre_T][out_stride]), and is written back
  const float* pre_proj = nullptr;
  const int* pre_ntok = nullptr;
  int pre_T = 0;
  // launch_skinny only: the Q8_0 matrices (seg[i].m: w at the segment's first 16-row tile,
  // d at its scales) are in the one-launch decode's matrix-core order
  int mma = 0;
  // launch_skinny only: the weight format (kQ8, kBF16 or kMX4)
  int wt = kQ8;
};

constexpr int kGemvKSmall = 2048;   // input length of the multi-column variants
constexpr int kGemvKMax = 8192;     // longest input the GEMV takes
constexpr int kGemvMaxHeads = 64;

hipError_t launch_gemv(int wt, int prologue, const GemvParams& p, int grid, hipStream_t s);
int gemv_cols_per_pass(int N);

// ---------------------------------------------------------------------------------------
// Per-head kernel: conv (verify/commit), L2 norms, gates, delta rule, read-out.
// ---------------------------------------------------------------------------------------
constexpr int kHeadCols = 16;      // value columns per wave (one partial sum of o^2 each)
constexpr int kMaxNcb = 128 / kHeadCols;   // partial sums a head has (d_v is 64 or 128)

// The sum of a head's ncb (1 .. kMaxNcb) partial sums of o^2, added in order j = 0 .. ncb - 1.
// Every load is issued at once (indices clamped into the head, the extra terms added as +0,
// which leaves the sum's bits unchanged): a loop over the runtime count waited for each
// load in turn.
__device__ __forceinline__ float sum_partials(const float* sp, int ncb) {
  float x[kMaxNcb];
#pragma unroll
  for (int j = 0; j < kMaxNcb; ++j) x[j] = sp[min(j, ncb - 1)];
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxNcb; ++j) a += j < ncb ? x[j] : 0.0f;
  return a;
}

struct HeadParams {
  int H = 0, dk = 0, dv = 0, C = 0, rank_f = 0, rank_g = 0;
  int B = 0, T = 0;               // sequences, tokens per sequence (column n = b*T + t)
  const float* proj = nullptr;    // [N][proj_stride]: a or p (C) | f_lr | g_lr | beta logits
  int proj_stride = 0;
  const float* act = nullptr;     // [N][C] activated q|k|v when proj holds pre-conv p, else null
  int wt = 0;
  PackedMat fb, gb;               // [H*dk][rank_f], [H*dv][rank_g]
  const float* a_log = nullptr;
  const float* dt_bias = nullptr;
  const float* alpha_gate = nullptr;  // [N][H*dk + H*dv]: alpha per key channel | output gate
  float* S = nullptr;             // [B][H][dk][dv]
  int write_state = 1;
  const int* ntok = nullptr;      // commit: tokens to apply per sequence (clamped 1..T)
  int write_out = 1;
  float* o = nullptr;             // [N][H*dv]
  float* gate = nullptr;          // [N][H*dv]
  float* ss = nullptr;            // [N][H][dv/kHeadCols] partial sums of o^2
  float l2_eps = 0.f;
  float q_scale = 0.f;            // d_k^-1/2 as fp32
  // commit only: the layer's conv window [B][3][C], rolled by the accepted tokens' logged
  // pre-conv projections (proj) once the replay is done (null: left alone)
  float* win_commit = nullptr;
  // [B] or null: a sequence with active[b] == 0 keeps its state (its outputs are still
  // computed from it)
  const int* active = nullptr;
  // verify with a commit folded in (pre_ntok != null): first the previous verify's accepted
  // tokens, pre_ntok[b] of them (clamped 1..pre_T), replayed from its log (rows
  // n = b pre_T + t of pre_proj / pre_act / pre_ag, laid out as proj / act / alpha_gate),
  // and the state written back once; then this call's T tokens as above
  const float* pre_proj = nullptr;
  const float* pre_act = nullptr;
  const float* pre_ag = nullptr;
  const int* pre_ntok = nullptr;
  int pre_T = 0;
  // fuse_gates = 1, decode (T = 1, no folded commit): compute the gates here instead of
  // reading alpha_gate: alpha of the head's rows from F_b (fb) and f_lr, the wave's
  // output-gate columns from G_b and g_lr (proj at C and C + rank_f), in the gate form
  // gate_form (row-major fb, gb).  fuse_gates = 2: the same for this call's T = 1 token
  // of a model with its own gate-tile-order copy (fbw/fbd, gbw/gbd; KDA form, rank_f in
  // {32, 64, 128}, d_k = 128) on the matrix cores, also written to ag_out ([N][H*dk + H*dv]
  // as alpha_gate) when that is set (a replayed commit reads them there)
  int fuse_gates = 0;
  float* ag_out = nullptr;
  int gate_form = 0;
  float gate_lb = 0.f;
  const int8_t* fbw = nullptr;
  const uint16_t* fbd = nullptr;
  const int8_t* gbw = nullptr;
  const uint16_t* gbd = nullptr;
};

hipError_t launch_head(const HeadParams& p, hipStream_t s);
// decode batches up to this many sequences run the gates inside the head kernel (row-major
// F_b, G_b with vector dots; a model's own gate-tile-order copy on the matrix cores)
constexpr int kFuseGatesMaxB = 8;
constexpr int kFuseGatesMaxBOwned = 16;

struct GatesParams {
  int N = 0, K = 0, V = 0, dk = 0, rank = 0, C = 0, wt = 0;
  int gate = 0;                   // forget-gate form (kGateKda / kGateSafe / kGateScalar)
  float gate_lb = 0.f;            // safe gate: lower bound of log(alpha)
  const float* proj = nullptr;    // [N][proj_stride]: f_lr at C, g_lr at C + rank
  int proj_stride = 0;
  PackedMat fb, gb;               // [K][rank], [V][rank]
  const float* a_log = nullptr;   // [H]
  const float* dt_bias = nullptr; // [K] ([H] for the scalar gate)
  float* out = nullptr;           // [N][K + V]: alpha | gate
  // Q8_0 F_b / G_b in gate-tile order (made for the one-launch decode; null if none): with
  // them, N > 1 runs on the int8 matrix cores
  const int8_t* fbw = nullptr;
  const uint16_t* fbd = nullptr;
  const int8_t* gbw = nullptr;
  const uint16_t* gbd = nullptr;
};
hipError_t launch_gates(const GatesParams& p, hipStream_t s);
// Whether the per-head kernel handles these low-rank shapes (equal ranks, a power-of-two
// number of 16-byte chunks per row, at most 10 chunk loads per thread).
bool head_supported(int dk, int wt, int rank_f, int rank_g);

// Conv + SiLU over T tokens per sequence from the committed window (left unchanged):
// act[b*T + t][c] from the pre-conv projections plog[b*T + t][c] (stride proj_stride).
// With pre_ntok (a commit folded in) the window first moves on by the previous verify's
// accepted tokens (pre_ntok[b], clamped 1..pre_T, rows b pre_T + t of pre_plog) and is
// written back.
hipError_t launch_conv_seq(const float* plog, int proj_stride, float* win, const float* conv_w,
                           float* act, int B, int T, int C, const float* pre_plog,
                           const int* pre_ntok, int pre_T, hipStream_t s);

// ---------------------------------------------------------------------------------------
// Chunked prefill.
// ---------------------------------------------------------------------------------------
// C[m][coff + n] = sum_k A[m][k] B[n][k]; B = BF16 rows from up to kMaxSegs stacked
// matrices ([rows][K] each, segment i starting at output column seg_first[i]); A = BF16
// [M][lda], plus optionally a second BF16 plane summed against the same B (an fp32
// operand as hi + lo).  K % 64 == 0.
struct GemmParams {
  const uint16_t* A = nullptr;    // BF16 [M][lda]
  const uint16_t* A2 = nullptr;   // optional second BF16 plane [M][lda] (the low half of an
                                  // fp32 operand split hi + lo), multiplied by the same B
  int lda = 0;
  const uint16_t* seg_b[kMaxSegs] = {};
  int seg_first[kMaxSegs] = {};
  int nseg = 0;
  int M = 0, N = 0, K = 0;        // K a multiple of 64
  float* C = nullptr;
  int ldc = 0, coff = 0;
};
hipError_t launch_gemm(const GemmParams& p, hipStream_t s);
// fp32 [n] -> BF16 planes hi = bf16(x), lo = bf16(x - hi); n a multiple of 4
hipError_t launch_split_planes(const float* x, uint16_t* hi, uint16_t* lo, int64_t n, hipStream_t s);

constexpr int kChunk = 64;          // tokens per chunk of the chunked delta rule

struct PrefillParams {
  int B = 0, L = 0, H = 0, dk = 0, dv = 0, C = 0, rank_f = 0, rank_g = 0;
  int nch = 0;                    // chunks per sequence
  const float* P = nullptr;       // [B*L][proj_stride]: p (C) | f_lr | g_lr | beta logits
  int proj_stride = 0;
  const float* win = nullptr;     // [B][3][C] initial conv window
  float* win_out = nullptr;       // [B][3][C] final window (may alias win; own kernel, after prep)
  const float* conv_w = nullptr;
  const float* a_log = nullptr;
  const float* dt_bias = nullptr;
  const float* onw = nullptr;     // [dv] or null
  const uint16_t* Fb = nullptr;   // forget-gate up-projection, BF16 [H*dk][rank_f] ([H][rank_f]
                                  // for the scalar gate)
  int gate = 0;                   // forget-gate form
  float gate_lb = 0.f;
  const uint16_t* Gb = nullptr;   // output-gate up-projection, BF16 [H*dv][rank_g]
  float l2_eps = 0.f, q_scale = 0.f, norm_eps = 0.f;
  // per-chunk preparation outputs, per (b, h, chunk), in matrix-core operand order: -W,
  // q 2^G, (k 2^(G_last - G))^T and A as BF16 hi/lo fragments, U in accumulator order,
  // dec = 2^G_last
  void *Wf = nullptr, *Qf = nullptr, *Kf = nullptr, *Af = nullptr;
  float *Uf = nullptr, *dec = nullptr;
  float* S = nullptr;             // [B][H][dk][dv] state, read then overwritten
  float* o = nullptr;             // [B*L][H*dv] scan outputs
  uint16_t *on_hi = nullptr, *on_lo = nullptr;   // [B*L][H*dv] gated norm as BF16 hi/lo planes
};
hipError_t launch_prefill_window(const PrefillParams& p, hipStream_t s);
hipError_t launch_chunk_prep(const PrefillParams& p, hipStream_t s);
hipError_t launch_chunk_scan(const PrefillParams& p, hipStream_t s);
hipError_t launch_chunk_gnorm(const PrefillParams& p, hipStream_t s);

// ---------------------------------------------------------------------------------------
// Packing.
// ---------------------------------------------------------------------------------------
hipError_t launch_pack(int wt, const float* src, int64_t rows, int64_t cols, void* dst,
                       hipStream_t s);
hipError_t launch_unpack_q8(const void* packed, int64_t rows, int64_t cols, uint16_t* d16,
                            int8_t* qs, hipStream_t s);
// An MXFP4-packed [rows][cols] matrix as the Q8_0 layout holding the same values (q8 has
// Q8_0's packed size); *bad is set if a nonzero block's scale has no fp16 power of two.
hipError_t launch_mx4_to_q8(const void* mx4, int64_t rows, int64_t cols, void* q8, int* bad,
                            hipStream_t s);
// A Q8_0-packed [rows][cols] matrix as [rows * rep][cols], each row repeated rep times
// (out has Q8_0's packed size for rows * rep rows); and n floats each repeated rep times.
hipError_t launch_q8_repeat_rows(const void* q8, int64_t rows, int64_t cols, int rep, void* out,
                                 hipStream_t s);
hipError_t launch_f32_repeat(const float* in, int64_t n, int rep, float* out, hipStream_t s);

}  // namespace kda

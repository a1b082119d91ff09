// Declarations of the one-launch decode step (persistent.hip) and the packed-weight handle
// it shares with the rest of the library.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kda {

struct PackedMat {
  const uint8_t* w = nullptr;   // F32/BF16 data, the Q8_0 byte plane (q + 128), or the
                                // MXFP4 code plane (two 4-bit codes a byte)
  const __half* d = nullptr;    // Q8_0 scale plane [rows][cols/32]
  const uint8_t* e = nullptr;   // MXFP4 scale plane [rows][cols/32] (E8M0: 2^(e - 127))
};

// ---------------------------------------------------------------------------------------
// One-launch decode step (batch 1, Q8_0 weights).
// ---------------------------------------------------------------------------------------
struct PersistLayer {
  PackedMat seg[6];               // W_q, W_k, W_v, F_a, G_a, W_beta  (rows [out][D])
  PackedMat wo;
  // the fused projection rows and W_o rearranged for the matrix cores (mma_order_* below)
  const int8_t* pw = nullptr;
  const uint16_t* pd = nullptr;
  const int8_t* ow = nullptr;
  const uint16_t* od = nullptr;
  // F_b and G_b rearranged for the matrix cores (gate_order_* below)
  const int8_t* fbw = nullptr;
  const uint16_t* fbd = nullptr;
  const int8_t* gbw = nullptr;
  const uint16_t* gbd = nullptr;
  const float* conv_w = nullptr;
  const float* a_log = nullptr;
  const float* dt_bias = nullptr;
  const float* o_norm_w = nullptr;
};

struct PersistParams {
  int n_layers = 0, D = 0, H = 0, dk = 0, dv = 0, C = 0, rank = 0, proj_rows = 0;
  int seg_first[6] = {};
  float eps = 0.f, l2_eps = 0.f, q_scale = 0.f;
  int gate_safe = 0;                     // 1: the lower-bounded gate (else KDA's)
  float gate_lb = 0.f;                   // its bound (log of alpha lies in (gate_lb, 0))
  const PersistLayer* layers = nullptr;  // device array [n_layers]
  float* S = nullptr;                    // [n_layers][H][dk][dv]
  float* win = nullptr;                  // [n_layers][3][C]
  const float* x_in = nullptr;           // [D]
  float* y_out = nullptr;                // [D]
  uint64_t* xbuf = nullptr;              // [2][D]      tagged residual stream
  uint64_t* pbuf = nullptr;              // [proj_rows] tagged projections
  uint64_t* obuf = nullptr;              // [V] tagged normalised, gated head outputs
  uint64_t* flags = nullptr;             // [3][kMaxPersistBlocks] tagged producer flags
  int* err = nullptr;                    // nonzero after a wait timed out (device word, kept
                                         // until the host resets it)
  int* err_host = nullptr;               // host-mapped copy of err: the host refuses further
                                         // steps on the model once it reads nonzero
  uint64_t timeout = 0;                  // wall-clock ticks a wait may take
  int poll_rounds = 48;                  // flag-poll rounds between two looks at the clock
  uint32_t epoch = 0;                    // token counter (tags = epoch * n_layers + layer + 1)
  int o_first_block = 0, o_blocks = 0;  // blocks [first, first + n) run the output projection,
                                         // 32 rows each
  int q_blocks = 0;                      // the projection blocks after them: the first q_blocks
                                         // take the q/k/v rows, 48 each, the next ones the
                                         // low-rank and beta rows, 16 each
};
constexpr int kMaxPersistBlocks = 1024;

// Q8_0 rows [0, rows) of up to six stacked matrices (segment i starts at row first[i]) with
// D columns, rearranged into the order the one-launch decode loads them in: tiles of 16
// rows, each 16 rows x D bytes as [4 waves][D/512 runs][2 halves][64 lanes][16 bytes] with
// the bytes as signed q (not q + 128), and the scales as [tile][4][64][D/512] fp16 bits.
// Rows past `rows` are zero.  Sizes: mma_order_bytes / mma_order_scales per matrix.
struct MmaSource {
  const uint8_t* w[6];
  const __half* d[6];
  int first[6];
  int nseg;
};
inline size_t mma_order_bytes(int rows, int D) { return (size_t)((rows + 15) / 16) * 16 * D; }
inline size_t mma_order_scales(int rows, int D) { return (size_t)((rows + 15) / 16) * 16 * (D / 32); }
hipError_t launch_mma_order(const MmaSource& src, int rows, int D, int8_t* w, uint16_t* d,
                            hipStream_t s);
// Q8_0 rows [0, rows) (rows a multiple of 16) of a matrix with `rank` columns (32, 64 or
// 128; NB = rank / 32 blocks per row), rearranged for the one-launch decode's gate tiles:
// per tile of 16 rows, [2 halves][NB blocks][16 rows][16 bytes] with the bytes as signed q
// (chunk (h, g, n) = bytes [32 g + 16 h, + 16) of row n), and the scales as [tile][NB][16]
// fp16 bits.  Sizes: rows * rank bytes and rows * NB scales.
hipError_t launch_gate_order(const uint8_t* w_src, const __half* d_src, int rows, int rank,
                             int8_t* w, uint16_t* d, hipStream_t s);
hipError_t launch_persistent(const PersistParams& p, int blocks, bool cooperative, hipStream_t s);
int persistent_max_blocks();            // co-resident blocks of one per CU, 0 if unavailable

}  // namespace kda

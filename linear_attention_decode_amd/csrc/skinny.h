// Q8_0, BF16 or MXFP4 weights times a few columns on the matrix cores (skinny.hip).
#pragma once
#include "kda_internal.h"

namespace kda {

// True when launch_skinny handles this product: Q8_0 weights, 8 < N <= 64 columns,
// K in {2048, 4096}; BF16 weights, 4 < N <= 64 columns, MXFP4 weights, 1 < N <= 64, K = 2048.
bool skinny_supported(int wt, int N, int K);
// True when launch_skinny handles a product whose Q8_0 matrices are in the one-launch
// decode's matrix-core order (GemvParams::mma): 1 <= N <= 64 columns, K in {1024, 2048}.
bool skinny_mma_supported(int N, int K);
// Device scratch the column preparation needs for N columns of length K.
size_t skinny_scratch_bytes(int N, int K);
// Same product, prologue and epilogue as launch_gemv(kQ8, prologue, g, ...), on MFMA.
hipError_t launch_skinny(int prologue, const GemvParams& g, void* scratch, hipStream_t s);

}  // namespace kda

// Host-side launch interface of the output projection (output.hip).  Not
// part of the public ABI.
#pragma once

#include "internal.hpp"

namespace mla {

struct OutputLaunch {
    int T, K, N;                 // rows, depth (H * V for u = W_O o), outputs (d_model)
    const void* x;               // [T][K] bf16
    const void* w;               // [N][K] bf16
    void* out;                   // [T][N] bf16
    float* part;                 // [kc][T][N] f32 depth-split partial sums
    int kc;                      // depth splits (output_splits)
    hipStream_t stream;
};

// Depth splits of the output projection for T rows (workspace partial slices).
int output_splits(int N, int K, long long T);
hipError_t launch_output(const OutputLaunch& a);

}  // namespace mla

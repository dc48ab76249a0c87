// Output projection of the attention layer, bf16: u = W_O [o_1; ...; o_H]
// ("DeepSeek-V2: MLA Explained", "MLA Full Formulas", section 3, the heads'
// outputs concatenated head after head and projected by W_O).  The decode's
// output o [T][H][V] is already that concatenation, row by row, so
//
//   u[t][n] = sum_k W[n][k] x[t][k],   x = o viewed as [T][H V], W = W_O.
//
// The weights (d_model x H V, 235 MB for DeepSeek-V3) dominate the traffic, so
// few rows run on the weight-streaming GEMM of stream_gemm.hpp with the depth
// split over workgroups (fp32 partial sums); a whole prompt's rows (1024 or
// more) on its 256 x 256 tile form.  A second kernel adds each output's
// partial sums in increasing split order (results do not depend on
// scheduling) and rounds to bf16.

#include "common.hpp"
#include "output.hpp"
#include "stream_gemm.hpp"

namespace mla {
namespace {

// grid: ceil(T N / 1024) workgroups of 256 threads, four consecutive outputs
// per thread (N % 32 == 0, so a thread's four never straddle a row).
__global__ __launch_bounds__(256) void output_finalize(const float* __restrict__ part, int kc, long long TN,
                                                       unsigned short* __restrict__ out) {
    const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= TN) return;
    f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
    for (int s = 1; s < kc; ++s) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(part + (size_t)s * TN + i);
        acc[0] += v[0];
        acc[1] += v[1];
        acc[2] += v[2];
        acc[3] += v[3];
    }
    u16x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = f32_to_bf16_bits(acc[e]);
    *reinterpret_cast<u16x4*>(out + i) = h;
}

}  // namespace

int output_splits(int N, int K, long long T) {
    if (T >= kQueryTileRows) return 1;
    return stream_gemm_splits(N, K, 32, T);
}

hipError_t launch_output(const OutputLaunch& a) {
    if (a.T == 0) return hipSuccess;
    const auto* x = static_cast<const unsigned short*>(a.x);
    const auto* w = static_cast<const unsigned short*>(a.w);
    if (a.T >= kQueryTileRows) {
        query_gemm_tiles<true><<<dim3((a.N + kBOut - 1) / kBOut, (a.T + kBRows - 1) / kBRows), 512, 0,
                                 a.stream>>>(x, a.T, a.K, w, nullptr, a.N, 2, 1, nullptr, 1.0f, nullptr,
                                             nullptr, 0, a.part);
    } else {
        const int n_ob = (a.N / 32 + kQWaves - 1) / kQWaves;
        stream_gemm_mfma<true><<<dim3(n_ob * a.kc, stream_gemm_row_groups(a.T)), kQWaves * kWave, 0, a.stream>>>(
            x, a.T, a.K, w, nullptr, a.N, 0, 2, 1, nullptr, 1.0f, nullptr, nullptr, a.part, n_ob);
    }
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const long long TN = (long long)a.T * a.N;
    output_finalize<<<(unsigned)((TN / 4 + 255) / 256), 256, 0, a.stream>>>(
        a.part, a.kc, TN, static_cast<unsigned short*>(a.out));
    return hipGetLastError();
}

}  // namespace mla

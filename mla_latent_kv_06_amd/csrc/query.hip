// Query path of MLA ("DeepSeek-V2: MLA Explained", "MLA Full Formulas",
// step 1, query compression), bf16 activations:
//
//   c_Q = W_DQ h                      stream_gemm_mfma (stream_gemm.hpp) with
//                                     the depth split across workgroups (fp32
//                                     partial sums)
//   c_Q = RMSNorm(c_Q) * gamma        optional: the latent norm V3 applies
//                                     after its compressed vectors ("KV
//                                     Compression -- DeepSeek-V3", "How it
//                                     works"); partial sums added in a fixed
//                                     order, c_Q rounded to bf16
//   q^C = W_UQ c_Q,  q^R = RoPE(W_QR c_Q)   stream_gemm_mfma over both weights;
//                                     the rotation is applied to the fp32
//                                     accumulators before the bf16 store
//
// With q_lora == 0 (full-rank queries) the last kernel reads h directly.
// The outputs are the decode's q_nope [T][H][N] and q_pe [T][H][R]: head
// blocks concatenated in head order, as the formula's [q_1; ...; q_H].

#include "common.hpp"
#include "query.hpp"
#include "stream_gemm.hpp"

namespace mla {
namespace {

// grid: T rows, 512 threads; DQ <= 2048 (validated).  Row t of c_Q: the
// partial sums of its kc chunks, added in increasing chunk order, then the
// optional RMSNorm * gamma, rounded to bf16.  Partial loads go out eight
// chunks at a time, unconditionally at clamped addresses (a load under a
// branch would be waited for inside it).
constexpr int kQFinThreads = 512;
__global__ __launch_bounds__(kQFinThreads) void query_latent_finalize(
    const float* __restrict__ part, int kc_count, int T, int DQ,
    const unsigned short* __restrict__ gamma, float eps, unsigned short* __restrict__ cq) {
    __shared__ float red[16];
    const int t = blockIdx.x, tid = threadIdx.x;
    constexpr int U = 4;                         // outputs per thread: o = tid + 512 u
    float x[U] = {0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < kc_count; g += 8) {
        float v[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int o = min(tid + kQFinThreads * u, DQ - 1);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kc = min(g + j, kc_count - 1);
                v[u][j] = part[((size_t)kc * T + t) * DQ + o] * (g + j < kc_count ? 1.f : 0.f);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j) x[u] += v[u][j];
    }
    float scale[U] = {1.f, 1.f, 1.f, 1.f};
    if (gamma != nullptr) {                      // uniform
        float ss = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (tid + kQFinThreads * u < DQ) ss += x[u] * x[u];
        ss = block_sum(ss, red);
        const float inv = 1.0f / sqrtf(ss / (float)DQ + eps);
#pragma unroll
        for (int u = 0; u < U; ++u)
            scale[u] = inv * bf16_bits_to_f32(gamma[min(tid + kQFinThreads * u, DQ - 1)]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int o = tid + kQFinThreads * u;
        if (o < DQ) cq[(size_t)t * DQ + o] = f32_to_bf16_bits(x[u] * scale[u]);
    }
}

}  // namespace

int query_splits(int d_q, int K, long long T) { return stream_gemm_splits(d_q, K, kNumCUs, T); }

hipError_t launch_query(const QueryLaunch& a) {
    if (a.T == 0) return hipSuccess;
    const unsigned short* x = static_cast<const unsigned short*>(a.h);
    int K = a.d_model;
    // many rows: 256 x 256 tiles, when the outputs fill whole tiles
    const bool tiles = a.T >= kQueryTileRows;
    if (a.q_lora > 0) {
        if (tiles && a.kc == 1 && a.q_lora % kBOut == 0) {
            query_gemm_tiles<true><<<dim3(a.q_lora / kBOut, (a.T + kBRows - 1) / kBRows), 512, 0, a.stream>>>(
                x, a.T, a.d_model, static_cast<const unsigned short*>(a.w_dq), nullptr, a.q_lora, 2, a.q_len,
                a.start_pos, a.rope_base, nullptr, nullptr, 0, a.part);
        } else {
            // c_Q partial sums: W_DQ as the single weight tensor, depth split a.kc ways
            const int n_ob = (a.q_lora / 32 + kQWaves - 1) / kQWaves;
            stream_gemm_mfma<true><<<dim3(n_ob * a.kc, stream_gemm_row_groups(a.T)), kQWaves * kWave, 0, a.stream>>>(
                x, a.T, a.d_model, static_cast<const unsigned short*>(a.w_dq), nullptr, a.q_lora, 0, 2, 1,
                a.start_pos, a.rope_base, nullptr, nullptr, a.part, n_ob);
        }
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
        query_latent_finalize<<<a.T, kQFinThreads, 0, a.stream>>>(
            a.part, a.kc, a.T, a.q_lora, static_cast<const unsigned short*>(a.gamma), a.eps, a.cq);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
        x = a.cq;
        K = a.q_lora;
    }
    const int HN = a.H * a.N, HR = a.H * a.R;
    if (tiles && HN % kBOut == 0 && HR % kBOut == 0 && a.R % 4 == 0) {
        query_gemm_tiles<false><<<dim3((HN + HR) / kBOut, (a.T + kBRows - 1) / kBRows), 512, 0, a.stream>>>(
            x, a.T, K, static_cast<const unsigned short*>(a.w_uq), static_cast<const unsigned short*>(a.w_qr), HN,
            a.R, a.q_len, a.start_pos, a.rope_base, static_cast<unsigned short*>(a.q_nope),
            static_cast<unsigned short*>(a.q_pe), HR, nullptr);
        return hipGetLastError();
    }
    const int n_mb = (HN + HR) / 32;
    const int n_ob = (n_mb + kQWaves - 1) / kQWaves;
    stream_gemm_mfma<false><<<dim3(n_ob, stream_gemm_row_groups(a.T)), kQWaves * kWave, 0, a.stream>>>(
        x, a.T, K, static_cast<const unsigned short*>(a.w_uq),
        static_cast<const unsigned short*>(a.w_qr), HN, HR, a.R, a.q_len, a.start_pos, a.rope_base,
        static_cast<unsigned short*>(a.q_nope), static_cast<unsigned short*>(a.q_pe), nullptr, n_ob);
    return hipGetLastError();
}

}  // namespace mla

// Latent-cache append: for every new token, x = W_kv,a h (d -> d_c + R), then
// [RMSNorm(x[0:d_c]) * gamma ; RoPE(x[d_c:], position)] is written into the
// token's paged slot ("KV Compression -- DeepSeek-V3", "How it works").
//
// Two kernels: a split-K projection writing fp32 partial sums to the
// workspace (for bf16 activations the weight-streaming MFMA GEMM of
// stream_gemm.hpp when d is a multiple of 64, else the MFMA kernel below;
// fp32 VALU for f32 activations), then one
// workgroup per token that adds the partials in a fixed order (so results do
// not depend on scheduling), normalises, rotates, rounds and stores.

#include "common.hpp"
#include "internal.hpp"
#include "stream_gemm.hpp"
#include "append_finalize.hpp"

namespace mla {
namespace {

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One wave per (32 outputs, 32 tokens, K chunk of at most kAppendChunk):
//   part[kc][t][o] = sum_{d in chunk} W[o][d] h[t][d]
// as x = h . W^T with both operands streamed straight from global memory;
// all of a chunk's fragments are loaded before the first MFMA, so a wave
// waits for memory once.  The result's lanes run along outputs, so each
// store instruction writes two full 128-byte rows of part.
//
// Work placement: the token blocks of one (output block, chunk) are
// neighbouring waves of one workgroup, so each W slice leaves HBM once and its
// second read hits the compute unit's caches.
// grid: P * kc_count workgroups, P = ceil(n_mb * n_nb / 4) per chunk.
__global__ __launch_bounds__(256) void append_gemm_mfma(const unsigned short* __restrict__ h,
                                                        const unsigned short* __restrict__ w,
                                                        int T, int d, int Dout, int kc_count,
                                                        int kchunk, float* __restrict__ part) {
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31, hf = lane >> 5;
    const int n_mb = Dout / 32, n_nb = (T + 31) / 32;
    const int P = (n_mb * n_nb + 3) / 4;
    const int kc = blockIdx.x / P;
    const int lj = (blockIdx.x - kc * P) * 4 + (threadIdx.x >> 6);
    const int nb = lj % n_nb, mb = lj / n_nb;
    if (kc >= kc_count || mb >= n_mb) return;
    const int o = mb * 32 + l32;
    const int t = nb * 32 + l32;
    const int k_lo = kc * kchunk, k_hi = min(d, k_lo + kchunk);
    const unsigned short* wp = w + (size_t)o * d + hf * 8;
    const unsigned short* hp = h + (size_t)min(t, T - 1) * d + hf * 8;
    const bool tok_ok = t < T;
    constexpr int NK = kAppendChunk / 16;
    bf16x8 av[NK], bv[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        const int k = k_lo + i * 16;
        av[i] = bf16x8{};
        bv[i] = bf16x8{};
        if (k < k_hi) {
            av[i] = *reinterpret_cast<const bf16x8*>(wp + k);
            if (tok_ok) bv[i] = *reinterpret_cast<const bf16x8*>(hp + k);
        }
    }
    f32x16 acc = {};
#pragma unroll
    for (int i = 0; i < NK; ++i) acc = mfma32(bv[i], av[i], acc);
    // acc[i] of lane (hf, l32): token nb*32 + 8 (i/4) + 4 hf + i%4, output o
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int tt = nb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (tt < T) part[((size_t)kc * T + tt) * Dout + o] = acc[i];
    }
}

// grid: ceil(T * Dout / 256); one thread per (token, output), whole K.
template <int ADT>
__global__ __launch_bounds__(256) void append_gemm_generic(const void* __restrict__ h,
                                                           const void* __restrict__ w, int T, int d,
                                                           int Dout, float* __restrict__ part) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long long)T * Dout) return;
    const int t = (int)(i / Dout), o = (int)(i % Dout);
    float acc = 0.f;
    for (int k = 0; k < d; ++k)
        acc += load_act<ADT>(w, (size_t)o * d + k) * load_act<ADT>(h, (size_t)t * d + k);
    part[i] = acc;
}

// grid: T tokens, 256 threads: append_finalize_token for token blockIdx.x.
template <int ADT, int CDT>
__global__ __launch_bounds__(256) void append_finalize(
    const float* __restrict__ part, int kc_count, int T, int DC, int DR,
    const void* __restrict__ gamma, float eps, float rope_base,
    const int* __restrict__ block_table, int max_blocks, const int* __restrict__ start_pos,
    int n_new, int BSZ, void* __restrict__ pool, float* __restrict__ pool_scale) {
    append_finalize_token<ADT, CDT>(blockIdx.x, part, kc_count, T, DC, DR, gamma, eps, rope_base,
                                    block_table, max_blocks, start_pos, n_new, BSZ, pool, pool_scale);
}

template <int ADT, int CDT>
hipError_t finalize(const AppendLaunch& a) {
    const int T = a.batch * a.n_new;
    append_finalize<ADT, CDT><<<T, 256, 0, a.stream>>>(
        a.part, a.kc, T, a.DC, a.DR, a.gamma, a.eps, a.rope_base, a.block_table, a.max_blocks,
        a.start_pos, a.n_new, a.BS, a.pool, a.pool_scale);
    return hipGetLastError();
}

}  // namespace

int append_stream_splits(int Dout, int d_model, long long T) {
    // the finalize adds at most 32 partial slices on its fast path
    return stream_gemm_splits(Dout, d_model, 32, T);
}

hipError_t launch_append_project(const AppendLaunch& a, bool mfma_gemm) {
    const int T = a.batch * a.n_new;
    if (T == 0) return hipSuccess;
    const int Dout = a.DC + a.DR;
    if (mfma_gemm && a.stream_gemm && a.kc == 1 && T >= kQueryTileRows && Dout % 4 == 0) {
        // a whole prompt: the 256 x 256 tile form, fp32 rows straight into the one slice
        query_gemm_tiles<true><<<dim3((Dout + kBOut - 1) / kBOut, (T + kBRows - 1) / kBRows), 512, 0, a.stream>>>(
            static_cast<const unsigned short*>(a.h), T, a.d_model, static_cast<const unsigned short*>(a.w_kv_a),
            nullptr, Dout, 2, 1, nullptr, 1.0f, nullptr, nullptr, 0, a.part);
    } else if (mfma_gemm && a.stream_gemm) {
        const int n_ob = (Dout / 32 + kQWaves - 1) / kQWaves;
        const dim3 grid(n_ob * a.kc, stream_gemm_row_groups(T));
        stream_gemm_mfma<true><<<grid, kQWaves * kWave, 0, a.stream>>>(
            static_cast<const unsigned short*>(a.h), T, a.d_model,
            static_cast<const unsigned short*>(a.w_kv_a), nullptr, Dout, 0, 2, 1, nullptr, 1.0f, nullptr,
            nullptr, a.part, n_ob);
    } else if (mfma_gemm) {
        const int P = ((Dout / 32) * ((T + 31) / 32) + 3) / 4;
        append_gemm_mfma<<<P * a.kc, 256, 0, a.stream>>>(
            static_cast<const unsigned short*>(a.h), static_cast<const unsigned short*>(a.w_kv_a), T,
            a.d_model, Dout, a.kc, a.kchunk, a.part);
    } else {
        const long long n = (long long)T * Dout;
        const unsigned grid = (unsigned)((n + 255) / 256);
        if (a.act_dtype == MLA_BF16)
            append_gemm_generic<MLA_BF16><<<grid, 256, 0, a.stream>>>(a.h, a.w_kv_a, T, a.d_model, Dout, a.part);
        else
            append_gemm_generic<MLA_F32><<<grid, 256, 0, a.stream>>>(a.h, a.w_kv_a, T, a.d_model, Dout, a.part);
    }
    return hipGetLastError();
}

hipError_t launch_append_finalize(const AppendLaunch& a) {
    if (a.batch * a.n_new == 0) return hipSuccess;
    if (a.act_dtype == MLA_BF16) {
        if (a.cache_dtype == MLA_BF16) return finalize<MLA_BF16, MLA_BF16>(a);
        if (a.cache_dtype == MLA_FP8_E4M3) return finalize<MLA_BF16, MLA_FP8_E4M3>(a);
        return finalize<MLA_BF16, MLA_F32>(a);
    }
    if (a.cache_dtype == MLA_BF16) return finalize<MLA_F32, MLA_BF16>(a);
    if (a.cache_dtype == MLA_FP8_E4M3) return finalize<MLA_F32, MLA_FP8_E4M3>(a);
    return finalize<MLA_F32, MLA_F32>(a);
}

hipError_t launch_append(const AppendLaunch& a, bool mfma_gemm) {
    if (hipError_t e = launch_append_project(a, mfma_gemm); e != hipSuccess) return e;
    return launch_append_finalize(a);
}

}  // namespace mla

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
constexpr int kQueryTileRows = 1024;             // rows from which the 256 x 256 tile kernel runs
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

// Many rows (a whole prompt): 256 outputs x 256 rows per workgroup of 8
// waves, two per SIMD; wave w owns outputs 64 (w % 4) .. +64 for rows 128
// (w / 4) .. +128 (8 accumulators, outputs on the MFMA rows).  The depth
// streams in 64-column chunks through the buffer-to-LDS path, two stages
// deep, 8 copies per wave per chunk (instruction i = w + 8 j covers rows
// 8 i .. +8 of the stage: weights, then activations), in the XOR tile
// layout of the streaming GEMM.  Output tiles never straddle the two weight
// tensors (both are whole multiples of 256 rows).
//   DOWN: fp32 c_Q partials part[row][o] (one depth slice).
//   else: q^C (bf16) or, past HN, q^R turned by RoPE: a lane holds four
//         consecutive outputs of one row, so each rotary pair is in-lane.
constexpr int kBRows = 256;
constexpr int kBOut = 256;
constexpr int kBStage = (kBOut + kBRows) * 128;      // 64 KB
constexpr int kBOutStride = 144;
constexpr int kBLds = 8 * 128 * kBOutStride > 2 * kBStage ? 8 * 128 * kBOutStride : 2 * kBStage;

template <bool DOWN>
__global__ __launch_bounds__(512, 1) void query_gemm_tiles(
    const unsigned short* __restrict__ x, int T, int K,
    const unsigned short* __restrict__ w0, const unsigned short* __restrict__ w1, int N0, int R,
    int q_len, const int* __restrict__ start_pos, float rope_base,
    unsigned short* __restrict__ out0, unsigned short* __restrict__ out1, int N1,
    float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kBLds];
    MLA_LDS unsigned char* lds = (MLA_LDS unsigned char*)smem;
    const int o0 = blockIdx.x * kBOut, r0 = blockIdx.y * kBRows;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hf = lane >> 5;
    const int r8 = lane >> 3, s8 = lane & 7;
    const int wo = w & 3, wt = w >> 2;
    const bool second = o0 >= N0;                     // uniform: the tile's weight tensor
    const unsigned short* wbase = second ? w1 + (size_t)(o0 - N0) * K : w0 + (size_t)o0 * K;
    const int rows_left = T - r0;
    const __amdgpu_buffer_rsrc_t w_r = make_rsrc(wbase, kBOut * K * 2);
    const __amdgpu_buffer_rsrc_t x_r = make_rsrc(x + (size_t)r0 * K, (rows_left < kBRows ? rows_left : kBRows) * K * 2);
    unsigned voff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int i = w + 8 * j;
        const int row = 8 * (j < 4 ? i : i - 32) + r8;
        voff[j] = (unsigned)row * (unsigned)(K * 2) + (unsigned)((s8 ^ qswz(row)) << 4);
    }
    const int n_chunks = K / 64;
    auto issue = [&](int c) {
        MLA_LDS unsigned char* st = lds + (c & 1) * kBStage;
        const unsigned col = c < n_chunks ? (unsigned)c * 128u : 0x80000000u;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(j < 4 ? w_r : x_r, (MLA_LDS void*)(st + (w + 8 * j) * 1024), 16,
                                                     voff[j] + col, 0, 0, 0);
    };
    f32x16 acc[2][4];
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[ob][tb] = f32x16{};
    issue(0);
    for (int c = 0; c < n_chunks; ++c) {
        stage_barrier();                              // everyone is done with chunk c - 1's stage
        issue(c + 1);
        __builtin_amdgcn_s_waitcnt(0x0F70 | 8);       // vmcnt(8): this wave's copies of chunk c landed
        stage_barrier();                              // ... and everyone's
        const MLA_LDS unsigned char* st = lds + (c & 1) * kBStage;
#pragma unroll
        for (int sx = 0; sx < 4; ++sx) {
            const int cx = 2 * sx + hf;
            bf16x8 wf[2], xf[4];
#pragma unroll
            for (int ob = 0; ob < 2; ++ob) {
                const int row = 64 * wo + 32 * ob + l32;
                wf[ob] = *reinterpret_cast<const MLA_LDS bf16x8*>(st + (8 * row + (cx ^ qswz(row))) * 16);
            }
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int row = 128 * wt + 32 * tb + l32;
                xf[tb] = *reinterpret_cast<const MLA_LDS bf16x8*>(st + kBOut * 128 + (8 * row + (cx ^ qswz(row))) * 16);
            }
#pragma unroll
            for (int ob = 0; ob < 2; ++ob)
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) acc[ob][tb] = sg_mfma32(wf[ob], xf[tb], acc[ob][tb]);
        }
    }
    wait_vmem_0();                                    // the record-less copies of the last chunk too
    __syncthreads();                                  // stages free for the store staging

    // acc[ob][tb][i]: output o0 + 64 wo + 32 ob + 8 (i/4) + 4 hf + i%4 of row
    // r0 + 128 wt + 32 tb + l32
    if constexpr (DOWN) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int tt = r0 + 128 * wt + 32 * tb + l32;
            if (tt >= T) continue;
#pragma unroll
            for (int ob = 0; ob < 2; ++ob)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 v = {acc[ob][tb][4 * g], acc[ob][tb][4 * g + 1], acc[ob][tb][4 * g + 2],
                                     acc[ob][tb][4 * g + 3]};
                    *reinterpret_cast<f32x4*>(part + (size_t)tt * N0 + o0 + 64 * wo + 32 * ob + 8 * g + 4 * hf) = v;
                }
        }
        return;
    }
    MLA_LDS unsigned char* ost = lds + w * (128 * kBOutStride);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int rl = 32 * tb + l32;                 // row within the wave's 128
        const int tc = min(r0 + 128 * wt + rl, T - 1);
        const int b = tc / q_len;
        const int pos = second ? start_pos[b] + (tc - b * q_len) : 0;
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[ob][tb][4 * g + e];
                if (second) {
                    // rotary pairs (v[0], v[1]) and (v[2], v[3]): channels
                    // r, r + 1 of a head's R, r even
#pragma unroll
                    for (int pr = 0; pr < 2; ++pr) {
                        const int orot = o0 - N0 + 64 * wo + 32 * ob + 8 * g + 4 * hf + 2 * pr;
                        const int r = orot % R;
                        const double inv_freq = pow((double)rope_base, -2.0 * (double)(r >> 1) / (double)R);
                        const double ang = (double)pos * inv_freq;
                        const double turns = rint(ang * 0.15915494309189535);
                        float sn, cs;
                        sincosf((float)fma(-turns, 6.283185307179586, ang), &sn, &cs);
                        const float x0 = v[2 * pr], x1 = v[2 * pr + 1];
                        v[2 * pr] = x0 * cs - x1 * sn;
                        v[2 * pr + 1] = x0 * sn + x1 * cs;
                    }
                }
                u16x4 hv;
#pragma unroll
                for (int e = 0; e < 4; ++e) hv[e] = f32_to_bf16_bits(v[e]);
                *reinterpret_cast<MLA_LDS u16x4*>(ost + rl * kBOutStride + (32 * ob + 8 * g + 4 * hf) * 2) = hv;
            }
    }
    // LDS operations of one wave complete in order: the reads see the writes
    const int n_out = second ? N1 : N0;
    unsigned short* dst = (second ? out1 : out0) + (second ? o0 - N0 : o0) + 64 * wo;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int rl = 8 * k + r8;
        const int tt = r0 + 128 * wt + rl;
        const u32x4 v = *reinterpret_cast<const MLA_LDS u32x4*>(ost + rl * kBOutStride + s8 * 16);
        if (tt < T) *reinterpret_cast<u32x4*>(dst + (size_t)tt * n_out + s8 * 8) = v;
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

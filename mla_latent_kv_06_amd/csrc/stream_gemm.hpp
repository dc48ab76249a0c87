// Weight-streaming MFMA GEMM for few rows (bf16): y = W x^T for every one of
// T rows of x, with W's rows (outputs) and x's rows both streamed HBM -> LDS;
// and its 256 x 256 tile form for many rows (a whole prompt).  Used by the
// query path (query.hip) and the cache append (append.hip).
// Kernel code only: included by the .hip files that launch it.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace mla {
namespace {

__device__ __forceinline__ f32x16 sg_mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// [W_UQ; W_QR] x^T (x = c_Q, or h for full-rank queries; any single weight
// tensor when HR == 0).  A workgroup of
// kQWaves waves owns 32 kQWaves consecutive outputs (wave w: outputs
// 32 w .. +32 of them) and computes them for every query row, in passes of
// kQRows rows.  The depth K is walked in chunks of 64 columns; each chunk of
// the workgroup's weight rows and of the pass's query rows is copied HBM ->
// LDS by the buffer-to-LDS path (no VGPR round trip), kQStages chunks deep,
// so kQStages - 1 chunks are in flight while one is multiplied.  (Measured on
// the V3 up-projection: 2-3 stages stream the weights at ~3 TB/s, 6 stages
// at ~2.6 TB/s; more copies in flight do not help this access pattern.)
//
// Copies: instruction i of a tile covers rows 8 i .. 8 i + 7 (8 lanes of 16
// bytes per 128-byte row); each wave issues the same number per stage (4 of
// the weight tile, 4 of the query tile), so s_waitcnt vmcnt(8 (kQStages - 1))
// says its copies of the oldest stage have landed, and a barrier makes that
// true for the workgroup.  Rows past the tensors' ends are outside the
// buffer resources and read nothing; their results are never stored.
//
// LDS tiles: chunk c (8 columns) of row t sits at 16-byte slot 8 t + (c ^
// g(t)), the XOR pattern of the split-KV tiles, so the 16-byte reads of 32
// consecutive rows (one MFMA operand) spread over the banks.
//
// acc[nb][i] of lane (hf, l32): row r0 + nb*32 + 8 (i/4) + 4 hf + i%4,
// output o.  RoPE pairs (x[2k], x[2k+1]) of a head's rotary block sit in
// lanes l32 and l32 ^ 1 (R is even and a block starts at a multiple of 32),
// exchanged with one DPP move.  The angle pos * base^(-2k/R) is formed in
// double and reduced modulo 2 pi before the fp32 sine / cosine, as in the
// cache append.
constexpr int kQWaves = 3;
constexpr int kQRows = 96;                        // query rows per pass (3 MFMA row blocks)
constexpr int kQStages = 3;
constexpr int kQTileBytes = 96 * 128;             // 96 rows x 64 bf16
__device__ __forceinline__ int qswz(int t) {
    return (((t & 3) << 1) | ((t >> 2) & 1)) ^ ((t >> 2) & 2);
}
__device__ __forceinline__ void wait_vmem_16() {
    // s_waitcnt vmcnt(16) (= 8 (kQStages - 1)): vmcnt bits 3:0 and 15:14;
    // expcnt / lgkmcnt unconstrained
    __builtin_amdgcn_s_waitcnt(0x0F70 | (16 & 15) | ((16 >> 4) << 14));
}
__device__ __forceinline__ void wait_vmem_0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Workgroup barrier that waits for this wave's LDS operations only: the
// copies of later stages stay in flight across it (a plain __syncthreads
// would also wait for them).
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// Buffer resource over [base, base + bytes): raw (untyped) access, gfx9 word 3.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

//
// A grid with gridDim.y > 1 spreads the row passes over workgroups (many
// rows: the weights are then re-read per pass, from the caches).
//
// PART (the query down-projection): one weight tensor (w_uq = W_DQ, HN its
// rows, HR = 0), the depth split over gridDim.x / n_ob workgroups, each
// writing fp32 partial sums part[split][row][output] for the finalize.
template <bool PART>
__global__ __launch_bounds__(kQWaves * kWave) void stream_gemm_mfma(
    const unsigned short* __restrict__ x, int T, int K,
    const unsigned short* __restrict__ w_uq, const unsigned short* __restrict__ w_qr,
    int HN, int HR, int R, int q_len, const int* __restrict__ start_pos, float rope_base,
    unsigned short* __restrict__ q_nope, unsigned short* __restrict__ q_pe,
    float* __restrict__ part, int n_ob) {
    static_assert(8 * (kQStages - 1) == 16, "wait_vmem_16 counts the copies of kQStages - 1 stages");
    __shared__ __attribute__((aligned(16))) unsigned char smem[kQStages * 2 * kQTileBytes];
    MLA_LDS unsigned char* lds = (MLA_LDS unsigned char*)smem;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hf = lane >> 5;
    const int ob = PART ? (int)blockIdx.x % n_ob : (int)blockIdx.x;
    const int split = PART ? (int)blockIdx.x / n_ob : 0;
    const int o_wg = ob * 32 * kQWaves;           // first output of the workgroup
    const int o = o_wg + 32 * w + l32;
    const int n_out = HN + HR;
    const bool active = o_wg + 32 * w < n_out;    // uniform per wave
    const bool rot = active && o_wg + 32 * w >= HN;
    const int row_bytes = K * 2;
    // chunks of 64 columns this workgroup walks: [c_lo, c_lo + n_chunks)
    const int all_chunks = K / 64;
    const int per_split = PART ? (all_chunks + (int)gridDim.x / n_ob - 1) / ((int)gridDim.x / n_ob)
                               : all_chunks;
    const int c_lo = min(all_chunks, split * per_split);
    const int n_chunks = min(all_chunks, c_lo + per_split) - c_lo;

    // this lane's part of a copy instruction: row 8 i + r8, 16-byte slot s8
    const int r8 = lane >> 3, s8 = lane & 7;
    // weight rows of copy instruction i (wave w issues i = w, w + 3, w + 6, w + 9)
    __amdgpu_buffer_rsrc_t wrs[4];
    unsigned wvo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = w + kQWaves * j;
        const int row = o_wg + 8 * i;              // first row of the instruction (uniform)
        const bool in_qr = row >= HN;
        const unsigned short* base = in_qr ? w_qr : w_uq;
        const int rows_avail = in_qr ? HR : HN;
        wrs[j] = make_rsrc(base, rows_avail * row_bytes);
        const int rr = (in_qr ? row - HN : row) + r8;
        wvo[j] = (unsigned)rr * row_bytes + (unsigned)((s8 ^ qswz(8 * i + r8)) << 4);
    }
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, T * row_bytes);

    // row passes: this workgroup takes passes blockIdx.y, blockIdx.y + gridDim.y, ...
    for (int r0 = (int)blockIdx.y * kQRows; r0 < T; r0 += kQRows * (int)gridDim.y) {
        const int nbs = min(3, (T - r0 + 31) / 32);
        unsigned xvo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = w + kQWaves * j;
            xvo[j] = (unsigned)(r0 + 8 * i + r8) * row_bytes + (unsigned)((s8 ^ qswz(8 * i + r8)) << 4);
        }
        // chunk c into stage c % kQStages.  A chunk past the end is issued
        // all the same (the wait counts stay fixed) at an offset beyond every
        // resource's range (offsets stay below 2^31), so it reads nothing.
        auto issue = [&](int c) {
            MLA_LDS unsigned char* st = lds + (c % kQStages) * 2 * kQTileBytes;
            const unsigned col = c < n_chunks ? (unsigned)(c_lo + c) * 128u : 0x80000000u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = w + kQWaves * j;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs[j], (MLA_LDS void*)(st + i * 1024), 16,
                                                         wvo[j] + col, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (MLA_LDS void*)(st + kQTileBytes + i * 1024),
                                                         16, xvo[j] + col, 0, 0, 0);
            }
        };
        f32x16 acc[3] = {f32x16{}, f32x16{}, f32x16{}};
#pragma unroll
        for (int c = 0; c < kQStages - 1; ++c) issue(c);
        for (int c = 0; c < n_chunks; ++c) {
            stage_barrier();                      // everyone is done with chunk c - 1's stage
            issue(c + kQStages - 1);
            wait_vmem_16();                       // this wave's copies of chunk c landed
            stage_barrier();                      // ... and everyone's
            const MLA_LDS unsigned char* st = lds + (c % kQStages) * 2 * kQTileBytes;
            // all of the chunk's fragments first, then the MFMAs: one LDS
            // round trip per chunk.  Row blocks past the pass's rows multiply
            // stale LDS data; MFMA rows are independent and those are never
            // stored.
            const int wrow = 32 * w + l32;
            bf16x8 wf[4], xf[3][4];
#pragma unroll
            for (int sx = 0; sx < 4; ++sx) {
                const int cx = 2 * sx + hf;       // 16-byte column slot of K-step sx
                wf[sx] = *reinterpret_cast<const MLA_LDS bf16x8*>(st + (8 * wrow + (cx ^ qswz(wrow))) * 16);
#pragma unroll
                for (int nb = 0; nb < 3; ++nb) {
                    const int xrow = 32 * nb + l32;
                    xf[nb][sx] = *reinterpret_cast<const MLA_LDS bf16x8*>(
                        st + kQTileBytes + (8 * xrow + (cx ^ qswz(xrow))) * 16);
                }
            }
#pragma unroll
            for (int sx = 0; sx < 4; ++sx)
#pragma unroll
                for (int nb = 0; nb < 3; ++nb) acc[nb] = sg_mfma32(xf[nb][sx], wf[sx], acc[nb]);
        }
        wait_vmem_0();                            // the record-less copies too
        __syncthreads();                          // before the next pass reuses the stages
        if (!active) continue;
        if constexpr (PART) {
#pragma unroll
            for (int nb = 0; nb < 3; ++nb) {
                if (nb >= nbs) break;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int tt = r0 + nb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
                    if (tt < T) part[((size_t)split * T + tt) * HN + o] = acc[nb][i];
                }
            }
            continue;
        }

        const int orot = o - HN;
        const int r = rot ? orot % R : 0;
        const bool odd = r & 1;
        const double inv_freq = pow((double)rope_base, -2.0 * (double)(r >> 1) / (double)R);
#pragma unroll
        for (int nb = 0; nb < 3; ++nb) {
            if (nb >= nbs) break;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int tt = r0 + nb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
                const float v = acc[nb][i];
                if (!rot) {
                    if (tt < T) q_nope[(size_t)tt * HN + o] = f32_to_bf16_bits(v);
                    continue;
                }
                // partner of the pair: lane l32 ^ 1 (quad permutation 1, 0, 3, 2)
                const float pv = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                                               __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
                const int tc = min(tt, T - 1);
                const int b = tc / q_len;
                const int pos = start_pos[b] + (tc - b * q_len);
                const double ang = (double)pos * inv_freq;
                const double turns = rint(ang * 0.15915494309189535);
                float sn, cs;
                sincosf((float)fma(-turns, 6.283185307179586, ang), &sn, &cs);
                const float x0 = odd ? pv : v, x1 = odd ? v : pv;
                const float y = odd ? x0 * sn + x1 * cs : x0 * cs - x1 * sn;
                if (tt < T) q_pe[(size_t)tt * HR + orot] = f32_to_bf16_bits(y);
            }
        }
    }
}

// Many rows (a whole prompt): 256 outputs x 256 rows per workgroup of 8
// waves, two per SIMD; wave w owns outputs 64 (w % 4) .. +64 for rows 128
// (w / 4) .. +128 (8 accumulators, outputs on the MFMA rows).  The depth
// streams in 64-column chunks through the buffer-to-LDS path, two stages
// deep, 8 copies per wave per chunk (instruction i = w + 8 j covers rows
// 8 i .. +8 of the stage: weights, then activations), in the XOR tile
// layout of the streaming GEMM.  Output tiles never straddle the two weight
// tensors (the first one is a whole multiple of 256 rows); in DOWN mode the
// last tile may be partial: its missing weight rows read nothing and its
// outputs past N0 are not stored.
//   DOWN: fp32 c_Q partials part[row][o] (one depth slice).
//   else: q^C (bf16) or, past HN, q^R turned by RoPE: a lane holds four
//         consecutive outputs of one row, so each rotary pair is in-lane.
constexpr int kQueryTileRows = 1024;             // rows from which the tile form runs
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
    const int w_rows = second ? kBOut : (N0 - o0 < kBOut ? N0 - o0 : kBOut);
    const __amdgpu_buffer_rsrc_t w_r = make_rsrc(wbase, w_rows * K * 2);
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
                    const int o = o0 + 64 * wo + 32 * ob + 8 * g + 4 * hf;     // N0 % 4 == 0
                    const f32x4 v = {acc[ob][tb][4 * g], acc[ob][tb][4 * g + 1], acc[ob][tb][4 * g + 2],
                                     acc[ob][tb][4 * g + 3]};
                    if (o < N0) *reinterpret_cast<f32x4*>(part + (size_t)tt * N0 + o) = v;
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

// Row-pass groups (gridDim.y) for T rows: one pass of kQRows rows each.
inline int stream_gemm_row_groups(long long T) {
    const long long g = (T + kQRows - 1) / kQRows;
    return (int)(g < 1 ? 1 : (g > 65535 ? 65535 : g));
}

// Depth splits for the PART mode: enough workgroups for the compute units
// together with the row-pass groups, at most max_splits and at most one per
// 64-column chunk (1 once the row passes alone fill the chip).
inline int stream_gemm_splits(int n_out, int K, int max_splits, long long T) {
    const long long n_ob = (n_out / 32 + kQWaves - 1) / kQWaves;
    const long long s = kNumCUs / (n_ob * stream_gemm_row_groups(T));
    return (int)(s < 1 ? 1 : (s > max_splits ? max_splits : (s > K / 64 ? K / 64 : s)));
}

}  // namespace
}  // namespace mla

// MLA prefill in the decompressed form, DeepSeek-V3 head shape (128 heads,
// latent 512, rotary 64, q_nope 128, v_head 128, cache blocks of 64 tokens).
//
// A prompt's attention costs 2 H (N + R + V) = 2 H 320 flops per (query, key)
// pair when keys and values are rebuilt from the latent ("DeepSeek-V2: MLA
// Explained", "MLA Full Formulas": k^C = W_UK c, v^C = W_UV c, keys
// [k^C ; k^R]), against 2 H (d_c + R + d_c) = 2 H 1088 in the absorbed form
// the decode uses.  With many query rows per sequence the rebuild is paid
// once per token and shared by every query, so prefill rebuilds:
//
//  1. gather:      the sequence's cache rows (paged) -> contiguous latents X
//                  [b][t][512] and rotary keys KR [b][t][64], bf16; an fp8
//                  cache gives X the codes' exact values, KR the dequantised
//                  values rounded to bf16, and its token scales to TS.
//  2. decompress:  K^C[b][h][t][:] = W_UK[h] X[b][t] and V^T[b][h][:][t] =
//                  W_UV[h] X[b][t] (times the token scale), bf16, on MFMA;
//                  V^T rows hold each 16-key group in the order the
//                  attention's softmax weights take (keys 0-3, 8-11, 4-7,
//                  12-15).
//  3. attention:   causal softmax attention of each head's queries [q^C ; q^R]
//                  over its keys [K^C ; KR] and values V, MFMA with an online
//                  softmax; query s of a sequence of L tokens and q_len queries
//                  sees tokens 0 .. L - q_len + s (the decode's rule).
//
// Workspace rows of sequence b start at b * Tpad (Tpad = max_blocks * 64
// rounded up to 256), so the host never reads lengths.  Token tiles past a
// sequence's length are skipped by every kernel; the gather zeroes the rows
// between the length and the next multiple of 256, which the decompression
// reads.

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"
#include "prefill.hpp"

namespace mla {
namespace {

constexpr int PH = 128;                 // heads
constexpr int PDC = 512;                // latent width
constexpr int PDR = 64;                 // rotary width
constexpr int PN = 128;                 // q_nope / k^C width
constexpr int PV = 128;                 // value width
constexpr int PBS = 64;                 // tokens per cache block
constexpr int kDTok = 256;              // tokens per rebuild tile (workspace rows round up to it)

__device__ __forceinline__ f32x16 pf_mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// XOR slot pattern of the LDS tiles: 16-byte chunk c of row t sits at slot
// c ^ g(t) of the row's 8 slots, so that the 16-byte reads of 16 consecutive
// rows at one chunk, and the 8-byte transposed reads of 4 rows x 2 chunks,
// land on disjoint banks.
__device__ __forceinline__ int pswz(int t) {
    return (((t & 3) << 1) | ((t >> 2) & 1)) ^ ((t >> 2) & 2);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t p_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt vmcnt(N), expcnt / lgkmcnt unconstrained (vmcnt: bits 3:0, 15:14)
template <int N>
__device__ __forceinline__ void p_wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier after this wave's LDS operations only: buffer-to-LDS
// copies of later stages stay in flight across it.
__device__ __forceinline__ void p_stage_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ int seq_len_of(const int* __restrict__ seq_lens, int b, int Tmax) {
    return min(max(seq_lens[b], 0), Tmax);
}

// ---------------------------------------------------------------------------
// 1. gather
// ---------------------------------------------------------------------------

// grid: batch * Tpad / 64 workgroups of 256; workgroup (b, k) handles tokens
// 64 k .. +64 of sequence b (cache block k of its table).
__global__ __launch_bounds__(256) void prefill_gather_kernel(
    const unsigned char* __restrict__ pool, const float* __restrict__ pool_scale, int fp8,
    const int* __restrict__ block_table, int max_blocks, const int* __restrict__ seq_lens,
    int Tmax, int Tpad, unsigned short* __restrict__ x, unsigned short* __restrict__ kr,
    float* __restrict__ ts) {
    const int per = Tpad / PBS;
    const int b = blockIdx.x / per, k = blockIdx.x - b * per;
    const int len = seq_len_of(seq_lens, b, Tmax);
    const int lim = (len + kDTok - 1) / kDTok * kDTok;   // the rebuild reads whole tiles
    if (k * PBS >= lim) return;
    const long long blk = k * PBS < len ? block_table[(size_t)b * max_blocks + k] : 0;
    const size_t row0 = (size_t)b * Tpad + (size_t)k * PBS;
    const int tid = threadIdx.x;
    if (!fp8) {
        // token-major rows: thread p takes chunk c (8 channels) of token r, so
        // consecutive threads read and write consecutive 16 bytes
        const unsigned short* src = reinterpret_cast<const unsigned short*>(pool) + (size_t)blk * PBS * (PDC + PDR);
        for (int p = tid; p < PBS * 72; p += 256) {          // 72 chunks of 8 channels per token
            const int r = p / 72, c = p - r * 72;
            const int t = k * PBS + r;
            const u16x8 v = t < len ? *reinterpret_cast<const u16x8*>(src + (size_t)r * (PDC + PDR) + c * 8)
                                    : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
            unsigned short* dst = c < 64 ? x + (row0 + r) * PDC + c * 8 : kr + (row0 + r) * PDR + (c - 64) * 8;
            *reinterpret_cast<u16x8*>(dst) = v;
        }
        return;
    }
    const unsigned char* src = pool + (size_t)blk * PBS * (PDC + PDR);
    const float* ssrc = pool_scale + (size_t)blk * PBS;
    for (int p = tid; p < PBS * 36; p += 256) {               // 36 chunks of 16 codes per row
        const int r = p / 36, c = p - r * 36;
        const int t = k * PBS + r;
        const bool live = t < len;
        const u32x4 raw = live ? *reinterpret_cast<const u32x4*>(src + ((size_t)r * 36 + c) * 16)
                               : u32x4{0u, 0u, 0u, 0u};
        const float s = live ? ssrc[r] : 0.f;
        if (c < 32) {
            // latent codes as their exact bf16 values; the scale is applied
            // to the decompressed keys and values
            u32x4 o[2];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                o[q >> 1][(q & 1) * 2 + 0] = __builtin_bit_cast(
                    unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[q], 1.0f, false));
                o[q >> 1][(q & 1) * 2 + 1] = __builtin_bit_cast(
                    unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[q], 1.0f, true));
            }
            unsigned short* dst = x + (row0 + r) * PDC + c * 16;
            *reinterpret_cast<u32x4*>(dst) = o[0];
            *reinterpret_cast<u32x4*>(dst + 8) = o[1];
            if (c == 0) ts[row0 + r] = s;
        } else {
            // rotary codes dequantised (code * scale) and rounded to bf16
            u16x8 o[2];
#pragma unroll
            for (int e = 0; e < 16; ++e)
                o[e >> 3][e & 7] = f32_to_bf16_bits(e4m3_to_f32((raw[e >> 2] >> (8 * (e & 3))) & 0xFFu) * s);
            unsigned short* dst = kr + (row0 + r) * PDR + (c - 32) * 16;
            *reinterpret_cast<u16x8*>(dst) = o[0];
            *reinterpret_cast<u16x8*>(dst + 8) = o[1];
        }
    }
}

// ---------------------------------------------------------------------------
// 2. decompression
// ---------------------------------------------------------------------------

// grid: H * (batch * Tpad / 256, rounded up to a multiple of 4) workgroups
// of 512.  Workgroup (h, b,
// tile) computes, for tokens t0 .. t0 + 256 of sequence b, the 256 outputs
// [W_UK[h] ; W_UV[h]] X^T: wave w owns outputs 64 (w % 4) .. +64 (waves with
// w % 4 < 2 the keys, the others the values) for tokens 128 (w / 4) .. +128.
// The depth 512 is walked in chunks of 64 columns, copied HBM -> LDS by the
// buffer-to-LDS path two stages deep (one chunk in flight while one is
// multiplied): per stage 256 weight rows and 256 token rows of 128 bytes, 64
// copy instructions, 8 per wave.  Instruction i covers rows 8 i .. 8 i + 7 of
// the stage (weights, then tokens), LDS bytes 1024 i .. +1024.  Two waves per
// SIMD; each byte copied into LDS feeds twice the products of a 128-token
// tile.
constexpr int kDOut = 256;
constexpr int kDWBytes = kDOut * 128;
constexpr int kDStage = kDWBytes + kDTok * 128;      // 64 KB
constexpr int kDOutStride = 144;                     // bytes per token row of the store staging
constexpr int kDLds = 8 * 128 * kDOutStride > 2 * kDStage ? 8 * 128 * kDOutStride : 2 * kDStage;

__global__ __launch_bounds__(512, 1) void prefill_decompress_kernel(
    const unsigned short* __restrict__ x, const float* __restrict__ ts,
    const unsigned short* __restrict__ w_uk, const unsigned short* __restrict__ w_uv,
    const int* __restrict__ seq_lens, int n_seq, int Tmax, int Tpad,
    unsigned short* __restrict__ kc, unsigned short* __restrict__ vv) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kDLds];
    MLA_LDS unsigned char* lds = (MLA_LDS unsigned char*)smem;
    // XCD = id % 8.  Each XCD's 32 concurrent workgroups cover 8 of its 16
    // heads x 4 consecutive token tiles (2 MB of weights + 1 MB of latents in
    // its L2): id / 8 = 32 g + 8 tl + hl, head = xcd + 8 hl + 64 (g % 2),
    // tile = 4 (g / 2) + tl.  The grid rounds the tiles up to a multiple of 4.
    const int xcd = blockIdx.x & 7, jj = blockIdx.x >> 3;
    const int g = jj >> 5, tl = (jj >> 3) & 3, hl = jj & 7;
    const int h = xcd + 8 * hl + 64 * (g & 1);
    const int tile = 4 * (g >> 1) + tl;
    const int ntt = Tpad / kDTok;
    const int b = tile / ntt, t0 = (tile - b * ntt) * kDTok;
    if (b >= n_seq) return;                          // rounding of the grid
    const int len = seq_len_of(seq_lens, b, Tmax);
    if (t0 >= len) return;                           // uniform
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hf = lane >> 5;
    const int r8 = lane >> 3, s8 = lane & 7;
    const int wo = w & 3, wt = w >> 2;               // output quarter, token half

    const __amdgpu_buffer_rsrc_t wk_r = p_rsrc(w_uk + (size_t)h * PN * PDC, PN * PDC * 2);
    const __amdgpu_buffer_rsrc_t wv_r = p_rsrc(w_uv + (size_t)h * PV * PDC, PV * PDC * 2);
    const __amdgpu_buffer_rsrc_t x_r = p_rsrc(x + ((size_t)b * Tpad + t0) * PDC, kDTok * PDC * 2);
    // instruction i = w + 8 j: j < 2 W_UK rows, j < 4 W_UV rows, else token rows
    unsigned voff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int i = w + 8 * j;
        const int row = 8 * (j < 2 ? i : (j < 4 ? i - 16 : i - 32)) + r8;
        voff[j] = (unsigned)row * (PDC * 2) + (unsigned)((s8 ^ pswz(row)) << 4);
    }
    auto issue = [&](int c) {
        MLA_LDS unsigned char* st = lds + (c & 1) * kDStage;
        const unsigned col = c < PDC / 64 ? (unsigned)c * 128u : 0x80000000u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const __amdgpu_buffer_rsrc_t r = j < 2 ? wk_r : (j < 4 ? wv_r : x_r);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (MLA_LDS void*)(st + (w + 8 * j) * 1024), 16,
                                                     voff[j] + col, 0, 0, 0);
        }
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[ob][tb] = f32x16{};
    // The K loop, compiled once per wave role: key waves put outputs on the
    // MFMA rows (K^C^T, stored per token), value waves put tokens on them
    // (V^T, stored per channel).  Both copies pass the same barriers.
    auto kloop = [&](auto value_waves) __attribute__((always_inline)) {
        constexpr bool VT = decltype(value_waves)::value;
        issue(0);
        for (int c = 0; c < PDC / 64; ++c) {
            p_stage_barrier();                       // everyone is done with chunk c - 1's stage
            issue(c + 1);
            p_wait_vmem<8>();                        // this wave's copies of chunk c landed
            p_stage_barrier();                       // ... and everyone's
            const MLA_LDS unsigned char* st = lds + (c & 1) * kDStage;
#pragma unroll
            for (int sx = 0; sx < 4; ++sx) {
                const int cx = 2 * sx + hf;          // 16-byte slot of K-step sx
                bf16x8 wf[2], xf[4];
#pragma unroll
                for (int ob = 0; ob < 2; ++ob) {
                    const int row = 64 * wo + 32 * ob + l32;
                    wf[ob] = *reinterpret_cast<const MLA_LDS bf16x8*>(st + (8 * row + (cx ^ pswz(row))) * 16);
                }
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const int row = 128 * wt + 32 * tb + l32;
                    xf[tb] = *reinterpret_cast<const MLA_LDS bf16x8*>(st + kDWBytes + (8 * row + (cx ^ pswz(row))) * 16);
                }
#pragma unroll
                for (int ob = 0; ob < 2; ++ob)
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb)
                        acc[ob][tb] = VT ? pf_mfma(xf[tb], wf[ob], acc[ob][tb]) : pf_mfma(wf[ob], xf[tb], acc[ob][tb]);
            }
        }
    };
    if (wo < 2)
        kloop(std::integral_constant<bool, false>{});
    else
        kloop(std::integral_constant<bool, true>{});
    p_wait_vmem<0>();                                // the record-less copies of chunk 8 too
    __syncthreads();                                 // stages free for the store staging

    MLA_LDS unsigned char* ost = lds + w * (128 * kDOutStride);
    if (wo >= 2) {
        // acc[ob][tb][i]: channel 64 (wo - 2) + 32 ob + l32 of token 128 wt +
        // 32 tb + 8 (i/4) + 4 hf + i%4.  V^T rows: keys of each 16-key group
        // in the order 0-3, 8-11, 4-7, 12-15 (position = key with bits 2 and 3
        // swapped), the order in which a lane half holds the softmax weights
        // of one MFMA K-step; the lane's 4 consecutive tokens stay 4
        // consecutive positions.  Staged as [64 channels][128 tokens] bf16
        // (rows of 272 bytes), stored as 256-byte row pieces.
        constexpr int VST = 272;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int tok = 32 * tb + 8 * g + 4 * hf;                    // first of 4
                const int pos = (tok & ~12) | ((tok & 4) << 1) | ((tok & 8) >> 1);
                float sc[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sc[e] = ts != nullptr ? ts[(size_t)b * Tpad + t0 + 128 * wt + tok + e] : 1.0f;
#pragma unroll
                for (int ob = 0; ob < 2; ++ob) {
                    u16x4 hv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) hv[e] = f32_to_bf16_bits(acc[ob][tb][4 * g + e] * sc[e]);
                    *reinterpret_cast<MLA_LDS u16x4*>(ost + (32 * ob + l32) * VST + pos * 2) = hv;
                }
            }
        }
        unsigned short* dst = vv + (((size_t)b * PH + h) * 128 + 64 * (wo - 2)) * Tpad + t0 + 128 * wt;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int ch = 4 * k + (lane >> 4), seg = lane & 15;
            const u32x4 v = *reinterpret_cast<const MLA_LDS u32x4*>(ost + ch * VST + seg * 16);
            *reinterpret_cast<u32x4*>(dst + (size_t)ch * Tpad + seg * 8) = v;
        }
        return;
    }
    // key waves.  acc[ob][tb][i]: output 64 wo + 32 ob + 8 (i/4) + 4 hf + i%4
    // of token 128 wt + 32 tb + l32.  Staged per wave as [token][64 outputs]
    // bf16 (rows of 144 bytes), then stored as 128-byte row pieces.
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int tok = 32 * tb + l32;
        const float sc = ts != nullptr ? ts[(size_t)b * Tpad + t0 + 128 * wt + tok] : 1.0f;
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u16x4 hv;
#pragma unroll
                for (int e = 0; e < 4; ++e) hv[e] = f32_to_bf16_bits(acc[ob][tb][4 * g + e] * sc);
                *reinterpret_cast<MLA_LDS u16x4*>(ost + tok * kDOutStride + (32 * ob + 8 * g + 4 * hf) * 2) = hv;
            }
    }
    // LDS operations of one wave complete in order: the reads see the writes
    unsigned short* dst = kc + (((size_t)b * PH + h) * Tpad + t0 + 128 * wt) * 128 + wo * 64;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int tok = 8 * k + r8;
        const u32x4 v = *reinterpret_cast<const MLA_LDS u32x4*>(ost + tok * kDOutStride + s8 * 16);
        *reinterpret_cast<u32x4*>(dst + (size_t)tok * 128 + s8 * 8) = v;
    }
}

// ---------------------------------------------------------------------------
// 3. causal attention
// ---------------------------------------------------------------------------

// grid: batch * H * nqb workgroups of 256 (nqb = ceil(q_len / 256)).  The 8
// XCDs take workgroups in turn (XCD = id % 8), so the ids are laid out to
// give all query blocks of one (sequence, head) to one XCD, longest first:
// they stream the same key and value tiles at about the same time, and the
// XCD's L2 serves all but the first read.
//
// Workgroup (b, h, qblk): queries s = 256 qblk .. +256 of sequence b, head h,
// on 8 waves of 32 queries (two waves per SIMD): wave w owns queries 256 qblk
// + 32 w + l32.  Key tiles of 64 tokens are copied HBM -> LDS three stages
// deep (two in flight while one is used): the 24 KB key tile [K^C | KR] (24
// chunks per token row: 16 of K^C, 8 of KR), chunk c of row t at 16-byte
// position (c / 8) * 512 + 8 t + (c % 8 ^ g(t)), and the 16 KB value tile,
// 128 channel rows of V^T (the tile's 64 keys, 8 chunks), chunk c of row r
// at 8 r + (c ^ g(r)); 40 copy instructions per tile (5 per wave),
// instruction i writing LDS bytes 1024 i .. +1024 of the stage.
//
// Per tile (64 keys), per wave:
//   S^T (64 keys x 32 queries) = K . Q^T      24 MFMA, K from LDS, Q in VGPRs
//   O^T (128 x 32)            += V^T . P^T    16 MFMA, V^T from LDS
// so a lane holds 32 scores of one query and the query's softmax statistics
// need one cross-lane exchange (lanes l and l + 32).
//
// Softmax: weights exp2(s * log2(e) * scale - m) with a per-query reference
// m that is raised only when a score exceeds it by more than kLazy (weights
// stay below 2^kLazy); raising it rescales the query's accumulators and sum
// (a wave-uniform branch, taken a few times per query).
constexpr int kPQ = 256;                 // queries per workgroup
constexpr int kPStages = 3;
constexpr int kPKBytes = PBS * (PN + PDR) * 2;      // 24 KB
constexpr int kPStage = kPKBytes + PBS * PV * 2;    // 40 KB
constexpr float kLazy = 8.0f;
constexpr int kPWaves = 8;               // waves per workgroup (4: 64 queries each, 8: 32)

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void prefill_attn_kernel(
    const unsigned short* __restrict__ q_nope,   // [batch * q_len][H][128]
    const unsigned short* __restrict__ q_pe,     // [batch * q_len][H][64]
    const unsigned short* __restrict__ kc,       // [batch][H][Tpad][128]
    const unsigned short* __restrict__ vv,       // [batch][H][128][Tpad]: V^T, keys permuted
    const unsigned short* __restrict__ kr,       // [batch * Tpad][64]
    const int* __restrict__ seq_lens, int Tmax, int Tpad, int q_len, int nqb, float scale_log2,
    unsigned short* __restrict__ out,            // [batch * q_len][H][128]
    float* __restrict__ lse) {                   // [batch * q_len][H]
    constexpr int QB = kPQ / (32 * NW);          // query blocks of 32 per wave
    constexpr int NCP = 40 / NW;                 // copy instructions per wave and tile
    static_assert(QB * 32 * NW == kPQ && NCP * NW == 40 && 16 % NW == 0 && 24 % NW == 0, "wave split");
    __shared__ __attribute__((aligned(16))) unsigned char smem[kPStages * kPStage];
    MLA_LDS unsigned char* lds = (MLA_LDS unsigned char*)smem;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hf = lane >> 5;
    const int r8 = lane >> 3, s8 = lane & 7;

    const int xcd = blockIdx.x & 7, jj = blockIdx.x >> 3;
    const int pair = (jj / nqb) * 8 + xcd;
    const int qblk = nqb - 1 - (jj - (jj / nqb) * nqb);
    const int b = pair / PH, h = pair - b * PH;
    const int len = seq_len_of(seq_lens, b, Tmax);
    const int base_vis = len - q_len;            // query s sees tokens < base_vis + s + 1
    const int q0 = qblk * kPQ;
    const int qa = q0 + 32 * QB * w;             // this wave's first query
    const int vis_blk = min(len, base_vis + min(q0 + kPQ, q_len));
    const int n_tiles = vis_blk > 0 ? (vis_blk + PBS - 1) / PBS : 0;
    const int vis_w = qa < q_len ? min(len, base_vis + min(qa + 32 * QB, q_len)) : 0;

    // ---- copies ----------------------------------------------------------------
    const size_t kv_base = ((size_t)b * PH + h) * Tpad * 128;
    const __amdgpu_buffer_rsrc_t kc_r = p_rsrc(kc + kv_base, (unsigned)Tpad * 256u);
    const __amdgpu_buffer_rsrc_t vv_r = p_rsrc(vv + kv_base, (unsigned)Tpad * 256u);
    const __amdgpu_buffer_rsrc_t kr_r = p_rsrc(kr + (size_t)b * Tpad * PDR, (unsigned)Tpad * 128u);
    // instruction i = w + NW j: i < 16 K^C (groups 0-1; token row 8 (i % 8)
    // + r8), i < 24 KR (group 2), else V^T (channel row 8 (i - 24) + r8, the
    // tile's 64 keys = 128 bytes of it).  Which tensor is fixed per j.
    constexpr int JKC = 16 / NW, JKR = 24 / NW;
    unsigned voff[NCP];
#pragma unroll
    for (int j = 0; j < NCP; ++j) {
        const int i = w + NW * j;
        if (j < JKR) {
            const int ii = j < JKC ? i : i - 16;
            const int row = 8 * (ii & 7) + r8;
            const int chunk = (j < JKC ? 8 * (ii >> 3) : 0) + (s8 ^ pswz(row));
            voff[j] = (unsigned)row * (j < JKC ? 256u : 128u) + (unsigned)chunk * 16u;
        } else {
            const int row = 8 * (i - 24) + r8;
            voff[j] = (unsigned)row * (unsigned)Tpad * 2u + (unsigned)((s8 ^ pswz(row)) << 4);
        }
    }
    auto issue = [&](int t) {
        MLA_LDS unsigned char* st = lds + (t % kPStages) * kPStage;
        const bool live = t < n_tiles;
#pragma unroll
        for (int j = 0; j < NCP; ++j) {
            const bool is_kr = j >= JKC && j < JKR;
            const __amdgpu_buffer_rsrc_t r = j < JKC ? kc_r : (is_kr ? kr_r : vv_r);
            const unsigned step = j < JKC ? 16384u : (is_kr ? 8192u : 128u);   // bytes per tile
            const unsigned off = live ? voff[j] + (unsigned)t * step : 0x80000000u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (MLA_LDS void*)(st + (w + NW * j) * 1024), 16, off,
                                                     0, 0, 0);
        }
    };
    // the first two tiles go out before the query loads
    issue(0);
    issue(1);

    // ---- this wave's queries as MFMA B fragments: lane (hf, l32) holds
    // channels 16 ks + 8 hf .. +8 of query qa + 32 qb + l32 (ks < 8: q^C, else q^R)
    bf16x8 qf[QB][12];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int s = qa + 32 * qb + l32;
        const size_t row = ((size_t)b * q_len + min(s, q_len - 1)) * PH + h;
        const bool ok = s < q_len;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(q_nope + row * PN + 16 * ks + 8 * hf);
            qf[qb][ks] = ok ? v : bf16x8{};
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(q_pe + row * PDR + 16 * ks + 8 * hf);
            qf[qb][8 + ks] = ok ? v : bf16x8{};
        }
    }

    // per-lane LDS offsets of the 16-byte operand reads: chunk 2 j + hf of
    // row l32 (plus a multiple of 32 rows), for the keys (j = K-step % 4) and
    // the value rows (j = the value K-step 2 hb + k2)
    int qk_off[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) qk_off[j] = (l32 * 8 + ((2 * j + hf) ^ pswz(l32 & 15))) * 16;

    f32x16 o[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int cm = 0; cm < 4; ++cm) o[qb][cm] = f32x16{};
    float m_ref[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_ref[qb] = kNegInf;
        l_run[qb] = 0.f;
    }

    // One tile: the scores of both halves (32 keys each) as two interleaved
    // MFMA chains, one maximum and reference check per query over the tile's
    // 64 keys, the weights, then the value product over four accumulators.
    // (A wave's dependent MFMAs would otherwise wait on each other; the
    // second wave of the SIMD fills the remaining gaps.)
    // LDS addresses: a per-lane base per tile (stage + lane offset), plus
    // constants that fit the instructions' offset field
    auto scores = [&](const MLA_LDS unsigned char* st, f32x16 (&sacc)[2][QB]) __attribute__((always_inline)) {
        const MLA_LDS unsigned char* kb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) kb[j] = st + qk_off[j];
        auto ka = [&](int hb, int ks) {
            return *reinterpret_cast<const MLA_LDS bf16x8*>(kb[ks & 3] + (hb * 32 * 128 + (ks >> 2) * 8192));
        };
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[hb][qb] = f32x16{};
        bf16x8 a0[2] = {ka(0, 0), ka(1, 0)}, a1[2] = {ka(0, 1), ka(1, 1)}, a2[2];
#pragma unroll
        for (int ks = 0; ks < 12; ++ks) {
            if (ks + 2 < 12) {
                a2[0] = ka(0, ks + 2);
                a2[1] = ka(1, ks + 2);
            }
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[hb][qb] = pf_mfma(a0[hb], qf[qb][ks], sacc[hb][qb]);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                a0[hb] = a1[hb];
                a1[hb] = a2[hb];
            }
        }
    };
    // lane: query qa + 32 qb + l32, keys t*64 + 32 hb + 8 (i/4) + 4 hf + i%4
    auto mask_tile = [&](int t, f32x16 (&sacc)[2][QB]) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int lim = base_vis + qa + 32 * qb + l32 - t * PBS - 4 * hf;   // last visible key, relative
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * hb + 8 * (i >> 2) + (i & 3) > lim) sacc[hb][qb][i] = kNegInf;
        }
    };
    // per-query maxima over the tile (log2 domain, both lanes of a query) and
    // the raise of the reference when they exceed it by more than kLazy
    auto raise_tile = [&](const f32x16 (&sacc)[2][QB]) __attribute__((always_inline)) {
        float mx[QB];
        bool raise[QB];
        bool any = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float hmax = max3f(sacc[0][qb][0], sacc[1][qb][0], sacc[0][qb][1]);
            hmax = max3f(hmax, sacc[1][qb][1], sacc[0][qb][2]);
#pragma unroll
            for (int i = 2; i < 15; ++i) hmax = max3f(hmax, sacc[1][qb][i], sacc[0][qb][i + 1]);
            hmax = fmaxf(hmax, sacc[1][qb][15]);
            hmax *= scale_log2;
            mx[qb] = fmaxf(hmax, __shfl_xor(hmax, 32, 64));
            raise[qb] = mx[qb] > m_ref[qb] + kLazy;
            any = any || raise[qb];
        }
        if (__builtin_amdgcn_ballot_w64(any) == 0) return;   // uniform
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float alpha = raise[qb] ? __builtin_amdgcn_exp2f(m_ref[qb] - mx[qb]) : 1.0f;
            m_ref[qb] = raise[qb] ? mx[qb] : m_ref[qb];
            l_run[qb] *= alpha;
#pragma unroll
            for (int cm = 0; cm < 4; ++cm)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[qb][cm][i] *= alpha;
        }
    };
    // weights exp2(s log2(e) scale - m) as bf16 B fragments of the value
    // product (pf[hb][qb][k2]), summed into l.  A query with nothing visible
    // yet has m_ref = -inf and only -inf scores: its weights are exp2(-inf) = 0.
    auto weights = [&](const f32x16 (&sacc)[2][QB], bf16x8 (&pf)[2][QB][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float m_use = m_ref[qb] == kNegInf ? 0.f : m_ref[qb];
            float ps = 0.f;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    u16x8 pu;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float pv = __builtin_amdgcn_exp2f(
                            __builtin_fmaf(sacc[hb][qb][8 * k2 + e], scale_log2, -m_use));
                        ps += pv;
                        pu[e] = f32_to_bf16_bits(pv);
                    }
                    pf[hb][qb][k2] = __builtin_bit_cast(bf16x8, pu);
                }
            l_run[qb] += ps;
        }
    };
    // O^T += V^T . P^T over the tile's 64 keys.  K-step kk = 2 hb + k2 covers
    // keys 32 hb + 16 k2 + {0..3, 8..11} (lanes 0-31) and {4..7, 12..15}
    // (lanes 32-63), matching P's layout; the V^T tile stores each 16-key
    // group in that order, so a lane's 8 keys are one 16-byte chunk (2 kk +
    // hf) of its channel row.  Consecutive MFMAs update different accumulators.
    auto values = [&](const MLA_LDS unsigned char* vt, const bf16x8 (&pf)[2][QB][2]) __attribute__((always_inline)) {
        auto va = [&](int kk, int cm) {
            return *reinterpret_cast<const MLA_LDS bf16x8*>(vt + qk_off[kk] + cm * 32 * 128);
        };
        bf16x8 v0 = va(0, 0), v1;
#pragma unroll
        for (int st16 = 0; st16 < 16; ++st16) {
            const int kk = st16 >> 2, cm = st16 & 3;      // kk = 2 hb + k2
            if (st16 + 1 < 16) v1 = va((st16 + 1) >> 2, (st16 + 1) & 3);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[qb][cm] = pf_mfma(v0, pf[kk >> 1][qb][kk & 1], o[qb][cm]);
            v0 = v1;
        }
    };

    for (int t = 0; t < n_tiles; ++t) {
        p_stage_barrier();                       // everyone is done with tile t - 1's stage
        issue(t + 2);
        p_wait_vmem<NCP * (kPStages - 1)>();     // this wave's copies of tile t landed
        p_stage_barrier();                       // ... and everyone's
        if (t * PBS >= vis_w) continue;          // nothing of this tile is visible to the wave
        const MLA_LDS unsigned char* st = lds + (t % kPStages) * kPStage;
        // does the tile reach past the first query's visible range?  (A half
        // past the wave's last query is then masked whole: its weights are 0.)
        const bool need_mask = t * PBS + PBS - 1 >= base_vis + qa + 1;
        f32x16 sacc[2][QB];
        bf16x8 pf[2][QB][2];
        scores(st, sacc);
        if (need_mask) mask_tile(t, sacc);
        raise_tile(sacc);
        weights(sacc, pf);
        values(st + kPKBytes, pf);
    }
    p_wait_vmem<0>();                            // the record-less copies too

    // ---- epilogue: out = O / l, lse = (m + log2 l) ln 2 ------------------------------
    // o[qb][cm][i]: channel 32 cm + 8 (i/4) + 4 hf + i%4 of query qa + 32 qb + l32
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int s = qa + 32 * qb + l32;
        const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);   // disjoint keys
        if (s >= q_len) continue;
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        const size_t row = ((size_t)b * q_len + s) * PH + h;
        unsigned short* dst = out + row * PV + 4 * hf;
#pragma unroll
        for (int cm = 0; cm < 4; ++cm)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u16x4 hv;
#pragma unroll
                for (int e = 0; e < 4; ++e) hv[e] = f32_to_bf16_bits(o[qb][cm][4 * g + e] * inv);
                *reinterpret_cast<u16x4*>(dst + 32 * cm + 8 * g) = hv;
            }
        if (hf == 0 && lse != nullptr) lse[row] = l_tot > 0.f ? (m_ref[qb] + __builtin_log2f(l_tot)) * kLn2 : kNegInf;
    }
}

}  // namespace

int prefill_tpad(int max_blocks) { return (max_blocks * PBS + kDTok - 1) / kDTok * kDTok; }

hipError_t launch_prefill(const PrefillLaunch& a) {
    if (a.batch == 0) return hipSuccess;
    const int Tmax = a.max_blocks * PBS, Tpad = prefill_tpad(a.max_blocks);
    if (a.stages & 1u) {
        prefill_gather_kernel<<<a.batch * (Tpad / PBS), 256, 0, a.stream>>>(
            static_cast<const unsigned char*>(a.pool), a.pool_scale, a.cache_dtype == MLA_FP8_E4M3 ? 1 : 0,
            a.block_table, a.max_blocks, a.seq_lens, Tmax, Tpad, a.x, a.kr, a.ts);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    if (a.stages & 2u) {
        const int n_tiles = a.batch * (Tpad / kDTok);
        prefill_decompress_kernel<<<PH * ((n_tiles + 3) / 4 * 4), 512, 0, a.stream>>>(
            a.x, a.cache_dtype == MLA_FP8_E4M3 ? a.ts : nullptr, static_cast<const unsigned short*>(a.w_uk),
            static_cast<const unsigned short*>(a.w_uv), a.seq_lens, a.batch, Tmax, Tpad, a.kc, a.vv);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    if (a.stages & 4u) {
        const int nqb = (a.q_len + kPQ - 1) / kPQ;
        prefill_attn_kernel<kPWaves><<<a.batch * PH * nqb, kPWaves * 64, 0, a.stream>>>(
            static_cast<const unsigned short*>(a.q_nope), static_cast<const unsigned short*>(a.q_pe), a.kc,
            a.vv, a.kr, a.seq_lens, Tmax, Tpad, a.q_len, nqb, a.scale * kLog2e,
            static_cast<unsigned short*>(a.out), a.lse);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mla

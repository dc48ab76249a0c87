// Absorbed-MLA decode for the DeepSeek-V3 head shape on gfx950 MFMA.
//
// Shape: 128 heads, latent d_c = 512, rotary R = 64, q_nope N = 128,
// v_head V = 128, cache blocks of 64 tokens, bf16 activations and weights,
// bf16 or fp8-e4m3 cache.  Three kernels, run in order on one stream:
//
//  1. absorb_q:  q_lat[r,h,:] = W_UK[h]^T q_nope[r,h,:]  (the query-side weight
//     absorption of "DeepSeek-V2: MLA Explained", "Optimization Note"), packed
//     with q_pe into one 576-wide bf16 query row per (row, head).
//  2. split_kv:  one workgroup per (sequence, query row, partition).  All 128
//     heads share every 64-token cache tile ("Latent Attention.", "Compress,
//     then rebuild": one latent serves every head), so heads form the dense
//     MFMA dimension: S^T = K_tile . Q^T, online softmax, O^T += V^T . P^T
//     with the latent columns of the same tile as values.  Writes the
//     partition's normalised o_lat and log-sum-exp.
//  3. combine:   merges partitions by log-sum-exp weights into o_lat, then
//     out[r,h,:] = W_UV[h] o_lat (the value-side absorption).
//
// All contractions accumulate in fp32; q_lat and the softmax weights P enter
// the MFMA as bf16, o_lat enters the W_UV product as a bf16 hi + lo pair.

#include "common.hpp"
#include "internal.hpp"

namespace mla {
namespace {

constexpr int H = 128;
constexpr int DC = 512;
constexpr int DR = 64;
constexpr int D = DC + DR;            // 576
constexpr int BS = 64;                // tokens per cache block = per tile
constexpr int ROWB = D * 2;           // 1152 bytes per bf16 row in memory
constexpr int GTILE = BS * ROWB;      // 73728 bytes per bf16 block in memory
constexpr int NCH = ROWB / 16;        // 72 16-byte chunks per bf16 row
constexpr int TILE = GTILE;           // LDS tile: same bytes, swizzled
constexpr int F8TILE = BS * D;        // 36864 bytes per fp8 tile
constexpr int F8CHUNKS = D / 16;      // 36 chunks per fp8 row

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS tile layout.  Chunk c (8 bf16 channels) of token row t lives at chunk
// position  P(t, c) = (c >> 3) * 512 + t * 8 + ((c & 7) ^ f(t)),
// f(t) = ((t & 3) << 1) | ((t >> 2) & 1): groups of 8 chunks are stored row
// by row, the chunk slot XOR-permuted per row.  Then
//  - 8 consecutive rows reading one chunk (the 16-byte score-operand reads)
//    hit 8 different slots, i.e. disjoint banks;
//  - 4 consecutive rows x 2 adjacent chunks (the transposed 8-byte value
//    reads of one 16-lane group) hit 8 different slots;
//  - every global->LDS instruction copies 8 rows x 128 contiguous bytes.
__device__ __forceinline__ int fswz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }
__device__ __forceinline__ int tpos(int t, int c) {
    return ((c >> 3) << 9) + (t << 3) + ((c & 7) ^ fswz(t));
}

// Buffer resource over [base, base + bytes): raw (untyped) access, gfx9 word 3.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ void wait_vmem_all() {
    // s_waitcnt vmcnt(0), leaving expcnt / lgkmcnt unconstrained
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// ---------------------------------------------------------------------------
// 1. q absorption
// ---------------------------------------------------------------------------

// grid: H * 4 * ceil(R / 64) workgroups of 256 threads.  Workgroup (h, cb, rb)
// produces q_lat[rb*64 .. +64][h][cb*128 .. +128]: q_lat^T = W_UK[h]^T q_nope^T
// with W_UK[h][:, cb*128 .. +128] staged in LDS (row stride padded to 264 B so
// the transposed reads of two half-waves fall in different banks).
constexpr int WT_STRIDE = 132;  // ushorts per staged W_UK row

__global__ __launch_bounds__(256) void absorb_q_kernel(
    const unsigned short* __restrict__ q_nope,  // [R][H][128]
    const unsigned short* __restrict__ q_pe,    // [R][H][64]
    const unsigned short* __restrict__ w_uk,    // [H][128][512]
    unsigned short* __restrict__ qbuf,          // [R][H][576]
    int R) {
    __shared__ __attribute__((aligned(16))) unsigned short wt[128 * WT_STRIDE];
    const int bid = blockIdx.x;
    const int h = bid % H;
    const int cb = (bid / H) & 3;
    const int rb = bid / (H * 4);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, in an SGPR
    const int l32 = lane & 31, hf = lane >> 5;

    {   // stage W_UK[h][n][cb*128 .. +128]: thread -> (n = tid/2, 64 columns)
        const int n = tid >> 1, half = tid & 1;
        const unsigned short* src = w_uk + ((size_t)h * 128 + n) * DC + cb * 128 + half * 64;
        unsigned short* dst = wt + n * WT_STRIDE + half * 64;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            u32x4 v = *reinterpret_cast<const u32x4*>(src + k * 8);
            *reinterpret_cast<unsigned long long*>(dst + k * 8) =
                (unsigned long long)v[0] | ((unsigned long long)v[1] << 32);
            *reinterpret_cast<unsigned long long*>(dst + k * 8 + 4) =
                (unsigned long long)v[2] | ((unsigned long long)v[3] << 32);
        }
    }
    // q_pe rides along in the workgroups of column block 0
    if (cb == 0) {
        for (int i = tid; i < 64 * 8; i += 256) {       // 64 rows x 8 chunks of 8
            const int r = rb * 64 + (i >> 3), c8 = i & 7;
            if (r < R) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(q_pe + ((size_t)r * H + h) * DR + c8 * 8);
                *reinterpret_cast<u32x4*>(qbuf + ((size_t)r * H + h) * D + DC + c8 * 8) = v;
            }
        }
    }
    __syncthreads();

    f32x16 acc[2] = {};
    const int cl = w * 32 + l32;                       // local latent column (M)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {                   // K = n, 16 per step
        bf16x8 a;
        u16x8 au;
#pragma unroll
        for (int j = 0; j < 8; ++j) au[j] = wt[(ks * 16 + hf * 8 + j) * WT_STRIDE + cl];
        a = __builtin_bit_cast(bf16x8, au);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int r = rb * 64 + nb * 32 + l32;
            bf16x8 bv = {};
            if (r < R)
                bv = *reinterpret_cast<const bf16x8*>(q_nope + ((size_t)r * H + h) * 128 + ks * 16 + hf * 8);
            acc[nb] = mfma32(a, bv, acc[nb]);
        }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int r = rb * 64 + nb * 32 + l32;
        if (r >= R) continue;
        unsigned short* dst = qbuf + ((size_t)r * H + h) * D + cb * 128 + w * 32 + 4 * hf;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const unsigned long long pk =
                (unsigned long long)f32_to_bf16_bits(acc[nb][4 * g + 0]) |
                ((unsigned long long)f32_to_bf16_bits(acc[nb][4 * g + 1]) << 16) |
                ((unsigned long long)f32_to_bf16_bits(acc[nb][4 * g + 2]) << 32) |
                ((unsigned long long)f32_to_bf16_bits(acc[nb][4 * g + 3]) << 48);
            *reinterpret_cast<unsigned long long*>(dst + 8 * g) = pk;
        }
    }
}

// ---------------------------------------------------------------------------
// 2. split-KV attention over the latent cache
// ---------------------------------------------------------------------------

// Issue the asynchronous copy of one bf16 cache block (64 rows x 1152 B,
// contiguous in memory) into an LDS tile.  Instruction i = 8 cg + q fills
// positions 64 i .. 64 i + 63: rows 8q .. 8q+7, chunk group cg.  Lane l takes
// row 8q + l/8 and slot l%8, i.e. chunk 8 cg + ((l%8) ^ f(l/8)).
__device__ __forceinline__ void issue_tile_bf16(const unsigned char* __restrict__ gtile,
                                                unsigned char* ltile, int w, int lane) {
    const unsigned lane_off = (lane >> 3) * ROWB + (((lane & 7) ^ fswz(lane >> 3)) << 4);
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(gtile, GTILE);
#pragma unroll
    for (int k = 0; k < 18; ++k) {
        const int i = w * 18 + k;                      // wave-uniform
        const int cg = i >> 3, q = i & 7;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (MLA_LDS void*)(ltile + i * 1024), 16,
                                                 lane_off, q * 8 * ROWB + cg * 128, 0, 0);
    }
}

// Zero rows valid .. 63 of an LDS tile (their cache slots hold no token).
__device__ __forceinline__ void zero_rows(unsigned char* ltile, int valid, int tid) {
    for (int p = valid * NCH + tid; p < BS * NCH; p += 256) {
        const int t = p / NCH, c = p - t * NCH;
        *reinterpret_cast<u32x4*>(ltile + tpos(t, c) * 16) = u32x4{0, 0, 0, 0};
    }
}

// Asynchronous copy of one fp8 cache block (64 rows x 576 B, contiguous) into
// row-major LDS staging, plus its 64 per-token scales.
__device__ __forceinline__ void issue_tile_fp8(const unsigned char* __restrict__ gtile,
                                               const float* __restrict__ gscale,
                                               unsigned char* lstage, float* lscale,
                                               int w, int lane) {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(gtile, F8TILE);
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const int i = w * 9 + k;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (MLA_LDS void*)(lstage + i * 1024), 16,
                                                 lane * 16, i * 1024, 0, 0);
    }
    if (w == 0 && lane < 16)
        __builtin_amdgcn_global_load_lds((const void*)(gscale + lane * 4), (MLA_LDS void*)lscale,
                                         16, 0, 0);
}

// fp8 staging -> dequantised bf16 swizzled tile (value * token scale, RNE).
// Rows at or beyond `valid` become zeros.
__device__ __forceinline__ void convert_tile_fp8(const unsigned char* lstage, const float* lscale,
                                                 unsigned char* ltile, int tid, int valid) {
#pragma unroll 1
    for (int k = 0; k < 9; ++k) {
        const int p = k * 256 + tid;                   // 2304 fp8 chunks
        const int t = p / F8CHUNKS, c = p - t * F8CHUNKS;
        u32x4 outw[2];
        if (t < valid) {
            const u32x4 raw = *reinterpret_cast<const u32x4*>(lstage + p * 16);
            const float sc = lscale[t];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(raw[q], false);
                const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(raw[q], true);
                const unsigned int p0 = f32_to_bf16_bits(lo[0] * sc) | ((unsigned)f32_to_bf16_bits(lo[1] * sc) << 16);
                const unsigned int p1 = f32_to_bf16_bits(hi[0] * sc) | ((unsigned)f32_to_bf16_bits(hi[1] * sc) << 16);
                outw[q >> 1][(q & 1) * 2 + 0] = p0;
                outw[q >> 1][(q & 1) * 2 + 1] = p1;
            }
        } else {
            outw[0] = u32x4{0, 0, 0, 0};
            outw[1] = u32x4{0, 0, 0, 0};
        }
        *reinterpret_cast<u32x4*>(ltile + tpos(t, 2 * c) * 16) = outw[0];
        *reinterpret_cast<u32x4*>(ltile + tpos(t, 2 * c + 1) * 16) = outw[1];
    }
}

// Workgroup (row, split): row = b * q_len + s handles query token s of
// sequence b for all 128 heads over cache tiles [t0, t1) of its visible range.
// Wave w owns heads 32w .. 32w+31 for the whole tile loop:
//   S^T (64 tokens x 32 heads) = K_tile (64 x 576) . Q_w^T   [2 x 36 MFMA]
//   O^T (512 cols x 32 heads) += V^T (512 x 64) . P^T        [16 x 4 MFMA]
// so softmax statistics and rescaling stay inside the wave.
template <bool FP8>
__global__ __launch_bounds__(256, 1) void split_kv_kernel(
    const unsigned short* __restrict__ qbuf,      // [R][H][576] bf16
    const unsigned char* __restrict__ pool,       // [blocks][64][576] bf16 | fp8
    const float* __restrict__ pool_scale,         // [blocks][64] (fp8)
    const int* __restrict__ block_table, int max_blocks,
    const int* __restrict__ seq_lens, int q_len, int num_splits, float scale_log2,
    float* __restrict__ part_o,                   // [R][S][H][512]
    float* __restrict__ part_lse) {               // [R][S][H]
    constexpr int LDS_BYTES = (FP8 ? (TILE + 2 * F8TILE + 2 * 256) : (2 * TILE)) + 16;
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, in an SGPR
    const int l32 = lane & 31, hf = lane >> 5;
    const int row = blockIdx.x / num_splits;
    const int split = blockIdx.x - row * num_splits;
    const int b = row / q_len, s = row - b * q_len;
    const int n_vis = seq_lens[b] - q_len + s + 1;
    const int n_tiles = n_vis > 0 ? (n_vis + BS - 1) / BS : 0;
    const int tps = (n_tiles + num_splits - 1) / num_splits;
    const int t0 = split * tps;
    const int t1 = min(n_tiles, t0 + tps);
    float* lse_dst = part_lse + ((size_t)row * num_splits + split) * H;
    if (t0 >= t1) {
        if (tid < H) lse_dst[tid] = kNegInf;
        return;
    }
    const int* btab = block_table + (size_t)b * max_blocks;
    const int head = w * 32 + l32;

    // this wave's 32 query rows, as MFMA B fragments: lane (hf, l32) holds
    // channels 16 ks + 8 hf .. +8 of head 32 w + l32
    bf16x8 qf[36];
    {
        const unsigned short* qrow = qbuf + ((size_t)row * H + head) * D + hf * 8;
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
    }

    unsigned char* tiles = smem;                       // bf16 tile(s)
    unsigned char* stage = smem + TILE;                // fp8 staging (FP8 only)
    float* sscale = reinterpret_cast<float*>(smem + TILE + 2 * F8TILE);

    auto valid_of = [&](int t) { return min(BS, n_vis - t * BS); };
    auto issue = [&](int t, int buf) {
        const size_t blk = (size_t)btab[t];
        if constexpr (FP8) {
            issue_tile_fp8(pool + blk * F8TILE, pool_scale + blk * BS, stage + buf * F8TILE,
                           sscale + buf * 64, w, lane);
        } else {
            issue_tile_bf16(pool + blk * GTILE, tiles + buf * TILE, w, lane);
        }
    };

    // Softmax without rescaling the accumulators: every weight of a pass is
    // exp2(s - m_ref) for one reference m_ref per head.  The first pass takes
    // m_ref from the first tile; if a later tile's maximum exceeds it by more
    // than kMaxLead (weights up to 2^64 stay far from fp32 overflow), the pass
    // is abandoned, one scan computes the exact maximum and a last pass runs
    // with it.  (Scaling O inside the loop would force the 256 accumulators out
    // of AGPRs.)
    // per-lane LDS byte offsets of the score-operand reads (chunk 2 ks + hf of
    // row l32, by ks % 4) and of the transposed value reads (by cm % 2): in a
    // 16-lane group, lane 4r + b reads row 4 hf + r, channels 4b .. 4b+3 of a
    // 16-channel column block
    int qk_off[4], tr_off[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) qk_off[j] = (l32 * 8 + ((2 * j + hf) ^ fswz(l32))) * 16;
    {
        const int r = (lane & 15) >> 2, g1 = (lane >> 4) & 1, b1 = (lane >> 1) & 1;
        const int f = (r << 1) | hf;                   // fswz(4 hf + r)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            tr_off[j] = ((4 * hf + r) * 8 + ((4 * j + 2 * g1 + b1) ^ f)) * 16 + (lane & 1) * 8;
    }
    constexpr float kMaxLead = 64.0f;
    // Overflow flags, one per tile parity: iteration t sets flag[t & 1] and
    // the top of iteration t + 1 reads it after the barrier, so no wave can
    // see a flag another wave sets later in the same iteration.
    int* abort_flag = reinterpret_cast<int*>(smem + LDS_BYTES - 16);
    f32x16 o[16];
    float m_ref = kNegInf, l_run = 0.f;
    int mode = 0;                        // 0: first-tile reference, 1: max scan, 2: exact reference
    for (;;) {
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] = f32x16{};
        l_run = 0.f;
        if (tid == 0) abort_flag[0] = abort_flag[1] = 0;
        bool aborted = false;
        issue(t0, 0);
        for (int t = t0; t < t1; ++t) {
            const int cur = (t - t0) & 1;
            const int valid = valid_of(t);
            wait_vmem_all();
            __syncthreads();             // tile t landed; previous tile fully consumed
            if (t > t0 && abort_flag[(t - 1) & 1]) { aborted = true; break; }
            if (t + 1 < t1) issue(t + 1, cur ^ 1);
            const unsigned char* tile;
            if constexpr (FP8) {
                convert_tile_fp8(stage + cur * F8TILE, sscale + cur * 64, tiles, tid, valid);
                __syncthreads();
                tile = tiles;
            } else {
                tile = tiles + cur * TILE;
                if (valid < BS) {        // last, partial tile of the sequence
                    zero_rows(tiles + cur * TILE, valid, tid);
                    __syncthreads();
                }
            }

            // Two halves of 32 tokens; each: scores for 32 tokens x 32 heads,
            // weights, then their contribution to O.
#pragma unroll 1
            for (int hb = 0; hb < 2; ++hb) {
                if (hb * 32 >= valid) break;
                // ---- S^T = K . Q^T: rows 32 hb + l32 -------------------------------
                f32x16 sacc = {};
#pragma unroll
                for (int ks = 0; ks < 36; ++ks) {
                    const bf16x8 av = *reinterpret_cast<const bf16x8*>(
                        tile + qk_off[ks & 3] + (ks >> 2) * 8192 + hb * 32 * 128);
                    sacc = mfma32(av, qf[ks], sacc);
                }
                // lane holds head `head`, tokens 32 hb + 8 (i/4) + 4 hf + (i%4)
                float sv[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) sv[i] = sacc[i] * scale_log2;
                if (valid < BS) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int tok = hb * 32 + (i >> 2) * 8 + 4 * hf + (i & 3);
                        if (tok >= valid) sv[i] = kNegInf;
                    }
                }
                float hmax = sv[0];
#pragma unroll
                for (int i = 1; i < 16; ++i) hmax = fmaxf(hmax, sv[i]);
                hmax = fmaxf(hmax, __shfl_xor(hmax, 32, 64));
                if (mode == 1) {
                    m_ref = fmaxf(m_ref, hmax);
                    continue;
                }
                if (mode == 0 && t == t0 && hb == 0) m_ref = hmax;
                // (cannot fire in the exact-reference pass: the scan saw the
                // same maxima, so at most three passes run)
                if (hmax > m_ref + kMaxLead) abort_flag[t & 1] = 1;

                float psum = 0.f;
                bf16x8 pf[2];
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    u16x8 pu;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float pv = __builtin_amdgcn_exp2f(sv[k2 * 8 + j] - m_ref);
                        psum += pv;
                        pu[j] = f32_to_bf16_bits(pv);
                    }
                    pf[k2] = __builtin_bit_cast(bf16x8, pu);
                }
                psum += __shfl_xor(psum, 32, 64);
                l_run += psum;

                // ---- O^T += V^T . P^T (latent columns of the same rows) -------------
                // K-step k2 covers tokens 32 hb + 16 k2 + {0..3, 8..11} (lanes
                // 0-31) and {4..7, 12..15} (lanes 32-63), matching P's layout.
#pragma unroll
                for (int cm = 0; cm < 16; ++cm) {
                    const unsigned char* vb = tile + tr_off[cm & 1] + (cm >> 1) * 8192;
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2) {
                        const int tb = hb * 32 + k2 * 16;
                        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                            (MLA_LDS bf16x4*)(vb + tb * 128));
                        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                            (MLA_LDS bf16x4*)(vb + (tb + 8) * 128));
                        const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                        o[cm] = mfma32(va, pf[k2], o[cm]);
                    }
                }
            }
        }
        if (!aborted) {
            __syncthreads();             // the last tile's overflow check
            aborted = abort_flag[(t1 - 1) & 1] != 0;
        }
        if (aborted) {
            __syncthreads();             // everyone has read the flag before it is reset
            mode = 1;
            m_ref = kNegInf;
            continue;
        }
        if (mode == 1) {
            mode = 2;
            __syncthreads();
            continue;
        }
        break;
    }

    // ---- epilogue: normalised partial o_lat and log-sum-exp ------------------------
    const float inv_l = 1.0f / l_run;
    float* po = part_o + (((size_t)row * num_splits + split) * H + head) * DC + 4 * hf;
#pragma unroll
    for (int cm = 0; cm < 16; ++cm)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 v = {o[cm][4 * g] * inv_l, o[cm][4 * g + 1] * inv_l, o[cm][4 * g + 2] * inv_l,
                       o[cm][4 * g + 3] * inv_l};
            *reinterpret_cast<f32x4*>(po + cm * 32 + g * 8) = v;
        }
    if (hf == 0) lse_dst[head] = (m_ref + __builtin_log2f(l_run)) * kLn2;
}

// ---------------------------------------------------------------------------
// 3. log-sum-exp combine of partitions, then out = W_UV o_lat
// ---------------------------------------------------------------------------

// grid: H * ceil(R / 32) workgroups (h fastest, so one head's row blocks share
// an XCD and its W_UV slice in L2).  Wave w combines rows 8w .. 8w+7 of the
// block into LDS, then computes out^T[32w .. +32][rows] = W_UV[h] o_lat^T.
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int R, int num_splits,
    const unsigned short* __restrict__ w_uv,    // [H][128][512]
    unsigned short* __restrict__ out,           // [R][H][128] bf16
    float* __restrict__ lse_out) {              // [R][H] or null
    __shared__ __attribute__((aligned(16))) unsigned char ol[2][32 * 1024];   // hi, lo bf16
    const int h = blockIdx.x % H;
    const int rb = blockIdx.x / H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, in an SGPR
    const int l32 = lane & 31, hf = lane >> 5;

    for (int rr = 0; rr < 8; ++rr) {
        const int rl = w * 8 + rr;                     // local row
        const int r = rb * 32 + rl;
        float acc[8] = {};
        float tot = 0.f, mx = kNegInf;
        if (r < R) {
            const float* lrow = part_lse + (size_t)r * num_splits * H + h;
            for (int s = lane; s < num_splits; s += 64) mx = fmaxf(mx, lrow[(size_t)s * H]);
            mx = wave_max(mx);
            if (mx != kNegInf) {
                for (int s = 0; s < num_splits; ++s) {
                    const float ls = lrow[(size_t)s * H];
                    if (ls == kNegInf) continue;
                    const float wt = __expf(ls - mx);
                    tot += wt;
                    const float* src = part_o + (((size_t)r * num_splits + s) * H + h) * DC + lane * 8;
                    const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
                    const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[j] += wt * v0[j];
                        acc[4 + j] += wt * v1[j];
                    }
                }
            }
            if (lse_out != nullptr && lane == 0)
                lse_out[(size_t)r * H + h] = (mx == kNegInf) ? kNegInf : mx + __logf(tot);
        }
        const float inv = tot > 0.f ? 1.0f / tot : 0.f;
        u16x8 hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float v = acc[j] * inv;
            hi[j] = f32_to_bf16_bits(v);
            lo[j] = f32_to_bf16_bits(v - bf16_bits_to_f32(hi[j]));
        }
        const int off = rl * 1024 + ((lane ^ (rl & 7)) << 4);   // chunk = lane (8 cols)
        *reinterpret_cast<u16x8*>(&ol[0][off]) = hi;
        *reinterpret_cast<u16x8*>(&ol[1][off]) = lo;
    }
    __syncthreads();

    f32x16 acc = {};
    const unsigned short* wrow = w_uv + ((size_t)h * 128 + w * 32 + l32) * DC + hf * 8;
#pragma unroll 4
    for (int ks = 0; ks < 32; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(wrow + ks * 16);
        const int ch = 2 * ks + hf;
        const int off = l32 * 1024 + ((ch ^ (l32 & 7)) << 4);
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&ol[0][off]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&ol[1][off]);
        acc = mfma32(a, bh, acc);
        acc = mfma32(a, bl, acc);
    }
    const int r = rb * 32 + l32;
    if (r < R) {
        unsigned short* dst = out + ((size_t)r * H + h) * 128 + w * 32 + 4 * hf;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const unsigned long long pk =
                (unsigned long long)f32_to_bf16_bits(acc[4 * g + 0]) |
                ((unsigned long long)f32_to_bf16_bits(acc[4 * g + 1]) << 16) |
                ((unsigned long long)f32_to_bf16_bits(acc[4 * g + 2]) << 32) |
                ((unsigned long long)f32_to_bf16_bits(acc[4 * g + 3]) << 48);
            *reinterpret_cast<unsigned long long*>(dst + 8 * g) = pk;
        }
    }
}

}  // namespace

bool is_v3_shape(const mla_dims& d) {
    return d.n_heads == H && d.kv_lora_rank == DC && d.qk_rope_dim == DR && d.qk_nope_dim == 128 &&
           d.v_head_dim == 128 && d.block_size == BS && d.act_dtype == MLA_BF16 &&
           (d.cache_dtype == MLA_BF16 || d.cache_dtype == MLA_FP8_E4M3);
}

hipError_t launch_decode_mfma(const DecodeLaunch& a, unsigned stages) {
    const int R = a.batch * a.q_len;
    if (R == 0) return hipSuccess;
    auto* qbuf = static_cast<unsigned short*>(a.qbuf);
    if (stages & MLA_STAGE_ABSORB_Q) {
        const int grid = H * 4 * ((R + 63) / 64);
        absorb_q_kernel<<<grid, 256, 0, a.stream>>>(
            static_cast<const unsigned short*>(a.q_nope), static_cast<const unsigned short*>(a.q_pe),
            static_cast<const unsigned short*>(a.w_uk), qbuf, R);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (stages & MLA_STAGE_SPLIT_KV) {
        const int grid = R * a.num_splits;
        const float scale_log2 = a.scale * kLog2e;
        if (a.cache_dtype == MLA_FP8_E4M3) {
            split_kv_kernel<true><<<grid, 256, 0, a.stream>>>(
                qbuf, static_cast<const unsigned char*>(a.pool), a.pool_scale, a.block_table,
                a.max_blocks, a.seq_lens, a.q_len, a.num_splits, scale_log2, a.part_o, a.part_lse);
        } else {
            split_kv_kernel<false><<<grid, 256, 0, a.stream>>>(
                qbuf, static_cast<const unsigned char*>(a.pool), nullptr, a.block_table,
                a.max_blocks, a.seq_lens, a.q_len, a.num_splits, scale_log2, a.part_o, a.part_lse);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (stages & MLA_STAGE_COMBINE) {
        const int grid = H * ((R + 31) / 32);
        combine_kernel<<<grid, 256, 0, a.stream>>>(a.part_o, a.part_lse, R, a.num_splits,
                                                   static_cast<const unsigned short*>(a.w_uv),
                                                   static_cast<unsigned short*>(a.out), a.lse);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mla

// Absorbed-MLA decode for the DeepSeek-V3 head shape on gfx950 MFMA.
//
// Shape: 128 heads, latent d_c = 512, rotary R = 64, q_nope N = 128,
// v_head V = 128, cache blocks of 64 tokens, bf16 activations and weights,
// bf16 or fp8-e4m3 cache.  Three kernels, run in order on one stream:
//
//  1. absorb_q:  q_lat[r,h,:] = W_UK[h]^T q_nope[r,h,:]  (the query-side weight
//     absorption of "DeepSeek-V2: MLA Explained", "Optimization Note"), packed
//     with q_pe into one 576-wide bf16 query row per (row, head).
//  2. split_kv:  each workgroup walks a range of (query row, cache tile) work
//     -- a fixed partition of one row, or an equal share of all rows' tiles
//     on the balanced schedule -- writing one piece per row it touches.  All
//     128 heads share every 64-token cache tile ("Latent Attention.", "Compress,
//     then rebuild": one latent serves every head), so heads form the dense
//     MFMA dimension: S^T = K_tile . Q^T, online softmax, O^T += V^T . P^T
//     with the latent columns of the same tile as values.  Writes each
//     piece's normalised o_lat (fp16) and log-sum-exp.
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
// position  P(t, c) = (c >> 3) * 512 + t * 8 + ((c & 7) ^ g(t)):  groups of 8
// chunks are stored row by row, the chunk slot XOR-permuted per row by
//   g(t) = f(t & 7) ^ (2 * bit3(t)),  f(u) = ((u & 3) << 1) | ((u >> 2) & 1).
// With either 32 or 64 LDS banks this keeps
//  - 16 consecutive rows reading one chunk (the 16-byte score-operand reads)
//    on disjoint banks, and
//  - 4 consecutive rows x 2 adjacent chunks (the 8-byte transposed value reads
//    of one 16-lane group) on disjoint banks,
// while every global->LDS instruction still copies 8 rows x 128 contiguous bytes.
__device__ __forceinline__ int fswz(int t) {
    return (((t & 3) << 1) | ((t >> 2) & 1)) ^ ((t >> 2) & 2);
}
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
// with W_UK[h][:, cb*128 .. +128] staged in LDS as [n][col] rows of 288 bytes
// (256 + 32 of padding).  The MFMA A operand (32 latent columns x 16 n) is
// read with the transposing ds_read_b64_tr_b16: a 16-lane group reads 4 rows
// x 16 columns and each lane receives one column's 4 values; the padding puts
// the 4 rows of a group on disjoint banks.
constexpr int WT_ROWB = 288;    // bytes per staged W_UK row

__global__ __launch_bounds__(256) void absorb_q_kernel(
    const unsigned short* __restrict__ q_nope,  // [R][H][128]
    const unsigned short* __restrict__ q_pe,    // [R][H][64]
    const unsigned short* __restrict__ w_uk,    // [H][128][512]
    unsigned short* __restrict__ qbuf,          // [R][H][576]
    int R) {
    __shared__ __attribute__((aligned(16))) unsigned char wt[128 * WT_ROWB];
    const int bid = blockIdx.x;
    const int h = bid % H;
    const int cb = (bid / H) & 3;
    const int rb = bid / (H * 4);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, in an SGPR
    const int l32 = lane & 31, hf = lane >> 5;

    // W_UK[h][n][cb*128 .. +128]: 128 rows x 16 chunks of 16 B, 8 per thread
    u32x4 wv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int i = k * 256 + tid, n = i >> 4, c = i & 15;
        wv[k] = *reinterpret_cast<const u32x4*>(w_uk + ((size_t)h * 128 + n) * DC + cb * 128 + c * 8);
    }
    // this wave's q_nope fragments (B operands), loaded together with W_UK
    bf16x8 qv[8][2];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int r = rb * 64 + nb * 32 + l32;
            qv[ks][nb] = r < R ? *reinterpret_cast<const bf16x8*>(
                                     q_nope + ((size_t)r * H + h) * 128 + ks * 16 + hf * 8)
                               : bf16x8{};
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
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int i = k * 256 + tid, n = i >> 4, c = i & 15;
        *reinterpret_cast<u32x4*>(wt + n * WT_ROWB + c * 16) = wv[k];
    }
    __syncthreads();

    // A fragment of K-step ks: lane (hf, l32) needs column w*32 + l32 at
    // n = 16 ks + 8 hf .. +8.  16-lane group g = lane / 16 covers columns
    // 16 (g & 1) .. +16 of this wave's 32 and n offset 8 (g >> 1); lane
    // 4 r + b of a group points at row r, columns 4 b .. 4 b + 3.
    const int g = lane >> 4, r4 = (lane & 15) >> 2, b4 = lane & 3;
    const int a_off = (8 * (g >> 1) + r4) * WT_ROWB + (w * 32 + 16 * (g & 1) + 4 * b4) * 2;
    f32x16 acc[2] = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {                   // K = n, 16 per step
        const unsigned char* base = wt + ks * 16 * WT_ROWB + a_off;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(base));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(base + 4 * WT_ROWB));
        const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[nb] = mfma32(a, qv[ks][nb], acc[nb]);
    }
    // The output tile (64 query rows x 128 latent columns) goes through LDS so
    // that each row's 256-byte segment is written by one contiguous store:
    // from the accumulators a lane holds 8-byte pieces of 32 different rows.
    constexpr int OROWB = 272;                  // bytes per staged output row
    __syncthreads();                            // every wave is done reading W_UK
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const unsigned long long pk =
                (unsigned long long)f32_to_bf16_bits(acc[nb][4 * gg + 0]) |
                ((unsigned long long)f32_to_bf16_bits(acc[nb][4 * gg + 1]) << 16) |
                ((unsigned long long)f32_to_bf16_bits(acc[nb][4 * gg + 2]) << 32) |
                ((unsigned long long)f32_to_bf16_bits(acc[nb][4 * gg + 3]) << 48);
            *reinterpret_cast<unsigned long long*>(
                wt + (nb * 32 + l32) * OROWB + (w * 32 + 8 * gg + 4 * hf) * 2) = pk;
        }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {               // 64 rows x 16 chunks, 4 per thread
        const int i = k * 256 + tid, rl = i >> 4, c = i & 15;
        const int r = rb * 64 + rl;
        if (r < R)
            *reinterpret_cast<u32x4*>(qbuf + ((size_t)r * H + h) * D + cb * 128 + c * 8) =
                *reinterpret_cast<const u32x4*>(wt + rl * OROWB + c * 16);
    }
}

// ---------------------------------------------------------------------------
// 2. split-KV attention over the latent cache
// ---------------------------------------------------------------------------

// LDS-typed byte pointer.  Tile helpers take these so that the compiler's
// alias analysis can tell the tile being read from the one being filled.
typedef MLA_LDS unsigned char lds_u8;

// Issue the asynchronous copy of one bf16 cache block (64 rows x 1152 B,
// contiguous in memory) into an LDS tile.  Instruction i = 8 cg + q fills
// positions 64 i .. 64 i + 63: rows 8q .. 8q+7, chunk group cg.  Lane l takes
// row 8q + l/8 and slot l%8, i.e. chunk 8 cg + ((l%8) ^ g(8q + l/8)).
__device__ __forceinline__ void issue_tile_bf16(const unsigned char* __restrict__ gtile,
                                                lds_u8* ltile, int w, int lane) {
    // row 8q + l/8 has g = f(l/8) ^ 2 (q & 1): two per-lane offsets
    const unsigned off0 = (lane >> 3) * ROWB + (((lane & 7) ^ fswz(lane >> 3)) << 4);
    const unsigned off1 = (lane >> 3) * ROWB + (((lane & 7) ^ fswz((lane >> 3) + 8)) << 4);
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(gtile, GTILE);
#pragma unroll
    for (int k = 0; k < 18; ++k) {
        const int i = w * 18 + k;                      // wave-uniform
        const int cg = i >> 3, q = i & 7;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (MLA_LDS void*)(ltile + i * 1024), 16,
                                                 (q & 1) ? off1 : off0, q * 8 * ROWB + cg * 128,
                                                 0, 0);
    }
}

// Copy instruction k (0..17) of wave w of the bf16 tile copy above.
__device__ __forceinline__ void issue_tile_bf16_part(__amdgpu_buffer_rsrc_t rsrc, lds_u8* ltile,
                                                     int w, int lane, int k) {
    const unsigned off0 = (lane >> 3) * ROWB + (((lane & 7) ^ fswz(lane >> 3)) << 4);
    const int i = w * 18 + k;
    const int cg = i >> 3, q = i & 7;
    // rows 8q + 8 .. +7 (q odd) have g = f(l/8) ^ 2: chunk slot bit 1 flips
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (MLA_LDS void*)(ltile + i * 1024), 16,
                                             (q & 1) ? (off0 ^ 32u) : off0, q * 8 * ROWB + cg * 128,
                                             0, 0);
}

// Zero rows valid .. 63 of an LDS tile (their cache slots hold no token).
__device__ __forceinline__ void zero_rows(lds_u8* ltile, int valid, int tid) {
    for (int p = valid * NCH + tid; p < BS * NCH; p += 256) {
        const int t = p / NCH, c = p - t * NCH;
        *reinterpret_cast<MLA_LDS u32x4*>(ltile + tpos(t, c) * 16) = u32x4{0, 0, 0, 0};
    }
}

// Asynchronous copy of one fp8 cache block (64 rows x 576 B, contiguous) into
// row-major LDS staging, plus its 64 per-token scales after it.
__device__ __forceinline__ void issue_tile_fp8(const unsigned char* __restrict__ gtile,
                                               const float* __restrict__ gscale,
                                               lds_u8* lstage, int w, int lane) {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(gtile, F8TILE);
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const int i = w * 9 + k;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (MLA_LDS void*)(lstage + i * 1024), 16,
                                                 lane * 16, i * 1024, 0, 0);
    }
    if (w == 0) {
        const __amdgpu_buffer_rsrc_t srs = make_rsrc(gscale, BS * 4);
        if (lane < 16)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (MLA_LDS void*)(lstage + F8TILE), 16,
                                                     lane * 16, 0, 0, 0);
    }
}

// fp8 scores: the staging tile keeps rows 37 chunks (592 bytes) apart, so the
// score operand reads of 16 consecutive rows (one 16-byte chunk each, row
// stride 148 dwords) fall on distinct banks.  Position p = 64 i + lane of copy
// instruction i holds chunk p % 37 of row p / 37; the 37th chunk of a row is
// padding (it repeats chunk 35).  37 instructions, spread over the 4 waves;
// the 64 scales follow the codes.
constexpr int F8ROW = 37;                       // 16-byte chunks per padded staging row
constexpr int F8SCODES = BS * F8ROW * 16;       // 37888 bytes
__device__ __forceinline__ void issue_tile_fp8_padded(const unsigned char* __restrict__ gtile,
                                                      const float* __restrict__ gscale,
                                                      lds_u8* lstage, int w, int lane) {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(gtile, F8TILE);
#pragma unroll 1
    for (int i = w; i < BS * F8ROW / 64; i += 4) {
        const int p = i * 64 + lane;
        const int t = p / F8ROW, c = p - t * F8ROW;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (MLA_LDS void*)(lstage + i * 1024), 16,
                                                 t * D + min(c, F8CHUNKS - 1) * 16, 0, 0, 0);
    }
    if (w == 0) {
        const __amdgpu_buffer_rsrc_t srs = make_rsrc(gscale, BS * 4);
        if (lane < 16)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (MLA_LDS void*)(lstage + F8SCODES), 16,
                                                     lane * 16, 0, 0, 0);
    }
}

// Padded fp8 staging -> bf16 tile of the codes' values, latent channels only
// (the scores read the codes themselves).  Rows at or beyond `valid` become
// zeros, and so do their token scales.
__device__ __forceinline__ void convert_tile_fp8_latent(lds_u8* lstage, lds_u8* ltile, int tid,
                                                        int valid) {
    MLA_LDS float* lscale = reinterpret_cast<MLA_LDS float*>(lstage + F8SCODES);
    if (tid < BS && tid >= valid) lscale[tid] = 0.f;
#pragma unroll 1
    for (int k = 0; k < 8; ++k) {
        const int p = k * 256 + tid;                   // 64 rows x 32 latent chunks
        const int t = p >> 5, c = p & 31;
        u32x4 outw[2];
        if (t < valid) {
            const u32x4 raw = *reinterpret_cast<const MLA_LDS u32x4*>(lstage + (t * F8ROW + c) * 16);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // codes 4q, 4q+1 and 4q+2, 4q+3 as bf16 pairs (exact: unit scale)
                const unsigned int p0 = __builtin_bit_cast(
                    unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[q], 1.0f, false));
                const unsigned int p1 = __builtin_bit_cast(
                    unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[q], 1.0f, true));
                outw[q >> 1][(q & 1) * 2 + 0] = p0;
                outw[q >> 1][(q & 1) * 2 + 1] = p1;
            }
        } else {
            outw[0] = u32x4{0, 0, 0, 0};
            outw[1] = u32x4{0, 0, 0, 0};
        }
        *reinterpret_cast<MLA_LDS u32x4*>(ltile + tpos(t, 2 * c) * 16) = outw[0];
        *reinterpret_cast<MLA_LDS u32x4*>(ltile + tpos(t, 2 * c + 1) * 16) = outw[1];
    }
}

// fp8 staging -> bf16 swizzled tile of the codes' values.  Every e4m3 value is
// a bf16 value (3 of 7 mantissa bits, a narrower exponent range), so the copy
// is exact; the token scale is applied to the scores and the weights instead.
// Rows at or beyond `valid` become zeros, and so do their token scales (past a
// sequence's end a block may hold anything).
__device__ __forceinline__ void convert_tile_fp8(lds_u8* lstage, lds_u8* ltile, int tid,
                                                 int valid) {
    MLA_LDS float* lscale = reinterpret_cast<MLA_LDS float*>(lstage + F8TILE);
    if (tid < BS && tid >= valid) lscale[tid] = 0.f;
#pragma unroll 1
    for (int k = 0; k < 9; ++k) {
        const int p = k * 256 + tid;                   // 2304 fp8 chunks
        const int t = p / F8CHUNKS, c = p - t * F8CHUNKS;
        u32x4 outw[2];
        if (t < valid) {
            const u32x4 raw = *reinterpret_cast<const MLA_LDS u32x4*>(lstage + p * 16);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // codes 4q, 4q+1 and 4q+2, 4q+3 as bf16 pairs (exact: unit scale)
                const unsigned int p0 = __builtin_bit_cast(
                    unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[q], 1.0f, false));
                const unsigned int p1 = __builtin_bit_cast(
                    unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[q], 1.0f, true));
                outw[q >> 1][(q & 1) * 2 + 0] = p0;
                outw[q >> 1][(q & 1) * 2 + 1] = p1;
            }
        } else {
            outw[0] = u32x4{0, 0, 0, 0};
            outw[1] = u32x4{0, 0, 0, 0};
        }
        *reinterpret_cast<MLA_LDS u32x4*>(ltile + tpos(t, 2 * c) * 16) = outw[0];
        *reinterpret_cast<MLA_LDS u32x4*>(ltile + tpos(t, 2 * c + 1) * 16) = outw[1];
    }
}

// ---------------------------------------------------------------------------
// work partition of the split-KV pass
// ---------------------------------------------------------------------------
//
// Query row r = b * q_len + s (token s of sequence b) sees the first
// seq_lens[b] - q_len + s + 1 cache tokens, i.e. tiles(r) 64-token tiles.
//  - num_splits > 0: row r is cut into num_splits equal ranges of whole tiles,
//    one workgroup each; partial slot r * num_splits + split.
//  - num_splits == 0 (balanced): the rows' tiles, concatenated in row order,
//    are cut into G equal ranges [i T / G, (i+1) T / G), one per workgroup
//    (T = total tiles, G = min(grid, ceil(T / 4)) <= T, so no range is empty;
//    workgroups past G have nothing to do).  A range may span several rows; each
//    (workgroup i, row r) piece writes partial slot i + r.  Slots are unique:
//    for i < i' the rows of i end no later than the rows of i' begin, so
//    i + r < i' + r'.  Row r's pieces occupy slots first(r) + r .. last(r) + r,
//    first / last being the workgroups holding its first / last tile.

__device__ __forceinline__ int row_tiles(const int* __restrict__ seq_lens, int q_len, int r) {
    const int b = r / q_len;
    const int n_vis = seq_lens[b] - q_len + (r - b * q_len) + 1;
    return n_vis > 0 ? (n_vis + BS - 1) / BS : 0;
}

// Workgroups of the balanced schedule for T tiles: at most one per compute
// unit (the grid), and at least kMinGroupTiles tiles each, so that a small
// batch does not pay a workgroup's fixed costs (query load, partial write,
// one more partial to merge) for a single tile.
constexpr int kMinGroupTiles = 4;
__device__ __forceinline__ long long balanced_groups(long long grid, long long T) {
    return min(grid, (T + kMinGroupTiles - 1) / kMinGroupTiles);
}

// Workgroup holding tile t of the concatenated tiles (T tiles over G groups).
__device__ __forceinline__ int group_of_tile(long long t, long long T, long long G) {
    return (int)(((t + 1) * G + T - 1) / T - 1);
}

// Block-wide scan of row tile counts: thread tid owns rows [tid*per, tid*per+per)
// (per = ceil(R / 256)).  Returns T; *excl / *mine receive the tiles before this
// thread's rows and in them.  sc: 260 ints of LDS scratch.
template <typename LdsInt>
__device__ __forceinline__ int scan_row_tiles(const int* __restrict__ seq_lens, int q_len, int R,
                                              LdsInt sc, int* excl, int* mine) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int per = (R + 255) / 256;
    int local = 0;
    for (int k = 0; k < per; ++k) {
        const int r = tid * per + k;
        if (r < R) local += row_tiles(seq_lens, q_len, r);
    }
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    if (lane == 63) sc[256 + w] = incl;
    __syncthreads();
    int off = 0;
    for (int k = 0; k < w; ++k) off += sc[256 + k];
    const int T = sc[256] + sc[257] + sc[258] + sc[259];
    *excl = off + incl - local;
    *mine = local;
    return T;
}

// A piece (row, tiles [t0, t1)): row = b * q_len + s is query token s of
// sequence b; the piece covers all 128 heads over those tiles of the row's
// visible range.  A workgroup handles one piece (fixed partitions) or the
// consecutive pieces its balanced share of the tile sequence spans.
// Wave w owns heads 32w .. 32w+31 for the whole tile loop; each 64-token tile
// is processed as two halves of 32 tokens:
//   S^T (32 tokens x 32 heads) = K_half (32 x 576) . Q_w^T   [36 MFMA]
//   O^T (512 cols x 32 heads) += V^T (512 x 32) . P^T         [32 MFMA]
// so softmax statistics stay inside the wave.  Q_w stays in VGPRs (its rotary
// part in LDS on the bf16 path) and O^T in AGPRs for the whole loop.
// F8S (fp8 cache only): the score product runs on the fp8 matrix cores, with
// the cache codes as they are and the queries quantised to e4m3 with one scale
// per (row, head); the value product stays bf16.
template <bool FP8, bool F8S = false>
__global__ __launch_bounds__(256, 1) void split_kv_kernel(
    const unsigned short* __restrict__ qbuf,      // [R][H][576] bf16
    const unsigned char* __restrict__ pool,       // [blocks][64][576] bf16 | fp8
    const float* __restrict__ pool_scale,         // [blocks][64] (fp8)
    const int* __restrict__ block_table, int max_blocks,
    const int* __restrict__ seq_lens, int R, int q_len, int num_splits, float scale_log2,
    unsigned short* __restrict__ part_o,          // [slots][H][512] fp16
    float* __restrict__ part_lse) {               // [slots][H]
    // bf16: two tiles + the rotary queries of all heads (16 KB) = 160 KiB;
    // fp8: one bf16 tile + two fp8 staging tiles with scales (rotary queries in VGPRs)
    constexpr bool QPE_LDS = !FP8;
    constexpr int QPE_BYTES = H * DR * 2;
    static_assert(FP8 || !F8S, "fp8 scores need an fp8 cache");
    constexpr int STAGE = (F8S ? F8SCODES : F8TILE) + 256;   // fp8 staging buffer: codes + scales
    constexpr int LDS_BYTES = FP8 ? (TILE + 2 * STAGE) : (2 * TILE + QPE_BYTES);
    constexpr int NQ = F8S ? 1 : (QPE_LDS ? 32 : 36);   // bf16 query K-steps kept in VGPRs
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[LDS_BYTES];
    lds_u8* smem = (lds_u8*)smem_raw;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, in an SGPR
    const int l32 = lane & 31, hf = lane >> 5;
    const int head = w * 32 + l32;

    // ---- this workgroup's pieces (row, tiles [t0, t1), partial slot) ---------------
    int cur_row = 0, cur_rs = 0, rng_a = 0, rng_b = 0;   // balanced: walk state
    bool fixed_pending = num_splits > 0;
    if (num_splits == 0) {
        MLA_LDS int* sc = reinterpret_cast<MLA_LDS int*>(smem);
        int excl, mine;
        const int T = scan_row_tiles(seq_lens, q_len, R, sc, &excl, &mine);
        const long long G = balanced_groups(gridDim.x, T);
        if ((long long)blockIdx.x >= G) return;      // uniform: the whole workgroup leaves
        rng_a = (int)((long long)blockIdx.x * T / G);
        rng_b = (int)((long long)(blockIdx.x + 1) * T / G);
        if (rng_a < rng_b && excl <= rng_a && rng_a < excl + mine) {
            const int per = (R + 255) / 256;
            int rs = excl;
            for (int k = 0; k < per; ++k) {
                const int r = tid * per + k;
                const int nt = r < R ? row_tiles(seq_lens, q_len, r) : 0;
                if (rng_a < rs + nt) {
                    sc[260] = r;
                    sc[261] = rs;
                    break;
                }
                rs += nt;
            }
        }
        __syncthreads();
        if (rng_a < rng_b) {
            cur_row = sc[260];
            cur_rs = sc[261];
        }
        __syncthreads();                 // scratch read before the tiles reuse it
    }
    auto next_piece = [&](int& row, int& t0, int& t1, int& slot) -> bool {
        if (num_splits > 0) {
            if (!fixed_pending) return false;
            fixed_pending = false;
            row = blockIdx.x / num_splits;
            const int split = blockIdx.x - row * num_splits;
            const int n_tiles = row_tiles(seq_lens, q_len, row);
            const int tps = (n_tiles + num_splits - 1) / num_splits;
            t0 = split * tps;
            t1 = min(n_tiles, t0 + tps);
            slot = blockIdx.x;
            if (t0 >= t1) {              // nothing visible in this range
                if (tid < H) part_lse[(size_t)slot * H + tid] = kNegInf;
                return false;
            }
            return true;
        }
        while (cur_rs < rng_b && cur_row < R) {
            const int r = cur_row, rs = cur_rs;
            const int nt = row_tiles(seq_lens, q_len, r);
            cur_row += 1;
            cur_rs += nt;
            const int lo = max(rng_a, rs) - rs, hi = min(rng_b, rs + nt) - rs;
            if (hi > lo) {
                row = r;
                t0 = lo;
                t1 = hi;
                slot = blockIdx.x + r;
                return true;
            }
        }
        return false;
    };

    int row, t0, t1, slot;
    for (int piece = 0; next_piece(row, t0, t1, slot); ++piece) {
        if (piece > 0) __syncthreads();      // the previous piece's epilogue is done with LDS
        const int b = row / q_len, s = row - b * q_len;
        const int n_vis = seq_lens[b] - q_len + s + 1;
        float* lse_dst = part_lse + (size_t)slot * H;
        const int* btab = block_table + (size_t)b * max_blocks;

        // bf16: tiles at 0 and TILE, rotary queries at 2 TILE.
        // fp8: the bf16 tile at 0, staging buffers at TILE and TILE + STAGE.
        lds_u8* qpe = smem + 2 * TILE;

        auto valid_of = [&](int t) { return min(BS, n_vis - t * BS); };
        // asynchronous load of tile t into `dst` (a bf16 tile, or fp8 staging)
        auto issue = [&](int t, lds_u8* dst) {
            const size_t blk = (size_t)btab[t];
            if constexpr (F8S) {
                issue_tile_fp8_padded(pool + blk * F8TILE, pool_scale + blk * BS, dst, w, lane);
            } else if constexpr (FP8) {
                issue_tile_fp8(pool + blk * F8TILE, pool_scale + blk * BS, dst, w, lane);
            } else {
                issue_tile_bf16(pool + blk * GTILE, dst, w, lane);
            }
        };
        // The first tile's copy goes out before the query loads, so that the two
        // memory round trips of a piece's start overlap.
        issue(t0, FP8 ? smem + TILE : smem);
        bool t0_in_flight = true;

        // this wave's 32 query rows, as MFMA B fragments: lane (hf, l32) holds
        // channels 16 ks + 8 hf .. +8 of head 32 w + l32
        bf16x8 qf[NQ];
        if constexpr (!F8S) {
            const unsigned short* qrow = qbuf + ((size_t)row * H + head) * D + hf * 8;
#pragma unroll
            for (int ks = 0; ks < NQ; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
        }
        // fp8 scores: the fp8 B fragments of K-step s (64 channels) hold channels
        // 64 s + 32 hf .. +32 of head 32 w + l32, divided by the head's scale
        // 2^e, the smallest power of two with amax <= 448 * 2^e, and rounded to
        // nearest even.  The division is exact, so the rounding sees the exact
        // quotient; |q| / 2^e <= 448 never saturates.
        [[maybe_unused]] i32x8 qc[F8S ? 9 : 1];
        [[maybe_unused]] float qscale = 1.f;
        if constexpr (F8S) {
            const unsigned short* qrow = qbuf + ((size_t)row * H + head) * D + hf * 32;
            u32x4 raw[9][4];
            float amax = 0.f;
#pragma unroll
            for (int s8 = 0; s8 < 9; ++s8)
#pragma unroll
                for (int j = 0; j < 4; ++j) raw[s8][j] = *reinterpret_cast<const u32x4*>(qrow + 64 * s8 + 8 * j);
#pragma unroll
            for (int s8 = 0; s8 < 9; ++s8)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const unsigned u = raw[s8][j][e];
                        amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32((unsigned short)u)),
                                                 fabsf(bf16_bits_to_f32((unsigned short)(u >> 16)))));
                    }
            amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
            // amax = f 2^E, 0.5 <= f < 1, and 448 = 0.875 2^9
            int ex = 0;
            const float fm = frexpf(amax, &ex);
            const int qe = amax > 0.f ? (fm <= 0.875f ? ex - 9 : ex - 8) : 0;
            qscale = ldexpf(1.0f, qe);
            const float inv = ldexpf(1.0f, -qe);
#pragma unroll
            for (int s8 = 0; s8 < 9; ++s8)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // 8 bf16 -> 8 e4m3 codes (2 dwords)
                    const u32x4 u = raw[s8][j];
                    int d0 = 0, d1 = 0;
                    d0 = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_bits_to_f32((unsigned short)u[0]) * inv,
                                                         bf16_bits_to_f32((unsigned short)(u[0] >> 16)) * inv, d0, false);
                    d0 = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_bits_to_f32((unsigned short)u[1]) * inv,
                                                         bf16_bits_to_f32((unsigned short)(u[1] >> 16)) * inv, d0, true);
                    d1 = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_bits_to_f32((unsigned short)u[2]) * inv,
                                                         bf16_bits_to_f32((unsigned short)(u[2] >> 16)) * inv, d1, false);
                    d1 = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_bits_to_f32((unsigned short)u[3]) * inv,
                                                         bf16_bits_to_f32((unsigned short)(u[3] >> 16)) * inv, d1, true);
                    qc[s8][2 * j] = d0;
                    qc[s8][2 * j + 1] = d1;
                }
        }
        if constexpr (QPE_LDS) {
            // q_pe of all heads: head h's chunk c (8 channels) at h*128 + ((c ^ g(h)) << 4)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = k * 256 + tid;               // 1024 chunks
                const int h = i >> 3, c = i & 7;
                const u32x4 v = *reinterpret_cast<const u32x4*>(qbuf + ((size_t)row * H + h) * D + DC + c * 8);
                *reinterpret_cast<MLA_LDS u32x4*>(qpe + h * 128 + ((c ^ fswz(h & 15)) << 4)) = v;
            }
        }
        const lds_u8* qpe_lane = qpe + head * 128;
        const int qpe_g = fswz(head & 15);


        // Per-lane LDS byte offsets.  Score operand (chunk 2 ks + hf of row
        // 32 hb + l32): by ks % 4.  Transposed value reads (in a 16-lane group,
        // lane 4r + b reads row 4 hf + r (+8), channels 4b .. 4b+3 of a 16-channel
        // block): by cm % 2 and by the +8 row offset.
        int qk_off[4], tr_off[2][2];
#pragma unroll
        for (int j = 0; j < 4; ++j) qk_off[j] = (l32 * 8 + ((2 * j + hf) ^ fswz(l32 & 15))) * 16;
        {
            const int r = (lane & 15) >> 2, g1 = (lane >> 4) & 1, b1 = (lane >> 1) & 1;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int t = 8 * e + 4 * hf + r;      // row within a 16-row group
                    tr_off[j][e] = (t * 8 + ((4 * j + 2 * g1 + b1) ^ fswz(t))) * 16 + (lane & 1) * 8;
                }
        }

        // Softmax without rescaling the accumulators: every weight of a pass is
        // exp2(s - m_ref) for one reference m_ref per head.  The first pass takes
        // m_ref from the first half-tile; if a later half-tile's maximum exceeds it
        // by more than kMaxLead (weights stay below 2^64, far from fp32 overflow)
        // the pass's result is discarded, one scan computes the exact maximum and
        // a last pass runs with it.  (Scaling O inside the loop would force the
        // 256 accumulators out of AGPRs.)  The waves vote after the loop, in LDS.
        constexpr float kMaxLead = 64.0f;
        f32x16 o[16];
        float m_ref = kNegInf, l_run = 0.f;
        bool overflow = false;
        int mode = 0;                        // 0: first-tile reference, 1: max scan, 2: exact reference

        // One tile: start the load of the next tile into `nxt` (when there is
        // one), then attend over the 64 cache rows in `tile`.  The two buffers
        // never overlap; saying so (restrict) lets the compiler keep the
        // transposed value reads from waiting on the load in flight.
        auto run_tile = [&](int t, const lds_u8* __restrict__ tile, lds_u8* __restrict__ nxt,
                            const lds_u8* __restrict__ stg, bool has_next) __attribute__((always_inline)) {
            (void)stg;
            const int valid = valid_of(t);
            // bf16: the next tile's 18 copy instructions of this wave are spread
            // over the two score chains (one every 4 MFMAs); issued as one burst
            // they hold the wave at issue while the address unit works through
            // the workgroup's 72 copies.  Without a next tile the resource has no
            // records and the copies read nothing.
            [[maybe_unused]] __amdgpu_buffer_rsrc_t nrs;
            if constexpr (FP8) {
                if (has_next) issue(t + 1, nxt);
            } else {
                nrs = make_rsrc(pool + (size_t)btab[has_next ? t + 1 : t] * GTILE, has_next ? GTILE : 0);
            }
#pragma unroll 1
            for (int hb = 0; hb < 2; ++hb) {
                if (hb * 32 >= valid) break;
                // ---- S^T = K . Q^T: rows 32 hb + l32 -----------------------------------
                const lds_u8* kbase = tile + hb * 32 * 128;
                auto ka = [&](int ks) {
                    return *reinterpret_cast<const MLA_LDS bf16x8*>(kbase + qk_off[ks & 3] + (ks >> 2) * 8192);
                };
                auto qb = [&](int ks) -> bf16x8 {
                    if (ks < NQ) return qf[ks];
                    const int c = 2 * (ks - 32) + hf;
                    return *reinterpret_cast<const MLA_LDS bf16x8*>(qpe_lane + ((c ^ qpe_g) << 4));
                };
                f32x16 sacc = {};
                float sv[16];
                // fp8: token scales of the lane's rows 32 hb + 8 (i/4) + 4 hf + (i%4)
                // (zero past the sequence end), applied to the scores and folded
                // into the weights, so that keys and values enter the products as
                // the codes' exact values
                [[maybe_unused]] float tsc[16];
                if constexpr (FP8) {
                    const MLA_LDS float* lsc =
                        reinterpret_cast<const MLA_LDS float*>(stg + (F8S ? F8SCODES : F8TILE));
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 ks4 = *reinterpret_cast<const MLA_LDS f32x4*>(lsc + hb * 32 + 8 * g + 4 * hf);
#pragma unroll
                        for (int j = 0; j < 4; ++j) tsc[4 * g + j] = ks4[j];
                    }
                }
                if constexpr (F8S) {
                    // codes of rows 32 hb + l32, channels 64 s + 32 hf .. +32: two
                    // consecutive 16-byte chunks of the padded staging row
                    const lds_u8* srow = stg + ((hb * 32 + l32) * F8ROW + 2 * hf) * 16;
                    auto kc = [&](int s8) {
                        const u32x4 lo = *reinterpret_cast<const MLA_LDS u32x4*>(srow + s8 * 64);
                        const u32x4 hi = *reinterpret_cast<const MLA_LDS u32x4*>(srow + s8 * 64 + 16);
                        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    };
                    i32x8 a0 = kc(0), a1 = kc(1), a2;
#pragma unroll
                    for (int s8 = 0; s8 < 9; ++s8) {
                        if (s8 + 2 < 9) a2 = kc(s8 + 2);
                        // e4m3 x e4m3, unit block scales (e8m0 127 = 1.0)
                        sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, qc[s8], sacc, 0, 0, 0, 127, 0, 127);
                        a0 = a1;
                        a1 = a2;
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) sv[i] = sacc[i] * qscale * tsc[i];
                } else {
                    bf16x8 a0 = ka(0), a1 = ka(1), a2;
#pragma unroll
                    for (int ks = 0; ks < 36; ++ks) {
                        if (ks + 2 < 36) a2 = ka(ks + 2);
                        sacc = mfma32(a0, qb(ks), sacc);
                        if constexpr (!FP8) {
                            if ((ks & 3) == 0) issue_tile_bf16_part(nrs, nxt, w, lane, hb * 9 + (ks >> 2));
                        }
                        a0 = a1;
                        a1 = a2;
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) sv[i] = FP8 ? sacc[i] * tsc[i] : sacc[i];
                }
                // lane holds head `head`, tokens 32 hb + 8 (i/4) + 4 hf + (i%4)
                if (valid < BS) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int tok = hb * 32 + (i >> 2) * 8 + 4 * hf + (i & 3);
                        if (tok >= valid) sv[i] = kNegInf;
                    }
                }
                // sv holds unscaled scores; the log2-domain score is sv * scale_log2
                // (scale_log2 > 0, so maxima commute with the scaling).  Maxima and
                // sums stay per lane here; the two lanes of a head (hf = 0, 1) are
                // combined once per pass, not per half-tile.
                float hmax = sv[0];
#pragma unroll
                for (int i = 1; i < 16; ++i) hmax = fmaxf(hmax, sv[i]);
                hmax *= scale_log2;
                if (mode == 1) {
                    m_ref = fmaxf(m_ref, hmax);
                    continue;
                }
                if (mode == 0 && t == t0 && hb == 0) m_ref = fmaxf(hmax, __shfl_xor(hmax, 32, 64));
                // (cannot hold in the exact-reference pass: the scan saw the same
                // maxima, so at most three passes run)
                overflow |= hmax > m_ref + kMaxLead;

                float psum = 0.f;
                bf16x8 pf[2];
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    u16x8 pu;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[k2 * 8 + j], scale_log2, -m_ref));
                        psum += pv;
                        pu[j] = f32_to_bf16_bits(FP8 ? pv * tsc[k2 * 8 + j] : pv);
                    }
                    pf[k2] = __builtin_bit_cast(bf16x8, pu);
                }
                l_run += psum;

                // ---- O^T += V^T . P^T (latent columns of the same rows) -----------------
                // K-step k2 covers tokens 32 hb + 16 k2 + {0..3, 8..11} (lanes 0-31)
                // and {4..7, 12..15} (lanes 32-63), matching P's layout.  Fragments
                // are read one step ahead; k2 runs outermost so that consecutive
                // MFMAs update different accumulators.
                auto va = [&](int k2, int cm) {
                    const lds_u8* vb = tile + (cm >> 1) * 8192 + (hb * 32 + k2 * 16) * 128;
                    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (MLA_LDS bf16x4*)(vb + tr_off[cm & 1][0]));
                    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (MLA_LDS bf16x4*)(vb + tr_off[cm & 1][1]));     // rows +8 are in the offset
                    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                };
                bf16x8 v0 = va(0, 0), v1;
#pragma unroll
                for (int st = 0; st < 32; ++st) {
                    const int k2 = st >> 4, cm = st & 15;
                    if (st + 1 < 32) v1 = va((st + 1) >> 4, (st + 1) & 15);
                    o[cm] = mfma32(v0, pf[k2], o[cm]);
                    v0 = v1;
                }
            }
        };

        for (;;) {
#pragma unroll
            for (int i = 0; i < 16; ++i) o[i] = f32x16{};
            l_run = 0.f;
            overflow = false;
            if (!t0_in_flight) issue(t0, FP8 ? smem + TILE : smem);   // a later pass
            t0_in_flight = false;
            for (int t = t0; t < t1; ++t) {
                const int cur = (t - t0) & 1;
                wait_vmem_all();
                __syncthreads();             // tile t landed; previous tile fully consumed
                const bool has_next = t + 1 < t1;
                if constexpr (FP8) {
                    lds_u8* st_cur = smem + TILE + cur * STAGE;
                    lds_u8* st_nxt = smem + TILE + (cur ^ 1) * STAGE;
                    if constexpr (F8S) {
                        convert_tile_fp8_latent(st_cur, smem, tid, valid_of(t));
                    } else {
                        convert_tile_fp8(st_cur, smem, tid, valid_of(t));
                    }
                    __syncthreads();
                    run_tile(t, smem, st_nxt, st_cur, has_next);
                } else {
                    lds_u8* cur_tile = smem + cur * TILE;
                    lds_u8* nxt_tile = smem + (cur ^ 1) * TILE;
                    if (valid_of(t) < BS) {  // last, partial tile of the sequence
                        zero_rows(cur_tile, valid_of(t), tid);
                        __syncthreads();
                    }
                    run_tile(t, cur_tile, nxt_tile, nullptr, has_next);
                }
            }
            // ---- vote: did any wave's weights run past the reference? ------------------
            wait_vmem_all();                 // (record-less copies of the last tile included)
            __syncthreads();                 // all waves are done with the tiles
            MLA_LDS int* votes = reinterpret_cast<MLA_LDS int*>(smem);
            if (lane == 0) votes[w] = __builtin_amdgcn_ballot_w64(overflow) != 0;
            __syncthreads();
            const bool redo = (votes[0] | votes[1] | votes[2] | votes[3]) != 0;
            __syncthreads();                 // votes read before the next pass reuses the tiles
            if (redo) {
                mode = 1;
                m_ref = kNegInf;
                continue;
            }
            if (mode == 1) {             // the scan's maxima: both lanes of each head
                m_ref = fmaxf(m_ref, __shfl_xor(m_ref, 32, 64));
                mode = 2;
                continue;
            }
            break;
        }
        l_run += __shfl_xor(l_run, 32, 64);  // the head's two lanes hold disjoint tokens

        // ---- epilogue: normalised partial o_lat (fp16) and log-sum-exp ---------------
        // The partial is a convex combination of latent rows: fp16 keeps it to
        // 2^-11 relative and halves the bytes every workgroup writes at the same
        // moment (and the combine reads).  A lane holds 16-byte pieces of 32
        // different head rows, so each wave transposes through its own LDS region
        // (the tiles are free after the vote barrier) and writes every head row as
        // one 1 KB store.  Row stride 520 halves: the 8-byte writes of 16
        // consecutive lanes (16 head rows) fall on distinct banks.  Waves start
        // at different rows so that concurrent stores spread over memory channels.
        constexpr int OSTR = 520;
        const float inv_l = 1.0f / l_run;
        MLA_LDS unsigned short* ost = reinterpret_cast<MLA_LDS unsigned short*>(smem + w * (32 * OSTR * 2));
#pragma unroll
        for (int cm = 0; cm < 16; ++cm)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u16x4 hv;
#pragma unroll
                for (int j = 0; j < 4; ++j) hv[j] = f32_to_f16_bits(o[cm][4 * g + j] * inv_l);
                *reinterpret_cast<MLA_LDS u16x4*>(ost + l32 * OSTR + cm * 32 + g * 8 + 4 * hf) = hv;
            }
        // LDS operations of one wave complete in order: the reads see the writes
        unsigned short* po = part_o + ((size_t)slot * H + w * 32) * DC + lane * 8;
        const int rot = (blockIdx.x * 4 + w) & 31;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int hh = (i + rot) & 31;
            const u32x4 v = *reinterpret_cast<const MLA_LDS u32x4*>(ost + hh * OSTR + lane * 8);
            *reinterpret_cast<u32x4*>(po + hh * DC) = v;
        }
        if (hf == 0) lse_dst[head] = (m_ref + __builtin_log2f(l_run)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// 3. log-sum-exp combine of partitions, then out = W_UV o_lat
// ---------------------------------------------------------------------------

// grid: H * ceil(R / 32) workgroups (h fastest, so one head's row blocks share
// an XCD and its W_UV slice in L2).  Workgroup (h, rb) handles rows rb*32 ..
// +32 of head h; wave w combines rows 8w .. 8w+7, then computes
// out^T[32w .. +32][rows] = W_UV[h] o_lat^T.  Every phase issues its global
// loads together (partition weights, then all partitions of 8 rows, then the
// whole W_UV slice) so each costs about one memory round trip.
__global__ __launch_bounds__(256) void combine_kernel(
    const unsigned short* __restrict__ part_o,  // [slots][H][512] fp16
    const float* __restrict__ part_lse,         // [slots][H]
    const int* __restrict__ seq_lens, int q_len, int R, int num_splits, int groups,
    const unsigned short* __restrict__ w_uv,    // [H][128][512]
    unsigned short* __restrict__ out,           // [R][H][128] bf16
    float* __restrict__ lse_out) {              // [R][H] or null
    __shared__ __attribute__((aligned(16))) unsigned char ol[2][32 * 1024];   // hi, lo bf16
    __shared__ float wts[32][kMaxSplits];       // normalised partition weights per local row
    const int h = blockIdx.x % H;
    const int rb = blockIdx.x / H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, in an SGPR
    const int l32 = lane & 31, hf = lane >> 5;
    __shared__ int pbase[32], pcnt[32];         // partial slots of each local row

    // ---- where each row's partials are (see the split-KV work partition)
    if (num_splits > 0) {
        if (tid < 32) {
            const bool in = rb * 32 + tid < R;
            pbase[tid] = in ? (rb * 32 + tid) * num_splits : 0;
            pcnt[tid] = in ? num_splits : 0;
        }
    } else {
        int* sc = reinterpret_cast<int*>(&wts[0][0]);
        int excl, mine;
        const int T = scan_row_tiles(seq_lens, q_len, R, sc, &excl, &mine);
        const int per = (R + 255) / 256;
        int rs = excl;
        for (int k = 0; k < per; ++k) {
            const int r = tid * per + k;
            if (r >= R) break;
            const int nt = row_tiles(seq_lens, q_len, r);
            if (r >= rb * 32 && r < rb * 32 + 32) {
                const int G = (int)balanced_groups(groups, T);
                const int f = nt > 0 ? group_of_tile(rs, T, G) : 0;
                const int l = nt > 0 ? group_of_tile(rs + nt - 1, T, G) : -1;
                pbase[r - rb * 32] = f + r;
                pcnt[r - rb * 32] = l - f + 1;
            }
            rs += nt;
        }
        if (tid < 32 && rb * 32 + tid >= R) {
            pbase[tid] = 0;
            pcnt[tid] = 0;
        }
    }
    __syncthreads();

    // ---- partition weights exp(lse_s - max) / sum and the merged lse; lanes
    // run over partitions (at most 256 = 4 x 64)
    int S = 0;                                  // most partials of this wave's rows
    {
        float lv[8][4];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const int base = pbase[w * 8 + rr], cnt = pcnt[w * 8 + rr];
            S = max(S, cnt);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sp = lane + 64 * j;
                lv[rr][j] = sp < cnt ? part_lse[((size_t)base + sp) * H + h] : kNegInf;
            }
        }
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const int rl = w * 8 + rr, r = rb * 32 + rl;
            const float mx = wave_max(fmaxf(fmaxf(lv[rr][0], lv[rr][1]), fmaxf(lv[rr][2], lv[rr][3])));
            float e[4], tot = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                e[j] = lv[rr][j] == kNegInf ? 0.f : __expf(lv[rr][j] - mx);
                tot += e[j];
            }
            tot = wave_sum(tot);
            const float inv = tot > 0.f ? 1.0f / tot : 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (lane + 64 * j < kMaxSplits) wts[rl][lane + 64 * j] = e[j] * inv;
            if (lse_out != nullptr && lane == 0 && r < R)
                lse_out[(size_t)r * H + h] = (mx == kNegInf) ? kNegInf : mx + __logf(tot);
        }
    }
    // (each wave reads back only its own rows' weights: LDS operations of one
    // wave complete in order)

    // ---- o_lat of rows 8w .. 8w+7: lane holds columns 8 lane .. 8 lane + 7.
    // A partition with no visible token has weight 0 and an unwritten partial:
    // select, never multiply, so whatever that memory holds cannot leak in.
    float acc[8][8];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[rr][j] = 0.f;
    const unsigned short* pcol = part_o + (size_t)h * DC + lane * 8;
#pragma unroll 2
    for (int sp = 0; sp < S; ++sp) {
        u32x4 v[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            // past a row's last partial the weight is 0: read its first one
            const int sl = pbase[w * 8 + rr] + (sp < pcnt[w * 8 + rr] ? sp : 0);
            v[rr] = *reinterpret_cast<const u32x4*>(pcol + (size_t)sl * H * DC);
        }
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const float wt = wts[w * 8 + rr][sp];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = f16_bits_to_f32((unsigned short)(v[rr][j >> 1] >> (16 * (j & 1))));
                acc[rr][j] += wt != 0.f ? wt * x : 0.f;
            }
        }
    }
    // W_UV slice of this wave's 32 output rows: all 32 fragments at once
    bf16x8 wa[32];
    {
        const unsigned short* wrow = w_uv + ((size_t)h * 128 + w * 32 + l32) * DC + hf * 8;
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) wa[ks] = *reinterpret_cast<const bf16x8*>(wrow + ks * 16);
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        const int rl = w * 8 + rr;
        u16x8 hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float v = acc[rr][j];
            hi[j] = f32_to_bf16_bits(v);
            lo[j] = f32_to_bf16_bits(v - bf16_bits_to_f32(hi[j]));
        }
        const int off = rl * 1024 + ((lane ^ (rl & 7)) << 4);   // chunk = lane (8 cols)
        *reinterpret_cast<u16x8*>(&ol[0][off]) = hi;
        *reinterpret_cast<u16x8*>(&ol[1][off]) = lo;
    }
    __syncthreads();

    f32x16 oacc = {};
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
        const int ch = 2 * ks + hf;
        const int off = l32 * 1024 + ((ch ^ (l32 & 7)) << 4);
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&ol[0][off]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&ol[1][off]);
        oacc = mfma32(wa[ks], bh, oacc);
        oacc = mfma32(wa[ks], bl, oacc);
    }
    // out rows (32 rows x 128 values of head h) through LDS, so that each
    // row's 256-byte segment is one contiguous store (a lane holds 8-byte
    // pieces of 32 different rows)
    constexpr int OROWB = 272;                  // bytes per staged output row
    __syncthreads();                            // every wave is done reading o_lat
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const unsigned long long pk =
            (unsigned long long)f32_to_bf16_bits(oacc[4 * g + 0]) |
            ((unsigned long long)f32_to_bf16_bits(oacc[4 * g + 1]) << 16) |
            ((unsigned long long)f32_to_bf16_bits(oacc[4 * g + 2]) << 32) |
            ((unsigned long long)f32_to_bf16_bits(oacc[4 * g + 3]) << 48);
        *reinterpret_cast<unsigned long long*>(&ol[0][l32 * OROWB + (w * 32 + 8 * g + 4 * hf) * 2]) = pk;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {               // 32 rows x 16 chunks, 2 per thread
        const int i = k * 256 + tid, rl = i >> 4, c = i & 15;
        const int r = rb * 32 + rl;
        if (r < R)
            *reinterpret_cast<u32x4*>(out + ((size_t)r * H + h) * 128 + c * 8) =
                *reinterpret_cast<const u32x4*>(&ol[0][rl * OROWB + c * 16]);
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
        // balanced scheduling: one workgroup per compute unit
        const int grid = a.num_splits > 0 ? R * a.num_splits : kNumCUs;
        const float scale_log2 = a.scale * kLog2e;
        if (a.cache_dtype == MLA_FP8_E4M3 && a.fp8_scores) {
            split_kv_kernel<true, true><<<grid, 256, 0, a.stream>>>(
                qbuf, static_cast<const unsigned char*>(a.pool), a.pool_scale, a.block_table,
                a.max_blocks, a.seq_lens, R, a.q_len, a.num_splits, scale_log2,
                static_cast<unsigned short*>(a.part_o), a.part_lse);
        } else if (a.cache_dtype == MLA_FP8_E4M3) {
            split_kv_kernel<true><<<grid, 256, 0, a.stream>>>(
                qbuf, static_cast<const unsigned char*>(a.pool), a.pool_scale, a.block_table,
                a.max_blocks, a.seq_lens, R, a.q_len, a.num_splits, scale_log2,
                static_cast<unsigned short*>(a.part_o), a.part_lse);
        } else {
            split_kv_kernel<false><<<grid, 256, 0, a.stream>>>(
                qbuf, static_cast<const unsigned char*>(a.pool), nullptr, a.block_table,
                a.max_blocks, a.seq_lens, R, a.q_len, a.num_splits, scale_log2,
                static_cast<unsigned short*>(a.part_o), a.part_lse);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (stages & MLA_STAGE_COMBINE) {
        const int grid = H * ((R + 31) / 32);
        combine_kernel<<<grid, 256, 0, a.stream>>>(static_cast<const unsigned short*>(a.part_o),
                                                   a.part_lse, a.seq_lens, a.q_len, R, a.num_splits,
                                                   kNumCUs,
                                                   static_cast<const unsigned short*>(a.w_uv),
                                                   static_cast<unsigned short*>(a.out), a.lse);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mla

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

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"
#include "append_finalize.hpp"

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

// Calls f(std::integral_constant<int, I>) for I = B .. E-1 in order: a loop
// whose index is a compile-time constant in every copy of the body.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// ---------------------------------------------------------------------------
// 1. q absorption
// ---------------------------------------------------------------------------

// The absorbed queries [q_lat ; q_pe] (576 bf16 per row and head) are stored
// in the order the split-KV kernels load them as MFMA B fragments: wave w of
// a workgroup holds heads 32 w .. 32 w + 31, and its K-step ks (channels
// 16 ks .. +16) is 64 lanes x 8 channels, lane hf * 32 + (head % 32) taking
// channels 16 ks + 8 hf .. +8.  So each fragment load is one contiguous
// 1 KB read.  Element offset of 8 channels c .. c + 7 (c a multiple of 8) of
// row r, head h:
__device__ __forceinline__ size_t q_frag_offset(int r, int h, int c) {
    return (((size_t)r * 4 + (h >> 5)) * 36 + (c >> 4)) * 512 + (((c >> 3) & 1) * 32 + (h & 31)) * 8;
}
static_assert(H == 128 && D == 576, "q_frag_offset assumes 4 head groups of 32 and 36 K-steps");

// grid: H * 4 * ceil(R / 64) workgroups of 256 threads.  Workgroup (h, cb, rb)
// produces q_lat[rb*64 .. +64][h][cb*128 .. +128]: q_lat^T = W_UK[h]^T q_nope^T
// with W_UK[h][:, cb*128 .. +128] staged in LDS as [n][col] rows of 288 bytes
// (256 + 32 of padding).  The MFMA A operand (32 latent columns x 16 n) is
// read with the transposing ds_read_b64_tr_b16: a 16-lane group reads 4 rows
// x 16 columns and each lane receives one column's 4 values; the padding puts
// the 4 rows of a group on disjoint banks.
constexpr int WT_ROWB = 288;    // bytes per staged W_UK row
// bytes per staged q_nope row (256 + 16): the 16-byte B-operand reads of 16
// consecutive rows start 68 dwords apart and cover all 64 banks
constexpr int QT_ROWB = 272;

__device__ __forceinline__ void absorb_q_block(
    int bid,                                    // workgroup of the grid above
    const unsigned short* __restrict__ q_nope,  // [R][H][128]
    const unsigned short* __restrict__ q_pe,    // [R][H][64]
    const unsigned short* __restrict__ w_uk,    // [H][128][512]
    unsigned short* __restrict__ qbuf,          // [R][H][576], fragment order (q_frag_offset)
    int R) {
    __shared__ __attribute__((aligned(16))) unsigned char wt[128 * WT_ROWB];
    __shared__ __attribute__((aligned(16))) unsigned char qt[64 * QT_ROWB];
    // head h = 16 (bid % 8) + (bid / 8) % 16: workgroup ids that share bid % 8
    // run on one XCD, so each XCD produces 16 consecutive heads, and the 128-byte
    // lines of the fragment-ordered query buffer (8 heads each) are filled
    // within one L2 rather than written in 16-byte pieces from eight
    static_assert(H == 128, "eight XCDs x 16 heads");
    const int h = (bid & 7) * 16 + ((bid >> 3) & 15);
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
    // q_nope of the 64 rows for head h: 64 rows x 16 chunks of 16 B, 4 per
    // thread (16 consecutive threads read one row's 256 bytes), at clamped
    // rows; staged in LDS for the MFMA B operands
    u32x4 qv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = k * 256 + tid, r = min(rb * 64 + (i >> 4), R - 1), c = i & 15;
        qv[k] = *reinterpret_cast<const u32x4*>(q_nope + ((size_t)r * H + h) * 128 + c * 8);
    }
    // q_pe rides along in the workgroups of column block 0: 64 rows x 8
    // chunks of 16 bytes, two per thread, loaded here with everything else
    // (unconditionally, at clamped rows) and stored at the end
    u32x4 pe[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int i = k * 256 + tid, r = min(rb * 64 + (i >> 3), R - 1), c8 = i & 7;
        pe[k] = *reinterpret_cast<const u32x4*>(q_pe + ((size_t)r * H + h) * DR + c8 * 8);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int i = k * 256 + tid, n = i >> 4, c = i & 15;
        *reinterpret_cast<u32x4*>(wt + n * WT_ROWB + c * 16) = wv[k];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = k * 256 + tid, rl = i >> 4, c = i & 15;
        *reinterpret_cast<u32x4*>(qt + rl * QT_ROWB + c * 16) = qv[k];
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
        for (int nb = 0; nb < 2; ++nb) {
            // B operand: row nb*32 + l32, n = 16 ks + 8 hf .. +8
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(qt + (nb * 32 + l32) * QT_ROWB + (ks * 16 + hf * 8) * 2);
            acc[nb] = mfma32(a, b, acc[nb]);
        }
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
            *reinterpret_cast<u32x4*>(qbuf + q_frag_offset(r, h, cb * 128 + c * 8)) =
                *reinterpret_cast<const u32x4*>(wt + rl * OROWB + c * 16);
    }
    if (cb == 0) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int i = k * 256 + tid, r = rb * 64 + (i >> 3), c8 = i & 7;
            if (r < R) *reinterpret_cast<u32x4*>(qbuf + q_frag_offset(r, h, DC + c8 * 8)) = pe[k];
        }
    }
}

__global__ __launch_bounds__(256) void absorb_q_kernel(const unsigned short* __restrict__ q_nope,
                                                      const unsigned short* __restrict__ q_pe,
                                                      const unsigned short* __restrict__ w_uk,
                                                      unsigned short* __restrict__ qbuf, int R) {
    absorb_q_block(blockIdx.x, q_nope, q_pe, w_uk, qbuf, R);
}

// The cache append's finalize (workgroups 0 .. T-1, one token each) and the
// query absorption (the rest) in one launch: they do not depend on each
// other, and the finalize's 64-odd latency-bound workgroups then run beside
// the absorption's bandwidth-bound ones instead of after them.
struct FinalizeArgs {
    const float* part;
    int kc, T, DC, DR;
    const void* gamma;
    float eps, rope_base;
    const int* block_table;
    int max_blocks;
    const int* start_pos;
    int n_new, BSZ;
    void* pool;
    float* pool_scale;
};
template <int CDT>
__global__ __launch_bounds__(256) void finalize_absorb_kernel(FinalizeArgs f,
                                                              const unsigned short* __restrict__ q_nope,
                                                              const unsigned short* __restrict__ q_pe,
                                                              const unsigned short* __restrict__ w_uk,
                                                              unsigned short* __restrict__ qbuf, int R) {
    if ((int)blockIdx.x < f.T)
        append_finalize_token<MLA_BF16, CDT>(blockIdx.x, f.part, f.kc, f.T, f.DC, f.DR, f.gamma, f.eps,
                                             f.rope_base, f.block_table, f.max_blocks, f.start_pos,
                                             f.n_new, f.BSZ, f.pool, f.pool_scale);
    else
        absorb_q_block(blockIdx.x - f.T, q_nope, q_pe, w_uk, qbuf, R);
}

// ---------------------------------------------------------------------------
// 2. split-KV attention over the latent cache
// ---------------------------------------------------------------------------

// LDS-typed byte pointer.  Tile helpers take these so that the compiler's
// alias analysis can tell the tile being read from the one being filled.
typedef MLA_LDS unsigned char lds_u8;

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
//  - num_splits == 0 (balanced): the tiles are cut into G equal ranges over
//    "entries" concatenated in order.  With 1 < q_len <= kPairQ an entry is a
//    sequence (Qs = q_len rows sharing its tiles, tiles(entry) = tiles of its
//    last row); otherwise an entry is a query row (Qs = 1).  Range g =
//    [g T / G, (g+1) T / G) of the T entry tiles is walked by Qs workgroups,
//    one per row s of each entry, on one XCD at the same time, so that the
//    rows of a sequence read each tile from HBM about once.  The piece of
//    (range g, entry e, row s) writes partial slot Qs (g + e) + s; a piece
//    whose row sees none of the range's tiles writes log-sum-exp -inf there.
//    Slots are unique: for g < g' the entries of g end no later than those of
//    g' begin, so g + e < g' + e'.  Row (e, s)'s pieces occupy slots
//    Qs (f + e) + s, Qs (f + 1 + e) + s, .. Qs (l + e) + s, f / l being the
//    ranges holding its entry's first / last tile; all below kNumCUs + R.

// Tiles seen by row s of a sequence of len tokens (q_len query rows).
__device__ __forceinline__ int tiles_from_len(int len, int q_len, int s) {
    const int n_vis = len - q_len + s + 1;
    return n_vis > 0 ? (n_vis + BS - 1) / BS : 0;
}
__device__ __forceinline__ int row_tiles(const int* __restrict__ seq_lens, int q_len, int r) {
    const int b = r / q_len;
    return tiles_from_len(seq_lens[b], q_len, r - b * q_len);
}

// Workgroups of the balanced schedule for T tiles: at most one per compute
// unit (the grid), and at least kMinGroupTiles tiles each.  One tile per
// workgroup is the fastest choice measured for a single 4096-token row (64
// workgroups: 24-27 us against 31 us with 16 workgroups of 4 tiles): spreading
// the tiles outweighs each workgroup's fixed costs (query load, partial write,
// one more partial to merge).
constexpr int kMinGroupTiles = 1;
// Largest q_len whose rows share tile ranges (sequence entries).
constexpr int kPairQ = 8;
static_assert(kNumCUs % 8 == 0 && kNumCUs / 8 >= kPairQ, "every XCD runs at least one range's rows");
__device__ __forceinline__ int sched_qs(int q_len) { return q_len <= kPairQ ? q_len : 1; }
// Tiles of entry e, and the query row of its row s.
__device__ __forceinline__ int entry_tiles(const int* __restrict__ seq_lens, int q_len, int e) {
    return q_len <= kPairQ ? row_tiles(seq_lens, q_len, e * q_len + q_len - 1) : row_tiles(seq_lens, q_len, e);
}
__device__ __forceinline__ int entry_row(int q_len, int e, int s) { return q_len <= kPairQ ? e * q_len + s : e; }
// Sequence of entry e, and the row (within its sequence) whose tiles are the entry's.
__device__ __forceinline__ int entry_seq(int q_len, int e) { return q_len <= kPairQ ? e : e / q_len; }
__device__ __forceinline__ int entry_last_s(int q_len, int e) { return q_len <= kPairQ ? q_len - 1 : e % q_len; }
// Ranges for T entry tiles on `grid` workgroups (a multiple of the 8 XCDs):
// each XCD runs ceil(G / 8) ranges x Qs rows, at most grid / 8 workgroups.
__device__ __forceinline__ long long balanced_groups(long long grid, long long T, int Qs) {
    return min(8 * ((grid / 8) / Qs), (T + kMinGroupTiles - 1) / kMinGroupTiles);
}


// Workgroup holding tile t of the concatenated tiles (T tiles over G groups).
__device__ __forceinline__ int group_of_tile(long long t, long long T, long long G) {
    return (int)(((t + 1) * G + T - 1) / T - 1);
}

// Block-wide scan of entry tile counts: thread tid owns entries [tid*per,
// tid*per+per) (per = ceil(E / 256)).  Returns T; *excl / *mine receive the
// tiles before this thread's entries and in them, *len0 the sequence length
// of its first entry (when it has one).  sc: 260 ints of LDS scratch.
template <typename LdsInt>
__device__ __forceinline__ int scan_entry_tiles(const int* __restrict__ seq_lens, int q_len, int E,
                                                LdsInt sc, int* excl, int* mine, int* len0) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int per = (E + 255) / 256;
    int local = 0;
    *len0 = 0;
    for (int k = 0; k < per; ++k) {
        const int e = tid * per + k;
        if (e < E) {
            const int len = seq_lens[entry_seq(q_len, e)];
            if (k == 0) *len0 = len;
            local += tiles_from_len(len, q_len, entry_last_s(q_len, e));
        }
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

// One workgroup's walk of the balanced schedule (workgroups of 256 threads).
// Workgroup id b runs on XCD b % 8; the XCD's ceil(G / 8) consecutive ranges
// go to its workgroups in order, Qs per range (row s = (b / 8) % Qs), so the
// rows of one range run side by side and consecutive ranges (a long row's
// pieces) share an L2.
struct BalancedWalk {
    int grp, s, rng_a, rng_b, cur_e, cur_es;
    int len_e, len;                      // sequence length of entry len_e, known from the scan
};
// Sets up the walk; false: this workgroup has nothing to do (uniform).
template <typename LdsInt>
__device__ __forceinline__ bool balanced_start(const int* __restrict__ seq_lens, int q_len, int R,
                                               LdsInt sc, BalancedWalk& wk) {
    const int tid = threadIdx.x;
    const int Qs = sched_qs(q_len), E = R / Qs;
    int excl, mine, len0;
    const int T = scan_entry_tiles(seq_lens, q_len, E, sc, &excl, &mine, &len0);
    const long long G = balanced_groups(gridDim.x, T, Qs);
    const int per = (int)((G + 7) / 8);
    const int bx = blockIdx.x & 7, bk = blockIdx.x >> 3;
    const int g = bk < per * Qs ? bx * per + bk / Qs : (int)G;
    if ((long long)g >= G) return false;
    wk.grp = g;
    wk.s = bk % Qs;
    wk.rng_a = (int)((long long)g * T / G);
    wk.rng_b = (int)((long long)(g + 1) * T / G);
    wk.cur_e = 0;
    wk.cur_es = 0;
    wk.len_e = -1;
    wk.len = 0;
    if (wk.rng_a < wk.rng_b && excl <= wk.rng_a && wk.rng_a < excl + mine) {
        // this thread's entries hold the range's first tile; with one entry
        // per thread (E <= 256) its tiles and length came with the scan
        const int pe = (E + 255) / 256;
        int es = excl;
        for (int k = 0; k < pe; ++k) {
            const int e = tid * pe + k;
            const int len = pe == 1 ? len0 : e < E ? seq_lens[entry_seq(q_len, e)] : 0;
            const int nt = pe == 1 ? mine : e < E ? tiles_from_len(len, q_len, entry_last_s(q_len, e)) : 0;
            if (wk.rng_a < es + nt) {
                sc[260] = e;
                sc[261] = es;
                sc[262] = len;
                break;
            }
            es += nt;
        }
    }
    __syncthreads();
    if (wk.rng_a < wk.rng_b) {
        wk.cur_e = sc[260];
        wk.cur_es = sc[261];
        wk.len_e = wk.cur_e;
        wk.len = sc[262];
    }
    __syncthreads();                     // scratch read before the caller reuses it
    return true;
}
// The walk's next piece (row, tiles [t0, t1), slot, and len, the length of
// the row's sequence); false when done.  A row that sees none of a range's
// tiles gets log-sum-exp -inf in its slot.
__device__ __forceinline__ bool balanced_next(BalancedWalk& wk, const int* __restrict__ seq_lens, int q_len,
                                              int R, float* __restrict__ part_lse, int& row, int& t0,
                                              int& t1, int& slot, int& len) {
    const int Qs = sched_qs(q_len), E = R / Qs;
    while (wk.cur_es < wk.rng_b && wk.cur_e < E) {
        const int e = wk.cur_e, es = wk.cur_es;
        len = e == wk.len_e ? wk.len : seq_lens[entry_seq(q_len, e)];
        const int nt = tiles_from_len(len, q_len, entry_last_s(q_len, e));
        wk.cur_e += 1;
        wk.cur_es += nt;
        const int lo = max(wk.rng_a, es) - es, hi = min(wk.rng_b, es + nt) - es;
        if (hi > lo) {
            row = entry_row(q_len, e, wk.s);
            slot = Qs * (wk.grp + e) + wk.s;
            t0 = lo;
            t1 = min(hi, tiles_from_len(len, q_len, row - (row / q_len) * q_len));
            if (t0 < t1) return true;
            if (threadIdx.x < H) part_lse[(size_t)slot * H + threadIdx.x] = kNegInf;
        }
    }
    return false;
}

template <bool FP8>
__global__ __launch_bounds__(256, 1) void split_kv_kernel(
    const unsigned short* __restrict__ qbuf,      // [R][H][576] bf16, fragment order (q_frag_offset)
    const unsigned char* __restrict__ pool,       // [blocks][64][576] bf16 | fp8
    const float* __restrict__ pool_scale,         // [blocks][64] (fp8)
    const int* __restrict__ block_table, int max_blocks,
    const int* __restrict__ seq_lens, int R, int q_len, int num_splits, float scale_log2,
    unsigned short* __restrict__ part_o,          // [slots][H][512] fp16
    float* __restrict__ part_lse) {               // [slots][H]
    // Only the fp8 cache runs here (a bf16 cache runs on split_kv_ring_kernel).
    static_assert(FP8, "split_kv_kernel serves the fp8 cache");
    // one bf16 tile + two fp8 staging tiles with scales; the queries (rotary
    // part included) stay in VGPRs
    constexpr int STAGE = F8TILE + 256;                     // fp8 staging buffer: codes + scales
    constexpr int LDS_BYTES = TILE + 2 * STAGE;
    constexpr int NQ = 36;                                  // bf16 query K-steps kept in VGPRs
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[LDS_BYTES];
    lds_u8* smem = (lds_u8*)smem_raw;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, in an SGPR
    const int l32 = lane & 31, hf = lane >> 5;
    const int head = w * 32 + l32;

    // ---- this workgroup's pieces (row, tiles [t0, t1), partial slot) ---------------
    BalancedWalk wk{};
    bool fixed_pending = num_splits > 0;
    if (num_splits == 0 && !balanced_start(seq_lens, q_len, R, reinterpret_cast<MLA_LDS int*>(smem), wk))
        return;                          // uniform: the whole workgroup leaves
    auto next_piece = [&](int& row, int& t0, int& t1, int& slot, int& len) -> bool {
        if (num_splits > 0) {
            if (!fixed_pending) return false;
            fixed_pending = false;
            row = blockIdx.x / num_splits;
            const int split = blockIdx.x - row * num_splits;
            len = seq_lens[row / q_len];
            const int n_tiles = tiles_from_len(len, q_len, row - (row / q_len) * q_len);
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
        return balanced_next(wk, seq_lens, q_len, R, part_lse, row, t0, t1, slot, len);
    };

    int row, t0, t1, slot, seq_len;
    for (int piece = 0; next_piece(row, t0, t1, slot, seq_len); ++piece) {
        if (piece > 0) __syncthreads();      // the previous piece's epilogue is done with LDS
        const int b = row / q_len, s = row - b * q_len;
        const int n_vis = seq_len - q_len + s + 1;
        float* lse_dst = part_lse + (size_t)slot * H;
        const int* btab = block_table + (size_t)b * max_blocks;

        // the bf16 tile at 0, staging buffers at TILE and TILE + STAGE

        auto valid_of = [&](int t) { return min(BS, n_vis - t * BS); };
        // asynchronous load of tile t into the fp8 staging buffer `dst`
        auto issue = [&](int t, lds_u8* dst) {
            const size_t blk = (size_t)btab[t];
            issue_tile_fp8(pool + blk * F8TILE, pool_scale + blk * BS, dst, w, lane);
        };
        // The first tile's copy goes out before the query loads, so that the two
        // memory round trips of a piece's start overlap.
        issue(t0, smem + TILE);
        bool t0_in_flight = true;

        // this wave's 32 query rows, as MFMA B fragments: lane (hf, l32) holds
        // channels 16 ks + 8 hf .. +8 of head 32 w + l32 (one 1 KB read per
        // K-step, q_frag_offset)
        bf16x8 qf[NQ];
        {
            const unsigned short* qrow = qbuf + q_frag_offset(row, 32 * w, 0) + lane * 8;
#pragma unroll
            for (int ks = 0; ks < NQ; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 512);
        }


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
            const int valid = valid_of(t);
            if (has_next) issue(t + 1, nxt);
#pragma unroll 1
            for (int hb = 0; hb < 2; ++hb) {
                if (hb * 32 >= valid) break;
                // ---- S^T = K . Q^T: rows 32 hb + l32 -----------------------------------
                const lds_u8* kbase = tile + hb * 32 * 128;
                auto ka = [&](int ks) {
                    return *reinterpret_cast<const MLA_LDS bf16x8*>(kbase + qk_off[ks & 3] + (ks >> 2) * 8192);
                };
                auto qb = [&](int ks) -> bf16x8 { return qf[ks]; };
                f32x16 sacc = {};
                float sv[16];
                // fp8: token scales of the lane's rows 32 hb + 8 (i/4) + 4 hf + (i%4)
                // (zero past the sequence end), applied to the scores and folded
                // into the weights, so that keys and values enter the products as
                // the codes' exact values
                float tsc[16];
                {
                    const MLA_LDS float* lsc =
                        reinterpret_cast<const MLA_LDS float*>(stg + F8TILE);
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 ks4 = *reinterpret_cast<const MLA_LDS f32x4*>(lsc + hb * 32 + 8 * g + 4 * hf);
#pragma unroll
                        for (int j = 0; j < 4; ++j) tsc[4 * g + j] = ks4[j];
                    }
                }
                {
                    bf16x8 a0 = ka(0), a1 = ka(1), a2;
#pragma unroll
                    for (int ks = 0; ks < 36; ++ks) {
                        if (ks + 2 < 36) a2 = ka(ks + 2);
                        sacc = mfma32(a0, qb(ks), sacc);
                        a0 = a1;
                        a1 = a2;
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) sv[i] = sacc[i] * tsc[i];
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
                        pu[j] = f32_to_bf16_bits(pv * tsc[k2 * 8 + j]);
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
            if (!t0_in_flight) issue(t0, smem + TILE);   // a later pass
            t0_in_flight = false;
            for (int t = t0; t < t1; ++t) {
                const int cur = (t - t0) & 1;
                wait_vmem_all();
                __syncthreads();             // tile t landed; previous tile fully consumed
                const bool has_next = t + 1 < t1;
                lds_u8* st_cur = smem + TILE + cur * STAGE;
                lds_u8* st_nxt = smem + TILE + (cur ^ 1) * STAGE;
                convert_tile_fp8(st_cur, smem, tid, valid_of(t));
                __syncthreads();
                run_tile(t, smem, st_nxt, st_cur, has_next);
            }
            // ---- vote: did any wave's weights run past the reference? ------------------
            wait_vmem_all();
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
// 2b. split-KV over a bf16 cache: half-tile ring, software-pipelined
// ---------------------------------------------------------------------------
//
// Same work partition, partial slots and results as split_kv_kernel, for a
// bf16 cache.  The cache streams through a ring of four 32-row half-tiles
// (4 x 36 KiB); the last 16 KiB of LDS pass softmax weights between waves.
//
// Two products per half-tile, split differently over the four waves:
//  - scores: wave w owns heads 32w .. 32w+31 (its queries stay in VGPRs):
//      S^T (32 tokens x 32 heads) = K_half (32 x 576) . Q_w^T      36 MFMA
//    and forms those heads' softmax weights P;
//  - values: wave w owns latent columns 128w .. 128w+127 of all 128 heads:
//      O^T (128 cols x 128 heads) += V^T (128 x 32) . P^T          32 MFMA
//    with every head block's weights read from LDS.  Each value fragment
//    then feeds four MFMAs (one per head block).
// The cache's blocks are token-major (1152-byte rows) and a half-tile stays
// token-major in LDS, so the score operand -- 8 channels of one token -- is
// one 16-byte LDS read, and the value operand -- 8 consecutive tokens of one
// latent channel -- comes from two transposing 8-byte reads.
// Loop iteration h (half h of the piece) runs, per wave:
//   S_{h+1} (36 MFMA, with the copy of half h+3: 9 instructions)
//   V_h     (32 MFMA, with the softmax of S_{h+1} threaded between them;
//            its weights go to LDS for iteration h+1)
// Every LDS operand is read well ahead of its use (four MFMAs for the score
// operands): with a shorter lead an LDS-fed 32x32x16 MFMA waits for its
// operand.  A scheduling barrier after every MFMA slot keeps this order;
// left alone, the compiler moves each read next to its use and gathers the
// vector work between the chains.  One barrier per half: half h+1 has landed
// (each wave waits for its own copies, the barrier for the others'), the
// weights P_h are in LDS, and every wave is done with half h-1, whose slot
// the copy of h+3 reuses, and with the weights of h-1, whose buffer P_{h+1}
// reuses.
constexpr int HROWS = 32;                 // tokens per half-tile (= the cache's sub-block)
constexpr int HALF = HROWS * ROWB;        // 36864 bytes
constexpr int NRING = 4;                  // ring slots
constexpr int PBUF = 4 * 2 * 1024;        // weights of one half: 4 head blocks x 2 K-steps x 1 KB
static_assert(HALF == 36 * 1024 && BS == 2 * HROWS, "a half-tile is 36 copies of 1 KB, half a block");

// Half-tile layout in LDS.  Token t's row (1152 bytes: 9 groups of 128
// bytes, 8 chunks of 8 channels each) sits at t * 1152, as in memory, with
// the chunks of every group permuted: logical chunk x of a group at 16-byte
// position x ^ tswz(t), tswz(t) = bit1(t) << 2 | bits 2..3 of t.  Rows are
// 4.5 x 256 bytes apart, so a row's bank offset is 128 (t & 1), and tswz
// separates the rest:
//  - score operand (16-byte reads of one chunk of 16 aligned rows): over
//    the 8 even or the 8 odd rows, tswz takes each of its 8 values once;
//  - value operand (transposing 8-byte reads, 32 lanes: 4 aligned rows x
//    4 aligned chunks): of the two even (odd) rows, tswz differs in bit 2,
//    so they fall on the two different 4-chunk halves of the group.
__device__ __forceinline__ int tswz(int t) { return (((t >> 1) & 1) << 2) | ((t >> 2) & 3); }

// Copy instruction k (0..8) of wave w for one half-tile: instruction
// i = 9 w + k moves bytes 1024 i .. +1024 of the half into the same bytes of
// the slot.  Lanes 8 j .. 8 j + 7 fill 128-byte group G = 8 i + j, i.e.
// group G % 9 of token G / 9 = 8 w + (8 k + j) / 9, and lane 8 j + p fills
// position p with logical chunk p ^ tswz(token).  copy_swizzles packs the 9
// tswz values of a lane (3 bits each, instruction k at bit 3 k).
__device__ __forceinline__ unsigned copy_swizzles(int w, int lane) {
    unsigned packed = 0;
#pragma unroll
    for (int k = 0; k < 9; ++k) packed |= (unsigned)tswz(8 * w + (8 * k + (lane >> 3)) / 9) << (3 * k);
    return packed;
}
__device__ __forceinline__ void issue_half_part(__amdgpu_buffer_rsrc_t rsrc, lds_u8* slot, int w,
                                                int lane, unsigned swz, int k) {
    const int i = w * 9 + k;
    const unsigned off = ((lane >> 3) << 7) + ((((unsigned)lane ^ (swz >> (3 * k))) & 7) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (MLA_LDS void*)(slot + i * 1024), 16, off, i * 1024,
                                             0, 0);
}

// Zero the latent channels (the first 1024 bytes of the row, whatever the
// chunk order) of tokens valid .. 31 of a half-tile slot: their cache slots
// hold no token, and the value product must not meet NaN there.
__device__ __forceinline__ void zero_half_tokens(lds_u8* slot, int valid, int tid) {
    for (int p = valid * 64 + tid; p < HROWS * 64; p += 256)
        *reinterpret_cast<MLA_LDS u16x8*>(slot + (p >> 6) * ROWB + (p & 63) * 16) = u16x8{};
}

// Workgroup barrier after this wave's vector memory operations up to the 9
// (18) most recent have completed, and its LDS operations.  __syncthreads()
// would wait for every copy in flight (its fence drains the whole vector
// memory counter).  The asm's memory clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void barrier_landed_but_9() {
    asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void barrier_landed_but_18() {
    asm volatile("s_waitcnt vmcnt(18) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Workgroup barrier after this wave's LDS operations (vector memory copies
// may stay in flight).
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Phase timers of the split-KV ring kernel, compiled only into the
// instrumented build (-DMLA_PHASE_STAMPS, libmla_phases.so; include/mla_debug.h).
// Each wave keeps lap timers in shader cycles (s_memtime): lap k adds the
// cycles since the previous lap, so the laps of a wave sum to its whole run.
// Laps: 0 / 1 / 2 the steady-state half-tiles' barrier wait, score chain and
// value chain (with the softmax threaded in); 8 kernel start (or the previous
// piece's end) to the piece's start (the schedule walk); 9 to the first
// half-tile landed (block table, queries, first copies); 10 the first half's
// scores and softmax; 12 the piece's last two half-tiles and the final value
// chain; 13 the vote (and any repeated pass); 14 the epilogue (partial o_lat
// and lse written).  Word 3 counts steady-state half-tiles, 4 the wave's
// cycles, 5 its pieces, 6 / 7 the low 32 bits of s_memrealtime (100 MHz) at
// its start and end.  Wave w of workgroup b < kNumCUs writes words
// 64 b + 16 w .. +16 of g_phase_stamps at its end.
#ifdef MLA_PHASE_STAMPS
constexpr int kPhaseWords = kNumCUs * 4 * 16;
}  // namespace
// (external linkage, so that the runtime finds the symbol by name)
__device__ unsigned g_phase_stamps[kPhaseWords];
namespace {
#define MLA_LAP(k)                                                                  \
    do {                                                                            \
        const unsigned long long t_ = __builtin_readcyclecounter();                 \
        ph_[k] += (unsigned)(t_ - ph_last_);                                        \
        ph_last_ = t_;                                                              \
    } while (0)
#define MLA_PHASE_COUNT(k) (++ph_[k])
#else
#define MLA_LAP(k) \
    do {           \
    } while (0)
#define MLA_PHASE_COUNT(k) \
    do {                   \
    } while (0)
#endif

__global__ __launch_bounds__(256, 1) void split_kv_ring_kernel(
    const unsigned short* __restrict__ qbuf,      // [R][H][576] bf16, fragment order (q_frag_offset)
    const unsigned char* __restrict__ pool,       // [blocks][64][576] bf16
    const int* __restrict__ block_table, int max_blocks,
    const int* __restrict__ seq_lens, int R, int q_len, int num_splits, float scale_log2,
    unsigned short* __restrict__ part_o,          // [slots][H][512] fp16
    float* __restrict__ part_lse) {               // [slots][H]
    constexpr int P_OFF = NRING * HALF;
    constexpr int LDS_BYTES = P_OFF + 2 * PBUF;           // 160 KiB
    constexpr int DIST = 4;                               // score operand lead, in MFMAs
    constexpr int NS = 36, NV = 32;                       // score / value MFMAs per half
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[LDS_BYTES];
    lds_u8* smem = (lds_u8*)smem_raw;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, in an SGPR
    const int l32 = lane & 31, hf = lane >> 5;
    const int head = w * 32 + l32;
    const unsigned cswz = copy_swizzles(w, lane);   // this lane's copy swizzles
#ifdef MLA_PHASE_STAMPS
    unsigned ph_[16] = {};
    const unsigned long long ph_start_ = __builtin_readcyclecounter();
    const unsigned long long ph_rt0_ = __builtin_amdgcn_s_memrealtime();
    unsigned long long ph_last_ = ph_start_;
#endif

    // ---- this workgroup's pieces: as in split_kv_kernel ----------------------------
    BalancedWalk wk{};
    bool fixed_pending = num_splits > 0;
    if (num_splits == 0 && !balanced_start(seq_lens, q_len, R, reinterpret_cast<MLA_LDS int*>(smem), wk))
        return;                          // uniform: the whole workgroup leaves
    auto next_piece = [&](int& row, int& t0, int& t1, int& slot, int& len) -> bool {
        if (num_splits > 0) {
            if (!fixed_pending) return false;
            fixed_pending = false;
            row = blockIdx.x / num_splits;
            const int split = blockIdx.x - row * num_splits;
            len = seq_lens[row / q_len];
            const int n_tiles = tiles_from_len(len, q_len, row - (row / q_len) * q_len);
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
        return balanced_next(wk, seq_lens, q_len, R, part_lse, row, t0, t1, slot, len);
    };

    lds_u8* pbuf = smem + P_OFF;
    int row, t0, t1, pslot, seq_len;
    for (int piece = 0; next_piece(row, t0, t1, pslot, seq_len); ++piece) {
        MLA_LAP(8);
        MLA_PHASE_COUNT(5);
        if (piece > 0) __syncthreads();      // the previous piece's epilogue is done with LDS
        const int b = row / q_len, s = row - b * q_len;
        const int n_vis = seq_len - q_len + s + 1;
        float* lse_dst = part_lse + (size_t)pslot * H;
        const int* btab = block_table + (size_t)b * max_blocks;
        // halves hfirst .. hlast of the row hold the piece's visible tokens;
        // only hlast can be partial
        const int vis_end = min(n_vis, t1 * BS);
        const int hfirst = 2 * t0, hlast = (vis_end - 1) / HROWS;
        auto slot_of = [&](int h) { return smem + ((h - hfirst) & (NRING - 1)) * HALF; };
        // slot and weight-buffer addresses as wave-uniform values, so that the
        // copies' LDS addresses (M0) come from scalar arithmetic
        auto slot_at = [&](int h) __attribute__((always_inline)) {
            return smem + __builtin_amdgcn_readfirstlane((h - hfirst) & (NRING - 1)) * HALF;
        };
        auto pbuf_of = [&](int h) __attribute__((always_inline)) {
            return pbuf + __builtin_amdgcn_readfirstlane((h - hfirst) & 1) * PBUF;
        };
        auto valid_half = [&](int h) { return min(HROWS, vis_end - h * HROWS); };
        // buffer resource of half h; past the last half, one without records
        // (its copies read nothing), so that every iteration issues 9 copies
        auto half_rsrc = [&](int h) {
            const bool real = h <= hlast;
            const size_t blk = (size_t)btab[real ? (h >> 1) : (hlast >> 1)];
            return make_rsrc(pool + blk * GTILE + (h & 1) * HALF, real ? HALF : 0);
        };
        auto issue_half = [&](int h) {
            const __amdgpu_buffer_rsrc_t rs = half_rsrc(h);
#pragma unroll
            for (int k = 0; k < 9; ++k) issue_half_part(rs, slot_of(h), w, lane, cswz, k);
        };
        // A piece's start: this wave's query rows (their addresses need only
        // the row, so they go out while the block table is read), the first
        // half's copy, then the next two halves' copies, so that the first
        // scores wait only for the first two groups of memory operations
        // (vector memory operations complete in order).
        // The query rows, as MFMA B fragments: lane (hf, l32) holds channels
        // 16 ks + 8 hf .. +8 of head 32 w + l32 (latent 0..31, rotary 32..35),
        // one 1 KB read per K-step (q_frag_offset).
        bf16x8 qf[36];
        {
            const unsigned short* qrow = qbuf + q_frag_offset(row, 32 * w, 0) + lane * 8;
#pragma unroll
            for (int ks = 0; ks < 36; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 512);
        }
        issue_half(hfirst);
        issue_half(hfirst + 1);
        issue_half(hfirst + 2);
        bool first_in_flight = true;

        // Per-lane LDS byte offsets.
        // Score operand of K-step ks (channels 16 ks + 8 hf .. +8 of one token
        // per lane): one 16-byte read of chunk 2 ks + hf of token ts = l32
        // with bits 2 and 3 exchanged, i.e. group ks / 4, position
        // (2 (ks % 4)) ^ hf ^ tswz(ts).  So the scores' accumulator row m
        // holds token m with bits 2 and 3 exchanged: lane (hf, l32) ends up
        // with tokens 16 (i/8) + 8 hf + i%8 in sv[i], the order in which the
        // value operand reads them.
        int s_off[4], v_off[2][2];
        {
            const int ts = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 >> 1) & 4);
            const int tau = tswz(ts) ^ hf;
#pragma unroll
            for (int c = 0; c < 4; ++c) s_off[c] = ts * ROWB + (((2 * c) ^ tau) << 4);
        }
        // Value operand: V^T for latent channels 32 cm + l32, K-step k2:
        // tokens 16 k2 + 8 hf .. +8, two transposing reads (tokens +0..3,
        // +4..7).  In 16-lane group g, lane 4 r + b points at token row
        // 16 k2 + 8 (g >> 1) + 4 e + r, channels 32 cm + 16 (g & 1) + 4 b .. +3
        // -- chunk 4 (cm & 1) + 2 (g & 1) + b / 2 of group cm / 2, half b & 1 --
        // and receives channel 32 cm + l32's four tokens.  v_off[cm & 1][e];
        // k2 adds 16 rows, which leaves tswz unchanged.
        {
            const int g = lane >> 4, r = (lane >> 2) & 3, b = lane & 3;
            const int x = 2 * (g & 1) + (b >> 1);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int t = 8 * (g >> 1) + 4 * e + r;
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    v_off[p][e] = t * ROWB + (((4 * p + x) ^ tswz(t)) << 4) + 8 * (b & 1);
            }
        }
        auto k_frag = [&](const lds_u8* sbase, int ks) __attribute__((always_inline)) -> bf16x8 {
            return *reinterpret_cast<const MLA_LDS bf16x8*>(sbase + s_off[ks & 3] + (ks >> 2) * 128);
        };
        auto v_frag = [&](const lds_u8* vbase, int cm, int k2) __attribute__((always_inline)) -> bf16x8 {
            const lds_u8* vb = vbase + (cm >> 1) * 128 + k2 * 16 * ROWB;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(vb + v_off[cm & 1][0]));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(vb + v_off[cm & 1][1]));
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        // weights of head block hb, K-step k2, as the MFMA B operand: 1 KB,
        // lane l at 16 l
        auto p_frag = [&](const lds_u8* pb, int hb, int k2) __attribute__((always_inline)) -> bf16x8 {
            return *reinterpret_cast<const MLA_LDS bf16x8*>(pb + (hb * 2 + k2) * 1024 + lane * 16);
        };

        // Softmax without rescaling the accumulators: every weight of a pass is
        // exp2(s - m_ref) for one reference m_ref per head.  The first pass takes
        // m_ref from the piece's first half-tile; if a later half-tile's maximum
        // exceeds it by more than kMaxLead (weights stay below 2^64, far from
        // fp32 overflow) the pass's result is discarded, one scan computes the
        // exact maximum and a last pass runs with it.  (Scaling O inside the loop
        // would force the 256 accumulators out of AGPRs.)  The waves vote after
        // the loop, in LDS.
        constexpr float kMaxLead = 64.0f;
        // o[4 c + hb]: O^T for latent columns 32 (4 w + c) .. +32 and heads
        // 32 hb .. +32
        f32x16 o[16];
        float m_ref = kNegInf, l_run = 0.f;
        bool overflow = false;
        int mode = 0;                        // 0: first-half reference, 1: max scan, 2: exact reference

        // scores of one half, unscaled, in VGPRs: lane (hf, l32) holds head
        // 32 w + l32, tokens 16 (i/8) + 8 hf + i%8 of the half in sv[i]
        float sv[16];
        bf16x8 pw[2];                        // this wave's weights of a half, per value K-step
        float hmax = kNegInf, psum = 0.f;
        int sv_valid = HROWS;                // rows of the half in sv that hold tokens
        lds_u8* pw_dst = pbuf;               // where the weights of the half in sv go

        // Softmax of the half held in sv as steps k = 0 .. 28, threaded between
        // the MFMAs of another chain.  The instructions of one step do not
        // depend on each other (a step's inputs come from earlier steps, at
        // least one MFMA apart), so each step issues without stalling the
        // wave: value i is scaled at step 8 + i, exponentiated at 9 + i and
        // summed at 10 + i.  MASKED (a partial last half): rows past the
        // sequence end are set to -inf in steps 0-3 and the rest follows four
        // steps later.  SCAN: steps 1-7 only, raising m_ref to the half's
        // maximum.  The weights end in LDS at pw_dst (this wave's head block).
        float mx[6];
        auto softmax_step = [&](auto kc, auto scan_c, auto mask_c) __attribute__((always_inline)) {
            constexpr bool SCAN = decltype(scan_c)::value;
            constexpr bool MASKED = decltype(mask_c)::value;
            constexpr int k = decltype(kc)::value - (MASKED ? 4 : 0);
            if constexpr (MASKED && k < 0) {
                constexpr int g = k + 4;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (16 * (g >> 1) + 4 * (g & 1) + j >= sv_valid - 8 * hf) sv[4 * g + j] = kNegInf;
            }
            if constexpr (k == 1) {
                mx[0] = max3f(sv[0], sv[1], sv[2]);
                mx[1] = max3f(sv[3], sv[4], sv[5]);
            }
            if constexpr (k == 2) {
                mx[2] = max3f(sv[6], sv[7], sv[8]);
                mx[3] = max3f(sv[9], sv[10], sv[11]);
            }
            if constexpr (k == 3) {
                mx[4] = max3f(sv[12], sv[13], sv[14]);
                mx[5] = max3f(sv[15], mx[0], mx[1]);
            }
            if constexpr (k == 4) mx[0] = max3f(mx[2], mx[3], mx[4]);
            if constexpr (k == 5) hmax = max3f(mx[0], mx[5], mx[5]);
            // the log2-domain score is sv * scale_log2 (scale_log2 > 0, so maxima
            // commute with the scaling).  Maxima and sums stay per lane; the two
            // lanes of a head (hf = 0, 1) combine once per pass.
            if constexpr (k == 6) hmax *= scale_log2;
            if constexpr (k == 7) {
                if constexpr (SCAN) {
                    m_ref = fmaxf(m_ref, hmax);
                } else {
                    // (cannot hold in the exact-reference pass: the scan saw the
                    // same maxima, so at most three passes run)
                    overflow |= hmax > m_ref + kMaxLead;
                }
            }
            if constexpr (!SCAN) {
                if constexpr (k >= 8 && k < 24) sv[k - 8] = __builtin_fmaf(sv[k - 8], scale_log2, -m_ref);
                if constexpr (k >= 9 && k < 25) sv[k - 9] = __builtin_amdgcn_exp2f(sv[k - 9]);
                if constexpr (k >= 10 && k < 26) psum += sv[k - 10];
                // weights 4 j .. 4 j + 3 as bf16 into pw (j = 0, 1 at steps 18, 19;
                // j = 2, 3 at steps 25, 26)
                if constexpr (k == 18 || k == 19 || k == 25 || k == 26) {
                    constexpr int j = (k == 18) ? 0 : (k == 19) ? 1 : (k == 25) ? 2 : 3;
                    u32x4 t = __builtin_bit_cast(u32x4, pw[j >> 1]);
                    t[(j & 1) * 2] = pack_bf16x2(sv[4 * j], sv[4 * j + 1]);
                    t[(j & 1) * 2 + 1] = pack_bf16x2(sv[4 * j + 2], sv[4 * j + 3]);
                    pw[j >> 1] = __builtin_bit_cast(bf16x8, t);
                }
                if constexpr (k == 27) {
                    l_run += psum;
                    psum = 0.f;
                }
                if constexpr (k == 28) {
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2)
                        *reinterpret_cast<MLA_LDS bf16x8*>(pw_dst + (w * 2 + k2) * 1024 + lane * 16) = pw[k2];
                }
            }
        };

        // The scores of half h into sv, plain (a piece's first half).
        auto first_scores = [&](int h) __attribute__((always_inline)) {
            const lds_u8* sb = slot_of(h);
            bf16x8 ring[DIST];
            f32x16 sacc = {};
            static_for<0, DIST>([&](auto mc) { ring[decltype(mc)::value] = k_frag(sb, decltype(mc)::value); });
            static_for<0, NS>([&](auto mc) __attribute__((always_inline)) {
                constexpr int m = decltype(mc)::value;
                const bf16x8 a = ring[m % DIST];
                if constexpr (m + DIST < NS) ring[m % DIST] = k_frag(sb, m + DIST);
                sacc = mfma32(a, qf[m], sacc);
                __builtin_amdgcn_sched_barrier(0);
            });
#pragma unroll
            for (int i = 0; i < 16; ++i) sv[i] = sacc[i];
        };
        // The weights of the half in sv, plain (SCAN: m_ref only).
        auto plain_softmax = [&](auto scan_c) __attribute__((always_inline)) {
            if (sv_valid < HROWS) {
                static_for<0, 33>([&](auto kc) { softmax_step(kc, scan_c, std::true_type{}); });
            } else {
                static_for<0, 29>([&](auto kc) { softmax_step(kc, scan_c, std::false_type{}); });
            }
        };

        // V_h: O^T += V^T . P^T for this wave's 4 column blocks and all 4 head
        // blocks.  Slot m = 16 k2 + 4 c + hb; the value fragment of (k2, c) is
        // read one column block ahead; the weights of head block hb, K-step 1
        // replace those of K-step 0 right after their last use (slot 12 + hb),
        // four MFMAs ahead of their first.  The first value fragment and the
        // K-step-0 weights (VPre) are read before the chain starts, inside the
        // score chain when there is one.  Step hook(m) runs after the MFMA of
        // slot m.
        struct VPre {
            bf16x8 va;
            bf16x8 pf[4];
        };
        auto v_prologue = [&](const lds_u8* __restrict__ vb, const lds_u8* __restrict__ pb)
                              __attribute__((always_inline)) {
            VPre p;
            p.va = v_frag(vb, 4 * w, 0);
            static_for<0, 4>([&](auto hc) { p.pf[decltype(hc)::value] = p_frag(pb, decltype(hc)::value, 0); });
            return p;
        };
        auto values_from = [&](const lds_u8* __restrict__ vb, const lds_u8* __restrict__ pb, const VPre& pre,
                               auto hook) __attribute__((always_inline)) {
            bf16x8 va[2], pf[4];
            va[0] = pre.va;
            static_for<0, 4>([&](auto hc) { pf[decltype(hc)::value] = pre.pf[decltype(hc)::value]; });
            static_for<0, NV>([&](auto mc) __attribute__((always_inline)) {
                constexpr int m = decltype(mc)::value;
                // head blocks in the order 1, 2, 3, 0 within a column block: the
                // chain starts away from accumulator 0, whose registers the
                // scores' accumulator borrows during the score chain
                constexpr int c = (m >> 2) & 3, hb = (m + 1) & 3;
                if constexpr ((m & 3) == 0 && m + 4 < NV) {      // next column block's fragment
                    constexpr int kn = (m + 4) >> 4, cn = ((m + 4) >> 2) & 3;
                    va[((m >> 2) + 1) & 1] = v_frag(vb, 4 * w + cn, kn);
                }
                o[4 * c + hb] = mfma32(va[(m >> 2) & 1], pf[hb], o[4 * c + hb]);
                if constexpr (m >= 12 && m < 16) pf[hb] = p_frag(pb, hb, 1);
                hook(std::integral_constant<int, m>{});
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        auto values = [&](const lds_u8* __restrict__ vb, const lds_u8* __restrict__ pb, auto hook)
                          __attribute__((always_inline)) {
            values_from(vb, pb, v_prologue(vb, pb), hook);
        };

        // One pipelined iteration: the scores S_{h+1} (into sv), with the copy
        // of half h+3 spread over them; then, unless SCAN, V_h with the weights
        // of h from LDS.  SOFT: the softmax of S_{h+1} is threaded between the
        // V_h MFMAs, from slot SOFT_LAG on, so that the first value MFMAs issue
        // while the score chain's results drain (a partial S_{h+1}, the piece's
        // last half, takes the plain masked softmax after the iteration
        // instead).  SCAN: scores only.
        constexpr int SOFT_LAG = 2;
        static_assert(28 + SOFT_LAG < NV, "the softmax steps fit in the value chain");
        auto iteration_body = [&](auto scan_c, auto soft_c, int h, const lds_u8* __restrict__ sb,
                                  const lds_u8* __restrict__ vb, lds_u8* __restrict__ cb,
                                  const lds_u8* __restrict__ pb) __attribute__((always_inline)) {
            constexpr bool SCAN = decltype(scan_c)::value;
            constexpr bool SOFT = decltype(soft_c)::value;
            const __amdgpu_buffer_rsrc_t crs = half_rsrc(h + 3);
            bf16x8 ring[DIST];
            f32x16 sacc = {};
            VPre pre;
            sv_valid = valid_half(h + 1);
            static_for<0, DIST>([&](auto mc) { ring[decltype(mc)::value] = k_frag(sb, decltype(mc)::value); });
            static_for<0, NS>([&](auto mc) __attribute__((always_inline)) {
                constexpr int m = decltype(mc)::value;
                const bf16x8 a = ring[m % DIST];
                if constexpr (m + DIST < NS) ring[m % DIST] = k_frag(sb, m + DIST);
                sacc = mfma32(a, qf[m], sacc);
                if constexpr (m % 4 == 0) issue_half_part(crs, cb, w, lane, cswz, m / 4);
                // the value chain's first operands, read while the scores finish
                if constexpr (!SCAN && m == NS - DIST) pre = v_prologue(vb, pb);
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (SOFT) MLA_LAP(1);
            // the scores leave the accumulator (SOFT: after the first value
            // MFMA, which does not wait for them)
            if constexpr (!SOFT) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sv[i] = sacc[i];
            }
            if constexpr (!SCAN) {
                pw_dst = (lds_u8*)pbuf_of(h + 1);
                values_from(vb, pb, pre, [&](auto mc) __attribute__((always_inline)) {
                    constexpr int m = decltype(mc)::value;
                    if constexpr (SOFT && m == 0) {
#pragma unroll
                        for (int i = 0; i < 16; ++i) sv[i] = sacc[i];
                    }
                    if constexpr (SOFT && m >= SOFT_LAG)
                        softmax_step(std::integral_constant<int, m - SOFT_LAG>{}, std::false_type{},
                                     std::false_type{});
                });
            }
        };
        auto iteration = [&](auto scan_c, auto soft_c, int h) __attribute__((always_inline)) {
            iteration_body(scan_c, soft_c, h, slot_at(h + 1), slot_at(h), slot_at(h + 3), pbuf_of(h));
        };
        // wait for half h and for every wave: h is a piece's first half (the
        // two later halves' copies may stay in flight) or the half after the
        // current one (one later half's copies may)
        auto landed = [&](int h, bool first) {
            if (first) barrier_landed_but_18();
            else barrier_landed_but_9();
            if (valid_half(h) < HROWS) {     // the last, partial half of the sequence
                zero_half_tokens((lds_u8*)slot_of(h), valid_half(h), tid);
                __syncthreads();
            }
        };

        for (;;) {
#pragma unroll
            for (int i = 0; i < 16; ++i) o[i] = f32x16{};
            l_run = 0.f;
            overflow = false;
            if (!first_in_flight) {              // a later pass
                issue_half(hfirst);
                issue_half(hfirst + 1);
                issue_half(hfirst + 2);
            }
            first_in_flight = false;
            landed(hfirst, true);
            MLA_LAP(9);
            first_scores(hfirst);
            sv_valid = valid_half(hfirst);
            pw_dst = (lds_u8*)pbuf_of(hfirst);
            if (mode == 0) {
                // the reference: the first half's maximum over both lanes of each
                // head (rows past the sequence end excluded)
                // (token 16 (i/8) + 8 hf + i%8 of the half: a constant against a
                // per-lane limit, so no per-element token index stays live)
                float mx0 = kNegInf;
                const int lim = sv_valid - 8 * hf;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if ((i >> 3) * 16 + (i & 7) < lim) mx0 = fmaxf(mx0, sv[i]);
                mx0 *= scale_log2;
                m_ref = fmaxf(mx0, __shfl_xor(mx0, 32, 64));
            }
            if (mode == 1) {
                plain_softmax(std::true_type{});
                for (int h = hfirst; h < hlast; ++h) {
                    landed(h + 1, false);
                    iteration(std::true_type{}, std::false_type{}, h);
                    plain_softmax(std::true_type{});
                }
            } else {
                plain_softmax(std::false_type{});
                // every half but the last is full: their softmax runs inside the
                // iteration that computes their scores
                MLA_LAP(10);
                for (int h = hfirst; h < hlast - 1; ++h) {
                    landed(h + 1, false);
                    MLA_LAP(0);
                    iteration(std::false_type{}, std::true_type{}, h);
                    MLA_LAP(2);
                    MLA_PHASE_COUNT(3);
                }
                if (hlast > hfirst) {
                    landed(hlast, false);
                    iteration(std::false_type{}, std::false_type{}, hlast - 1);
                    pw_dst = (lds_u8*)pbuf_of(hlast);
                    plain_softmax(std::false_type{});
                }
                barrier_lds();                   // the last half's weights are in LDS
                values(slot_of(hlast), pbuf_of(hlast), [](auto) {});
                MLA_LAP(12);
            }
            // ---- vote: did any wave's weights run past the reference? ------------------
            wait_vmem_all();                 // (record-less copies included)
            __syncthreads();                 // all waves are done with the ring
            MLA_LDS int* votes = reinterpret_cast<MLA_LDS int*>(smem);
            if (lane == 0) votes[w] = __builtin_amdgcn_ballot_w64(overflow) != 0;
            __syncthreads();
            const bool redo = (votes[0] | votes[1] | votes[2] | votes[3]) != 0;
            __syncthreads();                 // votes read before the next pass reuses the ring
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
        MLA_LAP(13);
        l_run += __shfl_xor(l_run, 32, 64);  // the head's two lanes hold disjoint tokens

        // ---- epilogue: normalised partial o_lat (fp16) and log-sum-exp ---------------
        // The partial is a convex combination of latent rows: fp16 keeps it to
        // 2^-11 relative and halves the bytes written (and read by the combine).
        // Wave w holds columns 128w .. 128w+127 of all 128 heads; each head's
        // sum of weights comes from the wave that owns the head's scores,
        // through LDS.  The accumulator layout scatters a lane's values over 32
        // column rows, so each wave transposes through its own LDS region (the
        // ring is free after the vote barrier) and writes 256-byte pieces of the
        // head rows.
        if (hf == 0) reinterpret_cast<MLA_LDS float*>(pbuf)[head] = l_run;
        barrier_lds();
        float inv_l[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) inv_l[hb] = 1.0f / reinterpret_cast<const MLA_LDS float*>(pbuf)[hb * 32 + l32];
        // staging: head row hh (0..127) of this wave at hh * OSTR halves, row
        // stride 136 halves (272 bytes): the 8-byte writes of 16 consecutive
        // lanes (16 head rows) fall on distinct banks
        constexpr int OSTR = 136;
        MLA_LDS unsigned short* ost = reinterpret_cast<MLA_LDS unsigned short*>(smem + w * (128 * OSTR * 2));
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u16x4 hv;
#pragma unroll
                    for (int j = 0; j < 4; ++j) hv[j] = f32_to_f16_bits(o[4 * c + hb][4 * g + j] * inv_l[hb]);
                    *reinterpret_cast<MLA_LDS u16x4*>(ost + (hb * 32 + l32) * OSTR + c * 32 + g * 8 + 4 * hf) = hv;
                }
        // LDS operations of one wave complete in order: the reads see the writes.
        // 128 head rows x 16 chunks of 16 bytes; lane l takes chunk l % 16 of
        // rows 4 i + l / 16.  Waves start at different rows so that concurrent
        // stores spread over memory channels.
        // (a buffer resource over the slot's partial keeps the addresses 32-bit)
        const __amdgpu_buffer_rsrc_t prs = make_rsrc(part_o + (size_t)pslot * H * DC, H * DC * 2);
        const int rot = (blockIdx.x * 4 + w) & 31;
#pragma unroll 4
        for (int i = 0; i < 32; ++i) {
            const int hh = 4 * ((i + rot) & 31) + (lane >> 4);
            const u32x4 v = *reinterpret_cast<const MLA_LDS u32x4*>(ost + hh * OSTR + (lane & 15) * 8);
            __builtin_amdgcn_raw_buffer_store_b128(v, prs, (hh * DC + w * 128 + (lane & 15) * 8) * 2, 0, 0);
        }
        if (hf == 0) lse_dst[head] = (m_ref + __builtin_log2f(l_run)) * kLn2;
        MLA_LAP(14);
    }
#ifdef MLA_PHASE_STAMPS
    ph_[4] = (unsigned)(ph_last_ - ph_start_);
    ph_[6] = (unsigned)ph_rt0_;
    ph_[7] = (unsigned)__builtin_amdgcn_s_memrealtime();
    if (blockIdx.x < (unsigned)kNumCUs && lane < 16) {
        unsigned v = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) v = lane == j ? ph_[j] : v;
        g_phase_stamps[blockIdx.x * 64 + w * 16 + lane] = v;
    }
#endif
}

// ---------------------------------------------------------------------------
// 3. log-sum-exp combine of partitions, then out = W_UV o_lat
// ---------------------------------------------------------------------------

// grid: H * ceil(R / 32) workgroups of 512 threads (h fastest, so one head's
// row blocks share an XCD and its W_UV slice in L2).  Workgroup (h, rb)
// handles rows rb*32 .. +32 of head h.  Its memory traffic is three
// independent reads issued up front -- this head's W_UV slice (as MFMA
// operands, wave w taking output values 16w .. 16w+15), the sequence lengths
// (to locate each row's partials), then every partial and log-sum-exp of the
// wave's 4 rows together -- so the kernel costs about two memory round trips.
//  1. merge: wave w merges rows 4w .. 4w+3 online over their partials (lane
//     holds latent columns 8 lane .. +8): o_lat = sum_p e^{lse_p} o_p / sum_p
//     e^{lse_p}, lse = log sum_p e^{lse_p};
//  2. out^T[16w .. +16][rows] = W_UV[h][16w .. +16] o_lat^T with o_lat from
//     LDS as a bf16 hi + lo pair (16x16x32 MFMA, 32 K-steps of 16 per pair).
constexpr int CMB_THREADS = 512;
constexpr int CMB_CHUNK = 4;                    // partials per row loaded together

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(CMB_THREADS) void combine_kernel(
    const unsigned short* __restrict__ part_o,  // [slots][H][512] fp16
    const float* __restrict__ part_lse,         // [slots][H]
    const int* __restrict__ seq_lens, int q_len, int R, int num_splits, int groups,
    const unsigned short* __restrict__ w_uv,    // [H][128][512]
    unsigned short* __restrict__ out,           // [R][H][128] bf16
    float* __restrict__ lse_out) {              // [R][H] or null
    // merged o_lat of the 32 rows, hi and lo bf16: row rl at rl * 1024 bytes,
    // 16-byte chunk c at position c ^ (rl & 7)
    __shared__ __attribute__((aligned(16))) unsigned char ol[2][32 * 1024];
    __shared__ int pbase[32], pcnt[32], red[2][CMB_THREADS / 64];
    __shared__ float xacc[CMB_THREADS / 64][512], xml[CMB_THREADS / 64][2];   // form B's wave results
    const int h = blockIdx.x % H;
    const int rb = blockIdx.x / H, r0 = rb * 32;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, in an SGPR

    // ---- sequence lengths first (their wait then leaves the W_UV loads in
    // flight): thread tid reads the length behind row tid (and, past 512
    // rows, every 512th after it); lanes 0..31 of wave 0 read this block's rows.
    const bool balanced = num_splits == 0;
    // balanced: entries of the schedule (sequences when Qs > 1, else rows);
    // a row's partials sit Qs slots apart
    const int Qs = sched_qs(q_len), E = R / Qs;
    const int pstr = balanced ? Qs : 1;
    const int len_main = seq_lens[entry_row(q_len, min(tid, E - 1), Qs - 1) / q_len];
    const int len_blk = seq_lens[min(r0 + (lane & 31), R - 1) / q_len];
    // tiles of a row from its sequence length
    auto tiles_of = [&](int r, int len) {
        const int n_vis = len - q_len + (r - (r / q_len) * q_len) + 1;
        return n_vis > 0 ? (n_vis + BS - 1) / BS : 0;
    };
    // (keeps the compiler from hoisting the W_UV loads above these: vector
    // memory loads complete in order, so the lengths would wait for W_UV)
    __builtin_amdgcn_sched_barrier(0);

    // ---- W_UV[h] rows 16w + (lane % 16), K-step ks: latent columns
    // 32 ks + 8 (lane / 16) .. +8 (the A operand of the 16x16x32 MFMA)
    bf16x8 wa[16];
    {
        const unsigned short* wrow = w_uv + ((size_t)h * 128 + 16 * w + (lane & 15)) * DC + (lane >> 4) * 8;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) wa[ks] = *reinterpret_cast<const bf16x8*>(wrow + ks * 32);
    }

    // ---- where each row's partials are (see the split-KV work partition).
    // The balanced schedule's table is computed whatever the schedule (the
    // branch-free form keeps the length loads ahead of W_UV's); a fixed
    // partition overrides it.
    {
        // tiles of all entries (T) and of the entries before this block's first
        const int e0 = r0 / Qs;
        int total = 0, before = 0;
        {
            const int nt = tiles_of(entry_row(q_len, tid, Qs - 1), len_main) * (tid < E ? 1 : 0);
            total = nt;
            before = tid < e0 ? nt : 0;
        }
        for (int e = tid + CMB_THREADS; e < E; e += CMB_THREADS) {
            const int nt = entry_tiles(seq_lens, q_len, e);
            total += nt;
            before += e < e0 ? nt : 0;
        }
#pragma unroll
        for (int d = 32; d > 0; d >>= 1) {
            total += __shfl_xor(total, d, 64);
            before += __shfl_xor(before, d, 64);
        }
        if (lane == 0) {
            red[0][w] = total;
            red[1][w] = before;
        }
        __syncthreads();
        if (w == 0) {
            int T = 0, rs = 0;
#pragma unroll
            for (int k = 0; k < CMB_THREADS / 64; ++k) {
                T += red[0][k];
                rs += red[1][k];
            }
            // lanes 0..31: the block's rows; an exclusive scan over their
            // entries (each entry counted at its first lane in the block)
            // gives the tiles before each row's entry
            const int r = r0 + (lane & 31);
            const int e = r / Qs, s = r - e * Qs;
            const int nt = tiles_of(entry_row(q_len, e, Qs - 1), len_blk) * ((lane < 32 && r < R) ? 1 : 0);
            const int c = (s == 0 || lane == 0) ? nt : 0;
            int incl = c;
#pragma unroll
            for (int d = 1; d < 32; d <<= 1) {
                const int y = __shfl_up(incl, d, 64);
                if ((lane & 31) >= d) incl += y;
            }
            const int first_lane = max(0, (lane & 31) - s);
            rs += __shfl(incl - c, first_lane, 64);
            if (lane < 32) {
                if (balanced) {
                    const int G = (int)balanced_groups(groups, T, Qs);
                    const int f = nt > 0 ? group_of_tile(rs, T, G) : 0;
                    const int l = nt > 0 ? group_of_tile(rs + nt - 1, T, G) : -1;
                    pbase[lane] = Qs * (f + e) + s;
                    pcnt[lane] = nt > 0 ? l - f + 1 : 0;
                } else {
                    pbase[lane] = r < R ? r * num_splits : 0;
                    pcnt[lane] = r < R ? num_splits : 0;
                }
            }
        }
    }
    __syncthreads();

    // ---- 1. merge.  A partial whose piece saw no token has log-sum-exp -inf
    // and unwritten memory: its weight is selected away, never multiplied, so
    // whatever that memory holds cannot leak in.  Two forms:
    //  A. (at most CMB_CHUNK partials per row, or many rows) wave w merges
    //     rows 4w .. 4w+3 itself, CMB_CHUNK partials per row at a time;
    //  B. (more partials, at most 8 rows) the waves split each row's
    //     partials (8 / rows waves per row, 16 partials each at a time) and
    //     the row's first wave merges their results through LDS, so that a
    //     long row costs one memory round trip instead of one per CMB_CHUNK.
    int S_blk = 0;
#pragma unroll
    for (int k = 0; k < 32; ++k) S_blk = max(S_blk, pcnt[k]);
    const int rows_b = min(32, R - r0);
    // per-lane merge of n partials into (m, l, acc): online log-sum-exp
    auto merge_into = [&](float& m_run, float& l_run, float (&acc)[8], const u32x4* v, const float* lv,
                          auto n_c) __attribute__((always_inline)) {
        constexpr int n = decltype(n_c)::value;
        float m_new = m_run;
#pragma unroll
        for (int j = 0; j < n; ++j) m_new = fmaxf(m_new, lv[j]);
        if (m_new == kNegInf) return;                 // nothing visible yet
        const float keep = m_run == kNegInf ? 0.f : __expf(m_run - m_new);
        float e[n], esum = 0.f;
#pragma unroll
        for (int j = 0; j < n; ++j) {
            e[j] = lv[j] == kNegInf ? 0.f : __expf(lv[j] - m_new);
            esum += e[j];
        }
        l_run = l_run * keep + esum;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float a = acc[c] * keep;
#pragma unroll
            for (int j = 0; j < n; ++j) {
                const float x = f16_bits_to_f32((unsigned short)(v[j][c >> 1] >> (16 * (c & 1))));
                a += e[j] != 0.f ? e[j] * x : 0.f;
            }
            acc[c] = a;
        }
        m_run = m_new;
    };
    // merged row rl of the block into LDS as bf16 hi + lo, and its lse
    auto emit_row = [&](int rl, float m_run, float l_run, const float (&acc)[8]) __attribute__((always_inline)) {
        const int r = r0 + rl;
        const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
        u16x8 hi, lo;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float x = acc[c] * inv;
            hi[c] = f32_to_bf16_bits(x);
            lo[c] = f32_to_bf16_bits(x - bf16_bits_to_f32(hi[c]));
        }
        const int off = rl * 1024 + ((lane ^ (rl & 7)) << 4);   // chunk = lane (8 columns)
        *reinterpret_cast<u16x8*>(&ol[0][off]) = hi;
        *reinterpret_cast<u16x8*>(&ol[1][off]) = lo;
        if (lse_out != nullptr && lane == 0 && r < R)
            lse_out[(size_t)r * H + h] = l_run > 0.f ? m_run + __logf(l_run) : kNegInf;
    };
    if (S_blk > CMB_CHUNK && rows_b <= 8) {
        // ---- form B
        constexpr int NB = 16;
        const int wpr = rows_b == 1 ? 8 : rows_b == 2 ? 4 : rows_b <= 4 ? 2 : 1;
        const int rl = w / wpr, sub = w - rl * wpr;
        float m_run = kNegInf, l_run = 0.f, acc[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = 0.f;
        if (rl < rows_b) {
            const int base = pbase[rl], cnt = pcnt[rl];
            const __amdgpu_buffer_rsrc_t prs = make_rsrc(part_o + (size_t)base * H * DC, cnt * pstr * H * DC * 2);
            const __amdgpu_buffer_rsrc_t lrs = make_rsrc(part_lse + (size_t)base * H, cnt * pstr * H * 4);
            for (int p0 = sub; p0 < cnt; p0 += NB * wpr) {
                u32x4 v[NB];
                float lv[NB];
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int sp = (p0 + j * wpr) * pstr;
                    v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        prs, lane * 16, sp * (H * DC * 2) + h * (DC * 2), 0));
                    lv[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                         lrs, 0, sp * (H * 4) + h * 4, 0));
                }
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    if (p0 + j * wpr >= cnt) lv[j] = kNegInf;
                merge_into(m_run, l_run, acc, v, lv, std::integral_constant<int, NB>{});
            }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) xacc[w][lane * 8 + c] = acc[c];
        if (lane == 0) {
            xml[w][0] = m_run;
            xml[w][1] = l_run;
        }
        __syncthreads();
        if (sub == 0 && rl < rows_b) {
            float M = kNegInf;
            for (int k = 0; k < wpr; ++k) M = fmaxf(M, xml[w + k][0]);
            float L = 0.f, a[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) a[c] = 0.f;
            if (M != kNegInf) {
                for (int k = 0; k < wpr; ++k) {
                    const float mk = xml[w + k][0];
                    const float f = mk == kNegInf ? 0.f : __expf(mk - M);
                    L += f * xml[w + k][1];
#pragma unroll
                    for (int c = 0; c < 8; ++c) a[c] += f != 0.f ? f * xacc[w + k][lane * 8 + c] : 0.f;
                }
            }
            emit_row(rl, M, L, a);
        }
    } else {
        // ---- form A
        int base[4], cnt[4], S = 0;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            base[rr] = pbase[4 * w + rr];
            cnt[rr] = pcnt[4 * w + rr];
            S = max(S, cnt[rr]);
        }
        float acc[4][8], m_run[4], l_run[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            m_run[rr] = kNegInf;
            l_run[rr] = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[rr][j] = 0.f;
        }
        // Per-row buffer resources over the row's partials and log-sum-exps: the
        // offsets stay 32-bit and wave-uniform, and a piece past the row's count
        // reads outside the range (zeros; its weight is selected away below).
        __amdgpu_buffer_rsrc_t prs[4], lrs[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            prs[rr] = make_rsrc(part_o + (size_t)base[rr] * H * DC, cnt[rr] * pstr * H * DC * 2);
            lrs[rr] = make_rsrc(part_lse + (size_t)base[rr] * H, cnt[rr] * pstr * H * 4);
        }
        for (int p0 = 0; p0 < S; p0 += CMB_CHUNK) {
            u32x4 v[4][CMB_CHUNK];
            float lv[4][CMB_CHUNK];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                for (int j = 0; j < CMB_CHUNK; ++j) {
                    const int sp = (p0 + j) * pstr;
                    v[rr][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                             prs[rr], lane * 16, sp * (H * DC * 2) + h * (DC * 2), 0));
                    lv[rr][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                              lrs[rr], 0, sp * (H * 4) + h * 4, 0));
                }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                for (int j = 0; j < CMB_CHUNK; ++j)
                    if (p0 + j >= cnt[rr]) lv[rr][j] = kNegInf;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                merge_into(m_run[rr], l_run[rr], acc[rr], v[rr], lv[rr], std::integral_constant<int, CMB_CHUNK>{});
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) emit_row(4 * w + rr, m_run[rr], l_run[rr], acc[rr]);
    }
    __syncthreads();

    // ---- 2. out^T (16 values x 32 rows) of this wave: N-block nb = rows
    // 16 nb .. +16; the B operand of K-step ks is row 16 nb + (lane % 16),
    // latent columns 32 ks + 8 (lane / 16) .. +8, i.e. chunk 4 ks + lane / 16
    f32x4 oacc[2] = {};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int rl = 16 * nb + (lane & 15), ch = 4 * ks + (lane >> 4);
            const int off = rl * 1024 + ((ch ^ (rl & 7)) << 4);
            const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&ol[0][off]);
            const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&ol[1][off]);
            oacc[nb] = mfma16(wa[ks], bh, oacc[nb]);
            oacc[nb] = mfma16(wa[ks], bl, oacc[nb]);
        }
    // out rows (32 rows x 128 values of head h) through LDS, so that each
    // row's 256-byte segment is written by contiguous 16-byte stores: lane
    // (g, n) holds values 16 w + 4 g .. +4 of row 16 nb + n
    constexpr int OROWB = 272;                  // bytes per staged output row
    __syncthreads();                            // every wave is done reading o_lat
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const unsigned long long pk =
            (unsigned long long)f32_to_bf16_bits(oacc[nb][0]) |
            ((unsigned long long)f32_to_bf16_bits(oacc[nb][1]) << 16) |
            ((unsigned long long)f32_to_bf16_bits(oacc[nb][2]) << 32) |
            ((unsigned long long)f32_to_bf16_bits(oacc[nb][3]) << 48);
        *reinterpret_cast<unsigned long long*>(
            &ol[0][(16 * nb + (lane & 15)) * OROWB + (16 * w + 4 * (lane >> 4)) * 2]) = pk;
    }
    __syncthreads();
    {                                           // 32 rows x 16 chunks, one per thread
        const int rl = tid >> 4, c = tid & 15;
        const int r = r0 + rl;
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

hipError_t launch_finalize_absorb(const AppendLaunch& ap, const DecodeLaunch& dp) {
    const int T = ap.batch * ap.n_new, R = dp.batch * dp.q_len;
    const int n_abs = R > 0 ? H * 4 * ((R + 63) / 64) : 0;
    if (T + n_abs == 0) return hipSuccess;
    const FinalizeArgs f{ap.part, ap.kc, T, ap.DC, ap.DR, ap.gamma, ap.eps, ap.rope_base, ap.block_table,
                         ap.max_blocks, ap.start_pos, ap.n_new, ap.BS, ap.pool, ap.pool_scale};
    const auto* qn = static_cast<const unsigned short*>(dp.q_nope);
    const auto* qp = static_cast<const unsigned short*>(dp.q_pe);
    const auto* wk = static_cast<const unsigned short*>(dp.w_uk);
    auto* qbuf = static_cast<unsigned short*>(dp.qbuf);
    if (ap.cache_dtype == MLA_FP8_E4M3)
        finalize_absorb_kernel<MLA_FP8_E4M3><<<T + n_abs, 256, 0, ap.stream>>>(f, qn, qp, wk, qbuf, R);
    else
        finalize_absorb_kernel<MLA_BF16><<<T + n_abs, 256, 0, ap.stream>>>(f, qn, qp, wk, qbuf, R);
    return hipGetLastError();
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
        if (a.cache_dtype == MLA_FP8_E4M3) {
            split_kv_kernel<true><<<grid, 256, 0, a.stream>>>(
                qbuf, static_cast<const unsigned char*>(a.pool), a.pool_scale, a.block_table,
                a.max_blocks, a.seq_lens, R, a.q_len, a.num_splits, scale_log2,
                static_cast<unsigned short*>(a.part_o), a.part_lse);
        } else {
            split_kv_ring_kernel<<<grid, 256, 0, a.stream>>>(
                qbuf, static_cast<const unsigned char*>(a.pool), a.block_table, a.max_blocks,
                a.seq_lens, R, a.q_len, a.num_splits, scale_log2,
                static_cast<unsigned short*>(a.part_o), a.part_lse);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (stages & MLA_STAGE_COMBINE) {
        const int grid = H * ((R + 31) / 32);
        combine_kernel<<<grid, CMB_THREADS, 0, a.stream>>>(static_cast<const unsigned short*>(a.part_o),
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

#ifdef MLA_PHASE_STAMPS
// Copies the ring kernel's phase timers (see g_phase_stamps) to host memory and
// clears them.  Only the instrumented build exports it.
extern "C" mla_status mla_debug_phase_stamps(void* host_dst, size_t bytes) {
    if (host_dst == nullptr) return MLA_ERR_NULL_POINTER;
    if (bytes != sizeof(unsigned) * mla::kPhaseWords) return MLA_ERR_BAD_SHAPE;
    if (hipDeviceSynchronize() != hipSuccess) return MLA_ERR_HIP;
    if (hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(mla::g_phase_stamps), bytes) != hipSuccess) return MLA_ERR_HIP;
    static unsigned zeros[mla::kPhaseWords];
    if (hipMemcpyToSymbol(HIP_SYMBOL(mla::g_phase_stamps), zeros, bytes) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}
#endif

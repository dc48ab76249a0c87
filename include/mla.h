/*
 * mla.h -- C ABI of libmla: absorbed Multi-head Latent Attention (MLA) decode
 * over a paged latent cache, and the cache append that fills it, on AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed (sources cited by page title and section):
 *
 *  - Cache contents.  Each token of each sequence holds one row of
 *    d_c + R values: the RMS-normalised latent c^ (d_c channels) followed by
 *    the rotary key k^R (R channels).  "KV Compression -- DeepSeek-V3",
 *    "How it works" (one map W_kv,a emits latent then pre-rotation key; the
 *    latent is RMS-normalised; 512 + 64 values per token per layer) and
 *    "DeepSeek-V2: MLA Explained", "Caching Strategy".
 *
 *  - Decode.  For sequence b, query row s and head i the result equals naive
 *    MLA attention ("DeepSeek-V2: MLA Explained", "MLA Full Formulas",
 *    sections 2 and 3):
 *        o_i = sum_j softmax_j( (q^C_i . W_UK[i] c^_j + q^R_i . k^R_j) * scale )
 *                    * W_UV[i] c^_j
 *    computed in the weight-absorbed order the pages describe ("DeepSeek-V2:
 *    MLA Explained", "Optimization Note"; "Latent Attention.", "Compress, then
 *    rebuild"): q_lat = W_UK[i]^T q^C_i once per step, scores against the
 *    cached latents, softmax, o_lat = sum_j p_j c^_j, then o_i = W_UV[i] o_lat.
 *    Per-head keys and values are never formed.  scale defaults to
 *    1/sqrt(qk_nope_dim + qk_rope_dim) (section 3's 1/sqrt(d_h + d_h^R)).
 *    Row s sees tokens 0 .. seq_lens[b] - q_len + s (causal between the q_len
 *    new tokens, which are already in the cache).
 *
 *  - Append.  For new token t of sequence b at position p = start_pos[b] + t:
 *        x = W_kv,a h ;  row = [ RMSNorm(x[0:d_c]) * gamma ; RoPE(x[d_c:], p) ]
 *    written to slot (block_table[b][p / block_size], p % block_size).
 *    RMSNorm: x / sqrt(mean(x^2) + eps).  RoPE: pair (x[2k], x[2k+1]) rotated
 *    by p * rope_base^(-2k/R).
 *
 * Conventions for every entry point:
 *
 *  - All tensors are dense, row-major (the cache pool's blocks: see
 *    mla_cache_block_bytes), in device memory owned by the caller.
 *    The library allocates nothing and keeps no state between calls; every
 *    call is reentrant.  Buffers must stay alive until `stream` passes the
 *    enqueued work.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; nothing synchronises the host.  seq_lens, start_pos and
 *    block_table are read on the device only.
 *  - Host-side validation runs before any launch.  A non-MLA_OK status means
 *    nothing was enqueued, except MLA_ERR_HIP, which reports a failed launch.
 *    mla_last_error() returns a message describing the last failure on the
 *    calling thread.
 *  - Device-side contract (not checked): block ids in block_table that a
 *    sequence's tokens reach lie in [0, num_blocks); 1 <= q_len <= seq_lens[b]
 *    (a row that would see no token produces zeros and lse = -inf).
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_OK = 0,
    MLA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL            */
    MLA_ERR_BAD_SHAPE = 2,           /* a size is out of range                */
    MLA_ERR_UNSUPPORTED = 3,         /* dims / dtype combination not built    */
    MLA_ERR_ALIGNMENT = 4,           /* a pointer is not 16-byte aligned      */
    MLA_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes < the size query      */
    MLA_ERR_HIP = 6,                 /* a HIP launch or runtime call failed   */
    MLA_STATUS_MAX_ = 0x7fffffff     /* not a status: keeps the enum int-wide, so
                                        mla_status_string may be given any value */
} mla_status;

typedef enum {
    MLA_F32 = 0,
    MLA_BF16 = 1,
    MLA_FP8_E4M3 = 2  /* OCP e4m3 ("e4m3fn"): bias 7, max 448, no infinities */
} mla_dtype;

/* Shape and storage types of one MLA layer.
 *
 * Two code paths exist:
 *  - the MFMA path, for the DeepSeek-V3 head shape: n_heads 128,
 *    kv_lora_rank 512, qk_rope_dim 64, qk_nope_dim 128, v_head_dim 128,
 *    block_size 64, act_dtype BF16, cache_dtype BF16 or FP8_E4M3;
 *  - a portable path for any other shape within the limits below
 *    (n_heads <= 1024, kv_lora_rank <= 1024, qk_rope_dim <= 256 and even,
 *    qk_nope_dim <= 512, v_head_dim <= 512, 1 <= block_size <= 4096),
 *    act_dtype F32 or BF16, cache_dtype F32, BF16 or FP8_E4M3.
 * Both compute in fp32 and give the same result up to rounding. */
typedef struct {
    int32_t n_heads;       /* H                                              */
    int32_t kv_lora_rank;  /* d_c: latent width                              */
    int32_t qk_rope_dim;   /* R = d_h^R: rotary key / query width            */
    int32_t qk_nope_dim;   /* N = d_h: per-head content query width          */
    int32_t v_head_dim;    /* V: per-head output width                       */
    int32_t block_size;    /* tokens per cache block                         */
    int32_t cache_dtype;   /* mla_dtype of the cache pool                    */
    int32_t act_dtype;     /* mla_dtype of q, weights, h, gamma and out      */
    float softmax_scale;   /* 0 => 1/sqrt(qk_nope_dim + qk_rope_dim)         */
    int32_t flags;         /* reserved: must be 0                            */
} mla_dims;

/* mla_dims.flags is reserved: no flag is defined and every call that takes
 * dims returns MLA_ERR_UNSUPPORTED when it is not 0. */

/* Status name, e.g. "MLA_ERR_BAD_SHAPE". Never NULL. */
const char* mla_status_string(mla_status status);

/* Message for the last non-OK status returned on the calling thread
 * ("" if none).  The pointer stays valid until the next call on the thread. */
const char* mla_last_error(void);

/* Bytes of one cache row: (kv_lora_rank + qk_rope_dim) * element size.
 * Returns 0 for an invalid dims pointer or dtype. */
size_t mla_cache_row_bytes(const mla_dims* dims);

/* Bytes of one cache block: block_size * mla_cache_row_bytes(dims).  The pool
 * is an array of these, num_blocks blocks of block_size * D elements
 * (D = kv_lora_rank + qk_rope_dim).  Inside a block the rows are
 * token-major for every cache dtype: token t's row of D elements at t * D
 * (latent channels 0 .. kv_lora_rank - 1, then the rotary key).
 * Only the library's own calls (mla_cache_append) need to write a pool; the
 * layout matters to callers that fill or read pools themselves.
 * With FP8_E4M3 the per-token fp32 scales live in a separate array
 * cache_scale[num_blocks][block_size]. */
size_t mla_cache_block_bytes(const mla_dims* dims);

/* Workspace bytes mla_cache_append needs for `batch * n_new` new tokens. */
mla_status mla_cache_append_workspace_size(const mla_dims* dims, int32_t batch,
                                           int32_t n_new, int32_t d_model,
                                           size_t* bytes);

/* Project, normalise, rotate and store `n_new` new tokens per sequence.
 *
 *  h             [batch][n_new][d_model]            act_dtype
 *  w_kv_a        [kv_lora_rank + qk_rope_dim][d_model] act_dtype; latent rows first
 *  kv_norm_gamma [kv_lora_rank]                     act_dtype
 *  rms_eps       RMSNorm epsilon (added to mean(x^2))
 *  rope_base     RoPE base (10000 for DeepSeek)
 *  block_table   [batch][max_blocks_per_seq] int32, device
 *  start_pos     [batch] int32, device: position of sequence b's first new token
 *  cache_pool    [num_blocks][block_size * (kv_lora_rank + qk_rope_dim)] cache_dtype
 *                (block layout: see mla_cache_block_bytes)
 *  cache_scale   [num_blocks][block_size] float, FP8_E4M3 only (else NULL):
 *                receives amax/448 of each written row; the row holds
 *                round-to-nearest-even(x / scale), saturated to +-448
 *  workspace     device scratch of at least mla_cache_append_workspace_size bytes
 *
 * Only the batch * n_new addressed rows (and their scales) are written.  bf16
 * and fp8 stores round to nearest even.  d_model must be a multiple of 8. */
mla_status mla_cache_append(const mla_dims* dims, int32_t batch, int32_t n_new,
                            int32_t d_model, const void* h, const void* w_kv_a,
                            const void* kv_norm_gamma, float rms_eps, float rope_base,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* start_pos, void* cache_pool,
                            float* cache_scale, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Split-KV partitions per query row that mla_decode_absorbed uses when
 * num_splits == 0 on shapes served by the portable kernels: a function of batch
 * and q_len only (the host never reads sequence lengths).  The DeepSeek-V3
 * shape (MFMA kernels) uses the balanced schedule for num_splits == 0 instead
 * (see mla_decode_absorbed). */
int32_t mla_decode_default_splits(const mla_dims* dims, int32_t batch, int32_t q_len);

/* Workspace bytes mla_decode_absorbed needs for this num_splits (0 included). */
mla_status mla_decode_workspace_size(const mla_dims* dims, int32_t batch,
                                     int32_t q_len, int32_t num_splits,
                                     size_t* bytes);

/* Stages of one decode, for mla_decode_absorbed_stages. */
enum {
    MLA_STAGE_ABSORB_Q = 1,  /* q_lat = W_UK^T q_nope, packed with q_pe        */
    MLA_STAGE_SPLIT_KV = 2,  /* per-partition attention over the latent cache */
    MLA_STAGE_COMBINE = 4,   /* log-sum-exp merge of partitions, then W_UV    */
    MLA_STAGE_ALL = 7
};

/* One absorbed-MLA decode step over a paged latent cache.
 *
 *  q_nope       [batch][q_len][n_heads][qk_nope_dim] act_dtype
 *  q_pe         [batch][q_len][n_heads][qk_rope_dim] act_dtype, already rotated
 *  w_uk         [n_heads][qk_nope_dim][kv_lora_rank] act_dtype (k^C = W_UK[i] c^)
 *  w_uv         [n_heads][v_head_dim][kv_lora_rank]  act_dtype (v^C = W_UV[i] c^)
 *  cache_pool   [num_blocks][block_size * (kv_lora_rank + qk_rope_dim)] cache_dtype
 *               (block layout: see mla_cache_block_bytes)
 *  cache_scale  [num_blocks][block_size] float (FP8_E4M3 only, else NULL):
 *               a cached value is float(code) * scale of its token
 *  block_table  [batch][max_blocks_per_seq] int32, device
 *  seq_lens     [batch] int32, device: tokens of sequence b, the q_len new
 *               ones included
 *  num_splits   split-KV partitions per (sequence, query row), at most 256.
 *               Partition k of a row that sees n tokens covers tokens
 *               [k*P, (k+1)*P) with P = ceil(n / (num_splits * block_size))
 *               * block_size; empty partitions are skipped.
 *               0 on the DeepSeek-V3 shape: balanced schedule.  The visible
 *               64-token tiles of all rows, concatenated in row order, are
 *               divided into equal contiguous ranges, one per workgroup
 *               (as many workgroups as compute units, fewer when there are
 *               fewer tiles); a range may cover parts of several rows, each
 *               giving one partition.  Ragged batches then keep every compute
 *               unit equally busy.  0 on other shapes: the default split count
 *               (mla_decode_default_splits).
 *  out          [batch][q_len][n_heads][v_head_dim] act_dtype
 *  lse          [batch][q_len][n_heads] float or NULL: natural-log
 *               log-sum-exp of the scaled scores (-inf for a row with no token)
 *  workspace    device scratch of at least mla_decode_workspace_size bytes
 *
 * The MFMA path needs q_nope, q_pe, w_uk, w_uv, cache_pool and out 16-byte
 * aligned.  seq_lens is not updated. */
mla_status mla_decode_absorbed(const mla_dims* dims, int32_t batch, int32_t q_len,
                               const void* q_nope, const void* q_pe,
                               const void* w_uk, const void* w_uv,
                               const void* cache_pool, const float* cache_scale,
                               const int32_t* block_table, int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, int32_t num_splits,
                               void* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/* mla_decode_absorbed restricted to the stages in `stages` (MLA_STAGE_* bits),
 * for timing or overlapping the stages separately.  Running ABSORB_Q, then
 * SPLIT_KV, then COMBINE with the same arguments and workspace equals one
 * mla_decode_absorbed call; each stage reads what the previous one left in
 * the workspace. */
mla_status mla_decode_absorbed_stages(const mla_dims* dims, int32_t batch, int32_t q_len,
                                      const void* q_nope, const void* q_pe,
                                      const void* w_uk, const void* w_uv,
                                      const void* cache_pool, const float* cache_scale,
                                      const int32_t* block_table,
                                      int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, int32_t num_splits,
                                      void* out, float* lse, void* workspace,
                                      size_t workspace_bytes, uint32_t stages,
                                      void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * mla_decode_absorbed with no workspace argument.  Its scratch is one
 * statically sized device array inside the library (MLA_NOALLOC_SCRATCH_BYTES
 * per GPU, held from the library's first use on that GPU until the process
 * ends); the call allocates nothing.
 *
 * Arguments, results and requirements as mla_decode_absorbed, and the same
 * kernels run.  The stream must belong to the current device.  A call whose
 * workspace (mla_decode_workspace_size for the same arguments) exceeds
 * MLA_NOALLOC_SCRATCH_BYTES returns MLA_ERR_WORKSPACE_TOO_SMALL and launches
 * nothing; with the balanced schedule on the DeepSeek-V3 shape that admits
 * batch * q_len up to 119.  Every call on one GPU uses the same array, which
 * keeps what the last call left: calls that overlap on one GPU (on several
 * streams, or on one stream from several host threads without ordering)
 * race and their results are undefined. */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
mla_status mla_decode_absorbed_noalloc(const mla_dims* dims, int32_t batch, int32_t q_len,
                                       const void* q_nope, const void* q_pe,
                                       const void* w_uk, const void* w_uv,
                                       const void* cache_pool, const float* cache_scale,
                                       const int32_t* block_table,
                                       int32_t max_blocks_per_seq,
                                       const int32_t* seq_lens, int32_t num_splits,
                                       void* out, float* lse, void* stream);

/* ---- one decode step with its cache append ---------------------------------
 *
 * mla_cache_append of the step's new tokens, then mla_decode_absorbed over
 * the cache that holds them, in one call.  Sequence b appends q_len tokens
 * (hidden states h [batch][q_len][d_model], positions start_pos[b] ..
 * start_pos[b] + q_len - 1) and the same tokens' queries attend to every
 * cached token, themselves included: seq_lens[b] = start_pos[b] + q_len,
 * which the caller keeps consistent (the two arrays are read on the device).
 * The path is the one of "DeepSeek-V2: MLA Explained", "MLA Full Formulas"
 * sections 2-3, in the absorbed form of its "Optimization Note".
 *
 * Results -- out, lse and every byte of the pool -- are bit for bit those of
 * the two calls made in that order on one stream.  With bf16 activations on
 * the DeepSeek-V3 head shape the append's per-token finalize (norm, rotation,
 * store) and the decode's query absorption, which do not depend on each
 * other, run as one launch.
 *  arguments   as mla_cache_append (n_new = q_len) and mla_decode_absorbed
 *  workspace   mla_decode_step_workspace_size bytes, 16-byte aligned: the
 *              decode's workspace, then the append's
 * Errors: those of the two calls (checked before anything is launched). */
enum {
    MLA_STEP_PROJECT = 1,          /* the append's projection x = W_kv,a h          */
    MLA_STEP_FINALIZE_ABSORB = 2,  /* the append's finalize + the query absorption  */
    MLA_STEP_SPLIT_KV = 4,         /* the decode's split-KV pass                     */
    MLA_STEP_COMBINE = 8,          /* the decode's combine and W_UV                  */
    MLA_STEP_ALL = 15
};
mla_status mla_decode_step_workspace_size(const mla_dims* dims, int32_t batch, int32_t q_len,
                                          int32_t d_model, int32_t num_splits, size_t* bytes);
mla_status mla_decode_step(const mla_dims* dims, int32_t batch, int32_t q_len, int32_t d_model,
                           const void* h, const void* w_kv_a, const void* kv_norm_gamma,
                           float rms_eps, float rope_base, const int32_t* start_pos,
                           const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                           void* cache_pool, float* cache_scale, const int32_t* block_table,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_splits,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);
/* mla_decode_step restricted to the MLA_STEP_* stages in `stages` (run in the
 * order above, each reading what the earlier ones left in the workspace and
 * the pool), for per-kernel timing; all of them equal one mla_decode_step. */
mla_status mla_decode_step_stages(const mla_dims* dims, int32_t batch, int32_t q_len, int32_t d_model,
                                  const void* h, const void* w_kv_a, const void* kv_norm_gamma,
                                  float rms_eps, float rope_base, const int32_t* start_pos,
                                  const void* q_nope, const void* q_pe, const void* w_uk,
                                  const void* w_uv, void* cache_pool, float* cache_scale,
                                  const int32_t* block_table, int32_t max_blocks_per_seq,
                                  const int32_t* seq_lens, int32_t num_splits, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, uint32_t stages,
                                  void* stream);

/* ---- debug check of the device-side contract --------------------------------
 *
 * The decode and the append read block_table and seq_lens on the device
 * without checking them.  This call checks them, on the device: for every
 * sequence b, 0 <= seq_lens[b] <= max_blocks_per_seq * block_size, and every
 * block id block_table[b][k], k < ceil(seq_lens[b] / block_size), lies in
 * [0, num_blocks).  It writes report[0] = the number of violations,
 * report[1], report[2] = the first one (smallest b, then k; k = -1 for a
 * length), or -1, -1.  report: 3 int32 in device memory, valid once `stream`
 * has passed the call.  One workgroup walks batch * (max_blocks_per_seq + 1)
 * entries: a debugging aid, not for every step.
 * Errors (nothing launched): MLA_ERR_BAD_SHAPE, MLA_ERR_NULL_POINTER. */
mla_status mla_check_block_table(const mla_dims* dims, int32_t batch, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                 int32_t num_blocks, int32_t* report, void* stream);

/* ---- output projection -----------------------------------------------------
 *
 * The layer's output side ("DeepSeek-V2: MLA Explained", "MLA Full Formulas",
 * section 3): the heads' outputs of a query row, concatenated head after head,
 * times W_O:  u = W_O [o_1; ...; o_H].
 *
 * mla_output_project: out[t][j] = sum_k w[j][k] x[t][k] for t < rows, j < n,
 * bf16 operands, fp32 accumulation, bf16 result.  With x the decode's output
 * [rows][n_heads][v_head_dim] read as [rows][n_heads * v_head_dim] and w = W_O
 * [d_model][n_heads * v_head_dim] this is u.  (Any bf16 product of this form
 * runs: e.g. the merged weights W_O W_UV [d_model][n_heads * kv_lora_rank]
 * applied to the heads' attention-weighted latents.)
 *  rows         0 .. 65536;  k a positive multiple of 64;  n a positive
 *               multiple of 32;  rows * k * 2 and n * k * 2 below 2^31
 *  x [rows][k], w [n][k], out [rows][n]: bf16, device, 16-byte aligned
 *  workspace    device scratch of at least mla_output_workspace_size bytes
 *               (fp32 partial sums of the depth-split product), 16-byte aligned
 * The partial sums are added in a fixed order: results do not depend on
 * scheduling.  Errors: MLA_ERR_BAD_SHAPE, MLA_ERR_NULL_POINTER,
 * MLA_ERR_ALIGNMENT, MLA_ERR_WORKSPACE_TOO_SMALL; nothing is launched then. */
mla_status mla_output_workspace_size(int32_t rows, int32_t k, int32_t n, size_t* bytes);
mla_status mla_output_project(int32_t rows, int32_t k, int32_t n, const void* x, const void* w,
                              void* out, void* workspace, size_t workspace_bytes, void* stream);

/* One decode step through the output projection: mla_decode_absorbed, whose
 * output o [batch][q_len][n_heads][v_head_dim] stays in the workspace, then
 * u = W_O [o_1; ...; o_H] as mla_output_project.
 *  w_o   [d_model][n_heads * v_head_dim] bf16 (columns h * v_head_dim .. +
 *        v_head_dim act on head h)
 *  u     [batch][q_len][d_model] bf16
 *  lse   as mla_decode_absorbed (or NULL)
 * Other arguments as mla_decode_absorbed; act_dtype must be MLA_BF16,
 * n_heads * v_head_dim a multiple of 64 and d_model a multiple of 32.
 * workspace: at least mla_decode_output_workspace_size bytes. */
mla_status mla_decode_output_workspace_size(const mla_dims* dims, int32_t batch, int32_t q_len,
                                            int32_t num_splits, int32_t d_model, size_t* bytes);
mla_status mla_decode_output(const mla_dims* dims, int32_t batch, int32_t q_len,
                             const void* q_nope, const void* q_pe,
                             const void* w_uk, const void* w_uv,
                             const void* cache_pool, const float* cache_scale,
                             const int32_t* block_table, int32_t max_blocks_per_seq,
                             const int32_t* seq_lens, int32_t num_splits, int32_t d_model,
                             const void* w_o, void* u, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---- query path ------------------------------------------------------------
 *
 * The decode's query inputs from the layer input ("DeepSeek-V2: MLA
 * Explained", "MLA Full Formulas", step 1, query compression).  For query row
 * s of sequence b, at position p = start_pos[b] + s:
 *     c_Q = W_DQ h                            (h itself when q_lora_rank == 0:
 *                                              full-rank queries)
 *     c_Q = RMSNorm(c_Q) * q_norm_gamma       when q_norm_gamma is not NULL
 *                                              (the norm V3 applies after its
 *                                              compressed vectors, "KV
 *                                              Compression -- DeepSeek-V3",
 *                                              "How it works"); NULL leaves
 *                                              the formula as printed
 *     q^C = W_UQ c_Q,   q^R = RoPE(W_QR c_Q, p)
 * split into head blocks [q_1; ...; q_H].  RoPE turns pairs (x[2k], x[2k+1])
 * of each head's rotary block by p * rope_base^(-2k/qk_rope_dim), as the cache
 * append turns the keys.  c_Q is rounded to bf16 between the two products;
 * accumulation is fp32.
 *
 *  h            [batch][q_len][d_model] bf16
 *  w_dq         [q_lora_rank][d_model] bf16 (NULL when q_lora_rank == 0)
 *  q_norm_gamma [q_lora_rank] bf16 or NULL (must be NULL when q_lora_rank == 0)
 *  w_uq         [n_heads * qk_nope_dim][f] bf16, f = q_lora_rank or d_model
 *  w_qr         [n_heads * qk_rope_dim][f] bf16
 *  start_pos    [batch] int32, device
 *  q_nope       [batch][q_len][n_heads][qk_nope_dim] bf16 (out): the decode's q_nope
 *  q_pe         [batch][q_len][n_heads][qk_rope_dim] bf16 (out): the decode's
 *               q_pe, rotated
 *  workspace    device scratch of mla_query_workspace_size bytes (0 bytes, and
 *               NULL allowed, when q_lora_rank == 0)
 *
 * Requirements (else MLA_ERR_BAD_SHAPE / MLA_ERR_UNSUPPORTED): act_dtype
 * MLA_BF16; d_model a multiple of 64 in [64, 65536]; q_lora_rank 0 or a
 * multiple of 64 up to 2048; n_heads *
 * qk_nope_dim and n_heads * qk_rope_dim multiples of 32; q_len and batch *
 * q_len at most 65536 (a whole prompt may be projected at once); every
 * operand under 2 GiB.  Every tensor 16-byte aligned.
 * Of mla_dims only the head shape and act_dtype are used (all fields are
 * validated as for the other calls). */
mla_status mla_query_workspace_size(const mla_dims* dims, int32_t batch, int32_t q_len,
                                   int32_t d_model, int32_t q_lora_rank, size_t* bytes);
mla_status mla_query_project(const mla_dims* dims, int32_t batch, int32_t q_len, int32_t d_model,
                             int32_t q_lora_rank, const void* h, const void* w_dq,
                             const void* q_norm_gamma, float rms_eps, const void* w_uq,
                             const void* w_qr, float rope_base, const int32_t* start_pos,
                             void* q_nope, void* q_pe, void* workspace, size_t workspace_bytes,
                             void* stream);

/* ---- prefill -----------------------------------------------------------------
 *
 * Causal attention of many query rows per sequence over the paged latent
 * cache, in the decompressed form ("DeepSeek-V2: MLA Explained", "MLA Full
 * Formulas", steps 2 and 3): for every token j of sequence b and head i the
 * keys and values are rebuilt,
 *     K_{j,i} = [W_UK[i] c_j ; k^R_j],   V_{j,i} = W_UV[i] c_j,
 * and query s (of q_len) attends to tokens 0 .. seq_lens[b] - q_len + s:
 *     out = softmax(q . K^T * scale) V.
 * The arguments and the result are those of mla_decode_absorbed with the same
 * q_len (rows with no visible token: zeros and lse -inf); the two calls differ
 * in cost.  Per (query, key) pair the rebuilt form costs 2 H (N + R + V)
 * flops against 2 H (2 kv_lora_rank + R) for the absorbed one, and the
 * rebuild, 4 H N kv_lora_rank flops per token, is shared by all of a
 * sequence's queries: the call for long prompts, chunked or not.
 *
 * Steps (MLA_PREFILL_* bits for mla_prefill_stages): gather the rows of each
 * sequence from the pool into the workspace; rebuild K^C and V (bf16, fp32
 * accumulation; an fp8 cache enters as the codes' exact values with the
 * token scale applied to the fp32 products, its rotary keys as code * scale
 * rounded to bf16); attend (bf16 MFMA, fp32 accumulation, softmax weights
 * rounded to bf16 for the value product).
 *
 *  q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale, block_table, seq_lens,
 *  out, lse      as for mla_decode_absorbed; lse may be NULL.
 *  workspace     mla_prefill_workspace_size bytes: about 66 KB per token of
 *                batch * max_blocks_per_seq * block_size (rebuilt keys and
 *                values of every head)
 *
 * Requirements (else MLA_ERR_UNSUPPORTED / MLA_ERR_BAD_SHAPE): the
 * DeepSeek-V3 shape (128 heads, kv_lora_rank 512, qk_rope_dim 64, qk_nope_dim
 * and v_head_dim 128, block_size 64, act_dtype MLA_BF16, cache MLA_BF16 or
 * MLA_FP8_E4M3, no flags); q_len in [1, 2^20]; max_blocks_per_seq in
 * [1, 65536] with batch * max_blocks_per_seq * 64 <= 2^22; every tensor
 * 16-byte aligned.  seq_lens[b] above max_blocks_per_seq * block_size is
 * taken as that maximum. */
enum {
    MLA_PREFILL_GATHER = 1,      /* pool rows -> contiguous latents / rotary keys */
    MLA_PREFILL_DECOMPRESS = 2,  /* K^C = W_UK c, V = W_UV c for every token      */
    MLA_PREFILL_ATTEND = 4,      /* causal attention over the rebuilt keys        */
    MLA_PREFILL_ALL = 7
};
mla_status mla_prefill_workspace_size(const mla_dims* dims, int32_t batch, int32_t q_len,
                                      int32_t max_blocks_per_seq, size_t* bytes);
mla_status mla_prefill(const mla_dims* dims, int32_t batch, int32_t q_len,
                       const void* q_nope, const void* q_pe, const void* w_uk,
                       const void* w_uv, const void* cache_pool, const float* cache_scale,
                       const int32_t* block_table, int32_t max_blocks_per_seq,
                       const int32_t* seq_lens, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream);
/* mla_prefill restricted to the steps in `stages` (MLA_PREFILL_* bits), for
 * timing them separately.  Each step reads what the previous one left in the
 * workspace. */
mla_status mla_prefill_stages(const mla_dims* dims, int32_t batch, int32_t q_len,
                              const void* q_nope, const void* q_pe, const void* w_uk,
                              const void* w_uv, const void* cache_pool,
                              const float* cache_scale, const int32_t* block_table,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens, void* out,
                              float* lse, void* workspace, size_t workspace_bytes,
                              uint32_t stages, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */

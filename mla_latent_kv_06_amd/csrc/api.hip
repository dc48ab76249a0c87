// C ABI of libmla (include/mla.h): argument validation, workspace layout and
// dispatch to the MFMA or portable kernels.  Every check runs on the host
// before anything is enqueued.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "internal.hpp"
#include "output.hpp"
#include "prefill.hpp"
#include "query.hpp"

namespace {

thread_local char g_err[512] = "";

mla_status fail(mla_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

mla_status ok() {
    g_err[0] = '\0';
    return MLA_OK;
}

size_t elem_bytes(int dt) {
    switch (dt) {
        case MLA_F32: return 4;
        case MLA_BF16: return 2;
        case MLA_FP8_E4M3: return 1;
        default: return 0;
    }
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mla_status check_dims(const mla_dims* d) {
    if (d == nullptr) return fail(MLA_ERR_NULL_POINTER, "dims is NULL");
    if (d->n_heads < 1 || d->n_heads > 1024)
        return fail(MLA_ERR_BAD_SHAPE, "n_heads=%d outside [1, 1024]", d->n_heads);
    if (d->kv_lora_rank < 1 || d->kv_lora_rank > 1024)
        return fail(MLA_ERR_BAD_SHAPE, "kv_lora_rank=%d outside [1, 1024]", d->kv_lora_rank);
    if (d->qk_rope_dim < 0 || d->qk_rope_dim > 256 || (d->qk_rope_dim & 1))
        return fail(MLA_ERR_BAD_SHAPE, "qk_rope_dim=%d must be even and in [0, 256]", d->qk_rope_dim);
    if (d->qk_nope_dim < 1 || d->qk_nope_dim > 512)
        return fail(MLA_ERR_BAD_SHAPE, "qk_nope_dim=%d outside [1, 512]", d->qk_nope_dim);
    if (d->v_head_dim < 1 || d->v_head_dim > 512)
        return fail(MLA_ERR_BAD_SHAPE, "v_head_dim=%d outside [1, 512]", d->v_head_dim);
    if (d->block_size < 1 || d->block_size > 4096)
        return fail(MLA_ERR_BAD_SHAPE, "block_size=%d outside [1, 4096]", d->block_size);
    if (elem_bytes(d->cache_dtype) == 0)
        return fail(MLA_ERR_UNSUPPORTED, "cache_dtype=%d unknown", d->cache_dtype);
    if (d->act_dtype != MLA_F32 && d->act_dtype != MLA_BF16)
        return fail(MLA_ERR_UNSUPPORTED, "act_dtype=%d must be MLA_F32 or MLA_BF16", d->act_dtype);
    if (!(d->softmax_scale >= 0.f) || std::isinf(d->softmax_scale))
        return fail(MLA_ERR_BAD_SHAPE, "softmax_scale must be finite and >= 0");
    if (d->flags != 0)
        return fail(MLA_ERR_UNSUPPORTED, "flags=0x%x: no flags are defined; pass 0", (unsigned)d->flags);
    return MLA_OK;
}

float resolved_scale(const mla_dims& d) {
    return d.softmax_scale > 0.f ? d.softmax_scale
                                 : 1.0f / std::sqrt((float)(d.qk_nope_dim + d.qk_rope_dim));
}

int default_splits(int batch, int q_len) {
    const long long rows = (long long)batch * q_len;
    if (rows <= 0) return 1;
    long long s = (mla::kNumCUs + rows - 1) / rows;
    if (s > 64) s = 64;
    return (int)(s < 1 ? 1 : s);
}

struct DecodeWs {
    size_t qbuf, part_o, part_lse, total;
};

// Partial slots of the split-KV pass: R * splits with a fixed split count;
// with balanced scheduling (MFMA shapes, num_splits == 0) one per (workgroup,
// row) piece, at most kNumCUs + R.
size_t partial_slots(const mla_dims& d, int batch, int q_len, int num_splits) {
    const size_t R = (size_t)batch * q_len;
    if (num_splits > 0) return R * num_splits;
    if (mla::is_v3_shape(d)) return mla::kNumCUs + R;
    return R * default_splits(batch, q_len);
}

DecodeWs decode_ws(const mla_dims& d, int batch, int q_len, int num_splits) {
    const bool mfma = mla::is_v3_shape(d);
    const size_t R = (size_t)batch * q_len, H = d.n_heads;
    const size_t slots = partial_slots(d, batch, q_len, num_splits);
    DecodeWs w;
    w.qbuf = 0;
    size_t qb = R * H * (d.kv_lora_rank + d.qk_rope_dim) * (mfma ? 2 : 4);
    w.part_o = align_up(qb, 256);
    // partial o_lat: fp16 on the MFMA path (normalised convex combinations of
    // latent rows, stored with 2^-11 relative precision), fp32 otherwise
    w.part_lse = w.part_o + align_up(slots * H * d.kv_lora_rank * (mfma ? 2 : 4), 256);
    w.total = w.part_lse + align_up(slots * H * sizeof(float), 256);
    return w;
}

int append_kc(int d_model) { return (d_model + mla::kAppendChunk - 1) / mla::kAppendChunk; }

// The append's MFMA projection runs on the weight-streaming GEMM when
// d_model is a multiple of 64 and its operands stay under 2 GiB (32-bit
// buffer ranges), else on the split-K kernel of append.hip.
bool append_streams(const mla_dims& d, long long T, int d_model) {
    const long long Dout = d.kv_lora_rank + d.qk_rope_dim;
    return d_model % 64 == 0 && T * d_model * 2 < (1ll << 31) && Dout * d_model * 2 < (1ll << 31);
}

// partial slices of the append's MFMA projection
int append_slices(const mla_dims& d, long long T, int d_model) {
    return append_streams(d, T, d_model)
               ? mla::append_stream_splits(d.kv_lora_rank + d.qk_rope_dim, d_model, T)
               : append_kc(d_model);
}

bool append_uses_mfma(const mla_dims& d, int d_model) {
    return d.act_dtype == MLA_BF16 && (d.kv_lora_rank + d.qk_rope_dim) % 32 == 0 &&
           d_model % 16 == 0;
}

// Validates a decode call and fills its launch description; *empty: nothing
// to launch (batch 0).
mla_status decode_prepare(const mla_dims* dims, int32_t batch, int32_t q_len, const void* q_nope,
                          const void* q_pe, const void* w_uk, const void* w_uv, const void* cache_pool,
                          const float* cache_scale, const int32_t* block_table,
                          int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_splits,
                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                          unsigned stages, void* stream, mla::DecodeLaunch& a, bool& mfma, bool& empty) {
    empty = false;
    if (mla_status st = check_dims(dims); st != MLA_OK) return st;
    const mla_dims& d = *dims;
    if (batch < 0 || q_len < 1 || q_len > 1024)
        return fail(MLA_ERR_BAD_SHAPE, "batch=%d must be >= 0 and q_len=%d in [1, 1024]", batch, q_len);
    if (num_splits < 0 || num_splits > mla::kMaxSplits)
        return fail(MLA_ERR_BAD_SHAPE, "num_splits=%d outside [0, %d]", num_splits, mla::kMaxSplits);
    if (stages == 0 || (stages & ~(unsigned)MLA_STAGE_ALL))
        return fail(MLA_ERR_BAD_SHAPE, "stages=0x%x: use MLA_STAGE_* bits", stages);
    if (batch == 0) {
        empty = true;
        return ok();
    }
    if (max_blocks_per_seq < 1) return fail(MLA_ERR_BAD_SHAPE, "max_blocks_per_seq must be >= 1");
    // 0: balanced scheduling on the MFMA path, the default split count otherwise
    const int splits = (num_splits == 0 && !mla::is_v3_shape(d)) ? default_splits(batch, q_len)
                                                                  : num_splits;
    if ((stages & MLA_STAGE_ABSORB_Q) && (!q_nope || !q_pe || !w_uk))
        return fail(MLA_ERR_NULL_POINTER, "q_nope, q_pe and w_uk are required");
    if ((stages & MLA_STAGE_SPLIT_KV) && (!cache_pool || !block_table || !seq_lens))
        return fail(MLA_ERR_NULL_POINTER, "cache_pool, block_table and seq_lens are required");
    if ((stages & MLA_STAGE_SPLIT_KV) && d.cache_dtype == MLA_FP8_E4M3 && !cache_scale)
        return fail(MLA_ERR_NULL_POINTER, "cache_scale is required for an FP8 cache");
    if ((stages & MLA_STAGE_COMBINE) && (!w_uv || !out))
        return fail(MLA_ERR_NULL_POINTER, "w_uv and out are required");
    if (!workspace) return fail(MLA_ERR_NULL_POINTER, "workspace is NULL");
    const DecodeWs ws = decode_ws(d, batch, q_len, num_splits);
    if (workspace_bytes < ws.total)
        return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes=%zu < %zu", workspace_bytes, ws.total);
    mfma = mla::is_v3_shape(d);
    if (mfma) {
        const void* ptrs[] = {q_nope, q_pe, w_uk, w_uv, cache_pool, out, workspace};
        for (const void* p : ptrs)
            if (p && !aligned16(p)) return fail(MLA_ERR_ALIGNMENT, "tensor at %p is not 16-byte aligned", p);
        if (cache_scale && ((uintptr_t)cache_scale & 15u))
            return fail(MLA_ERR_ALIGNMENT, "cache_scale is not 16-byte aligned");
    } else if (!aligned16(workspace)) {
        return fail(MLA_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
    }
    a = mla::DecodeLaunch{};
    a.H = d.n_heads;
    a.DC = d.kv_lora_rank;
    a.DR = d.qk_rope_dim;
    a.N = d.qk_nope_dim;
    a.V = d.v_head_dim;
    a.BS = d.block_size;
    a.cache_dtype = d.cache_dtype;
    a.act_dtype = d.act_dtype;
    a.scale = resolved_scale(d);
    a.batch = batch;
    a.q_len = q_len;
    a.num_splits = splits;
    a.q_nope = q_nope;
    a.q_pe = q_pe;
    a.w_uk = w_uk;
    a.w_uv = w_uv;
    a.pool = cache_pool;
    a.pool_scale = cache_scale;
    a.block_table = block_table;
    a.max_blocks = max_blocks_per_seq;
    a.seq_lens = seq_lens;
    a.out = out;
    a.lse = lse;
    char* base = static_cast<char*>(workspace);
    a.qbuf = base + ws.qbuf;
    a.part_o = base + ws.part_o;
    a.part_lse = reinterpret_cast<float*>(base + ws.part_lse);
    a.stream = static_cast<hipStream_t>(stream);
    return ok();
}

mla_status launch_status(hipError_t e) {
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

mla_status decode_impl(const mla_dims* dims, int32_t batch, int32_t q_len, const void* q_nope,
                       const void* q_pe, const void* w_uk, const void* w_uv, const void* cache_pool,
                       const float* cache_scale, const int32_t* block_table,
                       int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_splits,
                       void* out, float* lse, void* workspace, size_t workspace_bytes,
                       unsigned stages, void* stream) {
    mla::DecodeLaunch a;
    bool mfma = false, empty = false;
    if (mla_status st = decode_prepare(dims, batch, q_len, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale,
                                       block_table, max_blocks_per_seq, seq_lens, num_splits, out, lse,
                                       workspace, workspace_bytes, stages, stream, a, mfma, empty);
        st != MLA_OK || empty)
        return st;
    return launch_status(mfma ? mla::launch_decode_mfma(a, stages) : mla::launch_decode_generic(a, stages));
}

// Query path: shape checks shared by the sizing call and the entry point.
mla_status check_query_shape(const mla_dims* dims, int32_t batch, int32_t q_len, int32_t d_model,
                             int32_t q_lora_rank) {
    if (mla_status st = check_dims(dims); st != MLA_OK) return st;
    const mla_dims& d = *dims;
    if (d.act_dtype != MLA_BF16)
        return fail(MLA_ERR_UNSUPPORTED, "the query path needs act_dtype MLA_BF16");
    if (batch < 0 || q_len < 1 || q_len > 65536)
        return fail(MLA_ERR_BAD_SHAPE, "batch=%d must be >= 0 and q_len=%d in [1, 65536]", batch, q_len);
    if ((long long)batch * q_len > 65536)
        return fail(MLA_ERR_BAD_SHAPE, "batch * q_len = %lld exceeds 65536", (long long)batch * q_len);
    if (d_model < 64 || d_model > 65536 || d_model % 64)
        return fail(MLA_ERR_BAD_SHAPE, "d_model=%d must be a multiple of 64 in [64, 65536]", d_model);
    if (q_lora_rank < 0 || q_lora_rank > 2048 || q_lora_rank % 64)
        return fail(MLA_ERR_BAD_SHAPE, "q_lora_rank=%d must be 0 or a multiple of 64 up to 2048",
                    q_lora_rank);
    if ((d.n_heads * d.qk_nope_dim) % 32 || (d.n_heads * d.qk_rope_dim) % 32)
        return fail(MLA_ERR_UNSUPPORTED, "n_heads * qk_nope_dim and n_heads * qk_rope_dim must be "
                                         "multiples of 32");
    if (d.qk_rope_dim < 2)
        return fail(MLA_ERR_UNSUPPORTED, "the query path needs qk_rope_dim >= 2");
    const long long K = q_lora_rank ? q_lora_rank : d_model;
    if ((long long)batch * q_len * K * 2 >= (1ll << 31) ||
        (long long)d.n_heads * (d.qk_nope_dim + d.qk_rope_dim) * K * 2 >= (1ll << 31) ||
        (long long)q_lora_rank * d_model * 2 >= (1ll << 31))
        return fail(MLA_ERR_BAD_SHAPE, "a query-path operand exceeds 2 GiB");
    return MLA_OK;
}

struct QueryWs {
    size_t part, cq, total;
    int kc;
};

QueryWs query_ws(int batch, int q_len, int d_model, int q_lora_rank) {
    QueryWs w{};
    if (q_lora_rank == 0) return w;
    const size_t T = (size_t)batch * q_len;
    w.kc = mla::query_splits(q_lora_rank, d_model, (long long)T);
    w.part = 0;
    w.cq = align_up((size_t)w.kc * T * q_lora_rank * 4, 256);
    w.total = w.cq + align_up(T * q_lora_rank * 2, 256);
    return w;
}

// Prefill: shape checks shared by the sizing call and the entry point.
mla_status check_prefill_shape(const mla_dims* dims, int32_t batch, int32_t q_len,
                               int32_t max_blocks_per_seq) {
    if (mla_status st = check_dims(dims); st != MLA_OK) return st;
    const mla_dims& d = *dims;
    if (!mla::is_v3_shape(d))
        return fail(MLA_ERR_UNSUPPORTED, "the prefill serves the DeepSeek-V3 head shape "
                                         "(128 heads, 512 + 64, 128 / 128, blocks of 64, bf16 activations)");
    if (batch < 0 || q_len < 1 || q_len > (1 << 20))
        return fail(MLA_ERR_BAD_SHAPE, "batch=%d must be >= 0 and q_len=%d in [1, 2^20]", batch, q_len);
    if (max_blocks_per_seq < 1 || max_blocks_per_seq > (1 << 16))
        return fail(MLA_ERR_BAD_SHAPE, "max_blocks_per_seq=%d outside [1, 65536]", max_blocks_per_seq);
    if ((long long)batch * mla::prefill_tpad(max_blocks_per_seq) > (1ll << 22))
        return fail(MLA_ERR_BAD_SHAPE, "batch * max_blocks_per_seq * 64 exceeds 2^22 tokens");
    return MLA_OK;
}

struct PrefillWs {
    size_t x, kr, ts, kc, vv, total;
};

PrefillWs prefill_ws(int batch, int max_blocks) {
    const size_t rows = (size_t)batch * mla::prefill_tpad(max_blocks);
    PrefillWs w;
    w.x = 0;
    w.kr = align_up(rows * 512 * 2, 256);
    w.ts = w.kr + align_up(rows * 64 * 2, 256);
    w.kc = w.ts + align_up(rows * 4, 256);
    w.vv = w.kc + align_up(rows * 128 * 128 * 2, 256);
    w.total = w.vv + align_up(rows * 128 * 128 * 2, 256);
    return w;
}

mla_status prefill_impl(const mla_dims* dims, int32_t batch, int32_t q_len, const void* q_nope,
                        const void* q_pe, const void* w_uk, const void* w_uv, const void* cache_pool,
                        const float* cache_scale, const int32_t* block_table,
                        int32_t max_blocks_per_seq, const int32_t* seq_lens, void* out, float* lse,
                        void* workspace, size_t workspace_bytes, uint32_t stages, void* stream) {
    if (mla_status st = check_prefill_shape(dims, batch, q_len, max_blocks_per_seq); st != MLA_OK)
        return st;
    const mla_dims& d = *dims;
    if (stages == 0 || (stages & ~(uint32_t)MLA_PREFILL_ALL))
        return fail(MLA_ERR_BAD_SHAPE, "stages=0x%x: use MLA_PREFILL_* bits", stages);
    if (batch == 0) return ok();
    if ((stages & MLA_PREFILL_GATHER) && (!cache_pool || !block_table || !seq_lens))
        return fail(MLA_ERR_NULL_POINTER, "cache_pool, block_table and seq_lens are required");
    if ((stages & MLA_PREFILL_GATHER) && d.cache_dtype == MLA_FP8_E4M3 && !cache_scale)
        return fail(MLA_ERR_NULL_POINTER, "cache_scale is required for an FP8 cache");
    if ((stages & MLA_PREFILL_DECOMPRESS) && (!w_uk || !w_uv || !seq_lens))
        return fail(MLA_ERR_NULL_POINTER, "w_uk, w_uv and seq_lens are required");
    if ((stages & MLA_PREFILL_ATTEND) && (!q_nope || !q_pe || !out || !seq_lens))
        return fail(MLA_ERR_NULL_POINTER, "q_nope, q_pe, out and seq_lens are required");
    if (!workspace) return fail(MLA_ERR_NULL_POINTER, "workspace is NULL");
    const PrefillWs ws = prefill_ws(batch, max_blocks_per_seq);
    if (workspace_bytes < ws.total)
        return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes=%zu < %zu", workspace_bytes, ws.total);
    const void* ptrs[] = {q_nope, q_pe, w_uk, w_uv, cache_pool, out, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(MLA_ERR_ALIGNMENT, "tensor at %p is not 16-byte aligned", p);
    mla::PrefillLaunch a;
    a.cache_dtype = d.cache_dtype;
    a.scale = resolved_scale(d);
    a.batch = batch;
    a.q_len = q_len;
    a.q_nope = q_nope;
    a.q_pe = q_pe;
    a.w_uk = w_uk;
    a.w_uv = w_uv;
    a.pool = cache_pool;
    a.pool_scale = cache_scale;
    a.block_table = block_table;
    a.max_blocks = max_blocks_per_seq;
    a.seq_lens = seq_lens;
    a.out = out;
    a.lse = lse;
    char* base = static_cast<char*>(workspace);
    a.x = reinterpret_cast<unsigned short*>(base + ws.x);
    a.kr = reinterpret_cast<unsigned short*>(base + ws.kr);
    a.ts = reinterpret_cast<float*>(base + ws.ts);
    a.kc = reinterpret_cast<unsigned short*>(base + ws.kc);
    a.vv = reinterpret_cast<unsigned short*>(base + ws.vv);
    a.stages = stages;
    a.stream = static_cast<hipStream_t>(stream);
    const hipError_t e = mla::launch_prefill(a);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Output projection: shape checks shared by the sizing call and the entry point.
mla_status check_output_shape(int32_t rows, int32_t k, int32_t n) {
    if (rows < 0 || rows > 65536)
        return fail(MLA_ERR_BAD_SHAPE, "rows=%d outside [0, 65536]", rows);
    if (k < 64 || k % 64)
        return fail(MLA_ERR_BAD_SHAPE, "k=%d must be a positive multiple of 64", k);
    if (n < 32 || n % 32)
        return fail(MLA_ERR_BAD_SHAPE, "n=%d must be a positive multiple of 32", n);
    if ((long long)rows * k * 2 >= (1ll << 31) || (long long)n * k * 2 >= (1ll << 31))
        return fail(MLA_ERR_BAD_SHAPE, "an output-projection operand exceeds 2 GiB");
    return MLA_OK;
}

size_t output_ws_bytes(int32_t rows, int32_t k, int32_t n) {
    const int kc = mla::output_splits(n, k, rows);
    return align_up((size_t)kc * rows * n * 4, 256);
}

mla_status output_impl(int32_t rows, int32_t k, int32_t n, const void* x, const void* w, void* out,
                       void* workspace, size_t workspace_bytes, void* stream) {
    if (mla_status st = check_output_shape(rows, k, n); st != MLA_OK) return st;
    if (rows == 0) return ok();
    if (!x || !w || !out || !workspace)
        return fail(MLA_ERR_NULL_POINTER, "x, w, out and workspace are required");
    const void* ptrs[] = {x, w, out, workspace};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(MLA_ERR_ALIGNMENT, "tensor at %p is not 16-byte aligned", p);
    const size_t need = output_ws_bytes(rows, k, n);
    if (workspace_bytes < need)
        return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes=%zu < %zu", workspace_bytes, need);
    mla::OutputLaunch a;
    a.T = rows;
    a.K = k;
    a.N = n;
    a.x = x;
    a.w = w;
    a.out = out;
    a.part = static_cast<float*>(workspace);
    a.kc = mla::output_splits(n, k, rows);
    a.stream = static_cast<hipStream_t>(stream);
    const hipError_t e = mla::launch_output(a);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Decode followed by the output projection: the decode's output o stays in
// the workspace, after the decode's own scratch.
struct DecodeOutputWs {
    size_t decode, o, part, total;
};

DecodeOutputWs decode_output_ws(const mla_dims& d, int batch, int q_len, int num_splits, int d_model) {
    DecodeOutputWs w;
    const size_t R = (size_t)batch * q_len;
    w.decode = 0;
    w.o = align_up(decode_ws(d, batch, q_len, num_splits).total, 256);
    w.part = w.o + align_up(R * d.n_heads * d.v_head_dim * 2, 256);
    w.total = w.part + output_ws_bytes((int32_t)R, d.n_heads * d.v_head_dim, d_model);
    return w;
}

mla_status check_decode_output_shape(const mla_dims* dims, int32_t batch, int32_t q_len, int32_t num_splits,
                                     int32_t d_model) {
    if (mla_status st = check_dims(dims); st != MLA_OK) return st;
    if (dims->act_dtype != MLA_BF16)
        return fail(MLA_ERR_UNSUPPORTED, "the output projection needs act_dtype MLA_BF16");
    if (batch < 0 || q_len < 1 || q_len > 1024)
        return fail(MLA_ERR_BAD_SHAPE, "batch=%d must be >= 0 and q_len=%d in [1, 1024]", batch, q_len);
    if (num_splits < 0 || num_splits > mla::kMaxSplits)
        return fail(MLA_ERR_BAD_SHAPE, "num_splits=%d outside [0, %d]", num_splits, mla::kMaxSplits);
    return check_output_shape((int32_t)std::min<long long>((long long)batch * q_len, 65537),
                              dims->n_heads * dims->v_head_dim, d_model);
}

// Scratch of mla_decode_absorbed_noalloc: one array per GPU (each device
// holds its own copy), placed by the code object, never allocated by a call.
// In host code `scratch` names a host-side stand-in; the device address comes
// from hipGetSymbolAddress, once per device with that device current.
__device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

mla_status noalloc_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MLA_ERR_UNSUPPORTED, "device %d: at most %d devices are supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MLA_OK;
}

// Validates an append call and fills its launch description; *empty: nothing
// to launch (no new token).
mla_status append_prepare(const mla_dims* dims, int32_t batch, int32_t n_new, int32_t d_model,
                          const void* h, const void* w_kv_a, const void* kv_norm_gamma, float rms_eps,
                          float rope_base, const int32_t* block_table, int32_t max_blocks_per_seq,
                          const int32_t* start_pos, void* cache_pool, float* cache_scale, void* workspace,
                          size_t workspace_bytes, void* stream, mla::AppendLaunch& a, bool& mfma,
                          bool& empty) {
    empty = false;
    if (mla_status st = check_dims(dims); st != MLA_OK) return st;
    const mla_dims& d = *dims;
    if (batch < 0 || n_new < 0 || d_model < 1 || d_model % 8)
        return fail(MLA_ERR_BAD_SHAPE, "batch=%d n_new=%d d_model=%d (multiple of 8 required)", batch,
                    n_new, d_model);
    if (batch == 0 || n_new == 0) {
        empty = true;
        return ok();
    }
    if (!h || !w_kv_a || !kv_norm_gamma || !block_table || !start_pos || !cache_pool || !workspace)
        return fail(MLA_ERR_NULL_POINTER, "h, w_kv_a, kv_norm_gamma, block_table, start_pos, "
                                          "cache_pool and workspace are required");
    if (d.cache_dtype == MLA_FP8_E4M3 && !cache_scale)
        return fail(MLA_ERR_NULL_POINTER, "cache_scale is required for an FP8 cache");
    if (max_blocks_per_seq < 1) return fail(MLA_ERR_BAD_SHAPE, "max_blocks_per_seq must be >= 1");
    if (!(rms_eps >= 0.f) || !(rope_base > 0.f) || std::isinf(rope_base))
        return fail(MLA_ERR_BAD_SHAPE, "rms_eps must be >= 0 and rope_base finite and > 0");
    size_t need = 0;
    mla_cache_append_workspace_size(dims, batch, n_new, d_model, &need);
    if (workspace_bytes < need)
        return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes=%zu < %zu", workspace_bytes, need);
    mfma = append_uses_mfma(d, d_model);
    if (mfma && (!aligned16(h) || !aligned16(w_kv_a)))
        return fail(MLA_ERR_ALIGNMENT, "h and w_kv_a must be 16-byte aligned");
    if (!aligned16(workspace)) return fail(MLA_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
    a = mla::AppendLaunch{};
    a.DC = d.kv_lora_rank;
    a.DR = d.qk_rope_dim;
    a.BS = d.block_size;
    a.cache_dtype = d.cache_dtype;
    a.act_dtype = d.act_dtype;
    a.batch = batch;
    a.n_new = n_new;
    a.d_model = d_model;
    a.h = h;
    a.w_kv_a = w_kv_a;
    a.gamma = kv_norm_gamma;
    a.eps = rms_eps;
    a.rope_base = rope_base;
    a.block_table = block_table;
    a.max_blocks = max_blocks_per_seq;
    a.start_pos = start_pos;
    a.pool = cache_pool;
    a.pool_scale = cache_scale;
    a.part = static_cast<float*>(workspace);
    a.stream_gemm = mfma && append_streams(d, (long long)batch * n_new, d_model);
    a.kc = mfma ? append_slices(d, (long long)batch * n_new, d_model) : 1;
    a.kchunk = mfma ? mla::kAppendChunk : d_model;
    a.stream = static_cast<hipStream_t>(stream);
    return ok();
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
    switch (s) {
        case MLA_OK: return "MLA_OK";
        case MLA_ERR_NULL_POINTER: return "MLA_ERR_NULL_POINTER";
        case MLA_ERR_BAD_SHAPE: return "MLA_ERR_BAD_SHAPE";
        case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
        case MLA_ERR_ALIGNMENT: return "MLA_ERR_ALIGNMENT";
        case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
        case MLA_ERR_HIP: return "MLA_ERR_HIP";
        default: break;
    }
    return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error(void) { return g_err; }

size_t mla_cache_row_bytes(const mla_dims* d) {
    if (check_dims(d) != MLA_OK) return 0;
    return (size_t)(d->kv_lora_rank + d->qk_rope_dim) * elem_bytes(d->cache_dtype);
}

size_t mla_cache_block_bytes(const mla_dims* d) {
    const size_t row = mla_cache_row_bytes(d);
    return row ? row * (size_t)d->block_size : 0;
}

mla_status mla_cache_append_workspace_size(const mla_dims* dims, int32_t batch, int32_t n_new,
                                           int32_t d_model, size_t* bytes) {
    if (mla_status st = check_dims(dims); st != MLA_OK) return st;
    if (!bytes) return fail(MLA_ERR_NULL_POINTER, "bytes is NULL");
    if (batch < 0 || n_new < 0 || d_model < 1)
        return fail(MLA_ERR_BAD_SHAPE, "batch=%d n_new=%d d_model=%d", batch, n_new, d_model);
    const int kc = append_uses_mfma(*dims, d_model)
                       ? append_slices(*dims, (long long)batch * n_new, d_model) : 1;
    *bytes = align_up((size_t)kc * batch * n_new * (dims->kv_lora_rank + dims->qk_rope_dim) * 4, 256);
    return ok();
}

mla_status mla_cache_append(const mla_dims* dims, int32_t batch, int32_t n_new, int32_t d_model,
                            const void* h, const void* w_kv_a, const void* kv_norm_gamma,
                            float rms_eps, float rope_base, const int32_t* block_table,
                            int32_t max_blocks_per_seq, const int32_t* start_pos, void* cache_pool,
                            float* cache_scale, void* workspace, size_t workspace_bytes,
                            void* stream) {
    mla::AppendLaunch a;
    bool mfma = false, empty = false;
    if (mla_status st = append_prepare(dims, batch, n_new, d_model, h, w_kv_a, kv_norm_gamma, rms_eps,
                                       rope_base, block_table, max_blocks_per_seq, start_pos, cache_pool,
                                       cache_scale, workspace, workspace_bytes, stream, a, mfma, empty);
        st != MLA_OK || empty)
        return st;
    return launch_status(mla::launch_append(a, mfma));
}

int32_t mla_decode_default_splits(const mla_dims* dims, int32_t batch, int32_t q_len) {
    (void)dims;
    return default_splits(batch, q_len);
}

mla_status mla_decode_workspace_size(const mla_dims* dims, int32_t batch, int32_t q_len,
                                     int32_t num_splits, size_t* bytes) {
    if (mla_status st = check_dims(dims); st != MLA_OK) return st;
    if (!bytes) return fail(MLA_ERR_NULL_POINTER, "bytes is NULL");
    if (batch < 0 || q_len < 1 || q_len > 1024)
        return fail(MLA_ERR_BAD_SHAPE, "batch=%d q_len=%d", batch, q_len);
    if (num_splits < 0 || num_splits > mla::kMaxSplits)
        return fail(MLA_ERR_BAD_SHAPE, "num_splits=%d outside [0, %d]", num_splits, mla::kMaxSplits);
    *bytes = decode_ws(*dims, batch, q_len, num_splits).total;
    return ok();
}

mla_status mla_decode_absorbed(const mla_dims* dims, int32_t batch, int32_t q_len, const void* q_nope,
                               const void* q_pe, const void* w_uk, const void* w_uv,
                               const void* cache_pool, const float* cache_scale,
                               const int32_t* block_table, int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, int32_t num_splits, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(dims, batch, q_len, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale,
                       block_table, max_blocks_per_seq, seq_lens, num_splits, out, lse, workspace,
                       workspace_bytes, MLA_STAGE_ALL, stream);
}

mla_status mla_decode_absorbed_stages(const mla_dims* dims, int32_t batch, int32_t q_len,
                                      const void* q_nope, const void* q_pe, const void* w_uk,
                                      const void* w_uv, const void* cache_pool,
                                      const float* cache_scale, const int32_t* block_table,
                                      int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                      int32_t num_splits, void* out, float* lse, void* workspace,
                                      size_t workspace_bytes, uint32_t stages, void* stream) {
    return decode_impl(dims, batch, q_len, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale,
                       block_table, max_blocks_per_seq, seq_lens, num_splits, out, lse, workspace,
                       workspace_bytes, stages, stream);
}

mla_status mla_decode_absorbed_noalloc(const mla_dims* dims, int32_t batch, int32_t q_len,
                                       const void* q_nope, const void* q_pe, const void* w_uk,
                                       const void* w_uv, const void* cache_pool,
                                       const float* cache_scale, const int32_t* block_table,
                                       int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                       int32_t num_splits, void* out, float* lse, void* stream) {
    if (mla_status st = check_dims(dims); st != MLA_OK) return st;
    if (batch < 0 || q_len < 1 || q_len > 1024)
        return fail(MLA_ERR_BAD_SHAPE, "batch=%d must be >= 0 and q_len=%d in [1, 1024]", batch, q_len);
    if (num_splits < 0 || num_splits > mla::kMaxSplits)
        return fail(MLA_ERR_BAD_SHAPE, "num_splits=%d outside [0, %d]", num_splits, mla::kMaxSplits);
    if (batch == 0) return ok();
    const size_t need = decode_ws(*dims, batch, q_len, num_splits).total;
    if (need > MLA_NOALLOC_SCRATCH_BYTES)
        return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                    "this decode needs %zu bytes of scratch; the static scratch holds %zu "
                    "(use mla_decode_absorbed with a workspace)", need,
                    (size_t)MLA_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (mla_status st = noalloc_scratch(&ws); st != MLA_OK) return st;
    return decode_impl(dims, batch, q_len, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale,
                       block_table, max_blocks_per_seq, seq_lens, num_splits, out, lse, ws,
                       MLA_NOALLOC_SCRATCH_BYTES, MLA_STAGE_ALL, stream);
}

mla_status mla_check_block_table(const mla_dims* dims, int32_t batch, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_blocks,
                                 int32_t* report, void* stream) {
    if (mla_status st = check_dims(dims); st != MLA_OK) return st;
    if (batch < 0 || max_blocks_per_seq < 1 || num_blocks < 0)
        return fail(MLA_ERR_BAD_SHAPE, "batch=%d max_blocks_per_seq=%d num_blocks=%d", batch,
                    max_blocks_per_seq, num_blocks);
    if (!report) return fail(MLA_ERR_NULL_POINTER, "report is NULL");
    if (batch > 0 && (!block_table || !seq_lens))
        return fail(MLA_ERR_NULL_POINTER, "block_table and seq_lens are required");
    const hipError_t e = mla::launch_check_block_table(block_table, batch, max_blocks_per_seq, seq_lens,
                                                       dims->block_size, num_blocks, report,
                                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

mla_status mla_output_workspace_size(int32_t rows, int32_t k, int32_t n, size_t* bytes) {
    if (mla_status st = check_output_shape(rows, k, n); st != MLA_OK) return st;
    if (!bytes) return fail(MLA_ERR_NULL_POINTER, "bytes is NULL");
    *bytes = output_ws_bytes(rows, k, n);
    return ok();
}

mla_status mla_output_project(int32_t rows, int32_t k, int32_t n, const void* x, const void* w, void* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
    return output_impl(rows, k, n, x, w, out, workspace, workspace_bytes, stream);
}

mla_status mla_decode_output_workspace_size(const mla_dims* dims, int32_t batch, int32_t q_len,
                                            int32_t num_splits, int32_t d_model, size_t* bytes) {
    if (mla_status st = check_decode_output_shape(dims, batch, q_len, num_splits, d_model); st != MLA_OK)
        return st;
    if (!bytes) return fail(MLA_ERR_NULL_POINTER, "bytes is NULL");
    *bytes = decode_output_ws(*dims, batch, q_len, num_splits, d_model).total;
    return ok();
}

mla_status mla_decode_output(const mla_dims* dims, int32_t batch, int32_t q_len, const void* q_nope,
                             const void* q_pe, const void* w_uk, const void* w_uv, const void* cache_pool,
                             const float* cache_scale, const int32_t* block_table,
                             int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_splits,
                             int32_t d_model, const void* w_o, void* u, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (mla_status st = check_decode_output_shape(dims, batch, q_len, num_splits, d_model); st != MLA_OK)
        return st;
    if (batch == 0) return ok();
    if (!w_o || !u || !workspace) return fail(MLA_ERR_NULL_POINTER, "w_o, u and workspace are required");
    const DecodeOutputWs ws = decode_output_ws(*dims, batch, q_len, num_splits, d_model);
    if (workspace_bytes < ws.total)
        return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes=%zu < %zu", workspace_bytes, ws.total);
    char* base = static_cast<char*>(workspace);
    void* o = base + ws.o;
    if (mla_status st = decode_impl(dims, batch, q_len, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale,
                                    block_table, max_blocks_per_seq, seq_lens, num_splits, o, lse,
                                    base + ws.decode, ws.o - ws.decode, MLA_STAGE_ALL, stream);
        st != MLA_OK)
        return st;
    const int32_t R = batch * q_len;
    return output_impl(R, dims->n_heads * dims->v_head_dim, d_model, o, w_o, u, base + ws.part,
                       ws.total - ws.part, stream);
}

mla_status mla_query_workspace_size(const mla_dims* dims, int32_t batch, int32_t q_len,
                                   int32_t d_model, int32_t q_lora_rank, size_t* bytes) {
    if (mla_status st = check_query_shape(dims, batch, q_len, d_model, q_lora_rank); st != MLA_OK)
        return st;
    if (!bytes) return fail(MLA_ERR_NULL_POINTER, "bytes is NULL");
    *bytes = query_ws(batch, q_len, d_model, q_lora_rank).total;
    return ok();
}

mla_status mla_query_project(const mla_dims* dims, int32_t batch, int32_t q_len, int32_t d_model,
                             int32_t q_lora_rank, const void* h, const void* w_dq,
                             const void* q_norm_gamma, float rms_eps, const void* w_uq,
                             const void* w_qr, float rope_base, const int32_t* start_pos,
                             void* q_nope, void* q_pe, void* workspace, size_t workspace_bytes,
                             void* stream) {
    if (mla_status st = check_query_shape(dims, batch, q_len, d_model, q_lora_rank); st != MLA_OK)
        return st;
    const mla_dims& d = *dims;
    if (!(rms_eps >= 0.f) || !(rope_base > 0.f) || std::isinf(rope_base))
        return fail(MLA_ERR_BAD_SHAPE, "rms_eps must be >= 0 and rope_base finite and > 0");
    if (q_lora_rank == 0 && (w_dq || q_norm_gamma))
        return fail(MLA_ERR_BAD_SHAPE, "q_lora_rank 0 (full-rank queries) takes no w_dq or q_norm_gamma");
    if (batch == 0) return ok();
    if (!h || !w_uq || !w_qr || !start_pos || !q_nope || !q_pe)
        return fail(MLA_ERR_NULL_POINTER, "h, w_uq, w_qr, start_pos, q_nope and q_pe are required");
    if (q_lora_rank > 0 && (!w_dq || !workspace))
        return fail(MLA_ERR_NULL_POINTER, "w_dq and workspace are required when q_lora_rank > 0");
    const QueryWs ws = query_ws(batch, q_len, d_model, q_lora_rank);
    if (workspace_bytes < ws.total)
        return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes=%zu < %zu", workspace_bytes, ws.total);
    const void* ptrs[] = {h, w_dq, w_uq, w_qr, q_nope, q_pe, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(MLA_ERR_ALIGNMENT, "tensor at %p is not 16-byte aligned", p);
    mla::QueryLaunch a;
    a.H = d.n_heads;
    a.N = d.qk_nope_dim;
    a.R = d.qk_rope_dim;
    a.T = batch * q_len;
    a.q_len = q_len;
    a.d_model = d_model;
    a.q_lora = q_lora_rank;
    a.h = h;
    a.w_dq = w_dq;
    a.gamma = q_norm_gamma;
    a.eps = rms_eps;
    a.rope_base = rope_base;
    a.w_uq = w_uq;
    a.w_qr = w_qr;
    a.start_pos = start_pos;
    a.q_nope = q_nope;
    a.q_pe = q_pe;
    char* base = static_cast<char*>(workspace);
    a.part = q_lora_rank ? reinterpret_cast<float*>(base + ws.part) : nullptr;
    a.kc = ws.kc;
    a.cq = q_lora_rank ? reinterpret_cast<unsigned short*>(base + ws.cq) : nullptr;
    a.stream = static_cast<hipStream_t>(stream);
    const hipError_t e = mla::launch_query(a);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

mla_status mla_prefill_workspace_size(const mla_dims* dims, int32_t batch, int32_t q_len,
                                      int32_t max_blocks_per_seq, size_t* bytes) {
    if (!bytes) return fail(MLA_ERR_NULL_POINTER, "bytes is NULL");
    if (mla_status st = check_prefill_shape(dims, batch, q_len, max_blocks_per_seq); st != MLA_OK)
        return st;
    *bytes = prefill_ws(batch, max_blocks_per_seq).total;
    return ok();
}

mla_status mla_prefill(const mla_dims* dims, int32_t batch, int32_t q_len, const void* q_nope,
                       const void* q_pe, const void* w_uk, const void* w_uv, const void* cache_pool,
                       const float* cache_scale, const int32_t* block_table,
                       int32_t max_blocks_per_seq, const int32_t* seq_lens, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(dims, batch, q_len, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale,
                        block_table, max_blocks_per_seq, seq_lens, out, lse, workspace,
                        workspace_bytes, MLA_PREFILL_ALL, stream);
}

mla_status mla_prefill_stages(const mla_dims* dims, int32_t batch, int32_t q_len, const void* q_nope,
                              const void* q_pe, const void* w_uk, const void* w_uv,
                              const void* cache_pool, const float* cache_scale,
                              const int32_t* block_table, int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, uint32_t stages, void* stream) {
    return prefill_impl(dims, batch, q_len, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale,
                        block_table, max_blocks_per_seq, seq_lens, out, lse, workspace,
                        workspace_bytes, stages, stream);
}

mla_status mla_decode_step_workspace_size(const mla_dims* dims, int32_t batch, int32_t q_len,
                                          int32_t d_model, int32_t num_splits, size_t* bytes) {
    if (!bytes) return fail(MLA_ERR_NULL_POINTER, "bytes is NULL");
    size_t dec = 0, app = 0;
    if (mla_status st = mla_decode_workspace_size(dims, batch, q_len, num_splits, &dec); st != MLA_OK)
        return st;
    if (mla_status st = mla_cache_append_workspace_size(dims, batch, q_len, d_model, &app); st != MLA_OK)
        return st;
    *bytes = align_up(dec, 256) + app;
    return ok();
}

mla_status mla_decode_step_stages(const mla_dims* dims, int32_t batch, int32_t q_len, int32_t d_model,
                                  const void* h, const void* w_kv_a, const void* kv_norm_gamma,
                                  float rms_eps, float rope_base, const int32_t* start_pos,
                                  const void* q_nope, const void* q_pe, const void* w_uk,
                                  const void* w_uv, void* cache_pool, float* cache_scale,
                                  const int32_t* block_table, int32_t max_blocks_per_seq,
                                  const int32_t* seq_lens, int32_t num_splits, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, uint32_t stages,
                                  void* stream) {
    if (stages == 0 || (stages & ~(uint32_t)MLA_STEP_ALL))
        return fail(MLA_ERR_BAD_SHAPE, "stages=0x%x: use MLA_STEP_* bits", stages);
    size_t need = 0;
    if (mla_status st = mla_decode_step_workspace_size(dims, batch, q_len, d_model, num_splits, &need);
        st != MLA_OK)
        return st;
    if (batch == 0) return ok();
    if (!workspace) return fail(MLA_ERR_NULL_POINTER, "workspace is NULL");
    if (workspace_bytes < need)
        return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes=%zu < %zu", workspace_bytes, need);
    size_t dec_bytes = 0;
    mla_decode_workspace_size(dims, batch, q_len, num_splits, &dec_bytes);
    dec_bytes = align_up(dec_bytes, 256);
    char* ws = static_cast<char*>(workspace);
    mla::AppendLaunch ap;
    bool app_mfma = false, app_empty = false;
    if (mla_status st = append_prepare(dims, batch, q_len, d_model, h, w_kv_a, kv_norm_gamma, rms_eps,
                                       rope_base, block_table, max_blocks_per_seq, start_pos, cache_pool,
                                       cache_scale, ws + dec_bytes, workspace_bytes - dec_bytes, stream, ap,
                                       app_mfma, app_empty);
        st != MLA_OK)
        return st;
    mla::DecodeLaunch dp;
    bool dec_mfma = false, dec_empty = false;
    if (mla_status st = decode_prepare(dims, batch, q_len, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale,
                                       block_table, max_blocks_per_seq, seq_lens, num_splits, out, lse, ws,
                                       dec_bytes, MLA_STAGE_ALL, stream, dp, dec_mfma, dec_empty);
        st != MLA_OK)
        return st;
    auto decode = [&](unsigned st) {
        return dec_mfma ? mla::launch_decode_mfma(dp, st) : mla::launch_decode_generic(dp, st);
    };
    if (stages & MLA_STEP_PROJECT)
        if (hipError_t e = mla::launch_append_project(ap, app_mfma); e != hipSuccess) return launch_status(e);
    if (stages & MLA_STEP_FINALIZE_ABSORB) {
        if (dec_mfma) {                  // bf16 activations, V3 shape: one launch
            if (hipError_t e = mla::launch_finalize_absorb(ap, dp); e != hipSuccess) return launch_status(e);
        } else {
            if (hipError_t e = mla::launch_append_finalize(ap); e != hipSuccess) return launch_status(e);
            if (hipError_t e = decode(MLA_STAGE_ABSORB_Q); e != hipSuccess) return launch_status(e);
        }
    }
    const unsigned rest = ((stages & MLA_STEP_SPLIT_KV) ? MLA_STAGE_SPLIT_KV : 0u) |
                          ((stages & MLA_STEP_COMBINE) ? MLA_STAGE_COMBINE : 0u);
    if (rest) return launch_status(decode(rest));
    return ok();
}

mla_status mla_decode_step(const mla_dims* dims, int32_t batch, int32_t q_len, int32_t d_model,
                           const void* h, const void* w_kv_a, const void* kv_norm_gamma,
                           float rms_eps, float rope_base, const int32_t* start_pos,
                           const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                           void* cache_pool, float* cache_scale, const int32_t* block_table,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_splits,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
    return mla_decode_step_stages(dims, batch, q_len, d_model, h, w_kv_a, kv_norm_gamma, rms_eps, rope_base,
                                  start_pos, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale, block_table,
                                  max_blocks_per_seq, seq_lens, num_splits, out, lse, workspace,
                                  workspace_bytes, MLA_STEP_ALL, stream);
}

}  // extern "C"

// Host-side launch interface between the C ABI layer (api.hip) and the
// kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

// MI355X compute units; the default split count aims to give every CU work.
constexpr int kNumCUs = 256;
constexpr int kMaxSplits = 256;
constexpr int kAppendChunk = 256;     // d_model columns per split-K chunk of the MFMA projection

struct DecodeLaunch {
    // shape
    int H, DC, DR, N, V, BS;
    int cache_dtype, act_dtype;
    float scale;                 // softmax scale (natural units)
    int batch, q_len, num_splits;
    // tensors
    const void* q_nope;
    const void* q_pe;
    const void* w_uk;
    const void* w_uv;
    const void* pool;
    const float* pool_scale;
    const int32_t* block_table;
    int max_blocks;
    const int32_t* seq_lens;
    void* out;
    float* lse;
    // workspace carve-up
    void* qbuf;                  // [R][H][DC+DR]: bf16 in the split-KV kernels' fragment order
                                 // (MFMA path, q_frag_offset) or f32 row-major (portable)
    void* part_o;                // [R][S][H][DC]: fp16 on the MFMA path, fp32 otherwise
    float* part_lse;             // [R][S][H]
    hipStream_t stream;
};

struct AppendLaunch {
    int DC, DR, BS;
    int cache_dtype, act_dtype;
    int batch, n_new, d_model;
    const void* h;
    const void* w_kv_a;
    const void* gamma;
    float eps, rope_base;
    const int32_t* block_table;
    int max_blocks;
    const int32_t* start_pos;
    void* pool;
    float* pool_scale;
    float* part;                 // [KC][T][DC+DR] f32
    int kc;                      // partial slices in `part`
    int kchunk;                  // d_model columns per chunk (split-K kernel)
    bool stream_gemm = false;    // projection on the weight-streaming GEMM
    hipStream_t stream;
};

bool is_v3_shape(const mla_dims& d);

hipError_t launch_decode_mfma(const DecodeLaunch& a, unsigned stages);
hipError_t launch_decode_generic(const DecodeLaunch& a, unsigned stages);
hipError_t launch_append(const AppendLaunch& a, bool mfma_gemm);
// the append's two launches on their own: the projection into the partial
// sums, then the per-token finalize (launch_append runs both)
hipError_t launch_append_project(const AppendLaunch& a, bool mfma_gemm);
hipError_t launch_append_finalize(const AppendLaunch& a);
// the append's finalize and the decode's query absorption as one launch
// (bf16 activations, V3 decode shape; they are independent of each other)
hipError_t launch_finalize_absorb(const AppendLaunch& ap, const DecodeLaunch& dp);
hipError_t launch_check_block_table(const int* block_table, int batch, int max_blocks, const int* seq_lens,
                                    int block_size, int num_blocks, int* report, hipStream_t stream);

}  // namespace mla

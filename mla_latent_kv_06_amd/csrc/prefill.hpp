// Host-side launch interface of the prefill (prefill.hip).  Not part of the
// public ABI.
#pragma once

#include "internal.hpp"

namespace mla {

struct PrefillLaunch {
    int cache_dtype;
    float scale;                 // softmax scale (natural units)
    int batch, q_len;
    const void* q_nope;          // [batch][q_len][128][128] bf16
    const void* q_pe;            // [batch][q_len][128][64] bf16
    const void* w_uk;            // [128][128][512] bf16
    const void* w_uv;            // [128][128][512] bf16
    const void* pool;
    const float* pool_scale;
    const int32_t* block_table;
    int max_blocks;
    const int32_t* seq_lens;
    void* out;                   // [batch][q_len][128][128] bf16
    float* lse;                  // [batch][q_len][128]
    // workspace carve-up (rows of sequence b start at b * prefill_tpad)
    unsigned short* x;           // [batch][Tpad][512] gathered latents
    unsigned short* kr;          // [batch][Tpad][64] rotary keys
    float* ts;                   // [batch][Tpad] token scales (fp8 cache)
    unsigned short* kc;          // [batch][128][Tpad][128] content keys
    unsigned short* vv;          // [batch][128][Tpad][128] values
    unsigned stages;             // bits: 1 gather, 2 decompress, 4 attention
    hipStream_t stream;
};

// Workspace rows per sequence: max_blocks * 64 rounded up to 256 (the rebuild tile).
int prefill_tpad(int max_blocks);
hipError_t launch_prefill(const PrefillLaunch& a);

}  // namespace mla

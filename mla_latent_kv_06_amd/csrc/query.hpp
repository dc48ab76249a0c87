// Host-side launch interface of the query path (query.hip).  Not part of the
// public ABI.
#pragma once

#include "internal.hpp"

namespace mla {

struct QueryLaunch {
    int H, N, R;                 // heads, content and rotary query widths per head
    int T, q_len;                // query rows (batch * q_len) and rows per sequence
    int d_model, q_lora;         // q_lora == 0: full-rank queries (no compression)
    const void* h;               // [T][d_model] bf16
    const void* w_dq;            // [q_lora][d_model] bf16
    const void* gamma;           // [q_lora] bf16, or NULL: no latent norm
    float eps, rope_base;
    const void* w_uq;            // [H N][q_lora or d_model] bf16
    const void* w_qr;            // [H R][q_lora or d_model] bf16
    const int32_t* start_pos;    // [batch]: position of each sequence's first query row
    void* q_nope;                // [T][H][N] bf16
    void* q_pe;                  // [T][H][R] bf16
    float* part;                 // [kc][T][q_lora] f32 split-K partial sums
    int kc;                      // depth splits in `part` (query_splits)
    unsigned short* cq;          // [T][q_lora] bf16 compressed queries
    hipStream_t stream;
};

hipError_t launch_query(const QueryLaunch& a);

// Depth splits of the query down-projection for T rows (workspace partial
// slices).
int query_splits(int q_lora, int d_model, long long T);
// Depth splits of the cache append's projection on the weight-streaming
// GEMM for T rows (which needs d_model a multiple of 64 and operands under
// 2 GiB).
int append_stream_splits(int Dout, int d_model, long long T);

}  // namespace mla

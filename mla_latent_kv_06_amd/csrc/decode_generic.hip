// Portable absorbed-MLA decode for shapes outside the MFMA path (any head
// count and widths within the documented limits; f32 or bf16 activations;
// f32, bf16 or fp8 cache).  Plain fp32 VALU arithmetic, same three stages and
// workspace layout as the MFMA path:
//   absorb:  qbuf[r][h] = [W_UK[h]^T q_nope[r,h] ; q_pe[r,h]]      (fp32)
//   split:   per (row, partition, head) online softmax over the partition
//   combine: log-sum-exp merge, then W_UV[h] o_lat

#include "common.hpp"
#include "internal.hpp"

namespace mla {
namespace {

constexpr int NT = 256;
constexpr int MAX_PER_THREAD = 4;     // latent columns per thread (d_c <= 1024)

template <int CDT>
__device__ __forceinline__ float cache_val(const void* pool, const float* pscale, size_t phys,
                                           int D, int c, int bs) {
    if constexpr (CDT == MLA_FP8_E4M3) {
        const unsigned char code = static_cast<const unsigned char*>(pool)[phys * D + c];
        return e4m3_to_f32(code) * pscale[phys];
    } else if constexpr (CDT == MLA_BF16) {
        return bf16_bits_to_f32(static_cast<const unsigned short*>(pool)[cache_offset(phys, c, D)]);
    } else {
        return static_cast<const float*>(pool)[phys * D + c];
    }
}

// grid: R * H.  qbuf[(r*H + h)*(DC+DR) + c]
template <int ADT>
__global__ __launch_bounds__(NT) void g_absorb(const void* __restrict__ q_nope,
                                               const void* __restrict__ q_pe,
                                               const void* __restrict__ w_uk,
                                               float* __restrict__ qbuf, int H, int N, int DC,
                                               int DR) {
    __shared__ float qn[512];
    const int r = blockIdx.x / H, h = blockIdx.x % H;
    const size_t qi = (size_t)r * H + h;
    for (int n = threadIdx.x; n < N; n += NT) qn[n] = load_act<ADT>(q_nope, qi * N + n);
    __syncthreads();
    float* dst = qbuf + qi * (DC + DR);
    for (int c = threadIdx.x; c < DC; c += NT) {
        float acc = 0.f;
        for (int n = 0; n < N; ++n) acc += load_act<ADT>(w_uk, ((size_t)h * N + n) * DC + c) * qn[n];
        dst[c] = acc;
    }
    for (int k = threadIdx.x; k < DR; k += NT) dst[DC + k] = load_act<ADT>(q_pe, qi * DR + k);
}

// grid: R * S * H (head fastest).  One workgroup owns one (row, partition,
// head); tokens are processed 256 at a time: one score per thread, a
// block-wide max / sum, then every thread accumulates its latent columns.
template <int CDT>
__global__ __launch_bounds__(NT) void g_split(
    const float* __restrict__ qbuf, const void* __restrict__ pool, const float* __restrict__ pscale,
    const int* __restrict__ block_table, int max_blocks, const int* __restrict__ seq_lens,
    int q_len, int num_splits, int H, int DC, int DR, int BSZ, float scale,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
    __shared__ float q[1280];
    __shared__ float pw[NT];
    __shared__ long long prow[NT];
    __shared__ float red[16];
    const int h = blockIdx.x % H;
    const int rs = blockIdx.x / H;
    const int split = rs % num_splits, row = rs / num_splits;
    const int b = row / q_len, s = row % q_len;
    const int D = DC + DR;
    const int n_vis = seq_lens[b] - q_len + s + 1;
    const size_t oi = ((size_t)row * num_splits + split) * H + h;
    // partition of P tokens, P a multiple of the block size
    const long long per = n_vis > 0
        ? (long long)((n_vis + (long long)num_splits * BSZ - 1) / ((long long)num_splits * BSZ)) * BSZ
        : 0;
    const long long j0 = (long long)split * per;
    const long long j1 = min((long long)n_vis, j0 + per);
    if (j0 >= j1) {
        if (threadIdx.x == 0) part_lse[oi] = kNegInf;
        return;
    }
    for (int c = threadIdx.x; c < D; c += NT) q[c] = qbuf[((size_t)row * H + h) * D + c];
    __syncthreads();
    const int* btab = block_table + (size_t)b * max_blocks;
    float acc[MAX_PER_THREAD] = {};
    float m = kNegInf, l = 0.f;
    for (long long jb = j0; jb < j1; jb += NT) {
        const long long j = jb + threadIdx.x;
        float sc = kNegInf;
        if (j < j1) {
            const size_t phys = (size_t)btab[j / BSZ] * BSZ + (size_t)(j % BSZ);
            prow[threadIdx.x] = (long long)phys;
            float dot = 0.f;
            for (int c = 0; c < D; ++c) dot += q[c] * cache_val<CDT>(pool, pscale, phys, D, c, BSZ);
            sc = dot * scale;
        }
        const float cmax = block_max(sc, red);
        const float m_new = fmaxf(m, cmax);
        const float alpha = __expf(m - m_new);
        const float p = (j < j1) ? __expf(sc - m_new) : 0.f;
        pw[threadIdx.x] = p;
        const float psum = block_sum(p, red);      // also orders the pw / prow writes
        l = l * alpha + psum;
        m = m_new;
        const int cnt = (int)min((long long)NT, j1 - jb);
#pragma unroll
        for (int k = 0; k < MAX_PER_THREAD; ++k) acc[k] *= alpha;
        for (int jj = 0; jj < cnt; ++jj) {
            const float pj = pw[jj];
            const size_t phys = (size_t)prow[jj];
#pragma unroll
            for (int k = 0; k < MAX_PER_THREAD; ++k) {
                const int c = threadIdx.x + k * NT;
                if (c < DC) acc[k] += pj * cache_val<CDT>(pool, pscale, phys, D, c, BSZ);
            }
        }
        __syncthreads();
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int k = 0; k < MAX_PER_THREAD; ++k) {
        const int c = threadIdx.x + k * NT;
        if (c < DC) part_o[oi * DC + c] = acc[k] * inv;
    }
    if (threadIdx.x == 0) part_lse[oi] = m + __logf(l);
}

// grid: R * H.
template <int ADT>
__global__ __launch_bounds__(NT) void g_combine(const float* __restrict__ part_o,
                                                const float* __restrict__ part_lse, int num_splits,
                                                int H, int DC, int V, const void* __restrict__ w_uv,
                                                void* __restrict__ out, float* __restrict__ lse_out) {
    __shared__ float ol[1024];
    const int row = blockIdx.x / H, h = blockIdx.x % H;
    float mx = kNegInf;
    for (int s = 0; s < num_splits; ++s)
        mx = fmaxf(mx, part_lse[((size_t)row * num_splits + s) * H + h]);
    float tot = 0.f;
    for (int c = threadIdx.x; c < DC; c += NT) ol[c] = 0.f;
    if (mx != kNegInf) {
        for (int s = 0; s < num_splits; ++s) {
            const size_t oi = ((size_t)row * num_splits + s) * H + h;
            const float ls = part_lse[oi];
            if (ls == kNegInf) continue;
            const float wt = __expf(ls - mx);
            tot += wt;
            for (int c = threadIdx.x; c < DC; c += NT) ol[c] += wt * part_o[oi * DC + c];
        }
    }
    const float inv = tot > 0.f ? 1.0f / tot : 0.f;
    for (int c = threadIdx.x; c < DC; c += NT) ol[c] *= inv;
    __syncthreads();
    for (int v = threadIdx.x; v < V; v += NT) {
        float acc = 0.f;
        for (int c = 0; c < DC; ++c) acc += load_act<ADT>(w_uv, ((size_t)h * V + v) * DC + c) * ol[c];
        store_act<ADT>(out, ((size_t)row * H + h) * V + v, acc);
    }
    if (lse_out != nullptr && threadIdx.x == 0)
        lse_out[(size_t)row * H + h] = (mx == kNegInf) ? kNegInf : mx + __logf(tot);
}

template <int ADT, int CDT>
hipError_t run(const DecodeLaunch& a, unsigned stages) {
    const int R = a.batch * a.q_len;
    float* qbuf = static_cast<float*>(a.qbuf);
    if (stages & MLA_STAGE_ABSORB_Q) {
        g_absorb<ADT><<<R * a.H, NT, 0, a.stream>>>(a.q_nope, a.q_pe, a.w_uk, qbuf, a.H, a.N, a.DC,
                                                    a.DR);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    if (stages & MLA_STAGE_SPLIT_KV) {
        g_split<CDT><<<R * a.num_splits * a.H, NT, 0, a.stream>>>(
            qbuf, a.pool, a.pool_scale, a.block_table, a.max_blocks, a.seq_lens, a.q_len,
            a.num_splits, a.H, a.DC, a.DR, a.BS, a.scale, static_cast<float*>(a.part_o), a.part_lse);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    if (stages & MLA_STAGE_COMBINE) {
        g_combine<ADT><<<R * a.H, NT, 0, a.stream>>>(static_cast<const float*>(a.part_o), a.part_lse,
                                                    a.num_splits, a.H, a.DC,
                                                     a.V, a.w_uv, a.out, a.lse);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_decode_generic(const DecodeLaunch& a, unsigned stages) {
    if (a.batch * a.q_len == 0) return hipSuccess;
    if (a.act_dtype == MLA_BF16) {
        if (a.cache_dtype == MLA_BF16) return run<MLA_BF16, MLA_BF16>(a, stages);
        if (a.cache_dtype == MLA_FP8_E4M3) return run<MLA_BF16, MLA_FP8_E4M3>(a, stages);
        return run<MLA_BF16, MLA_F32>(a, stages);
    }
    if (a.cache_dtype == MLA_BF16) return run<MLA_F32, MLA_BF16>(a, stages);
    if (a.cache_dtype == MLA_FP8_E4M3) return run<MLA_F32, MLA_FP8_E4M3>(a, stages);
    return run<MLA_F32, MLA_F32>(a, stages);
}

}  // namespace mla

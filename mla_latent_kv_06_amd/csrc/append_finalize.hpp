// The cache append's last step for one new token (device code only, included
// by the kernels that run it): the split-K partial sums of x = W_kv,a h are
// added in a fixed order, then [RMSNorm(x[0:d_c]) * gamma ; RoPE(x[d_c:],
// position)] is rounded and stored into the token's paged slot ("KV
// Compression -- DeepSeek-V3", "How it works").
#pragma once

#include "common.hpp"

namespace mla {
namespace {

// Token t of the append, one workgroup of 256 threads.  Dout = DC + DR <= 1280
// (dims are validated).
//
// Everything that does not depend on the projection is started first so that
// its latency overlaps the partial loads: the token's position and cache
// slot, gamma, and the rotary sine / cosine.  RoPE turns pairs (x[2k],
// x[2k+1]) by pos * base^(-2k/R); the angle needs double precision (at
// position 2^17 an fp32 angle is off by up to 1/64 rad), so it is formed in
// double, reduced modulo 2 pi with one fma against the double nearest 2 pi
// (error below 1e-11 rad for positions under 2^20), and its fp32 sin / cos
// taken.  The split-K partials are summed chunk by chunk in increasing order.
template <int ADT, int CDT>
__device__ __forceinline__ void append_finalize_token(
    int t, const float* __restrict__ part, int kc_count, int T, int DC, int DR,
    const void* __restrict__ gamma, float eps, float rope_base,
    const int* __restrict__ block_table, int max_blocks, const int* __restrict__ start_pos,
    int n_new, int BSZ, void* __restrict__ pool, float* __restrict__ pool_scale) {
    __shared__ float y[1280];
    __shared__ float rsn[128], rcs[128];
    __shared__ float red[16];
    const int tid = threadIdx.x;
    const int Dout = DC + DR;
    const int b = t / n_new;
    const int pos = start_pos[b] + (t - b * n_new);
    const size_t phys = (size_t)block_table[(size_t)b * max_blocks + pos / BSZ] * BSZ + pos % BSZ;

    // Loads below are unconditional, at clamped (valid) addresses, with the
    // unused values selected away afterwards: a load under a branch would be
    // waited for inside that branch, one round trip each.
    if (Dout % 4 == 0 && DC % 2 == 0 && Dout <= 4 * 256 && kc_count <= 32) {
        // common shapes: thread tid owns outputs 4 tid .. 4 tid + 3 (16-byte
        // partial loads, every one in flight at once; a rotary pair (x[2k],
        // x[2k+1]) sits in one thread)
        const int o0 = 4 * tid, oc = min(o0, Dout - 4);
        const float keep_o = o0 < Dout ? 1.f : 0.f;
        f32x4 pv[32];
#pragma unroll
        for (int kc = 0; kc < 32; ++kc)
            pv[kc] = *reinterpret_cast<const f32x4*>(part + ((size_t)min(kc, kc_count - 1) * T + t) * Dout + oc);
        float g4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            g4[e] = load_act<ADT>(gamma, min(o0 + e, DC - 1)) * (o0 + e < DC ? 1.f : 0.f);
        if (tid < DR / 2) {
            const double ang = (double)pos * pow((double)rope_base, -2.0 * tid / (double)DR);
            const double turns = rint(ang * 0.15915494309189535);
            sincosf((float)fma(-turns, 6.283185307179586, ang), &rsn[tid], &rcs[tid]);
        }
        float x4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 32; ++kc) {
            const float keep = kc < kc_count ? keep_o : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) x4[e] += pv[kc][e] * keep;
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (o0 + e < DC) ss += x4[e] * x4[e];
        ss = block_sum(ss, red);                // also publishes rsn[], rcs[]
        const float inv = 1.0f / sqrtf(ss / (float)DC + eps);
        float yo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int o = o0 + e;
            if (o < DC) {
                yo[e] = x4[e] * inv * g4[e];
            } else {
                const int k = min((o - DC) >> 1, 127);
                const float x0 = x4[e & ~1], x1 = x4[e | 1];
                yo[e] = (e & 1) ? x0 * rsn[k] + x1 * rcs[k] : x0 * rcs[k] - x1 * rsn[k];
            }
        }
        if constexpr (CDT == MLA_FP8_E4M3) {
            float amax = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(yo[e]) * keep_o);
            amax = block_max(amax, red);
            const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
            unsigned int codes = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) codes |= (unsigned int)f32_to_e4m3_rne_sat(yo[e] / sc) << (8 * e);
            if (o0 < Dout)
                *reinterpret_cast<unsigned int*>(static_cast<unsigned char*>(pool) + phys * Dout + o0) = codes;
            if (tid == 0) pool_scale[phys] = sc;
        } else if constexpr (CDT == MLA_BF16) {
            // the token's row is contiguous: four outputs, one 8-byte store
            if (o0 < Dout) {
                u16x4 hv;
#pragma unroll
                for (int e = 0; e < 4; ++e) hv[e] = f32_to_bf16_bits(yo[e]);
                *reinterpret_cast<u16x4*>(static_cast<unsigned short*>(pool) + cache_offset(phys, o0, Dout)) = hv;
            }
        } else if (o0 < Dout) {
#pragma unroll
            for (int e = 0; e < 4; ++e) store_act<CDT>(pool, cache_offset(phys, o0 + e, Dout), yo[e]);
        }
        return;
    }
    constexpr int U = 5;                        // outputs per thread: o = tid + 256 u
    float gm[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int o = tid + 256 * u;
        gm[u] = load_act<ADT>(gamma, min(o, DC - 1)) * (o < DC ? 1.f : 0.f);
    }
    float x[U];
    if (Dout <= 3 * 256 && kc_count <= 32) {
        // common shapes: every partial load of the thread is in flight at once
        float pv[3][32];
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int o = tid + 256 * u;
            // (clamped reads are finite partial sums: a 0 / 1 factor drops them)
            const float keep_o = o < Dout ? 1.f : 0.f;
#pragma unroll
            for (int kc = 0; kc < 32; ++kc) {
                const float v = part[((size_t)min(kc, kc_count - 1) * T + t) * Dout + min(o, Dout - 1)];
                pv[u][kc] = v * (kc < kc_count ? keep_o : 0.f);
            }
        }
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            x[u] = 0.f;
#pragma unroll
            for (int kc = 0; kc < 32; ++kc) x[u] += pv[u][kc];
        }
        x[3] = x[4] = 0.f;
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int o = tid + 256 * u;
            x[u] = 0.f;
            if (o < Dout)
                for (int kc = 0; kc < kc_count; ++kc) x[u] += part[((size_t)kc * T + t) * Dout + o];
        }
    }
    if (tid < DR / 2) {
        const double ang = (double)pos * pow((double)rope_base, -2.0 * tid / (double)DR);
        const double turns = rint(ang * 0.15915494309189535);
        sincosf((float)fma(-turns, 6.283185307179586, ang), &rsn[tid], &rcs[tid]);
    }
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int o = tid + 256 * u;
        if (o < Dout) y[o] = x[u];
        if (o < DC) ss += x[u] * x[u];
    }
    ss = block_sum(ss, red);                    // also publishes y[], rsn[], rcs[]
    const float inv = 1.0f / sqrtf(ss / (float)DC + eps);
    float yo[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int o = tid + 256 * u;
        if (o < DC) {
            yo[u] = x[u] * inv * gm[u];
        } else if (o < Dout) {
            const int k = (o - DC) >> 1;
            const float x0 = y[DC + 2 * k], x1 = y[DC + 2 * k + 1];
            yo[u] = ((o - DC) & 1) ? x0 * rsn[k] + x1 * rcs[k] : x0 * rcs[k] - x1 * rsn[k];
        } else {
            yo[u] = 0.f;
        }
    }
    if constexpr (CDT == MLA_FP8_E4M3) {
        float amax = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) amax = fmaxf(amax, fabsf(yo[u]));
        amax = block_max(amax, red);
        const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
        unsigned char* dst = static_cast<unsigned char*>(pool) + phys * Dout;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int o = tid + 256 * u;
            if (o < Dout) dst[o] = static_cast<unsigned char>(f32_to_e4m3_rne_sat(yo[u] / sc));
        }
        if (tid == 0) pool_scale[phys] = sc;
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int o = tid + 256 * u;
            if (o < Dout) store_act<CDT>(pool, cache_offset(phys, o, Dout), yo[u]);
        }
    }
}

}  // namespace
}  // namespace mla

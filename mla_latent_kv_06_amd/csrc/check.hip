// Debug check of the paged cache's device-side contract (mla_check_block_table):
// the decode and the append trust block_table and seq_lens, so an id outside
// the pool would read or write outside it.  One workgroup walks every
// (sequence, block) entry a sequence's tokens reach and reports the number of
// violations and the first one (smallest b, then k), deterministically.

#include "common.hpp"
#include "internal.hpp"

namespace mla {
namespace {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void check_block_table_kernel(
    const int* __restrict__ block_table, int batch, int max_blocks, const int* __restrict__ seq_lens,
    int block_size, int num_blocks, int* __restrict__ report) {
    __shared__ int cnt[kCheckThreads / 64];
    __shared__ long long first[kCheckThreads / 64];
    const long long total = (long long)batch * (max_blocks + 1);
    int n = 0;
    long long f = -1;
    // entry e = b * (max_blocks + 1) + k: k < max_blocks is block k of sequence
    // b, k == max_blocks stands for sequence b's length
    for (long long e = threadIdx.x; e < total; e += kCheckThreads) {
        const int b = (int)(e / (max_blocks + 1)), k = (int)(e - (long long)b * (max_blocks + 1));
        const int len = seq_lens[b];
        bool bad;
        if (k == max_blocks) {
            bad = len < 0 || (long long)len > (long long)max_blocks * block_size;
        } else {
            const long long need = len > 0 ? ((long long)len + block_size - 1) / block_size : 0;
            const int id = block_table[(size_t)b * max_blocks + k];
            bad = k < need && (id < 0 || id >= num_blocks);
        }
        if (bad) {
            ++n;
            if (f < 0) f = e;                    // entries rise with e per thread
        }
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int o = 32; o > 0; o >>= 1) {
        n += __shfl_xor(n, o, 64);
        const long long g = __shfl_xor(f, o, 64);
        f = (f < 0) ? g : (g < 0 ? f : min(f, g));
    }
    if (lane == 0) {
        cnt[w] = n;
        first[w] = f;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int tn = 0;
        long long tf = -1;
        for (int i = 0; i < kCheckThreads / 64; ++i) {
            tn += cnt[i];
            if (first[i] >= 0 && (tf < 0 || first[i] < tf)) tf = first[i];
        }
        report[0] = tn;
        report[1] = tf < 0 ? -1 : (int)(tf / (max_blocks + 1));
        const int k = tf < 0 ? -1 : (int)(tf % (max_blocks + 1));
        report[2] = k == max_blocks ? -1 : k;
    }
}

}  // namespace

hipError_t launch_check_block_table(const int* block_table, int batch, int max_blocks, const int* seq_lens,
                                    int block_size, int num_blocks, int* report, hipStream_t stream) {
    check_block_table_kernel<<<1, kCheckThreads, 0, stream>>>(block_table, batch, max_blocks, seq_lens,
                                                              block_size, num_blocks, report);
    return hipGetLastError();
}

}  // namespace mla

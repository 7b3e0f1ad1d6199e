// schedule.hip -- longest-processing-time-first order of attention work items.
//
// Kept-block counts differ a lot between query blocks (the CDF rule keeps few
// blocks for peaked rows and many for flat ones, and the STA union adds a
// border-dependent number). Launching the items with the most kept blocks
// first lets the hardware dispatcher fill the tail with short items.
// Counting sort over counts 0..n in one workgroup (LDS histogram + scan).

#include "common.h"
#include "kernels.h"

namespace nabla {

constexpr int kLptThreads = 1024;

__global__ __launch_bounds__(kLptThreads) void lpt_order_kernel(const int32_t* __restrict__ counts,
                                                                 int64_t items, int n,
                                                                 int32_t* __restrict__ order) {
    __shared__ int hist[NABLA_MAX_BLOCKS + 1];
    __shared__ int chunk_sum[kLptThreads];
    const int t = threadIdx.x;
    const int nb = n + 1;  // count values 0..n
    for (int c = t; c < nb; c += kLptThreads) hist[c] = 0;
    __syncthreads();
    for (int64_t it = t; it < items; it += kLptThreads) {
        int c = counts[it];
        c = c < 0 ? 0 : (c > n ? n : c);
        atomicAdd(&hist[c], 1);
    }
    __syncthreads();
    // Exclusive scan in descending count order: slot position r = n - c.
    // Thread t owns a contiguous range of ranks [t*per, (t+1)*per).
    const int per = (nb + kLptThreads - 1) / kLptThreads;
    int local = 0;
    for (int r = t * per; r < (t + 1) * per && r < nb; ++r) local += hist[n - r];
    chunk_sum[t] = local;
    __syncthreads();
    // Hillis-Steele inclusive scan over the 1024 chunk sums.
    for (int off = 1; off < kLptThreads; off <<= 1) {
        const int add = t >= off ? chunk_sum[t - off] : 0;
        __syncthreads();
        chunk_sum[t] += add;
        __syncthreads();
    }
    int run = chunk_sum[t] - local;  // exclusive prefix of this thread's range
    for (int r = t * per; r < (t + 1) * per && r < nb; ++r) {
        const int c = n - r;
        const int hc = hist[c];
        hist[c] = run;  // becomes the next free slot of count c
        run += hc;
    }
    __syncthreads();
    for (int64_t it = t; it < items; it += kLptThreads) {
        int c = counts[it];
        c = c < 0 ? 0 : (c > n ? n : c);
        const int pos = atomicAdd(&hist[c], 1);
        order[pos] = (int32_t)it;
    }
}

hipError_t launch_lpt_order(const int32_t* counts, int64_t items, int n, int32_t* order,
                            hipStream_t stream) {
    lpt_order_kernel<<<1, kLptThreads, 0, stream>>>(counts, items, n, order);
    return hipGetLastError();
}

}  // namespace nabla

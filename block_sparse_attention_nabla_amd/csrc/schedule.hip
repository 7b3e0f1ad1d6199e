// schedule.hip -- order of attention work items (query or key blocks).
//
// Two goals. (1) Cache locality: every kept block pair re-reads a 32 KB K/V
// tile pair, and one head's K and V (41 MB at 80640 x 128) is re-read about a
// hundred times, so the items that run at the same time should belong to
// as few heads as possible -- and, since each of MI355X's 8 XCDs has its own
// L2, the items one XCD runs should come from the same head. Workgroup b of
// a launch runs on XCD b % 8 (round-robin dispatch), so the launch maps
// workgroup b to a (head part, position) pair: XCD x walks the parts
// x, x + 8, x + 16, ...; a part is an interleaved share of one head (every
// second, fourth or eighth item of its longest-first order).
// (2) Load balance: kept-block counts differ a lot between query blocks (the
// CDF rule keeps few blocks for peaked rows and many for flat ones), so
// within a head the longest items start first. XCDs also differ in speed
// (measured: the same number of block steps takes up to 4% longer on some
// XCDs than on others), so the XCDs that share a head take its items from a
// counter as they start rather than by a fixed interleave. Small problems,
// whose K/V all fit the Infinity Cache and whose few workgroups per CU make
// the longest items set the kernel's length, start the longest items of
// every head first instead.

#include "common.h"
#include "kernels.h"

namespace nabla {

constexpr int kLptThreads = 1024;

// One workgroup per head: counting sort of the head's `items` items by count
// (descending; counts clamped to [0, n]). order[h*items + p] = global item id
// of the head's p-th item. Also zeroes the head's claim counter, if any.
__global__ __launch_bounds__(kLptThreads) void head_lpt_kernel(const int32_t* __restrict__ counts,
                                                               int items, int n,
                                                               int32_t* __restrict__ order,
                                                               int32_t* __restrict__ claim) {
    __shared__ int hist[NABLA_MAX_BLOCKS + 1];
    __shared__ int chunk_sum[kLptThreads];
    const int t = threadIdx.x;
    const int64_t base = (int64_t)blockIdx.x * items;
    const int nb = n + 1;  // count values 0..n
    if (claim && t == 0) claim[blockIdx.x] = 0;
    for (int c = t; c < nb; c += kLptThreads) hist[c] = 0;
    __syncthreads();
    for (int it = t; it < items; it += kLptThreads) {
        int c = counts[base + it];
        c = c < 0 ? 0 : (c > n ? n : c);
        atomicAdd(&hist[c], 1);
    }
    __syncthreads();
    // Exclusive scan in descending count order: rank r <-> count n - r.
    // Thread t owns the contiguous ranks [t*per, (t+1)*per).
    const int per = (nb + kLptThreads - 1) / kLptThreads;
    int local = 0;
    for (int r = t * per; r < (t + 1) * per && r < nb; ++r) local += hist[n - r];
    chunk_sum[t] = local;
    __syncthreads();
    for (int off = 1; off < kLptThreads; off <<= 1) {  // inclusive scan of the chunk sums
        const int add = t >= off ? chunk_sum[t - off] : 0;
        __syncthreads();
        chunk_sum[t] += add;
        __syncthreads();
    }
    int run = chunk_sum[t] - local;
    for (int r = t * per; r < (t + 1) * per && r < nb; ++r) {
        const int c = n - r;
        const int hc = hist[c];
        hist[c] = run;  // next free position of count c
        run += hc;
    }
    __syncthreads();
    for (int it = t; it < items; it += kLptThreads) {
        int c = counts[base + it];
        c = c < 0 ? 0 : (c > n ? n : c);
        const int pos = atomicAdd(&hist[c], 1);
        order[base + pos] = (int32_t)(base + it);
    }
}

hipError_t launch_lpt_order(const int32_t* counts, int64_t BH, int items, int maxc,
                            int32_t* order, int32_t* claim, hipStream_t stream) {
    head_lpt_kernel<<<(unsigned)BH, kLptThreads, 0, stream>>>(counts, items, maxc, order, claim);
    return hipGetLastError();
}

__global__ __launch_bounds__(64) void zero_count_kernel(int32_t* __restrict__ bad) {
    if (threadIdx.x == 0) *bad = 0;
}

// One wave per row: the count in [0, n]; the first `count` entries in [0, n)
// and strictly ascending (each lane compares its entry with the previous
// lane's, lane 0 with the last entry of the previous 64).
__global__ __launch_bounds__(256) void check_lists_kernel(const int32_t* __restrict__ count,
                                                          const int32_t* __restrict__ idx,
                                                          int64_t rows, int n,
                                                          int32_t* __restrict__ bad) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;  // whole wave
    const int c = count[row];
    bool ok = c >= 0 && c <= n;
    if (ok) {
        const int32_t* l = idx + row * (int64_t)n;
        int prev_last = -1;
        for (int base = 0; base < c && ok; base += 64) {
            const int i = base + lane;
            const int v = i < c ? l[i] : 0;
            const int up = __shfl_up(v, 1);
            const int prev = lane == 0 ? prev_last : up;
            const bool wrong = i < c && (v < 0 || v >= n || (i > 0 && v <= prev));
            if (__ballot(wrong)) ok = false;
            prev_last = __shfl(v, 63);
        }
    }
    if (!ok && lane == 0) atomicAdd(bad, 1);
}

hipError_t launch_check_lists(const int32_t* count, const int32_t* idx, int64_t rows, int n,
                              int32_t* bad, hipStream_t stream) {
    zero_count_kernel<<<1, 64, 0, stream>>>(bad);
    if (rows > 0)
        check_lists_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(count, idx, rows, n, bad);
    return hipGetLastError();
}

XcdSchedule make_schedule(int64_t BH, int n) {
    int64_t a = BH, b = 8;  // gcd(BH, 8)
    while (b != 0) {
        const int64_t r = a % b;
        a = b;
        b = r;
    }
    const int g = (int)a;
    XcdSchedule s;
    // Parts per head: at least 2, so that two XCDs share each head and at most
    // four heads' K/V (4 x 41 MB at 80640 x 128) are live at once -- they fit
    // the 256 MB Infinity Cache, which eight live heads would overflow.
    s.parts = 8 / g < 2 ? 2 : 8 / g;
    s.units = BH * s.parts;                  // a multiple of 8
    s.cap = (n + s.parts - 1) / s.parts;     // positions per part
    s.n = n;
    s.grid = s.units * s.cap;
    s.mode = kSchedStatic;
    s.bh = BH;
    s.claim = nullptr;
    return s;
}

// Problems up to this many work items whose K/V (all heads) fit this many
// bytes use the position-major order.
constexpr int64_t kPosMajorItems = 16384;
constexpr int64_t kPosMajorBytes = 128ll << 20;

XcdSchedule make_balanced_schedule(int64_t BH, int n, int64_t kv_bytes_per_head, int32_t* claim) {
    XcdSchedule s = make_schedule(BH, n);
    if (BH * n <= kPosMajorItems && BH * kv_bytes_per_head <= kPosMajorBytes) {
        s.mode = kSchedPosMajor;
        s.grid = BH * n;
        return s;
    }
    if (claim) {
        s.mode = kSchedClaim;
        s.claim = claim;
        s.cap = (5 * n + 4 * s.parts - 1) / (4 * s.parts);  // a quarter to spare
        s.grid = s.units * s.cap;
    }
    return s;
}

}  // namespace nabla

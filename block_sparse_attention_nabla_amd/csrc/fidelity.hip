// fidelity.hip -- mask-fidelity diagnostic on gfx950.
//
// The per-block fidelity test that the review record of "NABLA: Neighborhood
// Adaptive Block-Level Attention" (arXiv 2507.13546, pith.science) asks for:
// how much of full attention's token-level probability mass lies inside the
// blocks a mask keeps, against the best blocks one could keep with the same
// per-row budget.
//
//   block_mass_kernel  M_ij = (1/N) sum_{s in block i} sum_{u in block j} P_su,
//                      P_su = exp(scale q_s.k_u - LSE_s) with the dense LSE
//                      (softmax over all S keys, eq. (2)); every key block.
//                      S^T = K Q^T on bf16 MFMA as in the forward kernel, the
//                      probabilities summed per tile in fp32 (deterministic).
//   recall_kernel      per row: sum of M over the kept list, and the sum of the
//                      row's c largest masses (c = kept count), found by radix
//                      selection of the c-th largest value (sums in double).

#include "common.h"
#include "kernels.h"

namespace nabla {

namespace {

template <int D>
struct MassTile {
    static constexpr int CPR = D / 8;                   // 16-byte chunks per row
    static constexpr int KSTB = 2 * D + 16;             // padded K row stride (bytes)
    static constexpr int LOADS = kBlockN * CPR / 128;   // chunks per thread per tile
};

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// One workgroup (2 waves x 32 queries) per query block, sweeping every key block.
template <int D>
__global__ __launch_bounds__(128) void block_mass_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const float* __restrict__ lse, int S,
                                                         int n, XcdSchedule sched,
                                                         float scale_log2,
                                                         float* __restrict__ mass) {
    using T = MassTile<D>;
    constexpr int KK = D / 16;
    constexpr int L = T::LOADS;
    __shared__ __attribute__((aligned(16))) char sK[kBlockN * T::KSTB];
    __shared__ float sPart[2][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, c = lane & 31;
    const int64_t item = scheduled_slot(sched, blockIdx.x);
    if (item < 0) return;  // padding slot (whole workgroup)
    const int64_t bh = item / n;
    const int qb = (int)(item % n);
    const int64_t head = bh * (int64_t)S * D;
    const uint16_t* kh = k + head;

    const int qrow = qb * kBlockN + wave * 32 + c;
    bf16x8_t qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(q + head + (int64_t)qrow * D + 16 * kk + 8 * h));
    // exp2 argument offset of this lane's query: LSE in log2 units.
    const float lse2 = lse[bh * (int64_t)S + qrow] * kLog2e;

    u32x4_t kr[L];
#define NABLA_MASS_FETCH(J)                                                    \
    do {                                                                       \
        const int64_t off_ = (int64_t)(J) * kBlockN * D;                       \
        _Pragma("unroll") for (int i_ = 0; i_ < L; ++i_)                       \
            kr[i_] = *reinterpret_cast<const u32x4_t*>(kh + off_ + (tid + 128 * i_) * 8); \
    } while (0)
#define NABLA_MASS_STAGE()                                                     \
    do {                                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < L; ++i_) {                     \
            const int e_ = tid + 128 * i_;                                     \
            *reinterpret_cast<u32x4_t*>(sK + (e_ / T::CPR) * T::KSTB + 16 * (e_ % T::CPR)) = kr[i_]; \
        }                                                                      \
    } while (0)

    const char* kbase = sK + c * T::KSTB + 16 * h;
    float* mrow = mass + item * (int64_t)n;
    const float inv_n = 1.0f / (float)kBlockN;
    float part = 0.f;  // lane (j % 64) keeps this wave's sum for key block j

    NABLA_MASS_FETCH(0);
    NABLA_MASS_STAGE();
    if (n > 1) NABLA_MASS_FETCH(1);
    __syncthreads();
    for (int j = 0; j < n; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            bf16x8_t a[KK];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(kbase + 32 * kt * T::KSTB + 32 * kk));
            f32x16_t s = zero16();
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) s = mfma_32x32x16(a[kk], qf[kk], s);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc += __builtin_amdgcn_exp2f(s[r] * scale_log2 - lse2);
        }
        const float tot = wave_sum_f(acc);
        if (lane == (j & 63)) part = tot;
        if ((j & 63) == 63 || j == n - 1) {
            sPart[wave][lane] = part;
            __syncthreads();
            const int j0 = j & ~63;
            if (wave == 0 && lane <= (j & 63))
                mrow[j0 + lane] = (sPart[0][lane] + sPart[1][lane]) * inv_n;
        }
        if (j + 1 < n) {
            __syncthreads();  // every wave has read K_j
            NABLA_MASS_STAGE();
            if (j + 2 < n) NABLA_MASS_FETCH(j + 2);
            __syncthreads();
        }
    }
#undef NABLA_MASS_FETCH
#undef NABLA_MASS_STAGE
}

constexpr int kRecallThreads = 256;

__device__ __forceinline__ double block_sum_d(double v, double* red, int t) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if ((t & 63) == 0) red[t >> 6] = v;
    __syncthreads();
    const double r = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return r;
}

// One workgroup per row (bh, i).
__global__ __launch_bounds__(kRecallThreads) void recall_kernel(
    const float* __restrict__ mass, int n, const int32_t* __restrict__ kv_count,
    const int32_t* __restrict__ kv_idx, float* __restrict__ recall, float* __restrict__ best) {
    __shared__ float mv[NABLA_MAX_BLOCKS];
    __shared__ int hcnt[256];
    __shared__ int wtot[4];
    __shared__ int sel_bin, sel_above;
    __shared__ double red[4];

    const int64_t row = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const float* M = mass + row * (int64_t)n;
    for (int j = t; j < n; j += kRecallThreads) mv[j] = M[j];
    int cnt = kv_count[row];
    cnt = cnt < 0 ? 0 : (cnt > n ? n : cnt);
    const int32_t* list = kv_idx + row * (int64_t)n;
    __syncthreads();

    // Mass inside the kept list (indices outside [0, n) contribute nothing).
    double rs = 0.0;
    for (int e = t; e < cnt; e += kRecallThreads) {
        const int j = list[e];
        if ((unsigned)j < (unsigned)n) rs += (double)mv[j];
    }
    rs = block_sum_d(rs, red, t);

    // c-th largest value tau: MSB-first radix select over the (non-negative)
    // fp32 bit patterns, counting entries strictly above each 8-bit bin.
    uint32_t prefix = 0, pmask = 0;
    int above = 0;
    if (cnt > 0) {
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            hcnt[t] = 0;
            __syncthreads();
            for (int j = t; j < n; j += kRecallThreads) {
                const uint32_t key = __float_as_uint(fmaxf(mv[j], 0.f));
                if ((key & pmask) == prefix) atomicAdd(&hcnt[(key >> shift) & 255], 1);
            }
            __syncthreads();
            const int m = hcnt[t];
            int incl = m;  // inclusive suffix sum over this wave's bins (higher lane = higher bin)
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int o = __shfl_down(incl, off);
                if (lane + off < 64) incl += o;
            }
            if (lane == 0) wtot[wave] = incl;
            if (t == 0) sel_bin = 256;
            __syncthreads();
            int higher = 0;
            for (int w = wave + 1; w < 4; ++w) higher += wtot[w];
            const int above_bin = above + higher + (incl - m);
            if (m > 0 && above_bin <= cnt - 1) atomicMin(&sel_bin, t);
            __syncthreads();
            const int b = sel_bin;  // < 256: the highest non-empty bin qualifies
            if (t == b) sel_above = above_bin;
            __syncthreads();
            above = sel_above;
            prefix |= (uint32_t)b << shift;
            pmask |= 0xffu << shift;
            __syncthreads();
        }
    }
    const float tau = __uint_as_float(prefix);
    double bs = 0.0;
    for (int j = t; j < n; j += kRecallThreads) {
        const float x = fmaxf(mv[j], 0.f);
        if (cnt > 0 && x > tau) bs += (double)x;
    }
    bs = block_sum_d(bs, red, t);
    if (t == 0) {
        recall[row] = (float)rs;
        best[row] = cnt > 0 ? (float)(bs + (double)(cnt - above) * (double)tau) : 0.f;
    }
}

}  // namespace

hipError_t launch_block_mass(const void* q, const void* k, const float* lse, int64_t BH, int S,
                             int D, float softmax_scale, float* mass, hipStream_t stream) {
    const int n = S / kBlockN;
    const XcdSchedule sched = make_schedule(BH, n);
    const float sl2 = softmax_scale * kLog2e;
    if (D == 128)
        block_mass_kernel<128><<<(unsigned)sched.grid, 128, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, lse, S, n, sched, sl2, mass);
    else
        block_mass_kernel<64><<<(unsigned)sched.grid, 128, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, lse, S, n, sched, sl2, mass);
    return hipGetLastError();
}

hipError_t launch_mask_recall(const float* mass, int64_t BH, int n, const int32_t* kv_count,
                              const int32_t* kv_idx, float* recall, float* best,
                              hipStream_t stream) {
    recall_kernel<<<(unsigned)(BH * n), kRecallThreads, 0, stream>>>(mass, n, kv_count, kv_idx,
                                                                     recall, best);
    return hipGetLastError();
}

}  // namespace nabla

// mask_kernels.hip -- the NABLA block-mask stage on gfx950.
//
// "NABLA: Neighborhood Adaptive Block-Level Attention", section 3.1.2,
// Algorithm 1 (pooling, reduced softmax, CDF binarisation) and section 3.1.3
// (union with the sliding-tile mask), followed by compaction of each mask row
// into an ascending list of kept key blocks.
//
//   pool_kernel      steps 2-5: block means of Q and K (HBM streaming, exact fp64 sums)
//   logits_kernel    steps 6-7 (logits part): Q_a K_a^T * scale per head, fp32 MFMA
//   select_wave_kernel steps 7-11: row softmax, sort-free CDF selection by radix
//                    select over the fp32 bit patterns of the probabilities,
//                    exact (fp64) order of the entries next to the cut, STA
//                    union, ascending compaction, optional dense/bit rows. The
//                    same kernel runs the Top-k selector the CDF rule is
//                    measured against; sta_select_kernel the static STA window
//                    alone (Table 1's baseline).
//   transpose_kernel the key-block -> query-block lists the backward pass uses

#include "common.h"
#include "kernels.h"

namespace nabla {

// ---------------------------------------------------------------------------
// Pooling: out[bh][i][d] = (1/N) * sum_{r<N} x[bh][i*N + r][d].
// One workgroup per (block, tensor); 256 threads stream the 64 x D bf16 block
// with 16-byte loads and sum each column in fp64, then reduce the partial rows
// in LDS in a fixed order (deterministic). A sum of 64 bf16 values (8-bit
// significands) is exact in fp64 unless their exponents span more than 39
// binades, and dividing by 64 is exact, so the fp64 means equal the exact
// block means. The kernel writes them in fp64 (for the exact re-check of
// near-tied probabilities in the selection), rounded to fp32 (the operands of
// the reduced-logit products) and the Euclidean norm of each mean (rounded up;
// it bounds the rounding error of those fp32 products).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k,
                                                   PoolOut out) {
    constexpr int CG = D / 8;           // 16-byte column groups per row
    constexpr int RPT = 256 / CG;       // rows covered per pass
    constexpr int PASSES = kBlockN / RPT;
    __shared__ double part[RPT][D];
    __shared__ double wsq[4];

    const int64_t blk = blockIdx.x;     // flattened bh * n + i
    const int tensor = blockIdx.y;      // 0: Q, 1: K
    const uint16_t* src = (tensor == 0 ? q : k) + blk * (int64_t)kBlockN * D;

    const int t = threadIdx.x;
    const int cg = t % CG, r0 = t / CG;
    // Every Q/K byte is read once here: non-temporal loads stream past the caches.
    uint4 raw[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        raw[p] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                                               src + (int64_t)(r0 + p * RPT) * D + cg * 8)));
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const uint32_t w[4] = {raw[p].x, raw[p].y, raw[p].z, raw[p].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += (double)bf16_bits_to_f32(w[e] & 0xffffu);
            acc[2 * e + 1] += (double)bf16_bits_to_f32(w[e] >> 16);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r0][cg * 8 + e] = acc[e];
    __syncthreads();
    double sq = 0.0;
    if (t < D) {
        double s = 0.0;
#pragma unroll 8
        for (int r = 0; r < RPT; ++r) s += part[r][t];
        const double mean = s * (1.0 / kBlockN);
        (tensor == 0 ? out.qa64 : out.ka64)[blk * D + t] = mean;
        (tensor == 0 ? out.qa : out.ka)[blk * D + t] = (float)mean;
        sq = mean * mean;
    }
    // Norm of the mean: fixed-order reduction over the D threads that hold it.
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
    if ((t & 63) == 0) wsq[t >> 6] = sq;
    __syncthreads();
    if (t == 0) {
        const double tot = (wsq[0] + wsq[1]) + (wsq[2] + wsq[3]);
        // Rounded up (with a relative margin far above the rounding of this sum).
        (tensor == 0 ? out.qnorm : out.knorm)[blk] = (float)(sqrt(tot) * (1.0 + 1e-6));
    }
}

// Largest key-block norm of each head: kmax[bh] = max_j knorm[bh][j].
__global__ __launch_bounds__(256) void head_max_kernel(const float* __restrict__ knorm, int n,
                                                       float* __restrict__ kmax) {
    __shared__ float wm[4];
    const int64_t bh = blockIdx.x;
    const int t = threadIdx.x;
    float m = 0.f;
    for (int j = t; j < n; j += 256) m = fmaxf(m, knorm[bh * n + j]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((t & 63) == 0) wm[t >> 6] = m;
    __syncthreads();
    if (t == 0) kmax[bh] = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
}

// ---------------------------------------------------------------------------
// Reduced logits: L[bh][i][j] = scale * sum_d Q_a[bh][i][d] * K_a[bh][j][d].
// Workgroup = 4 waves = a 64 x 64 tile of (i, j); each wave one 32 x 32 tile
// built from v_mfma_f32_32x32x2_f32 (fp32 in, fp32 accumulate). Each lane
// feeds the MFMAs from one float4 of Q_a and one of K_a per 8 values of d:
// lane-half h and component m stand for d = d0 + 4h + m on both operands.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void logits_kernel(const float* __restrict__ qa,
                                                     const float* __restrict__ ka,
                                                     float* __restrict__ logits, int n,
                                                     float scale) {
    // Each wave computes a 64 x 64 tile as 2 x 2 MFMA tiles of 32 x 32, so every
    // operand load feeds two products; the workgroup covers 128 x 128.
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = lane >> 5, c = lane & 31;
    const int64_t bh = blockIdx.z;
    const int i0 = blockIdx.x * 128 + 64 * (wave >> 1);
    const int j0 = blockIdx.y * 128 + 64 * (wave & 1);
    if (i0 >= n || j0 >= n) return;  // whole-wave exit; no barriers below
    const float* qrow[2];
    const float* krow[2];
    bool qok[2], kok[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int qi = i0 + 32 * t + c, kj = j0 + 32 * t + c;
        qok[t] = qi < n;
        kok[t] = kj < n;
        qrow[t] = qa + (bh * n + (qok[t] ? qi : 0)) * D;
        krow[t] = ka + (bh * n + (kok[t] ? kj : 0)) * D;
    }

    f32x16_t acc[2][2];
#pragma unroll
    for (int a_ = 0; a_ < 2; ++a_)
#pragma unroll
        for (int b_ = 0; b_ < 2; ++b_) acc[a_][b_] = zero16();
    // The next step's operands are loaded before this step's products.
    float4 na[2], nb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        na[t] = qok[t] ? *reinterpret_cast<const float4*>(qrow[t] + 4 * h) : make_float4(0, 0, 0, 0);
        nb[t] = kok[t] ? *reinterpret_cast<const float4*>(krow[t] + 4 * h) : make_float4(0, 0, 0, 0);
    }
#pragma unroll 2
    for (int d0 = 0; d0 < D; d0 += 8) {
        float4 a[2], b[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            a[t] = na[t];
            b[t] = nb[t];
            if (d0 + 8 < D) {
                na[t] = qok[t] ? *reinterpret_cast<const float4*>(qrow[t] + d0 + 8 + 4 * h) : make_float4(0, 0, 0, 0);
                nb[t] = kok[t] ? *reinterpret_cast<const float4*>(krow[t] + d0 + 8 + 4 * h) : make_float4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int tj = 0; tj < 2; ++tj) {
                acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[ti].x, b[tj].x, acc[ti][tj], 0, 0, 0);
                acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[ti].y, b[tj].y, acc[ti][tj], 0, 0, 0);
                acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[ti].z, b[tj].z, acc[ti][tj], 0, 0, 0);
                acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[ti].w, b[tj].w, acc[ti][tj], 0, 0, 0);
            }
    }
    // C layout: this lane holds column j0 + 32 tj + c and rows i0 + 32 ti + c_row(r, h).
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
        if (!kok[tj]) continue;
        const int kj = j0 + 32 * tj + c;
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = i0 + 32 * ti + c_row(r, h);
                if (i < n) logits[(bh * n + i) * (int64_t)n + kj] = acc[ti][tj][r] * scale;
            }
    }
}

// ---------------------------------------------------------------------------
// Block reductions over a 256-thread workgroup (fixed order => deterministic).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// STA window membership of key block j for query block i (clipped centred window).
__device__ __forceinline__ bool sta_contains(const StaParams& s, int i, int j) {
    const int ti = i / (s.tH * s.tW), yi = (i / s.tW) % s.tH, xi = i % s.tW;
    const int tj = j / (s.tH * s.tW), yj = (j / s.tW) % s.tH, xj = j % s.tW;
    const bool in_t = tj >= ti - (s.wt - 1) / 2 && tj <= ti + s.wt / 2;
    const bool in_h = yj >= yi - (s.wh - 1) / 2 && yj <= yi + s.wh / 2;
    const bool in_w = xj >= xi - (s.ww - 1) / 2 && xj <= xi + s.ww / 2;
    return in_t && in_h && in_w;  // clipping is implicit: j is always on the grid
}

// ---------------------------------------------------------------------------
// The static STA window alone (Table 1's STA rows): one workgroup (256 threads)
// per query-block row, ballot compaction in ascending order.
// ---------------------------------------------------------------------------
constexpr int kStaThreads = 256;

__global__ __launch_bounds__(kStaThreads) void sta_select_kernel(
    int n, StaParams sta, int32_t* __restrict__ kv_count, int32_t* __restrict__ kv_idx,
    uint8_t* __restrict__ dense_mask, uint32_t* __restrict__ bits, int words_per_row) {
    __shared__ int wcount[4];
    const int64_t row = blockIdx.x;  // flattened bh * n + i
    const int i = (int)(row % n);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int32_t* out_idx = kv_idx + row * (int64_t)n;
    int running = 0;
    for (int base = 0; base < n; base += kStaThreads) {
        const int j = base + t;
        const bool keep = j < n && sta_contains(sta, i, j);
        const unsigned long long bal = __ballot(keep);
        const int before = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wcount[wave] = __popcll(bal);
        __syncthreads();
        int off = running;
        for (int w = 0; w < wave; ++w) off += wcount[w];
        if (keep) out_idx[off + before] = j;
        if (dense_mask && j < n) dense_mask[row * (int64_t)n + j] = keep ? 1 : 0;
        if (bits && lane < 2) {
            const int word = (base + 64 * wave) / 32 + lane;
            if (word < words_per_row)
                bits[row * (int64_t)words_per_row + word] = (uint32_t)(bal >> (32 * lane));
        }
        running += wcount[0] + wcount[1] + wcount[2] + wcount[3];
        __syncthreads();
    }
    if (t == 0) kv_count[row] = running;
}

// ---------------------------------------------------------------------------
// Content selection + compaction, one wave per query-block row.
//
// kSelCdf:  keep j iff G_j <= thr (the NABLA rule, Algorithm 1), G_j = mass of
//           the entries strictly larger than p_j.
// kSelTopk: keep j iff fewer than k entries of the row are strictly larger than
//           p_j (the k largest, ties at the k-th value kept together): the same
//           selection with every entry weighing 1 and k - 1 as the bound.
//
// 1. p_j = exp(L_j - max) / sum in fp32 (L = the fp32 reduced logits).
// 2. The kept set {j : G_j <= thr} is {j : p_j >= tau} for the smallest value
//    tau whose strictly-larger mass is <= thr. tau is found MSB-first over the
//    uint32 bit patterns of the (non-negative) p_j, 8 bits per pass: a 256-bin
//    histogram of (count, weight) over the entries matching the prefix so far,
//    a suffix sum over bins, and the lowest non-empty bin whose weight-above
//    stays <= the bound. Masses are 2^-40 fixed-point integers, so every sum is
//    exact and independent of the order in which the atomics land. Once the
//    boundary bin holds at most 64 entries, it is finished exactly.
// 3. Exact order near the cut. fp32 rounding can order two nearly equal
//    probabilities differently from exact arithmetic, which changes a decision
//    even far from the threshold in mass. The rounding error of the fp32 logits
//    is bounded per row by E = err_unit * |Q_a[i]| * max_j |K_a[j]| (err_unit
//    covers the fp32 operands, the D-term fp32 dot product and the scaling),
//    and exp / division add a bound that depends on |L_j - max|; together they
//    give a window W in log-probability beyond which the fp32 order of two
//    entries is the exact order. Then:
//      p_j > tau e^W   -> kept (every entry that may lie above j is above tau,
//                         whose strictly-larger weight is <= the bound);
//      p_j < tau e^-W  -> dropped (every entry >= tau lies exactly above j);
//      otherwise (C1)  -> decided exactly: G*_j = weight of the entries above
//                         tau e^2W + weight of the entries of C2 = [tau e^-2W,
//                         tau e^2W] whose logit, recomputed in fp64 from the
//                         exact fp64 block means, is larger than j's.
//    The weights stay the fp32-derived fixed-point masses; only the order is
//    made exact. Rows whose window holds a single entry (almost all) keep the
//    radix result unchanged.
// 4. STA union and ascending compaction with ballots.
//
// Rows of up to 2048 blocks keep their values in registers (lane l holds
// j = l + 64 r; four rows per workgroup); longer rows (up to NABLA_MAX_BLOCKS)
// keep them in LDS (two rows per workgroup). No workgroup barrier is needed:
// every reduction is a wave shuffle and each wave owns its LDS slice.
// A histogram bin is one 64-bit word, (weight << kCntBits) + count, so each
// entry costs one LDS atomic; the fields cannot carry into each other (counts
// <= NABLA_MAX_BLOCKS < 2^kCntBits, weights sum to < 2^41). Each wave keeps
// kSelCopies copies of its histogram, lane l adding into copy l % kSelCopies:
// neighbouring key blocks tend to share a bin, and the copies spread those
// same-address atomics over different words.
// ---------------------------------------------------------------------------
constexpr int kSelCopies = 4;
constexpr int kCntBits = 14;
constexpr int kCandCap = 64;  // near-cut candidates held in LDS per row
static_assert(NABLA_MAX_BLOCKS < (1 << kCntBits), "bin counts must fit their field");

// Orders this wave's LDS accesses: the compiler may not move LDS operations
// across it, and the wave waits until its own LDS operations have completed.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

template <bool LROW>
struct SelLds {
    static constexpr int kRows = LROW ? 2 : 4;  // rows (waves) per workgroup
    static constexpr int kWords = (LROW ? NABLA_MAX_BLOCKS : 2048) / 32;
    unsigned long long hist[kSelCopies][256];  // also the row (as float) during step 3
    unsigned long long cw[kCandCap];           // candidate weights
    double cl[kCandCap];                       // candidate fp64 logits
    int cj[kCandCap];                          // candidate key blocks
    uint32_t decided[kWords];                  // exact decisions of C1 entries (bit per j)
    float row[LROW ? NABLA_MAX_BLOCKS : 1];    // p of rows longer than 2048 blocks
};

// Fixed-point weight of a probability (Top-k: 1 per entry).
template <int MODE>
__device__ __forceinline__ unsigned long long sel_weight(float p) {
    return MODE == kSelTopk ? 1ull : (unsigned long long)__float2ull_rn(p * 0x1p40f);
}

// fp64 logit of key block jj for the row's fp64 query mean (qv: this lane's
// D/64 components d = lane * DPL + c), reduced over the wave in a fixed order.
template <int D>
__device__ __forceinline__ double exact_logit(const double (&qv)[D / 64], const double* ka64_head,
                                              int jj, int lane, double scale) {
    constexpr int DPL = D / 64;
    const double* kr = ka64_head + (int64_t)jj * D + lane * DPL;
    double s = 0.0;
#pragma unroll
    for (int c = 0; c < DPL; ++c) s = fma(qv[c], kr[c], s);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    return s * scale;
}

template <int MODE, int VPL, bool LROW, int D>
__global__ __launch_bounds__(256) void select_wave_kernel(SelectArgs a) {
    using Lds = SelLds<LROW>;
    __shared__ __attribute__((aligned(16))) Lds lds_all[Lds::kRows];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * Lds::kRows + wave;
    if (row >= a.rows) return;  // whole wave; no workgroup barrier follows
    Lds& L = lds_all[wave];
    const int n = a.n;
    const int i = (int)(row % n);
    const int64_t bh = row / n;
    // Chunks of 64 entries: lane l of chunk r holds j = l + 64 r.
    const int nch = LROW ? (n + 63) / 64 : VPL;
    float pv[LROW ? 1 : VPL];
    auto val = [&](int r) -> float& {
        if constexpr (LROW) return L.row[lane + 64 * r];
        else return pv[r];
    };
    auto for_chunks = [&](auto&& f) {
        if constexpr (LROW) {
            for (int r = 0; r < nch; ++r) f(r);
        } else {
#pragma unroll
            for (int r = 0; r < VPL; ++r) f(r);
        }
    };

    // 1. row maximum; exponentials and their sum; p = e * (1 / z)
    const float* Lg = a.logits + row * (int64_t)n;
    float mx = -INFINITY;
    for_chunks([&](int r) {
        const int j = lane + 64 * r;
        const float x = j < n ? Lg[j] : -INFINITY;
        val(r) = x;
        mx = fmaxf(mx, x);
    });
    mx = wave_max(mx);
    float z = 0.f;
    for_chunks([&](int r) {
        const int j = lane + 64 * r;
        const float e = j < n ? expf(val(r) - mx) : 0.f;
        val(r) = e;
        z += e;
    });
    z = wave_sum(z);
    // One reciprocal for the row: its rounding is a factor common to every p of
    // the row, so it cancels in the ratios the exact-order window relies on.
    const float rz = 1.0f / z;
    for_chunks([&](int r) { val(r) = val(r) * rz; });

    uint32_t tau = 0;
    bool refined = false;
    float lo1 = 0.f, hi1 = 0.f;
    if (!a.keep_all) {
        // 2. radix select of tau: lane l owns bins 4l .. 4l+3.
        unsigned long long(*hw)[256] = L.hist;
        unsigned long long* mine_copy = hw[lane % kSelCopies];
        uint32_t prefix = 0, pmask = 0;
        unsigned long long above = 0;
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            // The weights are recomputed each pass rather than kept live across
            // passes (VPL 64-bit registers): the scale is made opaque per pass.
            float two40 = 0x1p40f;
            asm volatile("" : "+s"(two40));
#pragma unroll
            for (int cp = 0; cp < kSelCopies; ++cp)
#pragma unroll
                for (int b = 0; b < 4; ++b) hw[cp][4 * lane + b] = 0ull;
            wave_lds_sync();
            for_chunks([&](int r) {
                const int j = lane + 64 * r;
                const float p = val(r);
                const uint32_t key = __float_as_uint(p);
                if (j < n && (key & pmask) == prefix) {
                    const int d = (key >> shift) & 255;
                    const unsigned long long wgt =
                        MODE == kSelTopk ? 1ull : (unsigned long long)__float2ull_rn(p * two40);
                    atomicAdd(&mine_copy[d], (wgt << kCntBits) + 1ull);
                }
            });
            wave_lds_sync();
            unsigned long long m[4];
            int cb[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                unsigned long long packed = 0;
#pragma unroll
                for (int cp = 0; cp < kSelCopies; ++cp) packed += hw[cp][4 * lane + b];
                m[b] = packed >> kCntBits;
                cb[b] = (int)(packed & ((1ull << kCntBits) - 1ull));
            }
            const unsigned long long local = (m[0] + m[1]) + (m[2] + m[3]);
            unsigned long long incl = local;  // inclusive suffix sum over lanes
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const unsigned long long o = __shfl_down(incl, off);
                if (lane + off < 64) incl += o;
            }
            unsigned long long ab[4];  // weight strictly above each of this lane's bins
            ab[3] = above + (incl - local);
            ab[2] = ab[3] + m[3];
            ab[1] = ab[2] + m[2];
            ab[0] = ab[1] + m[1];
            int cand = 256;
#pragma unroll
            for (int b = 3; b >= 0; --b)
                if (cb[b] > 0 && ab[b] <= a.bound) cand = 4 * lane + b;
            int sel = cand;  // lowest qualifying bin of the wave
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) sel = min(sel, __shfl_xor(sel, off));
            // < 256: the highest non-empty bin always qualifies.
            unsigned long long mine = ab[0];
            int cmine = cb[0];
#pragma unroll
            for (int b = 1; b < 4; ++b)
                if ((sel & 3) == b) {
                    mine = ab[b];
                    cmine = cb[b];
                }
            above = __shfl(mine, sel >> 2);
            const int csel = __shfl(cmine, sel >> 2);  // entries in the selected bin
            prefix |= (uint32_t)sel << shift;
            pmask |= 0xffu << shift;
            wave_lds_sync();  // this pass's reads finish before the LDS is reused
            if (pass < 3 && csel <= 64) {
                // Few entries left: finish exactly. Each candidate's weight strictly
                // above is `above` plus the candidates with a larger bit pattern --
                // the same fixed-point sums the remaining passes would form, so tau
                // is the same. Candidates are compacted into LDS slots 0 .. csel-1
                // (keys in histogram copy 1 read as 32-bit words, weights in copy 0).
                uint32_t* hc = reinterpret_cast<uint32_t*>(hw[1]);
                unsigned long long* hm = hw[0];
                int base = 0;
                for_chunks([&](int r) {
                    const int j = lane + 64 * r;
                    const float p = val(r);
                    const uint32_t key = __float_as_uint(p);
                    const bool is_c = j < n && (key & pmask) == prefix;
                    const unsigned long long bal = __ballot(is_c);
                    if (is_c) {
                        const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
                        hc[pos] = key;
                        hm[pos] = sel_weight<MODE>(p);
                    }
                    base += __popcll(bal);
                });
                wave_lds_sync();
                const uint32_t my_key = lane < csel ? hc[lane] : 0u;
                unsigned long long acc = 0;
                for (int m2 = 0; m2 < csel; ++m2)
                    if (hc[m2] > my_key) acc += hm[m2];
                uint32_t t = (lane < csel && above + acc <= a.bound) ? my_key : 0xffffffffu;
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) t = min(t, (uint32_t)__shfl_xor((int)t, off));
                prefix = t;  // the largest candidate always qualifies
                wave_lds_sync();
                break;
            }
        }
        tau = prefix;

        // 3. exact order near the cut.
        const float tauf = __uint_as_float(tau);
        if (tauf >= 0x1p-100f) {
            const float E = a.err_unit * a.qnorm[row] * a.kmax[bh];
            // |L_j - max| of window entries, bounded via the cut's exponential
            // e_cut = tau * z (log <= 0), plus the window itself (< 1).
            const float X = fabsf(__logf(tauf * z)) + 2.f * E + 1.f;
            const float W = 2.f * E + 0x1p-23f * X + 0x1p-20f;
            const float g1 = __expf(W) * (1.f + 0x1p-20f), g2 = __expf(2.f * W) * (1.f + 0x1p-20f);
            hi1 = tauf * g1;
            lo1 = tauf / g1;
            const float hi2 = tauf * g2, lo2 = tauf / g2;
            int c2 = 0;
            for_chunks([&](int r) {
                const int j = lane + 64 * r;
                const float p = val(r);
                c2 += __popcll(__ballot(j < n && p >= lo2 && p <= hi2));
            });
            if (c2 >= 2) {
                refined = true;
                unsigned long long w_up = 0;  // weight of the entries above tau e^2W
                for_chunks([&](int r) {
                    const int j = lane + 64 * r;
                    const float p = val(r);
                    if (j < n && p > hi2) w_up += sel_weight<MODE>(p);
                });
                w_up = wave_sum_u64(w_up);
                // The row in LDS so entries can be addressed by index.
                float* prow = L.row;
                if constexpr (!LROW) {
                    prow = reinterpret_cast<float*>(L.hist);  // 8 KB = 2048 floats
                    for_chunks([&](int r) { prow[lane + 64 * r] = val(r); });
                }
                for (int w = lane; w < (n + 31) / 32; w += 64) L.decided[w] = 0u;
                constexpr int DPL = D / 64;
                double qv[DPL];
#pragma unroll
                for (int c = 0; c < DPL; ++c) qv[c] = a.qa64[row * D + lane * DPL + c];
                const double* kh64 = a.ka64 + bh * (int64_t)n * D;
                wave_lds_sync();
                if (c2 <= kCandCap) {
                    // Collect C2 (ascending j), compute fp64 logits, decide C2 entries.
                    int s = 0;
                    for (int base = 0; base < n; base += 64) {
                        const int j = base + lane;
                        const float p = j < n ? prow[j] : 0.f;
                        const bool in2 = j < n && p >= lo2 && p <= hi2;
                        const unsigned long long bal = __ballot(in2);
                        if (in2) {
                            const int pos = s + __popcll(bal & ((1ull << lane) - 1ull));
                            L.cj[pos] = j;
                            L.cw[pos] = sel_weight<MODE>(p);
                        }
                        s += __popcll(bal);
                    }
                    wave_lds_sync();
                    for (int m2 = 0; m2 < c2; ++m2) {
                        const double l64 = exact_logit<D>(qv, kh64, L.cj[m2], lane, a.scale64);
                        if (lane == 0) L.cl[m2] = l64;
                    }
                    wave_lds_sync();
                    if (lane < c2) {
                        const double lt = L.cl[lane];
                        unsigned long long g = w_up;
                        for (int m2 = 0; m2 < c2; ++m2)
                            if (L.cl[m2] > lt) g += L.cw[m2];
                        if (g <= a.bound) atomicOr(&L.decided[L.cj[lane] >> 5], 1u << (L.cj[lane] & 31));
                    }
                } else {
                    // Many near-equal entries (constant or duplicated blocks): every C1
                    // entry against every C2 entry, logits recomputed as needed.
                    for (int base = 0; base < n; base += 64) {
                        const int j = base + lane;
                        const float p = j < n ? prow[j] : 0.f;
                        unsigned long long bal = __ballot(j < n && p >= lo1 && p <= hi1);
                        while (bal) {
                            const int jj = base + __ffsll((long long)bal) - 1;
                            bal &= bal - 1;
                            const double lj = exact_logit<D>(qv, kh64, jj, lane, a.scale64);
                            unsigned long long g = w_up;
                            for (int b2 = 0; b2 < n; b2 += 64) {
                                const int l = b2 + lane;
                                const float pl = l < n ? prow[l] : 0.f;
                                unsigned long long bal2 = __ballot(l < n && pl >= lo2 && pl <= hi2);
                                while (bal2) {
                                    const int ll = b2 + __ffsll((long long)bal2) - 1;
                                    bal2 &= bal2 - 1;
                                    const double lv = exact_logit<D>(qv, kh64, ll, lane, a.scale64);
                                    if (lv > lj) g += sel_weight<MODE>(prow[ll]);
                                }
                            }
                            if (lane == 0 && g <= a.bound) L.decided[jj >> 5] |= 1u << (jj & 31);
                        }
                    }
                }
                wave_lds_sync();
            }
        }
    }

    // 4. decisions, STA union, ascending compaction (chunk r = blocks 64r .. 64r+63)
    int32_t* out_idx = a.kv_idx + row * (int64_t)n;
    int running = 0;
    for_chunks([&](int r) {
        if (64 * r < n) {
            const int j = lane + 64 * r;
            bool keep = false;
            if (j < n) {
                const float p = val(r);
                if (a.keep_all) keep = true;
                else if (!refined) keep = __float_as_uint(p) >= tau;
                else keep = p > hi1 || (p >= lo1 && ((L.decided[j >> 5] >> (j & 31)) & 1u));
                if (!keep && a.sta.on) keep = sta_contains(a.sta, i, j);
            }
            const unsigned long long bal = __ballot(keep);
            if (keep) out_idx[running + __popcll(bal & ((1ull << lane) - 1ull))] = j;
            if (a.dense_mask && j < n) a.dense_mask[row * (int64_t)n + j] = keep ? 1 : 0;
            if (a.bits && lane < 2) {
                const int word = 2 * r + lane;
                if (word < a.words_per_row)
                    a.bits[row * (int64_t)a.words_per_row + word] = (uint32_t)(bal >> (32 * lane));
            }
            running += __popcll(bal);
        }
    });
    if (lane == 0) a.kv_count[row] = running;
}

// ---------------------------------------------------------------------------
// Transpose of the kept-block relation: for key block j, the ascending list of
// query blocks i that keep it. Workgroup = one 32-column word of the row
// bitmasks; each wave owns 8 of those columns and walks the rows 64 at a time,
// compacting with a ballot (no atomics, deterministic, ascending).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_kernel(const uint32_t* __restrict__ bits, int n,
                                                        int words_per_row,
                                                        int32_t* __restrict__ q_count,
                                                        int32_t* __restrict__ q_idx) {
    const int wc = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int running[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) running[b] = 0;
    const uint32_t* col = bits + bh * (int64_t)n * words_per_row + wc;
    for (int i0 = 0; i0 < n; i0 += 64) {
        const int i = i0 + lane;
        const uint32_t word = i < n ? col[(int64_t)i * words_per_row] : 0u;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int j = 32 * wc + 8 * wave + b;
            const bool f = (word >> (8 * wave + b)) & 1u;
            const unsigned long long bal = __ballot(f);
            if (j < n && f)
                q_idx[(bh * n + j) * (int64_t)n + running[b] + __popcll(bal & ((1ull << lane) - 1ull))] = i;
            running[b] += __popcll(bal);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int j = 32 * wc + 8 * wave + b;
            if (j < n) q_count[bh * n + j] = running[b];
        }
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by the C ABI after validation).
// ---------------------------------------------------------------------------
hipError_t launch_pool(const void* q, const void* k, const PoolOut& out, int64_t BH, int n, int D,
                       hipStream_t stream) {
    dim3 grid((unsigned)(BH * n), 2);
    if (D == 128)
        pool_kernel<128><<<grid, 256, 0, stream>>>((const uint16_t*)q, (const uint16_t*)k, out);
    else
        pool_kernel<64><<<grid, 256, 0, stream>>>((const uint16_t*)q, (const uint16_t*)k, out);
    head_max_kernel<<<(unsigned)BH, 256, 0, stream>>>(out.knorm, n, out.kmax);
    return hipGetLastError();
}

hipError_t launch_logits(const float* qa, const float* ka, float* logits, int64_t BH, int n, int D,
                         float scale, hipStream_t stream) {
    dim3 grid((n + 127) / 128, (n + 127) / 128, (unsigned)BH);
    if (D == 128)
        logits_kernel<128><<<grid, 256, 0, stream>>>(qa, ka, logits, n, scale);
    else
        logits_kernel<64><<<grid, 256, 0, stream>>>(qa, ka, logits, n, scale);
    return hipGetLastError();
}

hipError_t launch_select(int mode, const SelectArgs& a, int D, hipStream_t stream) {
    const int n = a.n;
    if (mode == kSelSta) {
        sta_select_kernel<<<(unsigned)a.rows, kStaThreads, 0, stream>>>(
            n, a.sta, a.kv_count, a.kv_idx, a.dense_mask, a.bits, a.words_per_row);
        return hipGetLastError();
    }
#define NABLA_SEL(MODE_, VPL_, LROW_, D_)                                                        \
    select_wave_kernel<MODE_, VPL_, LROW_, D_>                                                   \
        <<<(unsigned)((a.rows + SelLds<LROW_>::kRows - 1) / SelLds<LROW_>::kRows),               \
           64 * SelLds<LROW_>::kRows, 0, stream>>>(a)
#define NABLA_SEL_D(MODE_, VPL_, LROW_)                                                          \
    do {                                                                                         \
        if (D == 128) NABLA_SEL(MODE_, VPL_, LROW_, 128);                                        \
        else NABLA_SEL(MODE_, VPL_, LROW_, 64);                                                  \
    } while (0)
#define NABLA_SEL_MODES(VPL_, LROW_)                                                             \
    do {                                                                                         \
        if (mode == kSelTopk) NABLA_SEL_D(kSelTopk, VPL_, LROW_);                                \
        else NABLA_SEL_D(kSelCdf, VPL_, LROW_);                                                  \
    } while (0)
    if (n <= 512) NABLA_SEL_MODES(8, false);
    else if (n <= 1024) NABLA_SEL_MODES(16, false);
    else if (n <= 1280) NABLA_SEL_MODES(20, false);
    else if (n <= 2048) NABLA_SEL_MODES(32, false);
    else NABLA_SEL_MODES(1, true);
#undef NABLA_SEL_MODES
#undef NABLA_SEL_D
#undef NABLA_SEL
    return hipGetLastError();
}

hipError_t launch_transpose(const uint32_t* bits, int64_t BH, int n, int words_per_row,
                            int32_t* q_count, int32_t* q_idx, hipStream_t stream) {
    dim3 grid((unsigned)words_per_row, (unsigned)BH);
    transpose_kernel<<<grid, 256, 0, stream>>>(bits, n, words_per_row, q_count, q_idx);
    return hipGetLastError();
}

}  // namespace nabla

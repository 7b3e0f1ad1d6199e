// mask_kernels.hip -- the NABLA block-mask stage on gfx950.
//
// "NABLA: Neighborhood Adaptive Block-Level Attention", section 3.1.2,
// Algorithm 1 (pooling, reduced softmax, CDF binarisation) and section 3.1.3
// (union with the sliding-tile mask), followed by compaction of each mask row
// into an ascending list of kept key blocks.
//
//   pool_kernel      steps 2-5: block means of Q and K (HBM streaming, fp32 sums)
//   logits_kernel    steps 6-7 (logits part): Q_a K_a^T * scale per head, fp32 MFMA
//   select_kernel    steps 7-11: row softmax, sort-free CDF selection by radix
//                    select over the fp32 bit patterns of the probabilities,
//                    STA union, ascending compaction, optional dense/bit rows.
//                    The same kernel also runs the two variant selectors the
//                    CDF rule is measured against: Top-k blocks per row, and
//                    the static STA window alone (Table 1's baseline).
//   transpose_kernel the key-block -> query-block lists the backward pass uses

#include "common.h"
#include "kernels.h"

namespace nabla {

// ---------------------------------------------------------------------------
// Pooling: out[bh][i][d] = (1/N) * sum_{r<N} x[bh][i*N + r][d].
// One workgroup per (block, tensor); 256 threads stream the 64 x D bf16 block
// with 16-byte loads, sum per column in fp32, then reduce the partial rows in
// LDS in a fixed order (deterministic).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k,
                                                   float* __restrict__ qa,
                                                   float* __restrict__ ka) {
    constexpr int CG = D / 8;           // 16-byte column groups per row
    constexpr int RPT = 256 / CG;       // rows covered per pass
    constexpr int PASSES = kBlockN / RPT;
    __shared__ float part[RPT][D];

    const int64_t blk = blockIdx.x;     // flattened bh * n + i
    const uint16_t* src = (blockIdx.y == 0 ? q : k) + blk * (int64_t)kBlockN * D;
    float* dst = (blockIdx.y == 0 ? qa : ka) + blk * D;

    const int t = threadIdx.x;
    const int cg = t % CG, r0 = t / CG;
    // Every Q/K byte is read once here: non-temporal loads stream past the caches.
    uint4 raw[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        raw[p] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                                               src + (int64_t)(r0 + p * RPT) * D + cg * 8)));
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const uint32_t w[4] = {raw[p].x, raw[p].y, raw[p].z, raw[p].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += bf16_bits_to_f32(w[e] & 0xffffu);
            acc[2 * e + 1] += bf16_bits_to_f32(w[e] >> 16);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r0][cg * 8 + e] = acc[e];
    __syncthreads();
    if (t < D) {
        float s = 0.f;
#pragma unroll 8
        for (int r = 0; r < RPT; ++r) s += part[r][t];
        dst[t] = s * (1.0f / kBlockN);
    }
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
// Selection + compaction: one workgroup (256 threads) per query block row.
//
// kSelCdf:  keep j iff G_j <= thr (the NABLA rule, Algorithm 1).
// kSelTopk: keep j iff fewer than k entries of the row are strictly larger than
//           p_j (the k largest, ties at the k-th value kept together). The
//           radix select below runs unchanged with every entry weighing 1
//           instead of its fixed-point mass, and with k - 1 as the bound.
// kSelSta:  keep j iff the STA window of i contains j; no softmax, no selection.
//
// p_j = exp(L_j - max) / sum is computed in fp32. The kept set is
// {j : G_j <= thr} with G_j = mass of entries strictly larger than p_j; it is
// exactly {j : p_j >= tau} for the smallest probability value tau whose
// strictly-larger mass is <= thr. tau is found MSB-first over the uint32 bit
// patterns of the (non-negative) p_j, 8 bits per pass: a 256-bin histogram of
// (count, mass) over the entries matching the prefix so far, a suffix sum over
// bins, and the lowest non-empty bin whose mass-above stays <= thr. Masses are
// summed as 2^-40 fixed-point integers, so the sums are exact and independent
// of the order the atomics land in.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 256;

template <int MODE>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ logits, int n, int keep_all, uint64_t bound, StaParams sta,
    int32_t* __restrict__ kv_count, int32_t* __restrict__ kv_idx,
    uint8_t* __restrict__ dense_mask, uint32_t* __restrict__ bits, int words_per_row) {
    __shared__ float pv[NABLA_MAX_BLOCKS];
    __shared__ unsigned long long hmass[256];
    __shared__ int hcnt[256];
    __shared__ unsigned long long wsum[4];
    __shared__ float wred[4];
    __shared__ int sel_bin;
    __shared__ unsigned long long sel_above;
    __shared__ int wcount[4];

    const int64_t row = blockIdx.x;  // flattened bh * n + i
    const int i = (int)(row % n);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    uint32_t tau = 0;
    if (MODE != kSelSta) {
        const float* L = logits + row * (int64_t)n;
        // 1. load the row, row maximum
        float mx = -INFINITY;
        for (int j = t; j < n; j += kSelThreads) {
            const float x = L[j];
            pv[j] = x;
            mx = fmaxf(mx, x);
        }
        mx = wave_max(mx);
        if (lane == 0) wred[wave] = mx;
        __syncthreads();
        mx = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
        __syncthreads();

        // 2. exponentials and their sum (fixed order per thread, then fixed tree)
        float z = 0.f;
        for (int j = t; j < n; j += kSelThreads) {
            const float e = expf(pv[j] - mx);
            pv[j] = e;
            z += e;
        }
        z = wave_sum(z);
        if (lane == 0) wred[wave] = z;
        __syncthreads();
        z = (wred[0] + wred[1]) + (wred[2] + wred[3]);
        for (int j = t; j < n; j += kSelThreads) pv[j] = pv[j] / z;
        __syncthreads();

        // 3. radix select of tau over the bit patterns of p
        uint32_t prefix = 0, pmask = 0;
        unsigned long long above = 0;  // weight (mass or count) strictly above the prefix range
        if (!keep_all) {
            for (int pass = 0; pass < 4; ++pass) {
                const int shift = 24 - 8 * pass;
                hmass[t] = 0ull;
                hcnt[t] = 0;
                __syncthreads();
                for (int j = t; j < n; j += kSelThreads) {
                    const float p = pv[j];
                    const uint32_t key = __float_as_uint(p);
                    if ((key & pmask) == prefix) {
                        const int d = (key >> shift) & 255;
                        const unsigned long long wgt =
                            MODE == kSelTopk ? 1ull : (unsigned long long)__float2ull_rn(p * 0x1p40f);
                        atomicAdd(&hmass[d], wgt);
                        atomicAdd(&hcnt[d], 1);
                    }
                }
                __syncthreads();
                // Suffix sum over bins: bin t needs the mass of bins > t. Each
                // thread owns bin t; inclusive suffix scan within the wave over
                // lanes (higher lane = higher bin), then add the higher waves.
                unsigned long long m = hmass[t];
                unsigned long long incl = m;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const unsigned long long o = __shfl_down(incl, off);
                    if (lane + off < 64) incl += o;
                }
                if (lane == 0) wsum[wave] = incl;  // total of this wave's 64 bins
                if (t == 0) sel_bin = 256;
                __syncthreads();
                unsigned long long higher = 0;
                for (int w = wave + 1; w < 4; ++w) higher += wsum[w];
                const unsigned long long mass_above_bin = above + higher + (incl - m);
                if (hcnt[t] > 0 && mass_above_bin <= bound) atomicMin(&sel_bin, t);
                __syncthreads();
                const int b = sel_bin;  // always < 256: the highest non-empty bin qualifies
                if (t == b) sel_above = mass_above_bin;
                __syncthreads();
                above = sel_above;
                prefix |= (uint32_t)b << shift;
                pmask |= 0xffu << shift;
                __syncthreads();
            }
        }
        tau = prefix;
    }  // MODE != kSelSta

    // 4. decisions, STA union, ascending compaction
    int32_t* out_idx = kv_idx + row * (int64_t)n;
    int running = 0;
    for (int base = 0; base < n; base += kSelThreads) {
        const int j = base + t;
        bool keep = false;
        if (j < n) {
            if (MODE != kSelSta) keep = keep_all || __float_as_uint(pv[j]) >= tau;
            if (!keep && sta.on) keep = sta_contains(sta, i, j);
        }
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
// The same selection with one wave per row, for rows of n <= 64 * VPL blocks:
// the row stays in registers (lane l holds j = l + 64 r), every reduction is a
// wave shuffle and the radix histograms live in a per-wave LDS slice, so no
// workgroup barrier is needed. Four rows per 256-thread workgroup.
// A histogram bin is one 64-bit word, (weight << kCntBits) + count, so each
// entry costs one LDS atomic; the fields cannot carry into each other (counts
// <= NABLA_MAX_BLOCKS < 2^kCntBits, weights sum to < 2^41). Each wave keeps
// kSelCopies copies of its histogram, lane l adding into copy l % kSelCopies:
// neighbouring key blocks tend to share a bin, and the copies spread those
// same-address atomics over different words.
// ---------------------------------------------------------------------------
constexpr int kSelWaveRows = 4;
constexpr int kSelCopies = 4;
constexpr int kCntBits = 14;
static_assert(NABLA_MAX_BLOCKS < (1 << kCntBits), "bin counts must fit their field");

// Orders this wave's LDS accesses: the compiler may not move LDS operations
// across it, and the wave waits until its own LDS operations have completed.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

template <int MODE, int VPL>
__global__ __launch_bounds__(256) void select_wave_kernel(
    const float* __restrict__ logits, int64_t rows, int n, int keep_all, uint64_t bound,
    StaParams sta, int32_t* __restrict__ kv_count, int32_t* __restrict__ kv_idx,
    uint8_t* __restrict__ dense_mask, uint32_t* __restrict__ bits, int words_per_row) {
    __shared__ __attribute__((aligned(16))) unsigned long long hist[kSelWaveRows][kSelCopies][256];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * kSelWaveRows + wave;
    if (row >= rows) return;  // whole wave; no workgroup barrier follows
    const int i = (int)(row % n);
    float pv[VPL];
    uint32_t tau = 0;
    if (MODE != kSelSta) {
        const float* L = logits + row * (int64_t)n;
        // 1. row maximum; 2. exponentials and their sum; p = e / z
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < VPL; ++r) {
            const int j = lane + 64 * r;
            pv[r] = j < n ? L[j] : -INFINITY;
            mx = fmaxf(mx, pv[r]);
        }
        mx = wave_max(mx);
        float z = 0.f;
#pragma unroll
        for (int r = 0; r < VPL; ++r) {
            const int j = lane + 64 * r;
            const float e = j < n ? expf(pv[r] - mx) : 0.f;
            pv[r] = e;
            z += e;
        }
        z = wave_sum(z);
#pragma unroll
        for (int r = 0; r < VPL; ++r) pv[r] = pv[r] / z;

        // 3. radix select of tau (see select_kernel): lane l owns bins 4l .. 4l+3.
        if (!keep_all) {
            unsigned long long(*hw)[256] = hist[wave];
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
#pragma unroll
                for (int r = 0; r < VPL; ++r) {
                    const int j = lane + 64 * r;
                    const uint32_t key = __float_as_uint(pv[r]);
                    if (j < n && (key & pmask) == prefix) {
                        const int d = (key >> shift) & 255;
                        const unsigned long long wgt =
                            MODE == kSelTopk ? 1ull : (unsigned long long)__float2ull_rn(pv[r] * two40);
                        atomicAdd(&mine_copy[d], (wgt << kCntBits) + 1ull);
                    }
                }
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
                    if (cb[b] > 0 && ab[b] <= bound) cand = 4 * lane + b;
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
#pragma unroll
                    for (int r = 0; r < VPL; ++r) {
                        const int j = lane + 64 * r;
                        const uint32_t key = __float_as_uint(pv[r]);
                        const bool is_c = j < n && (key & pmask) == prefix;
                        const unsigned long long bal = __ballot(is_c);
                        if (is_c) {
                            const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
                            hc[pos] = key;
                            hm[pos] = MODE == kSelTopk ? 1ull
                                                       : (unsigned long long)__float2ull_rn(pv[r] * 0x1p40f);
                        }
                        base += __popcll(bal);
                    }
                    wave_lds_sync();
                    const uint32_t my_key = lane < csel ? hc[lane] : 0u;
                    unsigned long long acc = 0;
                    for (int m2 = 0; m2 < csel; ++m2)
                        if (hc[m2] > my_key) acc += hm[m2];
                    uint32_t t = (lane < csel && above + acc <= bound) ? my_key : 0xffffffffu;
#pragma unroll
                    for (int off = 32; off >= 1; off >>= 1) t = min(t, (uint32_t)__shfl_xor((int)t, off));
                    prefix = t;  // the largest candidate always qualifies
                    wave_lds_sync();
                    break;
                }
            }
            tau = prefix;
        }
    }

    // 4. decisions, STA union, ascending compaction (chunk r = blocks 64r .. 64r+63)
    int32_t* out_idx = kv_idx + row * (int64_t)n;
    int running = 0;
#pragma unroll
    for (int r = 0; r < VPL; ++r) {
        if (64 * r < n) {
            const int j = lane + 64 * r;
            bool keep = false;
            if (j < n) {
                if (MODE != kSelSta) keep = keep_all || __float_as_uint(pv[r]) >= tau;
                if (!keep && sta.on) keep = sta_contains(sta, i, j);
            }
            const unsigned long long bal = __ballot(keep);
            if (keep) out_idx[running + __popcll(bal & ((1ull << lane) - 1ull))] = j;
            if (dense_mask && j < n) dense_mask[row * (int64_t)n + j] = keep ? 1 : 0;
            if (bits && lane < 2) {
                const int word = 2 * r + lane;
                if (word < words_per_row)
                    bits[row * (int64_t)words_per_row + word] = (uint32_t)(bal >> (32 * lane));
            }
            running += __popcll(bal);
        }
    }
    if (lane == 0) kv_count[row] = running;
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
hipError_t launch_pool(const void* q, const void* k, float* qa, float* ka, int64_t nblocks, int D,
                       hipStream_t stream) {
    dim3 grid((unsigned)nblocks, 2);
    if (D == 128)
        pool_kernel<128><<<grid, 256, 0, stream>>>((const uint16_t*)q, (const uint16_t*)k, qa, ka);
    else
        pool_kernel<64><<<grid, 256, 0, stream>>>((const uint16_t*)q, (const uint16_t*)k, qa, ka);
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

hipError_t launch_select(int mode, const float* logits, int64_t BH, int n, int keep_all,
                         uint64_t bound, const StaParams& sta, int32_t* kv_count, int32_t* kv_idx,
                         uint8_t* dense_mask, uint32_t* bits, int words_per_row,
                         hipStream_t stream) {
    const int64_t rows = BH * n;
    // Content selectors on rows of up to 2048 blocks: one wave per row (values in
    // registers). The STA window alone has no per-row reduction and runs faster
    // with a workgroup per row.
    if (n <= 2048 && mode != kSelSta) {
        const unsigned wgrid = (unsigned)((rows + kSelWaveRows - 1) / kSelWaveRows);
#define NABLA_SEL_WAVE(MODE_, VPL_)                                                             \
    select_wave_kernel<MODE_, VPL_><<<wgrid, 64 * kSelWaveRows, 0, stream>>>(                   \
        logits, rows, n, keep_all, bound, sta, kv_count, kv_idx, dense_mask, bits, words_per_row)
#define NABLA_SEL_WAVE_MODES(VPL_)                                                              \
    do {                                                                                        \
        if (mode == kSelTopk) NABLA_SEL_WAVE(kSelTopk, VPL_);                                   \
        else NABLA_SEL_WAVE(kSelCdf, VPL_);                                                     \
    } while (0)
        if (n <= 512) NABLA_SEL_WAVE_MODES(8);
        else if (n <= 1024) NABLA_SEL_WAVE_MODES(16);
        else if (n <= 1280) NABLA_SEL_WAVE_MODES(20);
        else NABLA_SEL_WAVE_MODES(32);
#undef NABLA_SEL_WAVE_MODES
#undef NABLA_SEL_WAVE
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)rows;
    if (mode == kSelTopk)
        select_kernel<kSelTopk><<<grid, kSelThreads, 0, stream>>>(
            logits, n, keep_all, bound, sta, kv_count, kv_idx, dense_mask, bits, words_per_row);
    else if (mode == kSelSta)
        select_kernel<kSelSta><<<grid, kSelThreads, 0, stream>>>(
            logits, n, keep_all, bound, sta, kv_count, kv_idx, dense_mask, bits, words_per_row);
    else
        select_kernel<kSelCdf><<<grid, kSelThreads, 0, stream>>>(
            logits, n, keep_all, bound, sta, kv_count, kv_idx, dense_mask, bits, words_per_row);
    return hipGetLastError();
}

hipError_t launch_transpose(const uint32_t* bits, int64_t BH, int n, int words_per_row,
                            int32_t* q_count, int32_t* q_idx, hipStream_t stream) {
    dim3 grid((unsigned)words_per_row, (unsigned)BH);
    transpose_kernel<<<grid, 256, 0, stream>>>(bits, n, words_per_row, q_count, q_idx);
    return hipGetLastError();
}

}  // namespace nabla

// attn_fwd.hip -- block-sparse flash-attention forward on gfx950.
//
// Computes eq. (4) of "NABLA: Neighborhood Adaptive Block-Level Attention"
// (section 2.2) with the NABLA/STA block mask of section 3.1.3: each query
// block attends only to the key blocks of its kept list. Online softmax over
// the kept blocks (flash-attention style), bf16 MFMA with fp32 accumulation.
//
// A wave owns 32 query rows of one 64-row query block. Per kept key block j:
//   S^T = K Q^T: A operand = K rows from LDS, B operand = Q^T in registers;
//   O^T += V^T P^T: B operand = P^T straight from the S^T accumulators (their
//   rows become the contraction slots), A operand = V^T read from the
//   row-major V tile with the transposing LDS read (ds_read_b64_tr_b16),
//   which hands each lane one column of four consecutive V rows -- matching
//   the accumulator's slot map, so neither P nor V is ever shuffled.
// K and V tiles are prefetched two blocks ahead into registers with plain
// 16-byte loads and written to padded LDS rows after the current block's
// reads (the pair kernel below double-buffers them), so global latency
// overlaps a whole block of compute. exp2 is used
// with log2(e) folded into the scale, and the output is rescaled only when a
// row maximum grows by more than 2^8; the block maximum is formed only when
// the exponentials taken against the running maximum could have reached that
// (softmax_lazy), which leaves every result unchanged and keeps the max
// reduction out of most steps. The output is divided by the sum of the bf16
// weights that entered the PV product (LSE uses the fp32 sum); that sum comes
// from four small MFMAs per block on the PV product's own B operands
// (weight_sum_operand). A wave raises its issue priority for the
// duration of a block step: a SIMD holds two waves, and one that is computing
// then goes ahead of one that is staging tiles or issuing its next loads,
// whose latency the prefetch already covers (measured: 3-5% faster).
//
// Two kernels share that per-block step:
//   attn_fwd_kernel       one query block per workgroup (2 waves);
//   attn_fwd_pair_kernel  two query blocks per workgroup (4 waves): the same
//                         tile position in two consecutive frames (blocks i
//                         and i + F in the block order of section 3.1.1),
//                         whose kept lists overlap strongly. The workgroup
//                         walks the ascending union of both lists, loads each
//                         K/V tile once, and each pair of waves computes only
//                         the blocks of its own list -- in the same order as
//                         the single kernel, so the results are bitwise equal.
//                         For D = 128 it moves its tiles by direct-to-LDS
//                         loads into swizzled unpadded rows (see its
//                         specialization below); D = 64 stages them through
//                         registers like the single kernel.
// The one-block kernel is bound by K/V tile traffic from beyond L2 (each kept
// pair reads a 32 KB tile pair); sharing tiles between the two blocks of a
// pair removes the loads of their common blocks, after which the pair kernel
// is bound by its block step (the softmax VALU work that does not co-issue
// with MFMA) and by waits on union steps that only one block keeps.

#include "common.h"
#include "kernels.h"

namespace nabla {

namespace {

constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

template <int D>
struct Tile {
    static constexpr int CPR = D / 8;            // 16-byte chunks per row
    static constexpr int KSTB = 2 * D + 16;      // K row stride (bytes): 16-byte pad
    static constexpr int VSTB = 2 * D + 64;      // V row stride (bytes): 64-byte pad
    static constexpr int CHUNKS = kBlockN * CPR; // 16-byte chunks per tile
};

// Per-wave state of 32 query rows.
template <int D>
struct RowState {
    static constexpr int KK = D / 16;  // MFMA k-steps over the head dimension
    static constexpr int DT = D / 32;  // 32-row d tiles of O^T
    bf16x8_t qf[KK];                   // Q^T as the B operand
    f32x16_t oacc[DT];                 // O^T accumulators
    // m_run: running maximum (log2 units), equal in both lanes of a query
    // column; l_run: sum of fp32 probabilities (for LSE), this lane's share of
    // the column's keys (the epilogue adds the two lanes' shares); w_run: sum
    // of the bf16-rounded probabilities that feed the PV product (the
    // output's normaliser) over all of the column's keys, in both lanes, up to
    // the previous block; w_pend: the last block's weight sum, added at the
    // start of the next block (its MFMA has finished by then; read at the end
    // of its own block it would stall the wave until the PV products drain).
    float m_run, l_run, w_run, w_pend;
};

// Lane l of a wave: query column c = l % 32, half h = l / 32.
template <int D>
__device__ __forceinline__ void load_rows(RowState<D>& st, const uint16_t* qrow_ptr, int h) {
#pragma unroll
    for (int kk = 0; kk < RowState<D>::KK; ++kk)
        st.qf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow_ptr + 16 * kk + 8 * h));
#pragma unroll
    for (int t = 0; t < RowState<D>::DT; ++t) st.oacc[t] = zero16();
    st.m_run = -INFINITY;
    st.l_run = 0.f;
    st.w_run = 0.f;
    st.w_pend = 0.f;
}

// Maximum over the lane pair (l, l ^ 32) that holds one query column: the
// VALU half-swap of gfx950 exchanges the two 32-lane halves without an LDS
// round trip (lane l < 32 finds x[l + 32] in the second result, lane l >= 32
// finds x[l - 32] in the first; each also sees its own value).
__device__ __forceinline__ float pair_max(float x) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(x, __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
}

// Online softmax of one block for query column c (keys split over this lane
// and lane ^ 32), with the output rescaled only when some row's maximum grows
// by more than 2^8 (probabilities then stay at most 2^8). The exponentials are
// first taken against the running maximum: each is >= 0, so a lane sum of at
// most 2^7 bounds all of its probabilities by 2^7, and a maximum that grew by
// more than 2^8 would have given a probability near 2^8 or above (the margin
// covers the rounding of the scaled logit and of exp2). Only when some lane's
// sum exceeds 2^7 (or is not finite, as on a row's first block) is the block
// maximum formed; if it grew by more than 2^8 the output is rescaled and the
// exponentials are taken again. The running maximum, and so every result, is
// the same as forming the block maximum first on every block.
template <int D>
__device__ __forceinline__ void softmax_lazy(RowState<D>& st, const f32x16_t (&s)[2], uint32_t (&pw)[2][8],
                                             float& rs, float scale_log2) {
    constexpr int DT = RowState<D>::DT;
    auto exps = [&]() {
        rs = -0.f;  // x + (-0) == x for every x, so the first add folds away
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // One rounding (fused), as the contracted form elsewhere.
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][2 * e], scale_log2, -st.m_run));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][2 * e + 1], scale_log2, -st.m_run));
                rs += p0 + p1;
                pw[kt][e] = pack_bf16x2(p0, p1);
            }
    };
    exps();
    if (__builtin_amdgcn_ballot_w64(!(rs <= 128.0f))) {
        float mx = s[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = __builtin_fmaxf(mx, s[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[1][r]);
        mx = pair_max(mx) * scale_log2;
        const bool grow = mx > st.m_run + kRescaleLog2;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? mx : st.m_run;
            const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
            st.l_run *= alpha;
            st.w_run *= alpha;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) st.oacc[t][r] *= alpha;
            st.m_run = m_new;
            exps();
        }
    }
}

// Sum of the bf16 weights by MFMA. v_mfma_f32_16x16x32_bf16 reads B (32 x 16)
// as lane l = 16 g + n supplying column n, k-slots 8 g .. 8 g + 7, and A
// (16 x 32) as lane l supplying row l % 16 at the same k-slots; lane l gets
// C[4 g + i][n], i = 0..3. Fed with the PV product's B operand of one 16-key
// slice, whose lane l holds 8 weights of query column l % 32 (half l / 32 of
// the slice's keys), the slots of group g belong to query n + 16 (g % 2). An
// A operand of ones at slot groups g with g % 2 == (row / 4) % 2 and zeros
// elsewhere -- in lane l, ones iff bit 4 of l equals bit 2 -- makes every
// C[4 g + i][n] the slice's full weight sum of query n + 16 (g % 2), which is
// lane l's own column l % 32. Four such products per block replace 16
// v_dot2c_f32_bf16, which do not co-execute with MFMA. Both helpers give the
// same operand: the second reads the lane id through an opaque instruction, so
// a kernel without registers to spare rebuilds it at each use instead of
// holding four registers across its loop.
__device__ __forceinline__ bf16x8_t weight_sum_operand(uint32_t l) {
    const uint32_t w = ((l >> 4) & 1) == ((l >> 2) & 1) ? 0x3f803f80u : 0u;
    return as_bf16x8(make_uint4(w, w, w, w));
}
__device__ __forceinline__ bf16x8_t weight_sum_operand_here() {
    uint32_t l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return weight_sum_operand(l);
}

// One kept key block: K tile at kbase (lane base for the S^T A operand), V
// tile at vbase (lane base for the transposing V^T reads).
// DEEP: read the K fragments further ahead of their products (all of tile 0,
// then tile 1's reads interleaved with tile 0's MFMAs, the order pinned with
// scheduling groups) -- 15 more registers; used where they fit 2 waves/SIMD.
template <int D, bool DEEP>
__device__ __forceinline__ void block_step(RowState<D>& st, const char* kbase, const char* vbase,
                                           float scale_log2, bf16x8_t wsel) {
    using T = Tile<D>;
    constexpr int KK = RowState<D>::KK, DT = RowState<D>::DT;
    __builtin_amdgcn_s_setprio(1);  // back to 0 at the end of the step
    st.w_run += st.w_pend;

    // S^T (64 keys x 32 queries) as two 32 x 32 tiles.
    f32x16_t s[2];
    if constexpr (DEEP) {
        bf16x8_t a0[KK], a1[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            a0[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(kbase + 32 * kk));
        s[0] = zero16();
        s[1] = zero16();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            a1[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(kbase + 32 * T::KSTB + 32 * kk));
            s[0] = mfma_32x32x16(a0[kk], st.qf[kk], s[0]);
        }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) s[1] = mfma_32x32x16(a1[kk], st.qf[kk], s[1]);
        // Groups: KK LDS reads, then (1 MFMA, 1 LDS read) x KK, then KK MFMAs.
        __builtin_amdgcn_sched_group_barrier(0x100, KK, 0);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, KK, 0);
    } else {
        // A fragments of each tile read before its products (the compiler keeps
        // about two reads in flight).
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            bf16x8_t a[KK];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(kbase + 32 * kt * T::KSTB + 32 * kk));
            s[kt] = zero16();
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) s[kt] = mfma_32x32x16(a[kk], st.qf[kk], s[kt]);
        }
    }

    float rs;
    uint32_t pw[2][8];  // bf16 probabilities, B operands of the PV product
    softmax_lazy(st, s, pw, rs, scale_log2);
    st.l_run += rs;
    f32x4_t wsum = {0.f, 0.f, 0.f, 0.f};

    // O^T += V^T P^T. For key tile kt and half u, B = S^T registers 8u..8u+7:
    // slot s is key 32kt + 16u + 8*(s/4) + 4h + s%4; the transposing reads
    // of rows 32kt + 16u + {0, 8} + 4h + jj deliver V^T with the same map.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bf16x8_t b = as_bf16x8(make_uint4(pw[kt][4 * u], pw[kt][4 * u + 1],
                                                    pw[kt][4 * u + 2], pw[kt][4 * u + 3]));
            wsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wsel, b, wsum, 0, 0, 0);
            const char* vrow = vbase + (32 * kt + 16 * u) * T::VSTB;
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16_t*)(vrow + 64 * t));
                const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16_t*)(vrow + 8 * T::VSTB + 64 * t));
                const uint2 ulo = __builtin_bit_cast(uint2, lo);
                const uint2 uhi = __builtin_bit_cast(uint2, hi);
                st.oacc[t] = mfma_32x32x16(as_bf16x8(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y)), b,
                                           st.oacc[t]);
            }
        }
    st.w_pend = wsum[0];
    __builtin_amdgcn_s_setprio(0);
}

// Epilogue: O[query][d] = O^T[d][query] / w. The lane holds query row `qrow`
// and d = 32t + 8g + 4h + e for register 4g + e of tile t.
template <int D>
__device__ __forceinline__ void store_rows(const RowState<D>& st, int64_t head, int64_t qrow, int h,
                                           void* __restrict__ o, int o_fp32, float* __restrict__ lse,
                                           int64_t lse_index) {
    constexpr int DT = RowState<D>::DT;
    const float w_sum = st.w_run + st.w_pend;
    const float l_sum = st.l_run + __shfl_xor(st.l_run, 32);
    const float inv_l = w_sum > 0.f ? 1.0f / w_sum : 0.f;
    if (o_fp32) {
        float* orow = static_cast<float*>(o) + head + qrow * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<float4*>(orow + 32 * t + 8 * g + 4 * h) =
                    make_float4(st.oacc[t][4 * g + 0] * inv_l, st.oacc[t][4 * g + 1] * inv_l,
                                st.oacc[t][4 * g + 2] * inv_l, st.oacc[t][4 * g + 3] * inv_l);
    } else {
        uint16_t* orow = static_cast<uint16_t*>(o) + head + qrow * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 w;
                w.x = pack_bf16x2(st.oacc[t][4 * g + 0] * inv_l, st.oacc[t][4 * g + 1] * inv_l);
                w.y = pack_bf16x2(st.oacc[t][4 * g + 2] * inv_l, st.oacc[t][4 * g + 3] * inv_l);
                *reinterpret_cast<uint2*>(orow + 32 * t + 8 * g + 4 * h) = w;
            }
    }
    if (lse && h == 0)
        lse[lse_index] = l_sum > 0.f ? (st.m_run + __log2f(l_sum)) * kLn2 : -INFINITY;
}

// Lane bases for LDS reads (everything else is an immediate offset).
// K rows for the S^T A operand: row 32 kt + c, bytes 32 kk + 16 h.
template <int D>
__device__ __forceinline__ const char* k_lane_base(const char* sK, int lane) {
    return sK + (lane & 31) * Tile<D>::KSTB + 16 * (lane >> 5);
}
// V^T via the transposing read: this lane supplies the address of row
// rbase + 4h + (lane % 16) / 4, columns 32 dt + 16 ((lane / 16) % 2) +
// 4 (lane % 4) .. +3, and receives V[rbase + 4h + jj][32 dt + lane % 32]
// for jj = 0..3 (rbase = 32 kt + 16 u, plus 8 for the upper four slots).
template <int D>
__device__ __forceinline__ const char* v_lane_base(const char* sV, int lane) {
    return sV + (4 * (lane >> 5) + ((lane & 15) >> 2)) * Tile<D>::VSTB +
           2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
}

}  // namespace

template <int D>
__global__ __launch_bounds__(128, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int S, int n, const int32_t* __restrict__ kv_count,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ order, XcdSchedule sched,
    float scale_log2, void* __restrict__ o, int o_fp32, float* __restrict__ lse) {
    using T = Tile<D>;
    constexpr int L = T::CHUNKS / 128;  // 16-byte chunks per thread per tile
    __shared__ __attribute__((aligned(16))) char sK[kBlockN * T::KSTB];
    __shared__ __attribute__((aligned(16))) char sV[kBlockN * T::VSTB];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, c = lane & 31;
    const int64_t item = scheduled_item(sched, order, blockIdx.x);
    if (item < 0) return;  // padding slot (whole workgroup)
    const int64_t bh = item / n;
    const int qb = (int)(item % n);
    int cnt = kv_count[item];
    cnt = cnt < 0 ? 0 : (cnt > n ? n : cnt);
    const int32_t* list = kv_idx + item * (int64_t)n;
    const int64_t head = bh * (int64_t)S * D;
    const uint16_t* kh = k + head;
    const uint16_t* vh = v + head;

    const int64_t qrow = (int64_t)qb * kBlockN + wave * 32 + c;
    RowState<D> st;
    load_rows<D>(st, q + head + qrow * D, h);

    // Staging: thread chunk e = tid + 128 i covers row e / CPR, chunk e % CPR.
    u32x4_t kr[L], vr[L];
#define NABLA_FETCH(IT)                                                        \
    do {                                                                       \
        int jj_ = list[(IT)];                                                  \
        jj_ = (unsigned)jj_ < (unsigned)n ? jj_ : 0;                           \
        const int64_t off_ = (int64_t)jj_ * kBlockN * D;                       \
        _Pragma("unroll") for (int i_ = 0; i_ < L; ++i_) {                     \
            const int e_ = tid + 128 * i_;                                     \
            kr[i_] = *reinterpret_cast<const u32x4_t*>(kh + off_ + e_ * 8);    \
            vr[i_] = *reinterpret_cast<const u32x4_t*>(vh + off_ + e_ * 8);    \
        }                                                                      \
    } while (0)
#define NABLA_STAGE()                                                          \
    do {                                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < L; ++i_) {                     \
            const int e_ = tid + 128 * i_;                                     \
            const int r_ = e_ / T::CPR, ch_ = e_ % T::CPR;                     \
            *reinterpret_cast<u32x4_t*>(sK + r_ * T::KSTB + 16 * ch_) = kr[i_];\
            *reinterpret_cast<u32x4_t*>(sV + r_ * T::VSTB + 16 * ch_) = vr[i_];\
        }                                                                      \
    } while (0)

    const char* kbase = k_lane_base<D>(sK, lane);
    const char* vbase = v_lane_base<D>(sV, lane);

    if (cnt > 0) {
        NABLA_FETCH(0);
        NABLA_STAGE();
        if (cnt > 1) NABLA_FETCH(1);
        __syncthreads();
    }
    for (int it = 0; it < cnt; ++it) {
        block_step<D, false>(st, kbase, vbase, scale_log2, weight_sum_operand_here());
        if (it + 1 < cnt) {
            __syncthreads();  // every wave has read K_j and V_j
            NABLA_STAGE();  // block it+1, fetched one iteration ago
            if (it + 2 < cnt) NABLA_FETCH(it + 2);
            __syncthreads();
        }
    }

#undef NABLA_FETCH
#undef NABLA_STAGE
    store_rows<D>(st, head, qrow, h, o, o_fp32, lse, bh * (int64_t)S + qrow);
}

// Two query blocks per workgroup: waves 0-1 serve block A, waves 2-3 block B
// (B = A + F, the same tile in the next frame; -1 when A is in the last frame
// of an odd frame count). The workgroup walks the ascending union of the two
// kept lists with two cursors: `cur` for the block being computed, `pre` two
// union steps ahead for the prefetch. Each union step carries two flags (in
// A's list, in B's list); a pair of waves computes a step only if its flag is
// set, so each block sees exactly its own kept blocks in ascending order.
// The K/V tiles are double-buffered in LDS (75.8 KB at D = 128; two workgroups
// still fit a CU): a wave stages the next step into the other buffer right
// after computing the current one, and one barrier per step suffices.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_pair_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int S, int n, int F, const int32_t* __restrict__ kv_count,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ order, XcdSchedule sched,
    float scale_log2, void* __restrict__ o, int o_fp32, float* __restrict__ lse) {
    using T = Tile<D>;
    constexpr int L = T::CHUNKS / 256;  // 16-byte chunks per thread per tile
    constexpr int KB = kBlockN * T::KSTB, VB = kBlockN * T::VSTB;
    __shared__ __attribute__((aligned(16))) char sK[2 * KB];
    __shared__ __attribute__((aligned(16))) char sV[2 * VB];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int grp = wave >> 1;  // 0: block A, 1: block B
    const int h = lane >> 5, c = lane & 31;
    const int64_t pair = scheduled_item(sched, order, blockIdx.x);
    if (pair < 0) return;  // padding slot (whole workgroup)
    // Pair p of a head: frames 2s and 2s+1 of tile position tp.
    const int np = sched.n;
    const int64_t bh = pair / np;
    const int p = (int)(pair % np);
    const int s2 = 2 * (p / F), tp = p % F;
    const int qa = s2 * F + tp;
    const int qbB = qa + F < n ? qa + F : -1;
    const int64_t itemA = bh * (int64_t)n + qa;
    const int64_t itemB = bh * (int64_t)n + (qbB < 0 ? qa : qbB);
    int cntA = kv_count[itemA];
    cntA = cntA < 0 ? 0 : (cntA > n ? n : cntA);
    int cntB = qbB < 0 ? 0 : kv_count[itemB];
    cntB = cntB < 0 ? 0 : (cntB > n ? n : cntB);
    const int32_t* listA = kv_idx + itemA * (int64_t)n;
    const int32_t* listB = kv_idx + itemB * (int64_t)n;
    const int64_t head = bh * (int64_t)S * D;
    const uint16_t* kh = k + head;
    const uint16_t* vh = v + head;

    const int my_qb = grp ? qbB : qa;
    const bool active = my_qb >= 0;
    const int64_t qrow = (int64_t)(active ? my_qb : qa) * kBlockN + (wave & 1) * 32 + c;
    RowState<D> st;
    load_rows<D>(st, q + head + qrow * D, h);
    const bf16x8_t wsel = weight_sum_operand(lane);

    // Union cursor: positions in both lists; the next element of each (n = end).
    struct Cursor {
        int ia, ib;
    };
    auto entry = [&](const int32_t* list, int i, int cntL) -> int {
        if (i >= cntL) return n;
        const int j = list[i];
        return (unsigned)j < (unsigned)n ? j : 0;
    };
    // Advance a cursor by one union step; returns the block and its flags.
    auto step = [&](Cursor& cu, int& j, int& flags) {
        const int ja = entry(listA, cu.ia, cntA);
        const int jb = entry(listB, cu.ib, cntB);
        j = ja < jb ? ja : jb;
        flags = (ja == j ? 1 : 0) | (jb == j ? 2 : 0);
        cu.ia += (flags & 1);
        cu.ib += (flags & 2) >> 1;
    };

    u32x4_t kr[L], vr[L];
#define NABLA_PFETCH(J)                                                        \
    do {                                                                       \
        const int64_t off_ = (int64_t)(J) * kBlockN * D;                       \
        _Pragma("unroll") for (int i_ = 0; i_ < L; ++i_) {                     \
            const int e_ = tid + 256 * i_;                                     \
            kr[i_] = *reinterpret_cast<const u32x4_t*>(kh + off_ + e_ * 8);    \
            vr[i_] = *reinterpret_cast<const u32x4_t*>(vh + off_ + e_ * 8);    \
        }                                                                      \
    } while (0)
#define NABLA_PSTAGE(B)                                                        \
    do {                                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < L; ++i_) {                     \
            const int e_ = tid + 256 * i_;                                     \
            const int r_ = e_ / T::CPR, ch_ = e_ % T::CPR;                     \
            char* kd_ = sK + (B) * KB + r_ * T::KSTB + 16 * ch_;                 \
            char* vd_ = sV + (B) * VB + r_ * T::VSTB + 16 * ch_;                 \
            *reinterpret_cast<u32x4_t*>(kd_) = kr[i_];                         \
            *reinterpret_cast<u32x4_t*>(vd_) = vr[i_];                         \
        }                                                                      \
    } while (0)

    const char* kbase = k_lane_base<D>(sK, lane);
    const char* vbase = v_lane_base<D>(sV, lane);

    // Union length: |A| + |B| - |A and B|, counted by walking the cursor.
    Cursor pre{0, 0};
    int f_cur = 0, f_next = 0;  // flags of the staged step and of the step in flight
    int j_tmp;
    if (cntA + cntB > 0) {
        int buf = 0;
        step(pre, j_tmp, f_cur);
        NABLA_PFETCH(j_tmp);
        NABLA_PSTAGE(0);
        if (pre.ia < cntA || pre.ib < cntB) {
            step(pre, j_tmp, f_next);
            NABLA_PFETCH(j_tmp);
        }
        __syncthreads();
        for (;;) {
            const int mine = grp ? (f_cur & 2) : (f_cur & 1);
            if (mine && active)
                block_step<D, true>(st, kbase + buf * KB, vbase + buf * VB, scale_log2, wsel);
            if (f_next == 0) break;  // the computed step was the last one
            // The other buffer's readers finished before the last barrier.
            NABLA_PSTAGE(buf ^ 1);  // the step fetched one iteration ago
            f_cur = f_next;
            f_next = 0;
            if (pre.ia < cntA || pre.ib < cntB) {
                step(pre, j_tmp, f_next);
                NABLA_PFETCH(j_tmp);
            }
            __syncthreads();
            buf ^= 1;
        }
    }

#undef NABLA_PFETCH
#undef NABLA_PSTAGE
    if (active) store_rows<D>(st, head, qrow, h, o, o_fp32, lse, bh * (int64_t)S + qrow);
}

// ---------------------------------------------------------------------------
// attn_fwd_pair_kernel for D = 128: the same walk and block step as the
// generic pair kernel, but the K/V tiles move global -> LDS by direct-to-LDS
// loads (global_load_lds_dwordx4: each wave instruction fills 1 KB = four
// 256-byte tile rows), with no staging registers and no LDS stores in the
// waves' instruction streams. Tile rows are unpadded; the 16-byte chunk ch of
// row r is stored at ch ^ (r % 16) in the K tile and at ch ^ 4 (r % 4) in the
// V tile, which keeps the K row reads (ds_read_b128, 16 consecutive rows) and
// the V transposing reads (ds_read_b64_tr_b16, four chunks of four
// consecutive rows) free of bank conflicts; each lane's read addresses are
// computed once (XOR patterns). The next union step's tiles are requested
// into the other buffer at the start of a step and waited for at its end (one
// barrier per step). The two buffers are separate arrays and the loop is
// unrolled by two, so every LDS access names its buffer statically and the
// compiler's wait counting never makes a read wait for loads into the other
// buffer. Same operations in the same order as attn_fwd_kernel: bitwise equal.
// ---------------------------------------------------------------------------
namespace {
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;
// s_waitcnt vmcnt(0), other counters unconstrained.
__device__ __forceinline__ void dma_wait_all() {
    __builtin_amdgcn_s_waitcnt((0 & 15) | ((0 >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier that waits for this wave's LDS accesses (lgkmcnt 0) but
// not for direct-to-LDS loads in flight (the caller waits for those), and that
// no memory access crosses.
__device__ __forceinline__ void dma_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// A workgroup-uniform pointer kept in scalar registers and opaque to the
// optimiser, so a 32-bit lane offset added to it selects the scalar-base +
// vector-offset address form.
__device__ __forceinline__ const char* uniform_cptr(const char* p) {
    uint64_t x = reinterpret_cast<uint64_t>(p);
    asm volatile("" : "+s"(x));
    return reinterpret_cast<const char*>(x);
}
// Mark a value as produced here: keeps a 32-bit offset from being folded into
// a hoisted 64-bit pointer, and keeps loop-invariant loads from being waited
// for inside the loop.
template <typename T_>
__device__ __forceinline__ void settle_v(T_& x) { asm volatile("" : "+v"(x)); }

// One kept block from swizzled tiles: K row reads at kl[kk] (+ 8192 for the
// second 32-key tile), V transposing reads at vl[t] (+ row offsets).
__device__ __forceinline__ void block_step_swz(RowState<128>& st, const char* kt0, const char* vt0,
                                               const uint32_t (&kl)[8], const uint32_t (&vl)[4],
                                               float scale_log2, bf16x8_t wsel) {
    constexpr int KK = 8, DT = 4;
    __builtin_amdgcn_s_setprio(1);
    st.w_run += st.w_pend;
    // S^T: all of key tile 0's K fragments read first, then tile 1's reads
    // interleaved with tile 0's products (order pinned with scheduling groups).
    f32x16_t s[2];
    {
        bf16x8_t a0[KK], a1[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) a0[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(kt0 + kl[kk]));
        s[0] = zero16();
        s[1] = zero16();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            a1[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(kt0 + 8192 + kl[kk]));
            s[0] = mfma_32x32x16(a0[kk], st.qf[kk], s[0]);
        }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) s[1] = mfma_32x32x16(a1[kk], st.qf[kk], s[1]);
        __builtin_amdgcn_sched_group_barrier(0x100, KK, 0);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, KK, 0);
    }
    float rs;
    uint32_t pw[2][8];
    softmax_lazy(st, s, pw, rs, scale_log2);
    st.l_run += rs;
    f32x4_t wsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bf16x8_t b = as_bf16x8(make_uint4(pw[kt][4 * u], pw[kt][4 * u + 1],
                                                    pw[kt][4 * u + 2], pw[kt][4 * u + 3]));
            wsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wsel, b, wsum, 0, 0, 0);
            const char* vrow = vt0 + (32 * kt + 16 * u) * 256;
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(vrow + vl[t]));
                const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(vrow + 8 * 256 + vl[t]));
                const uint2 ulo = __builtin_bit_cast(uint2, lo);
                const uint2 uhi = __builtin_bit_cast(uint2, hi);
                st.oacc[t] = mfma_32x32x16(as_bf16x8(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y)), b, st.oacc[t]);
            }
        }
    st.w_pend = wsum[0];
    __builtin_amdgcn_s_setprio(0);
}
}  // namespace

template <>
__global__ __launch_bounds__(256, 2) void attn_fwd_pair_kernel<128>(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int S, int n, int F, const int32_t* __restrict__ kv_count,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ order, XcdSchedule sched,
    float scale_log2, void* __restrict__ o, int o_fp32, float* __restrict__ lse) {
    constexpr int D = 128;
    constexpr int TB = kBlockN * 2 * D;  // 16 KB per tile
    __shared__ __attribute__((aligned(1024))) char sK0[TB];
    __shared__ __attribute__((aligned(1024))) char sV0[TB];
    __shared__ __attribute__((aligned(1024))) char sK1[TB];
    __shared__ __attribute__((aligned(1024))) char sV1[TB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 1;
    const int h = lane >> 5, c = lane & 31;
    const int64_t pair = scheduled_item(sched, order, blockIdx.x);
    if (pair < 0) return;
    const int np = sched.n;
    const int64_t bh = pair / np;
    const int p = (int)(pair % np);
    const int s2 = 2 * (p / F), tp = p % F;
    const int qa = s2 * F + tp;
    const int qbB = qa + F < n ? qa + F : -1;
    const int64_t itemA = bh * (int64_t)n + qa;
    const int64_t itemB = bh * (int64_t)n + (qbB < 0 ? qa : qbB);
    int cntA = kv_count[itemA];
    cntA = cntA < 0 ? 0 : (cntA > n ? n : cntA);
    int cntB = qbB < 0 ? 0 : kv_count[itemB];
    cntB = cntB < 0 ? 0 : (cntB > n ? n : cntB);
    const int32_t* listA = kv_idx + itemA * (int64_t)n;
    const int32_t* listB = kv_idx + itemB * (int64_t)n;
    const int64_t head = bh * (int64_t)S * D;
    const char* kh = reinterpret_cast<const char*>(k + head);
    const char* vh = reinterpret_cast<const char*>(v + head);

    const int my_qb = grp ? qbB : qa;
    const bool active = my_qb >= 0;
    const int64_t qrow = (int64_t)(active ? my_qb : qa) * kBlockN + (wave & 1) * 32 + c;
    RowState<D> st;
    load_rows<D>(st, q + head + qrow * D, h);
    const bf16x8_t wsel = weight_sum_operand(lane);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) settle_v(st.qf[kk]);

    // Read addresses (bytes within a tile).
    uint32_t kl[8], vl[4];
    {
        const int x = c & 15;
        const uint32_t kb = (uint32_t)(c * 256 + 16 * (h ^ (x & 1)) + 32 * (x >> 1));
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) kl[kk] = kb ^ (32u * kk);
        const int y = (lane & 15) >> 2, g = (lane >> 4) & 1;
        const uint32_t vb = (uint32_t)((4 * h + y) * 256 + 16 * (2 * g + ((lane & 3) >> 1)) + 8 * (lane & 1) + 64 * y);
#pragma unroll
        for (int t = 0; t < 4; ++t) vl[t] = vb ^ (64u * t);
    }
    // Direct-to-LDS loads: wave w fills row groups m = w + 4 i (rows 4m .. 4m + 3);
    // lane L writes physical chunk L % 16 of row 4m + L / 16 and fetches the
    // logical chunk stored there.
    uint32_t gk, gv;
    {
        const int r = 4 * wave + (lane >> 4);
        gk = (uint32_t)(r * 256 + 16 * ((lane & 15) ^ (r & 15)));
        gv = (uint32_t)(r * 256 + 16 * ((lane & 15) ^ (4 * (r & 3))));
    }
    auto dma = [&](int j, char* dk_, char* dv_) {
        const char* ks = uniform_cptr(kh + (int64_t)j * TB);
        const char* vs = uniform_cptr(vh + (int64_t)j * TB);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t ok = gk + 4096u * i, ov = gv + 4096u * i;
            settle_v(ok);
            settle_v(ov);
            __builtin_amdgcn_global_load_lds((gbl_void_t*)(ks + ok), (lds_void_t*)(dk_ + 1024 * (wave + 4 * i)), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((gbl_void_t*)(vs + ov), (lds_void_t*)(dv_ + 1024 * (wave + 4 * i)), 16, 0, 0);
        }
    };
    // Union cursor (workgroup-uniform).
    int ia = 0, ib = 0;
    auto adv = [&](int& j, int& flags) {
        const int ja0 = ia < cntA ? __builtin_amdgcn_readfirstlane(listA[ia]) : n;
        const int jb0 = ib < cntB ? __builtin_amdgcn_readfirstlane(listB[ib]) : n;
        const int ja = (unsigned)ja0 <= (unsigned)n ? ja0 : 0;
        const int jb = (unsigned)jb0 <= (unsigned)n ? jb0 : 0;
        j = ja < jb ? ja : jb;
        flags = j >= n ? 0 : ((ja == j ? 1 : 0) | (jb == j ? 2 : 0));
        ia += flags & 1;
        ib += (flags >> 1) & 1;
    };
    int j_cur, f_cur, j_nxt, f_nxt;
    adv(j_cur, f_cur);
    if (f_cur) {
        dma(j_cur, sK0, sV0);
        adv(j_nxt, f_nxt);
        dma_wait_all();
        dma_barrier();
        // One step: load the next step's tiles into the other buffer, compute
        // this step from its buffer, advance, wait, meet.
        auto one = [&](const char* ck, const char* cv, char* nk, char* nv) {
            // Next step's tiles; with no next step, any valid block (never read).
            dma(f_nxt ? j_nxt : (f_cur ? j_cur : 0), nk, nv);
            const int mine = grp ? (f_cur & 2) : (f_cur & 1);
            if (mine && active) block_step_swz(st, ck, cv, kl, vl, scale_log2, wsel);
            j_cur = j_nxt;
            f_cur = f_nxt;
            if (f_cur) adv(j_nxt, f_nxt);
            else f_nxt = 0;
            dma_wait_all();
            dma_barrier();
        };
        for (;;) {
            one(sK0, sV0, sK1, sV1);
            one(sK1, sV1, sK0, sV0);
            if (f_cur == 0) break;
        }
    }
    if (active) store_rows<D>(st, head, qrow, h, o, o_fp32, lse, bh * (int64_t)S + qrow);
}

namespace {

constexpr int kPairThreads = 256;

// Work of pair p of head bh (frames 2s, 2s+1 of tile position p % F): the mean
// of the two kept counts, in [0, n], as the longest-first key.
__global__ __launch_bounds__(kPairThreads) void pair_counts_kernel(const int32_t* __restrict__ kv_count,
                                                                   int n, int F, int np,
                                                                   int64_t total,
                                                                   int32_t* __restrict__ pc) {
    const int64_t g = (int64_t)blockIdx.x * kPairThreads + threadIdx.x;
    if (g >= total) return;
    const int64_t bh = g / np;
    const int p = (int)(g % np);
    const int qa = 2 * (p / F) * F + p % F;
    int a = kv_count[bh * n + qa];
    a = a < 0 ? 0 : (a > n ? n : a);
    int b = 0;
    if (qa + F < n) {
        b = kv_count[bh * n + qa + F];
        b = b < 0 ? 0 : (b > n ? n : b);
    }
    pc[g] = (a + b + 1) / 2;
}

}  // namespace

int pair_count(int n, int F) { return F * ((n / F + 1) / 2); }

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, int64_t BH, int S, int D,
                           const int32_t* kv_count, const int32_t* kv_idx, const int32_t* order,
                           const XcdSchedule& sched, float softmax_scale, void* o, bool o_fp32,
                           float* lse, hipStream_t stream) {
    const int n = S / kBlockN;
    const unsigned grid = (unsigned)sched.grid;
    const float sl2 = softmax_scale * kLog2e;
    if (D == 128)
        attn_fwd_kernel<128><<<grid, 128, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, S, n, kv_count, kv_idx,
            order, sched, sl2, o, o_fp32 ? 1 : 0, lse);
    else
        attn_fwd_kernel<64><<<grid, 128, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, S, n, kv_count, kv_idx,
            order, sched, sl2, o, o_fp32 ? 1 : 0, lse);
    return hipGetLastError();
}

hipError_t launch_pair_counts(const int32_t* kv_count, int64_t BH, int n, int F, int32_t* pc,
                              hipStream_t stream) {
    const int np = pair_count(n, F);
    const int64_t total = BH * np;
    const unsigned grid = (unsigned)((total + kPairThreads - 1) / kPairThreads);
    pair_counts_kernel<<<grid, kPairThreads, 0, stream>>>(kv_count, n, F, np, total, pc);
    return hipGetLastError();
}

hipError_t launch_attn_fwd_pairs(const void* q, const void* k, const void* v, int64_t BH, int S,
                                 int D, int F, const int32_t* kv_count, const int32_t* kv_idx,
                                 const int32_t* order, const XcdSchedule& sched,
                                 float softmax_scale, void* o, bool o_fp32, float* lse,
                                 hipStream_t stream) {
    const int n = S / kBlockN;
    const unsigned grid = (unsigned)sched.grid;
    const float sl2 = softmax_scale * kLog2e;
    if (D == 128)
        attn_fwd_pair_kernel<128><<<grid, 256, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, S, n, F, kv_count, kv_idx,
            order, sched, sl2, o, o_fp32 ? 1 : 0, lse);
    else
        attn_fwd_pair_kernel<64><<<grid, 256, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, S, n, F, kv_count, kv_idx,
            order, sched, sl2, o, o_fp32 ? 1 : 0, lse);
    return hipGetLastError();
}

}  // namespace nabla

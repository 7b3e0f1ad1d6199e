// attn_bwd.hip -- block-sparse flash-attention backward on gfx950.
//
// Gradients of eq. (4) of "NABLA: Neighborhood Adaptive Block-Level Attention"
// (section 2.2) with the block mask held constant (it is a piecewise-constant
// function of Q and K). The paper trains through this attention in both its
// fine-tuning (section 4.1) and pretraining (section 4.3) experiments.
//
//   delta_kernel  Delta_s = sum_d dO[s,d] * O[s,d]
//   dkdv_kernel   one workgroup per key block j, walking the query blocks that
//                 keep j:  dV_j += P^T dO_i,  dK_j += scale * dS^T Q_i
//   dq_kernel     one workgroup per query block i, walking its kept key blocks:
//                 dQ_i += scale * dS K_j
// with P = exp(scale * Q K^T - LSE) and dS = P * (dO V^T - Delta). Each output
// block is owned by one workgroup, so there are no atomics and results are
// deterministic.
//
// Operand layouts follow attn_fwd.hip. Tiles are staged row-major in padded
// LDS rows (prefetched two blocks ahead through registers). A 32 x 32
// accumulator's rows become the contraction slots of the next product's B
// operand, and the matching A operand -- a transposed tile (K^T, dO^T, Q^T) --
// is read with the transposing LDS read, which hands each lane one column of
// four consecutive tile rows in exactly that slot order.

#include "common.h"
#include "kernels.h"

namespace nabla {

namespace {

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

template <int D>
struct BTile {
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row
    // Row stride (bytes): the tiles are read both row-wise (16 rows x 16 B)
    // and transposed (4 rows x 64 B); a 32-byte pad keeps both at most 2-way.
    static constexpr int RSTB = 2 * D + 32;
    static constexpr int LOADS = kBlockN * CPR / 128;  // 16-byte chunks per thread per tile
};

// Transposed A operand: rows rbase + 4h + jj (jj = 0..3, and +8 for the upper
// four slots) of a row-major tile, column 32 t + lane % 32. `tbase` is this
// lane's address of row 4h + (lane % 16) / 4, columns 16 ((lane/16) % 2) +
// 4 (lane % 4) .. +3 (see attn_fwd.hip for the read's lane layout).
template <int RSTB>
__device__ __forceinline__ bf16x8_t tr_operand(const char* tbase, int rbase, int t) {
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t*)(tbase + rbase * RSTB + 64 * t));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t*)(tbase + (rbase + 8) * RSTB + 64 * t));
    const uint2 ulo = __builtin_bit_cast(uint2, lo);
    const uint2 uhi = __builtin_bit_cast(uint2, hi);
    return as_bf16x8(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
}

__device__ __forceinline__ const char* tr_lane_base(const char* tile, int lane, int rstb) {
    const int h = lane >> 5;
    return tile + (4 * h + ((lane & 15) >> 2)) * rstb + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
}

// Store a transposed accumulator set (rows d, column = this lane's token) as
// bf16 row `row_ptr[d]`, scaled by `mul`.
template <int DT>
__device__ __forceinline__ void store_t_acc(uint16_t* row_ptr, const f32x16_t* acc, float mul,
                                            int h) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint2 w;
            w.x = pack_bf16x2(acc[t][4 * g + 0] * mul, acc[t][4 * g + 1] * mul);
            w.y = pack_bf16x2(acc[t][4 * g + 2] * mul, acc[t][4 * g + 3] * mul);
            *reinterpret_cast<uint2*>(row_ptr + 32 * t + 8 * g + 4 * h) = w;
        }
}

}  // namespace

// ---------------------------------------------------------------------------
// Delta_s = dO_s . O_s (fp32). D/8 lanes per row, 8 elements each; O is bf16
// or fp32 (an fp32 forward output keeps Delta free of O's bf16 rounding).
// ---------------------------------------------------------------------------
template <int D, bool O_FP32>
__global__ __launch_bounds__(256) void delta_kernel(const void* __restrict__ o,
                                                    const uint16_t* __restrict__ d_o, int64_t rows,
                                                    float* __restrict__ delta) {
    constexpr int LPR = D / 8;  // lanes per row
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / LPR;
    const int part = (int)(gid % LPR);
    float s = 0.f;
    if (row < rows) {
        float ov[8];
        if constexpr (O_FP32) {
            const float* op = static_cast<const float*>(o) + row * D + part * 8;
            const float4 a0 = *reinterpret_cast<const float4*>(op);
            const float4 a1 = *reinterpret_cast<const float4*>(op + 4);
            ov[0] = a0.x; ov[1] = a0.y; ov[2] = a0.z; ov[3] = a0.w;
            ov[4] = a1.x; ov[5] = a1.y; ov[6] = a1.z; ov[7] = a1.w;
        } else {
            const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(o) + row * D + part * 8);
            const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ov[2 * e] = bf16_bits_to_f32(wa[e] & 0xffffu);
                ov[2 * e + 1] = bf16_bits_to_f32(wa[e] >> 16);
            }
        }
        const uint4 b = *reinterpret_cast<const uint4*>(d_o + row * D + part * 8);
        const uint32_t wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s += ov[2 * e] * bf16_bits_to_f32(wb[e] & 0xffffu);
            s += ov[2 * e + 1] * bf16_bits_to_f32(wb[e] >> 16);
        }
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (row < rows && part == 0) delta[row] = s;
}

// Register staging of two 64 x D tiles (A, B) of block `blk` of one head and
// their write to padded LDS rows. Thread chunk e = tid + 128 i covers row
// e / CPR, chunk e % CPR.
#define NABLA_BWD_FETCH(A_SRC, B_SRC, BLK)                                            \
    do {                                                                              \
        const int64_t off_ = (int64_t)(BLK) * kBlockN * D;                            \
        _Pragma("unroll") for (int i_ = 0; i_ < L; ++i_) {                            \
            const int e_ = tid + 128 * i_;                                            \
            ra[i_] = *reinterpret_cast<const u32x4_t*>((A_SRC) + off_ + e_ * 8);      \
            rb[i_] = *reinterpret_cast<const u32x4_t*>((B_SRC) + off_ + e_ * 8);      \
        }                                                                             \
    } while (0)
#define NABLA_BWD_STAGE(A_DST, B_DST)                                                 \
    do {                                                                              \
        _Pragma("unroll") for (int i_ = 0; i_ < L; ++i_) {                            \
            const int e_ = tid + 128 * i_;                                            \
            const int r_ = e_ / T::CPR, ch_ = e_ % T::CPR;                            \
            *reinterpret_cast<u32x4_t*>((A_DST) + r_ * T::RSTB + 16 * ch_) = ra[i_];  \
            *reinterpret_cast<u32x4_t*>((B_DST) + r_ * T::RSTB + 16 * ch_) = rb[i_];  \
        }                                                                             \
    } while (0)

// ---------------------------------------------------------------------------
// dK, dV for one 64-key block; wave w owns keys 32w .. 32w+31.
// Per query block i: S = Q_i K^T and dP = dO_i V^T (A = Q_i / dO_i rows from
// LDS, B = K^T / V^T in registers; accumulator rows = queries), then
// dV^T += dO_i^T P and dK^T += Q_i^T dS (A = transposed reads of the dO_i / Q_i
// tiles, B = P / dS from the accumulators).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta, int S, int n,
    const int32_t* __restrict__ q_count, const int32_t* __restrict__ q_idx,
    const int32_t* __restrict__ order, XcdSchedule sched, float scale, float scale_log2,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
    using T = BTile<D>;
    constexpr int KK = D / 16, DT = D / 32, L = T::LOADS;
    __shared__ __attribute__((aligned(16))) char sQ[kBlockN * T::RSTB];
    __shared__ __attribute__((aligned(16))) char sO[kBlockN * T::RSTB];
    __shared__ __attribute__((aligned(16))) float sL[kBlockN];
    __shared__ __attribute__((aligned(16))) float sDel[kBlockN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, c = lane & 31;
    const int64_t item = scheduled_item(sched, order, blockIdx.x);
    if (item < 0) return;  // padding slot (whole workgroup)
    const int64_t bh = item / n;
    const int kb = (int)(item % n);
    int cnt = q_count[item];
    cnt = cnt < 0 ? 0 : (cnt > n ? n : cnt);
    const int32_t* list = q_idx + item * (int64_t)n;
    const int64_t head = bh * (int64_t)S * D;
    const uint16_t* qh = q + head;
    const uint16_t* oh = d_o + head;
    const float* lh = lse + bh * (int64_t)S;
    const float* dh = delta + bh * (int64_t)S;

    // K^T and V^T as B operands: lane holds key krow, d = 16 kk + 8 h + 0..7.
    const int krow = kb * kBlockN + wave * 32 + c;
    bf16x8_t kf[KK], vf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        kf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(k + head + (int64_t)krow * D + 16 * kk + 8 * h));
        vf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(v + head + (int64_t)krow * D + 16 * kk + 8 * h));
    }
    f32x16_t dVt[DT], dKt[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) {
        dVt[t] = zero16();
        dKt[t] = zero16();
    }

    const char* qrow_base = sQ + c * T::RSTB + 16 * h;  // row 32 qt + c, bytes 32 kk + 16 h
    const char* orow_base = sO + c * T::RSTB + 16 * h;
    const char* qtr = tr_lane_base(sQ, lane, T::RSTB);
    const char* otr = tr_lane_base(sO, lane, T::RSTB);

    u32x4_t ra[L], rb[L];
    float rl = 0.f, rd = 0.f;  // LSE / Delta of one query row (threads < 64)
    if (cnt > 0) {
        int i0 = list[0];
        i0 = (unsigned)i0 < (unsigned)n ? i0 : 0;
        NABLA_BWD_FETCH(qh, oh, i0);
        if (tid < kBlockN) {
            rl = lh[(int64_t)i0 * kBlockN + tid];
            rd = dh[(int64_t)i0 * kBlockN + tid];
        }
        NABLA_BWD_STAGE(sQ, sO);
        if (tid < kBlockN) {
            sL[tid] = rl * kLog2e;
            sDel[tid] = rd;
        }
        if (cnt > 1) {
            int i1 = list[1];
            i1 = (unsigned)i1 < (unsigned)n ? i1 : 0;
            NABLA_BWD_FETCH(qh, oh, i1);
            if (tid < kBlockN) {
                rl = lh[(int64_t)i1 * kBlockN + tid];
                rd = dh[(int64_t)i1 * kBlockN + tid];
            }
        }
        __syncthreads();
    }
    for (int it = 0; it < cnt; ++it) {
        uint32_t pw[2][8], dsw[2][8];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            // S and dP tiles: rows = queries 32 qt + c_row(r, h), column = key c of this wave.
            f32x16_t sc = zero16(), dp = zero16();
            {
                bf16x8_t a[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow_base + 32 * qt * T::RSTB + 32 * kk));
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) sc = mfma_32x32x16(a[kk], kf[kk], sc);
            }
            {
                bf16x8_t a[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(orow_base + 32 * qt * T::RSTB + 32 * kk));
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) dp = mfma_32x32x16(a[kk], vf[kk], dp);
            }
            // Rows c_row(4g + e, h) = 32 qt + 8 g + 4 h + e: four consecutive rows per g.
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 l4 = *reinterpret_cast<const float4*>(sL + 32 * qt + 8 * g + 4 * h);
                const float4 d4 = *reinterpret_cast<const float4*>(sDel + 32 * qt + 8 * g + 4 * h);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    const float p = __builtin_amdgcn_exp2f(sc[r] * scale_log2 - lv[e]);
                    sc[r] = p;
                    dp[r] = p * (dp[r] - dv4[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pw[qt][e] = pack_bf16x2(sc[2 * e], sc[2 * e + 1]);
                dsw[qt][e] = pack_bf16x2(dp[2 * e], dp[2 * e + 1]);
            }
        }
        // dV^T += dO^T P, dK^T += Q^T dS: slot s of B is query
        // 32 qt + 16 u + 8 (s/4) + 4 h + s%4, matched by the transposed reads.
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16x8_t bp = as_bf16x8(make_uint4(pw[qt][4 * u], pw[qt][4 * u + 1],
                                                         pw[qt][4 * u + 2], pw[qt][4 * u + 3]));
                const bf16x8_t bs = as_bf16x8(make_uint4(dsw[qt][4 * u], dsw[qt][4 * u + 1],
                                                         dsw[qt][4 * u + 2], dsw[qt][4 * u + 3]));
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    dVt[t] = mfma_32x32x16(tr_operand<T::RSTB>(otr, 32 * qt + 16 * u, t), bp, dVt[t]);
                    dKt[t] = mfma_32x32x16(tr_operand<T::RSTB>(qtr, 32 * qt + 16 * u, t), bs, dKt[t]);
                }
            }
        if (it + 1 < cnt) {
            __syncthreads();  // every wave is done with this query block's tiles
            NABLA_BWD_STAGE(sQ, sO);
            if (tid < kBlockN) {
                sL[tid] = rl * kLog2e;
                sDel[tid] = rd;
            }
            if (it + 2 < cnt) {
                int i2 = list[it + 2];
                i2 = (unsigned)i2 < (unsigned)n ? i2 : 0;
                NABLA_BWD_FETCH(qh, oh, i2);
                if (tid < kBlockN) {
                    rl = lh[(int64_t)i2 * kBlockN + tid];
                    rd = dh[(int64_t)i2 * kBlockN + tid];
                }
            }
            __syncthreads();
        }
    }
    store_t_acc<DT>(dk + head + (int64_t)krow * D, dKt, scale, h);
    store_t_acc<DT>(dv + head + (int64_t)krow * D, dVt, 1.0f, h);
}

// ---------------------------------------------------------------------------
// dQ for one 64-query block; wave w owns queries 32w .. 32w+31.
// Per key block j: S^T = K_j Q^T and dP^T = V_j dO^T (A = K_j / V_j rows from
// LDS, B = Q^T / dO^T in registers; accumulator rows = keys), then
// dQ^T += K_j^T dS^T (A = transposed reads of the K_j tile, B = dS^T).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta, int S, int n,
    const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_idx,
    const int32_t* __restrict__ order, XcdSchedule sched, float scale, float scale_log2,
    uint16_t* __restrict__ dq) {
    using T = BTile<D>;
    constexpr int KK = D / 16, DT = D / 32, L = T::LOADS;
    __shared__ __attribute__((aligned(16))) char sK[kBlockN * T::RSTB];
    __shared__ __attribute__((aligned(16))) char sV[kBlockN * T::RSTB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

    const int qrow = qb * kBlockN + wave * 32 + c;
    bf16x8_t qf[KK], dof[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        qf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(q + head + (int64_t)qrow * D + 16 * kk + 8 * h));
        dof[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(d_o + head + (int64_t)qrow * D + 16 * kk + 8 * h));
    }
    const float l2 = lse[bh * (int64_t)S + qrow] * kLog2e;
    const float del = delta[bh * (int64_t)S + qrow];
    f32x16_t dQt[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) dQt[t] = zero16();

    const char* krow_base = sK + c * T::RSTB + 16 * h;  // row 32 kt + c, bytes 32 kk + 16 h
    const char* vrow_base = sV + c * T::RSTB + 16 * h;
    const char* ktr = tr_lane_base(sK, lane, T::RSTB);

    u32x4_t ra[L], rb[L];
    if (cnt > 0) {
        int j0 = list[0];
        j0 = (unsigned)j0 < (unsigned)n ? j0 : 0;
        NABLA_BWD_FETCH(kh, vh, j0);
        NABLA_BWD_STAGE(sK, sV);
        if (cnt > 1) {
            int j1 = list[1];
            j1 = (unsigned)j1 < (unsigned)n ? j1 : 0;
            NABLA_BWD_FETCH(kh, vh, j1);
        }
        __syncthreads();
    }
    for (int it = 0; it < cnt; ++it) {
        uint32_t dsw[2][8];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            // S^T and dP^T tiles: rows = keys 32 kt + c_row(r, h), column = query c.
            f32x16_t sc = zero16(), dp = zero16();
            {
                bf16x8_t a[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(krow_base + 32 * kt * T::RSTB + 32 * kk));
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) sc = mfma_32x32x16(a[kk], qf[kk], sc);
            }
            {
                bf16x8_t a[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(vrow_base + 32 * kt * T::RSTB + 32 * kk));
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) dp = mfma_32x32x16(a[kk], dof[kk], dp);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(sc[r] * scale_log2 - l2);
                dp[r] = p * (dp[r] - del);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) dsw[kt][e] = pack_bf16x2(dp[2 * e], dp[2 * e + 1]);
        }
        // dQ^T += K^T dS^T: slot s of B is key 32 kt + 16 u + 8 (s/4) + 4 h + s%4.
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16x8_t bs = as_bf16x8(make_uint4(dsw[kt][4 * u], dsw[kt][4 * u + 1],
                                                         dsw[kt][4 * u + 2], dsw[kt][4 * u + 3]));
#pragma unroll
                for (int t = 0; t < DT; ++t)
                    dQt[t] = mfma_32x32x16(tr_operand<T::RSTB>(ktr, 32 * kt + 16 * u, t), bs, dQt[t]);
            }
        if (it + 1 < cnt) {
            __syncthreads();  // every wave is done with this key block's tiles
            NABLA_BWD_STAGE(sK, sV);
            if (it + 2 < cnt) {
                int j2 = list[it + 2];
                j2 = (unsigned)j2 < (unsigned)n ? j2 : 0;
                NABLA_BWD_FETCH(kh, vh, j2);
            }
            __syncthreads();
        }
    }
    store_t_acc<DT>(dq + head + (int64_t)qrow * D, dQt, scale, h);
}

#undef NABLA_BWD_FETCH
#undef NABLA_BWD_STAGE

hipError_t launch_bwd_delta(const void* o, bool o_fp32, const void* d_o, int64_t rows, int D,
                            float* delta, hipStream_t stream) {
    const int64_t threads = rows * (D / 8);
    const unsigned grid = (unsigned)((threads + 255) / 256);
    const uint16_t* dop = (const uint16_t*)d_o;
    if (D == 128) {
        if (o_fp32) delta_kernel<128, true><<<grid, 256, 0, stream>>>(o, dop, rows, delta);
        else delta_kernel<128, false><<<grid, 256, 0, stream>>>(o, dop, rows, delta);
    } else {
        if (o_fp32) delta_kernel<64, true><<<grid, 256, 0, stream>>>(o, dop, rows, delta);
        else delta_kernel<64, false><<<grid, 256, 0, stream>>>(o, dop, rows, delta);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* d_o,
                           const float* lse, const float* delta, int64_t BH, int S, int D,
                           const int32_t* q_count, const int32_t* q_idx, const int32_t* order,
                           const XcdSchedule& sched, float softmax_scale, void* dk, void* dv,
                           hipStream_t stream) {
    const int n = S / kBlockN;
    const unsigned grid = (unsigned)sched.grid;
    const float sl2 = softmax_scale * kLog2e;
    if (D == 128)
        dkdv_kernel<128><<<grid, 128, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)d_o, lse,
            delta, S, n, q_count, q_idx, order, sched, softmax_scale, sl2, (uint16_t*)dk,
            (uint16_t*)dv);
    else
        dkdv_kernel<64><<<grid, 128, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)d_o, lse,
            delta, S, n, q_count, q_idx, order, sched, softmax_scale, sl2, (uint16_t*)dk,
            (uint16_t*)dv);
    return hipGetLastError();
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* d_o,
                         const float* lse, const float* delta, int64_t BH, int S, int D,
                         const int32_t* kv_count, const int32_t* kv_idx, const int32_t* order,
                         const XcdSchedule& sched, float softmax_scale, void* dq,
                         hipStream_t stream) {
    const int n = S / kBlockN;
    const unsigned grid = (unsigned)sched.grid;
    const float sl2 = softmax_scale * kLog2e;
    if (D == 128)
        dq_kernel<128><<<grid, 128, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)d_o, lse,
            delta, S, n, kv_count, kv_idx, order, sched, softmax_scale, sl2, (uint16_t*)dq);
    else
        dq_kernel<64><<<grid, 128, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)d_o, lse,
            delta, S, n, kv_count, kv_idx, order, sched, softmax_scale, sl2, (uint16_t*)dq);
    return hipGetLastError();
}

}  // namespace nabla

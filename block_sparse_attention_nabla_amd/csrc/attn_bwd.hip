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
// Operand layouts follow attn_fwd.hip. Both kernels split each (query block,
// key block) pair into four 32 x 32 quadrants, one per wave, so two
// workgroups -- two waves per SIMD -- share a CU. Tiles sit row-major in LDS:
// for D = 128 moved by direct-to-LDS loads into swizzled unpadded rows (two
// buffers), otherwise staged through registers into padded rows. A 32 x 32
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
    template <int NT>
    static constexpr int loads() { return kBlockN * CPR / NT; }  // 16-byte chunks per thread per tile
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

// Mark a value loaded before the main loop as produced here. The compiler's
// wait-count tracking otherwise carries such loads as possibly outstanding
// into the loop and waits for them at their first use in every iteration --
// a wait that, in issue order, also covers the tile prefetch of the previous
// iteration. With this the wait is taken once, here.
template <typename T>
__device__ __forceinline__ void settle(T& x) {
    asm volatile("" : "+v"(x));
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
// their write to padded LDS rows. Thread chunk e = tid + NT i covers row
// e / CPR, chunk e % CPR (NT = threads per workgroup).
#define NABLA_BWD_FETCH(A_SRC, B_SRC, BLK)                                            \
    do {                                                                              \
        const int64_t off_ = (int64_t)(BLK) * kBlockN * D;                            \
        _Pragma("unroll") for (int i_ = 0; i_ < L; ++i_) {                            \
            const int e_ = tid + NT * i_;                                            \
            ra[i_] = *reinterpret_cast<const u32x4_t*>((A_SRC) + off_ + e_ * 8);      \
            rb[i_] = *reinterpret_cast<const u32x4_t*>((B_SRC) + off_ + e_ * 8);      \
        }                                                                             \
    } while (0)
#define NABLA_BWD_STAGE(A_DST, B_DST)                                                 \
    do {                                                                              \
        _Pragma("unroll") for (int i_ = 0; i_ < L; ++i_) {                            \
            const int e_ = tid + NT * i_;                                            \
            const int r_ = e_ / T::CPR, ch_ = e_ % T::CPR;                            \
            *reinterpret_cast<u32x4_t*>((A_DST) + r_ * T::RSTB + 16 * ch_) = ra[i_];  \
            *reinterpret_cast<u32x4_t*>((B_DST) + r_ * T::RSTB + 16 * ch_) = rb[i_];  \
        }                                                                             \
    } while (0)

// ---------------------------------------------------------------------------
// dK, dV for one 64-key block on four waves. Wave w takes key half
// kh = w % 2 (keys 32 kh .. +31) and query half qh = w / 2. Per query block i
// of the key block's list:
//   1. S = Q_i K^T and dP = dO_i V^T for the quadrant (queries 32 qh .. +31) x
//      (its keys): A = Q_i / dO_i rows from LDS, B = K^T / V^T in registers,
//      accumulator rows = queries; P and dS = P * (dP - Delta) packed to bf16.
//   2. The packed quadrant goes to LDS; the wave with the same keys and the
//      other query half reads it back in the same lane layout (its lanes hold
//      the same key columns), so both then hold P and dS for all 64 queries.
//   3. dV^T += dO_i^T P and dK^T += Q_i^T dS for half of the head dimension,
//      d in [D/2 qh, D/2 (qh + 1)) (A = transposed reads of the dO_i / Q_i
//      tiles, B = P / dS).
// A wave thus holds half of the dK/dV accumulators of its keys (about 250
// registers), so two workgroups -- two waves per SIMD -- share a CU and one
// wave's products overlap the other's softmax. Every output element gets the
// same products in the same order as in a wave owning all of D: the split
// changes no result.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta, int S, int n,
    const int32_t* __restrict__ q_count, const int32_t* __restrict__ q_idx,
    const int32_t* __restrict__ order, XcdSchedule sched, float scale, float scale_log2,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
    using T = BTile<D>;
    constexpr int NT = 256;
    constexpr int KK = D / 16, DT = D / 32, DH = DT / 2, L = T::template loads<NT>();
    __shared__ __attribute__((aligned(16))) char sQ[kBlockN * T::RSTB];
    __shared__ __attribute__((aligned(16))) char sO[kBlockN * T::RSTB];
    __shared__ __attribute__((aligned(16))) float sL[kBlockN];
    __shared__ __attribute__((aligned(16))) float sDel[kBlockN];  // -Delta of the staged rows
    // Packed P (groups 0, 1) and dS (groups 2, 3) of each wave's quadrant,
    // [wave][group][lane]: lane-contiguous 16-byte words.
    __shared__ __attribute__((aligned(16))) u32x4_t sX[4][4][kWave];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, c = lane & 31;
    const int kh = wave & 1, qh = wave >> 1;
    const int64_t item = scheduled_item(sched, order, blockIdx.x);
    if (item < 0) return;  // padding slot (whole workgroup)
    const int64_t bh = item / n;
    const int kb = (int)(item % n);
    int cnt = q_count[item];
    cnt = cnt < 0 ? 0 : (cnt > n ? n : cnt);
    const int32_t* list = q_idx + item * (int64_t)n;
    const int64_t head = bh * (int64_t)S * D;
    const uint16_t* qh_ptr = q + head;
    const uint16_t* oh_ptr = d_o + head;
    const float* lh = lse + bh * (int64_t)S;
    const float* dh = delta + bh * (int64_t)S;

    // K^T and V^T as B operands: lane holds key krow, d = 16 kk + 8 h + 0..7.
    const int krow = kb * kBlockN + kh * 32 + c;
    bf16x8_t kf[KK], vf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        kf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(k + head + (int64_t)krow * D + 16 * kk + 8 * h));
        vf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(v + head + (int64_t)krow * D + 16 * kk + 8 * h));
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        settle(kf[kk]);
        settle(vf[kk]);
    }
    f32x16_t dVt[DH], dKt[DH];
#pragma unroll
    for (int t = 0; t < DH; ++t) {
        dVt[t] = zero16();
        dKt[t] = zero16();
    }

    // Rows 32 qh + c of the Q / dO tiles, bytes 32 kk + 16 h.
    const char* qrow_base = sQ + (32 * qh + c) * T::RSTB + 16 * h;
    const char* orow_base = sO + (32 * qh + c) * T::RSTB + 16 * h;
    // Transposed reads of this wave's half of the head dimension.
    const char* qtr = tr_lane_base(sQ, lane, T::RSTB) + 64 * DH * qh;
    const char* otr = tr_lane_base(sO, lane, T::RSTB) + 64 * DH * qh;
    const float* lrow = sL + 32 * qh + 4 * h;
    const float* drow = sDel + 32 * qh + 4 * h;

    u32x4_t ra[L], rb[L];
    float rl = 0.f, rd = 0.f;  // LSE / Delta of one query row (threads < 64)
    if (cnt > 0) {
        int i0 = list[0];
        i0 = (unsigned)i0 < (unsigned)n ? i0 : 0;
        NABLA_BWD_FETCH(qh_ptr, oh_ptr, i0);
        if (tid < kBlockN) {
            rl = lh[(int64_t)i0 * kBlockN + tid];
            rd = dh[(int64_t)i0 * kBlockN + tid];
        }
        NABLA_BWD_STAGE(sQ, sO);
        if (tid < kBlockN) {
            sL[tid] = rl * kLog2e;
            sDel[tid] = -rd;
        }
        if (cnt > 1) {
            int i1 = list[1];
            i1 = (unsigned)i1 < (unsigned)n ? i1 : 0;
            NABLA_BWD_FETCH(qh_ptr, oh_ptr, i1);
            if (tid < kBlockN) {
                rl = lh[(int64_t)i1 * kBlockN + tid];
                rd = dh[(int64_t)i1 * kBlockN + tid];
            }
        }
        __syncthreads();
    }
    // dV^T += dO^T P, dK^T += Q^T dS over the query halves in order (p0/s0:
    // queries 0..31, p1/s1: 32..63); slot s of B is query
    // 32 qt + 16 u + 8 (s/4) + 4 h + s%4, matched by the transposed reads.
    auto accumulate = [&](const uint32_t (&p0)[8], const uint32_t (&s0)[8], const uint32_t (&p1)[8],
                          const uint32_t (&s1)[8]) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t* pp = qt == 0 ? p0 : p1;
                const uint32_t* ss = qt == 0 ? s0 : s1;
                const bf16x8_t bp = as_bf16x8(make_uint4(pp[4 * u], pp[4 * u + 1], pp[4 * u + 2], pp[4 * u + 3]));
                const bf16x8_t bs = as_bf16x8(make_uint4(ss[4 * u], ss[4 * u + 1], ss[4 * u + 2], ss[4 * u + 3]));
#pragma unroll
                for (int t = 0; t < DH; ++t) {
                    dVt[t] = mfma_32x32x16(tr_operand<T::RSTB>(otr, 32 * qt + 16 * u, t), bp, dVt[t]);
                    dKt[t] = mfma_32x32x16(tr_operand<T::RSTB>(qtr, 32 * qt + 16 * u, t), bs, dKt[t]);
                }
            }
    };
    for (int it = 0; it < cnt; ++it) {
        uint32_t pw[8], dsw[8];
        {
            // S and dP quadrant: rows = queries 32 qh + c_row(r, h), column = key c.
            f32x16_t sc = zero16(), dp;
            // dP starts from -Delta of its rows, so the products yield dP - Delta.
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 d4 = *reinterpret_cast<const float4*>(drow + 8 * g);
                dp[4 * g + 0] = d4.x;
                dp[4 * g + 1] = d4.y;
                dp[4 * g + 2] = d4.z;
                dp[4 * g + 3] = d4.w;
            }
            {
                bf16x8_t a[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow_base + 32 * kk));
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) sc = mfma_32x32x16(a[kk], kf[kk], sc);
            }
            {
                bf16x8_t a[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(orow_base + 32 * kk));
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) dp = mfma_32x32x16(a[kk], vf[kk], dp);
            }
            // Rows c_row(4g + e, h) = 32 qh + 8 g + 4 h + e: four consecutive rows per g.
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 l4 = *reinterpret_cast<const float4*>(lrow + 8 * g);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    const float p = __builtin_amdgcn_exp2f(sc[r] * scale_log2 - lv[e]);
                    sc[r] = p;
                    dp[r] = p * dp[r];
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pw[e] = pack_bf16x2(sc[2 * e], sc[2 * e + 1]);
                dsw[e] = pack_bf16x2(dp[2 * e], dp[2 * e + 1]);
            }
        }
        // Hand the quadrant to the wave with the same keys and the other query half.
        sX[wave][0][lane] = u32x4_t{pw[0], pw[1], pw[2], pw[3]};
        sX[wave][1][lane] = u32x4_t{pw[4], pw[5], pw[6], pw[7]};
        sX[wave][2][lane] = u32x4_t{dsw[0], dsw[1], dsw[2], dsw[3]};
        sX[wave][3][lane] = u32x4_t{dsw[4], dsw[5], dsw[6], dsw[7]};
        __syncthreads();
        uint32_t po[8], so[8];
        {
            const u32x4_t x0 = sX[wave ^ 2][0][lane], x1 = sX[wave ^ 2][1][lane];
            const u32x4_t x2 = sX[wave ^ 2][2][lane], x3 = sX[wave ^ 2][3][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                po[e] = x0[e];
                po[4 + e] = x1[e];
                so[e] = x2[e];
                so[4 + e] = x3[e];
            }
        }
        if (qh == 0) accumulate(pw, dsw, po, so);
        else accumulate(po, so, pw, dsw);
        if (it + 1 < cnt) {
            __syncthreads();  // every wave is done with this query block's tiles
            NABLA_BWD_STAGE(sQ, sO);
            if (tid < kBlockN) {
                sL[tid] = rl * kLog2e;
                sDel[tid] = -rd;
            }
            if (it + 2 < cnt) {
                int i2 = list[it + 2];
                i2 = (unsigned)i2 < (unsigned)n ? i2 : 0;
                NABLA_BWD_FETCH(qh_ptr, oh_ptr, i2);
                if (tid < kBlockN) {
                    rl = lh[(int64_t)i2 * kBlockN + tid];
                    rd = dh[(int64_t)i2 * kBlockN + tid];
                }
            }
            __syncthreads();
        }
    }
    store_t_acc<DH>(dk + head + (int64_t)krow * D + 32 * DH * qh, dKt, scale, h);
    store_t_acc<DH>(dv + head + (int64_t)krow * D + 32 * DH * qh, dVt, 1.0f, h);
}

// ---------------------------------------------------------------------------
// dQ for one 64-query block. Four waves split each (query block, key block)
// pair into 32 x 32 quadrants: wave w takes queries 32 (w / 2) .. +31 and keys
// 32 (w % 2) .. +31 of every key block. Per key block j:
// S^T = K_j Q^T and dP^T = V_j dO^T for its quadrant (A = K_j / V_j rows from
// LDS, B = Q^T / dO^T in registers; accumulator rows = keys), then
// dQ^T += K_j^T dS^T over its 32 keys (A = transposed reads of the K_j tile).
// The two waves of a query half sum their partial dQ once, through LDS, at
// the end (D = 128 moves its tiles by direct-to-LDS loads: see its
// specialization below). Small per-wave state (about 220 registers) lets two workgroups --
// two waves per SIMD -- share a CU, so one wave's products overlap the other's
// softmax and LDS reads.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta, int S, int n,
    const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_idx,
    const int32_t* __restrict__ order, XcdSchedule sched, float scale, float scale_log2,
    uint16_t* __restrict__ dq) {
    using T = BTile<D>;
    constexpr int NT = 256;
    constexpr int KK = D / 16, DT = D / 32, L = T::template loads<NT>();
    // K and V tiles; after the loop, the partial dQ of the key-half-1 waves.
    constexpr int kTileBytes = kBlockN * T::RSTB;
    constexpr int kRedBytes = 2 * DT * 16 * kWave * 4;
    static_assert(kRedBytes <= 2 * kTileBytes, "reduction buffer exceeds the tile buffers");
    __shared__ __attribute__((aligned(16))) char sKV[2 * kTileBytes];
    char* const sK = sKV;
    char* const sV = sKV + kTileBytes;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, c = lane & 31;
    const int kh = wave & 1, qh = wave >> 1;
    const int64_t item = scheduled_item(sched, order, blockIdx.x);
    if (item < 0) return;  // padding slot (whole workgroup)
    const int64_t bh = item / n;
    const int qb = (int)(item % n);
    int cnt = kv_count[item];
    cnt = cnt < 0 ? 0 : (cnt > n ? n : cnt);
    const int32_t* list = kv_idx + item * (int64_t)n;
    const int64_t head = bh * (int64_t)S * D;
    const uint16_t* kh_ptr = k + head;
    const uint16_t* vh_ptr = v + head;

    const int qrow = qb * kBlockN + qh * 32 + c;
    bf16x8_t qf[KK], dof[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        qf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(q + head + (int64_t)qrow * D + 16 * kk + 8 * h));
        dof[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(d_o + head + (int64_t)qrow * D + 16 * kk + 8 * h));
    }
    float l2 = lse[bh * (int64_t)S + qrow] * kLog2e;
    float del = delta[bh * (int64_t)S + qrow];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        settle(qf[kk]);
        settle(dof[kk]);
    }
    settle(l2);
    settle(del);
    f32x16_t dQt[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) dQt[t] = zero16();

    // Rows 32 kh + c of the K / V tiles, bytes 32 kk + 16 h.
    const char* krow_base = sK + (32 * kh + c) * T::RSTB + 16 * h;
    const char* vrow_base = sV + (32 * kh + c) * T::RSTB + 16 * h;
    const char* ktr = tr_lane_base(sK, lane, T::RSTB);

    u32x4_t ra[L], rb[L];
    if (cnt > 0) {
        int j0 = list[0];
        j0 = (unsigned)j0 < (unsigned)n ? j0 : 0;
        NABLA_BWD_FETCH(kh_ptr, vh_ptr, j0);
        NABLA_BWD_STAGE(sK, sV);
        if (cnt > 1) {
            int j1 = list[1];
            j1 = (unsigned)j1 < (unsigned)n ? j1 : 0;
            NABLA_BWD_FETCH(kh_ptr, vh_ptr, j1);
        }
        __syncthreads();
    }
    for (int it = 0; it < cnt; ++it) {
        uint32_t dsw[8];
        {
            // S^T and dP^T quadrant: rows = keys 32 kh + c_row(r, h), column = query c.
            // dP^T starts from -Delta (a loop invariant: the compiler keeps it in
            // registers), so the products yield dP - Delta.
            f32x16_t sc = zero16(), dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) dp[r] = -del;
            {
                bf16x8_t a[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(krow_base + 32 * kk));
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) sc = mfma_32x32x16(a[kk], qf[kk], sc);
            }
            {
                bf16x8_t a[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(vrow_base + 32 * kk));
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) dp = mfma_32x32x16(a[kk], dof[kk], dp);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(sc[r] * scale_log2 - l2);
                dp[r] = p * dp[r];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) dsw[e] = pack_bf16x2(dp[2 * e], dp[2 * e + 1]);
        }
        // dQ^T += K^T dS^T: slot s of B is key 32 kh + 16 u + 8 (s/4) + 4 h + s%4.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bf16x8_t bs = as_bf16x8(make_uint4(dsw[4 * u], dsw[4 * u + 1], dsw[4 * u + 2], dsw[4 * u + 3]));
#pragma unroll
            for (int t = 0; t < DT; ++t)
                dQt[t] = mfma_32x32x16(tr_operand<T::RSTB>(ktr, 32 * kh + 16 * u, t), bs, dQt[t]);
        }
        if (it + 1 < cnt) {
            __syncthreads();  // every wave is done with this key block's tiles
            NABLA_BWD_STAGE(sK, sV);
            if (it + 2 < cnt) {
                int j2 = list[it + 2];
                j2 = (unsigned)j2 < (unsigned)n ? j2 : 0;
                NABLA_BWD_FETCH(kh_ptr, vh_ptr, j2);
            }
            __syncthreads();
        }
    }
    // Sum the two key halves: the kh = 1 wave parks its accumulators in LDS in
    // register order (lane-contiguous words), the kh = 0 wave adds and stores.
    __syncthreads();  // tiles no longer read
    float* red = reinterpret_cast<float*>(sKV) + qh * (DT * 16 * kWave);
    if (kh == 1) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) red[(t * 16 + r) * kWave + lane] = dQt[t][r];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) dQt[t][r] += red[(t * 16 + r) * kWave + lane];
        store_t_acc<DT>(dq + head + (int64_t)qrow * D, dQt, scale, h);
    }
}

// ---------------------------------------------------------------------------
// dq_kernel for D = 128: the same quadrant split and operations in the same
// order (bitwise equal results), but the K/V tiles move global -> LDS by
// direct-to-LDS loads (global_load_lds_dwordx4, 1 KB = four unpadded 256-byte
// rows per wave instruction) into two buffers: the next key block's tiles are
// requested at the start of a step and waited for at its end (one barrier per
// step), with no staging registers and no LDS stores in the waves' streams.
// Unpadded rows are swizzled per 16-byte chunk: K, read both row-wise and
// transposed, keeps chunk ch of row r at ch ^ (4 (r % 4) + (r / 4) % 4); V,
// read row-wise only, at ch ^ (r % 16); both read kinds are then free of bank
// conflicts, and each lane's 24 read addresses are computed once. The two
// buffers are separate arrays and the loop is unrolled by two with a
// branch-free step, so no LDS read waits for loads into the other buffer.
// ---------------------------------------------------------------------------
namespace {
typedef __attribute__((address_space(3))) void bwd_lds_void_t;
typedef __attribute__((address_space(1))) const void bwd_gbl_void_t;
// s_waitcnt vmcnt(0), other counters unconstrained.
__device__ __forceinline__ void bwd_wait_vm0() {
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}
// Workgroup barrier that waits for this wave's LDS accesses (lgkmcnt 0) but not
// for direct-to-LDS loads in flight, and that no memory access crosses.
__device__ __forceinline__ void bwd_tile_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// A workgroup-uniform pointer kept in scalar registers and opaque to the
// optimiser (scalar-base + 32-bit vector-offset loads).
__device__ __forceinline__ const char* bwd_uniform_ptr(const char* p) {
    uint64_t x = reinterpret_cast<uint64_t>(p);
    asm volatile("" : "+s"(x));
    return reinterpret_cast<const char*>(x);
}
// Swizzles of unpadded 256-byte rows (16 chunks of 16 B): chunk ch of row r at
// ch ^ swz(r). K is read row-wise and transposed: 4 (r % 4) + (r / 4) % 4 keeps
// both conflict-free; V is read row-wise only: r % 16.
__device__ __forceinline__ int swz_k(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swz_v(int r) { return r & 15; }
}  // namespace

template <>
__global__ __launch_bounds__(256, 2) void dq_kernel<128>(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta, int S, int n,
    const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_idx,
    const int32_t* __restrict__ order, XcdSchedule sched, float scale, float scale_log2,
    uint16_t* __restrict__ dq) {
    constexpr int D = 128, KK = 8, DT = 4;
    constexpr int TB = kBlockN * 2 * D;  // 16 KB
    __shared__ __attribute__((aligned(1024))) char sK0[TB];
    __shared__ __attribute__((aligned(1024))) char sV0[TB];
    __shared__ __attribute__((aligned(1024))) char sK1[TB];
    __shared__ __attribute__((aligned(1024))) char sV1[TB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, c = lane & 31;
    const int kh = wave & 1, qh = wave >> 1;
    const int64_t item = scheduled_item(sched, order, blockIdx.x);
    if (item < 0) return;
    const int64_t bh = item / n;
    const int qb = (int)(item % n);
    int cnt = kv_count[item];
    cnt = cnt < 0 ? 0 : (cnt > n ? n : cnt);
    const int32_t* list = kv_idx + item * (int64_t)n;
    const int64_t head = bh * (int64_t)S * D;
    const char* khp = reinterpret_cast<const char*>(k + head);
    const char* vhp = reinterpret_cast<const char*>(v + head);

    const int qrow = qb * kBlockN + qh * 32 + c;
    bf16x8_t qf[KK], dof[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        qf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(q + head + (int64_t)qrow * D + 16 * kk + 8 * h));
        dof[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(d_o + head + (int64_t)qrow * D + 16 * kk + 8 * h));
    }
    float l2 = lse[bh * (int64_t)S + qrow] * kLog2e;
    float del = delta[bh * (int64_t)S + qrow];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        settle(qf[kk]);
        settle(dof[kk]);
    }
    settle(l2);
    settle(del);
    f32x16_t dQt[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) dQt[t] = zero16();

    // Read addresses within a tile.
    uint32_t ka[KK], va[KK], ta[2][DT];
    {
        const int x = c & 15;
        const int row = 32 * kh + c;
        const uint32_t kb = (uint32_t)(row * 256 + 16 * ((h ^ (swz_k(x) & 1)) + 2 * (swz_k(x) >> 1)));
        const uint32_t vb = (uint32_t)(row * 256 + 16 * ((h ^ (swz_v(x) & 1)) + 2 * (swz_v(x) >> 1)));
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            ka[kk] = kb ^ (32u * kk);
            va[kk] = vb ^ (32u * kk);
        }
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
            const int xr = 8 * hi + 4 * (lane >> 5) + ((lane & 15) >> 2);
            const int c0 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
            const uint32_t tb = (uint32_t)(xr * 256 + 16 * (c0 ^ swz_k(xr)) + 8 * (lane & 1));
#pragma unroll
            for (int t = 0; t < DT; ++t) ta[hi][t] = tb ^ (64u * t);
        }
    }
    // Direct-to-LDS loads: wave w fills row groups m = w + 4 i.
    uint32_t gk, gv;
    {
        const int r0 = 4 * wave + (lane >> 4);
        gk = (uint32_t)(r0 * 256 + 16 * ((lane & 15) ^ swz_k(r0)));
        gv = (uint32_t)(r0 * 256 + 16 * ((lane & 15) ^ swz_v(r0)));
    }
    auto entry = [&](int i) {
        const int b = __builtin_amdgcn_readfirstlane(list[i]);
        return (unsigned)b < (unsigned)n ? b : 0;
    };
    auto fetch = [&](int j, char* dk_, char* dv_) {
        const char* ks = bwd_uniform_ptr(khp + (int64_t)j * TB);
        const char* vs = bwd_uniform_ptr(vhp + (int64_t)j * TB);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t ok = gk + 4096u * i, ov = gv + 4096u * i;
            settle(ok);
            settle(ov);
            __builtin_amdgcn_global_load_lds((bwd_gbl_void_t*)(ks + ok), (bwd_lds_void_t*)(dk_ + 1024 * (wave + 4 * i)), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((bwd_gbl_void_t*)(vs + ov), (bwd_lds_void_t*)(dv_ + 1024 * (wave + 4 * i)), 16, 0, 0);
        }
    };
    auto compute = [&](const char* sK, const char* sV) {
        uint32_t dsw[8];
        {
            // dP^T starts from -Delta (a loop invariant: the compiler keeps it in
            // registers), so the products yield dP - Delta.
            f32x16_t sc = zero16(), dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) dp[r] = -del;
            {
                bf16x8_t a[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(sK + ka[kk]));
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) sc = mfma_32x32x16(a[kk], qf[kk], sc);
            }
            {
                bf16x8_t a[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(sV + va[kk]));
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) dp = mfma_32x32x16(a[kk], dof[kk], dp);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(sc[r] * scale_log2 - l2);
                dp[r] = p * dp[r];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) dsw[e] = pack_bf16x2(dp[2 * e], dp[2 * e + 1]);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bf16x8_t bs = as_bf16x8(make_uint4(dsw[4 * u], dsw[4 * u + 1], dsw[4 * u + 2], dsw[4 * u + 3]));
            const char* rb = sK + (32 * kh + 16 * u) * 256;
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(rb + ta[0][t]));
                const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(rb + ta[1][t]));
                const uint2 ulo = __builtin_bit_cast(uint2, lo);
                const uint2 uhi = __builtin_bit_cast(uint2, hi);
                dQt[t] = mfma_32x32x16(as_bf16x8(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y)), bs, dQt[t]);
            }
        }
    };
    auto step = [&](int it, const char* cK, const char* cV, char* nK, char* nV) {
        fetch(entry(min(it + 1, cnt - 1)), nK, nV);
        compute(cK, cV);
        bwd_wait_vm0();
        bwd_tile_barrier();
    };
    if (cnt > 0) {
        fetch(entry(0), sK0, sV0);
        bwd_wait_vm0();
        bwd_tile_barrier();
        int it = 0;
        for (; it + 1 < cnt; it += 2) {
            step(it, sK0, sV0, sK1, sV1);
            step(it + 1, sK1, sV1, sK0, sV0);
        }
        if (it < cnt) step(it, sK0, sV0, sK1, sV1);
    }
    // Sum the two key halves through LDS (tiles no longer read).
    __syncthreads();
    float* red = reinterpret_cast<float*>(qh ? sV0 : sK0);
    if (kh == 1) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) red[(t * 16 + r) * kWave + lane] = dQt[t][r];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) dQt[t][r] += red[(t * 16 + r) * kWave + lane];
        store_t_acc<DT>(dq + head + (int64_t)qrow * D, dQt, scale, h);
    }
}

// ---------------------------------------------------------------------------
// dkdv_kernel for D = 128: the same quadrants and products in the same order
// (bitwise equal results), with the Q/dO tiles moved by direct-to-LDS loads
// into two buffers as in dq_kernel<128> (both tiles are read row-wise and
// transposed, so both use the K swizzle), and the second product split by
// output instead of by head dimension: the query-half-0 wave of a key half
// accumulates dV over all of D and the query-half-1 wave dK. Each wave then
// needs the other wave's half of only one of P and dS (the dV wave receives
// P, the dK wave dS), which halves the exchange and lets two workgroups fit
// the LDS. LSE and -Delta of the staged rows are double-buffered with the
// tiles (written by wave 0 from values it loaded a step earlier). Two
// barriers per step: one for the exchange, one for the tile buffers.
// ---------------------------------------------------------------------------
template <>
__global__ __launch_bounds__(256, 2) void dkdv_kernel<128>(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta, int S, int n,
    const int32_t* __restrict__ q_count, const int32_t* __restrict__ q_idx,
    const int32_t* __restrict__ order, XcdSchedule sched, float scale, float scale_log2,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
    constexpr int D = 128, KK = 8, DT = 4;
    constexpr int TB = kBlockN * 2 * D;  // 16 KB
    __shared__ __attribute__((aligned(1024))) char sQ0[TB];
    __shared__ __attribute__((aligned(1024))) char sO0[TB];
    __shared__ __attribute__((aligned(1024))) char sQ1[TB];
    __shared__ __attribute__((aligned(1024))) char sO1[TB];
    __shared__ __attribute__((aligned(16))) float sL0[kBlockN], sL1[kBlockN];
    __shared__ __attribute__((aligned(16))) float sD0[kBlockN], sD1[kBlockN];
    // The half of P (from dK waves) or dS (from dV waves) a wave hands over,
    // [wave][group][lane]: lane-contiguous 16-byte words.
    __shared__ __attribute__((aligned(16))) u32x4_t sX[4][2][kWave];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, c = lane & 31;
    const int kh = wave & 1, qh = wave >> 1;  // qh 0: dV wave, 1: dK wave
    // Workgroup-uniform (item < 2^31): the pointers derived from it stay in scalar registers.
    const int64_t item = __builtin_amdgcn_readfirstlane((int)scheduled_item(sched, order, blockIdx.x));
    if (item < 0) return;
    const int64_t bh = item / n;
    const int kb = (int)(item % n);
    int cnt = q_count[item];
    cnt = cnt < 0 ? 0 : (cnt > n ? n : cnt);
    const int32_t* list = q_idx + item * (int64_t)n;
    const int64_t head = bh * (int64_t)S * D;
    const char* qhp = reinterpret_cast<const char*>(q + head);
    const char* ohp = reinterpret_cast<const char*>(d_o + head);
    const float* lh = lse + bh * (int64_t)S;
    const float* dh = delta + bh * (int64_t)S;

    const int krow = kb * kBlockN + kh * 32 + c;
    bf16x8_t kf[KK], vf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        kf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(k + head + (int64_t)krow * D + 16 * kk + 8 * h));
        vf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(v + head + (int64_t)krow * D + 16 * kk + 8 * h));
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        settle(kf[kk]);
        settle(vf[kk]);
    }
    f32x16_t acc[DT];  // dV^T (qh = 0) or dK^T (qh = 1)
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] = zero16();

    // Read addresses within a tile: row 32 qh + c, chunk 2 kk + h (row reads),
    // and the transposed reads of rows 4 h + (lane % 16) / 4 (+8), d tile t.
    uint32_t ra[KK], ta[2][DT];
    {
        const int x = c & 15;
        const int row = 32 * qh + c;
        const uint32_t rb = (uint32_t)(row * 256 + 16 * ((h ^ (swz_k(x) & 1)) + 2 * (swz_k(x) >> 1)));
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) ra[kk] = rb ^ (32u * kk);
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
            const int xr = 8 * hi + 4 * (lane >> 5) + ((lane & 15) >> 2);
            const int c0 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
            const uint32_t tb = (uint32_t)(xr * 256 + 16 * (c0 ^ swz_k(xr)) + 8 * (lane & 1));
#pragma unroll
            for (int t = 0; t < DT; ++t) ta[hi][t] = tb ^ (64u * t);
        }
    }
    // Direct-to-LDS loads: wave w fills row groups m = w + 4 i of both tiles.
    uint32_t g0;
    {
        const int r0 = 4 * wave + (lane >> 4);
        g0 = (uint32_t)(r0 * 256 + 16 * ((lane & 15) ^ swz_k(r0)));
    }
    auto entry = [&](int i) {
        const int b = __builtin_amdgcn_readfirstlane(list[i]);
        return (unsigned)b < (unsigned)n ? b : 0;
    };
    auto fetch = [&](int i, char* dq_, char* do_) {
        const char* qs = bwd_uniform_ptr(qhp + (int64_t)i * TB);
        const char* os = bwd_uniform_ptr(ohp + (int64_t)i * TB);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t o = g0 + 4096u * j;
            settle(o);
            __builtin_amdgcn_global_load_lds((bwd_gbl_void_t*)(qs + o), (bwd_lds_void_t*)(dq_ + 1024 * (wave + 4 * j)), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((bwd_gbl_void_t*)(os + o), (bwd_lds_void_t*)(do_ + 1024 * (wave + 4 * j)), 16, 0, 0);
        }
    };
    float rl = 0.f, rd = 0.f;  // LSE / Delta of query row `lane` of the step after next (wave 0)
    // acc += T^T B over the query halves in order (b0: queries 0..31, b1: 32..63);
    // slot s of B is query 32 qt + 16 u + 8 (s/4) + 4 h + s%4, matched by the
    // transposed reads of tile T.
    auto accumulate = [&](const char* tile, const uint32_t (&b0)[8], const uint32_t (&b1)[8]) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t* bb = qt == 0 ? b0 : b1;
                const bf16x8_t b = as_bf16x8(make_uint4(bb[4 * u], bb[4 * u + 1], bb[4 * u + 2], bb[4 * u + 3]));
                const char* rbp = tile + (32 * qt + 16 * u) * 256;
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(rbp + ta[0][t]));
                    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(rbp + ta[1][t]));
                    const uint2 ulo = __builtin_bit_cast(uint2, lo);
                    const uint2 uhi = __builtin_bit_cast(uint2, hi);
                    acc[t] = mfma_32x32x16(as_bf16x8(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y)), b, acc[t]);
                }
            }
    };
    auto step = [&](int it, const char* cQ, const char* cO, const float* cL, const float* cD, char* nQ,
                    char* nO, float* nL, float* nD) {
        fetch(entry(min(it + 1, cnt - 1)), nQ, nO);
        if (wave == 0) {
            nL[lane] = rl * kLog2e;
            nD[lane] = -rd;
            const int i2 = entry(min(it + 2, cnt - 1));
            rl = lh[(int64_t)i2 * kBlockN + lane];
            rd = dh[(int64_t)i2 * kBlockN + lane];
        }
        uint32_t pw[8], dsw[8];
        {
            // S and dP quadrant: rows = queries 32 qh + c_row(r, h), column = key c.
            // dP starts from -Delta of its rows, so the products yield dP - Delta.
            f32x16_t sc = zero16(), dp;
            const float* lrow = cL + 32 * qh + 4 * h;
            const float* drow = cD + 32 * qh + 4 * h;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 d4 = *reinterpret_cast<const float4*>(drow + 8 * g);
                dp[4 * g + 0] = d4.x;
                dp[4 * g + 1] = d4.y;
                dp[4 * g + 2] = d4.z;
                dp[4 * g + 3] = d4.w;
            }
            {
                bf16x8_t a[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(cQ + ra[kk]));
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) sc = mfma_32x32x16(a[kk], kf[kk], sc);
            }
            {
                bf16x8_t a[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(cO + ra[kk]));
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) dp = mfma_32x32x16(a[kk], vf[kk], dp);
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 l4 = *reinterpret_cast<const float4*>(lrow + 8 * g);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    const float p = __builtin_amdgcn_exp2f(sc[r] * scale_log2 - lv[e]);
                    sc[r] = p;
                    dp[r] = p * dp[r];
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pw[e] = pack_bf16x2(sc[2 * e], sc[2 * e + 1]);
                dsw[e] = pack_bf16x2(dp[2 * e], dp[2 * e + 1]);
            }
        }
        // The dV wave hands over its dS and receives P, the dK wave the reverse
        // (one code path per role, so the half handed over is dead after its write).
        auto trade = [&](const uint32_t (&give)[8], uint32_t (&got)[8]) {
            sX[wave][0][lane] = u32x4_t{give[0], give[1], give[2], give[3]};
            sX[wave][1][lane] = u32x4_t{give[4], give[5], give[6], give[7]};
            bwd_tile_barrier();
            const u32x4_t x0 = sX[wave ^ 2][0][lane], x1 = sX[wave ^ 2][1][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                got[e] = x0[e];
                got[4 + e] = x1[e];
            }
        };
        uint32_t got[8];
        if (qh == 0) {
            trade(dsw, got);
            accumulate(cO, pw, got);   // dV^T += dO^T P
        } else {
            trade(pw, got);
            accumulate(cQ, got, dsw);  // dK^T += Q^T dS
        }
        bwd_wait_vm0();
        bwd_tile_barrier();
    };
    if (cnt > 0) {
        const int i0 = entry(0);
        fetch(i0, sQ0, sO0);
        if (wave == 0) {
            sL0[lane] = lh[(int64_t)i0 * kBlockN + lane] * kLog2e;
            sD0[lane] = -dh[(int64_t)i0 * kBlockN + lane];
            const int i1 = entry(min(1, cnt - 1));
            rl = lh[(int64_t)i1 * kBlockN + lane];
            rd = dh[(int64_t)i1 * kBlockN + lane];
        }
        bwd_wait_vm0();
        bwd_tile_barrier();
        int it = 0;
        for (; it + 1 < cnt; it += 2) {
            step(it, sQ0, sO0, sL0, sD0, sQ1, sO1, sL1, sD1);
            step(it + 1, sQ1, sO1, sL1, sD1, sQ0, sO0, sL0, sD0);
        }
        if (it < cnt) step(it, sQ0, sO0, sL0, sD0, sQ1, sO1, sL1, sD1);
    }
    if (qh == 0) store_t_acc<DT>(dv + head + (int64_t)krow * D, acc, 1.0f, h);
    else store_t_acc<DT>(dk + head + (int64_t)krow * D, acc, scale, h);
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
        dkdv_kernel<128><<<grid, 256, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)d_o, lse,
            delta, S, n, q_count, q_idx, order, sched, softmax_scale, sl2, (uint16_t*)dk,
            (uint16_t*)dv);
    else
        dkdv_kernel<64><<<grid, 256, 0, stream>>>(
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
        dq_kernel<128><<<grid, 256, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)d_o, lse,
            delta, S, n, kv_count, kv_idx, order, sched, softmax_scale, sl2, (uint16_t*)dq);
    else
        dq_kernel<64><<<grid, 256, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)d_o, lse,
            delta, S, n, kv_count, kv_idx, order, sched, softmax_scale, sl2, (uint16_t*)dq);
    return hipGetLastError();
}

}  // namespace nabla

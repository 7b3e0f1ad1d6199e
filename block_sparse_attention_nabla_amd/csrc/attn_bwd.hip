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
// deterministic. Operand layouts follow attn_fwd.hip: a 32 x 32 accumulator's
// rows become the contraction slots of the next MFMA's B operand, and the
// matching A operand is read from a transposed LDS copy with the same slot map.

#include "common.h"
#include "kernels.h"

namespace nabla {

template <int D>
struct BwdTile {
    static constexpr int RST = D + 8;        // row-major tile stride (bf16)
    static constexpr int TST = kBlockN + 4;  // transposed tile stride (tokens)
};

// 64 x D block: row-major copy (dst_rm, may be null) and/or transposed copy
// (dst_t[d][token], may be null). 128 threads.
template <int D>
__device__ __forceinline__ void stage_block(const uint16_t* __restrict__ src, uint16_t* dst_rm,
                                            uint16_t* dst_t, int tid) {
    constexpr int CG = D / 8;
    constexpr int RST = BwdTile<D>::RST, TST = BwdTile<D>::TST;
    if (dst_rm) {
#pragma unroll
        for (int e = tid; e < kBlockN * CG; e += 128) {
            const int row = e / CG, cg = e % CG;
            *reinterpret_cast<uint4*>(dst_rm + row * RST + cg * 8) =
                *reinterpret_cast<const uint4*>(src + row * D + cg * 8);
        }
    }
    if (dst_t) {
#pragma unroll
        for (int e = tid; e < (kBlockN / 4) * CG; e += 128) {
            const int kg = e / CG, dg = e % CG;
            uint4 r[4];
#pragma unroll
            for (int a = 0; a < 4; ++a)
                r[a] = *reinterpret_cast<const uint4*>(src + (kg * 4 + a) * D + dg * 8);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                uint32_t e4[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const uint32_t w = (b >> 1) == 0 ? r[a].x : (b >> 1) == 1 ? r[a].y
                                     : (b >> 1) == 2 ? r[a].z : r[a].w;
                    e4[a] = (b & 1) ? (w >> 16) : (w & 0xffffu);
                }
                uint2 out;
                out.x = e4[0] | (e4[1] << 16);
                out.y = e4[2] | (e4[3] << 16);
                *reinterpret_cast<uint2*>(dst_t + (dg * 8 + b) * TST + kg * 4) = out;
            }
        }
    }
}

// A operand from a transposed tile: row (32t + c), slots = tokens
// base + 8*(s/4) + 4h + s%4 for s = 0..7 (base = 32*tile + 16*u).
__device__ __forceinline__ bf16x8_t read_t_operand(const uint16_t* tile_row, int base, int h) {
    const uint2 lo = *reinterpret_cast<const uint2*>(tile_row + base + 4 * h);
    const uint2 hi = *reinterpret_cast<const uint2*>(tile_row + base + 8 + 4 * h);
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

__device__ __forceinline__ bf16x8_t pack_b_operand(const f32x16_t& x, int u) {
    uint4 p;
    p.x = pack_bf16x2(x[8 * u + 0], x[8 * u + 1]);
    p.y = pack_bf16x2(x[8 * u + 2], x[8 * u + 3]);
    p.z = pack_bf16x2(x[8 * u + 4], x[8 * u + 5]);
    p.w = pack_bf16x2(x[8 * u + 6], x[8 * u + 7]);
    return as_bf16x8(p);
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

// ---------------------------------------------------------------------------
// dK, dV for one 64-key block; wave w owns keys 32w .. 32w+31.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta, int S, int n,
    const int32_t* __restrict__ q_count, const int32_t* __restrict__ q_idx,
    const int32_t* __restrict__ order, XcdSchedule sched, float scale, float scale_log2,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
    constexpr int RST = BwdTile<D>::RST, TST = BwdTile<D>::TST;
    constexpr int KK = D / 16, DT = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t sQ[kBlockN * RST];
    __shared__ __attribute__((aligned(16))) uint16_t sQt[D * TST];
    __shared__ __attribute__((aligned(16))) uint16_t sdO[kBlockN * RST];
    __shared__ __attribute__((aligned(16))) uint16_t sdOt[D * TST];
    __shared__ float sL[kBlockN], sDel[kBlockN];

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

    for (int it = 0; it < cnt; ++it) {
        const int i = list[it];
        if ((unsigned)i >= (unsigned)n) continue;  // uniform across the workgroup
        const int64_t tok0 = (int64_t)i * kBlockN;
        stage_block<D>(q + head + tok0 * D, sQ, sQt, tid);
        stage_block<D>(d_o + head + tok0 * D, sdO, sdOt, tid);
        if (tid < kBlockN) {
            sL[tid] = lse[bh * (int64_t)S + tok0 + tid] * kLog2e;
            sDel[tid] = delta[bh * (int64_t)S + tok0 + tid];
        }
        __syncthreads();
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            // S and dP tiles: rows = queries 32qt + c_row(r, h), column = key c of this wave.
            f32x16_t sc = zero16(), dp = zero16();
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const bf16x8_t aq = as_bf16x8(
                    *reinterpret_cast<const uint4*>(sQ + (32 * qt + c) * RST + 16 * kk + 8 * h));
                const bf16x8_t ad = as_bf16x8(
                    *reinterpret_cast<const uint4*>(sdO + (32 * qt + c) * RST + 16 * kk + 8 * h));
                sc = mfma_32x32x16(aq, kf[kk], sc);
                dp = mfma_32x32x16(ad, vf[kk], dp);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qr = 32 * qt + c_row(r, h);
                const float p = exp2f(sc[r] * scale_log2 - sL[qr]);
                sc[r] = p;
                dp[r] = p * (dp[r] - sDel[qr]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16x8_t bp = pack_b_operand(sc, u);
                const bf16x8_t bs = pack_b_operand(dp, u);
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    dVt[t] = mfma_32x32x16(read_t_operand(sdOt + (32 * t + c) * TST, 32 * qt + 16 * u, h),
                                           bp, dVt[t]);
                    dKt[t] = mfma_32x32x16(read_t_operand(sQt + (32 * t + c) * TST, 32 * qt + 16 * u, h),
                                           bs, dKt[t]);
                }
            }
        }
        __syncthreads();
    }
    store_t_acc<DT>(dk + head + (int64_t)krow * D, dKt, scale, h);
    store_t_acc<DT>(dv + head + (int64_t)krow * D, dVt, 1.0f, h);
}

// ---------------------------------------------------------------------------
// dQ for one 64-query block; wave w owns queries 32w .. 32w+31.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta, int S, int n,
    const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_idx,
    const int32_t* __restrict__ order, XcdSchedule sched, float scale, float scale_log2,
    uint16_t* __restrict__ dq) {
    constexpr int RST = BwdTile<D>::RST, TST = BwdTile<D>::TST;
    constexpr int KK = D / 16, DT = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t sK[kBlockN * RST];
    __shared__ __attribute__((aligned(16))) uint16_t sKt[D * TST];
    __shared__ __attribute__((aligned(16))) uint16_t sV[kBlockN * RST];

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

    for (int it = 0; it < cnt; ++it) {
        const int j = list[it];
        if ((unsigned)j >= (unsigned)n) continue;  // uniform across the workgroup
        const int64_t tok0 = (int64_t)j * kBlockN;
        stage_block<D>(k + head + tok0 * D, sK, sKt, tid);
        stage_block<D>(v + head + tok0 * D, sV, nullptr, tid);
        __syncthreads();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            // S^T and dP^T tiles: rows = keys 32kt + c_row(r, h), column = query c.
            f32x16_t sc = zero16(), dp = zero16();
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const bf16x8_t ak = as_bf16x8(
                    *reinterpret_cast<const uint4*>(sK + (32 * kt + c) * RST + 16 * kk + 8 * h));
                const bf16x8_t av = as_bf16x8(
                    *reinterpret_cast<const uint4*>(sV + (32 * kt + c) * RST + 16 * kk + 8 * h));
                sc = mfma_32x32x16(ak, qf[kk], sc);
                dp = mfma_32x32x16(av, dof[kk], dp);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = exp2f(sc[r] * scale_log2 - l2);
                dp[r] = p * (dp[r] - del);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16x8_t bs = pack_b_operand(dp, u);
#pragma unroll
                for (int t = 0; t < DT; ++t)
                    dQt[t] = mfma_32x32x16(read_t_operand(sKt + (32 * t + c) * TST, 32 * kt + 16 * u, h),
                                           bs, dQt[t]);
            }
        }
        __syncthreads();
    }
    store_t_acc<DT>(dq + head + (int64_t)qrow * D, dQt, scale, h);
}

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

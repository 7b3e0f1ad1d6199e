// attn_fwd.hip -- block-sparse flash-attention forward on gfx950.
//
// Computes eq. (4) of "NABLA: Neighborhood Adaptive Block-Level Attention"
// (section 2.2) with the NABLA/STA block mask of section 3.1.3: each query
// block attends only to the key blocks of its kept list. Online softmax over
// the kept blocks (flash-attention style), bf16 MFMA with fp32 accumulation.
//
// Work item = one 64-row query block; workgroup = 2 waves of 32 query rows.
// Per kept key block j:
//   K_j  -> LDS row-major   (A operand of S^T = K Q^T),
//   V_j  -> LDS transposed  (A operand of O^T += V^T P^T),
//   Q^T  stays in registers (B operand), P^T goes from the S^T accumulators
//   straight into the B operand of the PV product: the accumulator's rows
//   (keys) become the contraction slots, and V^T is read with the same slot
//   -> key assignment, so no data movement is needed for P.
// exp2 is used throughout with log2(e) folded into the scale.

#include "common.h"
#include "kernels.h"

namespace nabla {

template <int D>
struct FwdTile {
    static constexpr int KST = D + 8;        // K row stride in LDS (bf16), 16-byte pad
    static constexpr int VST = kBlockN + 4;  // V^T row stride (keys), 8-byte pad
};

// Load one 64 x D K block into LDS row-major and the V block transposed
// (sVt[d][key]). 128 threads.
template <int D>
__device__ __forceinline__ void load_kv_block(const uint16_t* __restrict__ kb,
                                              const uint16_t* __restrict__ vb, uint16_t* sK,
                                              uint16_t* sVt, int tid) {
    constexpr int CG = D / 8;
    constexpr int KST = FwdTile<D>::KST, VST = FwdTile<D>::VST;
#pragma unroll
    for (int e = tid; e < kBlockN * CG; e += 128) {
        const int row = e / CG, cg = e % CG;
        *reinterpret_cast<uint4*>(sK + row * KST + cg * 8) =
            *reinterpret_cast<const uint4*>(kb + row * D + cg * 8);
    }
#pragma unroll
    for (int e = tid; e < (kBlockN / 4) * CG; e += 128) {
        const int kg = e / CG, dg = e % CG;
        uint4 r[4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
            r[a] = *reinterpret_cast<const uint4*>(vb + (kg * 4 + a) * D + dg * 8);
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
            *reinterpret_cast<uint2*>(sVt + (dg * 8 + b) * VST + kg * 4) = out;
        }
    }
}

template <int D>
__global__ __launch_bounds__(128) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int S, int n, const int32_t* __restrict__ kv_count,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ order, float scale_log2,
    void* __restrict__ o, int o_fp32, float* __restrict__ lse) {
    constexpr int KST = FwdTile<D>::KST, VST = FwdTile<D>::VST;
    constexpr int KK = D / 16;  // MFMA k-steps over the head dimension
    constexpr int DT = D / 32;  // 32-row d tiles of O^T
    __shared__ __attribute__((aligned(16))) uint16_t sK[kBlockN * KST];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[D * VST];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, c = lane & 31;
    const int64_t item = order[blockIdx.x];
    const int64_t bh = item / n;
    const int qb = (int)(item % n);
    int cnt = kv_count[item];
    cnt = cnt < 0 ? 0 : (cnt > n ? n : cnt);
    const int32_t* list = kv_idx + item * (int64_t)n;
    const int64_t head = bh * (int64_t)S * D;

    // Q^T as the B operand: lane holds query (wave*32 + c), d = 16*kk + 8*h + 0..7.
    const int qrow = qb * kBlockN + wave * 32 + c;
    bf16x8_t qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(q + head + (int64_t)qrow * D + 16 * kk + 8 * h));

    f32x16_t oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = zero16();
    // l_run: sum of the fp32 probabilities (for LSE); w_run: sum of the bf16-rounded
    // probabilities that feed the PV product (the output's normaliser).
    float m_run = -INFINITY, l_run = 0.f, w_run = 0.f;

    for (int it = 0; it < cnt; ++it) {
        const int j = list[it];
        if ((unsigned)j >= (unsigned)n) continue;  // uniform across the workgroup
        load_kv_block<D>(k + head + (int64_t)j * kBlockN * D, v + head + (int64_t)j * kBlockN * D, sK,
                         sVt, tid);
        __syncthreads();

        // S^T (64 keys x 32 queries) as two 32 x 32 tiles.
        f32x16_t s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            s[kt] = zero16();
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const bf16x8_t a = as_bf16x8(
                    *reinterpret_cast<const uint4*>(sK + (32 * kt + c) * KST + 16 * kk + 8 * h));
                s[kt] = mfma_32x32x16(a, qf[kk], s[kt]);
            }
        }
        // Online softmax for query column c (keys split over this lane and lane ^ 32).
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        float rs = 0.f, ws = 0.f;
        uint4 pb[2][2];  // bf16 probabilities, B operands of the PV product
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                uint32_t w4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = exp2f(s[kt][8 * u + 2 * e] * scale_log2 - m_new);
                    const float p1 = exp2f(s[kt][8 * u + 2 * e + 1] * scale_log2 - m_new);
                    rs += p0 + p1;
                    w4[e] = pack_bf16x2(p0, p1);
                    ws += bf16_bits_to_f32(w4[e] & 0xffffu) + bf16_bits_to_f32(w4[e] >> 16);
                }
                pb[kt][u] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
            }
        rs += __shfl_xor(rs, 32);
        ws += __shfl_xor(ws, 32);
        l_run = l_run * alpha + rs;
        w_run = w_run * alpha + ws;
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;

        // O^T += V^T P^T. For key tile kt and half u, B = S^T registers 8u..8u+7:
        // slot s is key 32kt + 16u + 8*(s/4) + 4h + s%4; V^T is read the same way.
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16x8_t b = as_bf16x8(pb[kt][u]);
                const int key0 = 32 * kt + 16 * u + 4 * h;
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    const uint16_t* vrow = sVt + (32 * t + c) * VST;
                    const uint2 lo = *reinterpret_cast<const uint2*>(vrow + key0);
                    const uint2 hi = *reinterpret_cast<const uint2*>(vrow + key0 + 8);
                    const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
                    oacc[t] = mfma_32x32x16(as_bf16x8(av), b, oacc[t]);
                }
            }
        __syncthreads();
    }

    // Epilogue: O[query][d] = O^T[d][query] / l. This lane holds query (wave*32 + c)
    // and d = 32t + 8g + 4h + e for register 4g + e of tile t.
    const float inv_l = w_run > 0.f ? 1.0f / w_run : 0.f;
    if (o_fp32) {
        float* orow = static_cast<float*>(o) + head + (int64_t)qrow * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<float4*>(orow + 32 * t + 8 * g + 4 * h) =
                    make_float4(oacc[t][4 * g + 0] * inv_l, oacc[t][4 * g + 1] * inv_l,
                                oacc[t][4 * g + 2] * inv_l, oacc[t][4 * g + 3] * inv_l);
    } else {
        uint16_t* orow = static_cast<uint16_t*>(o) + head + (int64_t)qrow * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 w;
                w.x = pack_bf16x2(oacc[t][4 * g + 0] * inv_l, oacc[t][4 * g + 1] * inv_l);
                w.y = pack_bf16x2(oacc[t][4 * g + 2] * inv_l, oacc[t][4 * g + 3] * inv_l);
                *reinterpret_cast<uint2*>(orow + 32 * t + 8 * g + 4 * h) = w;
            }
    }
    if (lse && h == 0)
        lse[bh * (int64_t)S + qrow] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, int64_t BH, int S, int D,
                           const int32_t* kv_count, const int32_t* kv_idx, const int32_t* order,
                           float softmax_scale, void* o, bool o_fp32, float* lse,
                           hipStream_t stream) {
    const int n = S / kBlockN;
    const unsigned grid = (unsigned)(BH * n);
    const float sl2 = softmax_scale * kLog2e;
    if (D == 128)
        attn_fwd_kernel<128><<<grid, 128, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, S, n, kv_count, kv_idx,
            order, sl2, o, o_fp32 ? 1 : 0, lse);
    else
        attn_fwd_kernel<64><<<grid, 128, 0, stream>>>(
            (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, S, n, kv_count, kv_idx,
            order, sl2, o, o_fp32 ? 1 : 0, lse);
    return hipGetLastError();
}

}  // namespace nabla

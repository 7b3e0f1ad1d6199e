// attn_fwd.hip -- block-sparse flash-attention forward on gfx950.
//
// Computes eq. (4) of "NABLA: Neighborhood Adaptive Block-Level Attention"
// (section 2.2) with the NABLA/STA block mask of section 3.1.3: each query
// block attends only to the key blocks of its kept list. Online softmax over
// the kept blocks (flash-attention style), bf16 MFMA with fp32 accumulation.
//
// Work item = one 64-row query block; workgroup = 2 waves of 32 query rows.
// Per kept key block j:
//   S^T = K Q^T: A operand = K rows from LDS, B operand = Q^T in registers;
//   O^T += V^T P^T: B operand = P^T straight from the S^T accumulators (their
//   rows become the contraction slots), A operand = V^T read from the
//   row-major V tile with the transposing LDS read (ds_read_b64_tr_b16),
//   which hands each lane one column of four consecutive V rows -- matching
//   the accumulator's slot map, so neither P nor V is ever shuffled.
// K and V tiles are prefetched two blocks ahead into registers with plain
// 16-byte loads and written to padded LDS rows after the current block's
// reads, so global latency overlaps a whole block of compute. exp2 is used
// with log2(e) folded into the scale, and the output is rescaled only when a
// row maximum grows by more than 2^8.

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
    static constexpr int LOADS = kBlockN * CPR / 128;  // 16-byte chunks per thread per tile
};

}  // namespace

template <int D>
__global__ __launch_bounds__(128, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int S, int n, const int32_t* __restrict__ kv_count,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ order, XcdSchedule sched,
    float scale_log2, void* __restrict__ o, int o_fp32, float* __restrict__ lse) {
    using T = Tile<D>;
    constexpr int KK = D / 16;  // MFMA k-steps over the head dimension
    constexpr int DT = D / 32;  // 32-row d tiles of O^T
    constexpr int L = T::LOADS;
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

    // Q^T as the B operand: lane holds query (wave*32 + c), d = 16*kk + 8*h + 0..7.
    const int qrow = qb * kBlockN + wave * 32 + c;
    bf16x8_t qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(q + head + (int64_t)qrow * D + 16 * kk + 8 * h));

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

    // Lane bases for LDS reads (everything else is an immediate offset).
    // K rows for the S^T A operand: row 32 kt + c, bytes 32 kk + 16 h.
    const char* kbase = sK + c * T::KSTB + 16 * h;
    // V^T via the transposing read: this lane supplies the address of row
    // rbase + 4h + (lane % 16) / 4, columns 32 dt + 16 ((lane / 16) % 2) +
    // 4 (lane % 4) .. +3, and receives V[rbase + 4h + jj][32 dt + lane % 32]
    // for jj = 0..3 (rbase = 32 kt + 16 u, plus 8 for the upper four slots).
    const char* vbase = sV + (4 * h + ((lane & 15) >> 2)) * T::VSTB +
                        2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    f32x16_t oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = zero16();
    // l_run: sum of fp32 probabilities (for LSE); w_run: sum of the bf16-rounded
    // probabilities that feed the PV product (the output's normaliser).
    float m_run = -INFINITY, l_run = 0.f, w_run = 0.f;
    const uint32_t ones_bf16x2 = 0x3f803f80u;

    if (cnt > 0) {
        NABLA_FETCH(0);
        NABLA_STAGE();
        if (cnt > 1) NABLA_FETCH(1);
        __syncthreads();
    }
    for (int it = 0; it < cnt; ++it) {
        // S^T (64 keys x 32 queries) as two 32 x 32 tiles; A fragments read first.
        f32x16_t s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            bf16x8_t a[KK];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                a[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(kbase + 32 * kt * T::KSTB + 32 * kk));
            s[kt] = zero16();
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) s[kt] = mfma_32x32x16(a[kk], qf[kk], s[kt]);
        }

        // Online softmax for query column c (keys split over this lane and lane ^ 32).
        float mx = s[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = __builtin_fmaxf(mx, s[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[1][r]);
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
        // Rescale only when some row's maximum grew by more than 2^8; otherwise
        // keep the old reference (probabilities then stay below 2^8).
        const bool grow = mx > m_run + kRescaleLog2;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
            w_run *= alpha;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
            m_run = m_new;
        }
        float rs = 0.f, ws = 0.f;
        uint32_t pw[2][8];  // bf16 probabilities, B operands of the PV product
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p0 = __builtin_amdgcn_exp2f(s[kt][2 * e] * scale_log2 - m_run);
                const float p1 = __builtin_amdgcn_exp2f(s[kt][2 * e + 1] * scale_log2 - m_run);
                rs += p0 + p1;
                pw[kt][e] = pack_bf16x2(p0, p1);
                ws = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[kt][e]),
                                                     __builtin_bit_cast(bf16x2_t, ones_bf16x2), ws,
                                                     false);
            }
        rs += __shfl_xor(rs, 32);
        ws += __shfl_xor(ws, 32);
        l_run += rs;
        w_run += ws;

        // O^T += V^T P^T. For key tile kt and half u, B = S^T registers 8u..8u+7:
        // slot s is key 32kt + 16u + 8*(s/4) + 4h + s%4; the transposing reads
        // of rows 32kt + 16u + {0, 8} + 4h + jj deliver V^T with the same map.
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16x8_t b = as_bf16x8(make_uint4(pw[kt][4 * u], pw[kt][4 * u + 1],
                                                        pw[kt][4 * u + 2], pw[kt][4 * u + 3]));
                const char* vrow = vbase + (32 * kt + 16 * u) * T::VSTB;
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_v4i16_t*)(vrow + 64 * t));
                    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_v4i16_t*)(vrow + 8 * T::VSTB + 64 * t));
                    const uint2 ulo = __builtin_bit_cast(uint2, lo);
                    const uint2 uhi = __builtin_bit_cast(uint2, hi);
                    oacc[t] = mfma_32x32x16(as_bf16x8(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y)), b,
                                            oacc[t]);
                }
            }
        if (it + 1 < cnt) {
            __syncthreads();  // every wave has read K_j and V_j
            NABLA_STAGE();  // block it+1, fetched one iteration ago
            if (it + 2 < cnt) NABLA_FETCH(it + 2);
            __syncthreads();
        }
    }

#undef NABLA_FETCH
#undef NABLA_STAGE

    // Epilogue: O[query][d] = O^T[d][query] / w. This lane holds query (wave*32 + c)
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
        lse[bh * (int64_t)S + qrow] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
}

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

}  // namespace nabla

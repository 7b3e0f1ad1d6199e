// kernels.h -- launchers of the gfx950 NABLA kernels (host side, after validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nabla.h"

namespace nabla {

// STA window in tile units (one tile = one block): grid tT x tH x tW tiles,
// window wt x wh x ww tiles. on == 0 disables the union.
struct StaParams {
    int on;
    int tT, tH, tW;
    int wt, wh, ww;
};

// Outputs of the pooling stage (all [BH, n, ...] in block order).
struct PoolOut {
    float* qa;      // fp32 block means of Q [BH, n, D] (operands of the reduced logits)
    float* ka;      // fp32 block means of K
    double* qa64;   // the exact block means in fp64 [BH, n, D]
    double* ka64;
    float* qnorm;   // |Q_a[i]|_2, rounded up [BH, n]
    float* knorm;   // |K_a[j]|_2, rounded up [BH, n]
    float* kmax;    // max_j |K_a[j]|_2 per head [BH]
};
hipError_t launch_pool(const void* q, const void* k, const PoolOut& out, int64_t BH, int n, int D,
                       hipStream_t stream);
hipError_t launch_logits(const float* qa, const float* ka, float* logits, int64_t BH, int n, int D,
                         float scale, hipStream_t stream);
// Row selectors of launch_select. bound: kSelCdf -> floor(thr * 2^40) (fixed-point
// mass); kSelTopk -> k - 1 (a count); kSelSta -> unused (no logits needed).
enum { kSelCdf = 0, kSelTopk = 1, kSelSta = 2 };
struct SelectArgs {
    const float* logits;   // fp32 reduced logits [rows, n] (unused by kSelSta)
    int64_t rows;          // BH * n
    int n;
    int keep_all;
    uint64_t bound;
    StaParams sta;
    const double* qa64;    // exact block means (PoolOut)
    const double* ka64;
    const float* qnorm;
    const float* kmax;
    double scale64;        // softmax scale in fp64 (1/sqrt(D))
    float err_unit;        // fp32 logit error bound per unit |Q_a| |K_a| (see select_wave_kernel)
    int32_t* kv_count;
    int32_t* kv_idx;
    uint8_t* dense_mask;
    uint32_t* bits;
    int words_per_row;
};
hipError_t launch_select(int mode, const SelectArgs& args, int D, hipStream_t stream);
hipError_t launch_transpose(const uint32_t* bits, int64_t BH, int n, int words_per_row,
                            int32_t* q_count, int32_t* q_idx, hipStream_t stream);

// Per-head longest-first order over `items` items per head whose counts lie in
// [0, maxc] (maxc <= NABLA_MAX_BLOCKS; others are clamped): order[h*items + p] =
// item id (h*items + i) of head h's p-th item, counts descending (ties in any order).
hipError_t launch_lpt_order(const int32_t* counts, int64_t BH, int items, int maxc,
                            int32_t* order, int32_t* claim, hipStream_t stream);

// XCD-aware launch geometry (see schedule.hip). Three ways to map workgroup b
// to a work item of a per-head longest-first order:
//  kSchedStatic   heads are split into `parts` interleaved shares so that
//                 `units` = BH * parts is a multiple of the 8 XCDs; workgroup b
//                 runs on XCD b % 8 and serves unit x + 8 * (m / cap), position
//                 part + parts * (m % cap), with x = b % 8, m = b / 8.
//  kSchedClaim    the same head-to-XCD mapping, but the `parts` XCDs that share
//                 a head take its positions in longest-first order from a
//                 per-head counter (claim[head], zeroed by the ordering kernel)
//                 as their workgroups start, so a faster XCD takes more items;
//                 cap carries a quarter more workgroups than items, and the
//                 ones that find a head exhausted exit at once.
//  kSchedPosMajor small problems (whose K/V fit the Infinity Cache): position
//                 p of every head before position p + 1 of any head, so the
//                 longest items of all heads start first.
enum : int { kSchedStatic = 0, kSchedClaim = 1, kSchedPosMajor = 2 };
struct XcdSchedule {
    int parts;
    int64_t units;
    int cap;
    int n;  // items per head
    int64_t grid;
    int mode;
    int64_t bh;
    int32_t* claim;
};
XcdSchedule make_schedule(int64_t BH, int n);
// Balanced schedule for an attention launch: kSchedPosMajor when the problem is
// small, else kSchedClaim with the per-head counters `claim` (BH int32).
XcdSchedule make_balanced_schedule(int64_t BH, int n, int64_t kv_bytes_per_head, int32_t* claim);

// Slot (head * n + position) of workgroup b under kSchedStatic, or -1 for a
// padding slot.
__device__ __forceinline__ int64_t scheduled_slot(const XcdSchedule& s, int64_t b) {
    const int64_t x = b % 8, m = b / 8;
    const int64_t unit = x + 8 * (m / s.cap);
    const int64_t head = unit / s.parts;
    const int part = (int)(unit % s.parts);
    const int64_t pos = part + (int64_t)s.parts * (m % s.cap);
    if (pos >= s.n) return -1;
    return head * s.n + pos;
}

// Work item of workgroup b (through a per-head order), or -1 for a workgroup
// with nothing to do. Every thread of the workgroup must call it (kSchedClaim
// broadcasts the claimed position through LDS).
__device__ __forceinline__ int64_t scheduled_item(const XcdSchedule& s, const int32_t* order,
                                                  int64_t b) {
    if (s.mode == kSchedPosMajor) {
        const int64_t pos = b / s.bh, head = b % s.bh;
        return pos < s.n ? order[head * s.n + pos] : -1;
    }
    if (s.mode == kSchedClaim) {
        __shared__ int claimed;
        const int64_t m = b / 8;
        const int64_t head = (b % 8 + 8 * (m / s.cap)) / s.parts;
        if (threadIdx.x == 0) claimed = atomicAdd(s.claim + head, 1);
        __syncthreads();
        const int64_t pos = claimed;
        return pos < s.n ? order[head * s.n + pos] : -1;
    }
    const int64_t slot = scheduled_slot(s, b);
    return slot < 0 ? -1 : order[slot];
}

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, int64_t BH, int S, int D,
                           const int32_t* kv_count, const int32_t* kv_idx, const int32_t* order,
                           const XcdSchedule& sched,
                           float softmax_scale, void* o, bool o_fp32, float* lse,
                           hipStream_t stream);

// Paired forward (attn_fwd_pair_kernel): pairs of query blocks (i, i + F), F =
// blocks per frame; pair_count(n, F) pairs per head (n % F == 0).
int pair_count(int n, int F);
hipError_t launch_pair_counts(const int32_t* kv_count, int64_t BH, int n, int F, int32_t* pc,
                              hipStream_t stream);
hipError_t launch_attn_fwd_pairs(const void* q, const void* k, const void* v, int64_t BH, int S,
                                 int D, int F, const int32_t* kv_count, const int32_t* kv_idx,
                                 const int32_t* order, const XcdSchedule& sched,
                                 float softmax_scale, void* o, bool o_fp32, float* lse,
                                 hipStream_t stream);

hipError_t launch_bwd_delta(const void* o, bool o_fp32, const void* d_o, int64_t rows, int D,
                            float* delta, hipStream_t stream);
hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* d_o,
                           const float* lse, const float* delta, int64_t BH, int S, int D,
                           const int32_t* q_count, const int32_t* q_idx, const int32_t* order,
                           const XcdSchedule& sched, float softmax_scale, void* dk, void* dv,
                           hipStream_t stream);
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* d_o,
                         const float* lse, const float* delta, int64_t BH, int S, int D,
                         const int32_t* kv_count, const int32_t* kv_idx, const int32_t* order,
                         const XcdSchedule& sched, float softmax_scale, void* dq,
                         hipStream_t stream);

// Mask-fidelity diagnostic (fidelity.hip): dense block masses from Q, K and the
// dense LSE; per-row recall of block lists and of the best blocks at equal count.
hipError_t launch_block_mass(const void* q, const void* k, const float* lse, int64_t BH, int S,
                             int D, float softmax_scale, float* mass, hipStream_t stream);
// Rows with a malformed list (see nabla_check_lists) counted into *bad (zeroed first).
hipError_t launch_check_lists(const int32_t* count, const int32_t* idx, int64_t rows, int n,
                              int32_t* bad, hipStream_t stream);
hipError_t launch_mask_recall(const float* mass, int64_t BH, int n, const int32_t* kv_count,
                              const int32_t* kv_idx, float* recall, float* best,
                              hipStream_t stream);

// Library-held scratch of the allocation-free forward (static_scratch.hip): the
// device address of this GPU's copy (the device of `stream`, or the current one
// for the null stream), looked up once per device.
constexpr size_t kStaticScratchBytes = NABLA_STATIC_SCRATCH_BYTES;
hipError_t static_scratch_ptr(hipStream_t stream, void** out);

// Token reordering (block order <-> raster order) of runs of P tokens; see reorder.hip.
hipError_t launch_reorder(const void* src, void* dst, uint32_t runs, uint32_t cpr, uint32_t P,
                          uint32_t tW, bool inverse, hipStream_t stream);

}  // namespace nabla

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

hipError_t launch_pool(const void* q, const void* k, float* qa, float* ka, int64_t nblocks, int D,
                       hipStream_t stream);
hipError_t launch_logits(const float* qa, const float* ka, float* logits, int64_t BH, int n, int D,
                         float scale, hipStream_t stream);
// Row selectors of launch_select. bound: kSelCdf -> floor(thr * 2^40) (fixed-point
// mass); kSelTopk -> k - 1 (a count); kSelSta -> unused (logits may be null).
enum { kSelCdf = 0, kSelTopk = 1, kSelSta = 2 };
hipError_t launch_select(int mode, const float* logits, int64_t BH, int n, int keep_all,
                         uint64_t bound, const StaParams& sta, int32_t* kv_count, int32_t* kv_idx,
                         uint8_t* dense_mask, uint32_t* bits, int words_per_row,
                         hipStream_t stream);
hipError_t launch_transpose(const uint32_t* bits, int64_t BH, int n, int words_per_row,
                            int32_t* q_count, int32_t* q_idx, hipStream_t stream);

// Per-head longest-first order over `items` items per head whose counts lie in
// [0, maxc] (maxc <= NABLA_MAX_BLOCKS; others are clamped): order[h*items + p] =
// item id (h*items + i) of head h's p-th item, counts descending (ties in any order).
hipError_t launch_lpt_order(const int32_t* counts, int64_t BH, int items, int maxc,
                            int32_t* order, hipStream_t stream);

// XCD-aware launch geometry (see schedule.hip): heads are split into `parts`
// interleaved shares so that `units` = BH * parts is a multiple of the 8 XCDs;
// workgroup b runs on XCD b % 8 and serves unit x + 8 * (m / cap), position
// m % cap, with x = b % 8, m = b / 8.
struct XcdSchedule {
    int parts;
    int64_t units;
    int cap;
    int n;
    int64_t grid;
};
XcdSchedule make_schedule(int64_t BH, int n);

// Slot (head * n + position) of workgroup b, or -1 for a padding slot.
__device__ __forceinline__ int64_t scheduled_slot(const XcdSchedule& s, int64_t b) {
    const int64_t x = b % 8, m = b / 8;
    const int64_t unit = x + 8 * (m / s.cap);
    const int64_t head = unit / s.parts;
    const int part = (int)(unit % s.parts);
    const int64_t pos = part + (int64_t)s.parts * (m % s.cap);
    if (pos >= s.n) return -1;
    return head * s.n + pos;
}

// Work item of workgroup b (through a per-head order), or -1 for a padding slot.
__device__ __forceinline__ int64_t scheduled_item(const XcdSchedule& s, const int32_t* order,
                                                  int64_t b) {
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
hipError_t launch_mask_recall(const float* mass, int64_t BH, int n, const int32_t* kv_count,
                              const int32_t* kv_idx, float* recall, float* best,
                              hipStream_t stream);

// Token reordering (block order <-> raster order) of runs of P tokens; see reorder.hip.
hipError_t launch_reorder(const void* src, void* dst, uint32_t runs, uint32_t cpr, uint32_t P,
                          uint32_t tW, bool inverse, hipStream_t stream);

}  // namespace nabla

// nabla_api.cpp -- the extern "C" entry points declared in include/nabla.h.
// Validate, carve the caller's workspace, enqueue the kernels on the caller's
// stream. No allocation, no synchronisation, no state.

#include <hip/hip_runtime.h>
#include <math.h>

#include "kernels.h"
#include "validate.h"

using namespace nabla;

namespace {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline char* ws_at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

#define NABLA_LAUNCH(expr)                          \
    do {                                            \
        if ((expr) != hipSuccess) return NABLA_ERR_HIP; \
    } while (0)

// Bound on |L' - L| per unit of |Q_a[i]|_2 |K_a[j]|_2 for the fp32 reduced logit
// L' = fl(fl(sum_d fl(qa_d) fl(ka_d)) * fl(1/sqrt(D))) against the exact
// L = (1/sqrt(D)) sum_d qa_d ka_d: the D-term fp32 dot product contributes
// gamma_(D+2) = (D+2)u/(1-(D+2)u) of sum_d |qa_d ka_d| <= |qa| |ka| (products
// possibly rounded too), the fp32 operands 2u, the fp32 scale and the final
// multiply 2u each -- (D + 8) u in all, u = 2^-24, with a 1% margin.
float logit_error_unit(int D, float scale) {
    const double u = 1.0 / 16777216.0;
    return (float)((D + 8) * u * 1.01 * (double)scale * (1.0 + 1e-6));
}

StaParams sta_params(const nabla_sta_t* sta) {
    StaParams sp{};
    if (sta) {
        sp.on = 1;
        sp.tT = sta->T;
        sp.tH = sta->Hs / sta->P;
        sp.tW = sta->Ws / sta->P;
        sp.wt = sta->win_t;
        sp.wh = sta->win_h / sta->P;
        sp.ww = sta->win_w / sta->P;
    }
    return sp;
}

// Pool, reduced logits, one selector (kSelCdf or kSelTopk), compaction and the
// optional transpose. Arguments other than the selector's are validated here.
nabla_status_t content_mask(int mode, int keep_all, uint64_t bound, const void* q, const void* k,
                            int32_t B, int32_t H, int32_t S, int32_t D, int32_t N,
                            const nabla_sta_t* sta, int32_t* kv_count, int32_t* kv_idx,
                            int32_t* q_count, int32_t* q_idx, uint8_t* dense_mask, void* workspace,
                            size_t workspace_bytes, void* stream) {
    Shape s;
    nabla_status_t st = check_shape(B, H, S, D, N, &s);
    if (st != NABLA_OK) return st;
    if (!q || !k || !kv_count || !kv_idx) return NABLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k)) return NABLA_ERR_INVALID_ARG;
    if ((q_count == nullptr) != (q_idx == nullptr)) return NABLA_ERR_INVALID_ARG;
    st = check_sta(sta, s);
    if (st != NABLA_OK) return st;
    const MaskWorkspace w = mask_workspace(s);
    if (!workspace || workspace_bytes < w.total || !aligned16(workspace)) return NABLA_ERR_WORKSPACE;

    PoolOut po;
    po.qa = reinterpret_cast<float*>(ws_at(workspace, w.qa));
    po.ka = reinterpret_cast<float*>(ws_at(workspace, w.ka));
    po.qa64 = reinterpret_cast<double*>(ws_at(workspace, w.qa64));
    po.ka64 = reinterpret_cast<double*>(ws_at(workspace, w.ka64));
    po.qnorm = reinterpret_cast<float*>(ws_at(workspace, w.qnorm));
    po.knorm = reinterpret_cast<float*>(ws_at(workspace, w.knorm));
    po.kmax = reinterpret_cast<float*>(ws_at(workspace, w.kmax));
    float* logits = reinterpret_cast<float*>(ws_at(workspace, w.logits));
    uint32_t* bits = q_idx ? reinterpret_cast<uint32_t*>(ws_at(workspace, w.bits)) : nullptr;
    hipStream_t hs = as_stream(stream);

    const float scale = 1.0f / sqrtf((float)s.D);
    NABLA_LAUNCH(launch_pool(q, k, po, s.BH, (int)s.n, (int)s.D, hs));
    // Reduced logits and selection, w.logit_heads heads at a time (the map
    // region holds that many heads; one chunk unless B*H*n*n*4 bytes exceed
    // kMaxLogitMapBytes). Every per-row and per-head array is offset to the
    // chunk's first head; the kernels index them from there.
    const int64_t n = s.n, dim = s.D;
    for (int64_t h0 = 0; h0 < s.BH; h0 += w.logit_heads) {
        const int64_t nh = s.BH - h0 < w.logit_heads ? s.BH - h0 : w.logit_heads;
        const int64_t r0 = h0 * n;  // first row of the chunk
        NABLA_LAUNCH(launch_logits(po.qa + r0 * dim, po.ka + r0 * dim, logits, nh, (int)n, (int)dim, scale, hs));
        SelectArgs a{};
        a.logits = logits;
        a.rows = nh * n;
        a.n = (int)n;
        a.keep_all = keep_all;
        a.bound = bound;
        a.sta = sta_params(sta);
        a.qa64 = po.qa64 + r0 * dim;
        a.ka64 = po.ka64 + r0 * dim;
        a.qnorm = po.qnorm + r0;
        a.kmax = po.kmax + h0;
        a.scale64 = 1.0 / sqrt((double)s.D);
        a.err_unit = logit_error_unit((int)s.D, scale);
        a.kv_count = kv_count + r0;
        a.kv_idx = kv_idx + r0 * n;
        a.dense_mask = dense_mask ? dense_mask + r0 * n : nullptr;
        a.bits = bits ? bits + r0 * w.words_per_row : nullptr;
        a.words_per_row = w.words_per_row;
        NABLA_LAUNCH(launch_select(mode, a, (int)s.D, hs));
    }
    if (q_idx)
        NABLA_LAUNCH(launch_transpose(bits, s.BH, (int)s.n, w.words_per_row, q_count, q_idx, hs));
    return NABLA_OK;
}

}  // namespace

extern "C" {

const char* nabla_status_string(nabla_status_t status) {
    switch (status) {
        case NABLA_OK: return "NABLA_OK";
        case NABLA_ERR_INVALID_ARG: return "NABLA_ERR_INVALID_ARG";
        case NABLA_ERR_UNSUPPORTED: return "NABLA_ERR_UNSUPPORTED";
        case NABLA_ERR_WORKSPACE: return "NABLA_ERR_WORKSPACE";
        case NABLA_ERR_HIP: return "NABLA_ERR_HIP";
    }
    return "NABLA_ERR_UNKNOWN";
}

size_t nabla_workspace_size(int32_t op, int32_t B, int32_t H, int32_t S, int32_t D, int32_t N) {
    Shape s;
    if (op == NABLA_OP_STA_MASK) D = kStaShapeD;  // the STA mask does not depend on D
    if (check_shape(B, H, S, D, N, &s) != NABLA_OK) return 0;
    switch (op) {
        case NABLA_OP_STA_MASK: return sta_workspace(s).total;
        case NABLA_OP_MASK: return mask_workspace(s).total;
        case NABLA_OP_FWD: return fwd_workspace(s).total;
        case NABLA_OP_BWD: return bwd_workspace(s).total;
    }
    return 0;
}

nabla_status_t nabla_build_mask(const void* q, const void* k, int32_t B, int32_t H, int32_t S,
                                int32_t D, int32_t N, float thr, const nabla_sta_t* sta,
                                int32_t* kv_count, int32_t* kv_idx, int32_t* q_count,
                                int32_t* q_idx, uint8_t* dense_mask, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (!(thr >= 0.0f) || isinf(thr)) return NABLA_ERR_INVALID_ARG;  // rejects NaN too
    return content_mask(kSelCdf, thr >= 1.0f, threshold_fixed(thr), q, k, B, H, S, D, N, sta,
                        kv_count, kv_idx, q_count, q_idx, dense_mask, workspace, workspace_bytes,
                        stream);
}

nabla_status_t nabla_build_topk_mask(const void* q, const void* k, int32_t B, int32_t H, int32_t S,
                                     int32_t D, int32_t N, int32_t topk, const nabla_sta_t* sta,
                                     int32_t* kv_count, int32_t* kv_idx, int32_t* q_count,
                                     int32_t* q_idx, uint8_t* dense_mask, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    if (topk < 1) return NABLA_ERR_INVALID_ARG;
    const int keep_all = N > 0 && S / N <= topk;
    return content_mask(kSelTopk, keep_all, (uint64_t)(topk - 1), q, k, B, H, S, D, N, sta,
                        kv_count, kv_idx, q_count, q_idx, dense_mask, workspace, workspace_bytes,
                        stream);
}

nabla_status_t nabla_build_sta_mask(int32_t B, int32_t H, int32_t S, int32_t N,
                                    const nabla_sta_t* sta, int32_t* kv_count, int32_t* kv_idx,
                                    int32_t* q_count, int32_t* q_idx, uint8_t* dense_mask,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    Shape s;
    nabla_status_t st = check_shape(B, H, S, kStaShapeD, N, &s);
    if (st != NABLA_OK) return st;
    if (!sta || !kv_count || !kv_idx) return NABLA_ERR_INVALID_ARG;
    if ((q_count == nullptr) != (q_idx == nullptr)) return NABLA_ERR_INVALID_ARG;
    st = check_sta(sta, s);
    if (st != NABLA_OK) return st;
    const StaWorkspace w = sta_workspace(s);
    if (!workspace || workspace_bytes < w.total || !aligned16(workspace)) return NABLA_ERR_WORKSPACE;

    uint32_t* bits = q_idx ? reinterpret_cast<uint32_t*>(ws_at(workspace, w.bits)) : nullptr;
    hipStream_t hs = as_stream(stream);
    SelectArgs a{};
    a.rows = s.BH * s.n;
    a.n = (int)s.n;
    a.sta = sta_params(sta);
    a.kv_count = kv_count;
    a.kv_idx = kv_idx;
    a.dense_mask = dense_mask;
    a.bits = bits;
    a.words_per_row = w.words_per_row;
    NABLA_LAUNCH(launch_select(kSelSta, a, (int)s.D, hs));
    if (q_idx)
        NABLA_LAUNCH(launch_transpose(bits, s.BH, (int)s.n, w.words_per_row, q_count, q_idx, hs));
    return NABLA_OK;
}

}  // extern "C"

namespace {

// The forward after its workspace has been provided (caller's or library-held).
nabla_status_t sparse_attn_fwd(const Shape& s, const void* q, const void* k, const void* v,
                               const int32_t* kv_count, const int32_t* kv_idx,
                               float softmax_scale, int32_t frame_blocks, void* o,
                               int32_t o_dtype, float* lse, void* workspace, hipStream_t hs) {
    const FwdWorkspace w = fwd_workspace(s);
    int32_t* order = reinterpret_cast<int32_t*>(ws_at(workspace, w.order));
    int32_t* claim = reinterpret_cast<int32_t*>(ws_at(workspace, w.claim));
    const bool o_fp32 = o_dtype == NABLA_DTYPE_FP32;
    const int n = (int)s.n;
    const int64_t kv_bytes = 2 * s.S * s.D * (int64_t)sizeof(uint16_t);  // one head's K and V
    if (frame_blocks > 0 && n / frame_blocks >= 2) {
        // Pairs of query blocks (i, i + F): the same tile in consecutive frames.
        const int np = pair_count(n, frame_blocks);
        int32_t* pc = reinterpret_cast<int32_t*>(ws_at(workspace, w.counts));
        const XcdSchedule sched = make_balanced_schedule(s.BH, np, kv_bytes, claim);
        NABLA_LAUNCH(launch_pair_counts(kv_count, s.BH, n, frame_blocks, pc, hs));
        NABLA_LAUNCH(launch_lpt_order(pc, s.BH, np, n, order, claim, hs));
        NABLA_LAUNCH(launch_attn_fwd_pairs(q, k, v, s.BH, (int)s.S, (int)s.D, frame_blocks, kv_count,
                                           kv_idx, order, sched, softmax_scale, o, o_fp32, lse, hs));
        return NABLA_OK;
    }
    const XcdSchedule sched = make_balanced_schedule(s.BH, n, kv_bytes, claim);
    NABLA_LAUNCH(launch_lpt_order(kv_count, s.BH, n, n, order, claim, hs));
    NABLA_LAUNCH(launch_attn_fwd(q, k, v, s.BH, (int)s.S, (int)s.D, kv_count, kv_idx, order, sched,
                                 softmax_scale, o, o_fp32, lse, hs));
    return NABLA_OK;
}

// Argument checks shared by both forward entry points.
nabla_status_t check_fwd_args(int32_t B, int32_t H, int32_t S, int32_t D, int32_t N, const void* q,
                              const void* k, const void* v, const int32_t* kv_count,
                              const int32_t* kv_idx, float softmax_scale, int32_t frame_blocks,
                              const void* o, int32_t o_dtype, Shape* s) {
    nabla_status_t st = check_shape(B, H, S, D, N, s);
    if (st != NABLA_OK) return st;
    if (!q || !k || !v || !o || !kv_count || !kv_idx) return NABLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return NABLA_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || isinf(softmax_scale)) return NABLA_ERR_INVALID_ARG;
    if (o_dtype != NABLA_DTYPE_BF16 && o_dtype != NABLA_DTYPE_FP32) return NABLA_ERR_INVALID_ARG;
    if (frame_blocks < 0 || (frame_blocks > 0 && s->n % frame_blocks != 0)) return NABLA_ERR_INVALID_ARG;
    return NABLA_OK;
}

}  // namespace

extern "C" {

nabla_status_t nabla_sparse_attn_fwd(const void* q, const void* k, const void* v, int32_t B,
                                     int32_t H, int32_t S, int32_t D, int32_t N,
                                     const int32_t* kv_count, const int32_t* kv_idx,
                                     float softmax_scale, int32_t frame_blocks, void* o,
                                     int32_t o_dtype, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    Shape s;
    nabla_status_t st = check_fwd_args(B, H, S, D, N, q, k, v, kv_count, kv_idx, softmax_scale,
                                       frame_blocks, o, o_dtype, &s);
    if (st != NABLA_OK) return st;
    const FwdWorkspace w = fwd_workspace(s);
    if (!workspace || workspace_bytes < w.total || !aligned16(workspace)) return NABLA_ERR_WORKSPACE;
    return sparse_attn_fwd(s, q, k, v, kv_count, kv_idx, softmax_scale, frame_blocks, o, o_dtype,
                           lse, workspace, as_stream(stream));
}

nabla_status_t nabla_sparse_attn_fwd_static(const void* q, const void* k, const void* v, int32_t B,
                                            int32_t H, int32_t S, int32_t D, int32_t N,
                                            const int32_t* kv_count, const int32_t* kv_idx,
                                            float softmax_scale, int32_t frame_blocks, void* o,
                                            int32_t o_dtype, float* lse, void* stream) {
    Shape s;
    nabla_status_t st = check_fwd_args(B, H, S, D, N, q, k, v, kv_count, kv_idx, softmax_scale,
                                       frame_blocks, o, o_dtype, &s);
    if (st != NABLA_OK) return st;
    if (fwd_workspace(s).total > kStaticScratchBytes) return NABLA_ERR_WORKSPACE;
    hipStream_t hs = as_stream(stream);
    void* scratch_ptr = nullptr;
    if (static_scratch_ptr(hs, &scratch_ptr) != hipSuccess) return NABLA_ERR_HIP;
    return sparse_attn_fwd(s, q, k, v, kv_count, kv_idx, softmax_scale, frame_blocks, o, o_dtype,
                           lse, scratch_ptr, hs);
}

nabla_status_t nabla_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                     int32_t o_dtype, const void* d_o, const float* lse, int32_t B, int32_t H,
                                     int32_t S, int32_t D, int32_t N, const int32_t* kv_count,
                                     const int32_t* kv_idx, const int32_t* q_count,
                                     const int32_t* q_idx, float softmax_scale, void* dq,
                                     void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    Shape s;
    nabla_status_t st = check_shape(B, H, S, D, N, &s);
    if (st != NABLA_OK) return st;
    if (!q || !k || !v || !o || !d_o || !lse || !kv_count || !kv_idx || !q_count || !q_idx ||
        !dq || !dk || !dv)
        return NABLA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, o, d_o, dq, dk, dv};
    for (const void* p : ptrs)
        if (!aligned16(p)) return NABLA_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || isinf(softmax_scale)) return NABLA_ERR_INVALID_ARG;
    if (o_dtype != NABLA_DTYPE_BF16 && o_dtype != NABLA_DTYPE_FP32) return NABLA_ERR_INVALID_ARG;
    const BwdWorkspace w = bwd_workspace(s);
    if (!workspace || workspace_bytes < w.total || !aligned16(workspace)) return NABLA_ERR_WORKSPACE;

    float* delta = reinterpret_cast<float*>(ws_at(workspace, w.delta));
    int32_t* order_q = reinterpret_cast<int32_t*>(ws_at(workspace, w.order_q));
    int32_t* order_kv = reinterpret_cast<int32_t*>(ws_at(workspace, w.order_kv));
    int32_t* claim = reinterpret_cast<int32_t*>(ws_at(workspace, w.claim));
    hipStream_t hs = as_stream(stream);
    NABLA_LAUNCH(launch_bwd_delta(o, o_dtype == NABLA_DTYPE_FP32, d_o, s.BH * s.S, (int)s.D, delta, hs));
    // Q, K, V and dO of one head are read by each backward kernel.
    const int64_t head_bytes = 4 * s.S * s.D * (int64_t)sizeof(uint16_t);
    const XcdSchedule sched = make_balanced_schedule(s.BH, (int)s.n, head_bytes, claim);
    NABLA_LAUNCH(launch_lpt_order(q_count, s.BH, (int)s.n, (int)s.n, order_kv, claim, hs));
    NABLA_LAUNCH(launch_bwd_dkdv(q, k, v, d_o, lse, delta, s.BH, (int)s.S, (int)s.D, q_count, q_idx,
                                 order_kv, sched, softmax_scale, dk, dv, hs));
    NABLA_LAUNCH(launch_lpt_order(kv_count, s.BH, (int)s.n, (int)s.n, order_q, claim, hs));
    NABLA_LAUNCH(launch_bwd_dq(q, k, v, d_o, lse, delta, s.BH, (int)s.S, (int)s.D, kv_count, kv_idx,
                               order_q, sched, softmax_scale, dq, hs));
    return NABLA_OK;
}

nabla_status_t nabla_block_mass(const void* q, const void* k, const float* lse, int32_t B, int32_t H,
                                int32_t S, int32_t D, int32_t N, float softmax_scale, float* mass,
                                void* stream) {
    Shape s;
    const nabla_status_t st = check_shape(B, H, S, D, N, &s);
    if (st != NABLA_OK) return st;
    if (!q || !k || !lse || !mass) return NABLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k)) return NABLA_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || isinf(softmax_scale)) return NABLA_ERR_INVALID_ARG;
    NABLA_LAUNCH(launch_block_mass(q, k, lse, s.BH, (int)s.S, (int)s.D, softmax_scale, mass,
                                   as_stream(stream)));
    return NABLA_OK;
}

nabla_status_t nabla_mask_recall(const float* mass, int32_t B, int32_t H, int32_t S, int32_t N,
                                 const int32_t* kv_count, const int32_t* kv_idx, float* recall,
                                 float* best_recall, void* stream) {
    Shape s;
    const nabla_status_t st = check_shape(B, H, S, kStaShapeD, N, &s);
    if (st != NABLA_OK) return st;
    if (!mass || !kv_count || !kv_idx || !recall || !best_recall) return NABLA_ERR_INVALID_ARG;
    NABLA_LAUNCH(launch_mask_recall(mass, s.BH, (int)s.n, kv_count, kv_idx, recall, best_recall,
                                    as_stream(stream)));
    return NABLA_OK;
}

nabla_status_t nabla_check_lists(const int32_t* count, const int32_t* idx, int32_t B, int32_t H,
                                 int32_t S, int32_t N, int32_t* bad_rows, void* stream) {
    Shape s;
    const nabla_status_t st = check_shape(B, H, S, kStaShapeD, N, &s);
    if (st != NABLA_OK) return st;
    if (!count || !idx || !bad_rows) return NABLA_ERR_INVALID_ARG;
    NABLA_LAUNCH(launch_check_lists(count, idx, s.BH * s.n, (int)s.n, bad_rows, as_stream(stream)));
    return NABLA_OK;
}

nabla_status_t nabla_reorder_tokens(const void* src, void* dst, int32_t B, int32_t T, int32_t Hs,
                                    int32_t Ws, int32_t P, int64_t row_bytes, int32_t inverse,
                                    void* stream) {
    ReorderGeom g;
    const nabla_status_t st = check_reorder(src, dst, B, T, Hs, Ws, P, row_bytes, inverse, &g);
    if (st != NABLA_OK || g.empty) return st;
    NABLA_LAUNCH(launch_reorder(src, dst, g.runs, g.cpr, g.P, g.tW, inverse != 0, as_stream(stream)));
    return NABLA_OK;
}

}  // extern "C"

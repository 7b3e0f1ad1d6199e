// validate.cpp -- argument checks and workspace layout (no HIP dependency).
#include "validate.h"

#include <math.h>

namespace nabla {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

nabla_status_t check_shape(int32_t B, int32_t H, int32_t S, int32_t D, int32_t N, Shape* out) {
    if (B <= 0 || H <= 0 || S <= 0 || D <= 0 || N <= 0) return NABLA_ERR_INVALID_ARG;
    if (S % N != 0) return NABLA_ERR_INVALID_ARG;
    if (N != 64) return NABLA_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return NABLA_ERR_UNSUPPORTED;
    const int64_t n = S / N;
    if (n > NABLA_MAX_BLOCKS) return NABLA_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)B * H;
    // Grid dimension limits of the kernels (one workgroup per block or row).
    if (BH * n > (int64_t)0x7fffffff) return NABLA_ERR_UNSUPPORTED;
    if (out) *out = Shape{B, H, S, D, N, n, BH};
    return NABLA_OK;
}

nabla_status_t check_sta(const nabla_sta_t* sta, const Shape& s) {
    if (!sta) return NABLA_OK;
    if (sta->T <= 0 || sta->Hs <= 0 || sta->Ws <= 0 || sta->P <= 0) return NABLA_ERR_INVALID_ARG;
    if ((int64_t)sta->P * sta->P != s.N) return NABLA_ERR_INVALID_ARG;
    if (sta->Hs % sta->P || sta->Ws % sta->P) return NABLA_ERR_INVALID_ARG;
    if ((int64_t)sta->T * sta->Hs * sta->Ws != s.S) return NABLA_ERR_INVALID_ARG;
    if (sta->win_t < 1 || sta->win_h < sta->P || sta->win_w < sta->P) return NABLA_ERR_INVALID_ARG;
    if (sta->win_h % sta->P || sta->win_w % sta->P) return NABLA_ERR_INVALID_ARG;
    return NABLA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

MaskWorkspace mask_workspace(const Shape& s) {
    MaskWorkspace w;
    const size_t pooled = (size_t)s.BH * s.n * s.D * sizeof(float);
    w.words_per_row = (int)((s.n + 31) / 32);
    const size_t norms = (size_t)s.BH * s.n * sizeof(float);
    w.qa = 0;
    w.ka = w.qa + align256(pooled);
    w.qa64 = w.ka + align256(pooled);
    w.ka64 = w.qa64 + align256(2 * pooled);
    w.qnorm = w.ka64 + align256(2 * pooled);
    w.knorm = w.qnorm + align256(norms);
    w.kmax = w.knorm + align256(norms);
    w.logits = w.kmax + align256((size_t)s.BH * sizeof(float));
    const size_t head_map = (size_t)s.n * s.n * sizeof(float);
    int64_t heads = (int64_t)(kMaxLogitMapBytes / head_map);
    w.logit_heads = heads < 1 ? 1 : (heads > s.BH ? s.BH : heads);
    w.bits = w.logits + align256((size_t)w.logit_heads * head_map);
    w.total = w.bits + align256((size_t)s.BH * s.n * w.words_per_row * sizeof(uint32_t));
    return w;
}

StaWorkspace sta_workspace(const Shape& s) {
    StaWorkspace w;
    w.words_per_row = (int)((s.n + 31) / 32);
    w.bits = 0;
    w.total = align256((size_t)s.BH * s.n * w.words_per_row * sizeof(uint32_t));
    return w;
}

FwdWorkspace fwd_workspace(const Shape& s) {
    FwdWorkspace w;
    w.order = 0;
    w.counts = align256((size_t)s.BH * s.n * sizeof(int32_t));
    w.claim = w.counts + align256((size_t)s.BH * s.n * sizeof(int32_t));
    w.total = w.claim + align256((size_t)s.BH * sizeof(int32_t));
    return w;
}

BwdWorkspace bwd_workspace(const Shape& s) {
    BwdWorkspace w;
    w.delta = 0;
    w.order_q = align256((size_t)s.BH * s.S * sizeof(float));
    w.order_kv = w.order_q + align256((size_t)s.BH * s.n * sizeof(int32_t));
    w.claim = w.order_kv + align256((size_t)s.BH * s.n * sizeof(int32_t));
    w.total = w.claim + align256((size_t)s.BH * sizeof(int32_t));
    return w;
}

nabla_status_t check_reorder(const void* src, void* dst, int32_t B, int32_t T, int32_t Hs,
                             int32_t Ws, int32_t P, int64_t row_bytes, int32_t inverse,
                             ReorderGeom* out) {
    if (B < 0 || T < 0 || Hs < 0 || Ws < 0 || P <= 0 || row_bytes <= 0) return NABLA_ERR_INVALID_ARG;
    if (row_bytes % 16 != 0) return NABLA_ERR_INVALID_ARG;
    if (Hs % P != 0 || Ws % P != 0) return NABLA_ERR_INVALID_ARG;
    if (inverse != 0 && inverse != 1) return NABLA_ERR_INVALID_ARG;
    const int64_t tokens = (int64_t)B * T * Hs * Ws;
    ReorderGeom g{0, 0, (uint32_t)P, 0, tokens == 0};
    if (g.empty) {
        if (out) *out = g;
        return NABLA_OK;
    }
    if (!src || !dst || !aligned16(src) || !aligned16(dst)) return NABLA_ERR_INVALID_ARG;
    // Index arithmetic of the kernel is 32-bit in runs and in chunks per run.
    if (row_bytes > ((int64_t)1 << 36)) return NABLA_ERR_UNSUPPORTED;
    const int64_t runs = tokens / P;
    const int64_t cpr = (int64_t)P * (row_bytes / 16);
    if (runs > 0x7fffffff || cpr > 0x7fffffff) return NABLA_ERR_UNSUPPORTED;
    // At most 2^40 chunks (16 TiB): far beyond any device, and no overflow below.
    if ((uint64_t)runs * (uint64_t)cpr > ((uint64_t)1 << 40)) return NABLA_ERR_UNSUPPORTED;
    const uint64_t bytes = (uint64_t)runs * (uint64_t)cpr * 16u;
    const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
    if (s < d + bytes && d < s + bytes) return NABLA_ERR_INVALID_ARG;  // overlap
    g.runs = (uint32_t)runs;
    g.cpr = (uint32_t)cpr;
    g.tW = (uint32_t)(Ws / P);
    if (out) *out = g;
    return NABLA_OK;
}

uint64_t threshold_fixed(float thr) {
    const double x = (double)thr * 1099511627776.0;  // 2^40
    return (uint64_t)floor(x);
}

}  // namespace nabla

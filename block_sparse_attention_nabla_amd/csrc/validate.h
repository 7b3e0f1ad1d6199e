// validate.h -- argument checks and workspace layout of the NABLA C ABI.
// Plain C++ with no HIP dependency: every check runs before any GPU work.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/nabla.h"

namespace nabla {

struct Shape {
    int64_t B, H, S, D, N, n, BH;
};

// Region offsets inside a caller-provided workspace (all 256-byte aligned).
// The reduced-logit map is held for `logit_heads` heads at a time: as many as
// fit kMaxLogitMapBytes (at least one), so the workspace grows with one head's
// n x n map instead of all B*H of them; the mask call walks the heads in
// chunks of that many.
constexpr size_t kMaxLogitMapBytes = (size_t)256 << 20;
struct MaskWorkspace {
    size_t qa, ka, qa64, ka64, qnorm, knorm, kmax, logits, bits, total;
    int64_t logit_heads;
    int words_per_row;
};
struct StaWorkspace {
    size_t bits, total;
    int words_per_row;
};
struct FwdWorkspace {
    size_t order, counts, claim, total;
};
struct BwdWorkspace {
    size_t delta, order_q, order_kv, claim, total;
};

nabla_status_t check_shape(int32_t B, int32_t H, int32_t S, int32_t D, int32_t N, Shape* out);
nabla_status_t check_sta(const nabla_sta_t* sta, const Shape& s);
bool aligned16(const void* p);

MaskWorkspace mask_workspace(const Shape& s);
StaWorkspace sta_workspace(const Shape& s);
FwdWorkspace fwd_workspace(const Shape& s);

// Shape checks of calls that have no head dimension (the STA-only mask, the
// recall of block lists) use this one.
constexpr int32_t kStaShapeD = 64;
BwdWorkspace bwd_workspace(const Shape& s);

// Token reordering geometry: `runs` moved units of P tokens, `cpr` 16-byte
// chunks per run, tW patches per frame row. empty = nothing to move.
struct ReorderGeom {
    uint32_t runs, cpr, P, tW;
    bool empty;
};
nabla_status_t check_reorder(const void* src, void* dst, int32_t B, int32_t T, int32_t Hs,
                             int32_t Ws, int32_t P, int64_t row_bytes, int32_t inverse,
                             ReorderGeom* out);

// Fixed-point threshold used by the selection kernel: floor(thr * 2^40).
uint64_t threshold_fixed(float thr);

}  // namespace nabla

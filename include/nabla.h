/*
 * nabla.h -- C ABI of the MI355X (gfx950) NABLA block-sparse attention library.
 *
 * NABLA ("Neighborhood Adaptive Block-Level Attention", arXiv 2507.13546) makes a
 * per-head block mask from average-pooled queries and keys (Algorithm 1,
 * section 3.1.2), optionally ORs it with a sliding-tile (STA) mask (section
 * 3.1.3), and runs attention only on the kept N x N blocks (eq. (4), section 2.2).
 *
 * Conventions shared by every entry point:
 *  - Tensors Q, K, V, O, dO, dQ, dK, dV are device pointers to contiguous bf16
 *    (bfloat16, 2 bytes) arrays of shape [B, H, S, D] (row-major; D fastest).
 *    Tokens must already be in block order: block i of a head is tokens
 *    [i*N, (i+1)*N) (the paper's token reordering, section 3.1.1, Figure 3).
 *  - n = S / N query (and key) blocks per head. Block lists are int32:
 *      kv_count [B, H, n]      number of kept key blocks of query block i,
 *      kv_idx   [B, H, n, n]   entries [0, kv_count) = kept key blocks, ascending;
 *                              later entries are unspecified (not written),
 *      q_count  [B, H, n]      number of query blocks that keep key block j,
 *      q_idx    [B, H, n, n]   entries [0, q_count) = those query blocks, ascending.
 *  - Supported now: N == 64, D in {64, 128}, S % N == 0, n <= NABLA_MAX_BLOCKS.
 *  - Ownership: the caller allocates every buffer, including the workspace
 *    (size from nabla_workspace_size). The library never allocates, frees or
 *    synchronises; it enqueues work on `stream` (a hipStream_t; NULL = the
 *    default stream) and returns. It keeps no state between calls; concurrent
 *    calls are safe when they use distinct output and workspace buffers.
 *  - Errors: every argument is validated before anything is enqueued; a
 *    non-OK status means nothing was launched (except NABLA_ERR_HIP, returned
 *    when a launch itself fails). Faults inside kernels surface at the
 *    caller's next synchronisation, as for any HIP kernel.
 */
#ifndef NABLA_H
#define NABLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NABLA_MAX_BLOCKS 8192

/* Symbols of this ABI are the only ones the shared library exports. */
#if defined(__GNUC__) || defined(__clang__)
#define NABLA_API __attribute__((visibility("default")))
#else
#define NABLA_API
#endif

typedef enum {
    NABLA_OK = 0,
    NABLA_ERR_INVALID_ARG = 1, /* null pointer, bad shape, bad threshold, bad STA geometry */
    NABLA_ERR_UNSUPPORTED = 2, /* valid but not implemented: N != 64, D not in {64,128}, n too big */
    NABLA_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than nabla_workspace_size() */
    NABLA_ERR_HIP = 4          /* a HIP launch or query failed */
} nabla_status_t;

/* Sliding-tile window (section 2.2, eq. (4)-(5); STA_mask(T, H, W, W_T, W_H, W_W)
 * of section 3.1.3). The latent grid is T frames of Hs x Ws tokens, tiled by
 * 1 x P x P tiles, so one tile is one block and N == P*P. The window is
 * win_t frames x win_h x win_w tokens (win_h, win_w multiples of P), centred on
 * the query tile -- (w-1)/2 tiles below, w/2 above on each axis -- and clipped
 * at the grid edges. Requires T*Hs*Ws == S, Hs % P == 0, Ws % P == 0, windows >= 1. */
typedef struct {
    int32_t T, Hs, Ws, P;
    int32_t win_t, win_h, win_w;
} nabla_sta_t;

/* Operations for nabla_workspace_size. NABLA_OP_MASK covers nabla_build_mask and
 * nabla_build_topk_mask; NABLA_OP_STA_MASK covers nabla_build_sta_mask (D ignored). */
enum { NABLA_OP_MASK = 0, NABLA_OP_FWD = 1, NABLA_OP_BWD = 2, NABLA_OP_STA_MASK = 3 };

/* Element type of the forward output O. */
enum { NABLA_DTYPE_BF16 = 0, NABLA_DTYPE_FP32 = 1 };

/* Bytes of device workspace the given operation needs (0 for invalid shapes).
 * NABLA_OP_MASK is linear in B*H*n except for the fp32 reduced-logit map,
 * which the mask call keeps for a chunk of heads at a time: as many heads as
 * fit 256 MiB of n x n maps, at least one (n = S/N). */
NABLA_API size_t nabla_workspace_size(int32_t op, int32_t B, int32_t H, int32_t S, int32_t D, int32_t N);

/* Human-readable name of a status code (static storage). */
NABLA_API const char* nabla_status_string(nabla_status_t status);

/*
 * Block mask (Algorithm 1, section 3.1.2, plus the STA union of section 3.1.3).
 * For every head and query block i:
 *   Q_a[i] = mean of the N query rows of block i, K_a[j] likewise (steps 2-5);
 *   p_ij   = softmax_j(Q_a[i] . K_a[j] / sqrt(D))                 (steps 6-7);
 *   keep j iff thr >= 1 or G_ij <= thr, G_ij = sum of p_il over l with
 *   p_il > p_ij -- the sort / cumulative-sum / ">= 1 - thr" binarisation of
 *   steps 8-11 with ties kept together;                            then
 *   keep j also if the STA window of i contains j (when sta != NULL).
 * Block means are summed exactly (fp64); logits, softmax and masses are fp32,
 * and the order of the probabilities next to the cut is resolved with fp64
 * logits, so the kept set follows the exact order of the reduced map (G is
 * within fp32 rounding of its exact value). Results are written as
 * the compact lists above; q_count/q_idx (needed by the backward pass) and
 * dense_mask (uint8 [B, H, n, n], 1 = kept) are optional (NULL = skip).
 * thr must be finite and >= 0. Every row keeps at least its largest entry.
 */
NABLA_API nabla_status_t nabla_build_mask(const void* q, const void* k, int32_t B, int32_t H, int32_t S,
                                int32_t D, int32_t N, float thr, const nabla_sta_t* sta,
                                int32_t* kv_count, int32_t* kv_idx, int32_t* q_count,
                                int32_t* q_idx, uint8_t* dense_mask, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Variant selector: Top-k blocks per row, the fixed-budget rule the CDF
 * selection is compared with (review record of arXiv 2507.13546 on
 * pith.science, referee comment on Appendix C, Theorem 1). Same pooling and
 * reduced softmax as nabla_build_mask; then, for every head and query block i,
 *   keep j iff fewer than topk entries p_il are strictly larger than p_ij
 * (the topk largest blocks; blocks tied at the topk-th value are all kept, so
 * a row keeps at least min(topk, n) blocks), then the STA union if sta != NULL.
 * topk >= 1 (NABLA_ERR_INVALID_ARG otherwise); topk >= n keeps every block.
 * Outputs, workspace (NABLA_OP_MASK) and errors as for nabla_build_mask.
 */
NABLA_API nabla_status_t nabla_build_topk_mask(const void* q, const void* k, int32_t B, int32_t H,
                                               int32_t S, int32_t D, int32_t N, int32_t topk,
                                               const nabla_sta_t* sta, int32_t* kv_count,
                                               int32_t* kv_idx, int32_t* q_count, int32_t* q_idx,
                                               uint8_t* dense_mask, void* workspace,
                                               size_t workspace_bytes, void* stream);

/*
 * Variant selector: the static sliding-tile mask alone (STA, section 2.2,
 * eq. (4)-(5); the STA rows of Table 1): keep j iff the clipped window centred
 * on query tile i contains tile j, for every one of the B*H heads. Needs no Q
 * or K. sta is required (same rules as in nabla_build_mask, with P*P == N and
 * T*Hs*Ws == S). Outputs as for nabla_build_mask; the workspace
 * (NABLA_OP_STA_MASK, only used when q_count/q_idx are requested, but always
 * checked) holds the row bitmasks of the transpose.
 */
NABLA_API nabla_status_t nabla_build_sta_mask(int32_t B, int32_t H, int32_t S, int32_t N,
                                              const nabla_sta_t* sta, int32_t* kv_count,
                                              int32_t* kv_idx, int32_t* q_count, int32_t* q_idx,
                                              uint8_t* dense_mask, void* workspace,
                                              size_t workspace_bytes, void* stream);

/*
 * Block-sparse attention forward (eq. (4) with the kept-block mask): for each
 * token s of query block i,
 *   O_s   = sum_u softmax_u(scale * q_s . k_u) v_u over the keys u of the kept
 *           blocks kv_idx[b, h, i, 0 .. kv_count),
 *   LSE_s = log sum_u exp(scale * q_s . k_u)   (natural log).
 * o: [B, H, S, D] output of type o_dtype (NABLA_DTYPE_BF16 or NABLA_DTYPE_FP32;
 * the arithmetic is the same, only the final store differs). lse: fp32 [B, H, S]
 * output, may be NULL (the backward pass needs it). softmax_scale > 0, finite
 * (the paper uses 1/sqrt(D)). The PV product uses the probabilities rounded to
 * bf16 and divides by the sum of those rounded weights; LSE uses the fp32 sum.
 * Kept-block indices must lie in [0, n) and counts in [0, n]; a row with
 * count 0 yields O = 0 and LSE = -inf. bf16 MFMA, fp32 accumulation and softmax.
 * frame_blocks (F) is a scheduling hint, 0 = none: the number of consecutive
 * blocks that make up one latent frame in the block order of section 3.1.1
 * (Figure 3), i.e. (Hs/P) * (Ws/P). With F > 0 (n % F == 0, else
 * NABLA_ERR_INVALID_ARG) and at least two frames, query blocks i and i + F --
 * the same tile position in consecutive frames, whose kept lists overlap
 * strongly in video latents -- share one workgroup that loads each K/V tile of
 * the union of their lists once. Outputs are bitwise identical either way
 * (every query block still visits its own kept blocks in ascending order).
 */
NABLA_API nabla_status_t nabla_sparse_attn_fwd(const void* q, const void* k, const void* v, int32_t B,
                                     int32_t H, int32_t S, int32_t D, int32_t N,
                                     const int32_t* kv_count, const int32_t* kv_idx,
                                     float softmax_scale, int32_t frame_blocks, void* o,
                                     int32_t o_dtype, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * Allocation-free variant of nabla_sparse_attn_fwd, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments, checks, kernels and
 * results (bitwise) without the workspace argument. Its scratch memory -- the
 * per-head work order and pair counts, 8 * B * H * S / N bytes plus alignment
 * -- lives in a library-held device array of NABLA_STATIC_SCRATCH_BYTES per
 * GPU, kept until the process ends; the call allocates and frees nothing.
 * Shapes that need more scratch than that (B * H * S / N above about one
 * million blocks) return NABLA_ERR_WORKSPACE before anything is launched.
 * Calls that overlap on one GPU share the array and race: serialise them
 * (one stream, or events). The array of the GPU that owns `stream` is used.
 */
#define NABLA_STATIC_SCRATCH_BYTES (8u << 20)
NABLA_API nabla_status_t nabla_sparse_attn_fwd_static(const void* q, const void* k, const void* v,
                                                      int32_t B, int32_t H, int32_t S, int32_t D,
                                                      int32_t N, const int32_t* kv_count,
                                                      const int32_t* kv_idx, float softmax_scale,
                                                      int32_t frame_blocks, void* o, int32_t o_dtype,
                                                      float* lse, void* stream);

/*
 * Block-sparse attention backward, for training through the NABLA mask: the
 * mask is built inside the training algorithm of section 3.1 and attention is
 * trained with it -- fine-tuning (section 4.1) and the 2B-DiT pretraining run of
 * section 4.3, whose iteration time (10.9 s dense vs 7.5 s sparse) includes this
 * pass. Gradients of eq. (4) with the mask held constant (the mask is a
 * piecewise-constant function of Q and K, so it carries no gradient):
 *   P = exp(scale * Q K^T - LSE) on kept blocks, Delta_s = dO_s . O_s,
 *   dV = P^T dO, dP = dO V^T, dS = P * (dP - Delta),
 *   dQ = scale * dS K, dK = scale * dS^T Q.
 * Inputs o (of type o_dtype, bf16 or fp32) and lse are the forward's outputs
 * for the same q, k, v, lists and scale; d_o is the output gradient (bf16). q_count/q_idx is the transpose of
 * kv_count/kv_idx (as produced by nabla_build_mask). dq, dk, dv: bf16 outputs.
 * Deterministic: no atomics on the gradients.
 */
NABLA_API nabla_status_t nabla_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                     int32_t o_dtype, const void* d_o, const float* lse, int32_t B, int32_t H,
                                     int32_t S, int32_t D, int32_t N, const int32_t* kv_count,
                                     const int32_t* kv_idx, const int32_t* q_count,
                                     const int32_t* q_idx, float softmax_scale, void* dq,
                                     void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * Mask-fidelity diagnostic, part 1: the true block mass of full attention, the
 * quantity of the per-block fidelity test asked for in the review record of
 * arXiv 2507.13546 (pith.science: the referee's first major comment and the
 * skeptic's falsifier). For every head, query block i and key block j:
 *   mass[b, h, i, j] = (1/N) sum_{s in block i} sum_{u in block j} exp(scale q_s . k_u - lse_s)
 * with lse the dense (all-keys) log-sum-exp of eq. (2) -- for instance the lse
 * that nabla_sparse_attn_fwd returns for lists that keep every block. Each row
 * then sums to 1. q, k: bf16 [B, H, S, D] in block order; lse: fp32 [B, H, S]
 * (natural log); mass: fp32 [B, H, n, n] output. softmax_scale > 0, finite. Costs
 * one dense Q K^T (2 S^2 D flop per head) on bf16 MFMA with fp32 sums; no
 * workspace; deterministic.
 */
NABLA_API nabla_status_t nabla_block_mass(const void* q, const void* k, const float* lse, int32_t B,
                                          int32_t H, int32_t S, int32_t D, int32_t N,
                                          float softmax_scale, float* mass, void* stream);

/*
 * Mask-fidelity diagnostic, part 2: for every row (b, h, i) of a block mass
 * (from nabla_block_mass) and block lists (from any nabla_build_*_mask),
 *   recall[b, h, i]      = sum of mass[b, h, i, j] over the kept j,
 *   best_recall[b, h, i] = sum of the c largest mass[b, h, i, :], c = kv_count --
 * the top-mass block oracle at the same per-row budget, so recall <= best_recall.
 * mass: fp32 [B, H, n, n]; kv_count/kv_idx as everywhere (indices outside [0, n)
 * are ignored, counts clamped to [0, n]); recall, best_recall: fp32 [B, H, n]
 * outputs. Sums in double, deterministic; no workspace. S and N as for the
 * other calls (S % N == 0, N == 64).
 */
NABLA_API nabla_status_t nabla_mask_recall(const float* mass, int32_t B, int32_t H, int32_t S,
                                           int32_t N, const int32_t* kv_count, const int32_t* kv_idx,
                                           float* recall, float* best_recall, void* stream);

/*
 * Block-list check. The attention and diagnostic kernels read lists defensively:
 * a count outside [0, n] is clamped into it and an entry outside [0, n) is read
 * as block 0, so a malformed list gives wrong results rather than an error (and
 * a non-ascending list is processed in its own order). Callers that build or
 * edit lists themselves can check them first: this counts the rows (b, h, i)
 * whose list is malformed -- kv_count outside [0, n], or among the first
 * kv_count entries one outside [0, n) or one not larger than its predecessor
 * (the lists every nabla_build_*_mask writes, kv and q lists alike, are
 * strictly ascending and pass) -- and writes the number to *bad_rows (one
 * device int32, overwritten, written by the GPU: read it after the stream has
 * reached this call). count: int32 [B, H, n]; idx: int32 [B, H, n, n], row
 * stride n; n = S / N with S % N == 0 and N == 64 as for the other calls.
 * NABLA_ERR_INVALID_ARG for null pointers. No workspace; enqueued on `stream`
 * like every call.
 */
NABLA_API nabla_status_t nabla_check_lists(const int32_t* count, const int32_t* idx, int32_t B,
                                           int32_t H, int32_t S, int32_t N, int32_t* bad_rows,
                                           void* stream);

/*
 * Token reordering, section 3.1.1 (Figure 3): "fractal flattening", applied to
 * the token sequence at the input of the network, and its inverse at the output.
 * Each of the B items holds T frames of Hs x Ws tokens; raster order is
 * (t, y, x) with x fastest. Block order groups the P x P tokens of each spatial
 * patch into P*P consecutive tokens, row-major inside the patch, patches
 * row-major inside the frame, frames in their original order: block-order
 * position ((t*(Hs/P) + y/P)*(Ws/P) + x/P)*P*P + (y%P)*P + x%P holds raster
 * token (t, y, x). With P*P == N the result is the block layout the other entry
 * points expect.
 * A token is an opaque row of row_bytes bytes, for example the C features of a
 * hidden state ([B, S, C] with row_bytes = C * element size) or one head's D
 * features ([B*H, S, D], passing B*H as B).
 *   inverse = 0: src in raster order -> dst in block order;
 *   inverse = 1: src in block order  -> dst in raster order.
 * src, dst: device pointers, 16-byte aligned, B*T*Hs*Ws*row_bytes bytes each,
 * not overlapping (out of place). row_bytes > 0 and a multiple of 16; P >= 1;
 * Hs and Ws multiples of P (NABLA_ERR_INVALID_ARG otherwise). B, T, Hs or Ws
 * equal to 0 is an empty permutation: NABLA_OK, nothing enqueued. A pure byte
 * permutation: dst is bit-exact. No workspace.
 */
NABLA_API nabla_status_t nabla_reorder_tokens(const void* src, void* dst, int32_t B, int32_t T,
                                              int32_t Hs, int32_t Ws, int32_t P, int64_t row_bytes,
                                              int32_t inverse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NABLA_H */

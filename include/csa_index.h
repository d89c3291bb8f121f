/*
 * csa_index.h -- C ABI of the MI355X (gfx950) CSA indexer score / top-k library.
 *
 * The operation (DeepSeek-V4 Compressed Sparse Attention indexer, the fused
 * "StreamIndex" score of MaxText PR #5079 "Add StreamIndex Kernel for CSA",
 * PR description and the BlockSpec review): for batch b, query row i and
 * compressed key entry j,
 *
 *     score[b,i,j] = scale * sum_h w[b,i,h] * ReLU( sum_t q[b,h,i,t] * k[b,j,t] )
 *
 * with bf16 inputs and fp32 accumulation (the same PR's commit that chunks the
 * head accumulation and runs bf16 einsums with float32 accumulation).
 *
 * Masks (MaxText PR #4915 "DSV4: Add indexer_save_selection and
 * indexer_sharded_topk", inline review of the indexer's future and segment
 * masks): with absolute row position p = q_offset[b] + i and compress rate m,
 * entry j is a future entry when j >= clamp(floor((p+1)/m), 0, W).  When
 * segment ids are given, entry j is also masked when k_seg[b,j] != q_seg[b,i].
 * A masked entry reads -inf in a score output and is never selected.
 *
 * Selection (same PR, description: masking and top-k selection consumed by
 * the sparse attention): per row, the top_k unmasked entries ordered by score
 * descending, equal scores going to the lower j, then -1 padding when fewer
 * than top_k entries are unmasked.  -0 and +0 scores compare equal.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates and frees nothing, never synchronises, and keeps no pointer
 *    after returning.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 *    default stream); buffers must stay alive until it completes.
 *  - Arguments are checked on the host before anything is enqueued.  On any
 *    error nothing is enqueued, the function returns a non-zero status and
 *    csa_last_error() describes the problem.  Shapes the kernels do not
 *    implement return CSA_ERR_UNSUPPORTED; there is no silent fallback.
 *  - bf16 tensors are passed as 16-bit bfloat16 patterns.
 *  - Device-resident q_offset / q_seg / k_seg values are never trusted for
 *    addressing: any int32 value is memory-safe (thresholds are clamped).
 *  - Functions never throw and are safe to call from several host threads.
 */
#ifndef CSA_INDEX_H
#define CSA_INDEX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum csa_status {
    CSA_OK = 0,
    CSA_ERR_INVALID_ARG = 1, /* null / misaligned pointer, bad size, inconsistent masks */
    CSA_ERR_UNSUPPORTED = 2, /* a shape or stride the kernels do not implement        */
    CSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required             */
    CSA_ERR_DEVICE = 4       /* the HIP runtime reported an error when launching       */
} csa_status;

/* Execution plan.  AUTO picks by shape; the others force one plan (every plan
 * computes bit-identical scores and selections). */
typedef enum csa_plan {
    CSA_PLAN_AUTO = 0,
    CSA_PLAN_ROW_TILES = 1, /* workgroups own blocks of query rows and walk K tiles;
                               W <= 65536 (entries are held in 16 bits), AUTO takes
                               SPLIT_ROWS beyond that                                */
    CSA_PLAN_SPLIT_ROWS = 2 /* long rows split over workgroups (decode), then a top-k pass */
} csa_plan;

/*
 * Problem description.  Element strides (not bytes).  The innermost dimension
 * is contiguous: D for q and k, H for w.
 *   q : [B,H,S,D] bf16 at q + b*q_sb + h*q_sh + i*q_ss + t
 *       (head-major q has q_sh = S*D, q_ss = D; sequence-major [B,S,H,D] has
 *        q_sh = D, q_ss = H*D)
 *   k : [B,W,D] bf16 at k + b*k_sb + j*k_sw + t   (decode: W = cache capacity)
 *   w : [B,S,H] bf16 at w + b*w_sb + i*w_ss + h
 * Supported: D in {32, 64, 128}; 1 <= H <= 128; q and k 16-byte aligned with
 * strides that are multiples of 8 elements; k_sw < 2^24; W <= 2^30; m >= 1;
 * finite scale.  Strides may be smaller than the row they step over: k_sw < D
 * makes entries overlap and k_sw = 0 repeats one entry (the kernels read the
 * D values at each entry's own address, whatever the stride).
 */
typedef struct csa_index_problem {
    int32_t B, S, H, D, W;
    int32_t compress_rate; /* m */
    float scale;
    int32_t plan;          /* csa_plan */
    int64_t q_sb, q_sh, q_ss;
    int64_t k_sb, k_sw;
    int64_t w_sb, w_ss;
} csa_index_problem;

/* Optional masks (device pointers).  masks == NULL means all fields NULL. */
typedef struct csa_index_masks {
    const int32_t *q_offset; /* [B] absolute position of row 0; NULL => 0          */
    const int32_t *q_seg;    /* [B,S] dense segment id of each row; NULL => none    */
    const int32_t *k_seg;    /* [B,W] dense segment id of each entry; NULL iff q_seg */
} csa_index_masks;

/*
 * Masked scores.  scores: [B,S,W] fp32, dense, 4-byte aligned; every element
 * is written (masked = -inf).
 */
csa_status csa_index_score(const csa_index_problem *p, const void *q, const void *k, const void *w,
                           const csa_index_masks *masks, float *scores, void *stream);

/*
 * Top-k of each row of a dense fp32 matrix scores [rows, W] (row stride W).
 * Entries equal to -inf or NaN are never selected.  idx: [rows, top_k] int32.
 * 1 <= top_k <= 2048.  Needs no workspace today: pass NULL / 0 (a size query
 * is provided so callers need not change if that ever changes).
 */
csa_status csa_index_topk(int64_t rows, int32_t W, int32_t top_k, const float *scores,
                          int32_t *idx, void *workspace, size_t workspace_bytes, void *stream);

csa_status csa_index_topk_workspace_size(int64_t rows, int32_t W, int32_t top_k, size_t *bytes);

/*
 * Fused score + selection.  idx: [B,S,top_k] int32 (dense).  scores: optional
 * [B,S,W] fp32 output (NULL = not written; the score matrix then never reaches
 * HBM on the row-tile plan).  workspace: device memory of at least
 * csa_index_workspace_size() bytes (may be NULL when that size is 0), 256-byte
 * aligned.  1 <= top_k <= 2048.
 */
csa_status csa_index_select(const csa_index_problem *p, const void *q, const void *k, const void *w,
                            const csa_index_masks *masks, int32_t top_k, int32_t *idx, float *scores,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes csa_index_select needs for this problem when scores == NULL
 * (0 when it needs none).  Host-only; checks the arguments like the call. */
csa_status csa_index_workspace_size(const csa_index_problem *p, int32_t top_k, size_t *bytes);

/*
 * csa_index_select without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The workspace csa_index_select would take
 * comes from a scratch buffer of CSA_NOALLOC_SCRATCH_BYTES that the library
 * holds in device memory, one per GPU, from the first call on that GPU until
 * the process ends; this function allocates and frees nothing.  Problems
 * whose workspace (csa_index_workspace_size) exceeds it return
 * CSA_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU
 * shares that GPU's buffer, so calls that overlap on one GPU (concurrent
 * streams, or host threads without ordering) race and must not be issued;
 * calls ordered on one stream are safe.  The kernels overwrite every part of
 * the buffer they later read, so no call depends on an earlier one's
 * contents.  Arguments and results are those of csa_index_select.
 */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

csa_status csa_index_select_noalloc(const csa_index_problem *p, const void *q, const void *k, const void *w,
                                    const csa_index_masks *masks, int32_t top_k, int32_t *idx, float *scores,
                                    void *stream);

/*
 * Backward of csa_index_score: the gradients of
 *     L = sum over unmasked (b,i,j) of grad[b,i,j] * score[b,i,j]
 * with respect to q, k and w (the vector-Jacobian product of the custom VJP
 * in MaxText PR #5079 "Add StreamIndex Kernel for CSA"; its review asks for a
 * fused backward that does not materialise the [B,H,S,W] per-head logits,
 * and none is materialised here).  With l = q[b,h,i,:] . k[b,j,:]:
 *     dw[b,i,h]   = scale * sum_j grad[b,i,j] * ReLU(l)
 *     dq[b,h,i,:] = scale * w[b,i,h] * sum_j grad[b,i,j] * [l > 0] * k[b,j,:]
 *     dk[b,j,:]   = scale * sum_i sum_h grad[b,i,j] * w[b,i,h] * [l > 0] * q[b,h,i,:]
 * Masked pairs (the masks of csa_index_score) take no part: grad at masked
 * positions is never read into a result and may hold anything finite or not.
 * The ReLU derivative at l = 0 is 0.  Logits are recomputed exactly as the
 * forward computes them; the gradient operands grad*[l>0] (for dq) and
 * grad*w*[l>0] (for dk) are rounded to bf16 once and contracted with fp32
 * accumulation; dw is an fp32 sum.
 *
 * grad: [B,S,W] fp32, dense.  Outputs are fp32, dense, every element written:
 * dq [B,H,S,D] (4-byte aligned), dk [B,W,D] (16-byte aligned), dw [B,S,H]
 * (4-byte aligned).  q, k, w, masks and the problem are as for
 * csa_index_score (p->plan is not used).  workspace: at least
 * csa_index_backward_workspace_size() bytes, 256-byte aligned (per-chunk
 * partial key gradients); results do not depend on its prior contents and
 * are deterministic.
 */
csa_status csa_index_score_backward(const csa_index_problem *p, const void *q, const void *k, const void *w,
                                    const csa_index_masks *masks, const float *grad, float *dq, float *dk,
                                    float *dw, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Indexer loss: per query row, the KL divergence between a target
 * distribution over the row's visible entries and the softmax of the row's
 * scores (the KL-divergence loss of calculate_indexer_loss in MaxText PR #4564
 * "Implement QK attention head chunking in MLA", there chunked over heads;
 * here the score's 32-head blocks are the chunks).  The pages give no
 * formula; with the masks of csa_index_score, a = target[b,i,:] and visible j:
 *     p_j   = a_j / sum_j a_j              (the target, L1-normalised)
 *     kl[b,i] = sum_j p_j (log p_j - log softmax(score[b,i,:])_j),  0 log 0 = 0
 *     grad[b,i,j] = d kl[b,i] / d score[b,i,j] = softmax_j - p_j  (0 if masked)
 * Rows with no visible entry or zero target mass get kl = 0 and a zero
 * gradient.  target: [B,S,W] fp32, dense, >= 0 at visible entries (any value
 * at masked ones, never read into a result).  kl: [B,S] fp32.  grad: NULL or
 * [B,S,W] fp32 dense; with NULL the scores never reach HBM (one fused pass
 * with an online log-sum-exp), otherwise the scores are written to grad and
 * then turned into the gradient in place (feed it to
 * csa_index_score_backward for dq, dk, dw).  p->plan is not used.
 * Computed in fp32 with fast exp/log.
 */
csa_status csa_index_kl_loss(const csa_index_problem *p, const void *q, const void *k, const void *w,
                             const csa_index_masks *masks, const float *target, float *kl, float *grad,
                             void *stream);

/* Workspace bytes csa_index_score_backward needs for this problem.  Host-only;
 * checks the problem like the call. */
csa_status csa_index_backward_workspace_size(const csa_index_problem *p, size_t *bytes);

/* Plan the library would run for this problem (CSA_PLAN_ROW_TILES or
 * CSA_PLAN_SPLIT_ROWS), or -1 if the problem is invalid.  Host-only. */
int32_t csa_index_resolve_plan(const csa_index_problem *p);

/* Static description of a status code. */
const char *csa_status_string(csa_status s);

/* Detail of the last error on the calling host thread ("" if none). */
const char *csa_last_error(void);

/* ABI version of this header (bumped on incompatible change). */
int32_t csa_index_abi_version(void);

#define CSA_INDEX_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* CSA_INDEX_H */

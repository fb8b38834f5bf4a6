/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (forward,
 * and the backward pass of the bf16 and fp16 forward).
 *
 * The forward entry points compute, for every batch entry b and head h,
 *
 *     S   = scale * Q K^T                      (N x N, never stored)
 *     A   = row-softmax(S), disallowed keys at -inf before the softmax
 *     O   = A V
 *     LSE = log(sum_j exp(S_ij)) over the allowed keys j   (natural log)
 *
 * which is scaled-dot-product attention as defined on the page "Ch.04
 * Attention optimisation: FlashAttention and sparse attention" (mdooai.com,
 * sections "Core formula" and "Key points of the formulas", including the
 * -inf masking rule of its sparse-attention paragraph).  It is computed tile
 * by tile with a running row maximum and running row sum, so S and A never
 * reach device memory: the IO-aware exact method summarised on the page
 * "FlashAttention: Fast and Memory-Efficient Exact Attention with
 * IO-Awareness" (ai-paper-library, Summary and Method), including its
 * block-sparse extension, and the five-stage map (tile Q/K/V, stage blocks on
 * chip, local scores with running normalisation, accumulate without the full
 * matrix, schedule for the accelerator) on the page "What is FlashAttention?"
 * (unite.ai, "Five-stage operating map").
 *
 * Allowed set of key j for query i (all conditions must hold):
 *   causal != 0        : j <= i
 *   key_len != NULL    : j < key_len[b]   (value clamped to [0, N])
 *   block_mask != NULL : block_mask[(i/128) * nb + (j/128)] != 0,
 *                        nb = ceil(N/128); one mask shared by every (b, h)
 * A query row with no allowed key gets O = 0 and LSE = -inf.
 *
 * Layout and ownership (every entry point):
 *   q, k, v, o : DEVICE pointers, contiguous [B, H, N, d], d innermost,
 *                16-byte aligned; owned by the caller.  o must not overlap
 *                q, k or v.
 *   lse        : DEVICE pointer to float [B, H, N] (4-byte aligned) or NULL
 *                (then no logsumexp is written); must not overlap q, k, v
 *                or o.
 *   key_len    : DEVICE pointer to int32 [B] or NULL.
 *   block_mask : DEVICE pointer to uint8 [nb * nb] or NULL; row = query
 *                block, column = key block, 128 x 128 tokens per block.
 *   scale      : the softmax scale (1/sqrt(d) for standard attention); any
 *                finite value.
 *   stream     : HIP stream the work is enqueued on (NULL = default stream).
 *   B, H, N    : >= 1, with B*H*ceil(N/16) < 2^31.
 *   d          : 64 or 128.
 *
 * Behaviour: each call validates its arguments on the host and returns a
 * status code before making any HIP call; on success the work is enqueued
 * asynchronously on `stream` (the call never synchronises and never
 * allocates device or host memory).  A failed launch returns FA_ERR_HIP and
 * the hipError_t is kept for fa_last_hip_error() on the calling thread.  The
 * library never prints or aborts.  Results are deterministic: no atomics,
 * identical bits from run to run for the same inputs and tile choice.
 * Non-finite inputs propagate unchecked.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL_PTR = 1,             /* q, k, v or o is NULL                        */
    FA_ERR_INVALID_SHAPE = 2,        /* B, H, H_kv or N < 1, H % H_kv != 0, or the
                                        grid would overflow                         */
    FA_ERR_UNSUPPORTED_HEAD_DIM = 3, /* d not in {64, 128}                          */
    FA_ERR_MISALIGNED = 4,           /* q/k/v/o not 16-byte, lse/key_len not 4-byte */
    FA_ERR_UNSUPPORTED_TILE = 5,     /* (Br, Bc) pair or dtype not built            */
    FA_ERR_HIP = 6,                  /* the kernel launch failed                    */
    FA_ERR_INVALID_ARG = 7           /* non-finite scale, o or lse overlapping an
                                        input or each other, unknown tile order     */
} fa_status;

/* Element type codes for fa_fwd_ex and fa_fwd_gqa.  FA_DTYPE_F16 (IEEE
 * half inputs and output, fp16 probabilities as the PV operand, fp32
 * arithmetic otherwise) is the other 16-bit format the page on
 * FlashAttention-2 adoption (tcdigital.jp, section on fp16/bf16 precision
 * support) names as the precisions the method is meant to run in.
 * FA_DTYPE_BF16_F32OUT is the bf16 path with o a float [B, H, N, d] array
 * that receives O before its final rounding (bf16 inputs, bf16
 * probabilities as the PV operand): the deviation study of the page "Is
 * Flash Attention Stable?" explainer (aibr.jp, sections 3 and 4) compares
 * outputs with an FP64 golden value, and with O left unrounded the effect of
 * the tiling is not hidden under the last rounding.  FA_DTYPE_BF16_ACC16 is
 * bf16 I/O with the running output rounded to bf16 after every key tile, a
 * model of an implementation that holds its partial output in the input
 * precision between tiles, so that the output is rounded once per rescaling
 * step (the section 3 explanation of why deviation falls as tiles grow);
 * it is a study mode, less accurate than FA_DTYPE_BF16 by design.  Both run
 * on the tile-study kernels (Br = Bc = 0 selects (128, 64)). */
enum {
    FA_DTYPE_BF16 = 0,
    FA_DTYPE_F32 = 1,
    FA_DTYPE_F16 = 2,
    FA_DTYPE_BF16_F32OUT = 3,
    FA_DTYPE_BF16_ACC16 = 4
};

/*
 * bf16 inputs and output (q, k, v, o point to bfloat16), fp32 arithmetic
 * inside: bf16 x bf16 products on the matrix cores with fp32 accumulation,
 * fp32 running max/sum, probabilities rounded to bf16 (round to nearest even)
 * only as the operand of the P V product, O rounded to bf16 once at the end.
 * Uses the library's tuned tile shape for (d, causal).
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int N, int d, float scale, int causal,
           const int32_t *key_len, const uint8_t *block_mask,
           hipStream_t stream);

/*
 * fp32 inputs and output, fp32 arithmetic throughout (fp32 matrix-core
 * products, probabilities never rounded to a 16-bit type).  Same arguments
 * and semantics as fa_fwd.  This is the higher-precision end of the precision
 * axis that the page "Is Flash Attention Stable?" explainer (aibr.jp,
 * section 3) sets against BF16, each compared with an FP64 golden value.
 */
int fa_fwd_f32(const float *q, const float *k, const float *v, float *o,
               float *lse, int B, int H, int N, int d, float scale, int causal,
               const int32_t *key_len, const uint8_t *block_mask,
               hipStream_t stream);

/*
 * Tile-size control for the numeric-deviation study of the page "Is Flash
 * Attention Stable?" explainer (aibr.jp, sections 3 and 4: block sizes Br and
 * Bc varied, output compared with an FP64 golden value).  Same arguments as
 * fa_fwd plus:
 *   dtype : FA_DTYPE_BF16 (q/k/v/o bfloat16), FA_DTYPE_F16 (IEEE half),
 *           FA_DTYPE_F32 (float), FA_DTYPE_BF16_F32OUT (q/k/v bfloat16,
 *           o float) or FA_DTYPE_BF16_ACC16 (bfloat16, running output
 *           rounded to bf16 after every key tile)
 *   Br    : query rows per tile;  Bc : key rows per tile.
 * Br = Bc = 0 selects the tuned default (what fa_fwd / fa_fwd_f32 use).  For
 * bf16 every Br, Bc in {16, 32, 64, 128} is built for d = 64 and 128 (the
 * tile-study kernel family; an explicit (128, 64) runs it, not the tuned
 * kernel that the default (128, 64) runs), plus the tuned (256, 64), which
 * does not take a block mask.  FA_DTYPE_BF16_F32OUT, FA_DTYPE_BF16_ACC16 and
 * fp32 build every Br, Bc in {16, 32, 64, 128} (fp32 default (128, 32));
 * fp16 builds (128, 64).  Unbuilt pairs return FA_ERR_UNSUPPORTED_TILE.
 */
int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int N, int d, float scale, int causal,
              const int32_t *key_len, const uint8_t *block_mask,
              hipStream_t stream, int dtype, int Br, int Bc);

/* Key-tile visit orders for fa_fwd_study. */
enum { FA_ORDER_ASCENDING = 0, FA_ORDER_DESCENDING = 1, FA_ORDER_SHUFFLED = 2 };

/*
 * Tile-order control for the deviation study: the page "Is Flash Attention
 * Stable?" explainer (aibr.jp, sections 2 and 3) varies the order in which
 * blocks/tiles are processed besides their sizes, and asks libraries to
 * expose such settings (section 6).  Same arguments as fa_fwd_ex plus
 *   tile_order : FA_ORDER_ASCENDING (key tiles 0, 1, ...; what every other
 *                entry point does), FA_ORDER_DESCENDING (last key tile
 *                first) or FA_ORDER_SHUFFLED (a fixed permutation: of a
 *                workgroup's n key tiles, visit i goes to tile
 *                (a*i + n/2) mod n, a the smallest integer >= round(0.618*n)
 *                coprime to n; tiles the block mask turns off are skipped).
 *                Other values: FA_ERR_INVALID_ARG.
 * The result is the same attention up to rounding; only the order of the
 * running-maximum/rescale steps changes.  Orders other than ascending run
 * on the tile-study kernels only (bf16 with an explicit Br, Bc in
 * {16, 32, 64, 128}, FA_DTYPE_BF16_F32OUT or FA_DTYPE_BF16_ACC16; d = 64 or
 * 128); other tiles return FA_ERR_UNSUPPORTED_TILE.
 */
int fa_fwd_study(const void *q, const void *k, const void *v, void *o, float *lse,
                 int B, int H, int N, int d, float scale, int causal,
                 const int32_t *key_len, const uint8_t *block_mask,
                 hipStream_t stream, int dtype, int Br, int Bc, int tile_order);

/*
 * Grouped-query attention: the H query heads of each batch entry are split
 * into H_kv consecutive groups of H / H_kv heads, and every head of group g
 * attends to key/value head g (H_kv = H: plain multi-head attention;
 * H_kv = 1: multi-query attention).  This is the head sharing that the page
 * on FlashAttention-2 adoption (tcdigital.jp, section on the synergy with
 * MQA/GQA) says the method combines with.  Same arguments as fa_fwd_ex
 * except:
 *   k, v : DEVICE pointers, contiguous [B, H_kv, N, d] (16-byte aligned)
 *   H_kv : key/value heads, >= 1, H must be a multiple of H_kv
 *          (else FA_ERR_INVALID_SHAPE).
 * q, o, lse keep their [B, H, ...] layouts; o must not overlap q, k or v.
 */
int fa_fwd_gqa(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int H, int H_kv, int N, int d, float scale, int causal,
               const int32_t *key_len, const uint8_t *block_mask,
               hipStream_t stream, int dtype, int Br, int Bc);

/*
 * Forward with a key-range split for grids too small to fill the GPU (few
 * heads, e.g. one GPU's share of a head-sharded problem): each query tile's
 * key tiles are shared out over several workgroups, each writing an fp32
 * partial O (normalised by its own row sum) and partial log-sum-exp to the
 * workspace, and a second kernel merges them per row,
 *     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,
 * the same combination that merges results computed on different key
 * ranges anywhere.  Same arguments as fa_fwd_gqa with the tuned tile, plus
 *   dtype     : FA_DTYPE_BF16 or FA_DTYPE_F16 (the other dtypes run
 *               unsplit, as fa_fwd_gqa with Br = Bc = 0)
 *   workspace : DEVICE memory owned by the caller (16-byte aligned) of
 *               workspace_bytes bytes, or NULL.  fa_fwd_workspace_size
 *               gives the bytes needed; when it is 0, or workspace is NULL,
 *               the call is fa_fwd_gqa with Br = Bc = 0.  A non-NULL
 *               workspace smaller than needed, misaligned, or overlapping an
 *               input or output: FA_ERR_INVALID_ARG.  Its contents on entry
 *               do not matter; every byte the split uses is written first.
 * The result equals the unsplit one up to rounding (the shares' rows are
 * combined in fp32 and rounded to the output type once).
 */
int fa_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int H_kv, int N, int d, float scale, int causal,
              const int32_t *key_len, const uint8_t *block_mask,
              hipStream_t stream, int dtype, void *workspace,
              size_t workspace_bytes);

/* Workspace bytes fa_fwd_ws may use for this shape and dtype (0: none is
 * used, or the arguments are invalid).  Independent of H_kv, masks and
 * scale: it covers the causal mask, which splits some grids that are not
 * split without it (a call without the causal mask then uses part of the
 * workspace, or none). */
size_t fa_fwd_workspace_size(int B, int H, int N, int d, int dtype);

/* Size of the library's static scratch (fa_fwd_noalloc): the largest
 * workspace fa_fwd_workspace_size returns for any shape.  A split is only
 * used on grids of at most 512 query tiles, with at most 1024 shares in
 * all, so its partials cover at most 1024 * 128 rows of d + 1 <= 129 floats. */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)1024 * 128 * 129 * 4)

/*
 * fa_fwd_ws for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same computation as fa_fwd_ws given the workspace fa_fwd_workspace_size
 * asks for (identical bits), with the key-range split's fp32 partials kept
 * in a static device array of FA_NOALLOC_SCRATCH_BYTES bytes inside the
 * library instead of a caller workspace.
 *   Arguments, layouts, status codes: as fa_fwd_ws without the workspace
 *   arguments.  The device is the current HIP device of the calling thread
 *   (stream must belong to it).
 *   Memory: the call allocates nothing.  The static array exists once per
 *   GPU the library runs on and is held until the process ends; its address
 *   on a device is looked up on the first call there (hipGetSymbolAddress).
 *   A shape whose split would need more than FA_NOALLOC_SCRATCH_BYTES returns
 *   FA_ERR_INVALID_SHAPE (no valid shape does: the constant is the largest
 *   split workspace).
 *   Concurrency: every call on one GPU uses that GPU's array.  Calls whose
 *   work overlaps in time on one GPU (different streams, or different host
 *   threads without ordering) race on it and may return wrong results; calls
 *   ordered on one stream do not.  Nothing in the array has to start at
 *   zero: every partial is written before it is read.
 */
int fa_fwd_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int H, int H_kv, int N, int d, float scale, int causal,
                   const int32_t *key_len, const uint8_t *block_mask,
                   hipStream_t stream, int dtype);

/*
 * Materialised ("baseline") attention: the same result as fa_fwd_ex computed
 * in the conventional order, for the comparison that the page "Is Flash
 * Attention Stable?" explainer (aibr.jp, opening dialogue and sections 3
 * and 4) makes between FlashAttention and a Baseline Attention, each against
 * an FP64 golden value at BF16.  Three kernels on `stream`:
 *   S = scale * Q K^T, every (query, key) pair of every head, written to
 *       `workspace` as [B, H, N, N] of the intermediate type (-inf where the
 *       key is not allowed);
 *   A = row-softmax(S) in place (fp32 arithmetic: max, sum of exp(S - max),
 *       then exp(S - max) / sum), LSE = max + log(sum) (natural log);
 *   O = A V (A rounded to the input type as the matrix-core operand, fp32
 *       accumulation, O rounded once to the output type).
 * Key tiles whose A entries are all exactly zero (past the causal diagonal
 * or key_len, masked blocks) are skipped in A V.  Arguments as fa_fwd_ex
 * (no tile choice) plus
 *   dtype       : FA_DTYPE_BF16, FA_DTYPE_F16, FA_DTYPE_F32 or
 *                 FA_DTYPE_BF16_F32OUT
 *   inter_dtype : type S and A are held in: FA_DTYPE_F32, or the input type
 *                 of a 16-bit dtype (FA_DTYPE_BF16 for FA_DTYPE_BF16 and
 *                 FA_DTYPE_BF16_F32OUT, FA_DTYPE_F16 for FA_DTYPE_F16:
 *                 S and A each rounded once when written).  Other pairs:
 *                 FA_ERR_UNSUPPORTED_TILE.
 *   workspace   : DEVICE memory owned by the caller, 16-byte aligned, of at
 *                 least fa_fwd_baseline_workspace_size(B, H, N, dtype,
 *                 inter_dtype) bytes (else FA_ERR_INVALID_ARG; NULL:
 *                 FA_ERR_NULL_PTR); overwritten (holds A afterwards).
 * k and v have H heads (no grouping).  Outputs and the workspace must not
 * overlap the inputs or each other (FA_ERR_INVALID_ARG).  Grids
 * B*H*ceil(N/128)^2 and B*H*N must be below 2^31 (FA_ERR_INVALID_SHAPE).
 */
int fa_fwd_baseline(const void *q, const void *k, const void *v, void *o, float *lse,
                    int B, int H, int N, int d, float scale, int causal,
                    const int32_t *key_len, const uint8_t *block_mask,
                    hipStream_t stream, int dtype, int inter_dtype,
                    void *workspace, size_t workspace_bytes);

/* Workspace bytes fa_fwd_baseline needs: B * H * N * N elements of the
 * intermediate type (0 for an unsupported (dtype, inter_dtype) pair or an
 * invalid shape). */
size_t fa_fwd_baseline_workspace_size(int B, int H, int N, int dtype, int inter_dtype);

/*
 * Backward pass: the gradients of the loss sum(dout * o) with respect to q,
 * k and v, for bf16 attention computed by fa_fwd / fa_fwd_gqa with the same
 * scale, causal flag, key_len and block_mask.  The pages give only the
 * forward definition (mdooai.com, "Core formula") and report training
 * speed-ups (ai-paper-library, Summary); the gradients are the chain rule on
 * that definition:
 *     P = exp(S - LSE), dV = P^T dO, dP = dO V^T, Delta_i = dO_i . O_i,
 *     dS = P (dP - Delta), dQ = scale dS K, dK = scale dS^T Q,
 * with P recomputed tile by tile from q, k and the forward's lse (never
 * stored); dK and dV of a shared key/value head sum over its query heads.
 *   q, o, dout : DEVICE bf16 [B, H, N, d]      k, v : bf16 [B, H_kv, N, d]
 *   lse        : DEVICE float [B, H, N], the forward's logsumexp (natural log)
 *   delta      : DEVICE float [B, H, N] workspace owned by the caller,
 *                overwritten (holds Delta after the call)
 *   dq         : DEVICE bf16 [B, H, N, d] output
 *   dk, dv     : DEVICE bf16 [B, H_kv, N, d] outputs
 * All 16-byte aligned (lse, delta, key_len: 4).  Outputs and workspace must
 * not overlap the inputs or each other (FA_ERR_INVALID_ARG).  Same status
 * codes and asynchronous, deterministic behaviour as the forward; d = 64 or
 * 128; H a multiple of H_kv.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o,
           const void *dout, const float *lse, float *delta, void *dq,
           void *dk, void *dv, int B, int H, int H_kv, int N, int d,
           float scale, int causal, const int32_t *key_len,
           const uint8_t *block_mask, hipStream_t stream);

/*
 * fa_bwd with an element type and an optional workspace.
 *   dtype     : FA_DTYPE_BF16 (what fa_bwd does) or FA_DTYPE_F16 (q, k, v,
 *               o, dout, dq, dk, dv all IEEE half; P and dS enter the
 *               matrix-core products rounded to fp16 instead of bf16, every
 *               other step as for bf16).  Other dtypes:
 *               FA_ERR_UNSUPPORTED_TILE.
 *   workspace : DEVICE memory owned by the caller (16-byte aligned) of
 *               workspace_bytes bytes, or NULL.  When a grid is too small
 *               for the GPU (few heads or key/value heads, short N), the
 *               work of each dK/dV workgroup (its query heads and query
 *               tiles) and of each dQ workgroup (its key tiles) is then
 *               split over several workgroups that write fp32 partials
 *               here; reduce kernels add them in a fixed order
 *               (deterministic) and round once.  fa_bwd_workspace_size
 *               gives the bytes needed; when it
 *               is 0, or workspace is NULL, no workspace is used and the
 *               result is that of fa_bwd.  A non-NULL workspace smaller than
 *               needed, misaligned, or overlapping an input or output:
 *               FA_ERR_INVALID_ARG.  Its contents on entry do not matter and
 *               are overwritten.
 * Same arguments, layouts and behaviour as fa_bwd otherwise; the forward
 * that produced o and lse is fa_fwd_ex / fa_fwd_gqa with the same dtype.
 */
int fa_bwd_ex(const void *q, const void *k, const void *v, const void *o,
              const void *dout, const float *lse, float *delta, void *dq,
              void *dk, void *dv, int B, int H, int H_kv, int N, int d,
              float scale, int causal, const int32_t *key_len,
              const uint8_t *block_mask, hipStream_t stream, int dtype,
              void *workspace, size_t workspace_bytes);

/* Workspace bytes fa_bwd_ex may use for this shape (0: none is used, or the
 * shape is invalid).  Independent of dtype and masks: it covers the causal
 * mask, which splits some grids that are not split without it (a call
 * without the causal mask then uses part of the workspace, or none). */
size_t fa_bwd_workspace_size(int B, int H, int H_kv, int N, int d);

/* Query rows (Br) and key rows (Bc) per tile that fa_fwd_ex would use for
 * (dtype, d, block mask given or not, Br, Bc); writes them to *br_out /
 * *bc_out.  Returns FA_OK or FA_ERR_UNSUPPORTED_TILE /
 * FA_ERR_UNSUPPORTED_HEAD_DIM / FA_ERR_NULL_PTR. */
int fa_tile_shape(int dtype, int d, int block_sparse, int Br, int Bc,
                  int *br_out, int *bc_out);

/* Error reporting.  The page "Is Flash Attention Stable?" explainer (aibr.jp,
 * section 6) asks attention libraries to expose their settings and to carry
 * hooks for detecting errors; every entry point above returns a status code,
 * and these two calls explain it. */

/* Static text for a status code; unknown codes give "unknown status".  Never
 * NULL; the string is owned by the library. */
const char *fa_status_string(int status);

/* hipError_t of the most recent FA_ERR_HIP on the calling thread (0 if none).
 * A thread-local value: calls on other threads do not change it. */
int fa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */

/*
 * msa.h -- C ABI of the MI355X (gfx950) MSA sparse-layer decode attention library.
 *
 * Three stages, one call each, in the write-into-output style of the Cacheon
 * "Kernel ABI" page (section "Core rules"): the caller allocates every output
 * (and poisons it), passes arguments in the order below together with the HIP
 * stream to run on, and gets nothing back.  Each call
 *   - writes every logical cell of its outputs, honouring the strides given;
 *   - never writes an input;
 *   - allocates nothing, keeps no pointer after it returns, synchronises
 *     nothing on the host and only enqueues work on `stream`, so it may be
 *     captured into a HIP graph and replayed with new input values at the
 *     same addresses (Cacheon "Slot contract", section "CUDA graph contract");
 *   - returns void.  When an argument is outside the supported domain the call
 *     enqueues nothing (outputs keep their poison) and records an error code
 *     that msa_get_last_error() returns.  A launch failure is recorded the
 *     same way and never retried.
 *
 * Tensors are passed as msa_tensor descriptors: a device pointer to element
 * [0,...,0], a dtype, and per-dimension sizes and strides counted in
 * elements.  The library reads descriptors on the host only.
 *
 * Notation: R request rows, T query tokens per row, N = R*T query tokens
 * (token n = r*T + t), B = 128 tokens per block/page, MB logical blocks per
 * row (block_table width), P physical pages in the pool, Hq/Hkv query/KV
 * heads, D head dim, Di index dim, k top-k width.
 *
 * Visibility (a reading: the pages leave it open): query token n = r*T + t
 * sees key positions [0, V(n)) with V(n) = max(0, seq_lens[r] - (T-1-t)),
 * i.e. the row's T new tokens are already in the cache and are causal among
 * themselves (1 + 3 speculative tokens per row in the vLLM design note
 * "MiniMax-M3 decode through the ATOM kernel library", "Supported
 * experiment").  Logical block j of row r lives in physical page
 * block_table[r][j].
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;   /* same typedef as hip_runtime_api.h */

typedef enum msa_dtype {
    MSA_F32 = 0,
    MSA_BF16 = 1,
    MSA_FP8_E4M3FN = 2,   /* OCP E4M3FN codes, one byte each */
    MSA_I32 = 3
} msa_dtype;

#define MSA_MAX_DIMS 4

typedef struct msa_tensor {
    void *data;                     /* device pointer to element [0,...,0]      */
    int32_t dtype;                  /* msa_dtype                                */
    int32_t ndim;
    int64_t shape[MSA_MAX_DIMS];
    int64_t stride[MSA_MAX_DIMS];   /* in elements; may be any value >= 0       */
} msa_tensor;

typedef enum msa_status {
    MSA_OK = 0,
    MSA_ERR_NULL = 1,          /* a required pointer is NULL                          */
    MSA_ERR_DTYPE = 2,         /* dtype outside the supported set                     */
    MSA_ERR_SHAPE = 3,         /* ndim or sizes disagree between arguments            */
    MSA_ERR_LAYOUT = 4,        /* innermost stride / alignment the kernels need       */
    MSA_ERR_UNSUPPORTED = 5,   /* block size, head dim, group size, k, ... not served */
    MSA_ERR_WORKSPACE = 6,     /* workspace missing or smaller than required          */
    MSA_ERR_ARG = 7,           /* a scalar argument is out of range                   */
    MSA_ERR_LAUNCH = 8,        /* the HIP runtime refused a launch                    */
    MSA_ERR_SCRATCH_LIMIT = 9, /* msa_decode_step_noalloc: sizes need more than its
                                  16 MiB of scratch                                   */
    MSA_ERR_SCRATCH_SETUP = 10 /* msa_decode_step_noalloc: the scratch array's device
                                  address could not be obtained                       */
} msa_status;

/*
 * Stage 1 -- block scores.  Cacheon "Kernel ABI", "Attention block slots",
 * attention.msa_block_score (a per-query block-max score sheet) and
 * attention.msa_prefill_block_score (the same sheet for prefill queries).  The
 * pages leave the score open; this library computes
 *     scores[n][j] = idx_scale * max_{s visible to n, s in block j}
 *                    sum_d q_idx[n][d] * index_k[block_table[r][j]][s - j*B][d]
 * and -inf when block j holds no key visible to token n.  FP8 codes are
 * decoded exactly; products and sums are fp32.
 *
 *   q_idx       [N, Di]     bf16 | f32      innermost stride 1
 *   index_k     [P, B, Di]  fp8e4m3fn | f32 innermost stride 1, rows 16-byte aligned
 *   block_table [R, MB]     i32             any strides
 *   seq_lens    [R]         i32             seq_lens[r] <= MB*B (larger is clamped)
 *   tokens_per_row  T >= 1, N = R*T
 *   block_size  must be 128
 *   idx_scale   > 0, finite (static per-tensor dequantisation scale)
 *   scores      [N, MB]     f32 OUT         any strides; or, with T > 1, [R, MB]:
 *               one row per request (the sheet's per-request form in the
 *               page), scores[r][j] = the max of scores[n][j] over the row's
 *               tokens n; served for rows of up to 16 tokens on the MFMA path
 *               and up to 4 on the vector path
 * Di must be 32, 64 or 128.  A visible block whose physical page id lies
 * outside [0, P) scores NaN (the page is not read).  With bf16 queries, an FP8
 * index and Di in {64, 128} the dot products run on bf16 MFMA tiles (one page
 * per wave for rows of up to 16 tokens, 128-query tiles beyond); otherwise on
 * vector ALUs in fp32.
 */
void msa_block_score(const msa_tensor *q_idx, const msa_tensor *index_k,
                     const msa_tensor *block_table, const msa_tensor *seq_lens,
                     int32_t tokens_per_row, int32_t block_size, float idx_scale,
                     msa_tensor *scores, hipStream_t stream);

/*
 * Stage 2 -- top-k block selection.  Cacheon "Kernel ABI", "Attention block
 * slots" (attention.decode consumes nonnegative block ids, -1 = none;
 * attention.msa_prefill_block_score: unused output cells are -1) and
 * "Correctness is target-owned" (selections are graded as sets, so the order
 * inside a row is free; this library emits ascending block ids).
 * Per score row: candidates are the finite and +inf scores (-inf and NaN are
 * not); the k largest are taken with ties broken toward the lower block id
 * and -0 equal to +0; they are written in ascending block id and the row is
 * padded with -1 when it has fewer than k candidates.  Deterministic.
 *
 *   scores   [N, MB]  f32  any strides, 1 <= MB <= 2048
 *   k        1 <= k <= MB
 *   topk_idx [N, k]   i32 OUT  any strides
 */
void msa_select_topk(const msa_tensor *scores, int32_t k, msa_tensor *topk_idx,
                     hipStream_t stream);

/*
 * Workspace bytes msa_sparse_decode needs for these sizes: split partials plus
 * one arrival counter per (query token, KV head).  Depends on the sizes only,
 * not on the device, the element types or the data.
 */
size_t msa_sparse_decode_workspace_bytes(int32_t rows, int32_t tokens_per_row,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t k);

/*
 * Stage 3 -- sparse attention over the selected pages.  Cacheon "Kernel ABI",
 * "Attention block slots", attention.decode: scaled-dot-product attention of
 * each query over exactly the supplied nonnegative block ids, excluding -1
 * entries and key positions at or beyond its visibility; query head h reads
 * KV head h / (Hq/Hkv) (attention.sdpa).  With static scalar scales (vLLM
 * design note, "Supported experiment"):
 *     logit_s = sm_scale * k_scale * sum_d q[n][h][d] * k_code[s][d]
 *     out[n][h] = v_scale * sum_s softmax(logit)_s * v_code[s]
 * over the visible keys s of the selected blocks; 0 when there is none.
 * Ids outside [0, MB) count as -1; a block whose page id lies outside [0, P)
 * is skipped; duplicate ids in one row count once.
 *
 *   q           [N, Hq, D]      bf16 | f32      innermost stride 1
 *   k_cache     [P, B, Hkv, D]  fp8e4m3fn | bf16 | f32   innermost stride 1, 16-byte
 *                               aligned rows (bf16: the dense cache of attention.decode)
 *   v_cache     [P, B, Hkv, D]  same dtype and shape as k_cache
 *   block_table [R, MB] i32, seq_lens [R] i32   as for msa_block_score
 *   topk_idx    [N, k] i32, shared by all KV heads, or [Hkv, N, k] i32, one
 *               selection per KV head (attention.decode's (Hkv, B, K) layout:
 *               query head h attends the blocks of topk_idx[h / (Hq/Hkv)]);
 *               any strides.  With T > 1 the rows may also be per request
 *               ([R, k] or [Hkv, R, k]): token r*T + t attends row r's blocks,
 *               each token with its own visibility
 *   tokens_per_row  T >= 1
 *   out         [N, Hq, D]      bf16 | f32 OUT  any strides
 *   sm_scale, k_scale, v_scale  finite floats
 *   block_size  must be 128
 *   workspace   device scratch of at least msa_sparse_decode_workspace_bytes(...)
 *               bytes, 256-byte aligned, owned by the caller.  Zero-fill it once
 *               before its first use; every call leaves its counters at zero
 *               again, so the same workspace can be reused (and replayed in a
 *               graph) without clearing.  Calls that share one workspace must
 *               not run concurrently.
 * D must be 64 or 128.  When Hq/Hkv == 16 with bf16 queries and FP8 or bf16
 * caches the QK^T and PV products run on bf16 MFMA tiles (FP8 decoded exactly,
 * P rounded to bf16); otherwise (f32 queries or caches, other head ratios) on
 * vector ALUs in fp32.
 */
void msa_sparse_decode(const msa_tensor *q, const msa_tensor *k_cache,
                       const msa_tensor *v_cache, const msa_tensor *block_table,
                       const msa_tensor *seq_lens, const msa_tensor *topk_idx,
                       int32_t tokens_per_row, msa_tensor *out,
                       float sm_scale, float k_scale, float v_scale, int32_t block_size,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Stages 2 and 3 in one call: msa_select_topk(scores, k, topk_idx), then
 * msa_sparse_decode over that selection, with the same arguments, domain and
 * bit-identical outputs (topk_idx and out are both written).  For callers that
 * hold a score sheet already.  When the attention runs on MFMA (bf16 queries,
 * FP8 caches, Hq/Hkv = 16) and MB <= 128 the selection is not a launch of its
 * own: each attention workgroup selects its token's blocks from the score row
 * with the same wave-level radix select as msa_select_topk, and one of them
 * stores topk_idx; otherwise the top-k kernel runs first.
 *
 *   scores      [N, MB] f32, N = R * tokens_per_row, MB = block_table's width,
 *               or [R, MB] (per request, T > 1)
 *   topk_idx    [N, k] i32 OUT (one selection for all KV heads: one index head),
 *               or [R, k] with a per-request sheet: one selection per request
 *   workspace   as for msa_sparse_decode (same size query, same contract)
 */
void msa_select_sparse_decode(const msa_tensor *scores, int32_t k, msa_tensor *topk_idx,
                              const msa_tensor *q, const msa_tensor *k_cache,
                              const msa_tensor *v_cache, const msa_tensor *block_table,
                              const msa_tensor *seq_lens, int32_t tokens_per_row, msa_tensor *out,
                              float sm_scale, float k_scale, float v_scale, int32_t block_size,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Workspace bytes msa_decode_step needs for these sizes (the same as
 * msa_sparse_decode_workspace_bytes).  Depends on the sizes only.
 */
size_t msa_decode_step_workspace_bytes(int32_t rows, int32_t tokens_per_row,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t k);

/*
 * The three stages in one call: msa_block_score, then msa_select_sparse_decode
 * with width k (msa_select_topk, then msa_sparse_decode), with the same
 * arguments, the same domain and bit-identical outputs (scores, topk_idx and
 * out are all written).
 *
 *   index_k and k_cache/v_cache must have the same pool size P.
 *   scores and topk_idx are both per token ([N, ..]) or both per request
 *   ([R, ..], T > 1: one selection shared by the request's tokens).
 *   workspace   at least msa_decode_step_workspace_bytes(...) bytes, 256-byte
 *               aligned, zero-filled once before first use; every call leaves
 *               its counters at zero again.  Calls sharing a workspace must
 *               not run concurrently.
 */
void msa_decode_step(const msa_tensor *q_idx, const msa_tensor *index_k, const msa_tensor *q,
                     const msa_tensor *k_cache, const msa_tensor *v_cache,
                     const msa_tensor *block_table, const msa_tensor *seq_lens,
                     int32_t tokens_per_row, int32_t k, int32_t block_size,
                     float idx_scale, float sm_scale, float k_scale, float v_scale,
                     msa_tensor *scores, msa_tensor *topk_idx, msa_tensor *out,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * msa_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments (less the workspace),
 * domain and outputs as msa_decode_step, bit-identical to it.
 *
 * The step's scratch (split partials and arrival counters) lives in a 16 MiB
 * device array inside the library, one per GPU, held until the process ends.
 * A call whose split plan needs more (with 16 query heads of dim 128: more
 * than about 1950 query tokens, 8 KiB of partials each; at most 2048 query
 * tokens x KV heads) is rejected with MSA_ERR_SCRATCH_LIMIT before anything
 * is enqueued.  The first call on a device
 * looks the array's address up and enqueues a kernel that zero-fills it on
 * `stream`; every call leaves its counters at zero again.  Nothing here calls
 * hipMalloc, hipFree or an allocating library routine.  All calls on one GPU
 * share the array: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialised by the caller.
 */
void msa_decode_step_noalloc(const msa_tensor *q_idx, const msa_tensor *index_k, const msa_tensor *q,
                             const msa_tensor *k_cache, const msa_tensor *v_cache,
                             const msa_tensor *block_table, const msa_tensor *seq_lens,
                             int32_t tokens_per_row, int32_t k, int32_t block_size,
                             float idx_scale, float sm_scale, float k_scale, float v_scale,
                             msa_tensor *scores, msa_tensor *topk_idx, msa_tensor *out,
                             hipStream_t stream);

/*
 * Workspace bytes msa_prefill_block_score needs: one arrival counter per
 * output row, the owner of every query-block row and the query-block score
 * sheet [num_q_heads, all_seqblock_q, parts, max_blocks] f32, parts = 1
 * unless block_size_q > 512.  Depends on these sizes only; 0 for sizes out of
 * range.
 */
size_t msa_prefill_block_score_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                               int32_t all_seqblock_q, int32_t max_blocks,
                                               int32_t block_size_q);

/*
 * Ragged prefill score-to-selection in one call.  Cacheon "Kernel ABI",
 * "Attention block slots", attention.msa_prefill_block_score (the V2 call:
 * score production and selection for the whole ragged batch, out_topk written
 * once, unused cells -1; indices are logical block ids within the request).
 *
 * Request b owns the query tokens [cu_seqlens[b], cu_seqlens[b+1]) of q (its
 * new tokens, in order) and the query-block rows [cu_seqblocks_q[b],
 * cu_seqblocks_q[b+1]) of out_topk, one per block_size_q new tokens
 * (ceil(new tokens / block_size_q) rows).  Its logical key sequence has
 * seq_lens[b] keys; logical block j lives in page block_table[slot_ids[b]][j].
 * For query head h and query block qb of request b (readings where the pages
 * leave it open):
 *   V      = min(seq_lens[b], prefix_lens[b] + qb * block_size_q)  keys visible
 *   ncand  = ceil(V / 128)     candidate blocks 0 .. ncand-1
 *   score_j = scale * max over the block's new tokens t and the keys s < V of
 *             block j of sum_d q[t][h][d] * index_k[page(j)][s - 128 j][d]
 *   forced = blocks j < init_blocks or j >= ncand - local_blocks
 *   out_topk[h][cu_seqblocks_q[b] + qb] = the forced blocks (lower ids first,
 *             at most topk), then the other candidates by score (ties to the
 *             lower id), up to topk in all; ascending ids, padded with -1.
 * Rows of out_topk that no request owns are all -1.  FP8 codes are decoded
 * exactly, products run on bf16 MFMA tiles with fp32 sums.  With MB <= 128
 * and at most 32 rows per work group (query blocks of at least 16 tokens x
 * heads) the selection runs inside the scoring launch; otherwise a selection
 * launch follows it.
 *
 *   q              [total_q, Hq, Di]  bf16   innermost stride 1, 16-byte aligned rows
 *   index_k        [P, 128, Di]       fp8e4m3fn  one index head; rows 16-byte aligned
 *   block_table    [slots, MB] i32    any strides, 1 <= MB <= 2048
 *   slot_ids, seq_lens, prefix_lens   [batch] i32 (seq_lens[b] <= MB*128)
 *   cu_seqlens, cu_seqblocks_q        [batch+1] i32, non-decreasing from 0
 *   block_size_q >= 1; block_size_k must be 128; topk >= 1;
 *   init_blocks, local_blocks >= 0; scale > 0, finite
 *   out_topk       [Hq, all_seqblock_q, topk] i32 OUT  any strides;
 *                  all_seqblock_q >= cu_seqblocks_q[batch]
 *   workspace      at least msa_prefill_block_score_workspace_bytes(batch, Hq,
 *                  all_seqblock_q, MB, block_size_q) bytes, 256-byte aligned,
 *                  owned by the caller.  Zero-fill it once before its first
 *                  use; every call leaves its counters at zero again, so it is
 *                  reused (and graph-replayed) without clearing.  Calls sharing
 *                  a workspace must not run concurrently.
 * Di must be 64 or 128; batch at most 8192.  The page-size and length hints
 * of the pages' signature (max_seqlen_q/k, max_seqblock_q) are not needed:
 * the call plans its work on the device.  Inputs outside this contract
 * (inconsistent offsets, page ids outside [0, P), NaN dot products) never
 * cause an access outside the given tensors, but their rows are unspecified.
 */
void msa_prefill_block_score(const msa_tensor *q, const msa_tensor *index_k,
                             const msa_tensor *block_table, const msa_tensor *slot_ids,
                             const msa_tensor *cu_seqlens, const msa_tensor *seq_lens,
                             const msa_tensor *prefix_lens, int32_t block_size_q,
                             int32_t block_size_k, int32_t topk, int32_t init_blocks,
                             int32_t local_blocks, float scale, const msa_tensor *cu_seqblocks_q,
                             msa_tensor *out_topk, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Error code recorded by the most recent failing call on this thread, then
 * reset to MSA_OK.  Returns MSA_OK when no call failed since the last read. */
int32_t msa_get_last_error(void);

/* Static description of an msa_status code (never NULL). */
const char *msa_error_string(int32_t code);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */

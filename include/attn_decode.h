/*
 * attn_decode.h -- C ABI of the split-KV decode / small-query attention
 * library for MI355X (gfx950).
 *
 * What the library computes (for each batch b, query position i, query head
 * hq, with KV head h = hq / G, G = Hq / Hkv, and the L valid keys of b):
 *
 *     O[b,i,hq,:] = sum_j softmax_j(scale * q . k_j) v_j
 *     LSE[b,hq,i] = ln sum_j exp(scale * q . k_j)
 *
 * This is the attention definition of the "SmallQ FlashAttention (Vector)"
 * README (section 接口) with the grouped-query sharing of the lpnh.cn
 * "pack_gqa 与 num_splits" article; the default scale is 1/sqrt(head_dim).
 * It is evaluated with online softmax (ai6s.net FlashAttention article,
 * section "FlashAttention 的数学细节"), over num_splits KV ranges whose
 * partial outputs and logsumexps are merged at the end (lpnh.cn article,
 * section "两个开关在 kernel 层面各做了什么").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers to tensors are DEVICE pointers owned by the caller.  The
 *   library never allocates, frees or keeps them; it keeps no state between
 *   calls except the thread-local record read by attn_last_plan() and the
 *   per-GPU scratch array of attn_decode_fwd_noalloc() (with its device
 *   address, looked up once per GPU).
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Work is enqueued on it and the call returns without waiting.
 * - All arguments are validated on the host before anything is enqueued.
 *   On any error nothing is launched and no output byte is written.
 * - Device-side data (block_table entries, cache_seqlens values) is the
 *   caller's contract: every block_table entry a sequence uses must name a
 *   page < num_pages, and 0 <= cache_seqlens[b] (+ new_len where keys are
 *   appended) <= max_seqlen_k.  Use attn_check_paged_inputs() on host
 *   copies to verify it in tests.  A length over max_seqlen_k gives wrong
 *   results (keys past the plan's last split are not attended) but leaves
 *   the workspace's arrival counters intact for later calls.
 * - Element types: q, k, v and out share one 16-bit type (ATTN_FP16 or
 *   ATTN_BF16); lse is float32.  Accumulation is float32 throughout.
 * - An empty sequence (L = 0) gives O = 0 and LSE = -inf.
 * - Tensors must be contiguous in the layouts stated below, 16-byte
 *   aligned for q/k/v/out and 4-byte aligned for lse, block_table and
 *   cache_seqlens; workspace must be 256-byte aligned.
 */
#ifndef ATTN_DECODE_H
#define ATTN_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 7

/* Status of every call.  Invalid parameters are refused with an error code
 * before any work is enqueued, as the MixedQuantSparseFlashMlaMetadata
 * article's two-phase API does (section 调用方式: ACLNN_ERR_PARAM_INVALID),
 * and a shape or feature outside the supported envelope is an explicit
 * error, never a silent fallback to another path (MXFlashAttn page,
 * sections 前向算子 API and 能力矩阵). */
typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL                     */
    ATTN_ERR_SHAPE = 2,       /* sizes are inconsistent (<= 0, Hq % Hkv != 0,   */
                              /* max_seqlen_k > max_pages_per_seq * page_size)  */
    ATTN_ERR_UNSUPPORTED = 3, /* valid, but outside the supported envelope      */
    ATTN_ERR_ARG = 4,         /* num_splits / pack_gqa / scale out of range     */
    ATTN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than plan requires   */
    ATTN_ERR_ALIGN = 6,       /* a pointer breaks the alignment rule            */
    ATTN_ERR_HIP = 7,         /* the HIP runtime reported an error              */
    ATTN_ERR_DATA = 8         /* attn_check_paged_inputs found a bad entry      */
} attn_status;

typedef enum { ATTN_FP16 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Paged decode problem.
 *   q, out        [batch, q_len, num_heads_q, head_dim]
 *   k_cache,
 *   v_cache       [num_pages, page_size, num_heads_kv, head_dim]
 *                 (block, token-in-block, head, dim: the PA_BBND layout of
 *                 the MixedQuantSparseFlashMlaMetadata article, section
 *                 参数说明)
 *   block_table   int32 [batch, max_pages_per_seq]; key j of sequence b is
 *                 slot j % page_size of page block_table[b][j / page_size]
 *   cache_seqlens int32 [batch], number of valid keys of each sequence
 *   lse           float32 [batch, num_heads_q, q_len]
 * Supported: head_dim 1..256; page_size a multiple of 16; q_len >= 1 (no
 * causal mask: every query row sees all L keys); any G = Hq / Hkv.  Head
 * dims are padded inside the kernel to 32, 64, 128 or 256; multiples of 8
 * move K/V in 16-byte loads, other head dims element by element (slower). */
typedef struct {
    int32_t batch;
    int32_t q_len;
    int32_t num_heads_q;
    int32_t num_heads_kv;
    int32_t head_dim;
    int32_t page_size;
    int32_t max_pages_per_seq;
    int32_t max_seqlen_k;  /* upper bound of cache_seqlens; drives the plan   */
    int32_t dtype;         /* attn_dtype                                       */
    int64_t sum_seqlen_k;  /* optional: sum of cache_seqlens (0 = not given).
                            * With it, an automatic plan (num_splits 0) also
                            * splits a ragged batch (max_seqlen_k over twice
                            * the mean length) whose longest sequence exceeds
                            * one and a half compute units' fair shares of
                            * all keys, into pieces of at most three fifths of
                            * a share (an
                            * addition to the pages' rule), raises a split
                            * count above 1 that leaves compute units idle
                            * until the workgroups fill them (another
                            * addition), and a split call
                            * may launch the compact list (see
                            * attn_plan.extra_blocks) instead of every
                            * (unit, split) pair, and a head-dim-64 or -32
                            * call may read 2 or 4 KV heads per unit
                            * (attn_plan.heads_per_row).  0 <= sum <= batch *
                            * max_seqlen_k, else ATTN_ERR_SHAPE; a wrong but
                            * in-range value changes only speed. */
} attn_decode_shape;

/* Dense small-query problem (the SmallQ README's [heads, qLen, headDim]
 * layout, with num_heads_kv <= num_heads_q sharing as above).
 *   q, out  [num_heads_q, q_len, head_dim]
 *   k, v    [num_heads_kv, kv_len, head_dim]
 *   lse     float32 [num_heads_q, q_len]
 * Supported: head_dim 1..256 (the SmallQ README's "any headDim", section
 * 任意 headDim 支持, up to this cap); any kv_len >= 0; q_len >= 1. */
typedef struct {
    int32_t num_heads_q;
    int32_t num_heads_kv;
    int32_t q_len;
    int32_t kv_len;
    int32_t head_dim;
    int32_t dtype;
} attn_dense_shape;

/* What a call runs.  Filled by the plan functions and recorded by every
 * forward call (see attn_last_plan). */
typedef struct {
    int32_t num_splits;      /* S: KV ranges per (sequence, head unit)        */
    int32_t pack_gqa;        /* 1: the G query heads of a KV head share a unit */
    int32_t rows_per_unit;   /* query rows per unit: q_len*G packed, q_len not */
                             /* (head groups of R KV heads: q_len*R*G)         */
    int32_t rows_per_block;  /* packed rows one workgroup carries: 16; at      */
                             /* head_dim 64 or 128, 32 for units of 17..32     */
                             /* rows and 64 beyond (KV read once per block)    */
    int32_t row_blocks;      /* ceil(rows_per_unit / rows_per_block)           */
    int32_t units;           /* batch * head units * row_blocks; a head unit  */
                             /* is a KV head (packed), a query head, or a     */
                             /* group of KV heads (heads_per_row > 1)          */
    int32_t grid;            /* workgroups of the split kernel: units * S, or */
                             /* units + extra_blocks with the compact list    */
    int32_t split_granule;   /* split lengths are multiples of this many keys  */
    int32_t num_cus;         /* compute units the plan was made for           */
    int32_t combine;         /* how S > 1 partials are merged: 0 none (S = 1), */
                             /* 2 inside the split kernel by the last split to */
                             /* finish (1, a separate launch, is not used)     */
    int32_t kernel;          /* diagnostic: 10000 (16-byte loads), 20000      */
                             /* (16-byte loads, head_dim a multiple of 8 below */
                             /* the tile's), 30000 (element loads) or 40000    */
                             /* (head groups) + 1000 if paged + tile head dim */
                             /* (32, 64, 128 or 256); + 100000 in the record  */
                             /* of a kvcache call whose split kernel wrote    */
                             /* the new keys itself (no separate append)      */
    int32_t split_keys;      /* C: split s covers keys [s*C, (s+1)*C) of every */
                             /* sequence, C = 16*ceil(ceil(max_seqlen_k/16)/S) */
    int32_t heads_per_row;   /* KV heads per unit: 1, or R = 2 (head_dim 64) */
                             /* or 4 (head_dim 32) when the call is paged,    */
                             /* num_heads_kv is a multiple of R, packed (G = 1 */
                             /* counts as packed unless pack_gqa is 0),        */
                             /* q_len * R * G <= 16 and sum_seqlen_k is       */
                             /* given: the R adjacent KV heads are read as    */
                             /* one 128-wide key row (the cache puts them     */
                             /* side by side), with all R heads' query rows;  */
                             /* units, rows_per_unit and the split rule then  */
                             /* count these head groups                       */
    int32_t extra_blocks;    /* 0: the grid is split-major, every (unit,      */
                             /* split) pair has a workgroup (empty splits     */
                             /* return at once).  > 0 (paged, S > 1, length   */
                             /* sum given, batch <= 1024, and a smaller grid): */
                             /* a compact list: extra_blocks workgroups take  */
                             /* the splits 1.. of the sequences that need     */
                             /* them (listed on the device from the lengths), */
                             /* then one workgroup per unit runs split 0.     */
                             /* extra_blocks = max(1, floor(sum_seqlen_k / C) */
                             /* x head units x row_blocks), enough for one    */
                             /* item each when the sum is right; with a wrong */
                             /* sum they loop over the items (same results).  */
    int64_t workspace_bytes; /* bytes of workspace the forward call needs     */
} attn_plan;

/* Plan a paged decode call without touching any device.
 *   num_splits: 0 = choose by rule, >= 1 = use this value (<= 1024).
 *   pack_gqa:  -1 = choose by rule, 0 = off, 1 = on (forced on when S > 1).
 *   num_cus:    compute units to plan for; 0 = 256 (one MI355X).  A caller
 *               that counts workgroup slots instead passes compute units x
 *               resident workgroups here and the plan's num_splits to the
 *               forward call (the forward calls plan with the device's
 *               compute units).
 * The rules are the lpnh.cn article's (section "pack_gqa 怎么选": row
 * efficiency with a 0.9 margin; section "num_splits 怎么选": one split when
 * the units reach 80% of the compute units or the KV spans at most 4 tiles
 * of 128 keys, else the smallest split count whose last-wave efficiency is
 * within 85% of the best), taken over compute units with an M tile of 16. */
attn_status attn_decode_plan(const attn_decode_shape* shape, int num_splits, int pack_gqa,
                             int num_cus, attn_plan* plan);

/* Paged decode forward (layouts above).
 *   softmax_scale <= 0 selects 1/sqrt(head_dim).
 *   lse may be NULL (not written).
 *   workspace / workspace_bytes: device scratch of at least
 *     plan.workspace_bytes (0 when S = 1, then workspace may be NULL).
 *     Layout: float32 partial outputs [S][rows][head_dim], then (at the
 *     next 256-byte boundary) float32 partial LSEs [S][rows], rows ordered
 *     (b, i, hq), then (next 256-byte boundary) int32 arrival counters
 *     [plan.units], one per 128-byte line (32 int32 apart, so the atomics
 *     of different units never share a line).  The counters must be zero
 *     before the first call that
 *     uses the workspace (fill it with zeros once); every call leaves them
 *     zero again.  Calls that share one workspace must not run concurrently.
 *     Only the partials of splits that hold keys of a sequence spanning two
 *     or more splits are written (an empty split adds nothing to the merge;
 *     a sequence within one split is written to out directly); the other
 *     entries keep whatever they held.
 * The plan uses the compute-unit count of the current device. */
attn_status attn_decode_fwd(const attn_decode_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* cache_seqlens, int num_splits, int pack_gqa,
                            float softmax_scale, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/* attn_decode_fwd for callers that cannot allocate or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, layouts, results and errors as
 * attn_decode_fwd, without workspace / workspace_bytes: a split call keeps
 * its partials and arrival counters in a scratch array the library holds in
 * each GPU's memory (16 MiB per GPU, from the first use of the library on
 * that GPU until the process ends).  The call allocates nothing.
 *   Limit: a plan (attn_decode_plan with the same shape and options) needs
 *   the scratch only when num_splits > 1; then it must fit: units * 128
 *   bytes of counters <= 512 KiB, and the partials (num_splits * rows *
 *   head_dim * 4 bytes, then num_splits * rows * 4 bytes, each rounded up to
 *   256 bytes; rows = batch * q_len * num_heads_q) <= 15.5 MiB.  A larger
 *   call returns ATTN_ERR_WORKSPACE and launches nothing.
 *   Every call on a GPU shares that GPU's scratch, which keeps the last
 *   call's partials; calls that overlap on one GPU (other streams or host
 *   threads) race and must be ordered by the caller.  The kernel leaves the
 *   counters at zero after every call.
 *   ATTN_ERR_HIP also when the scratch's device address cannot be found. */
attn_status attn_decode_fwd_noalloc(const attn_decode_shape* shape, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* cache_seqlens,
                                    int num_splits, int pack_gqa, float softmax_scale, void* out,
                                    float* lse, void* stream);

/* Paged decode forward with the options of the flash_attn_with_kvcache call
 * in the lpnh.cn article (section "num_splits 怎么选"): keys appended to the
 * cache in the same call, and a causal mask for q_len > 1 (speculative /
 * MTP verification).  Other arguments as in attn_decode_fwd, which is this
 * call with new_len = 0 and causal = 0.
 *   k_new, v_new  [batch, new_len, num_heads_kv, head_dim], 16-byte aligned;
 *                 may be NULL when new_len == 0.
 *   new_len       keys appended per sequence (>= 0).  They are written to
 *                 key positions cache_seqlens[b] .. cache_seqlens[b] +
 *                 new_len - 1 of k_cache / v_cache (the block table must map
 *                 those pages), then attention covers L_b = cache_seqlens[b]
 *                 + new_len keys.  cache_seqlens itself is not changed.
 *                 shape->max_seqlen_k must bound every L_b.  With at most
 *                 4 new keys per sequence on the kernels whose tiles go
 *                 straight to LDS (head_dim a multiple of 8 from 40 to
 *                 256, or head groups) and no varlen queries, the
 *                 attention kernel writes them itself and reads them from
 *                 k_new / v_new (one launch; the record of attn_last_plan
 *                 then has kernel + 100000), unless that would lower the
 *                 workgroups resident per CU of a grid larger than one
 *                 round; otherwise an append kernel runs first.  Either
 *                 way the cache ends the same, and keys past the block
 *                 table are not written.
 *   causal        0: every query row sees all L_b keys.  1: query i of q_len
 *                 sees keys j <= L_b - q_len + i (the queries are the last
 *                 q_len positions: bottom-right alignment); a row that sees
 *                 no key gets O = 0 and LSE = -inf.
 * Errors: new_len < 0 or causal not 0/1 -> ATTN_ERR_ARG; new_len > 0 with a
 * NULL k_new/v_new -> ATTN_ERR_NULL. */
attn_status attn_decode_kvcache_fwd(const attn_decode_shape* shape, const void* q, void* k_cache,
                                    void* v_cache, const int32_t* block_table,
                                    const int32_t* cache_seqlens, const void* k_new,
                                    const void* v_new, int new_len, int causal, int num_splits,
                                    int pack_gqa, float softmax_scale, void* out, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Paged decode forward with a different query count per sequence (varlen
 * Q, the cu_seqlens input of the lpnh.cn article's section "pack_gqa 怎么选",
 * which always packs the query heads of a KV head).
 *   q, out        [total_q, num_heads_q, head_dim]: the queries of sequence b
 *                 are rows cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1
 *   cu_seqlens_q  int32 [batch + 1], cu_seqlens_q[0] = 0, non-decreasing,
 *                 cu_seqlens_q[batch] = total_q, every difference <=
 *                 shape->q_len (shape->q_len is the largest query count)
 *   lse           float32 [num_heads_q, total_q], may be NULL
 *   causal        as in attn_decode_kvcache_fwd, with each sequence's own
 *                 query count
 * Other arguments as in attn_decode_kvcache_fwd; pack_gqa is always on, so
 * the plan (and workspace size) is attn_decode_plan's with pack_gqa = 1.
 * Errors: total_q > batch * q_len -> ATTN_ERR_SHAPE; cu_seqlens_q NULL ->
 * ATTN_ERR_NULL.  cu_seqlens_q's values are the caller's contract, like
 * cache_seqlens. */
attn_status attn_decode_varlen_fwd(const attn_decode_shape* shape, const void* q, void* k_cache,
                                   void* v_cache, const int32_t* block_table,
                                   const int32_t* cache_seqlens, const int32_t* cu_seqlens_q,
                                   int total_q, const void* k_new, const void* v_new, int new_len,
                                   int causal, int num_splits, float softmax_scale, void* out,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Plan a dense call (num_splits as above, by the same lpnh.cn rules; always
 * packed).  The dense problem is the SmallQ README's (section 接口), which
 * walks each head's keys in blocks on one core (section 支持范围); with few
 * heads that would leave most compute units idle, so the key range is also
 * split here, as for paged calls (an addition to the README). */
attn_status attn_dense_plan(const attn_dense_shape* shape, int num_splits, int num_cus,
                            attn_plan* plan);

/* Dense small-query forward: the SmallQ README's call (section 接口:
 * query [heads, qLen, headDim] against key/value [heads, kvLen, headDim],
 * any kvLen and head dim, section 任意 headDim 支持).  Layouts above; other
 * arguments as in attn_decode_fwd; partial rows ordered (hq, i). */
attn_status attn_dense_fwd(const attn_dense_shape* shape, const void* q, const void* k,
                           const void* v, int num_splits, float softmax_scale, void* out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Merge S partials into the final output: the combine step on its own, the
 * reduction of the per-split outputs by their logsumexps that the lpnh.cn
 * article describes for num_splits > 1 (section 两个开关在 kernel 层面各做了
 * 什么), written here as the max-shifted log-sum-exp merge.
 *   o_part   float32 [num_splits][rows][head_dim], rows = batch*q_len*num_heads
 *            ordered (b, i, h); lse_part float32 [num_splits][rows]
 *            (natural log; -inf marks an empty partial).
 *   out      16-bit [batch, q_len, num_heads, head_dim]
 *   lse      float32 [batch, num_heads, q_len], may be NULL.
 * Per row: M = max_s LSE_s, w_s = exp(LSE_s - M), O = sum w_s O_s / sum w_s,
 * LSE = M + ln sum w_s; all partials empty gives O = 0, LSE = -inf.
 * head_dim: any value in [1, 512]. */
attn_status attn_combine_fwd(int num_splits, int batch, int q_len, int num_heads, int head_dim,
                             int dtype, const float* o_part, const float* lse_part, void* out,
                             float* lse, void* stream);

/* Host check of the device-data contract of the paged layout (block
 * table and lengths of the PA_BBND cache, MixedQuantSparseFlashMlaMetadata
 * article, section 参数说明), with an explicit error code for a bad entry
 * (section 调用方式), on host copies of block_table
 * [batch, max_pages_per_seq] and cache_seqlens [batch]: every used entry in
 * [0, num_pages) and 0 <= L <= max_seqlen_k.  Returns ATTN_ERR_DATA and the
 * first offending sequence in *bad_batch (may be NULL) on failure. */
attn_status attn_check_paged_inputs(const attn_decode_shape* shape,
                                    const int32_t* block_table_host,
                                    const int32_t* cache_seqlens_host, int64_t num_pages,
                                    int32_t* bad_batch);

/* The same host check for an attn_decode_kvcache_fwd call that appends
 * new_len keys per sequence (the paged KV append of the MXFlashAttn page,
 * section 能力矩阵): every sequence's cache_seqlens[b] + new_len keys must
 * be <= max_seqlen_k and mapped by block-table entries in [0, num_pages).
 * A call that breaks this bound loses the keys past its last split.
 * new_len < 0 -> ATTN_ERR_ARG; otherwise as attn_check_paged_inputs, which
 * is this check with new_len = 0. */
attn_status attn_check_kvcache_inputs(const attn_decode_shape* shape,
                                      const int32_t* block_table_host,
                                      const int32_t* cache_seqlens_host, int64_t num_pages,
                                      int new_len, int32_t* bad_batch);

/* Plan recorded by the last successful forward call on this thread
 * (ATTN_ERR_ARG if none yet): which kernel ran, with what split count,
 * packing and grid.  This is the dispatch record the MXFlashAttn page asks
 * callers to check (section 前向算子 API, get_last_dispatch_info(), and
 * section 已知限制: assert which kernel actually ran). */
attn_status attn_last_plan(attn_plan* plan);

/* Static text for a status code (the explicit errors of the MXFlashAttn
 * page, section 前向算子 API, readable in logs). */
const char* attn_status_str(attn_status status);

/* ATTN_ABI_VERSION of the built library (this library's own compatibility
 * check; no page defines it). */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DECODE_H */

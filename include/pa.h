/*
 * pa.h -- C ABI of the MI355X (gfx950) paged split-KV decode library (libpa.so).
 *
 * One decode step is three asynchronous calls on one HIP stream:
 *
 *   pa_plan    length-proportional work planner: splits every request's KV range into a number of
 *              partitions proportional to its context length, under a workgroup budget of
 *              budget_mult x CU and a per-request ceiling (ROCm/ATOM PR #2366 "Route the paged decode
 *              to aiter's FlyDSL kernel with work planner", sections 1 and 3; ROCm/ATOM PR #2514
 *              "adapt the FlyDSL paged decode to aiter #5809 (explicit work plans)", Design).
 *   pa_decode  split-KV grouped-query decode over a block-table KV cache: one partial softmax state per
 *              (plan slot, query token, query head).  Query token i of a request with L query tokens
 *              and KV length S sees keys [0, n), n = S - (L - 1 - i), or with a sliding window of W
 *              keys [max(0, n - W), n): the window applies per token (opengfx1030/vllm-rdna PR #29,
 *              Change 1).
 *   pa_merge   log-sum-exp merge of a request's partials into the output rows; rows past the last
 *              cumulative query length and rows with no visible key are written as exact zeros
 *              (same vllm-rdna page, Change 1; ATOM #2366 review, "Claims checked and not upheld").
 *
 * pa_attention runs the same three steps with one launch fewer: the decode plans in place (for
 * batches of up to PA_INLINE_PLAN_SEQS requests) and stores the plan it used.  pa_prefill computes
 * prompt rows of a mixed batch (their query blocks planned, decoded and merged like requests), and
 * pa_attention_mixed a whole decodes-first mixed batch, the decodes and the prompts sharing one launch
 * where they fit it.
 *
 * Conventions shared by every entry point:
 *   - All array arguments are DEVICE pointers (memory of the current HIP device), except where a
 *     parameter says host.  The caller owns all memory; the library allocates nothing, keeps no
 *     global state, never synchronises and never copies device to host.  Every call is stream-ordered
 *     and may be captured in a HIP graph.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Integer arrays are int32, contiguous.  Floating arrays are contiguous, innermost dimension last.
 *   - Alignment: q, k_cache, v_cache, out and work_info 16 bytes; reduce_info and num_work 8 bytes;
 *     workspace 256 bytes (PA_INVALID_ARG otherwise).
 *   - Storage types: PA_F32 (IEEE binary32), PA_BF16 (bfloat16), PA_FP8_E4M3 (OCP E4M3 "fn" codes,
 *     dequantised value = decoded code x per-tensor scale).
 *   - Host-side argument checks run before any launch; a failing check returns a nonzero status and
 *     launches nothing.  Device-side preconditions (in-range block ids for every key below S, query
 *     lengths <= max_q_len, non-decreasing cumulative lengths, num_rows >= last cumulative length,
 *     non-negative context lengths) cannot be checked without a synchronisation; kernels clamp their
 *     indexing so a violation gives unspecified values in the affected rows but no out-of-bounds access.
 *
 * Memory layouts:
 *   q, out         [num_rows, num_q_heads, head_dim]
 *   k_cache,       [num_blocks, num_kv_heads, block_size, head_dim]   (one page = block_size tokens)
 *   v_cache
 *   block_tables   [num_seqs, max_blocks_per_seq]   page ids; entries past a request's last page unused
 *   context_lens   [num_seqs]                       S_b, the request's KV length (query tokens included)
 *   cu_query_lens  [num_seqs + 1] or NULL           cumulative query lengths; NULL = one row per request
 *   work_info      [capacity, 4]  (request, tile_begin, tile_end, S_b); unused slots (-1, 0, 0, 0)
 *   reduce_info    [num_seqs, 2]  (first_slot, num_partitions)
 *   num_work       [2]            (number of used slots, tiles in the largest slot); 8-byte aligned
 *   workspace      pa_workspace_bytes(...) bytes: fp32 partials written by pa_decode and read by
 *                  pa_merge
 *
 * Query head h reads kv head h / (num_q_heads / num_kv_heads).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_F32 = 0,
    PA_BF16 = 1,
    PA_FP8_E4M3 = 2
} pa_dtype;

typedef enum {
    PA_OK = 0,
    PA_INVALID_ARG = 1,   /* null pointer, negative size, inconsistent shapes or dtypes */
    PA_UNSUPPORTED = 2,   /* valid but outside what the kernels implement (head_dim, block size, ...) */
    PA_CAPACITY = 3,      /* plan capacity or workspace smaller than the call needs */
    PA_HIP_ERROR = 4      /* a HIP runtime call or kernel launch failed */
} pa_status;

/* Limits of this implementation (checked on the host). */
#define PA_MAX_SEQS 8192           /* pa_plan keeps per-request prefix sums in LDS */
#define PA_MAX_GROUP_ROWS 64       /* (num_q_heads / num_kv_heads) x max_q_len */
#define PA_INLINE_PLAN_SEQS 256    /* largest batch pa_attention plans inside the decode launch */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)   /* the device array behind pa_attention_noalloc */

/*
 * Number of plan slots a batch needs:
 *   min(num_seqs x max_partitions, max(num_seqs, ceil(budget_mult x cu_count / num_kv_heads)))
 * (ATOM #2366 review item 3).  Pure host arithmetic; no device access.
 * Returns PA_INVALID_ARG for num_seqs < 0, any other argument < 1, or a null capacity_out.
 */
pa_status pa_plan_capacity(int32_t num_seqs, int32_t num_kv_heads, int32_t cu_count,
                           int32_t budget_mult, int32_t max_partitions, int32_t* capacity_out);

/*
 * Bytes of workspace pa_decode, pa_merge and pa_attention use for a plan of `capacity` slots, in
 * this order, each region 256-byte aligned:
 *   fp32 partial outputs [capacity, max_q_len, num_q_heads, head_dim] and fp32 (max, sum) pairs
 *   [capacity, max_q_len, num_q_heads, 2];
 *   then (capacity > 0) the shared-slot region, used when every request is one slot (see
 *   pa_decode): partials and pairs as above for 3 x capacity pieces, then int32 (first piece,
 *   pieces) pairs [PA_INLINE_PLAN_SEQS].  A workspace without this region (workspace_bytes short of
 *   it) works, without shared slots.
 * Returns 0 if any argument is < 1 (capacity may be 0) or the size overflows.
 */
size_t pa_workspace_bytes(int32_t capacity, int32_t max_q_len, int32_t num_q_heads, int32_t head_dim);

/*
 * Build the work plan on the device from context_lens (device, [num_seqs]).
 *   cu_query_lens   [num_seqs + 1] or NULL; read only with a sliding window (query lengths L_b)
 *   tile_tokens     partition granularity in tokens (256 in the pages' deployment)
 *   sliding_window  0 = none; W > 0: the plan covers only the keys the decode reads under a window
 *                   of W keys per query token (ROCm/ATOM PR #2366 review: plan and kernel must agree
 *                   on the window)
 *   capacity        length of work_info; must be >= pa_plan_capacity(...) for the same arguments
 * Request b reads keys [lo_b, S_b): lo_b = 0 without a window, else max(0, S_b - (L_b - 1) - W).
 * Its tiles are those the range touches, [t0_b, t1_b) = [floor(lo_b / T), ceil(S_b / T)), and its
 * length E_b = S_b - lo_b.  Apportionment: every request with E_b > 0 gets
 *   min(max_partitions, t1_b - t0_b, 1 + floor((C - B') E_b / W))
 * partitions, C = the capacity formula, B' = number of requests with E_b > 0, W = sum E_b (64-bit);
 * the others get none.  Partition j of request b covers tiles
 * t0_b + [floor(j tiles_b / parts_b), floor((j + 1) tiles_b / parts_b)), tiles_b = t1_b - t0_b.
 * Without a window this is the plain rule over [0, S_b).  Every slot of work_info is
 * rewritten (unused ones to (-1, 0, 0, 0)), so a plan never carries data from an earlier call.
 * num_work receives the number of used slots and the tile count of the largest slot.
 * dispatch_info (nullable, [capacity, 4], 16-byte aligned) receives, besides the plan, an order in
 * which pa_decode can run the slots: the slots ranked by tile count (largest first, ties by slot
 * index, unused slots last), rank r at position r when r < half = ceil(capacity / 2) and at position
 * capacity + half - 1 - r otherwise, each entry (request, tile_begin, tile_end, slot).  Positions p
 * and p + half hold ranks p and capacity - 1 - p, so where two workgroups share a compute unit a large
 * slot pairs with a small one.  This is this library's scheduling, not part of the plan; plans of
 * more than 1024 slots get the identity order.
 * Negative S_b (a precondition violation) are planned as 0.
 * Errors: PA_INVALID_ARG (null pointers, num_seqs < 0, arguments < 1), PA_UNSUPPORTED
 * (num_seqs > PA_MAX_SEQS), PA_CAPACITY (capacity too small), PA_HIP_ERROR (launch failure).
 */
pa_status pa_plan(const int32_t* context_lens, const int32_t* cu_query_lens, int32_t num_seqs,
                  int32_t num_kv_heads, int32_t cu_count, int32_t budget_mult, int32_t max_partitions,
                  int32_t tile_tokens, int32_t sliding_window, int32_t capacity, int32_t* work_info,
                  int32_t* reduce_info, int32_t* num_work, int32_t* dispatch_info, void* stream);

/*
 * Split-KV decode: for every used plan slot w = (b, tile_begin, tile_end, .) and kv head g, one
 * workgroup computes, for each query token i of request b and each query head h of group g, the
 * softmax state of the keys [tile_begin x T, min(tile_end x T, S_b)) intersected with the token's
 * visible range [lo_i, n_i), n_i = S_b - (L_b - 1 - i), lo_i = 0 or, with a window, max(0, n_i - W):
 *   m = max score, l = sum exp(score - m), acc = sum exp(score - m) v,   score = scale x k_scale x (q . k)
 * (V is multiplied by v_scale), stored unnormalised in the workspace; a slot/token with no visible
 * key stores l = 0, acc = 0.  S_b is context_lens[b]; the plan must have been built from the same
 * lengths (a stale plan covers the wrong key ranges).
 * Arguments:
 *   q, q_dtype                 [num_rows, num_q_heads, head_dim], PA_F32 or PA_BF16
 *   k_cache, v_cache, kv_dtype [num_blocks, num_kv_heads, block_size, head_dim], PA_F32/PA_BF16/PA_FP8_E4M3
 *   block_tables               [num_seqs, max_blocks_per_seq]
 *   context_lens               [num_seqs]
 *   cu_query_lens              [num_seqs + 1] or NULL (then row b is request b's only token)
 *   max_q_len                  upper bound on every request's query length (1 when cu is NULL)
 *   sliding_window             0 = none; W > 0: token i sees only keys [max(0, n_i - W), n_i); the plan
 *                              must have been built with the same window
 *   scale, k_scale, v_scale    softmax scale (typically 1/sqrt(head_dim)) and per-tensor dequant scales
 *   work_info, reduce_info,    the plan from pa_plan (capacity slots); reduce_info is only read when
 *   num_work                   out is given and may then not be NULL
 *   dispatch_info              NULL, or pa_plan's dispatch order for the same plan: workgroup position
 *                              p then runs the slot dispatch_info[p] names (word 3) instead of slot p;
 *                              the states go to the same places either way (bf16 and fp8 caches; the
 *                              f32 kernel and shared slots keep slot order)
 *   tile_tokens                the plan's tile size; a multiple of block_size
 *   workspace                  pa_workspace_bytes(capacity, max_q_len, num_q_heads, head_dim) bytes;
 *                              at least the slot states (that size without the shared-slot region,
 *                              PA_CAPACITY below it), in which case slots are not shared
 *   out, out_dtype             NULL: write the partial states only (pa_merge combines them later).
 *                              Non-NULL: also merge, exactly as pa_merge with the same arguments
 *                              (out_dtype must equal q_dtype): the call is then the decode launch
 *                              followed by the merge launch on the same stream, and the merge's
 *                              checks run with the decode's, before either launch.
 * Supported: head_dim in {64, 128, 256}; block_size in {16, 64, 128};
 * (num_q_heads / num_kv_heads) x max_q_len <= PA_MAX_GROUP_ROWS; max_blocks_per_seq x block_size
 * <= 2^31 - 257 (key positions are 32-bit).  Anything else returns PA_UNSUPPORTED.
 * KV types bf16 and fp8 run on the matrix cores in bf16 (fp8 codes widen exactly to bf16; q is
 * rounded to bf16; probabilities are rounded to bf16 for the P.V product; accumulation is fp32).
 * KV type f32 runs in fp32 on the vector ALUs.
 * Shared slots: when 0 < capacity <= num_seqs <= PA_INLINE_PLAN_SEQS (every request at most one
 * slot once the plan fills the capacity), head_dim <= 128 and workspace_bytes covers
 * the shared-slot region (pa_workspace_bytes does), slot sizes follow the request lengths and one
 * workgroup per slot would leave the longest request to one workgroup.  The decode then cuts every
 * used slot of n tiles into X = max(1, ceil(n / p)) pieces, p = ceil((sum of the used slots' tiles +
 * used slots) / (2 x used slots)), piece k taking the slot's tiles [floor(k n / X),
 * floor((k + 1) n / X)); each piece is one workgroup, pieces are numbered slot by slot, and their
 * states go to the shared-slot region with each request's (first piece, pieces).  pa_merge decides
 * the same way from its own arguments (capacity, num_seqs, head_dim, workspace_bytes).
 */
pa_status pa_decode(const void* q, pa_dtype q_dtype, int32_t num_rows, int32_t num_q_heads,
                    int32_t head_dim, const void* k_cache, const void* v_cache, pa_dtype kv_dtype,
                    int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, const int32_t* cu_query_lens,
                    int32_t max_q_len, int32_t sliding_window, float scale, float k_scale,
                    float v_scale, const int32_t* work_info, const int32_t* reduce_info,
                    const int32_t* num_work, const int32_t* dispatch_info, int32_t capacity,
                    int32_t tile_tokens, void* workspace, size_t workspace_bytes, void* out,
                    pa_dtype out_dtype, void* stream);

/*
 * Log-sum-exp merge.  For output row r and head h: the owning request b is found by binary search
 * of r in cu_query_lens (row b when NULL); token i = r - cu[b].  Over the request's partials j with
 * l_j > 0:  M = max m_j,  out = sum_j e^(m_j - M) acc_j / sum_j e^(m_j - M) l_j, rounded to nearest
 * even in out_dtype.  Rows r >= cu[num_seqs] (or >= num_seqs without cu), requests without
 * partitions, and rows whose partials are all empty are written as +0.0.  Every element of out
 * ([num_rows, num_q_heads, head_dim]) is written.
 * out_dtype must equal the q dtype given to pa_decode (PA_F32 or PA_BF16).
 * Under pa_decode's shared-slot condition (0 < capacity <= num_seqs <= PA_INLINE_PLAN_SEQS,
 * head_dim <= 128, workspace_bytes covering the region) a request's partials are its pieces (in slot
 * order) rather than its slots; same formula.  The workspace must hold what pa_decode (out = NULL)
 * wrote with the same capacity, max_q_len, num_q_heads, head_dim and workspace_bytes.
 */
pa_status pa_merge(int32_t num_rows, int32_t num_q_heads, int32_t head_dim, int32_t num_seqs,
                   const int32_t* cu_query_lens, int32_t max_q_len, const int32_t* reduce_info,
                   int32_t capacity, const void* workspace, size_t workspace_bytes, void* out,
                   pa_dtype out_dtype, void* stream);

/*
 * The whole step -- plan, decode, merge -- on one stream, with results identical to pa_plan followed
 * by pa_decode (out = NULL) and pa_merge with the same arguments: work_info, reduce_info and num_work
 * receive the plan bit for bit as pa_plan writes it, the workspace the same partial states, and out
 * the same rows, when capacity is pa_plan_capacity's value.  Arguments are those of the three calls
 * (cu_count, budget_mult, max_partitions as for pa_plan; capacity and sliding_window as for pa_plan
 * and pa_decode); the plan buffers are outputs here.
 * With num_seqs <= PA_INLINE_PLAN_SEQS and a bf16 or fp8 cache, the decode launch evaluates the
 * planner's rule itself (every workgroup over all requests, one request per thread) and stores the
 * plan, so the step is two launches (decode, merge); otherwise it is the three launches.
 * Shared slots as in pa_decode, with the capacity formula's value in place of capacity when the
 * plan is made in place (the two agree when capacity is pa_plan_capacity's value).
 * Errors: the union of pa_plan's, pa_decode's and pa_merge's checks, before any launch.
 */
pa_status pa_attention(const void* q, pa_dtype q_dtype, int32_t num_rows, int32_t num_q_heads,
                       int32_t head_dim, const void* k_cache, const void* v_cache, pa_dtype kv_dtype,
                       int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t num_seqs, const int32_t* cu_query_lens,
                       int32_t max_q_len, int32_t sliding_window, float scale, float k_scale,
                       float v_scale, int32_t cu_count, int32_t budget_mult, int32_t max_partitions,
                       int32_t tile_tokens, int32_t capacity, int32_t* work_info,
                       int32_t* reduce_info, int32_t* num_work, void* workspace,
                       size_t workspace_bytes, void* out, pa_dtype out_dtype, void* stream);

/*
 * pa_attention for callers that cannot allocate memory: code under HIP graph capture, serving loops
 * and harnesses that forbid allocation.  Arguments are pa_attention's without the workspace; the
 * partial states go instead to a static device array of PA_NOALLOC_SCRATCH_BYTES that the library
 * holds on every device it runs on until the process ends.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library call).  The workspace it uses is pa_workspace_bytes(capacity,
 * max_q_len, num_q_heads, head_dim) bytes of the array when that fits, else the slot states alone (no
 * shared slots) when those fit; the results are pa_attention's with a workspace of that size.
 * Beyond the array, PA_CAPACITY before anything else.
 * The first call with a device current looks up that device's copy of the array (hipGetSymbolAddress)
 * and keeps it; make that first call outside graph capture.  All calls on one device share its array
 * and find it holding the last call's contents (nothing in it must start at zero): calls that
 * overlap on one device (concurrent streams or threads) race and give wrong results.
 * Errors: PA_CAPACITY (the states exceed the array), PA_UNSUPPORTED (device index >= 64),
 * PA_HIP_ERROR (no current device or the lookup failed), then those of pa_attention.
 */
pa_status pa_attention_noalloc(const void* q, pa_dtype q_dtype, int32_t num_rows, int32_t num_q_heads,
                               int32_t head_dim, const void* k_cache, const void* v_cache, pa_dtype kv_dtype,
                               int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs, const int32_t* cu_query_lens,
                               int32_t max_q_len, int32_t sliding_window, float scale, float k_scale,
                               float v_scale, int32_t cu_count, int32_t budget_mult, int32_t max_partitions,
                               int32_t tile_tokens, int32_t capacity, int32_t* work_info,
                               int32_t* reduce_info, int32_t* num_work, void* out, pa_dtype out_dtype,
                               void* stream);

/*
 * Prefill rows: attention of every query token of the given requests over its visible keys, written
 * normalised to out.  For the decode-first split of mixed batches (opengfx1030/vllm-rdna PR #29,
 * Change 2: decode and verify rows go to the split-KV decode, the rest to a prefill kernel on the
 * rebased remainder): the caller passes the prefill requests' slices,
 *   context_lens + nd, block_tables + nd rows, cu_query_lens + nd (absolute row numbers: row r of q
 *   and out is query token r - cu[b] of request b),
 * with q and out the whole batch's arrays and num_rows its row count.  Rows [cu[0], cu[num_seqs])
 * get attention, rows [cu[num_seqs], num_rows) zeros, rows before cu[0] are not touched.
 * Token i of a request with L tokens and S keys sees [0, S - (L - 1 - i)) (or its last
 * sliding_window keys), as in pa_decode; rows with no visible key are zeros.
 * Two forms, chosen by the caller:
 *   workspace NULL   each query block (64 / G tokens at head_dim <= 128, 16 / G at 256) is one
 *                    workgroup that streams every key the block sees, in one launch: the form for
 *                    short prompts, whose blocks see few keys.
 *   workspace given  each request's query tokens are cut into blocks of T = 256 / G tokens (128 / G
 *                    at head_dim 256), and the blocks are planned like requests -- the length-
 *                    proportional rule of pa_plan over the blocks' key ranges, with budget 1 x
 *                    cu_count, ceiling 256 and 256-token tiles.  Each plan slot (a block and a range of
 *                    its keys) is then one workgroup whose eight waves share every 32-key K/V chunk
 *                    through LDS, each wave holding 16 or 32 of the block's query rows; the slots'
 *                    states are merged into the rows.  A block behind a long prefix reads its keys with
 *                    several workgroups, and each K/V byte is read once per block of T tokens.  Three
 *                    launches: the blocks and their plan, the block kernel, the merge.
 *                    The workspace holds pa_prefill_workspace_bytes(num_rows, num_seqs, num_q_heads,
 *                    num_kv_heads, head_dim, cu_count) bytes, 256-byte aligned, owned by the caller, with
 *                    no initial contents needed; cu_count is the compute-unit count the budget is built
 *                    from (pa_device_cu_count).
 * Both forms compute the same rows up to rounding.
 * K/V of bf16 or fp8 caches only (PA_UNSUPPORTED for f32).  cu_query_lens is required.  Errors: as
 * pa_decode, plus, with a workspace, PA_INVALID_ARG (cu_count < 1, misaligned workspace),
 * PA_UNSUPPORTED (more than PA_MAX_SEQS blocks), PA_CAPACITY (workspace too small).
 */
pa_status pa_prefill(const void* q, pa_dtype q_dtype, int32_t num_rows, int32_t num_q_heads,
                     int32_t head_dim, const void* k_cache, const void* v_cache, pa_dtype kv_dtype,
                     int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t num_seqs, const int32_t* cu_query_lens,
                     int32_t sliding_window, float scale, float k_scale, float v_scale, int32_t cu_count,
                     void* workspace, size_t workspace_bytes, void* out, pa_dtype out_dtype, void* stream);

/*
 * Bytes of workspace pa_prefill's split form needs for num_rows rows of num_seqs prompt requests: the
 * query blocks' lengths, first rows and request indices (at most ceil(num_rows / T) + num_seqs blocks,
 * T as in pa_prefill), their plan (work_info for the capacity formula over the blocks, reduce_info,
 * num_work), and the fp32 partial states [capacity, T, num_q_heads, head_dim] plus (max, sum) pairs,
 * each region 256-byte aligned.
 * Returns 0 for invalid sizes or more than PA_MAX_SEQS blocks.  Pure host arithmetic.
 */
size_t pa_prefill_workspace_bytes(int32_t num_rows, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t cu_count);

/*
 * A mixed batch whose requests are ordered decodes first, in one call (opengfx1030/vllm-rdna PR #29,
 * Change 2: decode and verify rows to the split-KV decode, the rest to the prefill kernel).
 * Requests [0, num_decodes) are the decode part: each has at most max_q_len query tokens, their rows
 * are [0, num_decode_rows) (num_decode_rows = cu[num_decodes], as pa_split_decode_first reports it),
 * and they are planned, decoded and merged exactly as pa_attention does with num_seqs = num_decodes
 * and num_rows = num_decode_rows: the plan buffers (sized for num_decodes requests), the workspace and
 * out rows [0, num_decode_rows) receive the same values.  Requests [num_decodes, num_seqs) are
 * prompts, with the attention pa_prefill computes from the slices context_lens + num_decodes,
 * block_tables + num_decodes rows and cu_query_lens + num_decodes: out rows [num_decode_rows,
 * cu[num_seqs]) get their attention, rows [cu[num_seqs], num_rows) zeros.  Here each prompt query
 * block (up to 64 / G tokens for head_dim <= 128, 16 / G for 256) is one workgroup that streams every
 * key the block sees, with no workspace of its own: the form for short prompts beside decodes; long
 * prompt chunks behind a prefix belong in pa_prefill.
 * Where the decode part is planned in place and the prompts' query blocks fit the decode's query
 * rows per workgroup (or can be cut to fit while there are at most 64 prompt rows), the decode and
 * the prompts share one launch (decode workgroups first, the prompts' after them) followed by the
 * merge: two launches for the whole batch; otherwise the parts are launched apart.  Prompt query
 * blocks may then hold fewer tokens than pa_prefill's, which changes only how the work is cut.
 * cu_query_lens is required.  Errors: those of pa_attention on the decode part and of pa_prefill
 * on the prompts, plus PA_INVALID_ARG for num_decodes outside [0, num_seqs] or num_decode_rows
 * outside [0, num_rows]; all before any launch.
 */
pa_status pa_attention_mixed(const void* q, pa_dtype q_dtype, int32_t num_rows, int32_t num_q_heads,
                             int32_t head_dim, const void* k_cache, const void* v_cache,
                             pa_dtype kv_dtype, int32_t num_blocks, int32_t num_kv_heads,
                             int32_t block_size, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                             const int32_t* cu_query_lens, int32_t num_decodes, int32_t num_decode_rows,
                             int32_t max_q_len, int32_t sliding_window, float scale, float k_scale,
                             float v_scale, int32_t cu_count, int32_t budget_mult, int32_t max_partitions,
                             int32_t tile_tokens, int32_t capacity, int32_t* work_info,
                             int32_t* reduce_info, int32_t* num_work, void* workspace,
                             size_t workspace_bytes, void* out, pa_dtype out_dtype, void* stream);

/*
 * The decode-first split of a batch whose requests are ordered decodes first (opengfx1030/vllm-rdna
 * PR #29, Change 2, the builder's split): the leading requests with at most `threshold` query tokens
 * (1 + speculative tokens) are the decode part.  HOST array cu_query_lens_host [num_seqs + 1];
 * writes the number of decode requests and their rows (cu[nd] - cu[0]).  Pure host arithmetic.
 */
pa_status pa_split_decode_first(const int32_t* cu_query_lens_host, int32_t num_seqs, int32_t threshold,
                                int32_t* num_decodes, int32_t* num_decode_tokens);

/* Static, human-readable name of a status code. */
const char* pa_status_string(pa_status status);

/* Compute-unit count of a HIP device (the cu_count the planner's budget is built from). */
pa_status pa_device_cu_count(int32_t device, int32_t* cu_count_out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */

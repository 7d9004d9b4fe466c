/*
 * pa_probe.h -- read-only bandwidth probes of libpa_probe.so (MI355X, gfx950).
 *
 * These are measurement kernels for the benchmark, not part of the decode path: they read device
 * memory and compute nothing of the method.  They give the decode kernel its practical ceilings on
 * the same device in the same run:
 *
 *   pa_probe_read    a contiguous read of `bytes` (the device's practical streaming read rate);
 *   pa_probe_gather  exactly the K and V bytes that pa_decode reads for a plan -- for every used slot
 *                    (request b, tiles [tb, te)) of work_info and every kv head, the keys
 *                    [tb x T, min(te x T, S_b)) fetched 16 keys at a time through the block table --
 *                    with the decode's launch shape (one 4-wave workgroup per (slot, kv head)) and
 *                    load form (16-byte non-temporal buffer loads), and no arithmetic, staging or
 *                    epilogue.  The plan is the one pa_plan writes (ROCm/ATOM PR #2366 "Route the paged
 *                    decode to aiter's FlyDSL kernel with work planner", section 3: work_info holds
 *                    (request, tile_begin, tile_end, seq_ctx) per slot).
 *
 * Conventions as in pa.h: device pointers, caller-owned memory, asynchronous on `stream` (a
 * hipStream_t passed as void*), nothing allocated, host-side checks before any launch.
 * `sink` receives one 32-bit word per wave of the launch (an XOR of the bytes read, so the loads are
 * not removed); its contents carry no meaning.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read bytes [0, bytes) of src once, split into `workgroups` contiguous spans of whole KiB (the last
 * may be shorter), one 256-thread workgroup each.
 *   src         device buffer, 16-byte aligned
 *   sink        device uint32 [4 x workgroups], 4-byte aligned
 * Errors: PA_INVALID_ARG (null pointers, workgroups < 1, misalignment), PA_HIP_ERROR (launch).
 */
pa_status pa_probe_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink, void* stream);

/*
 * Read the K/V bytes of a plan as described above.  Arguments mean what they mean for pa_decode
 * (include/pa.h): caches [num_blocks, num_kv_heads, block_size, head_dim] of kv_dtype,
 * block_tables [num_seqs, max_blocks_per_seq], context_lens [num_seqs], work_info [capacity, 4] from
 * pa_plan -- or the decode's dispatch order (pa_plan's dispatch_info), whose entries also start with
 * the request and the tile range, so workgroups take the slots in that order -- and num_work [2] from
 * pa_plan (checked, not read).  Only the rows below S_b are read; an entry naming no request (the
 * plan's sentinel for an unused slot) reads nothing.
 *   sink        device uint32 [4 x capacity x num_kv_heads], 4-byte aligned
 * Errors: PA_INVALID_ARG (null pointers, sizes < 1, misalignment, unknown kv_dtype),
 * PA_UNSUPPORTED (head_dim not 64/128/256, block_size not 16/64/128, tile_tokens not a multiple of
 * block_size), PA_HIP_ERROR (launch).
 */
pa_status pa_probe_gather(const void* k_cache, const void* v_cache, pa_dtype kv_dtype, int32_t num_blocks,
                          int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                          const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t num_seqs, const int32_t* work_info, const int32_t* num_work, int32_t capacity,
                          int32_t tile_tokens, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */

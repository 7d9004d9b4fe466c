// pa_plan.hip -- the length-proportional work planner on gfx950.
//
// What it computes is stated in ROCm/ATOM PR #2366 "[MiniMax-M3] Route the paged decode to aiter's
// FlyDSL kernel with work planner" (section 1: a partition count proportional to each request's real
// context length under a 2 x CU workgroup budget; section 3: ceiling 256; review item 2: work entries
// hold begin/end tiles and the request's length; review item 3: the capacity formula; review, window
// logic: under a sliding window the plan covers the range the kernel reads).  The rounding of the
// shares is this library's reading, documented in pa.h.
//
// One workgroup of 1024 threads does the whole plan: the planned sequences' lengths are read once into
// LDS, then a reduction for the total length and the number of non-empty requests, the per-request
// counts, an exclusive scan into LDS, and one thread per slot fills work_info by binary-searching the
// scanned offsets.  Integer-only, 64-bit where products can exceed 32 bits, so the result is
// bit-identical to any other exact evaluation.  For the split prefill the same launch first cuts the
// prompt requests into query blocks (cut_blocks) and plans the blocks.
//
// Optionally the same launch writes a dispatch order for the decode (this library's scheduling, not
// part of the pages' plan): the slots ranked by tile count (largest first, ties by slot index, unused
// slots last), rank r placed at position r when r < half = ceil(C / 2) and at position C + half - 1 - r
// otherwise; plans of more than kDispatchMaxSlots slots keep the slot order.  Positions p and p + half hold ranks p and C - 1 - p; with two workgroups per compute
// unit (positions p and p + half share one when C x kv heads is twice the compute units) each unit
// pairs a large slot with a small one, and the largest slots start in the first dispatch round.
#include "pa_device.h"

namespace pa {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

// A slot's dispatch key: larger for more tiles, then for a lower slot index (slots < 2048), distinct
// for distinct slots.  Unused slots (tiles -1) key below every used one and padding (-2) below those.
// Exact while tiles < kRankKeyTiles; the clamp keeps every key inside 31 bits.
constexpr int kRankKeyTiles = (1 << 20) - 2;
constexpr int kClosedMaxSeqs = kDispatchMaxSlots / 4;
static_assert(kDispatchMaxSlots <= 2048, "slot indices take the key's low 11 bits");
__device__ __forceinline__ int rank_key(int tiles, int slot) {
    return ((min(tiles, kRankKeyTiles - 1) + 2) << 11) | (2047 - slot);
}

// Query blocks of a prefill batch as pseudo-requests for the planner, the decode and the merge: each
// request's query tokens [0, L_b) are cut into blocks of block_tokens, numbered request by request.
// Block j covering tokens [i0, i1) of request b gets
//   blk_cu[j] = cu[b] + i0                (its first row; blk_cu[max_blocks] = cu[num_seqs]),
//   blk_ctx[j] = S_b - (L_b - i1)         (the keys its last token sees, at least 0),
//   blk_req[j] = b                        (the request's block-table row),
// so that token i of the block sees blk_ctx[j] - (i1 - 1 - i) = S_b - (L_b - 1 - i) keys, the
// request's own per-token causal range (opengfx1030/vllm-rdna PR #29, Change 1).  Slots past the last
// block are empty blocks (blk_cu = cu[num_seqs], blk_ctx = 0, blk_req = 0).  Each thread takes a
// contiguous run of requests; a scan over the threads gives each run's first block.  The blocks'
// lengths and token counts also go to the planner's LDS arrays (the caller meets the barrier after).
__device__ void cut_blocks(const PlanBlocks& pb, int max_blocks, int32_t* s_len, int32_t* s_qlen) {
    __shared__ int scan_carry[kPlanWaves];
    __shared__ int s_total;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int32_t* const cu = pb.cu;
    const int per = (pb.num_reqs + kPlanThreads - 1) / kPlanThreads;
    const int b0 = min(tid * per, pb.num_reqs);
    const int b1 = min(b0 + per, pb.num_reqs);
    auto q_len = [&](int b) { return max(cu[b + 1] - cu[b], 0); };
    int local = 0;
    for (int b = b0; b < b1; ++b) local += (q_len(b) + pb.block_tokens - 1) / pb.block_tokens;
    const int incl = wave_incl_scan(local, lane);
    if (lane == 63) scan_carry[wave] = incl;
    __syncthreads();
    int j = incl - local;
    for (int w = 0; w < wave; ++w) j += scan_carry[w];
    if (tid == kPlanThreads - 1) s_total = j + local;
    for (int b = b0; b < b1; ++b) {
        const int L = q_len(b);
        const int S = max(pb.ctx[b], 0);
        const int row = cu[b];
        for (int i0 = 0; i0 < L && j < max_blocks; i0 += pb.block_tokens, ++j) {
            const int i1 = min(L, i0 + pb.block_tokens);
            const int ctx = max(S - (L - i1), 0);
            pb.blk_cu[j] = row + i0;
            pb.blk_ctx[j] = ctx;
            pb.blk_req[j] = b;
            s_len[j] = ctx;
            s_qlen[j] = i1 - i0;
        }
    }
    __syncthreads();
    const int end = cu[pb.num_reqs];
    for (int e = max(s_total, 0) + tid; e < max_blocks; e += kPlanThreads) {
        pb.blk_cu[e] = end;
        pb.blk_ctx[e] = 0;
        pb.blk_req[e] = 0;
        s_len[e] = 0;
        s_qlen[e] = 0;
    }
    if (tid == 0) pb.blk_cu[max_blocks] = end;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu, int num_seqs,
    int cap_formula, int capacity, int max_partitions, int tile_tokens, int window,
    int4* __restrict__ work_info, int2* __restrict__ reduce_info, int32_t* __restrict__ num_work,
    int4* __restrict__ dispatch_info, const PlanBlocks blocks) {
    __shared__ int32_t first[PA_MAX_SEQS + 1];
    __shared__ int32_t s_len[PA_MAX_SEQS];        // each planned sequence's length (>= 0) ...
    __shared__ int32_t s_qlen[PA_MAX_SEQS];       // ... and query tokens, read from memory once
    __shared__ int32_t s_tiles[kDispatchMaxSlots];
    __shared__ __align__(16) int32_t s_aux[kDispatchMaxSlots];   // a slot's key, or its rank within its request
    __shared__ int32_t s_rank[kDispatchMaxSlots];
    __shared__ int4 s_entry[kDispatchMaxSlots];
    __shared__ int4 s_qrp[kClosedMaxSeqs];
    __shared__ long long red_total[kPlanWaves];
    __shared__ int red_count[kPlanWaves];
    __shared__ int scan_carry[kPlanWaves];
    __shared__ int largest_of_wave[kPlanWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool ranked = dispatch_info && capacity > 0 && capacity <= kDispatchMaxSlots;
    // ranks from the closed form (O(requests) per slot) when the batch is small against the slots
    const bool closed = ranked && num_seqs <= kClosedMaxSeqs && 4 * num_seqs <= capacity;

    if (blocks.ctx) {
        cut_blocks(blocks, num_seqs, s_len, s_qlen);
    } else {
        for (int b = tid; b < num_seqs; b += kPlanThreads) {
            s_len[b] = max(context_lens[b], 0);
            s_qlen[b] = plan_q_len(cu, b);
        }
    }
    __syncthreads();

    // the key range request b reads: all of [0, S_b), or its window's union
    auto range_of = [&](int b) -> PlanRange {
        return plan_range(s_len[b], window > 0 ? s_qlen[b] : 1, window, tile_tokens);
    };

    // --- W = sum of the lengths read and B' = #{requests reading any key} ---
    long long total = 0;
    int nonempty = 0;
    for (int b = tid; b < num_seqs; b += kPlanThreads) {
        const int len = range_of(b).len;
        total += len;
        nonempty += (len > 0);
    }
    total = wave_sum_ll(total);
    for (int o = 32; o >= 1; o >>= 1) nonempty += __shfl_xor(nonempty, o, 64);
    if (lane == 0) {
        red_total[wave] = total;
        red_count[wave] = nonempty;
    }
    __syncthreads();
    total = 0;
    nonempty = 0;
    for (int w = 0; w < kPlanWaves; ++w) {
        total += red_total[w];
        nonempty += red_count[w];
    }
    const long long extra = static_cast<long long>(cap_formula) - nonempty;

    // --- per-request partition counts over a contiguous range per thread, then an exclusive scan ---
    const int per = (num_seqs + kPlanThreads - 1) / kPlanThreads;
    const int b0 = min(tid * per, num_seqs);
    const int b1 = min(b0 + per, num_seqs);
    int local = 0;
    for (int b = b0; b < b1; ++b) {
        const PlanRange r = range_of(b);
        const int parts = plan_parts(r.len, r.tiles, extra, total, max_partitions);
        first[b] = parts;
        local += parts;
        if (closed)     // (q, rem, parts): rem slots of q + 1 tiles, the others of q
            s_qrp[b] = parts > 0 ? make_int4(r.tiles / parts, r.tiles % parts, parts, 0) : make_int4(0, 0, 0, 0);
    }
    const int incl = wave_incl_scan(local, lane);
    if (lane == 63) scan_carry[wave] = incl;
    __syncthreads();
    int offset = incl - local;
    for (int w = 0; w < wave; ++w) offset += scan_carry[w];
    for (int b = b0; b < b1; ++b) {
        const int parts = first[b];
        first[b] = offset;
        offset += parts;
    }
    if (tid == kPlanThreads - 1) first[num_seqs] = offset;  // the last thread's offset is the grand total
    __syncthreads();

    const int used = first[num_seqs];
    for (int b = tid; b < num_seqs; b += kPlanThreads)
        reduce_info[b] = make_int2(first[b], first[b + 1] - first[b]);

    // --- one thread per slot ---
    const int cap4 = (capacity + 3) & ~3;                 // the keys are read four at a time
    if (ranked)
        for (int s = tid; s < cap4; s += kPlanThreads) {
            s_rank[s] = 0;
            if (s >= capacity) {                          // padding: below every slot, counts for none
                s_tiles[s] = -2;
                s_aux[s] = rank_key(-2, s);
            }
        }
    int largest = 0;
    for (int s = tid; s < capacity; s += kPlanThreads) {
        int4 e = make_int4(-1, 0, 0, 0);
        int tiles = -1;                                   // unused slots rank after every used one
        int owner = num_seqs, within = s - used;          // (closed form) an unused slot's terms
        if (s < used) {
            // last request whose first slot is <= s (it has at least one partition because s < used)
            int lo = 0, hi = num_seqs - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (first[mid] <= s) lo = mid;
                else hi = mid - 1;
            }
            const int b = lo;
            const int j = s - first[b];
            const int parts = first[b + 1] - first[b];
            const PlanRange pr = range_of(b);
            const int2 r = plan_tile_range(j, pr.tiles, parts);
            e = make_int4(b, pr.t0 + r.x, pr.t0 + r.y, s_len[b]);
            tiles = r.y - r.x;
            largest = max(largest, tiles);
            if (closed) {
                // the request's slots before this one of the same size: r.x - j q of them hold q + 1
                const int q = s_qrp[b].x;
                const int big_before = r.x - j * q;
                owner = b;
                within = tiles == q + 1 ? big_before : j - big_before;
            }
        }
        work_info[s] = e;
        if (ranked) {
            s_tiles[s] = tiles;
            s_aux[s] = closed ? within : rank_key(tiles, s);
            s_entry[s] = make_int4(e.x, e.y, e.z, owner);
        } else if (dispatch_info) {
            dispatch_info[s] = make_int4(e.x, e.y, e.z, s);    // beyond the ranked size: identity order
        }
    }
    for (int o = 32; o >= 1; o >>= 1) largest = max(largest, __shfl_xor(largest, o, 64));
    if (lane == 0) largest_of_wave[wave] = largest;
    __syncthreads();
    if (tid == 0) {
        for (int w = 0; w < kPlanWaves; ++w) largest = max(largest, largest_of_wave[w]);
        *reinterpret_cast<int2*>(num_work) = make_int2(used, largest);
    }
    if (!ranked) return;
    // rank of slot s: slots with more tiles, then slots with as many tiles and a lower index.  Each
    // slot's terms are split over `split` threads; the parts meet in s_rank through integer adds, whose
    // sum does not depend on their order.
    const int split = max(1, min(kPlanThreads / capacity, 16));
    if (closed) {
        // Closed form.  Request b' holds rem' slots of q' + 1 tiles and parts' - rem' of q', so for a
        // slot of t tiles owned by request b it contributes parts' slots with more tiles when q' > t,
        // rem' when q' = t; and, when b' < b, parts' - rem' slots with as many tiles when q' = t,
        // rem' when q' + 1 = t.  Add the owner's own earlier slots of t tiles.  An unused slot (t = -1,
        // owner past the last request) gets every used slot plus the unused ones before it.
        const int per_part = (num_seqs + split - 1) / split;
        for (int w = tid; w < capacity * split; w += kPlanThreads) {
            const int s = w / split;
            const int part = w - s * split;
            const int t = s_tiles[s];
            const int owner = s_entry[s].w;
            const int r0 = part * per_part;
            const int r1 = min(r0 + per_part, num_seqs);
            int count = part == 0 ? s_aux[s] : 0;
            for (int b = r0; b < r1; ++b) {
                const int4 v = s_qrp[b];
                const int more = v.x > t ? v.z : (v.x == t ? v.y : 0);
                const int same = v.x == t ? v.z - v.y : (v.x + 1 == t ? v.y : 0);
                count += more + (b < owner ? same : 0);
            }
            if (count) atomicAdd(&s_rank[s], count);
        }
    } else {
        // Pairwise: while every slot holds fewer than kRankKeyTiles tiles the order is that of the
        // distinct keys rank_key(tiles, slot), one difference per pair (read four keys at a time from
        // the padded array); otherwise the pairs are compared field by field.
        int top = 0;
        for (int w = 0; w < kPlanWaves; ++w) top = max(top, largest_of_wave[w]);
        const bool keyed = top < kRankKeyTiles;
        const int quads = cap4 / 4;
        const int per_part = (quads + split - 1) / split;
        for (int w = tid; w < capacity * split; w += kPlanThreads) {
            const int s = w / split;
            const int part = w - s * split;
            const int q0 = part * per_part;
            const int q1 = min(q0 + per_part, quads);
            int count = 0;
            if (keyed) {
                const int k = s_aux[s];
#pragma unroll 8
                for (int q = q0; q < q1; ++q) {
                    // keys lie in [0, 2^31): the differences cannot overflow; 1 exactly when key u > k
                    const int4 ku = reinterpret_cast<const int4*>(s_aux)[q];
                    count += min(max(ku.x - k, 0), 1) + min(max(ku.y - k, 0), 1) +
                             min(max(ku.z - k, 0), 1) + min(max(ku.w - k, 0), 1);
                }
            } else {
                const int t = s_tiles[s];
                for (int u = 4 * q0; u < 4 * q1; ++u) {
                    const int tu = s_tiles[u];
                    count += (tu > t) || (tu == t && u < s);
                }
            }
            if (count) atomicAdd(&s_rank[s], count);
        }
    }
    __syncthreads();
    const int half = (capacity + 1) / 2;
    for (int s = tid; s < capacity; s += kPlanThreads) {
        const int rank = s_rank[s];
        const int pos = rank < half ? rank : capacity + half - 1 - rank;
        const int4 e = s_entry[s];
        dispatch_info[pos] = make_int4(e.x, e.y, e.z, s);    // (request, tile_begin, tile_end, slot)
    }
}

}  // namespace

hipError_t launch_plan(const int32_t* context_lens, const int32_t* cu, int num_seqs, int cap_formula,
                       int capacity, int max_partitions, int tile_tokens, int window,
                       int32_t* work_info, int32_t* reduce_info, int32_t* num_work, int32_t* dispatch_info,
                       hipStream_t stream, const PlanBlocks* blocks) {
    const PlanBlocks pb = blocks ? *blocks : PlanBlocks{};
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, context_lens, cu, num_seqs,
                       cap_formula, capacity, max_partitions, tile_tokens, window,
                       reinterpret_cast<int4*>(work_info), reinterpret_cast<int2*>(reduce_info),
                       num_work, reinterpret_cast<int4*>(dispatch_info), pb);
    return hipGetLastError();
}

}  // namespace pa

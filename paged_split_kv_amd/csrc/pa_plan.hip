// pa_plan.hip -- the length-proportional work planner on gfx950.
//
// What it computes is stated in ROCm/ATOM PR #2366 "[MiniMax-M3] Route the paged decode to aiter's
// FlyDSL kernel with work planner" (section 1: a partition count proportional to each request's real
// context length under a 2 x CU workgroup budget; section 3: ceiling 256; review item 2: work entries
// hold begin/end tiles and the request's length; review item 3: the capacity formula; review, window
// logic: under a sliding window the plan covers the range the kernel reads).  The rounding of the
// shares is this library's reading, documented in pa.h.
//
// One workgroup of 1024 threads does the whole plan: a reduction for the total length and the number
// of non-empty requests, the per-request counts, an exclusive scan into LDS, and then one thread per
// slot fills work_info by binary-searching the scanned offsets.  Integer-only, 64-bit where
// products can exceed 32 bits, so the result is bit-identical to any other exact evaluation.
#include "pa_device.h"

namespace pa {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu, int num_seqs,
    int cap_formula, int capacity, int max_partitions, int tile_tokens, int window,
    int4* __restrict__ work_info, int2* __restrict__ reduce_info, int32_t* __restrict__ num_work) {
    __shared__ int32_t first[PA_MAX_SEQS + 1];
    __shared__ long long red_total[kPlanWaves];
    __shared__ int red_count[kPlanWaves];
    __shared__ int scan_carry[kPlanWaves];
    __shared__ int largest_of_wave[kPlanWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // the key range request b reads: all of [0, S_b), or its window's union
    auto range_of = [&](int b) -> PlanRange {
        return plan_range(max(context_lens[b], 0), window > 0 ? plan_q_len(cu, b) : 1, window, tile_tokens);
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
    int largest = 0;
    for (int s = tid; s < capacity; s += kPlanThreads) {
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
            work_info[s] = make_int4(b, pr.t0 + r.x, pr.t0 + r.y, max(context_lens[b], 0));
            largest = max(largest, r.y - r.x);
        } else {
            work_info[s] = make_int4(-1, 0, 0, 0);
        }
    }
    for (int o = 32; o >= 1; o >>= 1) largest = max(largest, __shfl_xor(largest, o, 64));
    if (lane == 0) largest_of_wave[wave] = largest;
    __syncthreads();
    if (tid == 0) {
        for (int w = 0; w < kPlanWaves; ++w) largest = max(largest, largest_of_wave[w]);
        *reinterpret_cast<int2*>(num_work) = make_int2(used, largest);
    }
}

}  // namespace

hipError_t launch_plan(const int32_t* context_lens, const int32_t* cu, int num_seqs, int cap_formula,
                       int capacity, int max_partitions, int tile_tokens, int window,
                       int32_t* work_info, int32_t* reduce_info, int32_t* num_work, hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, context_lens, cu, num_seqs,
                       cap_formula, capacity, max_partitions, tile_tokens, window,
                       reinterpret_cast<int4*>(work_info), reinterpret_cast<int2*>(reduce_info),
                       num_work);
    return hipGetLastError();
}

}  // namespace pa

// pa_device.h -- device-side helpers shared by the gfx950 kernels of libpa (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// ---------------------------------------------------------------------------------------------
// launch helpers (host)
// ---------------------------------------------------------------------------------------------
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------------------------------------
// element conversions (device)
// ---------------------------------------------------------------------------------------------

// bfloat16 bits -> float: the bf16 pattern is the upper half of the binary32 pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// OCP E4M3 ("fn") code -> bfloat16 bits, exact: every e4m3fn value is a bf16 value.
// Normal codes (exponent field e > 0): bf16 exponent = e - 7 + 127, mantissa bits shifted up by 4.
// Subnormal codes (e = 0): value m x 2^-9, built from a small integer in float.
// S.1111.111 is NaN.
__device__ __forceinline__ uint32_t fp8e4m3_to_bf16(uint32_t code) {
    const uint32_t mag = code & 0x7fu;
    const uint32_t sign = (code & 0x80u) << 8;
    uint32_t bits;
    if (mag >= 0x08u) {
        bits = (mag << 4) + (120u << 7);
        if (mag == 0x7fu) bits = 0x7fc0u;
    } else {
        bits = __float_as_uint(static_cast<float>(mag) * 0x1p-9f) >> 16;
    }
    return sign | bits;
}

// Four e4m3fn codes packed in a dword -> two dwords of bf16 pairs (codes 0,1 then 2,3).
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t codes, uint32_t& lo, uint32_t& hi) {
    lo = fp8e4m3_to_bf16(codes & 0xffu) | (fp8e4m3_to_bf16((codes >> 8) & 0xffu) << 16);
    hi = fp8e4m3_to_bf16((codes >> 16) & 0xffu) | (fp8e4m3_to_bf16(codes >> 24) << 16);
}

// ---------------------------------------------------------------------------------------------
// wavefront reductions (64 lanes)
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------------------------
// the planner's rule, shared by the plan kernel and the decode that plans in place (ROCm/ATOM PR
// #2366 section 1: partitions proportional to the request's length under the budget; section 3:
// ceiling; review item 2: contiguous tile ranges).  Integer-only, so every evaluation is identical.
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        int lo = __shfl_xor(static_cast<int>(v & 0xffffffffll), o, 64);
        int hi = __shfl_xor(static_cast<int>(v >> 32), o, 64);
        v += (static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo);
    }
    return v;
}

// Cross-lane steps through DPP (the vector ALU's lane-shifted operand; no LDS round trip).  Lanes
// with no source lane, or outside the row mask, read `ident`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_read(int v, int ident) {
    return __builtin_amdgcn_update_dpp(ident, v, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 within each 16-lane row, then the
// last lane of row 0 (and of row 2) is added to row 1 (row 3), then lane 31 to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v, int /*lane*/) {
    v += dpp_read<kDppRowShr1, 0xf>(v, 0);
    v += dpp_read<kDppRowShr2, 0xf>(v, 0);
    v += dpp_read<kDppRowShr4, 0xf>(v, 0);
    v += dpp_read<kDppRowShr8, 0xf>(v, 0);
    v += dpp_read<kDppRowBcast15, 0xa>(v, 0);
    v += dpp_read<kDppRowBcast31, 0xc>(v, 0);
    return v;
}

// Maximum over the 64 lanes of non-negative values (the same prefix pattern with max), uniform.
__device__ __forceinline__ int wave_max_nonneg(int v) {
    v = max(v, dpp_read<kDppRowShr1, 0xf>(v, 0));
    v = max(v, dpp_read<kDppRowShr2, 0xf>(v, 0));
    v = max(v, dpp_read<kDppRowShr4, 0xf>(v, 0));
    v = max(v, dpp_read<kDppRowShr8, 0xf>(v, 0));
    v = max(v, dpp_read<kDppRowBcast15, 0xa>(v, 0));
    v = max(v, dpp_read<kDppRowBcast31, 0xc>(v, 0));
    return __builtin_amdgcn_readlane(v, 63);
}

// Sum over the 64 lanes of values in [0, 2^31), exact in 64 bits: the low and high 16-bit halves
// are summed separately (each total stays below 2^22), uniform.
__device__ __forceinline__ long long wave_sum_nonneg(int v) {
    const int lo = __builtin_amdgcn_readlane(wave_incl_scan(v & 0xffff, 0), 63);
    const int hi = __builtin_amdgcn_readlane(wave_incl_scan(static_cast<int>(static_cast<unsigned>(v) >> 16), 0), 63);
    return (static_cast<long long>(hi) << 16) + lo;
}

// The key range a request reads and the tiles it spans.  Without a window the range is [0, S);
// with a window of W keys per token (the window applies per token) it is the union of the
// tokens' ranges, [max(0, S - (L - 1) - W), S).  The tiles are those the range touches,
// [floor(lo / T), ceil(S / T)); len = S - lo weighs the request in the apportionment.
struct PlanRange {
    int len;      // keys read
    int t0;       // first tile
    int tiles;    // tiles spanned (0 when len = 0)
};

__device__ __forceinline__ PlanRange plan_range(int s, int q_len, int window, int tile_tokens) {
    PlanRange r;
    long long lo = 0;
    if (window > 0) {
        lo = static_cast<long long>(s) - (static_cast<long long>(q_len) - 1) - window;
        lo = lo < 0 ? 0 : (lo > s ? s : lo);
    }
    const unsigned t = static_cast<unsigned>(tile_tokens);
    r.len = s - static_cast<int>(lo);
    r.t0 = static_cast<int>(static_cast<unsigned>(lo) / t);
    // s + T - 1 < 2^32, so the 32-bit unsigned division is exact
    r.tiles = r.len > 0 ? static_cast<int>((static_cast<unsigned>(s) + t - 1u) / t) - r.t0 : 0;
    return r;
}

// Partitions of a request reading `len` keys over `tiles` tiles: none when empty, else
// min(P, tiles, 1 + floor(extra * len / W)) with extra = capacity - (non-empty requests) >= 0 and W
// the batch's total.  The quotient takes the 32-bit unsigned division when both operands fit.
__device__ __forceinline__ int plan_parts(int len, int tiles, long long extra, long long total,
                                          int max_partitions) {
    if (len <= 0) return 0;
    const unsigned long long num = static_cast<unsigned long long>(extra) * static_cast<unsigned>(len);
    long long q;
    if ((num >> 32) == 0 && (static_cast<unsigned long long>(total) >> 32) == 0)
        q = static_cast<unsigned>(num) / static_cast<unsigned>(total);
    else
        q = static_cast<long long>(num / static_cast<unsigned long long>(total));
    long long p = 1 + q;
    if (p > tiles) p = tiles;
    if (p > max_partitions) p = max_partitions;
    return static_cast<int>(p);
}

// Query length of request b (1 without cumulative lengths); a decreasing pair counts as 0.
__device__ __forceinline__ int plan_q_len(const int32_t* cu, int b) {
    if (!cu) return 1;
    const int L = cu[b + 1] - cu[b];
    return L < 0 ? 0 : L;
}

// Tile range [floor(j * tiles / parts), floor((j + 1) * tiles / parts)) of partition j.
__device__ __forceinline__ int2 plan_tile_range(int j, int tiles, int parts) {
    const unsigned t = static_cast<unsigned>(tiles);
    if (static_cast<unsigned long long>(parts) * t < (1ull << 32)) {
        // (j + 1) * tiles <= parts * tiles fits 32 bits: exact unsigned division
        return make_int2(static_cast<int>((static_cast<unsigned>(j) * t) / static_cast<unsigned>(parts)),
                         static_cast<int>((static_cast<unsigned>(j + 1) * t) / static_cast<unsigned>(parts)));
    }
    return make_int2(static_cast<int>((static_cast<long long>(j) * t) / parts),
                     static_cast<int>((static_cast<long long>(j + 1) * t) / parts));
}

// Workspace layout (see pa_workspace_bytes): acc region then (m, l) region, each 256-byte aligned.
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace regions: acc [capacity, max_q_len, num_q_heads, head_dim] fp32, then (m, l) pairs
// [capacity, max_q_len, num_q_heads, 2] fp32 (m is the running max in base-2 units).
__host__ __device__ inline size_t workspace_acc_bytes(int capacity, int max_q_len, int hq, int d) {
    return align256(static_cast<size_t>(capacity) * max_q_len * hq * d * sizeof(float));
}

__host__ __device__ inline size_t workspace_ml_bytes(int capacity, int max_q_len, int hq) {
    return align256(static_cast<size_t>(capacity) * max_q_len * hq * 2 * sizeof(float));
}

// Owning request and token of output row r (-1 when the row is padding or otherwise unowned).
// With cumulative query lengths this is the last b with cu[b] <= r.  Up to 63 requests, lane l of the
// wave loads cu[l] for l <= num_seqs, and the range check, the owner (a ballot) and its bounds (lane
// reads) follow from that one round of loads.  Beyond, a 64-way search in which every lane loads one
// probe: one round of loads for up to 64 requests per level.  A cu that is not monotone (a violated
// precondition) may give a wrong owner but never a token outside [0, max_q_len).  All lanes of the
// wave must call it with the same r.
__device__ __forceinline__ int owner_of_row(const int32_t* cu, int num_seqs, int max_q_len, int r, int& i) {
    i = 0;
    int b = -1;
    if (cu) {
        const int lane = threadIdx.x & 63;
        if (num_seqs > 0 && num_seqs < 64) {
            const int v = lane <= num_seqs ? cu[lane] : 0x7fffffff;
            const int first = __builtin_amdgcn_readlane(v, 0);
            const int last = __builtin_amdgcn_readlane(v, num_seqs);
            if (r >= first && r < last) {
                const unsigned long long m = __builtin_amdgcn_ballot_w64(lane < num_seqs && v <= r);
                b = __builtin_popcountll(m) - 1;            // >= 0: lane 0 holds first <= r
                const int c0 = __builtin_amdgcn_readlane(v, b);
                const int c1 = __builtin_amdgcn_readlane(v, b + 1);
                i = r - c0;
                if (i < 0 || i >= c1 - c0) b = -1;
            }
        } else if (num_seqs > 0 && r >= cu[0] && r < cu[num_seqs]) {
            int lo = 0, hi = num_seqs;                    // cu[lo] <= r; answer in [lo, hi)
            while (hi - lo > 1) {
                const int step = (hi - lo + 63) >> 6;
                const int idx = lo + lane * step;
                const int v = idx < hi ? cu[idx] : 0x7fffffff;
                const unsigned long long m = __builtin_amdgcn_ballot_w64(v <= r);
                const int k = __builtin_popcountll(m);     // probes are monotone: lanes 0..k-1 hold
                const int nlo = lo + max(k - 1, 0) * step;
                hi = min(hi, nlo + step);
                lo = nlo;
            }
            b = lo;
            i = r - cu[b];
            if (i < 0 || i >= cu[b + 1] - cu[b]) b = -1;
        }
    } else if (r < num_seqs) {
        b = r;
    }
    if (i >= max_q_len) b = -1;
    if (b < 0) i = 0;
    return b;
}


// ---------------------------------------------------------------------------------------------
// kernel argument blocks and launchers (one definition, shared by the translation units)
// ---------------------------------------------------------------------------------------------
struct DecodeArgs {
    const void* q;
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int32_t* cu;          // nullable
    const int4* work_info;
    const int4* dispatch_info;  // nullable: workgroup position p runs dispatch_info[p] = (request,
                                // tile_begin, tile_end, slot), the plan's slots in dispatch order
    const int32_t* num_work;
    float* ws_acc;
    float* ws_ml;
    const int32_t* bt_index;    // nullable: request b's block-table row is bt_index[b] (query blocks)
    void* out;                  // prefill mode only: the normalised rows are written here
    int window;                 // 0: none; W > 0: each query token sees its last W visible keys
    // prefill mode: each workgroup takes a block of up to block_tokens query tokens of one request
    // (all its visible keys, one partition) and writes the normalised rows to out directly
    int prefill;
    int block_tokens;
    // planning in place (num_seqs <= kInlinePlanSeqs): every workgroup evaluates the planner's rule
    // itself; the plan is also stored to these buffers for the merge and the caller
    int plan_inline;
    int plan_cap;               // the capacity formula's value (not the buffer's capacity)
    int max_partitions;
    int4* plan_work_out;
    int2* plan_reduce_out;
    int32_t* plan_num_work_out;
    // shared slots: pieces != 0 cuts every slot into pieces (see piece_size), one workgroup each;
    // workgroup p streams piece p and writes its state as state p of the shared-slot region (ws_acc
    // and ws_ml then point there and capacity is the piece count's bound), and (first piece, pieces)
    // per request go to piece_reduce_out for the merge.  plan_slots is the plan's slot count (the
    // length of work_info).
    int pieces;
    int plan_slots;
    int2* piece_reduce_out;
    int out_bf16;
    int num_rows, num_q_heads, num_kv_heads, group;   // group = Hq / Hkv
    int num_blocks, block_size, max_blocks, num_seqs;
    int max_q_len, capacity, tile_tokens;
    float score_scale_log2;     // scale * k_scale * log2(e)
    float v_scale;
};

// A decode launch: workgroups [0, split) run part[0], workgroups [split, grid) run part[1] with
// workgroup indices counted from split.  A plain launch sets split past the grid; a mixed batch's
// launch runs its decode requests (in-place plan) as part[0] and its prompts' query blocks as part[1].
struct LaunchArgs {
    DecodeArgs part[2];
    int split;
};

struct MergeArgs {
    const int32_t* cu;          // nullable
    const int2* reduce_info;
    const float* ws_acc;
    const float* ws_ml;
    const int32_t* row_floor;   // nullable: rows below *row_floor are left untouched
    void* out;
    int num_rows, num_q_heads, num_seqs, max_q_len, capacity;
};

// Requests a decode workgroup can plan for in place: one per thread of its 4 waves.
constexpr int kInlinePlanSeqs = PA_INLINE_PLAN_SEQS;

// Shared slots: pieces are sized so that a plan of `used` slots makes at most kPieceFactor x used +
// used pieces (see piece_size), so 3 x capacity piece states always suffice.
constexpr int kPieceFactor = 2;
inline int piece_bound(int capacity) { return (kPieceFactor + 1) * capacity; }

// The decode deals each slot's chunks evenly over its waves when the plan's largest slot gives every
// wave at least this many 16-key chunks, and in units of the largest slot otherwise.
constexpr int kEvenDealChunks = 12;

// The shared-slot region, after the slot states: the piece states' acc and (m, l) for
// piece_bound(capacity) pieces, then the per-request (first piece, pieces) pairs for up to
// kInlinePlanSeqs requests.  Byte offsets from the workspace's start.
struct SharedRegion {
    size_t acc, ml, reduce, end;
};
inline SharedRegion shared_region(int capacity, int max_q_len, int hq, int d) {
    SharedRegion r;
    const int states = piece_bound(capacity);
    r.acc = workspace_acc_bytes(capacity, max_q_len, hq, d) + workspace_ml_bytes(capacity, max_q_len, hq);
    r.ml = r.acc + workspace_acc_bytes(states, max_q_len, hq, d);
    r.reduce = r.ml + workspace_ml_bytes(states, max_q_len, hq);
    r.end = r.reduce + align256(static_cast<size_t>(kInlinePlanSeqs) * 2 * sizeof(int32_t));
    return r;
}

// Whether a decode writes pieces rather than slot states: a pure function of arguments that pa_decode,
// pa_merge and pa_attention all receive, so each decides alike.  `one_slot_cap` is the plan capacity
// that makes every request at most one slot (<= num_seqs); the batch fits the per-request table; the
// workspace holds the region.
inline bool shares_slots(int one_slot_cap, int num_seqs, int head_dim, int capacity, int max_q_len, int hq,
                         size_t workspace_bytes) {
    return one_slot_cap > 0 && one_slot_cap <= num_seqs && num_seqs <= kInlinePlanSeqs && head_dim <= 128 &&
           workspace_bytes >= shared_region(capacity, max_q_len, hq, head_dim).end;
}

// A split prefill's requests, cut into query blocks by the plan launch itself before it plans them
// (the planned sequences are then the blocks: num_seqs = max_blocks); see cut_blocks in pa_plan.hip.
struct PlanBlocks {
    const int32_t* ctx;       // the requests' context lengths [num_reqs] (null: no blocks to cut)
    const int32_t* cu;        // their query rows [num_reqs + 1]
    int num_reqs, block_tokens;
    int32_t *blk_ctx, *blk_cu, *blk_req;   // per block [max_blocks] (blk_cu [max_blocks + 1])
};
hipError_t launch_plan(const int32_t* context_lens, const int32_t* cu, int num_seqs,
                       int cap_formula, int capacity, int max_partitions, int tile_tokens, int window,
                       int32_t* work_info, int32_t* reduce_info, int32_t* num_work, int32_t* dispatch_info,
                       hipStream_t stream, const PlanBlocks* blocks = nullptr);
// Plans of at most this many slots get a balanced dispatch order; larger ones the identity.
constexpr int kDispatchMaxSlots = 1024;
hipError_t launch_decode(const DecodeArgs& a, int head_dim, pa_dtype kv_dtype, bool q_f32,
                         hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int head_dim, bool out_bf16, hipStream_t stream);
// Query tokens per prefill workgroup for a group of G query heads per kv head (G * tokens rows).
int prefill_block_tokens(int head_dim, int group);
// Column blocks (16 query rows each) of a decode launch over `rows` query rows per workgroup.
inline int column_blocks(int rows) { return rows <= 16 ? 1 : (rows <= 32 ? 2 : 4); }
// One launch for a mixed batch: the decode part (in-place plan) and the prompts' query blocks, both
// with `ncb` column blocks; false when the kernel has no form for that shape (the caller then
// launches the parts apart).
bool mixed_launch_supported(int head_dim, pa_dtype kv_dtype, int ncb);
hipError_t launch_mixed(const DecodeArgs& dec, const DecodeArgs& pre, int head_dim, pa_dtype kv_dtype,
                        bool q_f32, int ncb, hipStream_t stream);
hipError_t launch_prefill(const DecodeArgs& a, int head_dim, pa_dtype kv_dtype, bool q_f32,
                          hipStream_t stream);
// Query rows (G heads x tokens) of one query block of the split prefill, per head_dim.
int prefill_tile_rows(int head_dim);
// The split prefill's query blocks: one workgroup per (plan slot, kv head) of a plan over the blocks
// (a as for launch_decode with context_lens, cu and bt_index describing the blocks; max_q_len the
// block's token bound), writing slot states like the decode.  bf16 or fp8 caches.
hipError_t launch_prefill_tiles(const DecodeArgs& a, int head_dim, pa_dtype kv_dtype, bool q_f32,
                                hipStream_t stream);

}  // namespace pa

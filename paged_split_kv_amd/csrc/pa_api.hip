// pa_api.hip -- the C ABI of libpa: host-side argument checks and kernel launches.
//
// Every check below runs before any launch and returns a status; nothing here allocates, copies,
// synchronises or reads device memory.
#include <limits.h>

#include <mutex>

#include "pa_device.h"

// The workspace of pa_attention_noalloc: a static device array that every device the library runs
// on holds until the process ends.  In host code the name `scratch` is a host-side stand-in, not a
// device address; host code uses only the address hipGetSymbolAddress returns for the current
// device (scratch_on_current_device).
static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool supported_head_dim(int d) { return d == 64 || d == 128 || d == 256; }
bool supported_block_size(int bs) { return bs == 16 || bs == 64 || bs == 128; }

// The kernels address a request's keys and its block-table row with 32-bit integers: every key a
// block table can reach (max_blocks_per_seq x block_size, with a chunk of slack) must fit.
bool table_reach_fits(int32_t max_blocks_per_seq, int32_t block_size) {
    return (long long)max_blocks_per_seq * block_size <= (long long)INT_MAX - 256;
}

pa_status capacity_formula(int32_t num_seqs, int32_t num_kv_heads, int32_t cu_count,
                           int32_t budget_mult, int32_t max_partitions, int32_t* out) {
    if (num_seqs < 0 || num_kv_heads < 1 || cu_count < 1 || budget_mult < 1 || max_partitions < 1)
        return PA_INVALID_ARG;
    const long long budget = ((long long)budget_mult * cu_count + num_kv_heads - 1) / num_kv_heads;
    const long long a = (long long)num_seqs * max_partitions;
    const long long b = num_seqs > budget ? (long long)num_seqs : budget;
    const long long c = a < b ? a : b;
    if (c > INT_MAX) return PA_INVALID_ARG;
    *out = (int32_t)c;
    return PA_OK;
}

pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_HIP_ERROR; }

}  // namespace

extern "C" size_t pa_workspace_bytes(int32_t capacity, int32_t max_q_len, int32_t num_q_heads, int32_t head_dim);

namespace {

// Bytes of the slot states alone (partials and (m, l) pairs), the least workspace a decode and merge
// need; 0 for invalid sizes.  pa_workspace_bytes adds the shared-slot region.
size_t slot_state_bytes(int32_t capacity, int32_t max_q_len, int32_t num_q_heads, int32_t head_dim) {
    if (capacity < 0 || max_q_len < 1 || num_q_heads < 1 || head_dim < 1) return 0;
    const unsigned long long states = (unsigned long long)capacity * max_q_len * num_q_heads;
    if (states > (1ull << 40)) return 0;
    return pa::workspace_acc_bytes(capacity, max_q_len, num_q_heads, head_dim) +
           pa::workspace_ml_bytes(capacity, max_q_len, num_q_heads);
}

}  // namespace

namespace {

pa_status check_plan(const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                     int32_t cu_count, int32_t budget_mult, int32_t max_partitions, int32_t tile_tokens,
                     int32_t sliding_window, int32_t capacity, const int32_t* work_info,
                     const int32_t* reduce_info, const int32_t* num_work, int32_t* cap) {
    if (num_seqs < 0 || tile_tokens < 1 || capacity < 0 || sliding_window < 0) return PA_INVALID_ARG;
    if (!num_work || (num_seqs > 0 && (!context_lens || !reduce_info)) || (capacity > 0 && !work_info))
        return PA_INVALID_ARG;
    if ((work_info && !aligned(work_info, 16)) || (reduce_info && !aligned(reduce_info, 8)) ||
        !aligned(num_work, 8))
        return PA_INVALID_ARG;
    if (num_seqs > PA_MAX_SEQS) return PA_UNSUPPORTED;
    const pa_status st = capacity_formula(num_seqs, num_kv_heads, cu_count, budget_mult, max_partitions, cap);
    if (st != PA_OK) return st;
    if (capacity < *cap) return PA_CAPACITY;
    return PA_OK;
}

// Checks of pa_decode; on success fills the kernel arguments and says whether there is nothing to
// decode (no slot or no request).
pa_status prepare_decode(const void* q, pa_dtype q_dtype, int32_t num_rows, int32_t num_q_heads,
                         int32_t head_dim, const void* k_cache, const void* v_cache, pa_dtype kv_dtype,
                         int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, const int32_t* cu_query_lens,
                         int32_t max_q_len, int32_t sliding_window, float scale, float k_scale,
                         float v_scale, const int32_t* work_info, const int32_t* reduce_info,
                         const int32_t* num_work, int32_t capacity, int32_t tile_tokens, void* workspace,
                         size_t workspace_bytes, void* out, pa_dtype out_dtype, pa::DecodeArgs* args,
                         bool* nothing) {
    if (num_rows < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_blocks < 0 || num_seqs < 0 ||
        max_blocks_per_seq < 0 || max_q_len < 1 || capacity < 0 || tile_tokens < 1 || head_dim < 1 ||
        block_size < 1 || sliding_window < 0)
        return PA_INVALID_ARG;
    if (q_dtype != PA_F32 && q_dtype != PA_BF16) return PA_INVALID_ARG;
    if (kv_dtype != PA_F32 && kv_dtype != PA_BF16 && kv_dtype != PA_FP8_E4M3) return PA_INVALID_ARG;
    if (num_q_heads % num_kv_heads != 0) return PA_INVALID_ARG;
    if (!cu_query_lens && (max_q_len != 1 || num_rows < num_seqs)) return PA_INVALID_ARG;
    if (!(scale == scale) || !(k_scale == k_scale) || !(v_scale == v_scale)) return PA_INVALID_ARG;
    if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PA_UNSUPPORTED;
    if (!table_reach_fits(max_blocks_per_seq, block_size)) return PA_UNSUPPORTED;
    if (tile_tokens % block_size != 0) return PA_UNSUPPORTED;
    const int group = num_q_heads / num_kv_heads;
    if ((long long)group * max_q_len > PA_MAX_GROUP_ROWS) return PA_UNSUPPORTED;
    if (capacity > 0) {
        if (!work_info || !num_work || !workspace) return PA_INVALID_ARG;
        if (num_seqs > 0 && (!q || !k_cache || !v_cache || !block_tables || !context_lens))
            return PA_INVALID_ARG;
    }
    if (out) {
        if (out_dtype != q_dtype) return PA_INVALID_ARG;
        if (num_seqs > 0 && !reduce_info) return PA_INVALID_ARG;
        if (!aligned(out, 16) || (reduce_info && !aligned(reduce_info, 8))) return PA_INVALID_ARG;
        if ((long long)num_rows * num_q_heads > (long long)INT_MAX) return PA_UNSUPPORTED;
    }
    if ((q && !aligned(q, 16)) || (k_cache && !aligned(k_cache, 16)) || (v_cache && !aligned(v_cache, 16)) ||
        (work_info && !aligned(work_info, 16)) || (workspace && !aligned(workspace, 256)) ||
        (num_work && !aligned(num_work, 8)))
        return PA_INVALID_ARG;
    // the slot states must fit; the shared-slot region is used only when it fits too
    const size_t need = slot_state_bytes(capacity, max_q_len, num_q_heads, head_dim);
    if (capacity > 0 && (need == 0 || workspace_bytes < need)) return PA_CAPACITY;
    *nothing = capacity == 0 || num_seqs == 0;

    pa::DecodeArgs& a = *args;
    a = pa::DecodeArgs{};
    a.q = q;
    a.k_cache = static_cast<const uint8_t*>(k_cache);
    a.v_cache = static_cast<const uint8_t*>(v_cache);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.cu = cu_query_lens;
    a.work_info = reinterpret_cast<const int4*>(work_info);
    a.num_work = num_work;
    a.ws_acc = static_cast<float*>(workspace);
    const size_t acc_bytes = pa::workspace_acc_bytes(capacity, max_q_len, num_q_heads, head_dim);
    a.ws_ml = workspace ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + acc_bytes) : nullptr;
    a.out = nullptr;                  // the decode writes partial states; a merge launch writes out
    a.out_bf16 = out_dtype == PA_BF16 ? 1 : 0;
    a.num_rows = num_rows;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = group;
    a.num_blocks = num_blocks;
    a.block_size = block_size;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.max_q_len = max_q_len;
    a.capacity = capacity;
    a.tile_tokens = tile_tokens;
    a.score_scale_log2 = scale * k_scale * pa::kLog2e;
    a.v_scale = v_scale;
    a.window = sliding_window;
    return PA_OK;
}

pa_status prepare_merge(int32_t num_rows, int32_t num_q_heads, int32_t head_dim, int32_t num_seqs,
                        const int32_t* cu_query_lens, int32_t max_q_len, const int32_t* reduce_info,
                        int32_t capacity, const void* workspace, size_t workspace_bytes, void* out,
                        pa_dtype out_dtype, pa::MergeArgs* args) {
    if (num_rows < 0 || num_q_heads < 1 || num_seqs < 0 || max_q_len < 1 || capacity < 0)
        return PA_INVALID_ARG;
    if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_INVALID_ARG;
    if (!cu_query_lens && max_q_len != 1) return PA_INVALID_ARG;
    if (!supported_head_dim(head_dim)) return PA_UNSUPPORTED;
    if (num_rows > 0 && !out) return PA_INVALID_ARG;
    if (num_seqs > 0 && (!reduce_info || (capacity > 0 && !workspace))) return PA_INVALID_ARG;
    if ((reduce_info && !aligned(reduce_info, 8)) || (workspace && !aligned(workspace, 256)) ||
        (out && !aligned(out, 16)))
        return PA_INVALID_ARG;
    // the slot states must fit; the shared-slot region is used only when it fits too
    const size_t need = slot_state_bytes(capacity, max_q_len, num_q_heads, head_dim);
    if (capacity > 0 && (need == 0 || workspace_bytes < need)) return PA_CAPACITY;
    if ((long long)num_rows * num_q_heads > (long long)INT_MAX) return PA_UNSUPPORTED;

    pa::MergeArgs& a = *args;
    a = pa::MergeArgs{};
    a.cu = cu_query_lens;
    a.reduce_info = reinterpret_cast<const int2*>(reduce_info);
    a.ws_acc = static_cast<const float*>(workspace);
    a.ws_ml = workspace ? reinterpret_cast<const float*>(
                              static_cast<const uint8_t*>(workspace) +
                              pa::workspace_acc_bytes(capacity, max_q_len, num_q_heads, head_dim))
                        : nullptr;
    a.out = out;
    a.num_rows = num_rows;
    a.num_q_heads = num_q_heads;
    a.num_seqs = (capacity > 0) ? num_seqs : 0;   // without slots every row is zero
    a.max_q_len = max_q_len;
    a.capacity = capacity;
    return PA_OK;
}

// Shared slots: with every request one slot (capacity <= batch) slot sizes follow the request
// lengths, and the longest request alone would set the time.  When head_dim <= 128, the batch is at
// most PA_INLINE_PLAN_SEQS requests and the workspace holds the shared-slot region, the decode cuts
// each slot into pieces, one workgroup each, and the merge folds a request's pieces like slots.  `one_slot_cap` is the capacity that decides
// "one slot each": the plan's capacity for pa_decode, the capacity formula's value for pa_attention's
// in-place plan.  pa_merge decides with its own arguments (pa::shares_slots), which are the same.
bool share_slots(pa::DecodeArgs& d, int head_dim, int one_slot_cap, void* workspace, size_t workspace_bytes) {
    if (d.prefill ||
        !pa::shares_slots(one_slot_cap, d.num_seqs, head_dim, d.capacity, d.max_q_len, d.num_q_heads, workspace_bytes))
        return false;
    const pa::SharedRegion r = pa::shared_region(d.capacity, d.max_q_len, d.num_q_heads, head_dim);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    d.pieces = pa::kPieceFactor;
    d.plan_slots = d.capacity;
    d.capacity = pa::piece_bound(d.capacity);
    d.ws_acc = reinterpret_cast<float*>(ws + r.acc);
    d.ws_ml = reinterpret_cast<float*>(ws + r.ml);
    d.piece_reduce_out = reinterpret_cast<int2*>(ws + r.reduce);
    return true;
}

// The merge of shared slots: each request's pieces, from the shared-slot region.
void merge_pieces(pa::MergeArgs& m, int head_dim, const void* workspace) {
    const pa::SharedRegion r = pa::shared_region(m.capacity, m.max_q_len, m.num_q_heads, head_dim);
    const uint8_t* ws = static_cast<const uint8_t*>(workspace);
    m.reduce_info = reinterpret_cast<const int2*>(ws + r.reduce);
    m.ws_acc = reinterpret_cast<const float*>(ws + r.acc);
    m.ws_ml = reinterpret_cast<const float*>(ws + r.ml);
    m.capacity = pa::piece_bound(m.capacity);
}

}  // namespace

namespace {

// Checks of pa_prefill; on success fills the kernel arguments.  block_tokens 0 takes the kernel's own
// block size (prefill_block_tokens).
pa_status prepare_prefill(const void* q, pa_dtype q_dtype, int32_t num_rows, int32_t num_q_heads,
                          int32_t head_dim, const void* k_cache, const void* v_cache, pa_dtype kv_dtype,
                          int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs, const int32_t* cu_query_lens,
                          int32_t sliding_window, float scale, float k_scale, float v_scale, void* out,
                          pa_dtype out_dtype, int block_tokens, pa::DecodeArgs* args) {
    if (num_rows < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_blocks < 0 || num_seqs < 0 ||
        max_blocks_per_seq < 0 || head_dim < 1 || block_size < 1 || sliding_window < 0)
        return PA_INVALID_ARG;
    if (q_dtype != PA_F32 && q_dtype != PA_BF16) return PA_INVALID_ARG;
    if (kv_dtype != PA_F32 && kv_dtype != PA_BF16 && kv_dtype != PA_FP8_E4M3) return PA_INVALID_ARG;
    if (out_dtype != q_dtype || num_q_heads % num_kv_heads != 0) return PA_INVALID_ARG;
    if (!(scale == scale) || !(k_scale == k_scale) || !(v_scale == v_scale)) return PA_INVALID_ARG;
    if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PA_UNSUPPORTED;
    if (!table_reach_fits(max_blocks_per_seq, block_size)) return PA_UNSUPPORTED;
    if (kv_dtype == PA_F32) return PA_UNSUPPORTED;
    const int group = num_q_heads / num_kv_heads;
    if (group > PA_MAX_GROUP_ROWS) return PA_UNSUPPORTED;
    if (!cu_query_lens || (num_rows > 0 && (!q || !out))) return PA_INVALID_ARG;
    if (num_seqs > 0 && (!k_cache || !v_cache || !block_tables || !context_lens)) return PA_INVALID_ARG;
    if ((q && !aligned(q, 16)) || (out && !aligned(out, 16)) || (k_cache && !aligned(k_cache, 16)) ||
        (v_cache && !aligned(v_cache, 16)))
        return PA_INVALID_ARG;
    if ((long long)num_rows * num_q_heads > (long long)INT_MAX) return PA_UNSUPPORTED;

    const int lb = block_tokens > 0 ? block_tokens : pa::prefill_block_tokens(head_dim, group);
    // blocks of all requests together: sum ceil(L_b / lb) <= num_rows / lb + num_seqs
    const long long blocks = (num_rows + lb - 1) / lb + (long long)num_seqs;
    if (blocks * num_kv_heads > (long long)INT_MAX / 2) return PA_UNSUPPORTED;
    pa::DecodeArgs& a = *args;
    a = pa::DecodeArgs{};
    a.q = q;
    a.k_cache = static_cast<const uint8_t*>(k_cache);
    a.v_cache = static_cast<const uint8_t*>(v_cache);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.cu = cu_query_lens;
    a.out = out;
    a.out_bf16 = out_dtype == PA_BF16 ? 1 : 0;
    a.num_rows = num_rows;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = group;
    a.num_blocks = num_blocks;
    a.block_size = block_size;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.max_q_len = lb;
    a.capacity = static_cast<int>(blocks);
    a.tile_tokens = 256;
    a.score_scale_log2 = scale * k_scale * pa::kLog2e;
    a.v_scale = v_scale;
    a.window = sliding_window;
    a.prefill = 1;
    a.block_tokens = lb;
    return PA_OK;
}

}  // namespace

namespace {

// The split prefill: each request's query tokens are cut into blocks of up to 64 query rows (32 at
// head_dim 256; block_tokens tokens of G query heads), and the blocks are planned, decoded and merged
// as pseudo-requests, so a block's keys spread over several workgroups like a long decode request's.
// Measured on a 512-token chunk behind a 16384-token prefix (Hq 12 / Hkv 2, head_dim 256): blocks of
// 16, 32 and 64 rows took 632, 404 and 496 us.
// Workspace regions, each 256-byte aligned: per-block lengths, first rows (max_blocks + 1) and
// request indices; the plan over the blocks (work_info [capacity], reduce_info [max_blocks],
// num_work [2]); the slot states of that plan.
// Workgroup budget of the split prefill's plan over query blocks, in workgroups per compute unit: the
// block kernel holds one workgroup per compute unit, so its slots run in one round.
constexpr int kPrefillBudget = 1;

struct PrefillLayout {
    int block_tokens, max_blocks, capacity;
    size_t blk_ctx, blk_cu, blk_req, work, reduce, num_work, states, end;
};

bool prefill_layout(int32_t num_rows, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t cu_count, PrefillLayout* L) {
    if (num_rows < 0 || num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 || cu_count < 1 ||
        num_q_heads % num_kv_heads != 0)
        return false;
    const int group = num_q_heads / num_kv_heads;
    if (group > PA_MAX_GROUP_ROWS) return false;
    L->block_tokens = pa::prefill_tile_rows(head_dim) / group;
    if (L->block_tokens < 1) L->block_tokens = 1;
    // blocks: sum over requests of ceil(L_b / T) <= num_rows / T + num_seqs
    const long long nb = ((long long)num_rows + L->block_tokens - 1) / L->block_tokens + num_seqs;
    if (nb > PA_MAX_SEQS) return false;
    L->max_blocks = (int)nb;
    int32_t cap = 0;
    if (capacity_formula(L->max_blocks, num_kv_heads, cu_count, kPrefillBudget, 256, &cap) != PA_OK) return false;
    L->capacity = cap;
    size_t at = 0;
    auto region = [&](size_t bytes) {
        const size_t here = at;
        at += pa::align256(bytes);
        return here;
    };
    L->blk_ctx = region(sizeof(int32_t) * (size_t)nb);
    L->blk_cu = region(sizeof(int32_t) * ((size_t)nb + 1));
    L->blk_req = region(sizeof(int32_t) * (size_t)nb);
    L->work = region(sizeof(int32_t) * 4 * (size_t)cap);
    L->reduce = region(sizeof(int32_t) * 2 * (size_t)nb);
    L->num_work = region(sizeof(int32_t) * 2);
    const size_t states = slot_state_bytes(cap, L->block_tokens, num_q_heads, head_dim);
    if (states == 0 && cap > 0) return false;
    L->states = region(states);
    L->end = at;
    return true;
}

}  // namespace

extern "C" {

size_t pa_prefill_workspace_bytes(int32_t num_rows, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t cu_count) {
    PrefillLayout L;
    return prefill_layout(num_rows, num_seqs, num_q_heads, num_kv_heads, head_dim, cu_count, &L) ? L.end : 0;
}

pa_status pa_plan_capacity(int32_t num_seqs, int32_t num_kv_heads, int32_t cu_count,
                           int32_t budget_mult, int32_t max_partitions, int32_t* capacity_out) {
    if (!capacity_out) return PA_INVALID_ARG;
    return capacity_formula(num_seqs, num_kv_heads, cu_count, budget_mult, max_partitions, capacity_out);
}

size_t pa_workspace_bytes(int32_t capacity, int32_t max_q_len, int32_t num_q_heads, int32_t head_dim) {
    const size_t slots = slot_state_bytes(capacity, max_q_len, num_q_heads, head_dim);
    if (slots == 0 || capacity == 0) return slots;
    // then the shared-slot region (up to three times as many piece states)
    return pa::shared_region(capacity, max_q_len, num_q_heads, head_dim).end;
}

pa_status pa_plan(const int32_t* context_lens, const int32_t* cu_query_lens, int32_t num_seqs,
                  int32_t num_kv_heads, int32_t cu_count, int32_t budget_mult, int32_t max_partitions,
                  int32_t tile_tokens, int32_t sliding_window, int32_t capacity, int32_t* work_info,
                  int32_t* reduce_info, int32_t* num_work, int32_t* dispatch_info, void* stream) {
    int32_t cap = 0;
    const pa_status st = check_plan(context_lens, num_seqs, num_kv_heads, cu_count, budget_mult,
                                    max_partitions, tile_tokens, sliding_window, capacity, work_info,
                                    reduce_info, num_work, &cap);
    if (st != PA_OK) return st;
    if (dispatch_info && !aligned(dispatch_info, 16)) return PA_INVALID_ARG;
    return from_hip(pa::launch_plan(context_lens, cu_query_lens, num_seqs, cap, capacity, max_partitions,
                                    tile_tokens, sliding_window, work_info, reduce_info, num_work, dispatch_info,
                                    pa::as_stream(stream)));
}

pa_status pa_decode(const void* q, pa_dtype q_dtype, int32_t num_rows, int32_t num_q_heads,
                    int32_t head_dim, const void* k_cache, const void* v_cache, pa_dtype kv_dtype,
                    int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, const int32_t* cu_query_lens,
                    int32_t max_q_len, int32_t sliding_window, float scale, float k_scale,
                    float v_scale, const int32_t* work_info, const int32_t* reduce_info,
                    const int32_t* num_work, const int32_t* dispatch_info, int32_t capacity, int32_t tile_tokens,
                    void* workspace, size_t workspace_bytes, void* out, pa_dtype out_dtype, void* stream) {
    pa::DecodeArgs a;
    bool nothing = false;
    const pa_status st = prepare_decode(q, q_dtype, num_rows, num_q_heads, head_dim, k_cache, v_cache,
                                        kv_dtype, num_blocks, num_kv_heads, block_size, block_tables,
                                        max_blocks_per_seq, context_lens, num_seqs, cu_query_lens,
                                        max_q_len, sliding_window, scale, k_scale, v_scale, work_info,
                                        reduce_info, num_work, capacity, tile_tokens, workspace,
                                        workspace_bytes, out, out_dtype, &a, &nothing);
    if (st != PA_OK) return st;
    if (dispatch_info && !aligned(dispatch_info, 16)) return PA_INVALID_ARG;
    a.dispatch_info = reinterpret_cast<const int4*>(dispatch_info);
    if (out) {
        // the merge's own checks too, so that a failure launches nothing
        pa::MergeArgs m;
        const pa_status sm = prepare_merge(num_rows, num_q_heads, head_dim, num_seqs, cu_query_lens, max_q_len,
                                           reduce_info, capacity, workspace, workspace_bytes, out, out_dtype, &m);
        if (sm != PA_OK) return sm;
    }
    if (nothing) {
        if (!out || num_rows == 0) return PA_OK;
        // nothing to decode: the merge's contract still writes every row (all zero here)
        return pa_merge(num_rows, num_q_heads, head_dim, 0, nullptr, 1, nullptr, 0, nullptr, 0, out,
                        out_dtype, stream);
    }
    share_slots(a, head_dim, capacity, workspace, workspace_bytes);
    const pa_status sd = from_hip(pa::launch_decode(a, head_dim, kv_dtype, q_dtype == PA_F32, pa::as_stream(stream)));
    if (sd != PA_OK || !out || num_rows == 0) return sd;
    // with out: the merge launch on the same stream, exactly as pa_merge with the same arguments
    return pa_merge(num_rows, num_q_heads, head_dim, num_seqs, cu_query_lens, max_q_len, reduce_info, capacity,
                    workspace, workspace_bytes, out, out_dtype, stream);
}

pa_status pa_merge(int32_t num_rows, int32_t num_q_heads, int32_t head_dim, int32_t num_seqs,
                   const int32_t* cu_query_lens, int32_t max_q_len, const int32_t* reduce_info,
                   int32_t capacity, const void* workspace, size_t workspace_bytes, void* out,
                   pa_dtype out_dtype, void* stream) {
    pa::MergeArgs a;
    const pa_status st = prepare_merge(num_rows, num_q_heads, head_dim, num_seqs, cu_query_lens,
                                       max_q_len, reduce_info, capacity, workspace, workspace_bytes, out,
                                       out_dtype, &a);
    if (st != PA_OK || num_rows == 0) return st;
    // pieces where pa_decode, given the same arguments, shared the slots
    if (a.num_seqs > 0 &&
        pa::shares_slots(capacity, num_seqs, head_dim, capacity, max_q_len, num_q_heads, workspace_bytes))
        merge_pieces(a, head_dim, workspace);
    return from_hip(pa::launch_merge(a, head_dim, out_dtype == PA_BF16, pa::as_stream(stream)));
}

pa_status pa_attention(const void* q, pa_dtype q_dtype, int32_t num_rows, int32_t num_q_heads,
                       int32_t head_dim, const void* k_cache, const void* v_cache, pa_dtype kv_dtype,
                       int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t num_seqs, const int32_t* cu_query_lens,
                       int32_t max_q_len, int32_t sliding_window, float scale, float k_scale,
                       float v_scale, int32_t cu_count, int32_t budget_mult, int32_t max_partitions,
                       int32_t tile_tokens, int32_t capacity, int32_t* work_info,
                       int32_t* reduce_info, int32_t* num_work, void* workspace,
                       size_t workspace_bytes, void* out, pa_dtype out_dtype, void* stream) {
    // every check of the three calls first, so a failure launches nothing
    int32_t cap = 0;
    pa_status st = check_plan(context_lens, num_seqs, num_kv_heads, cu_count, budget_mult,
                              max_partitions, tile_tokens, sliding_window, capacity, work_info,
                              reduce_info, num_work, &cap);
    if (st != PA_OK) return st;
    pa::DecodeArgs d;
    bool nothing = false;
    st = prepare_decode(q, q_dtype, num_rows, num_q_heads, head_dim, k_cache, v_cache, kv_dtype,
                        num_blocks, num_kv_heads, block_size, block_tables, max_blocks_per_seq,
                        context_lens, num_seqs, cu_query_lens, max_q_len, sliding_window, scale,
                        k_scale, v_scale, work_info, reduce_info, num_work, capacity, tile_tokens,
                        workspace, workspace_bytes, nullptr, q_dtype, &d, &nothing);
    if (st != PA_OK) return st;
    if (out_dtype != q_dtype) return PA_INVALID_ARG;
    pa::MergeArgs m;
    st = prepare_merge(num_rows, num_q_heads, head_dim, num_seqs, cu_query_lens, max_q_len, reduce_info,
                       capacity, workspace, workspace_bytes, out, out_dtype, &m);
    if (st != PA_OK) return st;

    hipStream_t s = pa::as_stream(stream);
    const bool in_place = !nothing && kv_dtype != PA_F32 && num_seqs <= PA_INLINE_PLAN_SEQS;
    if (in_place) {
        d.plan_inline = 1;
        d.plan_cap = cap;
        d.max_partitions = max_partitions;
        d.plan_slots = capacity;
        d.plan_work_out = reinterpret_cast<int4*>(work_info);
        d.plan_reduce_out = reinterpret_cast<int2*>(reduce_info);
        d.plan_num_work_out = num_work;
        if (share_slots(d, head_dim, cap, workspace, workspace_bytes)) merge_pieces(m, head_dim, workspace);
    } else {
        if (!nothing && share_slots(d, head_dim, capacity, workspace, workspace_bytes))
            merge_pieces(m, head_dim, workspace);
        st = from_hip(pa::launch_plan(context_lens, cu_query_lens, num_seqs, cap, capacity, max_partitions,
                                      tile_tokens, sliding_window, work_info, reduce_info, num_work, nullptr, s));
        if (st != PA_OK) return st;
    }
    if (!nothing) {
        st = from_hip(pa::launch_decode(d, head_dim, kv_dtype, q_dtype == PA_F32, s));
        if (st != PA_OK) return st;
    }
    if (num_rows == 0) return PA_OK;
    return from_hip(pa::launch_merge(m, head_dim, out_dtype == PA_BF16, s));
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The current device's copy of `scratch`: its address is looked up with hipGetSymbolAddress the first
// time a call is made with that device current, checked, and kept for later calls.
pa_status scratch_on_current_device(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return PA_HIP_ERROR;
    if (dev < 0 || dev >= kMaxDevices) return PA_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PA_HIP_ERROR;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_attention_noalloc(const void* q, pa_dtype q_dtype, int32_t num_rows, int32_t num_q_heads,
                               int32_t head_dim, const void* k_cache, const void* v_cache, pa_dtype kv_dtype,
                               int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs, const int32_t* cu_query_lens,
                               int32_t max_q_len, int32_t sliding_window, float scale, float k_scale,
                               float v_scale, int32_t cu_count, int32_t budget_mult, int32_t max_partitions,
                               int32_t tile_tokens, int32_t capacity, int32_t* work_info,
                               int32_t* reduce_info, int32_t* num_work, void* out, pa_dtype out_dtype,
                               void* stream) {
    // the whole workspace when it fits the array, else the slot states alone (no shared slots)
    size_t bytes = pa_workspace_bytes(capacity, max_q_len, num_q_heads, head_dim);
    if (bytes > PA_NOALLOC_SCRATCH_BYTES) bytes = slot_state_bytes(capacity, max_q_len, num_q_heads, head_dim);
    if (bytes > PA_NOALLOC_SCRATCH_BYTES) return PA_CAPACITY;
    void* ws = nullptr;
    const pa_status st = scratch_on_current_device(&ws);
    if (st != PA_OK) return st;
    return pa_attention(q, q_dtype, num_rows, num_q_heads, head_dim, k_cache, v_cache, kv_dtype, num_blocks,
                        num_kv_heads, block_size, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                        cu_query_lens, max_q_len, sliding_window, scale, k_scale, v_scale, cu_count, budget_mult,
                        max_partitions, tile_tokens, capacity, work_info, reduce_info, num_work, ws, bytes, out,
                        out_dtype, stream);
}

pa_status pa_prefill(const void* q, pa_dtype q_dtype, int32_t num_rows, int32_t num_q_heads,
                     int32_t head_dim, const void* k_cache, const void* v_cache, pa_dtype kv_dtype,
                     int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t num_seqs, const int32_t* cu_query_lens,
                     int32_t sliding_window, float scale, float k_scale, float v_scale, int32_t cu_count,
                     void* workspace, size_t workspace_bytes, void* out, pa_dtype out_dtype, void* stream) {
    // the checks of the prefill rows (the single-launch form's argument block is not used here)
    pa::DecodeArgs p;
    pa_status st = prepare_prefill(q, q_dtype, num_rows, num_q_heads, head_dim, k_cache, v_cache, kv_dtype,
                                   num_blocks, num_kv_heads, block_size, block_tables, max_blocks_per_seq,
                                   context_lens, num_seqs, cu_query_lens, sliding_window, scale, k_scale, v_scale,
                                   out, out_dtype, 0, &p);
    if (st != PA_OK) return st;
    if (!workspace) {
        // no workspace: each query block one workgroup streaming all its keys, in one launch
        if (num_rows == 0) return PA_OK;
        return from_hip(pa::launch_prefill(p, head_dim, kv_dtype, q_dtype == PA_F32, pa::as_stream(stream)));
    }
    if (cu_count < 1) return PA_INVALID_ARG;
    PrefillLayout L;
    if (!prefill_layout(num_rows, num_seqs, num_q_heads, num_kv_heads, head_dim, cu_count, &L)) return PA_UNSUPPORTED;
    if (!aligned(workspace, 256)) return PA_INVALID_ARG;
    if (workspace_bytes < L.end) return PA_CAPACITY;
    if (num_rows == 0) return PA_OK;

    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int32_t* blk_ctx = reinterpret_cast<int32_t*>(ws + L.blk_ctx);
    int32_t* blk_cu = reinterpret_cast<int32_t*>(ws + L.blk_cu);
    int32_t* blk_req = reinterpret_cast<int32_t*>(ws + L.blk_req);
    int32_t* work = reinterpret_cast<int32_t*>(ws + L.work);
    int32_t* reduce = reinterpret_cast<int32_t*>(ws + L.reduce);
    int32_t* num_work = reinterpret_cast<int32_t*>(ws + L.num_work);
    float* states = reinterpret_cast<float*>(ws + L.states);
    const hipStream_t s = pa::as_stream(stream);
    // one launch cuts the query blocks and plans them
    const pa::PlanBlocks blocks{context_lens, cu_query_lens, num_seqs, L.block_tokens, blk_ctx, blk_cu, blk_req};
    st = from_hip(pa::launch_plan(blk_ctx, blk_cu, L.max_blocks, L.capacity, L.capacity, 256, 256, sliding_window,
                                  work, reduce, num_work, nullptr, s, &blocks));
    if (st != PA_OK) return st;

    pa::DecodeArgs d = pa::DecodeArgs{};
    d.q = q;
    d.k_cache = static_cast<const uint8_t*>(k_cache);
    d.v_cache = static_cast<const uint8_t*>(v_cache);
    d.block_tables = block_tables;
    d.context_lens = blk_ctx;
    d.cu = blk_cu;
    d.bt_index = blk_req;
    d.work_info = reinterpret_cast<const int4*>(work);
    d.num_work = num_work;
    d.ws_acc = states;
    d.ws_ml = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(states) +
                                       pa::workspace_acc_bytes(L.capacity, L.block_tokens, num_q_heads, head_dim));
    d.out_bf16 = out_dtype == PA_BF16 ? 1 : 0;
    d.num_rows = num_rows;
    d.num_q_heads = num_q_heads;
    d.num_kv_heads = num_kv_heads;
    d.group = num_q_heads / num_kv_heads;
    d.num_blocks = num_blocks;
    d.block_size = block_size;
    d.max_blocks = max_blocks_per_seq;
    d.num_seqs = L.max_blocks;
    d.max_q_len = L.block_tokens;
    d.capacity = L.capacity;
    d.tile_tokens = 256;
    d.score_scale_log2 = scale * k_scale * pa::kLog2e;
    d.v_scale = v_scale;
    d.window = sliding_window;
    st = from_hip(pa::launch_prefill_tiles(d, head_dim, kv_dtype, q_dtype == PA_F32, s));
    if (st != PA_OK) return st;

    pa::MergeArgs m = pa::MergeArgs{};
    m.cu = blk_cu;
    m.reduce_info = reinterpret_cast<const int2*>(reduce);
    m.ws_acc = d.ws_acc;
    m.ws_ml = d.ws_ml;
    m.row_floor = cu_query_lens;             // rows before the first request's belong to other calls
    m.out = out;
    m.num_rows = num_rows;
    m.num_q_heads = num_q_heads;
    m.num_seqs = L.max_blocks;
    m.max_q_len = L.block_tokens;
    m.capacity = L.capacity;
    return from_hip(pa::launch_merge(m, head_dim, out_dtype == PA_BF16, s));
}

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
                             size_t workspace_bytes, void* out, pa_dtype out_dtype, void* stream) {
    if (num_seqs < 0 || num_decodes < 0 || num_decodes > num_seqs || num_rows < 0 ||
        num_decode_rows < 0 || num_decode_rows > num_rows || max_blocks_per_seq < 0)
        return PA_INVALID_ARG;
    if (!cu_query_lens) return PA_INVALID_ARG;
    // all requests are decodes, or none is: one of the two entry points alone
    if (num_decodes == num_seqs)
        return pa_attention(q, q_dtype, num_rows, num_q_heads, head_dim, k_cache, v_cache, kv_dtype,
                            num_blocks, num_kv_heads, block_size, block_tables, max_blocks_per_seq,
                            context_lens, num_seqs, cu_query_lens, max_q_len, sliding_window, scale,
                            k_scale, v_scale, cu_count, budget_mult, max_partitions, tile_tokens, capacity,
                            work_info, reduce_info, num_work, workspace, workspace_bytes, out, out_dtype,
                            stream);
    if (num_decodes == 0) {
        // prompts only: their query blocks in one launch, each block one partition (no workspace)
        pa::DecodeArgs p;
        const pa_status sp = prepare_prefill(q, q_dtype, num_rows, num_q_heads, head_dim, k_cache, v_cache,
                                             kv_dtype, num_blocks, num_kv_heads, block_size, block_tables,
                                             max_blocks_per_seq, context_lens, num_seqs, cu_query_lens,
                                             sliding_window, scale, k_scale, v_scale, out, out_dtype, 0, &p);
        if (sp != PA_OK || num_rows == 0) return sp;
        return from_hip(pa::launch_prefill(p, head_dim, kv_dtype, q_dtype == PA_F32, pa::as_stream(stream)));
    }

    // the decode part: requests [0, num_decodes), rows [0, num_decode_rows), planned in place
    int32_t cap = 0;
    pa_status st = check_plan(context_lens, num_decodes, num_kv_heads, cu_count, budget_mult,
                              max_partitions, tile_tokens, sliding_window, capacity, work_info,
                              reduce_info, num_work, &cap);
    if (st != PA_OK) return st;
    pa::DecodeArgs d;
    bool nothing = false;
    st = prepare_decode(q, q_dtype, num_decode_rows, num_q_heads, head_dim, k_cache, v_cache, kv_dtype,
                        num_blocks, num_kv_heads, block_size, block_tables, max_blocks_per_seq,
                        context_lens, num_decodes, cu_query_lens, max_q_len, sliding_window, scale,
                        k_scale, v_scale, work_info, reduce_info, num_work, capacity, tile_tokens,
                        workspace, workspace_bytes, nullptr, q_dtype, &d, &nothing);
    if (st != PA_OK) return st;
    if (out_dtype != q_dtype) return PA_INVALID_ARG;
    pa::MergeArgs m;
    st = prepare_merge(num_decode_rows, num_q_heads, head_dim, num_decodes, cu_query_lens, max_q_len,
                       reduce_info, capacity, workspace, workspace_bytes, out, out_dtype, &m);
    if (st != PA_OK) return st;

    // the prompts: requests [num_decodes, num_seqs), absolute rows of q and out (rows past the last
    // cumulative length are written as zeros)
    const int group = num_q_heads / num_kv_heads;
    const int ncb_dec = pa::column_blocks(group * max_q_len);
    const int lb_own = pa::prefill_block_tokens(head_dim, group);
    // one launch when the prompts' query blocks fit the decode's column blocks, or can be cut to fit
    // while few (at most 64 prompt rows: smaller blocks each read all their keys again)
    int lb = 0;
    if (pa::column_blocks(group * lb_own) == ncb_dec) lb = lb_own;
    else if (num_rows - num_decode_rows <= 64 && 16 * ncb_dec >= group) lb = 16 * ncb_dec / group;
    const bool in_place = !nothing && kv_dtype != PA_F32 && num_decodes <= PA_INLINE_PLAN_SEQS;
    const bool fused = in_place && lb > 0 && pa::mixed_launch_supported(head_dim, kv_dtype, ncb_dec);
    const size_t bt_off = (size_t)num_decodes * (size_t)max_blocks_per_seq;
    pa::DecodeArgs p;
    st = prepare_prefill(q, q_dtype, num_rows, num_q_heads, head_dim, k_cache, v_cache, kv_dtype,
                         num_blocks, num_kv_heads, block_size, block_tables ? block_tables + bt_off : nullptr,
                         max_blocks_per_seq, context_lens + num_decodes, num_seqs - num_decodes,
                         cu_query_lens + num_decodes, sliding_window, scale, k_scale, v_scale, out, out_dtype,
                         fused ? lb : 0, &p);
    if (st != PA_OK) return st;

    hipStream_t s = pa::as_stream(stream);
    if (in_place) {
        d.plan_inline = 1;
        d.plan_cap = cap;
        d.max_partitions = max_partitions;
        d.plan_slots = capacity;
        d.plan_work_out = reinterpret_cast<int4*>(work_info);
        d.plan_reduce_out = reinterpret_cast<int2*>(reduce_info);
        d.plan_num_work_out = num_work;
    } else {
        st = from_hip(pa::launch_plan(context_lens, cu_query_lens, num_decodes, cap, capacity, max_partitions,
                                      tile_tokens, sliding_window, work_info, reduce_info, num_work, nullptr, s));
        if (st != PA_OK) return st;
    }
    if (fused) {
        st = from_hip(pa::launch_mixed(d, p, head_dim, kv_dtype, q_dtype == PA_F32, ncb_dec, s));
        if (st != PA_OK) return st;
    } else {
        if (!nothing) {
            st = from_hip(pa::launch_decode(d, head_dim, kv_dtype, q_dtype == PA_F32, s));
            if (st != PA_OK) return st;
        }
        if (num_rows > 0) {
            st = from_hip(pa::launch_prefill(p, head_dim, kv_dtype, q_dtype == PA_F32, s));
            if (st != PA_OK) return st;
        }
    }
    if (num_decode_rows == 0) return PA_OK;
    return from_hip(pa::launch_merge(m, head_dim, out_dtype == PA_BF16, s));
}

pa_status pa_split_decode_first(const int32_t* cu_query_lens_host, int32_t num_seqs, int32_t threshold,
                                int32_t* num_decodes, int32_t* num_decode_tokens) {
    if (num_seqs < 0 || threshold < 1 || !num_decodes || !num_decode_tokens) return PA_INVALID_ARG;
    if (num_seqs > 0 && !cu_query_lens_host) return PA_INVALID_ARG;
    int32_t nd = 0;
    while (nd < num_seqs && cu_query_lens_host[nd + 1] - cu_query_lens_host[nd] <= threshold) ++nd;
    *num_decodes = nd;
    *num_decode_tokens = num_seqs > 0 ? cu_query_lens_host[nd] - cu_query_lens_host[0] : 0;
    return PA_OK;
}

const char* pa_status_string(pa_status status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_INVALID_ARG: return "invalid argument";
        case PA_UNSUPPORTED: return "unsupported configuration";
        case PA_CAPACITY: return "plan capacity or workspace too small";
        case PA_HIP_ERROR: return "HIP runtime error";
        default: return "unknown status";
    }
}

pa_status pa_device_cu_count(int32_t device, int32_t* cu_count_out) {
    if (!cu_count_out) return PA_INVALID_ARG;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
        return PA_HIP_ERROR;
    *cu_count_out = v;
    return PA_OK;
}

}  // extern "C"

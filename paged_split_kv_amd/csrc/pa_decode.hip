// pa_decode.hip -- split-KV grouped-query paged decode on gfx950 (MI355X).
//
// What is computed (opengfx1030/vllm-rdna PR #29, Change item 1; ROCm/ATOM PR #2366 sections 1 and 3):
// for every plan slot w = (request b, tiles [tb, te)) and kv head g, the softmax state of the keys
// [tb*T, min(te*T, S_b)) for each query token i of request b (visible keys [0, S_b - (L_b-1-i))) and
// each query head of group g.  The state (running max m in base-2 units, sum l, unnormalised acc)
// goes to the workspace; pa_merge combines a request's slots.
//
// Design (bf16 / fp8 caches, the matrix-core kernel):
//  * one workgroup of NW waves (4; 8 when every request is one slot) per (slot, kv head).  The
//    slot's keys are cut into 16-key chunks (a chunk never straddles a page: pages hold 16, 64 or
//    128 tokens and slots start on tile boundaries); wave w takes units w, w+NW, ... of consecutive
//    chunks.  When the plan's largest slot gives each of its waves at least kEvenDealChunks chunks
//    (launches long enough to be bound by bandwidth), and in the 8-wave form, the unit is the slot
//    itself split NW ways, so every slot streams on all its waves from the start; otherwise it is the
//    largest slot split NW ways, so a small slot runs fewer, fully loaded waves and its loads do not
//    delay the largest slot's in a latency-bound launch.  The NW states merge in LDS at the end.
//  * when every request is one slot, pa_attention's in-place plan can also cut the slots into pieces
//    of about half the mean slot, one workgroup each (shared slots, see piece_size): the states are
//    then per piece, the merge folds a request's pieces, and the piece-size bound stands for the
//    largest slot in the choice of dealing.
//  * all query rows of the group -- G heads x L verify tokens, M = G*L <= 64 -- form the columns
//    of 16-wide MFMA blocks, so each K/V byte is read from HBM once per (slot, kv head) whatever L is.
//  * each chunk's K and V (16 x D each) are fetched PF chunks ahead into registers with 16-byte
//    coalesced non-temporal buffer loads, written to a per-wave LDS buffer with an XOR swizzle on
//    the 16-byte column, and read back in matrix-core operand order.  Rows past the slot's last key
//    are written as zeros, so whatever a page holds past the context (even NaN) never reaches the
//    products.
//  * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16: output lane l holds query row (l & 15) and keys
//    4*(l >> 4) + j, so the per-row softmax max needs only 2 cross-lane steps (gfx950 row swaps)
//    and the probabilities are already in the B-operand order of O^T = V^T . P^T (16x16x16, or
//    16x16x32 over two chunks at once), whose output lane again holds query row (l & 15): the
//    per-row rescale factors stay in-lane.
//  * head_dim 256 instead splits the head dimension across groups of two waves (four at four row
//    blocks; see Mfma::DS), so two workgroups per CU fit without spilling.
//  * fp8 (OCP e4m3fn) codes are widened exactly to bf16 in registers; k_scale folds into the score
//    scale and v_scale into the final state.  Probabilities are rounded to bf16 for P.V.
// The fp32-cache kernel is plain vector code (fp32 throughout) with the same outputs.
#include <climits>

#include "pa_device.h"

namespace pa {


namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Word 3 of a raw buffer resource on gfx9 parts (32-bit data format, no swizzle): loads past the
// resource's byte count return zero without touching memory.
constexpr int kRawBufferWord3 = 0x00020000;
// Cache-policy operand of a buffer load that marks it non-temporal (the nt bit on gfx950).
constexpr int kLoadNonTemporal = 2;

// Request geometry of slot work item: first row, query length (clamped), KV length.
struct SlotInfo {
    int b, row0, L, S;
    int k_lo, k_hi;   // key range of the slot
};

// From work entry w = (b, tile_begin, tile_end, .); `live` says the entry is among the used ones.
__device__ __forceinline__ bool entry_info(const DecodeArgs& a, int4 w, bool live, SlotInfo& si) {
    const int b = w.x;
    if (!live || b < 0 || b >= a.num_seqs) return false;
    const int S = max(a.context_lens[b], 0);
    int row0 = b, L = 1;
    if (a.cu) {
        row0 = a.cu[b];
        L = a.cu[b + 1] - row0;
    }
    L = min(max(L, 0), a.max_q_len);
    if (row0 < 0 || row0 >= a.num_rows) L = 0;
    else L = min(L, a.num_rows - row0);
    // keys covered by this slot, clipped to the context and to the block table's reach
    const long long lo = static_cast<long long>(max(w.y, 0)) * a.tile_tokens;
    long long hi = static_cast<long long>(max(w.z, 0)) * a.tile_tokens;
    hi = min(hi, static_cast<long long>(S));
    hi = min(hi, static_cast<long long>(a.max_blocks) * a.block_size);
    si.b = b;
    si.row0 = row0;
    si.L = L;
    si.S = S;
    si.k_lo = static_cast<int>(min(lo, static_cast<long long>(S)));
    si.k_hi = static_cast<int>(max(hi, static_cast<long long>(si.k_lo)));
    return true;
}

__device__ __forceinline__ bool slot_info(const DecodeArgs& a, int slot, SlotInfo& si) {
    // the slot's work entry and the used-slot count are independent loads
    const int4 w = a.work_info[slot];
    const int used = *a.num_work;
    return entry_info(a, w, slot < used, si);
}

// ---------------------------------------------------------------------------------------------
// planning in place: the plan of a batch of at most kInlinePlanSeqs requests, evaluated by every
// workgroup with one request per thread, so the decode needs no separate planning launch.  The
// workgroup keeps its own slot's entry; kv head 0's workgroups store the entries, workgroup 0 the
// per-request ranges and the slot counts, so the buffers end up as the plan kernel writes them.
// ---------------------------------------------------------------------------------------------
// Shared slots.  When the capacity leaves every request one slot, slot sizes follow the request
// lengths and one workgroup per slot leaves the longest request to a single workgroup.  Then every
// slot of n tiles is cut into X = max(1, ceil(n / per)) pieces, per = ceil((sum of the slots' tiles +
// slots) / (factor x slots)), so a plan of `used` slots makes at most factor x used + used pieces;
// piece k covers the slot's tiles [floor(k n / X), floor((k + 1) n / X)), the plan's own split rule
// one level down.  Pieces are numbered slot by slot, in slot order, so a request's pieces are
// consecutive; the in-place plan and a plan read from work_info give the same pieces.
__device__ __forceinline__ long long piece_size(long long tiles_total, int used, int factor) {
    const long long den = static_cast<long long>(factor) * max(used, 1);
    return max(1LL, (tiles_total + used + den - 1) / den);
}

__device__ __forceinline__ int pieces_of(int n, long long per) {
    return max(1, static_cast<int>((n + per - 1) / per));
}

// A request's slots hold q = floor(tiles / parts) or q + 1 tiles; pieces of all its slots.
__device__ __forceinline__ int request_pieces(int tiles, int parts, long long per) {
    if (parts <= 0) return 0;
    const int q = tiles / parts;
    const int big = tiles - q * parts;             // slots of q + 1 tiles
    return (parts - big) * pieces_of(q, per) + big * pieces_of(q + 1, per);
}

// Tiles, relative to the request's first tile, of the request's piece `off`: its slot j is the last
// one whose earlier slots hold at most `off` pieces (slots before j: j of q tiles at least, and
// floor(j tiles / parts) - j q of them with q + 1), found by bisection.
__device__ __forceinline__ int2 request_piece_tiles(int off, int tiles, int parts, long long per) {
    const int q = tiles / parts;
    const int xq = pieces_of(q, per);
    const int xb = pieces_of(q + 1, per);
    auto before = [&](int j) -> int {              // pieces of slots 0 .. j-1
        const int nb = plan_tile_range(j, tiles, parts).x - j * q;
        return j * xq + nb * (xb - xq);
    };
    int lo = 0, hi = parts - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (before(mid) <= off) lo = mid;
        else hi = mid - 1;
    }
    const int2 t = plan_tile_range(lo, tiles, parts);
    const int n = t.y - t.x;
    const int2 u = plan_tile_range(off - before(lo), n, pieces_of(n, per));
    return make_int2(t.x + u.x, t.x + u.y);
}

// Shared slots over a plan read from work_info (at most kInlinePlanSeqs slots, one per thread):
// workgroup p's piece, the piece count and bound, and (workgroup 0) the requests' piece ranges.
template <int NW>
__device__ void pieces_from_plan(const DecodeArgs& a, int p, int4& wk, int2& nwk) {
    static_assert(NW * 64 >= kInlinePlanSeqs, "one slot per thread");
    __shared__ long long s_tiles[NW];
    __shared__ int s_count[NW], s_below[NW];
    __shared__ int s_pfirst[kInlinePlanSeqs + 1];
    __shared__ int s_req[kInlinePlanSeqs];
    __shared__ int2 s_range[kInlinePlanSeqs];
    __shared__ int4 s_pentry;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool lead = blockIdx.x == 0;             // writes the requests' piece ranges
    const int used = min(max(__builtin_amdgcn_readfirstlane(a.num_work[0]), 0), a.plan_slots);
    const int4 e = tid < used ? a.work_info[tid] : make_int4(-1, 0, 0, 0);
    const int n = tid < used ? max(e.z - e.y, 0) : 0;
    const long long wt = wave_sum_nonneg(n);
    if (lane == 0) s_tiles[wave] = wt;
    if (lead && tid < kInlinePlanSeqs) {
        s_req[tid] = e.x;
        s_range[tid] = make_int2(0, 0);            // requests without slots: no pieces
    }
    __syncthreads();
    long long total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) total += s_tiles[w];
    const long long per = piece_size(total, used, a.pieces);
    const int X = tid < used ? pieces_of(n, per) : 0;
    const int incl = wave_incl_scan(X, lane);
    if (lane == 63) s_count[wave] = incl;
    __syncthreads();
    int before = 0, pused = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        before += w < wave ? s_count[w] : 0;
        pused += s_count[w];
    }
    const int pfirst = before + incl - X;          // = pused past the last slot
    if (tid < kInlinePlanSeqs) s_pfirst[tid] = pfirst;
    if (tid == 0) s_pfirst[kInlinePlanSeqs] = pused;
    const int below = __popcll(__builtin_amdgcn_ballot_w64(tid < used && pfirst <= p));
    if (lane == 0) s_below[wave] = below;
    __syncthreads();
    int owner = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w) owner += s_below[w];
    if (p < pused && tid == owner) {
        const int2 u = plan_tile_range(p - pfirst, n, X);
        s_pentry = make_int4(e.x, e.y + u.x, e.y + u.y, e.w);
    }
    if (lead && tid < used) {
        // a request's slots are consecutive: the first of them records the request's pieces,
        // [its first piece, the first piece past the request's last slot)
        const int b = e.x;
        if (b >= 0 && b < a.num_seqs && (tid == 0 || s_req[tid - 1] != b)) {
            int k = tid + 1;
            while (k < used && s_req[k] == b) ++k;
            s_range[b] = make_int2(pfirst, s_pfirst[k] - pfirst);
        }
    }
    __syncthreads();
    if (lead && tid < a.num_seqs) a.piece_reduce_out[tid] = s_range[tid];
    wk = p < pused ? s_pentry : make_int4(-1, 0, 0, 0);
    nwk = make_int2(pused, static_cast<int>(min(per, static_cast<long long>(INT_MAX))));   // pieces <= per tiles
}

// Up to 64 requests: every wave evaluates the whole plan on its own, with no barrier.
__device__ __forceinline__ void plan_in_wave(const DecodeArgs& a, int slot, int g, int4& wk, int2& nwk) {
    const int lane = threadIdx.x & 63;
    const bool real = lane < a.num_seqs;
    const int S = real ? max(a.context_lens[lane], 0) : 0;
    const PlanRange pr = plan_range(S, real && a.window > 0 ? plan_q_len(a.cu, lane) : 1, a.window, a.tile_tokens);
    const int len = pr.len;
    const int tiles = pr.tiles;
    const long long total = wave_sum_nonneg(len);
    const int nonempty = __popcll(__builtin_amdgcn_ballot_w64(len > 0));
    const int parts = plan_parts(len, tiles, static_cast<long long>(a.plan_cap) - nonempty, total,
                                 a.max_partitions);
    const int incl = wave_incl_scan(parts, lane);
    const int first = incl - parts;
    const int used = __builtin_amdgcn_readlane(incl, 63);
    const int big = wave_max_nonneg(parts > 0 ? (tiles + parts - 1) / parts : 0);   // largest part
    // the requests whose first slot is <= slot are a prefix; its last one owns the slot
    const int owner = __popcll(__builtin_amdgcn_ballot_w64(real && first <= slot)) - 1;
    wk = make_int4(-1, 0, 0, 0);
    if (slot < used) {
        const int o = max(owner, 0);
        const int2 t = plan_tile_range(slot - __builtin_amdgcn_readlane(first, o),
                                       __builtin_amdgcn_readlane(tiles, o), __builtin_amdgcn_readlane(parts, o));
        const int t0 = __builtin_amdgcn_readlane(pr.t0, o);
        wk = make_int4(o, t0 + t.x, t0 + t.y, __builtin_amdgcn_readlane(S, o));
    }
    nwk = make_int2(used, big);
    if (threadIdx.x < 64) {
        if (blockIdx.x == 0 && real) a.plan_reduce_out[lane] = make_int2(first, parts);
        if (lane == 0) {
            if (g == 0 && slot < a.plan_slots) a.plan_work_out[slot] = wk;
            if (blockIdx.x == 0) *reinterpret_cast<int2*>(a.plan_num_work_out) = nwk;
        }
    }
    if (!a.pieces) return;
    // shared slots: this workgroup streams piece `slot` instead (see piece_size)
    const long long per = piece_size(wave_sum_nonneg(tiles), used, a.pieces);
    const int np = request_pieces(tiles, parts, per);
    const int pincl = wave_incl_scan(np, lane);
    const int pfirst = pincl - np;
    const int pused = __builtin_amdgcn_readlane(pincl, 63);
    if (threadIdx.x < 64 && blockIdx.x == 0 && real) a.piece_reduce_out[lane] = make_int2(pfirst, np);
    const int po = __popcll(__builtin_amdgcn_ballot_w64(real && pfirst <= slot)) - 1;
    wk = make_int4(-1, 0, 0, 0);
    if (slot < pused) {
        const int o = max(po, 0);
        const int2 t = request_piece_tiles(slot - __builtin_amdgcn_readlane(pfirst, o),
                                           __builtin_amdgcn_readlane(tiles, o), __builtin_amdgcn_readlane(parts, o), per);
        const int t0 = __builtin_amdgcn_readlane(pr.t0, o);
        wk = make_int4(o, t0 + t.x, t0 + t.y, __builtin_amdgcn_readlane(S, o));
    }
    nwk = make_int2(pused, static_cast<int>(min(per, static_cast<long long>(INT_MAX))));   // pieces <= per tiles
}

template <int NW>
__device__ void plan_in_place(const DecodeArgs& a, int slot, int g, int4& wk, int2& nwk) {
    static_assert(NW * 64 >= kInlinePlanSeqs, "one request per thread");
    if (a.num_seqs <= 64) {
        plan_in_wave(a, slot, g, wk, nwk);
        return;
    }
    __shared__ long long s_total[NW], s_tiles[NW];
    __shared__ int s_nonempty[NW], s_slots[NW], s_below[NW], s_largest[NW], s_pieces[NW], s_pbelow[NW];
    __shared__ int4 s_entry, s_pentry;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = tid;
    const bool real = r < a.num_seqs;
    const int S = real ? max(a.context_lens[r], 0) : 0;
    const PlanRange pr = plan_range(S, real && a.window > 0 ? plan_q_len(a.cu, r) : 1, a.window, a.tile_tokens);
    const int len = pr.len;
    const int tiles = pr.tiles;

    // W = sum of the lengths read and B' = #{requests reading any key}
    const long long wsum = wave_sum_nonneg(len);
    const int wne = __popcll(__builtin_amdgcn_ballot_w64(len > 0));
    const long long wtiles = a.pieces ? wave_sum_nonneg(tiles) : 0;
    if (lane == 0) {
        s_total[wave] = wsum;
        s_nonempty[wave] = wne;
        s_tiles[wave] = wtiles;
    }
    __syncthreads();
    long long total = 0, tiles_total = 0;
    int nonempty = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        total += s_total[w];
        nonempty += s_nonempty[w];
        tiles_total += s_tiles[w];
    }

    // this request's partitions, their exclusive scan, and the largest partition in tiles
    const int parts = plan_parts(len, tiles, static_cast<long long>(a.plan_cap) - nonempty, total,
                                 a.max_partitions);
    const int incl = wave_incl_scan(parts, lane);
    const int big = wave_max_nonneg(parts > 0 ? (tiles + parts - 1) / parts : 0);   // largest part
    if (lane == 63) s_slots[wave] = incl;
    if (lane == 0) s_largest[wave] = big;
    __syncthreads();
    int before = 0, used = 0, largest = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        before += w < wave ? s_slots[w] : 0;
        used += s_slots[w];
        largest = max(largest, s_largest[w]);
    }
    const int first = before + incl - parts;

    // shared slots: this request's pieces and their scan within the wave
    int np = 0, pincl = 0;
    const long long per = a.pieces ? piece_size(tiles_total, used, a.pieces) : 1;
    if (a.pieces) {
        np = request_pieces(tiles, parts, per);
        pincl = wave_incl_scan(np, lane);
    }

    // the requests whose first slot is <= slot are a prefix; its last one owns the slot
    const int below = __popcll(__builtin_amdgcn_ballot_w64(real && first <= slot));
    if (lane == 0) s_below[wave] = below;
    if (lane == 63) s_pieces[wave] = pincl;
    if (blockIdx.x == 0 && real) a.plan_reduce_out[r] = make_int2(first, parts);
    __syncthreads();
    int owner = -1, pbefore = 0, pused = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        owner += s_below[w];
        pbefore += w < wave ? s_pieces[w] : 0;
        pused += s_pieces[w];
    }
    if (slot < used && r == owner) {
        const int2 t = plan_tile_range(slot - first, tiles, parts);
        s_entry = make_int4(r, pr.t0 + t.x, pr.t0 + t.y, S);
    }
    const int pfirst = pbefore + pincl - np;
    if (a.pieces) {
        const int pbelow = __popcll(__builtin_amdgcn_ballot_w64(real && pfirst <= slot));
        if (lane == 0) s_pbelow[wave] = pbelow;
        if (blockIdx.x == 0 && real) a.piece_reduce_out[r] = make_int2(pfirst, np);
    }
    __syncthreads();
    wk = slot < used ? s_entry : make_int4(-1, 0, 0, 0);
    nwk = make_int2(used, largest);
    if (tid == 0) {
        if (g == 0 && slot < a.plan_slots) a.plan_work_out[slot] = wk;
        if (blockIdx.x == 0) *reinterpret_cast<int2*>(a.plan_num_work_out) = nwk;
    }
    if (!a.pieces) return;
    // shared slots: this workgroup streams piece `slot` of the last request whose first piece is
    // <= slot
    int powner = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w) powner += s_pbelow[w];
    if (slot < pused && r == powner) {
        const int2 t = request_piece_tiles(slot - pfirst, tiles, parts, per);
        s_pentry = make_int4(r, pr.t0 + t.x, pr.t0 + t.y, S);
    }
    __syncthreads();
    wk = slot < pused ? s_pentry : make_int4(-1, 0, 0, 0);
    nwk = make_int2(pused, static_cast<int>(min(per, static_cast<long long>(INT_MAX))));   // pieces <= per tiles
}

// ---------------------------------------------------------------------------------------------
// prefill blocks: request b's query tokens [i0, i1), block_tokens at a time.  Every wave scans the
// cumulative query lengths 64 requests at a time and finds the request holding block qb; no barrier.
// ---------------------------------------------------------------------------------------------
struct PrefillBlock {
    int b, i0, i1;
};

__device__ __forceinline__ bool find_prefill_block(const DecodeArgs& a, int qb, PrefillBlock& out) {
    const int lane = threadIdx.x & 63;
    const int Lb = a.block_tokens;
    int before = 0;                                  // blocks of the requests already scanned
    for (int c0 = 0; c0 < a.num_seqs; c0 += 64) {
        const int r = c0 + lane;
        int L = 0;
        if (r < a.num_seqs) L = max(a.cu[r + 1] - a.cu[r], 0);
        const int n = (L + Lb - 1) / Lb;
        const int incl = wave_incl_scan(n, lane);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (qb < before + total) {
            // the owner is the first request whose blocks end past qb
            const unsigned long long m = __builtin_amdgcn_ballot_w64(r < a.num_seqs && before + incl > qb);
            const int o = __builtin_ctzll(m);
            const int first = before + __builtin_amdgcn_readlane(incl, o) - __builtin_amdgcn_readlane(n, o);
            const int j = qb - first;
            out.b = c0 + o;
            out.i0 = j * Lb;
            out.i1 = min(__builtin_amdgcn_readlane(L, o), out.i0 + Lb);
            return true;
        }
        before += total;
    }
    return false;
}

// Zero a row past the last prefill request's rows (rows before cu[0] belong to other calls).
template <int D>
__device__ __forceinline__ void zero_prefill_tail_row(const DecodeArgs& a, int r, int lane) {
    if (r >= a.num_rows || r < a.cu[a.num_seqs]) return;
    const size_t base = static_cast<size_t>(r) * a.num_q_heads * D;
    const int n4 = a.num_q_heads * D / 4;
    for (int e = lane; e < n4; e += 64) {
        if (a.out_bf16) *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + base + 4 * e) = make_uint2(0u, 0u);
        else *reinterpret_cast<float4*>(static_cast<float*>(a.out) + base + 4 * e) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// ---------------------------------------------------------------------------------------------
// matrix-core kernel (bf16 or fp8 caches)
// ---------------------------------------------------------------------------------------------
template <int D, int NCB, bool KV8, int NWAVES = 4>
struct Mfma {
    static constexpr int ESZ = KV8 ? 1 : 2;            // bytes per cache element in HBM
    static constexpr int GRB = D * ESZ;                // HBM bytes per cache row (one token, one kv head)
    static constexpr int GCPR = GRB / 16;              // 16-byte HBM columns per row
    static constexpr int NLD = 16 * GRB / 1024;        // 16-byte loads per lane per 16-row chunk
    static constexpr int LRB = D * 2;                  // LDS bytes per row (always bf16)
    static constexpr int LCPR = LRB / 16;              // 16-byte LDS columns per row
    static constexpr int SWM = (LCPR < 16 ? LCPR : 16) - 1;  // XOR swizzle mask on the column
    static constexpr int KSTEPS = D / 32;              // k-steps of the S^T product
    static constexpr int DT = D / 16;                  // 16-wide d tiles of the P.V product
    static constexpr int NW = NWAVES;                  // waves per workgroup
    // Chunk dealing (see the streaming loop): the 4-wave form splits each slot evenly over its waves
    // when the plan's largest slot is long enough, and deals units of the largest slot otherwise.
    // The 8-wave form, used when every request is one slot (slot sizes then follow the request
    // lengths), always splits each slot evenly, so short slots still run every wave and the longest
    // gets twice the waves of a 4-wave group.
    static constexpr bool EVEN = NW > 4;
    // head_dim 256 (DS): the waves work in groups of SPLIT that split the head dimension, each group
    // walking its own stream of the slot's chunks (chunks s, s + NS, ...).  A wave loads its SL
    // columns of K and V row-major (coalesced 16-byte pieces), stages them in LDS (K in a tile it
    // reads back at once in operand order, V in tiles of two parities for the transposed reads), and
    // the group's partial scores are summed through LDS.  The per-wave state is 1/SPLIT of the
    // full one, so operands, accumulators and a deep prefetch fit the registers of two workgroups
    // per CU, while only SPLIT waves repeat each chunk's softmax.
    static constexpr bool DS = D == 256;
    static constexpr int SPLIT = NCB >= 4 ? 4 : 2;     // waves sharing a chunk (DS)
    static constexpr int NS = NW / SPLIT;              // chunk streams per workgroup (DS)
    static constexpr int SL = D / SPLIT;               // head-dimension columns per wave (DS)
    static constexpr int KSW = SL / 32;                // k-steps of the partial S^T product (DS)
    static constexpr int DTW = SL / 16;                // d tiles of the P.V product per wave (DS)
    static constexpr int VGC = SL * ESZ / 16;          // 16-byte HBM columns of a wave's K or V row slice
    static constexpr int VLD = 16 * VGC / 64;          // 16-byte K (and V) loads per lane per chunk (DS)
    static constexpr int VLRB = SL * 2;                // LDS bytes per K or V row slice (bf16)
    static constexpr int VSWM = (VLRB / 16 < 16 ? VLRB / 16 : 16) - 1;
    static constexpr int PFD = KV8 ? (NCB == 1 ? 6 : (NCB == 2 ? 4 : 2)) : (NCB == 1 ? 3 : (NCB == 2 ? 2 : 3));   // chunks in flight per wave (DS)
    static constexpr int XBUF = 2 * NCB * NW * 64 * 16;  // partial-score exchange, two parities (DS)
    // chunks in flight per wave: as many as the registers hold without spilling (scratch traffic would
    // itself be waited for in order and stall the pipeline); an fp8 chunk takes half the registers
    // (head_dim 64 and 128; head_dim 256 uses PFD)
    static constexpr int PF_BF16 = D == 64 ? (NCB <= 2 ? 4 : 3) : (NCB == 1 ? 2 : (NCB == 2 ? 3 : 2));
    static constexpr int PF_FP8 = D == 64 ? (NCB <= 2 ? 8 : 6) : (NCB <= 2 ? 4 : 2);
    static constexpr int PF = DS ? PFD : (KV8 ? PF_FP8 : PF_BF16);
    // chunks per compute step: two where the registers allow, so each step runs two independent
    // score chains and one softmax pass over 32 keys (the per-chunk latency of a lone wave drops)
    static constexpr int CG = (D <= 128 && NCB == 1 && PF % 2 == 0) ? 2 : 1;
    static constexpr int WAVE_LDS = CG * 2 * 16 * LRB; // K then V of each chunk of a step, per wave
    // DS: per wave two V tiles (chunk parity) and one K tile, then the exchange
    static constexpr int STAGE_LDS = DS ? NW * 3 * 16 * VLRB + XBUF : NW * WAVE_LDS;
    static constexpr int ROWS = 16 * NCB;              // query rows per workgroup (padded)
    static constexpr int APITCH = D + 4;               // fp32 pitch of the LDS merge buffer
    static constexpr int MERGE_LDS = (NW * ROWS + 2 * ROWS + ROWS * APITCH) * 4;
    static constexpr int LDS = STAGE_LDS > MERGE_LDS ? STAGE_LDS : MERGE_LDS;
    // Per-wave designs whose state (ROWS x D accumulators, then m and l per row) fits the wave's
    // own staging tile park it there and merge the NW states per element while storing: one
    // barrier instead of a barrier per wave.
    static constexpr bool PARK = !DS && (ROWS * APITCH + 2 * ROWS) * 4 <= WAVE_LDS;
    // Waves per SIMD the register budget is cut for: 2 (two workgroups per CU, 256 registers per lane)
    // where operands and accumulators fit, else 1 (512 registers) rather than spilling.
    static constexpr int WAVES = (D == 64 || (D == 128 && NCB == 1) || DS) ? 2 : 1;

};

// Byte offset of 16-byte column c of row r in a per-wave bf16 LDS tile (XOR swizzle on the column).
template <int LRB, int SWM>
__device__ __forceinline__ int lds_col(int r, int c) {
    return r * LRB + ((c ^ (r & SWM)) << 4);
}

// The same for the head-split path's bf16 V tiles, whose reads are the transposed 8-byte ones: with 16
// columns a row the XOR is ((r & 7) << 1) | ((r >> 3) & 1), so rows r and r ^ 1, which a read cycle
// takes together, land on different bank groups (verify decode 45.4 -> 45.3 us).
template <int LRB, int SWM>
__device__ __forceinline__ int lds_vcol(int r, int c) {
    const int x = SWM == 15 ? (((r & 7) << 1) | ((r >> 3) & 1)) : (r & SWM);
    return r * LRB + ((c ^ x) << 4);
}

// Rescale threshold of the running maximum, in base-2 units: probabilities stay below 2^8.
constexpr float kRescaleSlack = 8.0f;

// Max and sum over the lanes l, l ^ 16, l ^ 32 and l ^ 48 (one query row's four lane groups) with
// gfx950's row swaps: permlane16_swap exchanges the odd 16-lane rows of its first operand with the
// even rows of its second, permlane32_swap the upper half of the first with the lower half of the
// second, so with both operands x each lane ends up holding x of itself and of its partner, one in
// each result.  Vector ALU only, no LDS round trip; every lane of the four gets the same value.
__device__ __forceinline__ float max_over_row_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_over_row_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// MIXED: the launch holds two parts (see LaunchArgs); otherwise every workgroup runs part[0].
template <int D, int NCB, bool KV8, bool QF32, int NWAVES, bool MIXED>
__global__ __launch_bounds__((64 * NWAVES), (Mfma<D, NCB, KV8, NWAVES>::WAVES)) void decode_mfma_kernel(const LaunchArgs L) {
    using C = Mfma<D, NCB, KV8, NWAVES>;
    const bool second = MIXED && static_cast<int>(blockIdx.x) >= L.split;
    // a copy (the fields become scalar selects): through a pointer chosen at run time the compiler
    // could no longer treat the arguments as invariant and reloaded them in the loop
    const DecodeArgs a = second ? L.part[1] : L.part[0];
    const int bid = static_cast<int>(blockIdx.x) - (second ? L.split : 0);
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform by construction; said so, so that everything derived from it (chunk indices,
    // page ids, buffer resources) stays in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int work_groups = a.capacity * a.num_kv_heads;
    if (bid >= work_groups) {
        // prefill: trailing workgroups write the rows past the last request as zeros
        if (a.prefill) zero_prefill_tail_row<D>(a, (bid - work_groups) * C::NW + wave, lane);
        return;
    }
    // the workgroup's position among the plan's slots; its slot is the position itself, or with a
    // dispatch order the slot that order puts there
    int slot = bid / a.num_kv_heads;
    const int g = bid - slot * a.num_kv_heads;

    // ---- slot geometry.  Dependent loads are kept to three levels: the work entry; then the
    // request's length, cumulative query lengths and (speculatively, over the plan's tile range)
    // this wave's page ids; then queries and K/V. ----
    int4 wk;
    int2 nwk;                                      // (used slots, largest slot in tiles)
    SlotInfo si;                                   // filled here in prefill mode, after the pages otherwise
    long long key_lo, key_hi;                      // the keys this workgroup covers, before clipping
    if (a.prefill) {
        // one block of query tokens: all keys its tokens see, from the first token's window start
        PrefillBlock pb;
        if (!find_prefill_block(a, slot, pb)) return;
        const int b0 = __builtin_amdgcn_readfirstlane(pb.b);
        const int i0 = __builtin_amdgcn_readfirstlane(pb.i0);
        const int i1 = __builtin_amdgcn_readfirstlane(pb.i1);
        const int Sb = __builtin_amdgcn_readfirstlane(max(a.context_lens[b0], 0));
        const int c0 = __builtin_amdgcn_readfirstlane(a.cu[b0]);
        const int Lr = __builtin_amdgcn_readfirstlane(a.cu[b0 + 1]) - c0;
        si.b = b0;
        si.row0 = c0 + i0;
        si.L = i1 - i0;
        si.S = Sb - (Lr - i1);                     // keys visible to the block's last token
        if (si.row0 < 0 || si.row0 >= a.num_rows) si.L = 0;
        else si.L = min(si.L, a.num_rows - si.row0);
        key_hi = max(si.S, 0);
        key_lo = a.window > 0 ? max(0LL, (key_hi - (si.L - 1) - a.window)) & ~15LL : 0;
        wk = make_int4(b0, 0, 0, Sb);
        nwk = make_int2(0, 0);
    } else {
        if (a.plan_inline) {
            plan_in_place<C::NW>(a, slot, g, wk, nwk);
        } else if (a.pieces) {
            pieces_from_plan<C::NW>(a, slot, wk, nwk);
        } else {
            wk = a.dispatch_info ? a.dispatch_info[slot] : a.work_info[slot];
            nwk = *reinterpret_cast<const int2*>(a.num_work);
        }
        wk = make_int4(__builtin_amdgcn_readfirstlane(wk.x), __builtin_amdgcn_readfirstlane(wk.y),
                       __builtin_amdgcn_readfirstlane(wk.z), __builtin_amdgcn_readfirstlane(wk.w));
        if (a.dispatch_info && !a.plan_inline && !a.pieces) slot = wk.w;   // word 3: the slot index
        nwk = make_int2(__builtin_amdgcn_readfirstlane(nwk.x), __builtin_amdgcn_readfirstlane(nwk.y));
        if (slot >= nwk.x) return;
        key_lo = static_cast<long long>(max(wk.y, 0)) * a.tile_tokens;
        key_hi = static_cast<long long>(max(wk.z, 0)) * a.tile_tokens;
    }
    const int b = wk.x;
    if (b < 0 || b >= a.num_seqs) return;
    // query blocks of a prefill read their request's block-table row
    const int bt_b = a.bt_index ? __builtin_amdgcn_readfirstlane(a.bt_index[b]) : b;
    const int* bt_row = a.block_tables + static_cast<size_t>(bt_b) * a.max_blocks;
    const long long reach = static_cast<long long>(a.max_blocks) * a.block_size;
    const int plan_lo = static_cast<int>(min(key_lo, reach));
    const int plan_hi = static_cast<int>(max(min(key_hi, reach), static_cast<long long>(plan_lo)));
    const int plan_chunks = (plan_hi - plan_lo + 15) >> 4;

    // Chunks are dealt to waves in units of `unit` consecutive chunks: wave w owns units w, w + NW, ...
    // of the slot and its k-th chunk is chunk_of(k).  Even dealing: the unit is this slot split over
    // the NW waves, so every slot streams on all its waves from the start, which keeps the most loads
    // in flight while the launch is bound by bandwidth.  Unit dealing: the unit is the plan's largest
    // slot split over the NW waves, so that slot's waves and every other wave with a full unit carry
    // the same load and finish together, while a smaller slot runs fewer streaming waves; in a short,
    // latency-bound launch this keeps the small slots' loads from delaying the largest slot's.  The
    // choice is uniform over the launch (from the plan's largest slot).  Any unit >= 1 covers every
    // chunk of every slot exactly once.  (A prefill block is its own slot: its chunks are split
    // evenly over the waves.)
    const int cpt = a.tile_tokens >> 4;          // 16-key chunks per tile
    const long long largest_chunks = static_cast<long long>(max(nwk.y, 1)) * cpt;
    const bool even = a.prefill || C::EVEN || largest_chunks >= static_cast<long long>(C::NW) * kEvenDealChunks;
    const long long unit_chunks = even ? plan_chunks : largest_chunks;
    const int unit = static_cast<int>(min(max(1LL, (unit_chunks + C::NW - 1) / C::NW), 1LL << 30));
    // Every slot of the plan (and every prefill block) spans at most NW units, so a wave's live
    // chunks are all in its first unit: k < unit takes no division.  Past that (only the empty
    // padding chunks, or a plan whose largest-slot word understates a slot) the general form applies.
    auto chunk_of = [&](int k) -> int {
        if constexpr (C::DS) return k * C::NS + wave / C::SPLIT;   // the wave group's stream
        if (k < unit) return wave * unit + k;
        const int j = k / unit;
        return (wave + C::NW * j) * unit + (k - j * unit);
    };
    // pages hold 16, 64 or 128 tokens: key -> (page ordinal, row) by shift and mask
    const int page_shift = __builtin_ctz(a.block_size);

    // Every memory instruction of the streaming loop is issued unconditionally, so each iteration
    // issues the same number of vector loads and the compiler can wait for exactly the chunk it
    // stages (vmcnt counts in order) rather than for every load in flight.  Loads that have nothing
    // to fetch go through buffer resources with no records: they return zeros and touch no memory.
    // Page ids are fetched 2 x PF chunks ahead, each just before the K/V loads PF chunks ahead, so
    // waiting for chunk k's K/V also covers the page id needed to issue chunk k + PF.
    const __amdgpu_buffer_rsrc_t bt_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int*>(bt_row), 0, a.max_blocks * 4, kRawBufferWord3);
    auto page_load = [&](int k) -> int {       // page id of the wave's k-th chunk; 0 past the plan
        const int c = chunk_of(k);
        const unsigned off = c < plan_chunks ? static_cast<unsigned>((plan_lo + 16 * c) >> page_shift) * 4u
                                             : 0xfffffff0u;
        return __builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, off, 0, 0);
    };
    int pfirst[C::PF], pnext[C::PF];
#pragma unroll
    for (int st = 0; st < C::PF; ++st) pfirst[st] = page_load(st);
#pragma unroll
    for (int st = 0; st < C::PF; ++st) pnext[st] = page_load(st + C::PF);

    if (!a.prefill) {
        const int S = __builtin_amdgcn_readfirstlane(max(a.context_lens[b], 0));
        int row0 = b, L = 1;
        if (a.cu) {
            row0 = __builtin_amdgcn_readfirstlane(a.cu[b]);
            L = __builtin_amdgcn_readfirstlane(a.cu[b + 1]) - row0;
        }
        L = min(max(L, 0), a.max_q_len);
        if (row0 < 0 || row0 >= a.num_rows) L = 0;
        else L = min(L, a.num_rows - row0);
        si.b = b;
        si.row0 = row0;
        si.L = L;
        si.S = S;
    }
    si.k_hi = min(plan_hi, max(si.S, 0));
    si.k_lo = min(plan_lo, si.k_hi);
    const int G = a.group;
    const int M = G * si.L;                       // valid query rows (<= ROWS)
    const int col = lane & 15;                    // MFMA column = query row within a block
    const int grp = lane >> 4;                    // 4 lane groups

    // ---- query operands (B of S^T = K.Q^T): qop[cb][s] = q[row][32s + 8*grp .. +8] as bf16 ----
    constexpr int NKS = C::DS ? C::KSW : C::KSTEPS;   // k-steps of this wave's S^T product
    constexpr int NDT = C::DS ? C::DTW : C::DT;       // d tiles of this wave's O^T
    const int dcol0 = C::DS ? (wave % C::SPLIT) * C::SL : 0;   // this wave's first head-dimension column
    bf16x8_t qop[NCB][NKS];
    int nvis[NCB];                                // keys visible to this lane's query row: [nlo, nvis)
    int nlo[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int n = 16 * cb + col;
        const bool valid = n < M;
        const int i = valid ? n / G : 0;
        const int h = g * G + (valid ? n - i * G : 0);
        nvis[cb] = valid ? si.S - (si.L - 1 - i) : 0;
        nlo[cb] = a.window > 0 ? max(nvis[cb] - a.window, 0) : 0;
        const size_t qoff = (static_cast<size_t>(si.row0 + i) * a.num_q_heads + h) * D;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const int d0 = dcol0 + 32 * s + 8 * grp;
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (valid) {
                if constexpr (QF32) {
                    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + qoff + d0);
                    const float4 x = p[0], y = p[1];
                    v[0] = pack_bf16x2(x.x, x.y);
                    v[1] = pack_bf16x2(x.z, x.w);
                    v[2] = pack_bf16x2(y.x, y.y);
                    v[3] = pack_bf16x2(y.z, y.w);
                } else {
                    v = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.q) + qoff + d0);
                }
            }
            qop[cb][s] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    // bounds over the workgroup's rows: the first token sees the fewest keys, the last token's window
    // starts latest; a step whose keys all lie in [nlo_hi, nvis_lo) needs no mask (rows past the
    // request's own rows take unmasked scores then, but they are never written)
    const int nvis_lo = si.S - (si.L - 1);
    const int nlo_hi = a.window > 0 ? max(si.S - a.window, 0) : 0;
    float m_run[NCB], l_run[NCB];                 // running reference max (base 2) and lane-partial sum
    float4_t acc[NCB][NDT];                       // O^T tile: lane holds d = dcol0 + 16t + 4*grp + j, row = col
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        m_run[cb] = -INFINITY;
        l_run[cb] = 0.f;
#pragma unroll
        for (int t = 0; t < NDT; ++t) acc[cb][t] = float4_t{0.f, 0.f, 0.f, 0.f};
    }

    const int nkeys = si.k_hi - si.k_lo;
    const int nchunks = nkeys > 0 ? (nkeys + 15) >> 4 : 0;
    const size_t head_stride = static_cast<size_t>(a.block_size) * C::GRB;   // HBM bytes per (block, kv head)
    uint8_t* const wlds = lds + wave * C::WAVE_LDS;   // chunk c of a step: K at c * 32 rows, then V

    // this wave's number of chunks: its full units, plus the ragged last unit if it owns it
    const int full_units = nchunks / unit;
    const int rem = nchunks - full_units * unit;
    int my_chunks = (full_units > wave ? (full_units - wave + C::NW - 1) / C::NW : 0) * unit;
    if (rem > 0 && full_units % C::NW == wave) my_chunks += rem;
    if constexpr (C::DS) my_chunks = (nchunks - wave / C::SPLIT + C::NS - 1) / C::NS;   // its stream's

    float* const mbuf = reinterpret_cast<float*>(lds);     // [NW][ROWS]  (after the stream)
    float* const lbuf = mbuf + C::NW * C::ROWS;             // [ROWS]
    float* const Mbuf = lbuf + C::ROWS;                     // [ROWS]
    float* const abuf = Mbuf + C::ROWS;                     // [ROWS][APITCH]
    if constexpr (C::DS) {
        // ---- head-split stream: every wave takes every chunk, SL columns of it ----
        constexpr int PF = C::PF;
        u32x4_t kreg[PF][C::VLD], vreg[PF][C::VLD];
        int nvalid_st[PF];
        // The 16-byte piece of the wave's slice that lane `lane` holds in load step it: row r, column c
        // of the slice.  Row-major, except fp8 slices of 8 columns, which widen to 16 LDS columns a row:
        // there each group of eight lanes takes half of two adjacent rows, so that the eight lanes
        // storing in one cycle do not meet on the same banks (columns c and c + 4 of a row would).
        auto vpiece_row = [&](int it) -> int {
            if constexpr (KV8 && C::VGC == 8) return 8 * it + 2 * (lane >> 4) + ((lane >> 2) & 1);
            return (it * 64 + lane) / C::VGC;
        };
        auto vpiece_col = [&](int it) -> int {
            if constexpr (KV8 && C::VGC == 8) return 4 * ((lane >> 3) & 1) + (lane & 3);
            return (it * 64 + lane) % C::VGC;
        };
        // this wave's K and V columns, 16-byte pieces, row-major, non-temporal; a chunk past the
        // slot, the context or on an invalid page loads zeros (no records)
        auto issue = [&](int st, int k, int page) {
            const int key0 = si.k_lo + 16 * chunk_of(k);
            const int blk = __builtin_amdgcn_readfirstlane(page);
            const bool live = k < my_chunks && blk >= 0 && blk < a.num_blocks;
            const int nv = live ? max(min(16, si.k_hi - key0), 0) : 0;
            nvalid_st[st] = nv;
            const int off = key0 & (a.block_size - 1);
            const size_t base = nv > 0 ? (static_cast<size_t>(blk) * a.num_kv_heads + g) * head_stride +
                                             static_cast<size_t>(off) * C::GRB
                                       : 0;
            const int records = nv > 0 ? 16 * C::GRB : 0;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t*>(a.k_cache + base), 0, records, kRawBufferWord3);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t*>(a.v_cache + base), 0, records, kRawBufferWord3);
#pragma unroll
            for (int it = 0; it < C::VLD; ++it) {
                const int r = vpiece_row(it);
                const int c = vpiece_col(it);
                const int o = r * C::GRB + dcol0 * C::ESZ + 16 * c;
                kreg[st][it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, kLoadNonTemporal));
                vreg[st][it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, kLoadNonTemporal));
            }
        };
        // two V tiles per wave (chunk parity), then one K tile per wave, then the partial-score
        // exchange [2][NCB][NW][64]
        uint8_t* const vlds0 = lds + wave * 2 * 16 * C::VLRB;
        uint8_t* const klds = lds + C::NW * 2 * 16 * C::VLRB + wave * 16 * C::VLRB;
        float4_t* const xbuf = reinterpret_cast<float4_t*>(lds + C::NW * 3 * 16 * C::VLRB);
        const int tr_row = 4 * grp + ((lane >> 2) & 3);
        const int tr_d0 = 4 * (lane & 3);

        // Stage A of chunk k (slot st of the load ring): K columns to the wave's K tile and V columns to
        // V tile k & 1, as bf16 rows (rows >= nv zero); K read back in operand order (lane: key row
        // lane & 15, columns 32s + 8*(lane >> 4) .. + 8 of the wave's slice); the loads PF chunks
        // ahead; then the partial S^T over this wave's columns into exchange buffer k & 1.  The K tile
        // is written and read by this wave alone, and a wave's LDS operations complete in order, so
        // the next chunk's K may reuse it.
        auto stage_a = [&](int st, int k) {
            const int nv = nvalid_st[st];
            uint8_t* const vlds = vlds0 + (k & 1) * 16 * C::VLRB;
            compiler_fence();
#pragma unroll
            for (int it = 0; it < C::VLD; ++it) {
                const int r = vpiece_row(it);
                const int c = vpiece_col(it);
                u32x4_t kv = kreg[st][it];
                u32x4_t vv = vreg[st][it];
                if (nv < 16) {
                    const u32x4_t z = {0u, 0u, 0u, 0u};
                    kv = r < nv ? kv : z;
                    vv = r < nv ? vv : z;
                }
                if constexpr (!KV8) {
                    *reinterpret_cast<u32x4_t*>(klds + lds_col<C::VLRB, C::VSWM>(r, c)) = kv;
                    *reinterpret_cast<u32x4_t*>(vlds + lds_vcol<C::VLRB, C::VSWM>(r, c)) = vv;
                } else {
                    // 16 fp8 codes -> 16 bf16 values = two LDS columns (2c, 2c+1), widened exactly
                    u32x4_t klo, khi, vlo, vhi;
#pragma unroll
                    for (int w = 0; w < 2; ++w) {
                        klo[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kv[w], 1.0f, false));
                        klo[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kv[w], 1.0f, true));
                        khi[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kv[w + 2], 1.0f, false));
                        khi[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kv[w + 2], 1.0f, true));
                        vlo[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vv[w], 1.0f, false));
                        vlo[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vv[w], 1.0f, true));
                        vhi[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vv[w + 2], 1.0f, false));
                        vhi[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vv[w + 2], 1.0f, true));
                    }
                    const int o0 = lds_col<C::VLRB, C::VSWM>(r, 2 * c);
                    const int o1 = lds_col<C::VLRB, C::VSWM>(r, 2 * c + 1);
                    *reinterpret_cast<u32x4_t*>(klds + o0) = klo;
                    *reinterpret_cast<u32x4_t*>(klds + o1) = khi;
                    *reinterpret_cast<u32x4_t*>(vlds + o0) = vlo;
                    *reinterpret_cast<u32x4_t*>(vlds + o1) = vhi;
                }
            }
            bf16x8_t kop[C::KSW];
#pragma unroll
            for (int ks = 0; ks < C::KSW; ++ks)
                kop[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                           klds + lds_col<C::VLRB, C::VSWM>(col, 4 * ks + grp)));
            compiler_fence();
            const int page = pnext[st];
            pnext[st] = page_load(k + 2 * PF);
            issue(st, k + PF, page);
            float4_t* const xb = xbuf + (k & 1) * NCB * C::NW * 64;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if (cb > 0 && 16 * cb >= M) break;     // a block past the request's rows: nothing
                float4_t sp = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < C::KSW; ++ks)
                    sp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks], qop[cb][ks], sp, 0, 0, 0);
                xb[(cb * C::NW + wave) * 64 + lane] = sp;
            }
        };

        // Stage B of chunk k (its keys from key0, nv of them): the summed scores (fixed wave order,
        // so every wave sees the same values), the online softmax, and P.V over this wave's columns.
        auto stage_b = [&](int k, int key0, int nv) {
            const uint8_t* const vlds = vlds0 + (k & 1) * 16 * C::VLRB;
            short4_t vop[C::DTW];
#pragma unroll
            for (int t = 0; t < C::DTW; ++t) {
                const int d0 = 16 * t + tr_d0;
                // fp8 V tiles keep the K layout (their stores take two columns per lane)
                const int off = (KV8 ? lds_col<C::VLRB, C::VSWM>(tr_row, d0 >> 3)
                                     : lds_vcol<C::VLRB, C::VSWM>(tr_row, d0 >> 3)) + ((d0 & 7) << 1);
                typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
                typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
                const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(vlds + off));
                vop[t] = __builtin_bit_cast(short4_t, v);
            }
            const float4_t* const xb = xbuf + (k & 1) * NCB * C::NW * 64;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if (cb > 0 && 16 * cb >= M) break;
                const int w0 = cb * C::NW + (wave / C::SPLIT) * C::SPLIT;   // the group's first wave
                float4_t sc = xb[w0 * 64 + lane];
#pragma unroll
                for (int w = 1; w < C::SPLIT; ++w) sc += xb[(w0 + w) * 64 + lane];
                // lane holds keys key0 + 4*grp + j for query row 16cb + col
                const int lim = min(nv, nvis[cb] - key0);
                const int low = nlo[cb] - key0;
                float x[4];
                float mt = -INFINITY;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kj = 4 * grp + j;
                    x[j] = (kj < lim && kj >= low) ? sc[j] * a.score_scale_log2 : -INFINITY;
                    mt = fmaxf(mt, x[j]);
                }
                mt = max_over_row_groups(mt);
                const bool grow = mt > m_run[cb] + kRescaleSlack;
                if (__builtin_amdgcn_ballot_w64(grow)) {
                    const float mnew = grow ? mt : m_run[cb];
                    const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[cb] - mnew);
                    l_run[cb] *= alpha;
#pragma unroll
                    for (int t = 0; t < NDT; ++t) acc[cb][t] *= alpha;
                    m_run[cb] = mnew;
                }
                const float mref = m_run[cb] == -INFINITY ? 0.f : m_run[cb];
                float p[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    p[j] = __builtin_amdgcn_exp2f(x[j] - mref);
                    l_run[cb] += p[j];
                }
                const u32x2_t pc = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
                const short4_t pop = __builtin_bit_cast(short4_t, pc);
#pragma unroll
                for (int t = 0; t < C::DTW; ++t)
                    acc[cb][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop[t], pop, acc[cb][t], 0, 0, 0);
            }
        };

#pragma unroll
        for (int st = 0; st < PF; ++st) issue(st, st, pfirst[st]);
        // Software pipeline over the chunks: iteration k runs stage A of chunk k, then stage B of
        // chunk k - 1 (whose partial scores every wave wrote before the previous barrier), then one
        // barrier.  Stage A of chunk k overwrites tile and exchange buffer k & 1, last read by stage
        // B of chunk k - 2 before that barrier.  The trip count is the same for every wave.
        // rounds of the longest stream (stream 0's), so every wave meets every barrier
        const int rounds = ((nchunks + C::NS - 1) / C::NS + PF - 1) / PF;
        int key0_prev = 0, nv_prev = 0;
        for (int k0 = 0; k0 < rounds * PF; k0 += PF) {
#pragma unroll
            for (int st = 0; st < PF; ++st) {
                const int k = k0 + st;
                const int nv = nvalid_st[st];
                stage_a(st, k);
                if (k > 0 && k - 1 < my_chunks) stage_b(k - 1, key0_prev, nv_prev);
                key0_prev = si.k_lo + 16 * chunk_of(k);
                nv_prev = nv;
                __syncthreads();
            }
        }
        if (rounds > 0 && rounds * PF - 1 < my_chunks) stage_b(rounds * PF - 1, key0_prev, nv_prev);
        // the waves of a group hold the same (m, l); the NS group states merge in LDS, each wave
        // adding its columns of acc
        const int stream = wave / C::SPLIT;
        const bool lead = wave % C::SPLIT == 0;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) l_run[cb] = sum_over_row_groups(l_run[cb]);
        __syncthreads();   // staging and exchange buffers are free from here on
        if (lead && grp == 0) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) mbuf[stream * C::ROWS + 16 * cb + col] = m_run[cb];
        }
        __syncthreads();
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int n = 16 * cb + col;
            float Mx = -INFINITY;
#pragma unroll
            for (int q = 0; q < C::NS; ++q) Mx = fmaxf(Mx, mbuf[q * C::ROWS + n]);
            const float f = __builtin_amdgcn_exp2f(m_run[cb] - (Mx == -INFINITY ? 0.f : Mx));
            l_run[cb] *= f;
#pragma unroll
            for (int t = 0; t < C::DTW; ++t) acc[cb][t] *= f;
            if (wave == 0 && grp == 0) Mbuf[n] = Mx;
        }
#pragma unroll
        for (int q = 0; q < C::NS; ++q) {
            if (stream == q) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const int n = 16 * cb + col;
#pragma unroll
                    for (int t = 0; t < C::DTW; ++t) {
                        float4_t* dst = reinterpret_cast<float4_t*>(abuf + n * C::APITCH + dcol0 + 16 * t + 4 * grp);
                        *dst = (q == 0) ? acc[cb][t] : (*dst + acc[cb][t]);
                    }
                    if (lead && grp == 0) lbuf[n] = (q == 0) ? l_run[cb] : (lbuf[n] + l_run[cb]);
                }
            }
            __syncthreads();
        }
    } else {

    u32x4_t kreg[C::PF][C::NLD], vreg[C::PF][C::NLD];
    int nvalid_st[C::PF];
    // The 16-byte piece of a chunk that lane `lane` holds in load step it: row r, 16-byte HBM column
    // c.  By default the pieces go to the lanes in row-major order.  With fp8 at head_dim 128 (8 HBM
    // columns a row) each widened piece fills LDS columns 2c and 2c + 1 of a 16-column row, and eight
    // lanes of a row storing columns 2c would meet on the same banks (columns c and c + 4); so there
    // each group of eight lanes takes half of two adjacent rows instead (four lanes, 64 contiguous
    // bytes, per row), whose swizzled columns then differ in their low three bits.
    auto piece_row = [&](int it) -> int {
        if constexpr (KV8 && C::GCPR == 8) return 8 * it + 2 * (lane >> 4) + ((lane >> 2) & 1);
        return (it * 64 + lane) / C::GCPR;
    };
    auto piece_col = [&](int it) -> int {
        if constexpr (KV8 && C::GCPR == 8) return 4 * ((lane >> 3) & 1) + (lane & 3);
        return (it * 64 + lane) % C::GCPR;
    };
    // K and V of the wave's k-th chunk from page `page`: 16 rows of GRB bytes each, one 16-byte
    // load per lane and step, non-temporal.  A chunk past the wave's work, past the context or on an
    // invalid page loads zeros (no records) and stages as an empty chunk.
    auto issue = [&](int st, int k, int page) {
        const int c = chunk_of(k);
        const int key0 = si.k_lo + 16 * c;
        const int blk = __builtin_amdgcn_readfirstlane(page);
        const bool live = k < my_chunks && blk >= 0 && blk < a.num_blocks;
        const int nv = live ? max(min(16, si.k_hi - key0), 0) : 0;
        nvalid_st[st] = nv;
        const int off = key0 & (a.block_size - 1);
        const size_t base = nv > 0 ? (static_cast<size_t>(blk) * a.num_kv_heads + g) * head_stride +
                                         static_cast<size_t>(off) * C::GRB
                                   : 0;
        const int records = nv > 0 ? 16 * C::GRB : 0;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(a.k_cache + base), 0, records, kRawBufferWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(a.v_cache + base), 0, records, kRawBufferWord3);
#pragma unroll
        for (int it = 0; it < C::NLD; ++it) {
            const int off = (piece_row(it) * C::GCPR + piece_col(it)) * 16;
            kreg[st][it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                           rk, off, 0, kLoadNonTemporal));
            vreg[st][it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                           rv, off, 0, kLoadNonTemporal));
        }
    };

    // Write a staged chunk into the wave's LDS tiles as bf16 rows; rows >= nv are zero.
    auto stage = [&](int st, int nv, bool full, int cbuf) {
        uint8_t* const klds = wlds + cbuf * 2 * 16 * C::LRB;
        uint8_t* const vlds = klds + 16 * C::LRB;
#pragma unroll
        for (int it = 0; it < C::NLD; ++it) {
            const int r = piece_row(it);
            const int c = piece_col(it);
            u32x4_t kv = kreg[st][it];
            u32x4_t vv = vreg[st][it];
            if (!full) {
                const bool ok = r < nv;
                const u32x4_t z = {0u, 0u, 0u, 0u};
                kv = ok ? kv : z;
                vv = ok ? vv : z;
            }
            if constexpr (!KV8) {
                const int off = lds_col<C::LRB, C::SWM>(r, c);
                *reinterpret_cast<u32x4_t*>(klds + off) = kv;
                *reinterpret_cast<u32x4_t*>(vlds + off) = vv;
            } else {
                // 16 fp8 codes -> 16 bf16 values = two LDS columns (2c, 2c+1), widened exactly
                u32x4_t klo, khi, vlo, vhi;
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    klo[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kv[w], 1.0f, false));
                    klo[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kv[w], 1.0f, true));
                    khi[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kv[w + 2], 1.0f, false));
                    khi[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kv[w + 2], 1.0f, true));
                    vlo[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vv[w], 1.0f, false));
                    vlo[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vv[w], 1.0f, true));
                    vhi[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vv[w + 2], 1.0f, false));
                    vhi[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vv[w + 2], 1.0f, true));
                }
                const int o0 = lds_col<C::LRB, C::SWM>(r, 2 * c);
                const int o1 = lds_col<C::LRB, C::SWM>(r, 2 * c + 1);
                *reinterpret_cast<u32x4_t*>(klds + o0) = klo;
                *reinterpret_cast<u32x4_t*>(klds + o1) = khi;
                *reinterpret_cast<u32x4_t*>(vlds + o0) = vlo;
                *reinterpret_cast<u32x4_t*>(vlds + o1) = vhi;
            }
        }
    };

    // Per-lane address of the transposed V read for d-tile 0: lane (16G + 4k + m) reads the 4 bf16
    // of row 4G + k at d = 4m; the hardware hands lane 16G + i the column d = i of rows 4G..4G+3.
    const int tr_row = 4 * grp + ((lane >> 2) & 3);
    const int tr_d0 = 4 * (lane & 3);

#pragma unroll
    for (int st = 0; st < C::PF; ++st) issue(st, st, pfirst[st]);

    // whole rounds of PF chunks; the padding chunks past my_chunks are empty and fetch nothing
    constexpr int CG = C::CG;
    const int rounds = (my_chunks + C::PF - 1) / C::PF;
    for (int k0 = 0; k0 < rounds * C::PF; k0 += C::PF) {
#pragma unroll
        for (int sg = 0; sg < C::PF; sg += CG) {
            // stage the step's CG chunks, each followed by the loads PF chunks ahead
            int key0[CG], nvc[CG];
#pragma unroll
            for (int c = 0; c < CG; ++c) {
                const int st = sg + c;
                const int k = k0 + st;
                key0[c] = si.k_lo + 16 * chunk_of(k);
                nvc[c] = nvalid_st[st];
                compiler_fence();
                if (nvc[c] == 16) stage(st, 16, true, c);   // uniform: only a ragged last chunk is partial
                else stage(st, nvc[c], false, c);
                compiler_fence();
                const int page = pnext[st];            // fetched before chunk k's K/V: already here
                pnext[st] = page_load(k + 2 * C::PF);
                issue(st, k + C::PF, page);
            }

            // K operands (A of S^T): row = col, d = 32s + 8*grp .. +8; V^T operands (A of
            // O^T = V^T.P^T): d = 16t + col, keys 4*grp + j, via transposed reads
            bf16x8_t kop[CG][C::KSTEPS];
            short4_t vop[CG][C::DT];
#pragma unroll
            for (int c = 0; c < CG; ++c) {
                const uint8_t* klds = wlds + c * 2 * 16 * C::LRB;
                const uint8_t* vlds = klds + 16 * C::LRB;
#pragma unroll
                for (int s = 0; s < C::KSTEPS; ++s)
                    kop[c][s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                                 klds + lds_col<C::LRB, C::SWM>(col, 4 * s + grp)));
#pragma unroll
                for (int t = 0; t < C::DT; ++t) {
                    const int d0 = 16 * t + tr_d0;
                    const int off = lds_col<C::LRB, C::SWM>(tr_row, d0 >> 3) + ((d0 & 7) << 1);
                    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
                    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
                    const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(vlds + off));
                    vop[c][t] = __builtin_bit_cast(short4_t, v);
                }
            }
            compiler_fence();

#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if (cb > 0 && 16 * cb >= M) break;     // a block past the request's rows: nothing
                float4_t sacc[CG];
#pragma unroll
                for (int c = 0; c < CG; ++c) {
                    sacc[c] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < C::KSTEPS; ++s)
                        sacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[c][s], qop[cb][s], sacc[c], 0, 0, 0);
                }
                // lane holds keys key0[c] + 4*grp + j of each chunk for query row 16cb + col
                float x[CG][4];
                float mt = -INFINITY;
                bool whole = true;                       // every key of the step visible to every row
#pragma unroll
                for (int c = 0; c < CG; ++c)
                    whole = whole && nvc[c] == 16 && key0[c] + 16 <= nvis_lo && key0[c] >= nlo_hi;
                if (whole) {
#pragma unroll
                    for (int c = 0; c < CG; ++c)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            x[c][j] = sacc[c][j] * a.score_scale_log2;
                            mt = fmaxf(mt, x[c][j]);
                        }
                } else {
#pragma unroll
                    for (int c = 0; c < CG; ++c) {
                        const int lim = min(nvc[c], nvis[cb] - key0[c]);
                        const int low = nlo[cb] - key0[c];    // window start relative to the chunk
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int kj = 4 * grp + j;
                            x[c][j] = (kj < lim && kj >= low) ? sacc[c][j] * a.score_scale_log2 : -INFINITY;
                            mt = fmaxf(mt, x[c][j]);
                        }
                    }
                }
                mt = max_over_row_groups(mt);
                // lazy rescale: move the reference only when the row max passes it by the slack
                const bool grow = mt > m_run[cb] + kRescaleSlack;
                if (__builtin_amdgcn_ballot_w64(grow)) {
                    const float mnew = grow ? mt : m_run[cb];
                    // a row with no visible key yet keeps (-inf, 0, 0): never form -inf - -inf
                    const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[cb] - mnew);
                    l_run[cb] *= alpha;
#pragma unroll
                    for (int t = 0; t < C::DT; ++t) acc[cb][t] *= alpha;
                    m_run[cb] = mnew;
                }
                const float mref = m_run[cb] == -INFINITY ? 0.f : m_run[cb];
                uint32_t pk[CG][2];
#pragma unroll
                for (int c = 0; c < CG; ++c) {
                    float p[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        p[j] = __builtin_amdgcn_exp2f(x[c][j] - mref);
                        l_run[cb] += p[j];
                    }
                    pk[c][0] = pack_bf16x2(p[0], p[1]);
                    pk[c][1] = pack_bf16x2(p[2], p[3]);
                }
                if constexpr (CG == 2) {
                    // one K = 32 product per d tile over both chunks: the contraction index 8*grp + jj
                    // stands for key 4*grp + jj of the first chunk (jj < 4) or of the second (jj >= 4),
                    // which is exactly what this lane holds of P and of the transposed V reads
                    const u32x4_t pc = {pk[0][0], pk[0][1], pk[1][0], pk[1][1]};
                    const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, pc);
#pragma unroll
                    for (int t = 0; t < C::DT; ++t) {
                        const u32x2_t va = __builtin_bit_cast(u32x2_t, vop[0][t]);
                        const u32x2_t vb = __builtin_bit_cast(u32x2_t, vop[1][t]);
                        const u32x4_t vc = {va[0], va[1], vb[0], vb[1]};
                        acc[cb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vc), pop,
                                                                             acc[cb][t], 0, 0, 0);
                    }
                } else {
                    const u32x2_t pc = {pk[0][0], pk[0][1]};
                    const short4_t pop = __builtin_bit_cast(short4_t, pc);
#pragma unroll
                    for (int t = 0; t < C::DT; ++t)
                        acc[cb][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop[0][t], pop, acc[cb][t], 0, 0, 0);
                }
            }
        }
    }

    // ---- merge the wave states in LDS ----
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        l_run[cb] = sum_over_row_groups(l_run[cb]);
    }
    if constexpr (C::PARK) {
        // the wave's own tile: no other wave reads it, and this wave's reads of it are done (LDS
        // operations of a wave complete in order)
        float* const ws = reinterpret_cast<float*>(wlds);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int n = 16 * cb + col;
#pragma unroll
            for (int t = 0; t < C::DT; ++t)
                *reinterpret_cast<float4_t*>(ws + n * C::APITCH + 16 * t + 4 * grp) = acc[cb][t];
            if (grp == 0) {
                ws[C::ROWS * C::APITCH + n] = m_run[cb];
                ws[C::ROWS * C::APITCH + C::ROWS + n] = l_run[cb];
            }
        }
        __syncthreads();
    } else {
    __syncthreads();   // staging buffers are free from here on
    if (grp == 0) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) mbuf[wave * C::ROWS + 16 * cb + col] = m_run[cb];
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int n = 16 * cb + col;
        float Mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < C::NW; ++w) Mx = fmaxf(Mx, mbuf[w * C::ROWS + n]);
        const float mref = Mx == -INFINITY ? 0.f : Mx;
        const float f = __builtin_amdgcn_exp2f(m_run[cb] - mref);
        l_run[cb] *= f;
#pragma unroll
        for (int t = 0; t < C::DT; ++t) acc[cb][t] *= f;
        if (wave == 0 && grp == 0) Mbuf[n] = Mx;
    }
#pragma unroll
    for (int w = 0; w < C::NW; ++w) {
        if (wave == w) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int n = 16 * cb + col;
#pragma unroll
                for (int t = 0; t < C::DT; ++t) {
                    float4_t* dst = reinterpret_cast<float4_t*>(abuf + n * C::APITCH + 16 * t + 4 * grp);
                    *dst = (w == 0) ? acc[cb][t] : (*dst + acc[cb][t]);
                }
                if (grp == 0) lbuf[n] = (w == 0) ? l_run[cb] : (lbuf[n] + l_run[cb]);
            }
        }
        __syncthreads();
    }
    }
    }

    // merged state of row n, columns 4*d4 .. +4: from the LDS state, or from the NW parked states
    // (max of the wave maxima, each wave rescaled to it, summed in wave order)
    auto state_at = [&](int n, int d4, float& m, float& l) -> float4_t {
        if constexpr (C::PARK) {
            float mw[C::NW];
            float Mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < C::NW; ++w) {
                mw[w] = reinterpret_cast<const float*>(lds + w * C::WAVE_LDS)[C::ROWS * C::APITCH + n];
                Mx = fmaxf(Mx, mw[w]);
            }
            const float mref = Mx == -INFINITY ? 0.f : Mx;
            float4_t v = float4_t{0.f, 0.f, 0.f, 0.f};
            l = 0.f;
#pragma unroll
            for (int w = 0; w < C::NW; ++w) {
                const float* ws = reinterpret_cast<const float*>(lds + w * C::WAVE_LDS);
                const float f = __builtin_amdgcn_exp2f(mw[w] - mref);
                v += f * *reinterpret_cast<const float4_t*>(ws + n * C::APITCH + 4 * d4);
                l += f * ws[C::ROWS * C::APITCH + C::ROWS + n];
            }
            m = Mx;
            return v;
        } else {
            m = Mbuf[n];
            l = lbuf[n];
            return *reinterpret_cast<const float4_t*>(abuf + n * C::APITCH + 4 * d4);
        }
    };

    // ---- write the slot's states: rows n < M, token i = n / G, head g*G + n % G ----
    constexpr int D4 = D / 4;
    if (!a.prefill) {
        const size_t slot_base = static_cast<size_t>(slot) * a.max_q_len;
        for (int e = tid; e < M * D4; e += 64 * C::NW) {
            const int n = e / D4;
            const int d4 = e - n * D4;
            const int i = n / G;
            const int h = g * G + (n - i * G);
            const size_t st = (slot_base + i) * a.num_q_heads + h;
            float mn, ln;
            float4_t v = state_at(n, d4, mn, ln);
            v *= a.v_scale;
            *reinterpret_cast<float4_t*>(a.ws_acc + st * D + 4 * d4) = v;
            if (d4 == 0) *reinterpret_cast<float2*>(a.ws_ml + st * 2) = make_float2(mn, ln);
        }
        return;
    }
    // a prefill block holds its rows' whole softmax state: the rows are written normalised
    for (int e = tid; e < M * D4; e += 64 * C::NW) {
        const int n = e / D4;
        const int d4 = e - n * D4;
        const int i = n / G;
        const int h = g * G + (n - i * G);
        float mn, l;
        const float4_t sv = state_at(n, d4, mn, l);
        const float inv = l > 0.f ? a.v_scale / l : 0.f;
        const float4_t v = sv * inv;
        const size_t o = (static_cast<size_t>(si.row0 + i) * a.num_q_heads + h) * D + 4 * d4;
        if (a.out_bf16) {
            uint2 w;
            w.x = pack_bf16x2(v[0], v[1]);
            w.y = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o) = w;
        } else {
            *reinterpret_cast<float4_t*>(static_cast<float*>(a.out) + o) = v;
        }
    }
}

// ---------------------------------------------------------------------------------------------
// fp32-cache kernel: plain vector ALU code, fp32 throughout
// ---------------------------------------------------------------------------------------------
template <int D, bool QF32>
__global__ __launch_bounds__(256) void decode_f32_kernel(const DecodeArgs a) {
    __shared__ float qbuf[4][D];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int slot = blockIdx.x / a.num_kv_heads;
    const int g = blockIdx.x - slot * a.num_kv_heads;
    SlotInfo si;
    if (a.pieces) {
        // shared slots: this workgroup's piece (slot is then the piece index)
        int4 wk;
        int2 nwk;
        pieces_from_plan<4>(a, slot, wk, nwk);
        if (!entry_info(a, wk, slot < nwk.x, si)) return;
    } else if (!slot_info(a, slot, si)) {
        return;
    }
    const int G = a.group;
    const int M = G * si.L;
    constexpr int E = D / 64;
    const int* bt_row = a.block_tables + static_cast<size_t>(si.b) * a.max_blocks;
    const float* kc = reinterpret_cast<const float*>(a.k_cache);
    const float* vc = reinterpret_cast<const float*>(a.v_cache);

    for (int n = wave; n < M; n += 4) {
        const int i = n / G;
        const int h = g * G + (n - i * G);
        const int nv = si.S - (si.L - 1 - i);
        const int lo = a.window > 0 ? max(si.k_lo, nv - a.window) : si.k_lo;
        const int hi = min(si.k_hi, nv);
        const size_t qoff = (static_cast<size_t>(si.row0 + i) * a.num_q_heads + h) * D;
        compiler_fence();
        for (int d = lane; d < D; d += 64) {
            if constexpr (QF32) qbuf[wave][d] = static_cast<const float*>(a.q)[qoff + d];
            else qbuf[wave][d] = bf16_to_f32(static_cast<const uint16_t*>(a.q)[qoff + d]);
        }
        compiler_fence();
        float m = -INFINITY, l = 0.f;
        float acc[E];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = 0.f;
        for (int base = lo; base < hi; base += 64) {
            const int p = base + lane;
            int blk = -1;
            float x = -INFINITY;
            if (p < hi) {
                blk = bt_row[p / a.block_size];
                if (blk < 0 || blk >= a.num_blocks) blk = -1;
            }
            if (blk >= 0) {
                const float* kp = kc + ((static_cast<size_t>(blk) * a.num_kv_heads + g) * a.block_size + p % a.block_size) * D;
                float dot = 0.f;
                for (int d = 0; d < D; d += 4) {
                    const float4 kv = *reinterpret_cast<const float4*>(kp + d);
                    dot = fmaf(qbuf[wave][d], kv.x, dot);
                    dot = fmaf(qbuf[wave][d + 1], kv.y, dot);
                    dot = fmaf(qbuf[wave][d + 2], kv.z, dot);
                    dot = fmaf(qbuf[wave][d + 3], kv.w, dot);
                }
                x = dot * a.score_scale_log2;
            }
            const float mt = wave_max(x);
            const float mnew = fmaxf(m, mt);
            const float mref = mnew == -INFINITY ? 0.f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(m - mref);
            const float pr = blk >= 0 ? __builtin_amdgcn_exp2f(x - mref) : 0.f;
            l = l * alpha + wave_sum(pr);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] *= alpha;
            const int cnt = min(64, hi - base);
            for (int k = 0; k < cnt; ++k) {
                const int bk = __builtin_amdgcn_readlane(blk, k);
                if (bk < 0) continue;
                const float pk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pr), k));
                const int pos = base + k;
                const float* vp = vc + ((static_cast<size_t>(bk) * a.num_kv_heads + g) * a.block_size + pos % a.block_size) * D;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[e] = fmaf(pk, vp[lane + 64 * e], acc[e]);
            }
            m = mnew;
        }
        const size_t st = (static_cast<size_t>(slot) * a.max_q_len + i) * a.num_q_heads + h;
#pragma unroll
        for (int e = 0; e < E; ++e) a.ws_acc[st * D + lane + 64 * e] = acc[e] * a.v_scale;
        if (lane == 0) *reinterpret_cast<float2*>(a.ws_ml + st * 2) = make_float2(m, l);
    }
}

// Workgroups of one part: its slots (or query blocks) times kv heads, and in prefill mode a trailing
// workgroup per NW rows for the zero fill of the rows past the last request.
template <int NW>
unsigned part_workgroups(const DecodeArgs& a) {
    unsigned n = static_cast<unsigned>(a.capacity) * static_cast<unsigned>(a.num_kv_heads);
    if (a.prefill) n += static_cast<unsigned>((a.num_rows + NW - 1) / NW);
    return n;
}

template <int D, int NCB, bool KV8, int NW = 4>
hipError_t launch_mfma_q(const DecodeArgs& a, bool qf32, dim3 grid, hipStream_t stream) {
    (void)grid;
    LaunchArgs L;
    L.part[0] = a;
    L.part[1] = a;
    L.split = INT_MAX;
    const dim3 g(part_workgroups<NW>(a));
    const dim3 block(64 * NW);
    if (qf32) hipLaunchKernelGGL((decode_mfma_kernel<D, NCB, KV8, true, NW, false>), g, block, 0, stream, L);
    else hipLaunchKernelGGL((decode_mfma_kernel<D, NCB, KV8, false, NW, false>), g, block, 0, stream, L);
    return hipGetLastError();
}

template <int D, int NCB, bool KV8>
hipError_t launch_mixed_q(const DecodeArgs& dec, const DecodeArgs& pre, bool qf32, hipStream_t stream) {
    constexpr int NW = 4;
    LaunchArgs L;
    L.part[0] = dec;
    L.part[1] = pre;
    L.split = static_cast<int>(part_workgroups<NW>(dec));
    const dim3 g(static_cast<unsigned>(L.split) + part_workgroups<NW>(pre));
    const dim3 block(64 * NW);
    if (qf32) hipLaunchKernelGGL((decode_mfma_kernel<D, NCB, KV8, true, NW, true>), g, block, 0, stream, L);
    else hipLaunchKernelGGL((decode_mfma_kernel<D, NCB, KV8, false, NW, true>), g, block, 0, stream, L);
    return hipGetLastError();
}

template <int D, bool KV8>
hipError_t launch_mixed_ncb(const DecodeArgs& dec, const DecodeArgs& pre, int ncb, bool qf32, hipStream_t stream) {
    if (ncb == 1) return launch_mixed_q<D, 1, KV8>(dec, pre, qf32, stream);
    if (ncb == 2) return launch_mixed_q<D, 2, KV8>(dec, pre, qf32, stream);
    return launch_mixed_q<D, 4, KV8>(dec, pre, qf32, stream);
}

template <int D, bool KV8>
hipError_t launch_mfma_ncb(const DecodeArgs& a, int ncb, bool qf32, dim3 grid, hipStream_t stream) {
    // every request one slot (the capacity is the batch): slot sizes follow the request lengths
    // and the longest requests set the time, so eight waves share each slot evenly -- unless the
    // slots are shared (cut into pieces of about half the mean slot, see piece_size), which the
    // four-wave form streams faster (measured: fp8 workload step 171 against 175 us)
    const bool one_slot_each = !a.prefill && (a.plan_inline ? a.plan_cap : a.capacity) <= a.num_seqs;
    if constexpr (D <= 128) {
        if (ncb == 1 && one_slot_each && !a.pieces) return launch_mfma_q<D, 1, KV8, 8>(a, qf32, grid, stream);
    }
    if (ncb == 1) return launch_mfma_q<D, 1, KV8>(a, qf32, grid, stream);
    if (ncb == 2) return launch_mfma_q<D, 2, KV8>(a, qf32, grid, stream);
    return launch_mfma_q<D, 4, KV8>(a, qf32, grid, stream);
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, pa_dtype kv, int ncb, bool qf32, dim3 grid, hipStream_t stream) {
    if (kv == PA_F32) {
        if (qf32) hipLaunchKernelGGL((decode_f32_kernel<D, true>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((decode_f32_kernel<D, false>), grid, dim3(256), 0, stream, a);
        return hipGetLastError();
    }
    if (kv == PA_BF16) return launch_mfma_ncb<D, false>(a, ncb, qf32, grid, stream);
    return launch_mfma_ncb<D, true>(a, ncb, qf32, grid, stream);
}

}  // namespace

int prefill_block_tokens(int head_dim, int group) {
    // rows per workgroup: 64 (four 16-row matrix blocks) where the operands fit in registers, one
    // block for head_dim 256, more only when a single token's heads need them
    int rows = head_dim <= 128 ? 64 : 16;
    while (rows < group && rows < PA_MAX_GROUP_ROWS) rows *= 2;
    return group > 0 ? (rows / group > 0 ? rows / group : 1) : 1;
}

hipError_t launch_prefill(const DecodeArgs& a, int head_dim, pa_dtype kv_dtype, bool q_f32,
                          hipStream_t stream) {
    const int ncb = column_blocks(a.group * a.block_tokens);
    const dim3 grid(static_cast<unsigned>(a.capacity) * static_cast<unsigned>(a.num_kv_heads));
    switch (head_dim) {
        case 64: return launch_d<64>(a, kv_dtype, ncb, q_f32, grid, stream);
        case 128: return launch_d<128>(a, kv_dtype, ncb, q_f32, grid, stream);
        default: return launch_d<256>(a, kv_dtype, ncb, q_f32, grid, stream);
    }
}

bool mixed_launch_supported(int head_dim, pa_dtype kv_dtype, int ncb) {
    return (head_dim == 64 || head_dim == 128 || head_dim == 256) &&
           (kv_dtype == PA_BF16 || kv_dtype == PA_FP8_E4M3) && ncb >= 1 && ncb <= 4 && ncb != 3;
}

hipError_t launch_mixed(const DecodeArgs& dec, const DecodeArgs& pre, int head_dim, pa_dtype kv_dtype,
                        bool q_f32, int ncb, hipStream_t stream) {
    if (!mixed_launch_supported(head_dim, kv_dtype, ncb)) return hipErrorInvalidValue;
    const bool kv8 = kv_dtype == PA_FP8_E4M3;
    switch (head_dim) {
        case 64: return kv8 ? launch_mixed_ncb<64, true>(dec, pre, ncb, q_f32, stream)
                            : launch_mixed_ncb<64, false>(dec, pre, ncb, q_f32, stream);
        case 128: return kv8 ? launch_mixed_ncb<128, true>(dec, pre, ncb, q_f32, stream)
                             : launch_mixed_ncb<128, false>(dec, pre, ncb, q_f32, stream);
        default: return kv8 ? launch_mixed_ncb<256, true>(dec, pre, ncb, q_f32, stream)
                            : launch_mixed_ncb<256, false>(dec, pre, ncb, q_f32, stream);
    }
}

hipError_t launch_decode(const DecodeArgs& a, int head_dim, pa_dtype kv_dtype, bool q_f32,
                         hipStream_t stream) {
    const int ncb = column_blocks(a.group * a.max_q_len);
    const dim3 grid(static_cast<unsigned>(a.capacity) * static_cast<unsigned>(a.num_kv_heads));
    if (grid.x == 0) return hipSuccess;
    switch (head_dim) {
        case 64: return launch_d<64>(a, kv_dtype, ncb, q_f32, grid, stream);
        case 128: return launch_d<128>(a, kv_dtype, ncb, q_f32, grid, stream);
        default: return launch_d<256>(a, kv_dtype, ncb, q_f32, grid, stream);
    }
}

}  // namespace pa

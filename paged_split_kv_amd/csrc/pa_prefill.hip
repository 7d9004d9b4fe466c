// pa_prefill.hip -- the prompt rows of a mixed batch, as planned query blocks (gfx950).
//
// What is computed (opengfx1030/vllm-rdna PR #29, Change items 1 and 2: prompt rows after the decode
// requests go to a prefill path; every query token i of a request with L tokens and S keys sees the
// keys [0, S - (L-1-i)), or its last W of them under a sliding window): pa_prefill's split form cuts
// each request's query tokens into blocks, plans the blocks like requests (ROCm/ATOM PR #2366,
// sections 1 and 3), and this kernel computes, for every plan slot (block b, tiles [tb, te)) and kv
// head g, the softmax state of the slot's keys for each query row of the block; pa_merge combines a
// block's slots into its rows.
//
// Unlike a decode slot, a block holds many query rows (G heads x up to ROWS / G tokens), so the
// product is a dense one and the kernel is organised for the matrix cores rather than for streaming:
//  * one workgroup of 8 waves (two per SIMD) per (slot, kv head); wave w owns RB blocks of 16 query
//    rows (rows 16 RB w .. 16 RB (w+1) - 1 of the block) and all D columns of their accumulators,
//    which with the query operands fit the 256 registers of a wave with no copies between register
//    files;
//  * the slot's keys go in chunks of 32, loaded with 16-byte coalesced non-temporal loads as bf16
//    rows into LDS tiles, K and V each with an XOR swizzle of its own on the 16-byte column: bf16
//    caches at head_dim >= 128 straight from HBM into a ring of four LDS chunk buffers (each half of
//    the waves loading one 16-key half of every chunk), fp8 (widened on the way) and head_dim 64
//    through registers into two; every wave then reads the whole chunk, so each K/V byte is fetched
//    once per workgroup and read from LDS by 8 waves;
//  * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (keys as rows, query rows as columns), the online
//    softmax in base 2 with lazy rescaling, and O^T = V^T . P^T on the same instruction over the 32
//    keys (V^T from the LDS transpose read), as in the decode kernel;
//  * the waves' rows are disjoint, so each wave writes its states straight from registers.
#include "pa_device.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(4))) int cint4;

// Word 3 of a raw buffer resource (32-bit data format, no swizzle): loads past the byte count return
// zero without touching memory.  Cache-policy operand 2 marks a load non-temporal.
constexpr int kRawWord3 = 0x00020000;
constexpr int kNonTemporal = 2;
// Rescale threshold of the running maximum, in base-2 units: probabilities stay below 2^8.
constexpr float kSlack = 8.0f;

// One direct load: each lane reads 16 bytes at its offset in the (scalar) buffer resource and the
// unit writes them to LDS at dst + 16 * lane, with zeros for lanes past the byte count.  The block
// names no register as output (the data goes to LDS only), and it is hand-written so that the
// compiler does not count it: otherwise it waits for every direct load in flight before each
// transposed LDS read.  The caller waits with explicit vector-memory counts before reading the data.
__device__ __forceinline__ void lds_load16(u32x4_t rsrc, const lds_void* dst, int voffset) {
    const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<size_t>(dst));
    asm volatile("buffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "{m0}"(m0), "v"(voffset), "s"(rsrc)
                 : "memory");
}

// The four words of a raw buffer resource over [base, base + records).
__device__ __forceinline__ u32x4_t raw_rsrc(const uint8_t* base, int records) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return u32x4_t{static_cast<uint32_t>(p), static_cast<uint32_t>(p >> 32) & 0xffffu,
                   static_cast<uint32_t>(records), static_cast<uint32_t>(kRawWord3)};
}

template <int D, bool KV8>
struct Tile {
    static constexpr int NW = 8;                       // waves (two per SIMD)
    static constexpr int NT = 64 * NW;
    static constexpr int RB = D == 256 ? 1 : 2;        // 16-row blocks per wave
    static constexpr int ROWS = NW * 16 * RB;          // query rows per workgroup
    static constexpr int KC = 32;                      // keys per chunk
    static constexpr int ESZ = KV8 ? 1 : 2;            // bytes per cached element
    static constexpr int GRB = D * ESZ;                // HBM bytes per key row
    static constexpr int PPR = GRB / 16;               // 16-byte HBM pieces per key row
    static constexpr int PIECES = KC * PPR;            // per chunk, of K (and of V)
    static constexpr int NL = (PIECES + NT - 1) / NT;  // pieces per thread per chunk
    static constexpr int LRB = D * 2;                  // LDS bytes per row (bf16)
    static constexpr int LCPR = LRB / 16;              // 16-byte LDS columns per row
    static constexpr int SWM = (LCPR < 16 ? LCPR : 16) - 1;
    static constexpr int TILE = KC * LRB;              // one K or V tile
    // bf16 caches at head_dim >= 128 load chunks straight into LDS (no staging registers), NBUF
    // chunks deep; fp8 (widened on the way) and head_dim 64 stage through registers, two deep
    static constexpr bool DMA = !KV8 && D >= 128;
    static constexpr int NBUF = DMA ? 4 : 2;           // LDS chunk buffers
    static constexpr int NLD = DMA ? 2 * PIECES / NT : 0;   // direct loads per thread per chunk (K and V)
    static constexpr int LDS = NBUF * 2 * TILE;        // K and V of NBUF chunks
    static constexpr int KS = D / 32;                  // k-steps of S^T
    static constexpr int DT = D / 16;                  // d tiles of O^T
    static_assert(NT % PPR == 0 || PIECES <= NT, "a wave's pieces lie in one half-chunk");
    static_assert(!DMA || (PIECES % NT == 0 && PPR == LCPR), "direct loads: whole 1 KB runs per wave");
};

// XOR swizzles of the 16-byte columns, one per tile (measured with the kernel's own read patterns;
// rows of 256 bytes and up all start on the same bank):
//  * K tiles are read 16 rows x one column per quarter wave (16-byte reads): r & 15 keeps those
//    reads at the full LDS rate;
//  * V tiles are read by the transposing 8-byte reads, each half wave taking 8 rows x two adjacent
//    columns: r & 15 puts rows r and r ^ 1 on the same two columns, so with 16 columns a row the V
//    XOR is even on rows 0-7 and odd on rows 8-15, which spreads them over 16 distinct columns.
template <int SWM>
__device__ __forceinline__ int kxor(int r) { return r & SWM; }
template <int SWM>
__device__ __forceinline__ int vxor(int r) {
    if constexpr (SWM == 15) return ((r & 7) << 1) | ((r >> 3) & 1);
    else return r & SWM;
}

// Byte offset of 16-byte column c of row r of a bf16 tile whose row r columns are XORed with x.
template <int LRB>
__device__ __forceinline__ int tile_col(int r, int c, int x) {
    return r * LRB + ((c ^ x) << 4);
}

__device__ __forceinline__ float row_max4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float row_sum4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 16 fp8 (e4m3fn) codes -> 16 bf16 values (exact), as two 16-byte LDS columns.
__device__ __forceinline__ void widen_fp8(const u32x4_t& v, u32x4_t& lo, u32x4_t& hi) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        lo[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[w], 1.0f, false));
        lo[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[w], 1.0f, true));
        hi[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[w + 2], 1.0f, false));
        hi[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[w + 2], 1.0f, true));
    }
}

template <int D, bool KV8, bool QF32>
__global__ __launch_bounds__(512, 2) void prefill_tile_kernel(const DecodeArgs a) {
    using C = Tile<D, KV8>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;                         // MFMA column: query row within a block
    const int grp = lane >> 4;                         // lane group: keys 4 grp .. 4 grp + 3
    const int slot = static_cast<int>(blockIdx.x) / a.num_kv_heads;
    const int g = static_cast<int>(blockIdx.x) - slot * a.num_kv_heads;

    // ---- the slot: block b, its rows and keys ----
    const int used = __builtin_amdgcn_readfirstlane(a.num_work[0]);
    if (slot >= used) return;
    const int4 wk = a.work_info[slot];
    const int b = __builtin_amdgcn_readfirstlane(wk.x);
    if (b < 0 || b >= a.num_seqs) return;
    const int S = __builtin_amdgcn_readfirstlane(max(a.context_lens[b], 0));
    const int row0 = __builtin_amdgcn_readfirstlane(a.cu[b]);
    int L = __builtin_amdgcn_readfirstlane(a.cu[b + 1]) - row0;
    L = min(max(L, 0), a.max_q_len);
    if (row0 < 0 || row0 >= a.num_rows) L = 0;
    else L = min(L, a.num_rows - row0);
    const int bt_b = a.bt_index ? __builtin_amdgcn_readfirstlane(a.bt_index[b]) : b;
    const long long reach = static_cast<long long>(a.max_blocks) * a.block_size;
    const long long lo64 = static_cast<long long>(max(__builtin_amdgcn_readfirstlane(wk.y), 0)) * a.tile_tokens;
    long long hi64 = static_cast<long long>(max(__builtin_amdgcn_readfirstlane(wk.z), 0)) * a.tile_tokens;
    hi64 = min(min(hi64, static_cast<long long>(S)), reach);
    const int k_lo = static_cast<int>(min(lo64, hi64));
    const int k_hi = static_cast<int>(hi64 > lo64 ? hi64 : lo64);
    const int nchunks = k_hi > k_lo ? (k_hi - k_lo + C::KC - 1) / C::KC : 0;
    const int G = a.group;
    const int M = G * L;                               // valid query rows (<= ROWS)

    // page ids of chunk k's two 16-key halves (0 past the block table's reach: such halves load nothing)
    const int* bt_row = a.block_tables + static_cast<size_t>(bt_b) * a.max_blocks;
    const __amdgpu_buffer_rsrc_t bt_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int*>(bt_row), 0, a.max_blocks * 4, kRawWord3);
    const int page_shift = __builtin_ctz(a.block_size);
    auto page_load = [&](int k, int half) -> int {
        const long long key = static_cast<long long>(k_lo) + C::KC * static_cast<long long>(k) + 16 * half;
        const unsigned off = key < k_hi ? static_cast<unsigned>(key >> page_shift) * 4u : 0xfffffff0u;
        return __builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, off, 0, 0);
    };

    // ---- query operands (B of S^T): qop[rb][s] = q[row][32 s + 8 grp .. + 8] as bf16 ----
    bf16x8_t qop[C::RB][C::KS];
    int nvis[C::RB], nlo[C::RB];                       // this lane's row sees keys [nlo, nvis)
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
        const int n = 16 * (C::RB * wave + rb) + col;
        const bool valid = n < M;
        const int i = valid ? n / G : 0;
        const int h = g * G + (valid ? n - i * G : 0);
        nvis[rb] = valid ? S - (L - 1 - i) : 0;
        nlo[rb] = a.window > 0 ? max(nvis[rb] - a.window, 0) : 0;
        const size_t qoff = (static_cast<size_t>(row0 + i) * a.num_q_heads + h) * D;
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            const int d0 = 32 * s + 8 * grp;
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
            qop[rb][s] = __builtin_bit_cast(bf16x8_t, v);
        }
    }
    // the fewest keys any row sees and the latest window start: chunks inside need no mask
    const int nvis_min = S - (L - 1);
    const int nlo_max = a.window > 0 ? max(S - a.window, 0) : 0;
    // row blocks of this wave holding rows of the block (wave-uniform)
    const int live_rb = min(max((M - 16 * C::RB * wave + 15) / 16, 0), C::RB);

    float m_run[C::RB], l_run[C::RB];
    float4_t acc[C::RB][C::DT];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
#pragma unroll
        for (int t = 0; t < C::DT; ++t) acc[rb][t] = float4_t{0.f, 0.f, 0.f, 0.f};
    }

    // ---- chunk loads: register set st holds one chunk's K and V pieces; every iteration issues the
    // same loads (a chunk past the slot, or a half on an invalid page, goes through a resource with no
    // records and loads zeros), so the waits are exact ----
    const size_t head_stride = static_cast<size_t>(a.block_size) * C::GRB;   // bytes per (page, kv head)
    u32x4_t kreg[2][C::NL], vreg[2][C::NL];
    int nv_of[2];
    auto issue = [&](int st, int k, int page0, int page1) {
        const int key0 = k_lo + C::KC * k;
        const int nv = k < nchunks ? min(C::KC, k_hi - key0) : 0;
        nv_of[st] = nv;
        __amdgpu_buffer_rsrc_t rk[2], rv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int blk = __builtin_amdgcn_readfirstlane(h ? page1 : page0);
            const bool ok = nv > 16 * h && blk >= 0 && blk < a.num_blocks;
            const int off = (key0 + 16 * h) & (a.block_size - 1);
            const size_t base = ok ? (static_cast<size_t>(blk) * a.num_kv_heads + g) * head_stride +
                                         static_cast<size_t>(off) * C::GRB
                                   : 0;
            const int records = ok ? 16 * C::GRB : 0;
            rk[h] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.k_cache + base), 0, records, kRawWord3);
            rv[h] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.v_cache + base), 0, records, kRawWord3);
        }
#pragma unroll
        for (int it = 0; it < C::NL; ++it) {
            const int f = it * C::NT + tid;
            const int r = f / C::PPR;
            const int c = f - r * C::PPR;
            // a wave's pieces of one load lie in one half of the chunk (wave-uniform)
            const int h = __builtin_amdgcn_readfirstlane(min(r, C::KC - 1) >> 4);
            const unsigned o = f < C::PIECES ? static_cast<unsigned>((r - 16 * h) * C::GRB + 16 * c) : 0xfffffff0u;
            kreg[st][it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(h ? rk[1] : rk[0], o, 0, kNonTemporal));
            vreg[st][it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(h ? rv[1] : rv[0], o, 0, kNonTemporal));
        }
    };
    // register set st -> LDS tiles of parity p (rows at or past nv as zeros)
    auto stage = [&](int st, int p) {
        uint8_t* const kt = lds + p * C::TILE;
        uint8_t* const vt = lds + (C::NBUF + p) * C::TILE;
        const int nv = nv_of[st];
#pragma unroll
        for (int it = 0; it < C::NL; ++it) {
            const int f = it * C::NT + tid;
            if (C::PIECES % C::NT != 0 && f >= C::PIECES) continue;
            const int r = f / C::PPR;
            const int c = f - r * C::PPR;
            const u32x4_t z = {0u, 0u, 0u, 0u};
            const u32x4_t kv = r < nv ? kreg[st][it] : z;
            const u32x4_t vv = r < nv ? vreg[st][it] : z;
            if constexpr (!KV8) {
                *reinterpret_cast<u32x4_t*>(kt + tile_col<C::LRB>(r, c, kxor<C::SWM>(r))) = kv;
                *reinterpret_cast<u32x4_t*>(vt + tile_col<C::LRB>(r, c, vxor<C::SWM>(r))) = vv;
            } else {
                u32x4_t klo, khi, vlo, vhi;
                widen_fp8(kv, klo, khi);
                widen_fp8(vv, vlo, vhi);
                const int kx = kxor<C::SWM>(r), vx = vxor<C::SWM>(r);
                *reinterpret_cast<u32x4_t*>(kt + tile_col<C::LRB>(r, 2 * c, kx)) = klo;
                *reinterpret_cast<u32x4_t*>(kt + tile_col<C::LRB>(r, 2 * c + 1, kx)) = khi;
                *reinterpret_cast<u32x4_t*>(vt + tile_col<C::LRB>(r, 2 * c, vx)) = vlo;
                *reinterpret_cast<u32x4_t*>(vt + tile_col<C::LRB>(r, 2 * c + 1, vx)) = vhi;
            }
        }
    };

    // ---- the products on the chunk in LDS tiles of parity p (keys key0 .. key0 + nv - 1) ----
    const int tr_row = 4 * grp + ((lane >> 2) & 3);
    const int tr_d0 = 4 * (lane & 3);
    auto compute = [&](int p, int key0, int nv) {
        const uint8_t* const kt = lds + p * C::TILE;
        const uint8_t* const vt = lds + (C::NBUF + p) * C::TILE;
        if (live_rb == 0) return;
        // S^T for the two 16-key halves: lane holds keys 16 kb + 4 grp + j of row block rb's row col
        // (2 RB independent accumulation chains; blocks past the rows compute on zero queries).  The K
        // operands are read KP steps ahead of their products, so LDS latency overlaps the matrix cores.
        constexpr int KP = C::KS < 4 ? C::KS : 4;
        bf16x8_t kop[C::KS][2];
        auto kread = [&](int s) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                kop[s][kb] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t*>(kt + tile_col<C::LRB>(16 * kb + col, 4 * s + grp, kxor<C::SWM>(16 * kb + col))));
        };
#pragma unroll
        for (int s = 0; s < KP; ++s) kread(s);
        float4_t sc[2][C::RB];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb) sc[kb][rb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    sc[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[s][kb], qop[rb][s], sc[kb][rb], 0, 0, 0);
            if (s + KP < C::KS) kread(s + KP);
        }
        // V^T operands (A of O^T += V^T . P^T over the 32 keys): contraction index 8 grp + j is key
        // 4 grp + j of the first half for j < 4 and key 16 + 4 grp + j - 4 of the second for j >= 4, as
        // P's registers lie.  The first VP tiles are read before the softmax, which then hides them.
        constexpr int VP = C::DT < 4 ? C::DT : 4;
        bf16x8_t vop[C::DT];
        auto vread = [&](int t) {
            const int d0 = 16 * t + tr_d0;
            const int o0 = tile_col<C::LRB>(tr_row, d0 >> 3, vxor<C::SWM>(tr_row)) + ((d0 & 7) << 1);
            const int o1 = tile_col<C::LRB>(16 + tr_row, d0 >> 3, vxor<C::SWM>(16 + tr_row)) + ((d0 & 7) << 1);
            const bf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(vt + o0));
            const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(vt + o1));
            const u32x2_t a0 = __builtin_bit_cast(u32x2_t, v0);
            const u32x2_t a1 = __builtin_bit_cast(u32x2_t, v1);
            const u32x4_t vc = {a0[0], a0[1], a1[0], a1[1]};
            vop[t] = __builtin_bit_cast(bf16x8_t, vc);
        };
#pragma unroll
        for (int t = 0; t < VP; ++t) vread(t);
        // a chunk inside every row's visible range takes no mask (uniform); otherwise the scores past a
        // row's range become -inf in place, so both cases share one softmax
        if (!(nv == C::KC && key0 + C::KC <= nvis_min && key0 >= nlo_max)) {
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb) {
                const int lim = min(nv, nvis[rb] - key0);
                const int low = nlo[rb] - key0;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int q = 16 * (j >> 2) + 4 * grp + (j & 3);
                    if (!(q < lim && q >= low)) sc[j >> 2][rb][j & 3] = -INFINITY;
                }
            }
        }
        bf16x8_t pop[C::RB];
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = sc[j >> 2][rb][j & 3] * a.score_scale_log2;
            float mt = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
            mt = row_max4(mt);
            const bool grow = mt > m_run[rb] + kSlack;
            if (__builtin_amdgcn_ballot_w64(grow)) {
                const float mnew = grow ? mt : m_run[rb];
                const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - mnew);
                l_run[rb] *= alpha;
#pragma unroll
                for (int t = 0; t < C::DT; ++t) acc[rb][t] *= alpha;
                m_run[rb] = mnew;
            }
            const float mref = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
            float pr[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                pr[j] = __builtin_amdgcn_exp2f(x[j] - mref);
                l_run[rb] += pr[j];
            }
            const u32x4_t pc = {pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                                pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
            pop[rb] = __builtin_bit_cast(bf16x8_t, pc);
        }
#pragma unroll
        for (int t = 0; t < C::DT; ++t) {
#pragma unroll
            for (int rb = 0; rb < C::RB; ++rb)
                acc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[t], pop[rb], acc[rb][t], 0, 0, 0);
            if (t + VP < C::DT) vread(t + VP);
        }
    };

    if constexpr (C::DMA) {
        // ---- direct loads: chunk k goes to LDS buffer k % NBUF.  The first NW / 2 waves load the first
        // 16 keys of every chunk and the others the last 16, so a wave finds one page and builds one pair
        // of resources per chunk.  Lane l of a load instruction writes the 16 bytes at its base + 16 l, so
        // the lane fetches the piece whose swizzled place is there (the same layout stage() writes); rows
        // past the slot's last key, or on an invalid page, are past the resource's byte count and land as
        // zeros.  Page ids come through scalar loads, so the vector-memory counter counts only the chunk
        // loads: NLD per chunk. ----
        constexpr int HW = C::NW / 2;                  // waves per half-chunk
        constexpr int WPOS = 16 * C::LCPR / HW;        // a wave's 16-byte places in a half of a tile
        constexpr int ITS = WPOS / 64;                 // its loads per tile and chunk
        static_assert(WPOS % 64 == 0 && 2 * ITS == C::NLD, "whole loads per wave");
        const int half = wave / HW;                    // wave-uniform
        const int p0w = 16 * C::LCPR * half + WPOS * (wave - HW * half);   // the wave's first place
        int ko[ITS], vo[ITS];                          // per lane: its pieces' offsets in the half's rows
#pragma unroll
        for (int it = 0; it < ITS; ++it) {
            const int pos = p0w + 64 * it + lane;
            const int r = pos / C::LCPR;
            const int c = pos - r * C::LCPR;           // the place; the piece that belongs there:
            ko[it] = (r - 16 * half) * C::GRB + 16 * (c ^ kxor<C::SWM>(r));
            vo[it] = (r - 16 * half) * C::GRB + 16 * (c ^ vxor<C::SWM>(r));
        }
        const uint8_t* const kg = a.k_cache + static_cast<size_t>(g) * head_stride;
        const uint8_t* const vg = a.v_cache + static_cast<size_t>(g) * head_stride;
        const size_t page_stride = static_cast<size_t>(a.num_kv_heads) * head_stride;
        // the block table is read-only here: through the constant address space a wave-uniform index
        // is a scalar load
        cint4* const cbt = (cint4*)(bt_row);
        // the page of this wave's half of chunk k, -1 past the slot (loads nothing)
        auto spage = [&](int k) -> int {
            if (k >= nchunks) return -1;
            const int key = k_lo + C::KC * k + 16 * half;
            if (key >= k_hi) return -1;
            return cbt[key >> page_shift];
        };
        auto dma = [&](int k, int page) {
            const int key = k_lo + C::KC * k + 16 * half;
            const int nvh = k < nchunks ? min(max(k_hi - key, 0), 16) : 0;
            const bool ok = nvh > 0 && page >= 0 && page < a.num_blocks;
            const size_t off = ok ? static_cast<size_t>(page) * page_stride +
                                        static_cast<size_t>(key & (a.block_size - 1)) * C::GRB
                                  : 0;
            const int records = ok ? nvh * C::GRB : 0;
            const u32x4_t rk = raw_rsrc(kg + off, records);
            const u32x4_t rv = raw_rsrc(vg + off, records);
            const uint8_t* const kt = lds + (k % C::NBUF) * C::TILE + 16 * p0w;
            const uint8_t* const vt = lds + (C::NBUF + k % C::NBUF) * C::TILE + 16 * p0w;
#pragma unroll
            for (int it = 0; it < ITS; ++it) {
                lds_load16(rk, (const lds_void*)(kt + 1024 * it), ko[it]);
                lds_load16(rv, (const lds_void*)(vt + 1024 * it), vo[it]);
            }
        };
        // The loop: iteration k waits for chunk k's loads (NBUF - 2 younger chunks may stay in flight)
        // and meets the barrier, so every wave's part of chunk k is in LDS and every wave is done with
        // chunk k - 1; it loads chunk k + NBUF - 1 into chunk k - 1's buffer, then computes chunk k.
        // The barrier carries no memory fence (that would wait for every load in flight); the compiler
        // fences keep LDS accesses on their side of it.
        // The query loads land first: the compiler does not see the direct loads, so once it knows the
        // query operands are in registers it adds no wait of its own for them inside the loop.
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
        asm volatile("" ::: "memory");
        for (int j = 0; j < C::NBUF - 1; ++j) dma(j, spage(j));
        int np = spage(C::NBUF - 1);
        constexpr int kWaitChunk = (C::NBUF - 2) * C::NLD;     // loads younger than chunk k's
        static_assert(kWaitChunk < 64, "vmcnt field");
        // unrolled NBUF times, so each buffer is a constant: the K reads then take their buffer in the
        // instructions' 16-bit offset field (K tiles in the first 64 KB); the V tiles lie past its
        // reach, so their reads keep an address per buffer
        for (int k0 = 0; k0 < nchunks; k0 += C::NBUF) {
#pragma unroll
            for (int par = 0; par < C::NBUF; ++par) {
                const int k = k0 + par;
                if (k >= nchunks) break;               // uniform: every wave leaves here together
                __builtin_amdgcn_s_waitcnt((kWaitChunk & 15) | (7 << 4) | (15 << 8) | ((kWaitChunk >> 4) << 14));
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                dma(k + C::NBUF - 1, np);
                const int key0 = k_lo + C::KC * k;
                compute(par, key0, min(C::KC, k_hi - key0));
                np = spage(k + C::NBUF);
            }
        }
        // the last loads (past the slot: zeros) land before the workgroup's LDS is released
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    } else {
        // ---- pipeline: LDS parity k & 1 holds chunk k; register set (k + 1) & 1 holds chunk k + 1 in
        // flight.  Iteration k loads the page ids of chunk k + 3, issues chunk k + 2 into the free register
        // set, computes chunk k, stages chunk k + 1 into the other parity (last read in iteration k - 1,
        // before that iteration's barrier) and meets the barrier.  Every wave runs the same trip count. ----
        int pg[2][2];                                      // page ids of chunks k + 2 and k + 3 (by parity)
        {
            const int p00 = page_load(0, 0), p01 = page_load(0, 1);
            const int p10 = page_load(1, 0), p11 = page_load(1, 1);
            pg[0][0] = page_load(2, 0);
            pg[0][1] = page_load(2, 1);
            issue(0, 0, p00, p01);
            issue(1, 1, p10, p11);
            pg[1][0] = page_load(3, 0);
            pg[1][1] = page_load(3, 1);
        }
        stage(0, 0);
        __syncthreads();
        for (int k0 = 0; k0 < nchunks; k0 += 2) {
    #pragma unroll
            for (int par = 0; par < 2; ++par) {
                const int k = k0 + par;
                if (par == 1 && k >= nchunks) break;       // uniform: every wave leaves here together
                const int q0 = pg[par][0], q1 = pg[par][1];
                pg[par][0] = page_load(k + 4, 0);
                pg[par][1] = page_load(k + 4, 1);
                const int nv = nv_of[par];
                issue(par, k + 2, q0, q1);
                compute(par, k_lo + C::KC * k, nv);
                stage(par ^ 1, par ^ 1);
                __syncthreads();
            }
        }
    }

    // ---- states: rows n < M of this wave, token i = n / G, head g G + n % G ----
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
        if (rb >= live_rb) break;
        const float l = row_sum4(l_run[rb]);
        const int n = 16 * (C::RB * wave + rb) + col;
        if (n >= M) continue;
        const int i = n / G;
        const int h = g * G + (n - i * G);
        const size_t st = (static_cast<size_t>(slot) * a.max_q_len + i) * a.num_q_heads + h;
#pragma unroll
        for (int t = 0; t < C::DT; ++t)
            *reinterpret_cast<float4_t*>(a.ws_acc + st * D + 16 * t + 4 * grp) = acc[rb][t] * a.v_scale;
        if (grp == 0) *reinterpret_cast<float2*>(a.ws_ml + st * 2) = make_float2(m_run[rb], l);
    }
}

template <int D, bool KV8>
hipError_t launch_tiles_d(const DecodeArgs& a, bool q_f32, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.capacity) * static_cast<unsigned>(a.num_kv_heads));
    const dim3 block(Tile<D, KV8>::NT);
    if (q_f32) hipLaunchKernelGGL((prefill_tile_kernel<D, KV8, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((prefill_tile_kernel<D, KV8, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace

static_assert(Tile<64, false>::ROWS == Tile<128, false>::ROWS && Tile<64, true>::ROWS == Tile<128, true>::ROWS &&
                  Tile<256, true>::ROWS == Tile<256, false>::ROWS,
              "one block size per head_dim, whatever the cache dtype");
int prefill_tile_rows(int head_dim) { return head_dim == 256 ? Tile<256, false>::ROWS : Tile<128, false>::ROWS; }

hipError_t launch_prefill_tiles(const DecodeArgs& a, int head_dim, pa_dtype kv_dtype, bool q_f32, hipStream_t stream) {
    if (a.capacity == 0 || a.num_kv_heads == 0) return hipSuccess;
    const bool kv8 = kv_dtype == PA_FP8_E4M3;
    switch (head_dim) {
        case 64: return kv8 ? launch_tiles_d<64, true>(a, q_f32, stream) : launch_tiles_d<64, false>(a, q_f32, stream);
        case 128: return kv8 ? launch_tiles_d<128, true>(a, q_f32, stream) : launch_tiles_d<128, false>(a, q_f32, stream);
        default: return kv8 ? launch_tiles_d<256, true>(a, q_f32, stream) : launch_tiles_d<256, false>(a, q_f32, stream);
    }
}

}  // namespace pa

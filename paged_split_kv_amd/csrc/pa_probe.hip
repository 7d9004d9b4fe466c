// pa_probe.hip -- read-only bandwidth probes that give the benchmark its ceilings (libpa_probe.so,
// declared in include/pa_probe.h).  They are measurement kernels, not part of the decode path: they
// read memory and compute nothing of the method.
//
//  * pa_probe_read streams a contiguous buffer once: the practical HBM read rate of the device.
//  * pa_probe_gather reads exactly the K and V bytes that a decode launch over the same plan reads --
//    every key of every used plan slot, for every kv head, through the block table, in 16-key chunks
//    -- with the decode's launch shape (one 4-wave workgroup per (slot, kv head)) and its load form
//    (16-byte non-temporal buffer loads, page ids fetched ahead), and nothing else: the ceiling of a
//    decode whose arithmetic, staging and epilogue were free.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"
#include "pa_probe.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer resource (32-bit data format, no swizzle): loads past the resource's byte
// count return zero without touching memory.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kLoadNonTemporal = 2;

__device__ __forceinline__ uint32_t fold(u32x4_t v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// Contiguous read: workgroup w streams bytes [w * span, min((w + 1) * span, bytes)); each wave step
// reads 1 KiB (64 lanes x 16 bytes) and PF steps are in flight per wave.
template <int PF>
__global__ __launch_bounds__(256) void probe_read_kernel(const uint8_t* src, size_t bytes, size_t span,
                                                         uint32_t* sink) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t begin = static_cast<size_t>(blockIdx.x) * span;
    const size_t end = begin + span < bytes ? begin + span : bytes;
    const long long steps = begin < end ? static_cast<long long>((end - begin + 1023) / 1024) : 0;
    // wave w takes 1 KiB steps w, w + 4, ...
    const long long mine = steps > wave ? (steps - wave + 3) / 4 : 0;
    u32x4_t reg[PF];
    auto issue = [&](int st, long long k) {
        const size_t off = begin + static_cast<size_t>(wave + 4 * k) * 1024;
        const bool live = k < mine;
        const size_t left = live ? end - off : 0;
        const int records = static_cast<int>(left < 1024 ? left : 1024);
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(src + (live ? off : 0)), 0, records, kRawBufferWord3);
        reg[st] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 0, kLoadNonTemporal));
    };
    uint32_t acc = 0;
#pragma unroll
    for (int st = 0; st < PF; ++st) issue(st, st);
    const long long rounds = (mine + PF - 1) / PF;
    for (long long k0 = 0; k0 < rounds * PF; k0 += PF) {
#pragma unroll
        for (int st = 0; st < PF; ++st) {
            acc ^= fold(reg[st]);
            issue(st, k0 + st + PF);
        }
    }
    acc ^= __shfl_xor(acc, 32, 64);
    if (lane == 0) sink[blockIdx.x * 4 + wave] = acc;
}

struct GatherArgs {
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int4* work_info;
    uint32_t* sink;
    int num_blocks, num_kv_heads, block_size, max_blocks, num_seqs, tile_tokens, row_bytes;
};

// Gather: workgroup (slot, kv head g) reads the keys [tile_begin * T, min(tile_end * T, S_b)) of its
// plan slot; the slot's 16-key chunks are split evenly over the 4 waves (consecutive runs), each chunk
// is 16 rows of row_bytes of K and of V (only the rows below S_b are read), NL 1-KiB loads each.
template <int NL, int PF>
__global__ __launch_bounds__(256) void probe_gather_kernel(const GatherArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slot = blockIdx.x / a.num_kv_heads;
    const int g = blockIdx.x - slot * a.num_kv_heads;
    // an unused slot's entry names no request (the plan's sentinel), in slot order and in the decode's
    // dispatch order alike, where unused slots do not sit at the end
    const int4 w = a.work_info[slot];
    const int b = __builtin_amdgcn_readfirstlane(w.x);
    if (b < 0 || b >= a.num_seqs) return;
    const int S = __builtin_amdgcn_readfirstlane(max(a.context_lens[b], 0));
    const long long reach = static_cast<long long>(a.max_blocks) * a.block_size;
    long long lo = static_cast<long long>(max(w.y, 0)) * a.tile_tokens;
    long long hi = static_cast<long long>(max(w.z, 0)) * a.tile_tokens;
    hi = hi < S ? hi : S;
    hi = hi < reach ? hi : reach;
    lo = lo < hi ? lo : hi;
    const int k_lo = static_cast<int>(lo), k_hi = static_cast<int>(hi);
    const int nchunks = (k_hi - k_lo + 15) >> 4;
    const int unit = (nchunks + 3) >> 2;
    const int c0 = wave * unit;
    const int mine = max(min(nchunks - c0, unit), 0);
    const int page_shift = __builtin_ctz(a.block_size);
    const int* bt_row = a.block_tables + static_cast<size_t>(b) * a.max_blocks;
    const __amdgpu_buffer_rsrc_t bt_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int*>(bt_row), 0, a.max_blocks * 4, kRawBufferWord3);
    auto page_load = [&](int k) -> int {
        const unsigned off = k < mine ? static_cast<unsigned>((k_lo + 16 * (c0 + k)) >> page_shift) * 4u : 0xfffffff0u;
        return __builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, off, 0, 0);
    };
    const size_t head_stride = static_cast<size_t>(a.block_size) * a.row_bytes;
    u32x4_t kreg[PF][NL], vreg[PF][NL];
    auto issue = [&](int st, int k, int page) {
        const int key0 = k_lo + 16 * (c0 + k);
        const int blk = __builtin_amdgcn_readfirstlane(page);
        const bool live = k < mine && blk >= 0 && blk < a.num_blocks;
        const int nv = live ? min(16, k_hi - key0) : 0;
        const size_t base = nv > 0 ? (static_cast<size_t>(blk) * a.num_kv_heads + g) * head_stride +
                                         static_cast<size_t>(key0 & (a.block_size - 1)) * a.row_bytes
                                   : 0;
        const int records = nv > 0 ? nv * a.row_bytes : 0;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.k_cache + base), 0, records, kRawBufferWord3);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.v_cache + base), 0, records, kRawBufferWord3);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            kreg[st][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, (i * 64 + lane) * 16, 0, kLoadNonTemporal));
            vreg[st][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, (i * 64 + lane) * 16, 0, kLoadNonTemporal));
        }
    };
    int pnext[PF];
#pragma unroll
    for (int st = 0; st < PF; ++st) issue(st, st, page_load(st));
#pragma unroll
    for (int st = 0; st < PF; ++st) pnext[st] = page_load(st + PF);
    uint32_t acc = 0;
    const int rounds = (mine + PF - 1) / PF;
    for (int k0 = 0; k0 < rounds * PF; k0 += PF) {
#pragma unroll
        for (int st = 0; st < PF; ++st) {
#pragma unroll
            for (int i = 0; i < NL; ++i) acc ^= fold(kreg[st][i]) ^ fold(vreg[st][i]);
            const int page = pnext[st];
            pnext[st] = page_load(k0 + st + 2 * PF);
            issue(st, k0 + st + PF, page);
        }
    }
    acc ^= __shfl_xor(acc, 32, 64);
    if (lane == 0) a.sink[blockIdx.x * 4 + wave] = acc;
}

template <int NL, int PF>
hipError_t launch_gather(const GatherArgs& a, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((probe_gather_kernel<NL, PF>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

extern "C" {

pa_status pa_probe_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink, void* stream) {
    if (!src || !sink || workgroups < 1) return PA_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3)) return PA_INVALID_ARG;
    if (bytes == 0) return PA_OK;
    const size_t span = ((bytes + workgroups - 1) / workgroups + 1023) & ~static_cast<size_t>(1023);
    const unsigned grid = static_cast<unsigned>((bytes + span - 1) / span);
    hipLaunchKernelGGL((probe_read_kernel<8>), dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<const uint8_t*>(src), bytes, span, sink);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_HIP_ERROR;
}

pa_status pa_probe_gather(const void* k_cache, const void* v_cache, pa_dtype kv_dtype, int32_t num_blocks,
                          int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                          const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t num_seqs, const int32_t* work_info, const int32_t* num_work, int32_t capacity,
                          int32_t tile_tokens, uint32_t* sink, void* stream) {
    if (!k_cache || !v_cache || !block_tables || !context_lens || !work_info || !num_work || !sink)
        return PA_INVALID_ARG;
    if (num_blocks < 1 || num_kv_heads < 1 || num_seqs < 0 || capacity < 0 || max_blocks_per_seq < 1 ||
        tile_tokens < 1)
        return PA_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(k_cache) & 15) || (reinterpret_cast<uintptr_t>(v_cache) & 15) ||
        (reinterpret_cast<uintptr_t>(work_info) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3))
        return PA_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PA_UNSUPPORTED;
    if (block_size != 16 && block_size != 64 && block_size != 128) return PA_UNSUPPORTED;
    if (tile_tokens % block_size) return PA_UNSUPPORTED;
    const int elem = kv_dtype == PA_F32 ? 4 : (kv_dtype == PA_BF16 ? 2 : (kv_dtype == PA_FP8_E4M3 ? 1 : 0));
    if (!elem) return PA_INVALID_ARG;
    const unsigned grid = static_cast<unsigned>(capacity) * static_cast<unsigned>(num_kv_heads);
    if (grid == 0) return PA_OK;
    GatherArgs a;
    a.k_cache = static_cast<const uint8_t*>(k_cache);
    a.v_cache = static_cast<const uint8_t*>(v_cache);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.work_info = reinterpret_cast<const int4*>(work_info);
    a.sink = sink;
    a.num_blocks = num_blocks;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.tile_tokens = tile_tokens;
    a.row_bytes = head_dim * elem;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    switch (16 * a.row_bytes / 1024) {          // 1-KiB loads per lane per 16-key chunk
        case 1: e = launch_gather<1, 8>(a, grid, s); break;
        case 2: e = launch_gather<2, 4>(a, grid, s); break;
        case 4: e = launch_gather<4, 2>(a, grid, s); break;
        case 8: e = launch_gather<8, 2>(a, grid, s); break;
        default: e = launch_gather<16, 1>(a, grid, s); break;
    }
    return e == hipSuccess ? PA_OK : PA_HIP_ERROR;
}

}  // extern "C"

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

// Two floats -> packed bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
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

// Workspace layout (see pa_workspace_bytes): acc region then (m, l) region, each 256-byte aligned.
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct WorkspaceView {
    float* acc;   // [capacity, max_q_len, num_q_heads, head_dim]
    float* ml;    // [capacity, max_q_len, num_q_heads, 2]   (running max in base-2 units, sum)
};

__host__ __device__ inline size_t workspace_acc_bytes(int capacity, int max_q_len, int hq, int d) {
    return align256(static_cast<size_t>(capacity) * max_q_len * hq * d * sizeof(float));
}

__host__ __device__ inline size_t workspace_ml_bytes(int capacity, int max_q_len, int hq) {
    return align256(static_cast<size_t>(capacity) * max_q_len * hq * 2 * sizeof(float));
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
    const int32_t* num_work;
    float* ws_acc;
    float* ws_ml;
    int num_rows, num_q_heads, num_kv_heads, group;   // group = Hq / Hkv
    int num_blocks, block_size, max_blocks, num_seqs;
    int max_q_len, capacity, tile_tokens;
    float score_scale_log2;     // scale * k_scale * log2(e)
    float v_scale;
};

struct MergeArgs {
    const int32_t* cu;          // nullable
    const int2* reduce_info;
    const float* ws_acc;
    const float* ws_ml;
    void* out;
    int num_rows, num_q_heads, num_seqs, max_q_len, capacity;
};

hipError_t launch_plan(const int32_t* context_lens, int num_seqs, int cap_formula, int capacity,
                       int max_partitions, int tile_tokens, int32_t* work_info, int32_t* reduce_info,
                       int32_t* num_work, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int head_dim, pa_dtype kv_dtype, bool q_f32,
                         hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int head_dim, bool out_bf16, hipStream_t stream);

}  // namespace pa

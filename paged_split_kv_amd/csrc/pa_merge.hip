// pa_merge.hip -- log-sum-exp merge of a request's split-KV states into the output rows (gfx950).
//
// For output row r and query head h (opengfx1030/vllm-rdna PR #29, Change item 1: each block finds
// its request by binary search over cu_query_lens; tokens past cu[-1] and zero-length requests come
// out as zeros):
//   b = last request with cu[b] <= r, token i = r - cu[b];
//   over the request's partials j with l_j > 0:  M = max m_j,
//   out = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j       (m is kept in base-2 units)
// Every element of out is written.
#include "pa_device.h"

namespace pa {


namespace {

// (m, l, acc) <- the log-sum-exp merge of two states (m in base-2 units; an empty state has m = -inf
// and l = 0 and contributes nothing; two empty states stay empty).
__device__ __forceinline__ void fold_state(float& m, float& l, float4& acc, float m2, float l2, const float4& a2) {
    const float mn = fmaxf(m, m2);
    const bool none = mn == -INFINITY;
    const float f1 = none ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    const float f2 = none ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
    l = l * f1 + l2 * f2;
    acc.x = acc.x * f1 + a2.x * f2;
    acc.y = acc.y * f1 + a2.y * f2;
    acc.z = acc.z * f1 + a2.z * f2;
    acc.w = acc.w * f1 + a2.w * f2;
    m = mn;
}

// One workgroup of NT threads per (row, head) and column part: the head dimension is split into CS
// parts of D / CS columns, each its own workgroup (every part reads all partials' (m, l) and its own
// columns of acc; the parts write disjoint columns).  Thread t owns the 16-byte column dc = t % NDC of
// its part and the partials j = pg, pg + NPG, ... with pg = t / NDC; it folds them into a running
// (max, sum, acc) with independent loads, then the NPG states of a column are combined in a fixed
// tree (lanes of a wave, then the waves through LDS).
// CS = 4 when there are fewer (row, head) pairs than compute units: a request split into hundreds of
// partials is then read by four workgroups on four compute units.
template <int D, bool OUT_BF16, int NT, int CS>
__global__ __launch_bounds__(NT) void merge_kernel(const MergeArgs a) {
    constexpr int NDC = D / 4 / CS;     // float4 columns of this part
    constexpr int NPG = NT / NDC;       // partial groups
    constexpr int NW = NT / 64;         // waves
    static_assert(NDC <= 64 && 64 % NDC == 0, "a wave holds whole partial groups");
    __shared__ float4 s_acc[NW][NDC];
    __shared__ float s_m[NW][NDC];
    __shared__ float s_l[NW][NDC];

    const int tid = threadIdx.x;
    const int pair = blockIdx.x / CS;
    const int part = blockIdx.x - pair * CS;
    const int dc = tid % NDC + part * NDC;       // float4 column within the head dimension
    const int pg = tid / NDC;
    const int r = pair / a.num_q_heads;
    const int h = pair - r * a.num_q_heads;
    if (a.row_floor && r < *a.row_floor) return;     // the whole workgroup: before any barrier

    int i;
    const int b = owner_of_row(a.cu, a.num_seqs, a.max_q_len, r, i);
    float m = -INFINITY, l = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (b >= 0) {
        const int2 ri = a.reduce_info[b];
        const int first = max(ri.x, 0);
        const int parts = max(min(ri.y, a.capacity - first), 0);
        const size_t step = static_cast<size_t>(a.max_q_len) * a.num_q_heads;       // states per slot
        const size_t st0 = (static_cast<size_t>(first) * a.max_q_len + i) * a.num_q_heads + h;
        // U partials in flight per thread: every load is issued before any is used (indices past
        // the last partial repeat it and are dropped), so a thread waits for memory once per batch
        // rather than twice per partial; empty partials (l = 0) are dropped by selects, not branches
        constexpr int U = NPG >= 32 ? 8 : 4;
        for (int j0 = pg; j0 < parts; j0 += U * NPG) {
            float2 ml[U];
            float4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const size_t st = st0 + static_cast<size_t>(min(j0 + u * NPG, parts - 1)) * step;
                ml[u] = *reinterpret_cast<const float2*>(a.ws_ml + st * 2);
                v[u] = *reinterpret_cast<const float4*>(a.ws_acc + st * D + 4 * dc);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool use = j0 + u * NPG < parts && ml[u].y > 0.f;
                const float mn = fmaxf(m, ml[u].x);
                const float fo = __builtin_amdgcn_exp2f(m - mn);      // 0 while m = -inf
                const float fn = __builtin_amdgcn_exp2f(ml[u].x - mn);
                l = use ? l * fo + ml[u].y * fn : l;
                acc.x = use ? acc.x * fo + v[u].x * fn : acc.x;
                acc.y = use ? acc.y * fo + v[u].y * fn : acc.y;
                acc.z = use ? acc.z * fo + v[u].z * fn : acc.z;
                acc.w = use ? acc.w * fo + v[u].w * fn : acc.w;
                m = use ? mn : m;
            }
        }
    }
    // Fold the NPG group states of each column in a fixed tree: group pg sits in lanes of wave
    // pg / (64 / NDC), so the first steps pair lanes NDC, 2 NDC, ... apart inside the wave, then one
    // thread per column folds the waves' states through LDS.
#pragma unroll
    for (int d = NDC; d < 64; d <<= 1) {
        const float m2 = __shfl_xor(m, d, 64);
        const float l2 = __shfl_xor(l, d, 64);
        float4 a2;
        a2.x = __shfl_xor(acc.x, d, 64);
        a2.y = __shfl_xor(acc.y, d, 64);
        a2.z = __shfl_xor(acc.z, d, 64);
        a2.w = __shfl_xor(acc.w, d, 64);
        fold_state(m, l, acc, m2, l2, a2);
    }
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (lane < NDC) {
        s_acc[wave][lane] = acc;
        s_m[wave][lane] = m;
        s_l[wave][lane] = l;
    }
    __syncthreads();
    if (tid >= NDC) return;
    m = s_m[0][tid];
    l = s_l[0][tid];
    acc = s_acc[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) fold_state(m, l, acc, s_m[w][tid], s_l[w][tid], s_acc[w][tid]);
    const float den = l;
    const float4 num = acc;
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const float4 o = den > 0.f ? make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
    const size_t base = (static_cast<size_t>(r) * a.num_q_heads + h) * D + 4 * dc;
    if constexpr (OUT_BF16) {
        uint2 w;
        w.x = pack_bf16x2(o.x, o.y);
        w.y = pack_bf16x2(o.z, o.w);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + base) = w;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + base) = o;
    }
}

// Compute units of the current device (the launch shapes below are chosen against it).
int device_cu_count() {
    int dev = 0, cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu < 1)
        return 256;
    return cu;
}

template <int D>
hipError_t launch_merge_d(const MergeArgs& a, bool out_bf16, dim3 grid, hipStream_t stream) {
    const unsigned cu = static_cast<unsigned>(device_cu_count());
    // fewer (row, head) pairs than compute units: each pair's columns split over four workgroups
    if (grid.x < cu) {
        const dim3 g4(grid.x * 4);
        if (out_bf16) hipLaunchKernelGGL((merge_kernel<D, true, 256, 4>), g4, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((merge_kernel<D, false, 256, 4>), g4, dim3(256), 0, stream, a);
    } else if (grid.x >= 8 * cu) {
        // many pairs (large batches, typically with few partials each): one wave per pair, so the
        // launch fits the compute units in one round instead of queueing 256-thread workgroups
        // (eight 256-thread workgroups per compute unit would be two rounds at 32 resident waves)
        if (out_bf16) hipLaunchKernelGGL((merge_kernel<D, true, 64, 1>), grid, dim3(64), 0, stream, a);
        else hipLaunchKernelGGL((merge_kernel<D, false, 64, 1>), grid, dim3(64), 0, stream, a);
    } else {
        if (out_bf16) hipLaunchKernelGGL((merge_kernel<D, true, 256, 1>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((merge_kernel<D, false, 256, 1>), grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int head_dim, bool out_bf16, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(static_cast<long long>(a.num_rows) * a.num_q_heads));
    if (grid.x == 0) return hipSuccess;
    switch (head_dim) {
        case 64: return launch_merge_d<64>(a, out_bf16, grid, stream);
        case 128: return launch_merge_d<128>(a, out_bf16, grid, stream);
        default: return launch_merge_d<256>(a, out_bf16, grid, stream);
    }
}

}  // namespace pa

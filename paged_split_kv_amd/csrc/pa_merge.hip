// pa_merge.hip -- log-sum-exp merge of a request's split-KV states into the output rows (gfx950).
//
// For output row r and query head h (opengfx1030/vllm-rdna PR #29, Change item 1: each block finds
// its request by binary search over cu_query_lens; tokens past cu[-1] and zero-length requests come
// out as zeros):
//   b = last request with cu[b] <= r, token i = r - cu[b];
//   over the request's partials j with l_j > 0:  M = max m_j,
//   out = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j       (m is kept in base-2 units)
// One wave per (row, head): lanes split the head dimension for the weighted sum and the partial list
// for the max.  Every element of out is written.
#include "pa_device.h"

namespace pa {


namespace {

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int r = wid / a.num_q_heads;
    const int h = wid - r * a.num_q_heads;
    if (r >= a.num_rows) return;

    int b = -1, i = 0;
    if (a.cu) {
        if (a.num_seqs > 0 && r >= a.cu[0] && r < a.cu[a.num_seqs]) {
            int lo = 0, hi = a.num_seqs - 1;          // last b with cu[b] <= r
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (a.cu[mid] <= r) lo = mid;
                else hi = mid - 1;
            }
            b = lo;
            i = r - a.cu[b];
            if (i >= a.cu[b + 1] - a.cu[b]) b = -1;
        }
    } else if (r < a.num_seqs) {
        b = r;
    }
    if (i >= a.max_q_len) b = -1;

    float num[E];
#pragma unroll
    for (int e = 0; e < E; ++e) num[e] = 0.f;
    float den = 0.f;

    if (b >= 0) {
        const int2 ri = a.reduce_info[b];
        const int first = max(ri.x, 0);
        const int parts = max(min(ri.y, a.capacity - first), 0);
        const size_t step = static_cast<size_t>(a.max_q_len) * a.num_q_heads;       // states per slot
        const size_t st0 = (static_cast<size_t>(first) * a.max_q_len + i) * a.num_q_heads + h;
        float Mx = -INFINITY;
        for (int j = lane; j < parts; j += 64) {
            const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + (st0 + j * step) * 2);
            if (ml.y > 0.f) Mx = fmaxf(Mx, ml.x);
        }
        Mx = wave_max(Mx);
        if (Mx != -INFINITY) {
            for (int j = 0; j < parts; ++j) {
                const size_t st = st0 + j * step;
                const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + st * 2);
                if (!(ml.y > 0.f)) continue;
                const float f = __builtin_amdgcn_exp2f(ml.x - Mx);
                den = fmaf(f, ml.y, den);
                const float* src = a.ws_acc + st * D;
#pragma unroll
                for (int e = 0; e < E; ++e) num[e] = fmaf(f, src[lane + 64 * e], num[e]);
            }
        }
    }

    const size_t o = (static_cast<size_t>(r) * a.num_q_heads + h) * D;
    const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float v = den > 0.f ? num[e] * inv : 0.f;
        if constexpr (OUT_BF16) static_cast<uint16_t*>(a.out)[o + lane + 64 * e] = f32_to_bf16(v);
        else static_cast<float*>(a.out)[o + lane + 64 * e] = v;
    }
}

template <int D>
hipError_t launch_merge_d(const MergeArgs& a, bool out_bf16, dim3 grid, hipStream_t stream) {
    if (out_bf16) hipLaunchKernelGGL((merge_kernel<D, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((merge_kernel<D, false>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int head_dim, bool out_bf16, hipStream_t stream) {
    const long long waves = static_cast<long long>(a.num_rows) * a.num_q_heads;
    const dim3 grid(static_cast<unsigned>((waves + 3) / 4));
    if (grid.x == 0) return hipSuccess;
    switch (head_dim) {
        case 64: return launch_merge_d<64>(a, out_bf16, grid, stream);
        case 128: return launch_merge_d<128>(a, out_bf16, grid, stream);
        default: return launch_merge_d<256>(a, out_bf16, grid, stream);
    }
}

}  // namespace pa

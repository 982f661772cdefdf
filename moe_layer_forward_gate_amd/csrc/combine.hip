// Gather: y[t] = sum over the token's slots j of the weighted expert outputs.
//
// [hotelren §2.1 step 6] and [hotelren §2.3] combine_kernel: the k expert
// outputs are summed with their gating weights; [pptc §2.1] the k outputs share
// slices of one buffer and are accumulated into the result. The weights were
// applied in the down-projection epilogue, which wrote slot (t, j), K split s to row
// (t*kt + j)*S + s; this pass adds the first nrow rows of each token's stride rows in
// a fixed order (slot 0 first), so the result does not depend on scheduling, and
// rounds once to the output dtype. (With the shared slices merged into one sum only
// the first k+1 slots of a token are written.) Each thread handles 4 consecutive
// columns (d % 4 == 0).
#include "common.h"

namespace moe {
namespace {

// the partial rows are read once: non-temporal loads keep them out of the caches
__device__ __forceinline__ float4 load_once(const float4* p) {
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(t[0], t[1], t[2], t[3]);
}

// U rows are loaded at once (rows past kt are not loaded and not added), then added in
// order, so every batch is one round trip to memory.
template <bool BF16, int U>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ow, int T, int kt, int stride,
                                                      int d, void* __restrict__ y) {
    const int d4 = d / 4;
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)T * d4) return;
    const int t = (int)(i / d4), c4 = (int)(i - (size_t)t * d4);
    const float4* src = reinterpret_cast<const float4*>(ow + (size_t)t * stride * d) + c4;
    // rows are added in order 0, 1, 2, ...
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < kt; j += U) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (j + u < kt) v[u] = load_once(&src[(size_t)(j + u) * d4]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (j + u < kt) {
                s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
            }
        }
    }
    if (BF16) {
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(s.x) | ((uint32_t)f32_to_bf16(s.y) << 16);
        o.y = (uint32_t)f32_to_bf16(s.z) | ((uint32_t)f32_to_bf16(s.w) << 16);
        reinterpret_cast<uint2*>(y)[i] = o;
    } else {
        reinterpret_cast<float4*>(y)[i] = s;
    }
}

}  // namespace

hipError_t launch_combine(const float* ow, int T, int nrow, int stride, int d, void* y, bool y_bf16,
                          hipStream_t s) {
    if (nrow > stride) return hipErrorInvalidValue;
    const size_t n = (size_t)T * (d / 4);
    // decode batches (under 2^18 threads): every row of a thread in one batch of up to 32
    // loads, on 64-thread workgroups so the few thousand threads spread over many CUs;
    // larger batches: 256-thread workgroups, 8 rows a batch (enough threads hide the latency)
    if (n < (1u << 18)) {
        dim3 grid((unsigned)((n + 63) / 64));
        if (y_bf16)
            hipLaunchKernelGGL((combine_kernel<true, 32>), grid, dim3(64), 0, s, ow, T, nrow, stride, d, y);
        else
            hipLaunchKernelGGL((combine_kernel<false, 32>), grid, dim3(64), 0, s, ow, T, nrow, stride, d, y);
    } else {
        dim3 grid((unsigned)((n + 255) / 256));
        if (y_bf16)
            hipLaunchKernelGGL((combine_kernel<true, 8>), grid, dim3(256), 0, s, ow, T, nrow, stride, d, y);
        else
            hipLaunchKernelGGL((combine_kernel<false, 8>), grid, dim3(256), 0, s, ow, T, nrow, stride, d, y);
    }
    return hipGetLastError();
}

}  // namespace moe

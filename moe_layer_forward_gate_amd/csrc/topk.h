// Wavefront routines of the Gate kernels: the (logit desc, id asc) top-k with its
// weights, and wave-wide sums.
#pragma once
#include "common.h"

namespace moe {
namespace {

// Order key: larger key = larger logit, then lower expert id. -0.0 is folded to
// +0.0 so the two compare equal, as they do as floats.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, off, kWave);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, kWave);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Wave sums of N = 2^M values at once (a transposed butterfly: at each of the first M
// steps a lane keeps half of its values and adds its partner's copy of them, then the
// last 6-M steps fold single values): N - 1 + 6 - M shuffles instead of 6 N. Lane l
// returns the sum of value l >> (6 - M).
template <int N>
__device__ __forceinline__ float wave_sum_many(float (&v)[N]) {
    constexpr int M = N == 1 ? 0 : N == 2 ? 1 : N == 4 ? 2 : N == 8 ? 3 : N == 16 ? 4 : 5;
    static_assert((1 << M) == N && N <= 32, "power of two up to 32");
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int s = 0; s < M; ++s) {
        const int off = 32 >> s;
        const bool upper = lane & off;
#pragma unroll
        for (int i = 0; i < (N >> (s + 1)); ++i) {
            const int h = N >> (s + 1);
            const float send = upper ? v[i] : v[i + h];
            const float keep = upper ? v[i + h] : v[i];
            v[i] = keep + __shfl_xor(send, off, kWave);
        }
    }
    float r = v[0];
#pragma unroll
    for (int off = 32 >> M; off > 0; off >>= 1) r += __shfl_xor(r, off, kWave);
    return r;
}

// One wave: top-k of logits[0..E) (bias already added), weights, shared gate.
// `logits` may live in LDS; E <= 128, k <= 64. With kGateClamp the routed logits are
// first clamped to [-50, 50] ([0539edu §5.2]: the gate's clip option bounds the logits
// before the softmax), so the top-k and the weights both see the clamped values. With
// kGateRaw the weights are the chosen logits themselves ([hotelren §3.2]: the top-k is
// taken on the raw logits with no softmax; [hotelren §2.3]: the combine weights each
// expert by that gating score).
__device__ void wave_topk_write(const float* logits, int E, int k, int gflags, int t, int32_t* idx,
                                float* w, float* gs, int32_t* ids_copy = nullptr) {
    const bool has_shared = (gflags & kGateShared) != 0;
    const bool clamp = (gflags & kGateClamp) != 0;
    const bool raw = (gflags & kGateRaw) != 0;
    auto logit = [&](int e) {
        const float v = logits[e];
        return clamp ? fminf(fmaxf(v, -kGateClampAbs), kGateClampAbs) : v;
    };
    const int lane = threadIdx.x % kWave;
    uint64_t k0 = lane < E ? topk_key(logit(lane), lane) : 0ull;
    uint64_t k1 = lane + kWave < E ? topk_key(logit(lane + kWave), lane + kWave) : 0ull;
    int my_e = -1;     // lane j < k keeps slot j's expert
    for (int j = 0; j < k; ++j) {
        uint64_t m = wave_max_u64(k0 > k1 ? k0 : k1);
        int e = (int)(0xFFFFFFFFu - (uint32_t)m);
        if (k0 == m) k0 = 0ull;
        if (k1 == m) k1 = 0ull;
        if (lane == j) my_e = e;
    }
    // softmax over the chosen logits, relative to slot 0 (the maximum)
    float l0 = __shfl(my_e >= 0 ? logit(my_e) : 0.0f, 0, kWave);
    float ex = lane < k ? expf(logit(my_e) - l0) : 0.0f;
    float sum = wave_sum(ex);
    if (lane < k) {
        idx[(size_t)t * k + lane] = my_e;
        w[(size_t)t * k + lane] = raw ? logit(my_e) : ex / sum;
        if (ids_copy) ids_copy[t * k + lane] = my_e;
    }
    if (has_shared && lane == 0) {
        float z = logits[E];
        gs[t] = 1.0f / (1.0f + expf(-z));
    }
}

}  // namespace
}  // namespace moe

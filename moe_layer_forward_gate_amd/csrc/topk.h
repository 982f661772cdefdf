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

// One DPP move of a 64-bit value (both halves with the same lane pattern).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

// Wave-wide maximum, the same in every lane. Inside each row of 16 lanes four DPP steps
// pair every lane with one of each other group (quad swaps at distance 1 and 2, then the
// mirror inside each half row and inside the row), so every lane ends with its row's
// maximum; the four row maxima are then read into scalar registers and compared there.
// All 64 lanes must be active. (DPP moves stay in the vector unit; a shuffle goes
// through the LDS crossbar and waits on it at each of its steps.)
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    uint64_t o;
    o = dpp_u64<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v = o > v ? o : v;
    o = dpp_u64<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v = o > v ? o : v;
    o = dpp_u64<0x141>(v);  // row_half_mirror
    v = o > v ? o : v;
    o = dpp_u64<0x140>(v);  // row_mirror
    v = o > v ? o : v;
    uint64_t m = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r);
        const uint64_t x = ((uint64_t)hi << 32) | lo;
        m = x > m ? x : m;
    }
    return m;
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

// One wave, all 64 lanes active (the maximum and the sums read other lanes through
// DPP and readlanes): top-k of logits[0..E) (bias already added), weights, shared gate.
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
    // softmax over the chosen logits, relative to slot 0 (the maximum); the k terms are
    // added in slot order
    const float mine = my_e >= 0 ? logit(my_e) : 0.0f;
    const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), 0));
    const float ex = lane < k ? expf(mine - l0) : 0.0f;
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
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

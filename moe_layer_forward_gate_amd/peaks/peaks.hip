// Microbenchmarks of the two rates the MoE kernels are held against on this GPU: a
// streaming HBM read (each wave reads its own contiguous region 16 bytes per lane,
// several loads in flight) and bf16 MFMA issue (v_mfma_f32_16x16x32_bf16 on a 4 x 8 grid
// of independent accumulators per wave, operands in registers, no memory traffic), once
// with constant operands and once with random operands that change every MFMA: the
// multipliers' switching activity sets the power draw, and with it the clock the chip
// holds, so only the second rate is reachable by a GEMM on real data.
// Built into libmoe_peaks.so, separate from libmoe; used by bench.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kU = 16;  // loads in flight per lane

template <bool NT>  // NT: non-temporal loads (the data is read once)
__global__ __launch_bounds__(256) void read_stream(const u32x4* __restrict__ p, size_t chunks_per_wave,
                                                   uint32_t* __restrict__ out) {
    const int lane = threadIdx.x % 64;
    const size_t wave = (size_t)blockIdx.x * 4 + threadIdx.x / 64;
    const u32x4* q = p + wave * chunks_per_wave * 64 + lane;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t c = 0; c < chunks_per_wave; c += kU) {
        u32x4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) v[u] = NT ? __builtin_nontemporal_load(&q[(c + u) * 64]) : q[(c + u) * 64];
#pragma unroll
        for (int u = 0; u < kU; ++u) acc ^= v[u];
    }
    out[wave * 64 + lane] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ __launch_bounds__(512) void mfma_issue(int iters, float* __restrict__ out) {
    bf16x8 a[4], b[8];
    for (int j = 0; j < 4; ++j)
        for (int i = 0; i < 8; ++i) a[j][i] = (__bf16)(threadIdx.x * 0.001f + i + j);
    for (int j = 0; j < 8; ++j)
        for (int i = 0; i < 8; ++i) b[j][i] = (__bf16)(i * 0.5f - j);
    f32x4 acc[4][8];
    for (int m = 0; m < 4; ++m)
        for (int n = 0; n < 8; ++n) acc[m][n] = f32x4{(float)m, (float)n, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = 0; n < 8; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b[n], acc[m][n], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    float s = 0.f;
    for (int m = 0; m < 4; ++m)
        for (int n = 0; n < 8; ++n) s += acc[m][n][0] + acc[m][n][3];
    out[blockIdx.x * 512 + threadIdx.x] = s;
}

// 32-bit integer mix (the finaliser of the MurmurHash3 family) for operand bits
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

// bf16 values +-[1, 2) with random mantissas: sign bit 15, exponent of 1.0, mantissa bits 0-6
__device__ __forceinline__ bf16x8 random_bf16x8(uint32_t seed) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t h = mix32(seed * 4u + (uint32_t)i);
        w[i] = (0x3F803F80u | (h & 0x007F007Fu)) | (h & 0x80008000u);
    }
    return __builtin_bit_cast(bf16x8, w);
}

// The same MFMA grid as mfma_issue, with two sets of random operands used in turn, so
// consecutive MFMAs of a wave never see the same inputs.
__global__ __launch_bounds__(512) void mfma_issue_random(int iters, float* __restrict__ out) {
    const uint32_t t = blockIdx.x * 512u + threadIdx.x;
    bf16x8 a[2][4], b[2][8];
    for (int s = 0; s < 2; ++s) {
        for (int j = 0; j < 4; ++j) a[s][j] = random_bf16x8(t * 64u + s * 32u + j);
        for (int j = 0; j < 8; ++j) b[s][j] = random_bf16x8(t * 64u + s * 32u + 8u + j);
    }
    f32x4 acc[4][8];
    for (int m = 0; m < 4; ++m)
        for (int n = 0; n < 8; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int n = 0; n < 8; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s][m], b[s ^ (n & 1)][n], acc[m][n], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    float sum = 0.f;
    for (int m = 0; m < 4; ++m)
        for (int n = 0; n < 8; ++n) sum += acc[m][n][0] + acc[m][n][3];
    out[blockIdx.x * 512 + threadIdx.x] = sum;
}

float time_ms(hipEvent_t a, hipEvent_t b) {
    float ms = 0.f;
    hipEventElapsedTime(&ms, a, b);
    return ms;
}

}  // namespace

namespace {
template <bool NT>
double read_gbps(size_t bytes, int waves, int reps) {
    if (waves <= 0 || waves % 4 || reps <= 0) return -1.0;
    const size_t cpw = bytes / 1024 / (size_t)waves / kU * kU;
    if (cpw == 0) return -1.0;
    u32x4* d = nullptr;
    uint32_t* o = nullptr;
    if (hipMalloc(&d, cpw * 1024 * waves) != hipSuccess) return -2.0;
    if (hipMalloc(&o, (size_t)waves * 64 * 4) != hipSuccess) { hipFree(d); return -2.0; }
    double r = -3.0;
    hipEvent_t a, b;
    if (hipMemset(d, 1, cpw * 1024 * waves) == hipSuccess && hipEventCreate(&a) == hipSuccess &&
        hipEventCreate(&b) == hipSuccess) {
        hipLaunchKernelGGL(read_stream<NT>, dim3(waves / 4), dim3(256), 0, 0, d, cpw, o);
        hipEventRecord(a, 0);
        for (int i = 0; i < reps; ++i)
            hipLaunchKernelGGL(read_stream<NT>, dim3(waves / 4), dim3(256), 0, 0, d, cpw, o);
        hipEventRecord(b, 0);
        if (hipEventSynchronize(b) == hipSuccess)
            r = (double)cpw * 1024 * waves * reps / (time_ms(a, b) * 1e-3) / 1e9;
        hipEventDestroy(a);
        hipEventDestroy(b);
    }
    hipFree(o);
    hipFree(d);
    return r;
}
}  // namespace

extern "C" {

// Streaming read rate in GB/s over `bytes` (rounded down to whole 16-KB rounds per wave)
// read by `waves` waves; returns a negative value on a HIP error.
__attribute__((visibility("default"))) double moe_peak_read_gbps(size_t bytes, int waves, int reps) {
    return read_gbps<false>(bytes, waves, reps);
}
// The same with non-temporal loads.
__attribute__((visibility("default"))) double moe_peak_read_nt_gbps(size_t bytes, int waves, int reps) {
    return read_gbps<true>(bytes, waves, reps);
}

// bf16 MFMA rate in TFLOP/s with `wgs` workgroups of 8 waves; negative on a HIP error.
__attribute__((visibility("default"))) double moe_peak_mfma_tflops(int wgs, int iters) {
    if (wgs <= 0 || iters <= 0) return -1.0;
    float* o = nullptr;
    if (hipMalloc(&o, (size_t)wgs * 512 * 4) != hipSuccess) return -2.0;
    double r = -3.0;
    hipEvent_t a, b;
    if (hipEventCreate(&a) == hipSuccess && hipEventCreate(&b) == hipSuccess) {
        hipLaunchKernelGGL(mfma_issue, dim3(wgs), dim3(512), 0, 0, 10, o);
        hipEventRecord(a, 0);
        hipLaunchKernelGGL(mfma_issue, dim3(wgs), dim3(512), 0, 0, iters, o);
        hipEventRecord(b, 0);
        if (hipEventSynchronize(b) == hipSuccess)
            r = (double)wgs * 8 * iters * 32 * 16384.0 / (time_ms(a, b) * 1e-3) / 1e12;
        hipEventDestroy(a);
        hipEventDestroy(b);
    }
    hipFree(o);
    return r;
}

// The same with random operands that change every MFMA (64 MFMAs per wave per iteration).
__attribute__((visibility("default"))) double moe_peak_mfma_random_tflops(int wgs, int iters) {
    if (wgs <= 0 || iters <= 0) return -1.0;
    float* o = nullptr;
    if (hipMalloc(&o, (size_t)wgs * 512 * 4) != hipSuccess) return -2.0;
    double r = -3.0;
    hipEvent_t a, b;
    if (hipEventCreate(&a) == hipSuccess && hipEventCreate(&b) == hipSuccess) {
        hipLaunchKernelGGL(mfma_issue_random, dim3(wgs), dim3(512), 0, 0, 10, o);
        hipEventRecord(a, 0);
        hipLaunchKernelGGL(mfma_issue_random, dim3(wgs), dim3(512), 0, 0, iters, o);
        hipEventRecord(b, 0);
        if (hipEventSynchronize(b) == hipSuccess)
            r = (double)wgs * 8 * iters * 64 * 16384.0 / (time_ms(a, b) * 1e-3) / 1e12;
        hipEventDestroy(a);
        hipEventDestroy(b);
    }
    hipFree(o);
    return r;
}

}  // extern "C"

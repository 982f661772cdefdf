// Scatter kernel: one workgroup of 16 waves runs scatter_block (scatter.h); and the
// physical scatter of token rows into the tiled up-projection operand.
#include "scatter.h"

namespace moe {
namespace {

constexpr int kScatterWaves = 16;

__global__ __launch_bounds__(1024) void scatter_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                      int V, int bm, ScatterOut o) {
    __shared__ ScatterSmem<kScatterWaves> sm;
    scatter_block<kScatterWaves>(idx, T, E, k, V, bm, o, sm);
}

// Token rows into the tiled up operand ([0539edu §2.2] Scatter: the tokens of one
// expert become one contiguous batch). Padded row q lies in tile g = q / bm of the
// expert e with tile_start[e] <= g < tile_start[e+1]; its local row q - tile_start[e]*bm
// is sorted row offsets[e] + local, i.e. token sorted_c[...] / kt, or zeros past the
// expert's last row. Rows of shared virtual experts past the first are not written
// (identical to the first's). Layout [R/16][d/32][64 lanes][8 bf16]: block (q/16, ks), lane l
// holds row 16*(q/16) + l%16, K 32*ks + 8*(l/16) .. +7 -- an MFMA A fragment -- so the
// GEMM stages each 1 KB block with one contiguous LDS-DMA instead of 16 row pieces.
// One wave per (16-row block, 128-wide K chunk): four 16-byte loads and stores per lane.
__global__ __launch_bounds__(256) void pack_a_kernel(GemmArgs a) {
    const int lane = threadIdx.x % kWave;
    const int u = blockIdx.x * 4 + threadIdx.x / kWave;
    const int KC = a.d / 128;
    if (u >= a.tile_start[a.Et] * (a.bm / 16) * KC) return;
    const int mb = u / KC, kc = u - (u / KC) * KC;
    const int g = mb / (a.bm / 16);
    int c = 0;
    for (int j0 = 0; j0 <= a.Et; j0 += kWave) {
        const int j = j0 + lane;
        c += __popcll(__ballot(j <= a.Et && a.tile_start[j] <= g));
    }
    const int e = c - 1;
    // shared virtual experts E0, E0+1, .. all hold every token in order: only E0's rows
    // are written, and the GEMM reads them for the others
    if (e > a.Et - a.kt + a.k) return;
    const int local = mb * 16 + lane % 16 - a.tile_start[e] * a.bm;
    const bool valid = local < a.offsets[e + 1] - a.offsets[e];
    u32x4 v[4];
    if (valid) {
        const bf16_t* src = a.x + (size_t)(a.sorted_c[a.offsets[e] + local] / a.kt) * a.d + kc * 128 + 8 * (lane / 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const u32x4*>(src + 32 * i);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = u32x4{0u, 0u, 0u, 0u};
    }
    u32x4* dst = reinterpret_cast<u32x4*>(a.xp) + ((size_t)mb * (a.d / 32) + kc * 4) * 64 + lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i * 64] = v[i];
}

}  // namespace

hipError_t launch_pack_a(const GemmArgs& a, hipStream_t s) {
    if (a.d % 128 || a.bm % 16) return hipErrorInvalidValue;
    const size_t waves = (size_t)a.max_tiles * (a.bm / 16) * (a.d / 128);
    hipLaunchKernelGGL(pack_a_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* idx, int T, int E, int k, int V, int bm, const ScatterOut& o,
                          hipStream_t s) {
    if (E > kMaxExperts || E + V > kMaxEt) return hipErrorInvalidValue;
    hipLaunchKernelGGL(scatter_kernel, dim3(1), dim3(kScatterWaves * kWave), 0, s, idx, T, E, k, V, bm, o);
    return hipGetLastError();
}

}  // namespace moe

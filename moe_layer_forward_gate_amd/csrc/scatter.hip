// Scatter kernel: one workgroup of 16 waves runs scatter_block (scatter.h).
#include "scatter.h"

namespace moe {
namespace {

constexpr int kScatterWaves = 16;

__global__ __launch_bounds__(1024) void scatter_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                      int V, int bm, ScatterOut o) {
    __shared__ ScatterSmem<kScatterWaves> sm;
    scatter_block<kScatterWaves>(idx, T, E, k, V, bm, o, sm);
}

}  // namespace

hipError_t launch_scatter(const int32_t* idx, int T, int E, int k, int V, int bm, const ScatterOut& o,
                          hipStream_t s) {
    if (E > kMaxExperts || E + V > kMaxEt) return hipErrorInvalidValue;
    hipLaunchKernelGGL(scatter_kernel, dim3(1), dim3(kScatterWaves * kWave), 0, s, idx, T, E, k, V, bm, o);
    return hipGetLastError();
}

}  // namespace moe

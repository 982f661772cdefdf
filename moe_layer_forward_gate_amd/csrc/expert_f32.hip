// Expert compute in fp32 (VALU FMA), for fp32 layers.
//
// Same grouped structure and epilogues as the MFMA path ([hotelren §2.1 steps
// 4-5], [hotelren §2.3] expert_gemm_kernel / combine weighting), on weights in
// their natural [E][K][N] layout. Workgroup tile 64 rows x 64 columns, K step 16,
// each thread a 4 x 4 block (the up kernel keeps gate and up accumulators for the
// same 4 x 4 block of H). fp32 layers are small; this path favours plainness.
#include "common.h"

namespace moe {
namespace {

constexpr int BM = kBMf32;  // 64
constexpr int BN = 64;
constexpr int BK = 16;
constexpr int GN = 8;

template <bool UP>
__global__ __launch_bounds__(256) void expert_gemm_f32(GemmF32Args a) {
    const int K = UP ? a.d : a.F;
    const int N = UP ? a.F : a.d;
    const int NT = N / BN;
    Tile tl;
    if (!decode_tile(a.tile_start, a.offsets, a.Et, NT, GN, BM, tl)) return;

    __shared__ float as[BK][BM + 4];
    __shared__ float bs[UP ? 2 : 1][BK][BN];

    const int tid = threadIdx.x;
    const int ty = tid / 16, tx = tid % 16;
    // A: thread loads a float4 of row tid/4 at K offset (tid%4)*4
    const int ar = tid / 4, akq = (tid % 4) * 4;
    const bool a_ok = ar < tl.rows;
    const float* a_row;
    {
        const int p = tl.seg0 + tl.row0 + (a_ok ? ar : 0);
        if (UP) a_row = a.x + (size_t)(a.sorted_c[p] / a.kt) * a.d;
        else a_row = a.h + (size_t)p * a.F;
    }
    // B: thread loads a float4 of K row tid/16 at column (tid%16)*4
    const int bk = tid / 16, bn4 = (tid % 16) * 4;
    const float* bg = (UP ? a.wg : a.wd) + (size_t)tl.e * K * N + (size_t)tl.n * BN + bn4;
    const float* bu = UP ? a.wu + (size_t)tl.e * K * N + (size_t)tl.n * BN + bn4 : nullptr;

    float accg[4][4], accu[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) accg[i][j] = accu[i][j] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += BK) {
        float4 av = a_ok ? *reinterpret_cast<const float4*>(a_row + k0 + akq) : make_float4(0.f, 0.f, 0.f, 0.f);
        as[akq + 0][ar] = av.x;
        as[akq + 1][ar] = av.y;
        as[akq + 2][ar] = av.z;
        as[akq + 3][ar] = av.w;
        *reinterpret_cast<float4*>(&bs[0][bk][bn4]) = *reinterpret_cast<const float4*>(bg + (size_t)(k0 + bk) * N);
        if (UP)
            *reinterpret_cast<float4*>(&bs[UP ? 1 : 0][bk][bn4]) =
                *reinterpret_cast<const float4*>(bu + (size_t)(k0 + bk) * N);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float4 x4 = *reinterpret_cast<const float4*>(&as[kk][ty * 4]);
            float4 g4 = *reinterpret_cast<const float4*>(&bs[0][kk][tx * 4]);
            const float xv[4] = {x4.x, x4.y, x4.z, x4.w};
            const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) accg[i][j] = fmaf(xv[i], gv[j], accg[i][j]);
            if (UP) {
                float4 u4 = *reinterpret_cast<const float4*>(&bs[UP ? 1 : 0][kk][tx * 4]);
                const float uv[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) accu[i][j] = fmaf(xv[i], uv[j], accu[i][j]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = ty * 4 + i;
        if (r >= tl.rows) continue;
        const int p = tl.seg0 + tl.row0 + r;
        if (UP) {
            float4 o;
            o.x = silu(accg[i][0]) * accu[i][0];
            o.y = silu(accg[i][1]) * accu[i][1];
            o.z = silu(accg[i][2]) * accu[i][2];
            o.w = silu(accg[i][3]) * accu[i][3];
            *reinterpret_cast<float4*>(a.h + (size_t)p * a.F + tl.n * BN + tx * 4) = o;
        } else {
            const int c = a.sorted_c[p];
            const int t = c / a.kt, j = c - t * a.kt;
            const float wgt = j < a.k ? a.topk_w[(size_t)t * a.k + j] : a.gs[t];
            float4 o = make_float4(accg[i][0] * wgt, accg[i][1] * wgt, accg[i][2] * wgt, accg[i][3] * wgt);
            *reinterpret_cast<float4*>(a.ow + (size_t)c * a.d + tl.n * BN + tx * 4) = o;
        }
    }
}

}  // namespace

hipError_t launch_expert_up_f32(const GemmF32Args& a, hipStream_t s) {
    const int NTp = (a.F / BN + GN - 1) / GN * GN;
    dim3 grid((unsigned)((a.max_tiles * NTp + kXcds - 1) / kXcds * kXcds));
    hipLaunchKernelGGL((expert_gemm_f32<true>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_expert_down_f32(const GemmF32Args& a, hipStream_t s) {
    const int NTp = (a.d / BN + GN - 1) / GN * GN;
    dim3 grid((unsigned)((a.max_tiles * NTp + kXcds - 1) / kXcds * kXcds));
    hipLaunchKernelGGL((expert_gemm_f32<false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe

// Expert compute on bf16 MFMA: grouped GEMMs over the by-expert row order.
//
// [hotelren §2.1 steps 4-5] each chosen expert's weights are loaded and its
// matrix products run; [0539edu §2.2] expert weights are stored expert-major and
// consecutively, and the kernel keeps weight slices in on-chip memory;
// [hotelren §2.3] expert_gemm_kernel is tailored to the expert weight layout;
// [mhpq §3.3] tensor-core fragments in 16x16 tiles on the original hardware.
//
// Up:   H[p, f] = silu(x[t(p)] . Wg[e][:, f]) * (x[t(p)] . Wu[e][:, f])
// Down: O[c(p), n] = wgt(c) * (H[p] . Wd[e][:, n]); wgt is the routing weight of
//       slot c (or the shared gate for a shared slice), so the top-k weighting of
//       the Gather stage is applied in this epilogue ([pptc §2.1] fused
//       aggregation).
//
// Workgroup tile 128 rows x 128 columns, K step 64, 4 waves in a 2 x 2 grid of
// 64 x 64, each wave 4 x 4 v_mfma_f32_16x16x32_bf16 accumulators. Both operands
// are staged in LDS in MFMA fragment order (one 1 KB block = 16 rows x 32 K, lane
// l holding row l%16, K 8*(l/16)..+7), so every fragment read is one conflict-free
// 16-byte-per-lane ds_read. Expert weights arrive from create-time packing already
// in that order (bf16: [Et][N/16][K/32][64][8]; int8: [E][N/16][K/64][64][16],
// bytes 0-7 the first 32-K half and 8-15 the second), so a weight tile is a
// straight 16-byte-per-lane copy; int8 is widened to bf16 on the way to LDS
// (exact: |q| <= 127 fits bf16's significand) and its per-column scale is
// applied to the fp32 accumulator in the epilogue. The next K step is loaded to
// registers while the current one is multiplied; one barrier per K step.
// Up-projection columns are packed gate/up interleaved per 16 columns, so each
// lane holds the gate and up accumulators of the same (row, f) and the SiLU*mul
// runs in registers.
#include "common.h"

namespace moe {
namespace {

constexpr int BM = kBM;    // 128
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int GN = 8;      // column tiles per group (see decode_tile)
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w, int sh) {
    // bytes sh/8 and sh/8+1 of w as two bf16 (exact widening of small integers)
    const float f0 = (float)(int)(int8_t)(w >> sh);
    const float f1 = (float)(int)(int8_t)(w >> (sh + 8));
    return (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
}

__device__ __forceinline__ u32x4 i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    u32x4 r;
    r.x = i8x2_to_bf16x2(lo, 0);
    r.y = i8x2_to_bf16x2(lo, 16);
    r.z = i8x2_to_bf16x2(hi, 0);
    r.w = i8x2_to_bf16x2(hi, 16);
    return r;
}

// Global -> registers for K step kt: 4 A chunks (16 B of one row each) and the
// weight tile's lane chunks.
template <bool INT8, int NBQ>
__device__ __forceinline__ void gload_tiles(u32x4 (&ra)[4], u32x4 (&rb)[NBQ], const bf16_t* const (&a_ptr)[4],
                                            const bool (&a_ok)[4], const u32x4* b_base, int kt, int K, int tid) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        ra[i] = a_ok[i] ? *reinterpret_cast<const u32x4*>(a_ptr[i] + k0) : u32x4{0u, 0u, 0u, 0u};
    if constexpr (INT8) {
        const int KB = K / 64;
#pragma unroll
        for (int i = 0; i < NBQ; ++i) {
            const int q = tid + kThreads * i;
            const int nb = q / 64, ln = q % 64;
            rb[i] = b_base[((size_t)nb * KB + kt) * 64 + ln];
        }
    } else {
        const int KS = K / 32;
#pragma unroll
        for (int i = 0; i < NBQ; ++i) {
            const int q = tid + kThreads * i;
            const int blk = q / 64, ln = q % 64;
            const int nb = blk / 2, ks = blk % 2;
            rb[i] = b_base[((size_t)nb * KS + kt * 2 + ks) * 64 + ln];
        }
    }
}

// Registers -> LDS (fragment order); int8 weights are widened to bf16 here.
template <bool INT8, int NBQ>
__device__ __forceinline__ void sstore_tiles(const u32x4 (&ra)[4], const u32x4 (&rb)[NBQ], const int (&a_lds)[4],
                                             u32x4* la, u32x4* lb, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) la[a_lds[i]] = ra[i];
    if constexpr (INT8) {
#pragma unroll
        for (int i = 0; i < NBQ; ++i) {
            const int q = tid + kThreads * i;
            const int nb = q / 64, ln = q % 64;
            lb[(nb * 2 + 0) * 64 + ln] = i8x8_to_bf16x8(rb[i].x, rb[i].y);
            lb[(nb * 2 + 1) * 64 + ln] = i8x8_to_bf16x8(rb[i].z, rb[i].w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < NBQ; ++i) lb[tid + kThreads * i] = rb[i];
    }
}

template <bool INT8, bool UP>
__global__ __launch_bounds__(kThreads, 2) void expert_gemm(GemmArgs a) {
    const int K = UP ? a.d : a.F;
    const int N = UP ? 2 * a.F : a.d;
    const int NT = N / BN;
    Tile tl;
    if (!decode_tile(a.tile_start, a.offsets, a.Et, NT, GN, BM, tl)) return;

    __shared__ u32x4 lds[2][2][(BM / 16) * (BK / 32) * 64];  // [buf][A|B][blocks*64 lanes]

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- A rows: thread loads rows tid/8 + 32*i, 16 B at K offset (tid%8)*8
    const int a_kc = tid % 8;
    const bf16_t* a_ptr[4];
    bool a_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = tid / 8 + 32 * i;
        a_ok[i] = r < tl.rows;
        const int p = tl.seg0 + tl.row0 + (a_ok[i] ? r : 0);
        if (UP) {
            const int c = a.sorted_c[p];
            a_ptr[i] = a.x + (size_t)(c / a.kt) * a.d + a_kc * 8;
        } else {
            a_ptr[i] = a.h + (size_t)p * a.F + a_kc * 8;
        }
    }
    // LDS slot of each A chunk: block (r/16, kc/4), lane (r%16) + 16*(kc%4)
    int a_lds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = tid / 8 + 32 * i;
        a_lds[i] = ((r / 16) * 2 + a_kc / 4) * 64 + (r % 16) + 16 * (a_kc % 4);
    }

    // ---- B tile
    const u32x4* b_base;
    if (INT8) {
        const int KB = K / 64;
        const int8_t* wb = (const int8_t*)(UP ? a.wgu : a.wdn) + (size_t)tl.e * N * K;
        b_base = reinterpret_cast<const u32x4*>(wb) + (size_t)(tl.n * 8) * KB * 64;
    } else {
        const int KS = K / 32;
        const bf16_t* wb = (const bf16_t*)(UP ? a.wgu : a.wdn) + (size_t)tl.e * N * K;
        b_base = reinterpret_cast<const u32x4*>(wb) + (size_t)(tl.n * 8) * KS * 64;
    }

    constexpr int NBQ = INT8 ? 2 : 4;
    u32x4 ra[4], rb[NBQ];
    const int KT = K / BK;
    gload_tiles<INT8, NBQ>(ra, rb, a_ptr, a_ok, b_base, 0, K, tid);
    sstore_tiles<INT8, NBQ>(ra, rb, a_lds, lds[0][0], lds[0][1], tid);
    __syncthreads();

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) gload_tiles<INT8, NBQ>(ra, rb, a_ptr, a_ok, b_base, kt + 1, K, tid);
        const u32x4* la = lds[buf][0];
        const u32x4* lb = lds[buf][1];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 af[4], bfg[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                af[mb] = __builtin_bit_cast(bf16x8, la[((wm * 4 + mb) * 2 + ks) * 64 + lane]);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                bfg[nb] = __builtin_bit_cast(bf16x8, lb[((wn * 4 + nb) * 2 + ks) * 64 + lane]);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], bfg[nb], acc[mb][nb], 0, 0, 0);
        }
        if (kt + 1 < KT) sstore_tiles<INT8, NBQ>(ra, rb, a_lds, lds[buf ^ 1][0], lds[buf ^ 1][1], tid);
        __syncthreads();
    }

    // ---- epilogue: lane holds column lane%16 of each 16x16 block, rows 4*(lane/16)+i
    const int col16 = lane % 16;
    const int rq = 4 * (lane / 16);
    if (UP) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int f = (tl.n * 4 + wn * 2 + q) * 16 + col16;
            float sg = 1.f, su = 1.f;
            if (INT8) {
                sg = a.s_gate[(size_t)tl.e * a.F + f];
                su = a.s_up[(size_t)tl.e * a.F + f];
            }
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = wm * 64 + mb * 16 + rq + i;
                    if (r < tl.rows) {
                        const float g = acc[mb][2 * q][i] * sg;
                        const float u = acc[mb][2 * q + 1][i] * su;
                        const size_t p = (size_t)tl.seg0 + tl.row0 + r;
                        a.h[p * a.F + f] = f32_to_bf16(silu(g) * u);
                    }
                }
        }
    } else {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 64 + mb * 16 + rq + i;
                if (r < tl.rows) {
                    const int c = a.sorted_c[tl.seg0 + tl.row0 + r];
                    const int t = c / a.kt, j = c - t * a.kt;
                    const float wgt = j < a.k ? a.topk_w[(size_t)t * a.k + j] : a.gs[t];
                    float* orow = a.ow + (size_t)c * a.d;
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) {
                        const int n = tl.n * BN + wn * 64 + nb * 16 + col16;
                        float v = acc[mb][nb][i] * wgt;
                        if (INT8) v *= a.s_down[(size_t)tl.e * a.d + n];
                        orow[n] = v;
                    }
                }
            }
    }
}

}  // namespace

hipError_t launch_expert_up_bf16(const GemmArgs& a, bool int8, hipStream_t s) {
    const int NT = 2 * a.F / BN;
    const int NTp = (NT + GN - 1) / GN * GN;
    // a multiple of 8 workgroups, so every XCD gets ceil(tiles / 8) slots
    dim3 grid((unsigned)((a.max_tiles * NTp + kXcds - 1) / kXcds * kXcds));
    if (int8)
        hipLaunchKernelGGL((expert_gemm<true, true>), grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((expert_gemm<false, true>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_expert_down_bf16(const GemmArgs& a, bool int8, hipStream_t s) {
    const int NT = a.d / BN;
    const int NTp = (NT + GN - 1) / GN * GN;
    dim3 grid((unsigned)((a.max_tiles * NTp + kXcds - 1) / kXcds * kXcds));
    if (int8)
        hipLaunchKernelGGL((expert_gemm<true, false>), grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((expert_gemm<false, false>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe

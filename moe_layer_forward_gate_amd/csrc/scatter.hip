// Scatter kernels: one workgroup of 16 waves runs scatter_block (scatter.h), or one
// wavefront runs scatter_wave for small batches; and the physical scatter of token rows
// into the tiled up-projection operand.
#include "scatter.h"

namespace moe {
namespace {

constexpr int kScatterWaves = 16;

__global__ __launch_bounds__(1024) void scatter_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                      int V, int bm, ScatterOut o) {
    __shared__ ScatterSmem<kScatterWaves> sm;
    scatter_block<kScatterWaves>(idx, T, E, k, V, bm, o, sm);
}

// Small batches: one wavefront does it all (no workgroup barriers).
__global__ __launch_bounds__(64) void scatter_wave_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                          int V, int bm, ScatterOut o) {
    __shared__ ScatterWaveSmem sm;
    scatter_wave(idx, T, E, k, V, bm, o, sm);
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
    // a separate down-projection tiling: its tile table, tile_start_h[e] = sum over e' < e of
    // ceil(n_e' / bm_h), by the first wave (a prefix sum 64 experts at a time)
    if (a.tile_start_h != a.tile_start && u == 0) {
        int carry = 0;
        if (lane == 0) a.tile_start_h[0] = 0;
        for (int j0 = 0; j0 < a.Et; j0 += kWave) {
            const int e = j0 + lane;
            int t = e < a.Et ? (a.offsets[e + 1] - a.offsets[e] + a.bm_h - 1) / a.bm_h : 0;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int y = __shfl_up(t, o, kWave);
                if (lane >= o) t += y;
            }
            if (e < a.Et) a.tile_start_h[e + 1] = carry + t;
            carry += __shfl(t, kWave - 1, kWave);
        }
    }
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

// ---- the scatter over many workgroups, for large batches: three launches
// count: chunk c (kChunk assignments, one per lane of 16 waves) -- per-wave ranks from
//   ballots over the expert-id bits, per-wave counts, their prefix over the chunk's
//   waves; writes cnt[c][e] and each assignment's rank inside its chunk;
// scan: one workgroup turns cnt[.][e] into each chunk's offset within expert e (in place,
//   chunk order), and builds counts, offsets and the tile table as scatter_block does;
// place: sorted position = offsets[e] + chunk offset + rank inside the chunk.
// The result is the same unique stable order.
constexpr int kChunk = 1024;

__global__ __launch_bounds__(1024) void scatter_count(const int32_t* __restrict__ idx, int N, int E,
                                                     int32_t* __restrict__ cnt, int32_t* __restrict__ lrank) {
    __shared__ int hist[16][kMaxExperts];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    for (int i = tid; i < 16 * E; i += 1024) hist[i / E][i % E] = 0;
    const int a = blockIdx.x * kChunk + tid;
    const bool valid = a < N;
    const int e = valid ? idx[a] : 0;
    __syncthreads();
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 7; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(valid && bit);
        same &= bit ? bb : ~bb;
    }
    const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (kWave - lane));
    const int rank = __popcll(same & lt_mask);
    if (valid && rank == 0) hist[wave][e] = __popcll(same);  // the group's lowest lane
    __syncthreads();
    if (tid < E) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const int h = hist[w][tid];
            hist[w][tid] = run;
            run += h;
        }
        cnt[(size_t)blockIdx.x * E + tid] = run;
    }
    __syncthreads();
    if (valid) lrank[a] = hist[wave][e] + rank;
}

__global__ __launch_bounds__(1024) void scatter_scan(int N, int T, int E, int V, int bm, int C,
                                                    int32_t* __restrict__ cnt, ScatterOut o) {
    __shared__ int ecnt[kMaxEt];
    __shared__ int offs[kMaxEt + 1];
    __shared__ int tiles[kMaxEt];
    __shared__ int tstart[kMaxEt + 1];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int Et = E + V;
    if (tid < E) {
        // chunk offsets within expert tid, in chunk order; loads go out 16 at a time
        int run = 0;
        for (int c0 = 0; c0 < C; c0 += 16) {
            int v[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) v[q] = c0 + q < C ? cnt[(size_t)(c0 + q) * E + tid] : 0;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                if (c0 + q < C) cnt[(size_t)(c0 + q) * E + tid] = run;
                run += v[q];
            }
        }
        ecnt[tid] = run;
    } else if (tid < Et) {
        ecnt[tid] = T;  // shared virtual experts hold every token
    }
    __syncthreads();
    if (wave == 0) wave_exclusive_scan(ecnt, Et, offs);
    if (wave == 1)
        for (int e = lane; e < Et; e += kWave) tiles[e] = (ecnt[e] + bm - 1) / bm;
    __syncthreads();
    if (wave == 1) wave_exclusive_scan(tiles, Et, tstart);
    __syncthreads();
    for (int e = tid; e <= Et; e += 1024) {
        if (e < Et) o.counts[e] = ecnt[e];
        o.offsets[e] = offs[e];
        o.tile_start[e] = tstart[e];
        if (e < E && o.user_counts) o.user_counts[e] = ecnt[e];
        if (e <= E && o.user_offsets) o.user_offsets[e] = offs[e];
    }
}

__global__ __launch_bounds__(256) void scatter_place(const int32_t* __restrict__ idx, int N, int T, int E, int k,
                                                     int V, const int32_t* __restrict__ cnt,
                                                     const int32_t* __restrict__ lrank, ScatterOut o) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int kt = k + V;
    if (i < N) {
        const int e = idx[i];
        const int pos = o.offsets[e] + cnt[(size_t)(i / kChunk) * E + e] + lrank[i];
        const int t = i / k, j = i - t * k;
        o.sorted_c[pos] = t * kt + j;
        if (o.user_sorted) o.user_sorted[pos] = i;
    } else if (i < N + V * T) {
        // shared virtual experts: every token, in order
        const int q = i - N, v = q / T, t = q - v * T;
        o.sorted_c[i] = t * kt + k + v;
    }
}

// A routing given by the caller ([pptc §3.4]: the engine consumes routing results made
// elsewhere, token-major [T][k]); an id outside [0, E) would index past the expert
// tables, so it is read as expert 0 at weight 0 and adds nothing to the output.
__global__ __launch_bounds__(256) void route_in_kernel(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                       int N, int E, int32_t* __restrict__ idx_out,
                                                       float* __restrict__ w_out) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < N) {
        const int e = idx[i];
        const bool ok = e >= 0 && e < E;
        idx_out[i] = ok ? e : 0;
        w_out[i] = ok ? w[i] : 0.0f;
    }
}

}  // namespace

hipError_t launch_route_in(const int32_t* idx, const float* w, int N, int E, int32_t* idx_out, float* w_out,
                           hipStream_t s) {
    if (N <= 0) return hipSuccess;
    hipLaunchKernelGGL(route_in_kernel, dim3((N + 255) / 256), dim3(256), 0, s, idx, w, N, E, idx_out, w_out);
    return hipGetLastError();
}

size_t scatter_wide_workspace(int N, int E) {
    const size_t C = ((size_t)N + kChunk - 1) / kChunk;
    return (C * E + (size_t)N) * sizeof(int32_t);
}

hipError_t launch_scatter_wide(const int32_t* idx, int T, int E, int k, int V, int bm, const ScatterOut& o,
                               int32_t* work, hipStream_t s) {
    if (E > kMaxExperts || E + V > kMaxEt) return hipErrorInvalidValue;
    const int N = T * k;
    const int C = (N + kChunk - 1) / kChunk;
    int32_t* cnt = work;
    int32_t* lrank = work + (size_t)C * E;
    hipLaunchKernelGGL(scatter_count, dim3(C), dim3(1024), 0, s, idx, N, E, cnt, lrank);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(scatter_scan, dim3(1), dim3(1024), 0, s, N, T, E, V, bm, C, cnt, o);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int tot = N + V * T;
    hipLaunchKernelGGL(scatter_place, dim3((tot + 255) / 256), dim3(256), 0, s, idx, N, T, E, k, V,
                       (const int32_t*)cnt, (const int32_t*)lrank, o);
    return hipGetLastError();
}

hipError_t launch_pack_a(const GemmArgs& a, hipStream_t s) {
    if (a.d % 128 || a.bm % 16) return hipErrorInvalidValue;
    const size_t waves = (size_t)a.max_tiles * (a.bm / 16) * (a.d / 128);
    hipLaunchKernelGGL(pack_a_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* idx, int T, int E, int k, int V, int bm, const ScatterOut& o,
                          hipStream_t s) {
    if (E > kMaxExperts || E + V > kMaxEt) return hipErrorInvalidValue;
    if (T * k <= kScatterWaveMaxN)
        hipLaunchKernelGGL(scatter_wave_kernel, dim3(1), dim3(kWave), 0, s, idx, T, E, k, V, bm, o);
    else
        hipLaunchKernelGGL(scatter_kernel, dim3(1), dim3(kScatterWaves * kWave), 0, s, idx, T, E, k, V, bm, o);
    return hipGetLastError();
}

}  // namespace moe

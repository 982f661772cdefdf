// Scatter as a workgroup-level routine (scatter_block) and as a one-wavefront routine for
// small batches (scatter_wave), shared by the standalone scatter kernel and the decode
// gate kernels that end with the scatter.
//
// [0539edu §2.2] Scatter stage; [hotelren §2.3] dispatch_kernel sends each token
// to its k experts' input buffers; [mhpq §2.1] tokens of one expert form one
// contiguous batch for a single GEMM; [pptc §3.3] expert_offsets is a prefix sum.
//
// Assignment a = t*k + j. Wave w owns the contiguous range of assignments
// [w*chunk, (w+1)*chunk):
//   1. per-wave expert histograms (LDS atomics; counts do not depend on order);
//   2. per-expert exclusive scan over waves, then over experts -> offsets;
//   3. each wave walks its range 64 assignments at a time; lanes holding the same
//      expert are found with 7 ballots over the expert-id bits, the rank of a lane
//      among them is a popcount of the lower lanes, and the group's lowest lane
//      advances the wave's running cursor for that expert.
// The result is the unique stable order (ascending a within each expert); no
// global atomics are used, so it is the same on every run.
//
// Shared virtual experts (the shared FFN split into V slices of d_ff columns)
// are appended as experts E..E+V-1, each holding every token in order.
#pragma once

#include "common.h"

namespace moe {

constexpr int kMaxEt = kMaxExperts + kMaxVirtual;  // <= 191: the scan covers 192 entries

template <int NWAVES>
struct ScatterSmem {
    int hist[NWAVES * kMaxExperts];  // per-wave counts, then cursors
    int cnt[kMaxEt];
    int offs[kMaxEt + 1];
    int tiles[kMaxEt];
    int tstart[kMaxEt + 1];
};

// exclusive scan of v[0..n) (n <= 191) by one wave; writes out[0..n], out[n] = total
__device__ inline void wave_exclusive_scan(const int* v, int n, int* out) {
    const int lane = threadIdx.x % kWave;
    int a[3];
    int s = 0;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        int e = lane * 3 + i;
        a[i] = e < n ? v[e] : 0;
        s += a[i];
    }
    int incl = s;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += o;
    }
    int run = incl - s;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        int e = lane * 3 + i;
        if (e <= n) out[e] = run;
        run += a[i];
    }
}

// The whole scatter, run by one workgroup of NWAVES waves (needs NWAVES >= 2).
template <int NWAVES>
__device__ void scatter_block(const int32_t* __restrict__ idx, int T, int E, int k, int V, int bm,
                              const ScatterOut& o, ScatterSmem<NWAVES>& sm) {
    const int nthr = NWAVES * kWave;
    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int N = T * k;
    const int kt = k + V;
    const int Et = E + V;
    const int chunk = (N + NWAVES - 1) / NWAVES;
    const int a0 = min(N, wave * chunk), a1 = min(N, a0 + chunk);

    for (int i = tid; i < NWAVES * E; i += nthr) sm.hist[i] = 0;
    __syncthreads();
    for (int a = a0 + lane; a < a1; a += kWave) atomicAdd(&sm.hist[wave * E + idx[a]], 1);
    __syncthreads();
    for (int e = tid; e < Et; e += nthr) {
        if (e < E) {
            int c = 0;
            for (int w = 0; w < NWAVES; ++w) {
                const int h = sm.hist[w * E + e];
                sm.hist[w * E + e] = c;  // assignments of this expert in earlier waves
                c += h;
            }
            sm.cnt[e] = c;
        } else {
            sm.cnt[e] = T;
        }
    }
    __syncthreads();
    if (wave == 0) wave_exclusive_scan(sm.cnt, Et, sm.offs);
    if (wave == 1) {
        for (int e = lane; e < Et; e += kWave) sm.tiles[e] = (sm.cnt[e] + bm - 1) / bm;
    }
    __syncthreads();
    if (wave == 1) wave_exclusive_scan(sm.tiles, Et, sm.tstart);
    for (int i = tid; i < NWAVES * E; i += nthr) sm.hist[i] += sm.offs[i % E];
    __syncthreads();

    // stable ranks; the expert ids of 8 rounds are fetched at once
    const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (kWave - lane));
    for (int base = a0; base < a1; base += 8 * kWave) {
        int ev[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int a = base + r * kWave + lane;
            ev[r] = a < a1 ? idx[a] : 0;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int a = base + r * kWave + lane;
            const bool valid = a < a1;
            const int e = ev[r];
            uint64_t same = __ballot(valid);
#pragma unroll
            for (int b = 0; b < 7; ++b) {
                const bool bit = (e >> b) & 1;
                const uint64_t bb = __ballot(valid && bit);
                same &= bit ? bb : ~bb;
            }
            if (valid) {
                const int rank = __popcll(same & lt_mask);
                const int pos = sm.hist[wave * E + e] + rank;
                const int t = a / k, j = a - t * k;
                o.sorted_c[pos] = t * kt + j;
                if (o.user_sorted) o.user_sorted[pos] = a;
                if (rank == 0) sm.hist[wave * E + e] += __popcll(same);
            }
        }
    }
    // shared virtual experts: every token, in order
    for (int i = tid; i < V * T; i += nthr) {
        const int v = i / T, t = i - v * T;
        o.sorted_c[N + i] = t * kt + k + v;
    }
    for (int e = tid; e <= Et; e += nthr) {
        if (e < Et) o.counts[e] = sm.cnt[e];
        o.offsets[e] = sm.offs[e];
        o.tile_start[e] = sm.tstart[e];
        if (e < E && o.user_counts) o.user_counts[e] = sm.cnt[e];
        if (e <= E && o.user_offsets) o.user_offsets[e] = sm.offs[e];
    }
}

// ---- the same scatter run by one wavefront, for small batches (a few hundred
// assignments): no workgroup barriers, one expert cursor array. A wave's LDS operations
// execute in order; lds_order() keeps the compiler from moving LDS accesses across the
// phase boundaries and waits for the phase's LDS writes.
constexpr int kScatterWaveMaxN = 256;  // assignments up to which one wavefront is faster

struct ScatterWaveSmem {
    int cnt[kMaxEt];
    int offs[kMaxEt + 1];
    int cur[kMaxEt];  // tiles per expert, then the running cursor of each expert
    int tstart[kMaxEt + 1];
};

__device__ __forceinline__ void lds_order() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ inline void scatter_wave(const int32_t* __restrict__ idx, int T, int E, int k, int V, int bm,
                                    const ScatterOut& o, ScatterWaveSmem& sm) {
    const int lane = threadIdx.x % kWave;
    const int N = T * k;
    const int kt = k + V;
    const int Et = E + V;
    for (int e = lane; e < Et; e += kWave) sm.cnt[e] = e < E ? 0 : T;  // shared slices: every token
    lds_order();
    for (int a = lane; a < N; a += kWave) atomicAdd(&sm.cnt[idx[a]], 1);
    lds_order();
    wave_exclusive_scan(sm.cnt, Et, sm.offs);
    for (int e = lane; e < Et; e += kWave) sm.cur[e] = (sm.cnt[e] + bm - 1) / bm;
    lds_order();
    wave_exclusive_scan(sm.cur, Et, sm.tstart);
    lds_order();
    for (int e = lane; e < E; e += kWave) sm.cur[e] = sm.offs[e];
    lds_order();
    // stable ranks, 64 assignments a round: lanes holding the same expert are found with
    // 7 ballots over the expert-id bits; the group's lowest lane advances the cursor
    const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (kWave - lane));
    for (int base = 0; base < N; base += kWave) {
        const int a = base + lane;
        const bool valid = a < N;
        const int e = valid ? idx[a] : 0;
        uint64_t same = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 7; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t bb = __ballot(valid && bit);
            same &= bit ? bb : ~bb;
        }
        const int rank = __popcll(same & lt_mask);
        if (valid) {
            const int pos = sm.cur[e] + rank;
            const int t = a / k, j = a - t * k;
            o.sorted_c[pos] = t * kt + j;
            if (o.user_sorted) o.user_sorted[pos] = a;
        }
        lds_order();
        if (valid && rank == 0) sm.cur[e] += __popcll(same);
        lds_order();
    }
    // shared virtual experts: every token, in order
    for (int i = lane; i < V * T; i += kWave) {
        const int v = i / T, t = i - v * T;
        o.sorted_c[N + i] = t * kt + k + v;
    }
    for (int e = lane; e <= Et; e += kWave) {
        if (e < Et) o.counts[e] = sm.cnt[e];
        o.offsets[e] = sm.offs[e];
        o.tile_start[e] = sm.tstart[e];
        if (e < E && o.user_counts) o.user_counts[e] = sm.cnt[e];
        if (e <= E && o.user_offsets) o.user_offsets[e] = sm.offs[e];
    }
}

}  // namespace moe
